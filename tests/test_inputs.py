"""CPU checks of the seeded inputs themselves: properties that GPU tests rely on
to reach a code path (no GPU, no library)."""
import math

import numpy as np
import torch

from exact_attention_channel_amd import workloads as W


def _anchor_gaps(x, chunk=64, qtile=128):
    """Largest (query-tile anchor - key-chunk anchor) over all visible pairs, per
    channel, in log2 units.  Anchors: the integer nearest to the running sum of
    g (log2 units) at the chunk's last token; a query tile's anchor is its first
    chunk's."""
    g = x["g"].float().numpy()[0]                       # [T, HQ, K]
    P = np.cumsum(g.astype(np.float64), axis=0) / math.log(2)
    L = P.shape[0]
    nch = (L + chunk - 1) // chunk
    R = np.stack([np.rint(P[min(chunk * c + chunk - 1, L - 1)]) for c in range(nch)])
    best = -np.inf
    for I in range((L + qtile - 1) // qtile):
        RQ = R[min(2 * I, nch - 1)]
        best = max(best, float((RQ[None] - R[:min(2 * I + 2, nch)]).max()))
    return best


def test_rising_channel_inputs_reach_rebalancing():
    """The rising-channel GPU cases need an anchor gap above 8 log2 units (the
    kernel's rebalancing threshold) while the rising channel adds nothing to any
    score (its k is zero)."""
    c = W.Prefill("rise", 2, 256, 4, 2, 64, 64, torch.bfloat16, rise_ch0_log2=0.1, seed=24)
    x = W.make_prefill(c)
    gap = _anchor_gaps(x)
    assert 8 < gap <= 16, gap
    assert float(x["k"][..., 0].abs().max()) == 0.0


def operand_exponents(x, chunk=64):
    """Largest |R_c - P2_j| (the rescaled keys' exponent) and |P2_i - RQ| (the
    rescaled queries', RQ the anchor of the first chunk of the 128-row query
    tile) over every (segment, head, channel), in log2 units; anchors are the
    integer nearest to P2 at each chunk's last token."""
    g = x["g"].float().numpy().astype(np.float64)
    cu = x["cu_seqlens"]
    segs = ([(b, 0, g.shape[1]) for b in range(g.shape[0])] if cu is None
            else [(0, a, b) for a, b in zip(cu[:-1].tolist(), cu[1:].tolist())])
    ek = eq = 0.0
    for b, lo, hi in segs:
        if hi <= lo:
            continue
        P = np.cumsum(g[b, lo:hi], axis=0) / math.log(2)
        L = P.shape[0]
        A = np.stack([np.rint(P[min(chunk * c + chunk - 1, L - 1)]) for c in range((L + chunk - 1) // chunk)])
        cidx = np.arange(L) // chunk
        ek = max(ek, float(np.abs(A[cidx] - P).max()))
        eq = max(eq, float(np.abs(P - A[cidx & ~1]).max()))
    return ek, eq


def test_benchmark_workloads_stay_in_the_half_operand_range():
    """The prefill workloads take the factorised path: both exponents within
    8 log2 units (the bound past which the pre-pass sends a (sequence, head)
    to the exact path)."""
    for c in (W.PREFILL_T1024_BF16, W.PREFILL_T8192_BF16, W.VARLEN_W2048_BF16):
        ek, eq = operand_exponents(W.make_prefill(c))
        assert ek <= 8 and eq <= 8, (c.name, ek, eq)


def test_strong_decay_inputs_leave_the_half_operand_range():
    """The GPU tests of the exact path use decays that overflow the half
    operands: g = -0.5 softplus(N) (about 37 log2 units per chunk) and
    channels decaying by 2 nats per token (185 per chunk; beyond float32 too)."""
    s = W.Prefill("s", 1, 1024, 4, 2, 128, 128, torch.bfloat16, g_mode="neg_softplus", g_std=0.5,
                  seed=61)
    f = W.Prefill("f", 1, 1024, 4, 2, 128, 128, torch.bfloat16, fast_ch=4, fast_g=-2.0, seed=63)
    assert min(operand_exponents(W.make_prefill(s))) > 30
    assert min(operand_exponents(W.make_prefill(f))) > 130


def test_default_workloads_stay_below_rebalancing():
    """The benchmark workload never rebalances (its decay sums fall), so its
    timing is the common path's."""
    x = W.make_prefill(W.PREFILL_T8192_BF16)
    assert _anchor_gaps(x) <= 8


def _pairs(lengths, window=0):
    """Allowed (i, j) pairs per head: 0 <= i - j < window (no window: i - j >= 0)."""
    tot = 0
    for n in lengths:
        if window <= 0 or n <= window:
            tot += n * (n + 1) // 2
        else:
            tot += window * (window + 1) // 2 + (n - window) * window
    return tot


def test_workload_recipes_match_the_stated_configurations():
    """Shapes, seeded varlen lengths and algorithmic work of the five workloads
    (the counting rule: 2*HQ*(K+V) FLOPs per allowed pair)."""
    c = W.PREFILL_T8192_BF16
    assert (c.B, c.T, c.HQ, c.H, c.K, c.V, c.window) == (1, 8192, 16, 4, 128, 128, 0)
    assert 2 * c.HQ * (c.K + c.V) * _pairs([c.T]) == 274_911_461_376
    v = W.VARLEN_W2048_BF16
    lens = W.varlen_lengths(v)
    assert lens == [3312, 4076, 1218, 2710, 896, 2878, 3871, 3993, 3569, 1298, 2295, 2293, 1177,
                    3015, 822, 1209]
    assert sum(lens) == 38_632 and all(512 <= n <= 4096 for n in lens)
    assert _pairs(lens, v.window) == 48_349_525
    assert round(2 * v.HQ * (v.K + v.V) * _pairs(lens, v.window) / 1e9, 2) == 792.16
    u = W.PREFILL_T1024_BF16
    assert (u.B, u.T, u.HQ, u.H, u.K, u.V) == (2, 1024, 8, 4, 64, 64)
    assert 2 * u.HQ * (u.K + u.V) * u.B * _pairs([u.T]) == 2_149_580_800
    t = W.PREFILL_T128_FP32
    assert (t.B, t.T, t.HQ, t.H, t.K, t.V, t.dtype) == (1, 128, 2, 1, 64, 64, torch.float32)
    d = W.DECODE_T32768_BF16
    assert (d.B, d.T_kv, d.HQ, d.H, d.K, d.V, d.C) == (64, 32768, 32, 8, 128, 128, 64)
    cache_bytes = (d.B * d.T_kv * d.HQ * d.K * 2 + d.B * d.T_kv * d.H * d.V * 2
                   + d.B * (d.T_kv // d.C) * d.HQ * d.K * 4)
    step_bytes = cache_bytes + d.B * d.HQ * d.K * 2 + d.B * d.HQ * d.K * 4 + d.B * d.HQ * d.V * 2
    assert step_bytes == 22_013_804_544
