"""Pins for the fp64 oracle: checks against facts fixed outside the oracle itself.

Every test here runs on the CPU.  The oracle (``oracle/wall_oracle.c``) is
compared with
  * hand-derived worked examples (tests/golden/, each citing its passage),
  * a library routine (torch's scaled_dot_product_attention on CPU in fp64)
    for the special cases the pages reduce to plain attention,
  * closed forms (causal prefix mean, sink renormalisation, ALiBi-style gate,
    window of one token),
  * invariants (rows of weights sum to one, GQA == repeated MHA, packing and
    shift invariance for varlen), and
  * an mpmath brute force at 50 digits on tiny shapes.
Each is chosen so that a plausible slip in the oracle -- a flipped sign of the
decay, an exclusive instead of inclusive prefix, a wrong GQA head, a dropped
gate or sink term, an off-by-one window -- fails at least one of them.
"""
import json
import math
import os
import re

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f64 = torch.float64


def _val(x):
    """Evaluate a fixture entry: a number or an expression with lnX / log / exp."""
    if isinstance(x, (int, float)):
        return float(x)
    expr = re.sub(r"ln(\d+(?:\.\d+)?)", r"log(\1)", x)
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "exp": math.exp}))


def _rand(shape, seed, scale=1.0):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=gen, dtype=torch.float32) * scale)


def _inputs(B=2, T=37, HQ=4, H=2, K=16, V=8, seed=0, g_scale=0.05):
    q = _rand((B, T, HQ, K), seed)
    k = _rand((B, T, H, K), seed + 1)
    v = _rand((B, T, H, V), seed + 2)
    g = _rand((B, T, HQ, K), seed + 3, g_scale)
    return q, k, v, g


def _sdpa(q, k, v, scale, attn_mask=None, causal=True):
    """torch SDPA on CPU fp64; q [B,T,HQ,K], k [B,T,HQ,K], v [B,T,HQ,V] -> [B,T,HQ,V]."""
    qt, kt, vt = (x.to(f64).transpose(1, 2).contiguous() for x in (q, k, v))
    if attn_mask is not None:
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask, scale=scale)
    else:
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.transpose(1, 2).numpy()


def _rep(x, HQ):
    return x.repeat_interleave(HQ // x.shape[2], dim=2)


# ---------------------------------------------------------------- worked examples

def test_golden_two_token_decay():
    fx = json.load(open(os.path.join(GOLDEN, "two_token_decay.json")))
    t = lambda key: torch.tensor([_val(x) for x in fx[key]], dtype=torch.float32).reshape(1, 2, 1, 1)
    o, lse = oracle.wall_attn(t("q"), t("k"), t("v"), t("g"), scale=fx["scale"], return_lse=True)
    exp_o = [_val(x) for x in fx["expected_o"]]
    exp_l = [_val(x) for x in fx["expected_lse"]]
    # inputs such as ln(3)/2 are rounded to float32 before the oracle sees them
    np.testing.assert_allclose(o.reshape(-1), exp_o, rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse.reshape(-1), exp_l, rtol=0, atol=2e-6)


def test_golden_two_token_gate_sink_window():
    fx = json.load(open(os.path.join(GOLDEN, "two_token_gate_sink_window.json")))
    t = lambda key: torch.tensor([_val(x) for x in fx[key]], dtype=torch.float32).reshape(1, 2, 1, 1)
    gs = torch.tensor([_val(x) for x in fx["g_scalar"]], dtype=torch.float32).reshape(1, 2, 1)
    sink = torch.tensor([_val(x) for x in fx["sink_bias"]], dtype=torch.float32)
    o, lse = oracle.wall_attn(t("q"), t("k"), t("v"), t("g"), scale=fx["scale"], g_scalar=gs,
                              sink_bias=sink, return_lse=True)
    np.testing.assert_allclose(o.reshape(-1), [_val(x) for x in fx["expected_o"]], atol=2e-6)
    np.testing.assert_allclose(lse.reshape(-1), [_val(x) for x in fx["expected_lse"]], atol=2e-6)
    o1, lse1 = oracle.wall_attn(t("q"), t("k"), t("v"), t("g"), scale=fx["scale"], g_scalar=gs,
                                sink_bias=sink, window_size=1, return_lse=True)
    assert abs(o1.reshape(-1)[1] - _val(fx["window_1_expected_o_row1"])) < 2e-6
    assert abs(lse1.reshape(-1)[1] - _val(fx["window_1_expected_lse_row1"])) < 2e-6


# ---------------------------------------------------------------- library routines

def test_g_zero_is_softmax_attention():
    """README introduction: g = 0 recovers vanilla softmax attention."""
    q, k, v, g = _inputs(seed=10)
    g.zero_()
    HQ, K = q.shape[2], q.shape[3]
    scale = K ** -0.5
    o = oracle.wall_attn(q, k, v, g, scale=scale)
    ref = _sdpa(q, _rep(k, HQ), _rep(v, HQ), scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_decay_equals_rescaled_softmax_attention():
    """exp(P_i - P_j) = e^{P_i} e^{-P_j}: Wall Attention is SDPA on (q e^P, k e^-P).

    P here is torch's own cumulative sum (inclusive), and the attention is
    torch's SDPA, so this checks the oracle's prefix direction, sign and GQA
    head mapping through an independent route.
    """
    q, k, v, g = _inputs(seed=20, g_scale=0.1)
    HQ, K = q.shape[2], q.shape[3]
    scale = 0.3
    P = torch.cumsum(g.to(f64), dim=1)
    qs = q.to(f64) * torch.exp(P)
    ks = _rep(k, HQ).to(f64) * torch.exp(-P)
    ref = _sdpa(qs, ks, _rep(v, HQ), scale)
    o = oracle.wall_attn(q, k, v, g, scale=scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-11)


def test_channel_constant_decay_is_scalar_decay():
    """g[t,hq,n] = gamma_t for all n: the score is scale * e^{G_i - G_j} q_i.k_j."""
    B, T, HQ, H, K, V = 1, 29, 2, 1, 8, 4
    q, k, v, _ = _inputs(B, T, HQ, H, K, V, seed=30)
    gam = _rand((B, T, HQ, 1), 33, 0.4)
    g = gam.expand(B, T, HQ, K).contiguous()
    scale = K ** -0.5
    o = oracle.wall_attn(q, k, v, g, scale=scale)
    G = torch.cumsum(gam.to(f64), dim=1)[..., 0]                       # [B,T,HQ]
    logits = torch.einsum("bihn,bjhn->bhij", q.to(f64), _rep(k, HQ).to(f64)) * scale
    logits = logits * torch.exp(G.transpose(1, 2)[..., :, None] - G.transpose(1, 2)[..., None, :])
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    w = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)
    ref = torch.einsum("bhij,bjhv->bihv", w, _rep(v, HQ).to(f64)).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-11)


def test_scalar_gate_constant_is_alibi():
    """g_scalar = c for every token adds c*(i-j): an ALiBi bias of slope c."""
    q, k, v, g = _inputs(B=1, T=41, seed=40)
    g.zero_()
    HQ, K = q.shape[2], q.shape[3]
    T = q.shape[1]
    c = -0.125
    gs = torch.full((1, T, HQ), c, dtype=torch.float32)
    o = oracle.wall_attn(q, k, v, g, scale=K ** -0.5, g_scalar=gs)
    i = torch.arange(T, dtype=f64)
    bias = c * (i[:, None] - i[None, :])
    bias = bias.masked_fill(i[None, :] > i[:, None], float("-inf"))
    ref = _sdpa(q, _rep(k, HQ), _rep(v, HQ), K ** -0.5, attn_mask=bias)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_window_band_matches_masked_softmax():
    """FlexAttention rule 0 <= i - j < W, with g = 0, through SDPA's boolean mask."""
    q, k, v, g = _inputs(B=2, T=53, seed=50)
    g.zero_()
    HQ, K = q.shape[2], q.shape[3]
    T = q.shape[1]
    for W in (1, 2, 7, 16, 52, 53, 200):
        o = oracle.wall_attn(q, k, v, g, scale=K ** -0.5, window_size=W)
        i = torch.arange(T)
        d = i[:, None] - i[None, :]
        band = (d >= 0) & (d < W)
        ref = _sdpa(q, _rep(k, HQ), _rep(v, HQ), K ** -0.5, attn_mask=band)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12, err_msg=f"W={W}")


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("window", [None, 5])
def test_zero_query_gives_causal_prefix_mean(window):
    """q = 0 makes every visible score 0: o_i is the mean of the visible v_j."""
    q, k, v, g = _inputs(B=2, T=45, seed=60, g_scale=0.3)
    q.zero_()
    HQ = q.shape[2]
    o = oracle.wall_attn(q, k, v, g, window_size=window)
    vr = _rep(v, HQ).to(f64)
    T = q.shape[1]
    ref = np.zeros(o.shape)
    for i in range(T):
        lo = 0 if window is None else max(0, i - window + 1)
        ref[:, i] = vr[:, lo:i + 1].mean(dim=1).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def test_weights_sum_to_one():
    """v == 1: without a sink o == 1; with a sink o == 1 - exp(sink - lse)."""
    q, k, v, g = _inputs(B=1, T=33, seed=70, g_scale=0.2)
    v = torch.ones_like(v)
    HQ, T = q.shape[2], q.shape[1]
    gs = _rand((1, T, HQ), 71, 0.1)
    o = oracle.wall_attn(q, k, v, g, g_scalar=gs)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
    sink = _rand((HQ,), 72)
    o, lse = oracle.wall_attn(q, k, v, g, g_scalar=gs, sink_bias=sink, return_lse=True)
    sink_mass = np.exp(sink.numpy().astype(np.float64)[None, None, :] - lse)
    np.testing.assert_allclose(o, (1.0 - sink_mass)[..., None] * np.ones(o.shape), atol=1e-13)


def test_sink_renormalises_closed_form():
    """A value-less sink logit b: o = o0 / (1 + e^{b - lse0}), lse = log(e^{lse0} + e^b)."""
    q, k, v, g = _inputs(seed=80)
    HQ = q.shape[2]
    o0, l0 = oracle.wall_attn(q, k, v, g, return_lse=True)
    sink = _rand((HQ,), 81, 2.0)
    o1, l1 = oracle.wall_attn(q, k, v, g, sink_bias=sink, return_lse=True)
    b = sink.numpy().astype(np.float64)[None, None, :]
    np.testing.assert_allclose(o1, o0 / (1.0 + np.exp(b - l0))[..., None], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, np.logaddexp(l0, b), rtol=0, atol=1e-13)


def test_window_one_returns_own_value():
    """W = 1: o_i = v_i; with a sink, o_i = v_i * sigmoid(s_ii - sink), s_ii = scale q_i.k_i."""
    q, k, v, g = _inputs(B=1, T=19, seed=90, g_scale=0.5)
    HQ, K = q.shape[2], q.shape[3]
    o = oracle.wall_attn(q, k, v, g, window_size=1)
    vr = _rep(v, HQ).to(f64).numpy()
    np.testing.assert_allclose(o, vr, rtol=0, atol=1e-14)
    sink = _rand((HQ,), 91)
    o = oracle.wall_attn(q, k, v, g, window_size=1, sink_bias=sink)
    sii = (q.to(f64) * _rep(k, HQ).to(f64)).sum(-1).numpy() * K ** -0.5
    sig = 1.0 / (1.0 + np.exp(sink.numpy().astype(np.float64)[None, None, :] - sii))
    np.testing.assert_allclose(o, vr * sig[..., None], rtol=0, atol=1e-13)


def test_window_at_least_length_is_no_window():
    q, k, v, g = _inputs(B=1, T=31, seed=100)
    a = oracle.wall_attn(q, k, v, g)
    for W in (31, 32, 1000):
        np.testing.assert_array_equal(oracle.wall_attn(q, k, v, g, window_size=W), a)


# ---------------------------------------------------------------- invariants

def test_gqa_equals_repeated_mha():
    q, k, v, g = _inputs(B=1, T=27, HQ=6, H=2, seed=110)
    a = oracle.wall_attn(q, k, v, g)
    b = oracle.wall_attn(q, _rep(k, 6), _rep(v, 6), g)
    np.testing.assert_array_equal(a, b)
    # a wrong group mapping (hq % H instead of hq // (HQ/H)) would differ:
    kb = k[:, :, [0, 1, 0, 1, 0, 1]]
    vb = v[:, :, [0, 1, 0, 1, 0, 1]]
    assert np.abs(oracle.wall_attn(q, kb, vb, g) - a).max() > 1e-3


def test_varlen_packing_invariance():
    """Packed sequences (cu_seqlens, B == 1) give each sequence's own output."""
    lens = [5, 17, 1, 33, 12]
    HQ, H, K, V = 4, 2, 8, 8
    seqs = [_inputs(1, L, HQ, H, K, V, seed=120 + s, g_scale=0.2) for s, L in enumerate(lens)]
    gs = [_rand((1, L, HQ), 140 + s, 0.1) for s, L in enumerate(lens)]
    sink = _rand((HQ,), 150)
    cat = lambda idx: torch.cat([s[idx] for s in seqs], dim=1)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    for W in (None, 4):
        packed = oracle.wall_attn(cat(0), cat(1), cat(2), cat(3), g_scalar=torch.cat(gs, 1),
                                  sink_bias=sink, window_size=W, cu_seqlens=cu)
        alone = np.concatenate([oracle.wall_attn(*s, g_scalar=gsi, sink_bias=sink, window_size=W)
                                for s, gsi in zip(seqs, gs)], axis=1)
        np.testing.assert_allclose(packed, alone, rtol=0, atol=1e-14)


def test_prefix_shift_invariance():
    """Adding a constant to g at a segment start shifts P uniformly: no change."""
    q, k, v, g = _inputs(B=2, T=23, seed=160, g_scale=0.2)
    a = oracle.wall_attn(q, k, v, g)
    g2 = g.clone()
    g2[:, 0] += 0.75
    b = oracle.wall_attn(q, k, v, g2)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # while the same constant added mid-sequence does change later rows
    g3 = g.clone()
    g3[:, 11] += 0.75
    c = oracle.wall_attn(q, k, v, g3)
    np.testing.assert_allclose(a[:, :11], c[:, :11], rtol=0, atol=1e-12)
    assert np.abs(a[:, 12:] - c[:, 12:]).max() > 1e-3


def test_rows_subset_matches_full():
    q, k, v, g = _inputs(B=2, T=40, seed=170)
    full = oracle.wall_attn(q, k, v, g).reshape(80, q.shape[2], -1)
    rows = [0, 5, 39, 40, 41, 79]
    part = oracle.wall_attn(q, k, v, g, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


# ---------------------------------------------------------------- brute force

def test_mpmath_bruteforce_tiny():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    B, T, HQ, H, K, V = 1, 6, 2, 1, 3, 2
    q, k, v, g = _inputs(B, T, HQ, H, K, V, seed=180, g_scale=0.7)
    gs = _rand((B, T, HQ), 181, 0.3)
    sink = _rand((HQ,), 182)
    scale, W = 0.61, 4
    o, lse = oracle.wall_attn(q, k, v, g, scale=scale, g_scalar=gs, sink_bias=sink,
                              window_size=W, return_lse=True)
    mp = lambda x: mpmath.mpf(float(x))
    for hq in range(HQ):
        for i in range(T):
            logits = []
            for j in range(max(0, i - W + 1), i + 1):
                acc = mpmath.mpf(0)
                for n in range(K):
                    dec = mpmath.mpf(0)
                    for u in range(j + 1, i + 1):     # decay accumulated strictly after j up to i
                        dec += mp(g[0, u, hq, n])
                    acc += mp(q[0, i, hq, n]) * mp(k[0, j, 0, n]) * mpmath.exp(dec)
                gate = mpmath.fsum(mp(gs[0, u, hq]) for u in range(j + 1, i + 1))
                logits.append((j, mpmath.mpf(scale) * acc + gate))
            Z = mpmath.fsum(mpmath.exp(s) for _, s in logits) + mpmath.exp(mp(sink[hq]))
            for c in range(V):
                num = mpmath.fsum(mpmath.exp(s) * mp(v[0, j, 0, c]) for j, s in logits)
                assert abs(float(num / Z) - o[0, i, hq, c]) < 1e-13
            assert abs(float(mpmath.log(Z)) - lse[0, i, hq]) < 1e-13


# ---------------------------------------------------------------- decode side

def test_prefix_log2_is_cumsum_over_ln2():
    q, k, v, g = _inputs(B=2, T=50, seed=190)
    P2 = oracle.prefix_log2(g)
    ref = np.cumsum(g.numpy().astype(np.float64), axis=1) / math.log(2.0)
    np.testing.assert_allclose(P2, ref, rtol=0, atol=1e-13)
    cu = torch.tensor([0, 7, 30, 50], dtype=torch.int32)
    g1 = g[:1]
    P2v = oracle.prefix_log2(g1, cu_seqlens=cu)
    parts = [np.cumsum(g1[:, a:b].numpy().astype(np.float64), axis=1) / math.log(2.0)
             for a, b in zip(cu[:-1].tolist(), cu[1:].tolist())]
    np.testing.assert_allclose(P2v, np.concatenate(parts, axis=1), rtol=0, atol=1e-13)


def test_cache_anchor_and_inverse():
    """R_c is P2 at the chunk's last token; k_tilde * 2^(P2 - R) gives back k."""
    B, T, HQ, H, K, C = 2, 150, 4, 2, 8, 64
    _, k, _, g = _inputs(B, T, HQ, H, K, 4, seed=200, g_scale=0.1)
    P2 = oracle.prefix_log2(g).astype(np.float32)
    kt, rc = oracle.build_kv_cache(k, P2, chunk_size=C)
    assert rc.shape == (B, 3, HQ, K)
    for c, last in enumerate([63, 127, 149]):
        np.testing.assert_array_equal(rc[:, c], P2[:, last].astype(np.float64))
    cidx = np.arange(T) // C
    back = kt * np.exp2(P2.astype(np.float64) - rc[:, cidx])
    np.testing.assert_allclose(back, _rep(k, HQ).numpy().astype(np.float64), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("sink", [False, True])
def test_decode_from_cache_equals_forward_last_row(sink):
    """README "Decode": decode over the pre-rescaled cache reproduces the forward."""
    B, T, HQ, H, K, V, C = 2, 150, 4, 2, 16, 8, 64
    q, k, v, g = _inputs(B, T, HQ, H, K, V, seed=210, g_scale=0.1)
    sb = _rand((HQ,), 211) if sink else None
    o_full, l_full = oracle.wall_attn(q, k, v, g, sink_bias=sb, return_lse=True)
    P2 = oracle.prefix_log2(g).astype(np.float32)
    kt, rc = oracle.build_kv_cache(k, P2, chunk_size=C)
    od, ld = oracle.decode(q[:, -1:], v, P2[:, -1:], kt.astype(np.float32), rc.astype(np.float32),
                           sink_bias=sb, cache_chunk_size=C, return_lse=True)
    # the float32 cache and P2 round at ~1e-7 relative
    np.testing.assert_allclose(od[:, 0], o_full[:, -1], rtol=0, atol=2e-6)
    np.testing.assert_allclose(ld[:, 0], l_full[:, -1], rtol=0, atol=2e-6)


# ---------------------------------------------------------------- decode with serving options

def _cache_for(k, g, C=64):
    P2 = oracle.prefix_log2(g).astype(np.float32)
    kt, rc = oracle.build_kv_cache(k, P2, chunk_size=C)
    return P2, kt.astype(np.float32), rc.astype(np.float32)


@pytest.mark.parametrize("window", [None, 1, 37, 100])
def test_decode_ext_window_gate_equals_forward_row(window):
    """Decode over the cache with a window and the gate cache reproduces the
    forward's last row with the same window and g_scalar (README "Decode" and
    "Tests"; the forward is pinned to SDPA and closed forms above)."""
    B, T, HQ, H, K, V = 2, 150, 4, 2, 16, 8
    q, k, v, g = _inputs(B, T, HQ, H, K, V, seed=220, g_scale=0.1)
    gs = _rand((B, T, HQ), 221, 0.1)
    sb = _rand((HQ,), 222)
    o_full, l_full = oracle.wall_attn(q, k, v, g, g_scalar=gs, sink_bias=sb, window_size=window,
                                      return_lse=True)
    P2, kt, rc = _cache_for(k, g)
    G2 = (np.cumsum(gs.numpy().astype(np.float64), axis=1) / math.log(2.0)).astype(np.float32)
    od, ld = oracle.decode_ext(q[:, -1:], v, P2[:, -1:], kt, rc, sink_bias=sb, gate_cache=G2,
                               gate_curr=G2[:, -1:], window_size=window, return_lse=True)
    np.testing.assert_allclose(od[:, 0], o_full[:, -1], rtol=0, atol=2e-6)
    np.testing.assert_allclose(ld[:, 0], l_full[:, -1], rtol=4e-7, atol=2e-6)


def test_decode_ext_lengths_equal_truncated_forward():
    """Row b holding len_b tokens of a longer cache decodes as the forward over
    its first len_b tokens (query at len_b - 1); len_b = 0 gives o = 0 and
    lse = the sink logit."""
    B, T, HQ, H, K, V = 3, 140, 4, 2, 16, 8
    q, k, v, g = _inputs(B, T, HQ, H, K, V, seed=230, g_scale=0.1)
    sb = _rand((HQ,), 231)
    P2, kt, rc = _cache_for(k, g)
    lens = [0, 65, 140]
    qs = torch.stack([q[b, max(L - 1, 0)] for b, L in enumerate(lens)])[:, None]
    ps = np.stack([P2[b, max(L - 1, 0)] for b, L in enumerate(lens)])[:, None]
    od, ld = oracle.decode_ext(qs, v, ps, kt, rc, sink_bias=sb,
                               cache_seqlens=np.array(lens, dtype=np.int32), return_lse=True)
    np.testing.assert_array_equal(od[0], 0.0)
    np.testing.assert_array_equal(ld[0, 0], sb.numpy().astype(np.float64))
    for b in (1, 2):
        L = lens[b]
        of, lf = oracle.wall_attn(q[b:b + 1, :L], k[b:b + 1, :L], v[b:b + 1, :L], g[b:b + 1, :L],
                                  sink_bias=sb, return_lse=True)
        np.testing.assert_allclose(od[b, 0], of[0, -1], rtol=0, atol=2e-6)
        # the float32 cache rounds each score at ~2^-24 relative
        np.testing.assert_allclose(ld[b, 0], lf[0, -1], rtol=4e-7, atol=2e-6)
