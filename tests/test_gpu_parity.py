"""GPU parity of libwallattn against the fp64 oracle (run on an MI355X).

Every test calls the HIP library through its C ABI (via the thin binding)
and compares with ``oracle`` on identical seeded inputs:
  * element by element at sizes the oracle finishes in seconds, spanning
    several tiles and a ragged tail;
  * on sampled rows at the full workload sizes, in the launch configuration
    the benchmark times;
  * bit-exact for the tile skipping and varlen indexing (q = 0 probes);
  * decode: cache build, decode over an oracle-built cache, the whole
    decode pipeline against the forward's last row, and streaming.
Tolerances (max-abs against the unrounded fp64 oracle): 2e-2 for bf16
inputs, 1e-4 for fp32 inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_channel_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
DEV = "cuda:0"


def lse_tol(dtype, ref):
    """Prefill lse bound: the output bound for bf16 inputs (the scores are
    moderate on every prefill case); for fp32 inputs 1e-4 plus the float32
    representation of lse itself, 2^-22 |lse|."""
    if dtype == torch.bfloat16:
        return TOL[dtype] + 0.0 * np.abs(ref)
    return TOL[dtype] + 2.0 ** -22 * np.abs(ref)


@pytest.fixture(scope="module")
def wa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_channel_amd as lib
    lib.load_library()  # raises if the HIP library is missing
    return lib


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_gpu(wa, x, return_lse=True):
    d = to_dev(x)
    o, lse = wa.wall_attn(d["q"], d["k"], d["v"], d["g"], scale=d["scale"], g_scalar=d["g_scalar"],
                          sink_bias=d["sink_bias"], window_size=d["window_size"],
                          cu_seqlens=d["cu_seqlens"], return_lse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_oracle(x, rows=None):
    return oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"], g_scalar=x["g_scalar"],
                            sink_bias=x["sink_bias"], window_size=x["window_size"],
                            cu_seqlens=x["cu_seqlens"], rows=rows, return_lse=True)


def assert_repeatable(wa, x, o, lse, what):
    """A second launch on the same inputs returns the same bits (no atomics,
    fixed reduction orders)."""
    o2, lse2 = run_gpu(wa, x)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), what + ": second launch differs"


def check(got, ref, tol, what):
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err), err.shape)
    tol_a = np.broadcast_to(np.asarray(tol, dtype=np.float64), err.shape)
    print(f"{what}: max-abs err {err.max():.3e} at {i} (tol {tol_a[i]:.3g})", flush=True)
    assert np.isfinite(got).all(), what
    bad = err > tol_a
    assert not bad.any(), (f"{what}: {bad.sum()} elements over tolerance; max-abs error "
                           f"{err.max():.3e} at {i}")


def cfg(name, B, T, HQ, H, K, V, dtype, **kw):
    return W.Prefill(name, B, T, HQ, H, K, V, dtype, **kw)


SMALL = [
    cfg("bf16_T300_ragged", 2, 300, 4, 2, 64, 64, torch.bfloat16, seed=11),
    cfg("bf16_T200_D128_gate_sink_window70", 1, 200, 4, 1, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=70, seed=12),
    cfg("bf16_T257_K64_V128_gqa4", 1, 257, 8, 2, 64, 128, torch.bfloat16, sink=True, seed=13),
    cfg("bf16_T191_K128_V64", 2, 191, 2, 2, 128, 64, torch.bfloat16, g_scalar_std=0.02, seed=14),
    cfg("bf16_T1", 3, 1, 4, 2, 64, 64, torch.bfloat16, sink=True, seed=15),
    cfg("bf16_T64_window1", 1, 64, 2, 1, 64, 64, torch.bfloat16, window=1, seed=16),
    cfg("bf16_varlen_window100", 1, 0, 4, 2, 64, 64, torch.bfloat16, nseq=9, len_lo=1, len_hi=300,
        window=100, g_scalar_std=0.01, sink=True, seed=17),
    cfg("f32_T190_D128_V64_gate_sink_window", 1, 190, 4, 2, 128, 64, torch.float32,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=77, seed=18),
    cfg("f32_varlen", 1, 0, 2, 1, 64, 64, torch.float32, nseq=6, len_lo=1, len_hi=200, seed=19),
    cfg("f32_T1", 1, 1, 2, 1, 64, 64, torch.float32, seed=20),
    cfg("bf16_T450_D128_gqa8_gate_sink_window300", 1, 450, 8, 1, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=300, seed=23),
    # the decay sum of channel 0 rises 0.1 log2 units per token (that channel
    # of k is zero): the second query tile's anchor lies ~13 log2 units above
    # the first key chunk's, so the kernel rebalances that tile pair with
    # sigma = 5 (query operand times 2^-5, scores times 2^5)
    cfg("bf16_T256_rising_channel_sigma", 2, 256, 4, 2, 64, 64, torch.bfloat16,
        rise_ch0_log2=0.1, g_scalar_std=0.01, sink=True, seed=24),
    cfg("bf16_T256_D128_rising_channel_sigma_window100", 1, 256, 4, 1, 128, 128, torch.bfloat16,
        rise_ch0_log2=0.1, window=100, seed=25),
    # 64 packed sequences x 8 heads x up to 11 chunks: more pre-pass
    # workgroups than the GPU holds at once, so the pre-pass runs its
    # (key/value head, chunk) pair order
    cfg("bf16_varlen64_gqa4_pair_order", 1, 0, 8, 2, 64, 64, torch.bfloat16, nseq=64, len_lo=1,
        len_hi=700, g_scalar_std=0.01, sink=True, seed=26),
    # long enough for steady tile pairs with K=128, V=64 and with K=64, V=128
    # (the latter windowed: ceil((W-1)/32) odd, so the window start is rounded
    # down to a chunk)
    cfg("bf16_T700_K128_V64_gqa2_gate_sink", 1, 700, 4, 2, 128, 64, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, seed=27),
    cfg("bf16_varlen_K64_V128_window200", 1, 0, 4, 1, 64, 128, torch.bfloat16, nseq=6,
        len_lo=100, len_hi=900, window=200, seed=28),
    # long rows on few heads: many steady tile pairs per workgroup, windowed
    # with gate and sink, and three long packed sequences
    cfg("bf16_T1536_window700_gate_sink", 1, 1536, 4, 2, 64, 64, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=700, seed=29),
    cfg("bf16_varlen3_long_D128_sink", 1, 0, 2, 1, 128, 128, torch.bfloat16, nseq=3,
        len_lo=600, len_hi=1500, sink=True, seed=30),
]


@pytest.mark.parametrize("c", SMALL, ids=[c.name for c in SMALL])
def test_prefill_small_full(wa, c):
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, TOL[c.dtype], c.name + " o")
    check(lse, rl, lse_tol(c.dtype, rl), c.name + " lse")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_varlen_with_empty_sequences(wa, dtype):
    """cu_seqlens with zero-length sequences first and in the middle."""
    c = cfg("varlen_empty", 1, 0, 4, 2, 64, 64, dtype, nseq=9, len_lo=0, len_hi=90, window=33,
            g_scalar_std=0.01, sink=True, seed=41)
    x = W.make_prefill(c)
    assert x["q"].shape[1] == 350
    x["cu_seqlens"] = torch.tensor([0, 0, 13, 13, 13, 124, 141, 141, 292, 350], dtype=torch.int32)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, TOL[dtype], "varlen with empty sequences o")
    check(lse, rl, lse_tol(dtype, rl), "varlen with empty sequences lse")


def test_prefill_extreme_sink(wa):
    """A sink logit far above (+25) or below (-25) every score."""
    c = SMALL[1]
    x = W.make_prefill(c)
    x["sink_bias"] = torch.tensor([25.0, -25.0, 0.0, 5.0])
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, TOL[c.dtype], "extreme sink o")
    check(lse, rl, lse_tol(c.dtype, rl), "extreme sink lse")


def test_config_tiny_fp32_full(wa):
    c = W.PREFILL_T128_FP32
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, 1e-4, c.name)


def test_config_usage_bf16_full(wa):
    c = W.PREFILL_T1024_BF16
    x = W.make_prefill(c)
    o, _ = run_gpu(wa, x)
    ro, _ = run_oracle(x)
    check(o, ro, 2e-2, c.name)


def test_config_usage_bf16_g_zero_is_softmax_attention(wa):
    """README introduction: g = 0 gives vanilla softmax attention."""
    c = W.Prefill(W.PREFILL_T1024_BF16.name + "_g0", 2, 1024, 8, 4, 64, 64, torch.bfloat16,
                  g_mode="zero", seed=2)
    x = W.make_prefill(c)
    o, _ = run_gpu(wa, x)
    ro, _ = run_oracle(x)
    check(o, ro, 2e-2, c.name + " vs oracle")
    rep = lambda t: t.float().repeat_interleave(2, dim=2).transpose(1, 2).double()
    sd = torch.nn.functional.scaled_dot_product_attention(
        x["q"].float().transpose(1, 2).double(), rep(x["k"]), rep(x["v"]), is_causal=True,
        scale=x["scale"]).transpose(1, 2).numpy()
    check(o, sd, 2e-2, c.name + " vs SDPA")


REF_OVERFLOW = [
    cfg("bf16_T700_D128_rising_gate", 1, 700, 4, 2, 128, 128, torch.bfloat16, g_mode="neg_softplus",
        g_std=0.05, sink=True, seed=21),
    cfg("bf16_varlen_window150_K64_rising_gate", 1, 0, 4, 2, 64, 64, torch.bfloat16, nseq=5,
        len_lo=40, len_hi=500, window=150, seed=22),
]


@pytest.mark.parametrize("c", REF_OVERFLOW, ids=[c.name for c in REF_OVERFLOW])
def test_prefill_gate_favouring_old_keys(wa, c):
    """A positive g_scalar (the running gate sum grows along the sequence) puts
    the largest scores on the oldest visible keys, hundreds of log2 units above
    the newest ones: the kernel's per-row reference taken from the newest keys
    cannot hold those probabilities, and the recompute with the exact row max
    must give the oracle's result."""
    x = W.make_prefill(c)
    shape = x["q"].shape[:3]
    x["g_scalar"] = torch.full(shape, 0.5, dtype=c.dtype)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, TOL[c.dtype], c.name + " o")
    check(lse, rl, lse_tol(c.dtype, rl), c.name + " lse")
    assert_repeatable(wa, x, o, lse, c.name)  # the recompute path, run twice


WIDE = [
    # decay sums that leave the anchored operands' range: the pre-pass sends
    # these (sequence, head) pairs to the attention kernels' exact path
    cfg("bf16_T1024_strong_decay_gate_sink", 1, 1024, 4, 2, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.5, g_scalar_std=0.01, sink=True, seed=61),
    cfg("bf16_T1024_strong_decay_window300", 1, 1024, 4, 2, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.5, window=300, seed=62),
    cfg("bf16_T1024_fast_channels", 1, 1024, 4, 2, 128, 128, torch.bfloat16, fast_ch=4,
        fast_g=-2.0, sink=True, seed=63),
    # only query head 0 decays fast: heads 1..3 stay on the factorised kernel
    cfg("bf16_T700_K64_fast_channels_head0", 2, 700, 4, 2, 64, 64, torch.bfloat16, fast_ch=3,
        fast_g=-2.0, fast_heads=1, g_scalar_std=0.01, seed=64),
    cfg("bf16_varlen_fast_channels_window90", 1, 0, 4, 1, 128, 64, torch.bfloat16, nseq=5,
        len_lo=1, len_hi=400, fast_ch=8, fast_g=-2.0, window=90, sink=True, seed=65),
    cfg("f32_T1024_fast_channels_gate", 1, 1024, 2, 1, 64, 128, torch.float32, fast_ch=4,
        fast_g=-2.0, g_scalar_std=0.01, sink=True, seed=66),
    # fp32 operands hold -0.5 softplus decays (no exact path)
    cfg("f32_T600_strong_decay", 1, 600, 2, 1, 128, 64, torch.float32, g_mode="neg_softplus",
        g_std=0.5, seed=67),
]


@pytest.mark.parametrize("c", WIDE, ids=[c.name for c in WIDE])
def test_prefill_out_of_operand_range(wa, c):
    """Strong decays (Wall Attention README, "Features": anchors keep every
    exp2 bounded only while a chunk's decay span is representable) give the
    oracle's result, never NaN."""
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, TOL[c.dtype], c.name + " o")
    check(lse, rl, lse_tol(c.dtype, rl), c.name + " lse")
    assert_repeatable(wa, x, o, lse, c.name)  # the exact path, run twice


def boundary_rows(bos, eos, step=64, extra=()):
    rows = set()
    for t in range(bos, eos, step):
        for d in (-1, 0, 1):
            if bos <= t + d < eos:
                rows.add(t + d)
    rows.update(r for r in extra if bos <= r < eos)
    rows.update([bos, eos - 1])
    return rows


def test_config_long_8k_every_row(wa):
    """Every row of the 8K workload (8192 x 16 heads) against the oracle."""
    c = W.PREFILL_T8192_BF16
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    ro, rl = run_oracle(x)
    check(o, ro, 2e-2, c.name)
    check(lse, rl, lse_tol(c.dtype, rl), c.name + " lse")


def test_config_long_8k_deterministic(wa):
    """Two launches of the benchmark workload give identical bits."""
    x = W.make_prefill(W.PREFILL_T8192_BF16)
    a, la = run_gpu(wa, x)
    b, lb = run_gpu(wa, x)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_config_varlen_window_rows(wa):
    """Packed varlen workload: every 4th row of every sequence plus the rows
    around each 32-, 64- and 128-row tile boundary and the window edge."""
    c = W.VARLEN_W2048_BF16
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    cu = x["cu_seqlens"].tolist()
    rows = set()
    for s in range(len(cu) - 1):
        bos, eos = cu[s], cu[s + 1]
        rows |= set(range(bos, eos, 4))
        rows |= boundary_rows(bos, eos, step=32, extra=(bos + 2047, bos + 2048, bos + 2049))
    rows = sorted(rows)
    ro, rl = run_oracle(x, rows=rows)
    N = o.shape[1]
    check(o.reshape(N, c.HQ, c.V)[rows], ro, 2e-2, c.name + f" ({len(rows)} rows)")
    check(lse.reshape(N, c.HQ)[rows], rl, lse_tol(c.dtype, rl), c.name + " lse")
    assert_repeatable(wa, x, o, lse, c.name)


# ----------------------------------------------------------------------------- indexing probes

def probe_inputs(c, dtype):
    """q = 0 so every visible weight is exactly 2^0 = 1; v carries key offsets."""
    x = W.make_prefill(c)
    x["q"] = torch.zeros_like(x["q"]).to(dtype)
    x["g_scalar"] = None
    x["sink_bias"] = None
    for key in ("k", "v", "g"):
        x[key] = x[key].to(dtype)
    # value channels: (j - bos) mod 64 and (j - bos) div 64, exact in bf16 and fp32
    N = x["q"].shape[0] * x["q"].shape[1]
    cu = x["cu_seqlens"].tolist() if x["cu_seqlens"] is not None else [c.T * b for b in range(c.B + 1)]
    off = torch.zeros(N, dtype=torch.float32)
    for s in range(len(cu) - 1):
        off[cu[s]:cu[s + 1]] = torch.arange(cu[s + 1] - cu[s], dtype=torch.float32)
    v = torch.zeros(N, c.H, c.V, dtype=torch.float32)
    v[:, :, 0] = (off % 64)[:, None]
    v[:, :, 1] = torch.floor(off / 64)[:, None]
    x["v"] = v.reshape(x["v"].shape).to(dtype)
    return x, cu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("which", ["long8k", "varlen_w2048", "small_window"])
def test_block_skip_indexing_exact(wa, which, dtype):
    if which == "long8k":
        c = W.PREFILL_T8192_BF16
    elif which == "varlen_w2048":
        c = W.VARLEN_W2048_BF16
    else:
        c = cfg("probe_small", 1, 0, 2, 1, 64, 64, dtype, nseq=7, len_lo=1, len_hi=400, window=129,
                seed=21)
    x, cu = probe_inputs(c, dtype)
    o, lse = run_gpu(wa, x)
    N = o.shape[0] * o.shape[1]
    cnt_gpu = np.rint(np.exp(lse.reshape(N, c.HQ)))
    # expected visible-key counts from the mask definition: min(i - bos + 1, W)
    Wn = c.window if c.window > 0 else 10 ** 9
    exp_cnt = np.zeros(N)
    for s in range(len(cu) - 1):
        i = np.arange(cu[s + 1] - cu[s])
        exp_cnt[cu[s]:cu[s + 1]] = np.minimum(i + 1, Wn)
    assert np.array_equal(cnt_gpu, np.repeat(exp_cnt[:, None], c.HQ, 1)), "visible-key counts differ"
    # the oracle agrees on the same counts (sampled rows)
    rows = sorted(set(np.linspace(0, N - 1, 40).astype(int).tolist()) | {N - 1})
    _, rl = run_oracle(x, rows=rows)
    assert np.array_equal(np.rint(np.exp(rl)), cnt_gpu[rows])
    if dtype == torch.float32:
        # o * count recovers the sum of (j - bos) over the visible keys exactly
        o2 = o.reshape(N, c.HQ, c.V)
        # each channel's sum is an exact integer below 2^24; round them separately
        tot = np.rint(o2[:, :, 0] * cnt_gpu) + 64 * np.rint(o2[:, :, 1] * cnt_gpu)
        exp_sum = np.zeros(N)
        for s in range(len(cu) - 1):
            i = np.arange(cu[s + 1] - cu[s])
            lo = np.maximum(0, i - Wn + 1)
            exp_sum[cu[s]:cu[s + 1]] = (lo + i) * (i - lo + 1) / 2
        assert np.array_equal(tot, np.repeat(exp_sum[:, None], c.HQ, 1)), "visible-key ranges differ"


def test_deterministic(wa):
    c = SMALL[1]
    x = W.make_prefill(c)
    a, la = run_gpu(wa, x)
    b, lb = run_gpu(wa, x)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


