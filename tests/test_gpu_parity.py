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
    """lse carries the score rounding of the rescaled operands, which grows
    with the score magnitude: allow the output tolerance plus a relative part
    (2^-9 of |lse| for the half operands of bf16 inputs, 2^-18 for fp32)."""
    rel = 2.0 ** -9 if dtype == torch.bfloat16 else 2.0 ** -18
    return TOL[dtype] + rel * np.abs(ref)


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


def boundary_rows(bos, eos, step=64, extra=()):
    rows = set()
    for t in range(bos, eos, step):
        for d in (-1, 0, 1):
            if bos <= t + d < eos:
                rows.add(t + d)
    rows.update(r for r in extra if bos <= r < eos)
    rows.update([bos, eos - 1])
    return rows


def test_config_long_8k_sampled(wa):
    c = W.PREFILL_T8192_BF16
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    T = c.T
    rng = np.random.default_rng(3)
    rows = set(range(0, T, 509)) | set(rng.integers(0, T, 24).tolist())
    rows |= {127, 128, 129, 4095, 4096, 8063, 8064, 8190, 8191}
    rows = sorted(rows)
    ro, rl = run_oracle(x, rows=rows)
    check(o.reshape(T, c.HQ, c.V)[rows], ro, 2e-2, c.name)
    check(lse.reshape(T, c.HQ)[rows], rl, lse_tol(c.dtype, rl), c.name + " lse")


def test_config_varlen_window_sampled(wa):
    c = W.VARLEN_W2048_BF16
    x = W.make_prefill(c)
    o, lse = run_gpu(wa, x)
    cu = x["cu_seqlens"].tolist()
    rng = np.random.default_rng(4)
    rows = set()
    for s in range(len(cu) - 1):
        bos, eos = cu[s], cu[s + 1]
        rows |= {bos, bos + 1, eos - 1, eos - 2, min(eos - 1, bos + 127), min(eos - 1, bos + 128),
                 min(eos - 1, bos + 2047), min(eos - 1, bos + 2048), min(eos - 1, bos + 2111)}
        rows |= set(rng.integers(bos, eos, 2).tolist())
    rows = sorted(rows)
    ro, rl = run_oracle(x, rows=rows)
    N = o.shape[1]
    check(o.reshape(N, c.HQ, c.V)[rows], ro, 2e-2, c.name)
    check(lse.reshape(N, c.HQ)[rows], rl, lse_tol(c.dtype, rl), c.name + " lse")


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


# ----------------------------------------------------------------------------- decode

def small_decode(B=3, T=300, HQ=8, H=2, K=128, V=128, dtype=torch.bfloat16, seed=31, sink=True):
    c = cfg("dec", B, T, HQ, H, K, V, dtype, sink=sink, seed=seed)
    return W.make_prefill(c)


def test_prefix_log2_matches_oracle(wa):
    x = small_decode(T=333)
    P2 = wa.wall_attn_prefix_log2(x["g"].to(DEV)).cpu().numpy()
    ref = oracle.prefix_log2(x["g"])
    check(P2, ref, 1e-4, "prefix_log2")
    c = cfg("dec_varlen", 1, 0, 4, 2, 64, 64, torch.bfloat16, nseq=5, len_lo=1, len_hi=200, seed=32)
    y = W.make_prefill(c)
    P2 = wa.wall_attn_prefix_log2(y["g"].to(DEV), cu_seqlens=y["cu_seqlens"].to(DEV)).cpu().numpy()
    check(P2, oracle.prefix_log2(y["g"], cu_seqlens=y["cu_seqlens"]), 1e-4, "prefix_log2 varlen")


@pytest.mark.parametrize("B,T", [(3, 300), (32, 1100)], ids=["chunk_order", "pair_order"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_build_cache_matches_oracle(wa, dtype, B, T):
    # 32 x 18 chunks x 8 heads exceed the workgroups the GPU holds at once:
    # the cache build then runs its (key/value head, chunk) pair order
    x = small_decode(B=B, T=T, dtype=dtype)
    P2 = torch.from_numpy(oracle.prefix_log2(x["g"]).astype(np.float32))
    kt, rc = wa.build_wall_kv_cache(x["k"].to(DEV), P2.to(DEV), chunk_size=64)
    rkt, rrc = oracle.build_kv_cache(x["k"], P2, chunk_size=64)
    assert np.array_equal(rc.cpu().numpy().astype(np.float64), rrc), "anchors must copy P2"
    assert kt.dtype == wa.cache_dtype(dtype)
    # round-to-nearest of a float32 product whose exp2 and multiply add ~2^-22
    rel = (2.0 ** -11 if dtype == torch.bfloat16 else 0.0) + 2.0 ** -21
    got = kt.float().cpu().numpy().astype(np.float64)
    # half subnormals (below 2^-14) round to a multiple of 2^-24
    absol = 2.0 ** -25 if dtype == torch.bfloat16 else 1e-30
    assert np.all(np.abs(got - rkt) <= rel * np.abs(rkt) + absol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_over_oracle_cache(wa, dtype):
    x = small_decode(T=300, dtype=dtype, B=2, HQ=8, H=2, K=64, V=128)
    P2 = oracle.prefix_log2(x["g"]).astype(np.float32)
    rkt, rrc = oracle.build_kv_cache(x["k"], P2, chunk_size=64)
    kt = torch.from_numpy(rkt).to(wa.cache_dtype(dtype))   # cache rounded on the CPU
    rc = torch.from_numpy(rrc.astype(np.float32))
    pc = torch.from_numpy(P2[:, -1:].copy())
    q = x["q"][:, -1:].contiguous()
    o, lse = wa.wall_attn_decode(q.to(DEV), x["v"].to(DEV), pc.to(DEV), kt.to(DEV), rc.to(DEV),
                                 sink_bias=x["sink_bias"].to(DEV), scale=x["scale"])
    ro, rl = oracle.decode(q, x["v"], pc, kt, rc, sink_bias=x["sink_bias"], scale=x["scale"],
                           return_lse=True)
    check(o.float().cpu().numpy(), ro, TOL[dtype], "decode over oracle cache")
    check(lse.cpu().numpy(), rl, lse_tol(dtype, rl), "decode lse")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 4096])
def test_decode_pipeline_equals_forward_last_row(wa, T):
    x = small_decode(T=T, B=2)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64)
    o, lse = wa.wall_attn_decode(d["q"][:, -1:].contiguous(), d["v"], P[:, -1:].contiguous(), kt,
                                 rc, sink_bias=d["sink_bias"], scale=d["scale"])
    torch.cuda.synchronize()
    rows = [b * T + T - 1 for b in range(x["q"].shape[0])]
    ro, rl = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"],
                              sink_bias=x["sink_bias"], rows=rows, return_lse=True)
    check(o[:, 0].float().cpu().numpy(), ro, 2e-2, f"decode T={T} vs oracle forward")
    check(lse[:, 0].cpu().numpy(), rl, lse_tol(torch.bfloat16, rl), f"decode lse T={T}")
    # and the GPU prefill's last row
    of = wa.wall_attn(d["q"], d["k"], d["v"], d["g"], scale=d["scale"], sink_bias=d["sink_bias"])
    check(o[:, 0].float().cpu().numpy(), of[:, -1].float().cpu().numpy(), 2e-2,
          f"decode T={T} vs GPU prefill")


def test_decode_streaming_matches_forward(wa):
    """Token-by-token decode reproduces every row of the forward (README "Tests")."""
    x = small_decode(T=150, B=1, HQ=4, H=2, K=64, V=64, seed=33)
    d = to_dev(x)
    ro, _ = run_oracle(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    worst = 0.0
    for t in range(1, 151):
        kt, rc = wa.build_wall_kv_cache(d["k"][:, :t].contiguous(), P[:, :t].contiguous())
        o, _ = wa.wall_attn_decode(d["q"][:, t - 1:t].contiguous(), d["v"][:, :t].contiguous(),
                                   P[:, t - 1:t].contiguous(), kt, rc, sink_bias=d["sink_bias"],
                                   scale=d["scale"])
        err = np.abs(o[0, 0].float().cpu().numpy() - ro[0, t - 1]).max()
        worst = max(worst, err)
    print(f"streaming worst max-abs {worst:.3e}", flush=True)
    assert worst <= 2e-2


def test_config_decode_32k_sampled(wa):
    """Full decode workload (B=64, T_kv=32768, HQ=32, H=8, D=128, C=64) in the benchmark's
    launch configuration.

    Kernel parity: for sampled batch rows the cache rows are replaced by an oracle-built
    cache (fp64 prefix and rescaling, rounded to the cache dtype on the CPU) and the GPU
    decode is compared with the oracle decoding that same cache.  The end-to-end pipeline
    (GPU prefix, GPU cache, GPU decode) is also compared with the oracle's forward last
    row and the error is printed: with a random-walk decay over 32K tokens the decode
    scores reach ~1e5 and the softmax is nearly an argmax with near ties, so a 16-bit
    cache cannot reproduce every row to 2e-2 (see the design notes); the end-to-end bound
    is asserted on the well-conditioned T_kv <= 4096 cases above.
    """
    c = W.DECODE_T32768_BF16
    x = W.make_decode(c, device=DEV)
    P = wa.wall_attn_prefix_log2(x["g"])
    kt, rc = wa.build_wall_kv_cache(x["k"], P, chunk_size=c.C)
    pc = P[:, -1:].contiguous()
    del P
    o_e2e, _ = wa.wall_attn_decode(x["q"], x["v"], pc, kt, rc, sink_bias=x["sink_bias"],
                                   scale=x["scale"], cache_chunk_size=c.C)
    torch.cuda.synchronize()
    rows = (0, 41, 63)
    ref = {}
    for b in rows:
        gb = x["g"][b:b + 1].cpu()
        P2 = oracle.prefix_log2(gb).astype(np.float32)
        rkt, rrc = oracle.build_kv_cache(x["k"][b:b + 1].cpu(), P2, chunk_size=c.C)
        kt_b = torch.from_numpy(rkt).to(kt.dtype)
        rc_b = torch.from_numpy(rrc.astype(np.float32))
        pc_b = torch.from_numpy(P2[:, -1:].copy())
        kt[b:b + 1].copy_(kt_b.to(DEV))
        rc[b:b + 1].copy_(rc_b.to(DEV))
        pc[b:b + 1].copy_(pc_b.to(DEV))
        ref[b] = oracle.decode(x["q"][b:b + 1].cpu(), x["v"][b:b + 1].cpu(), pc_b, kt_b, rc_b,
                               sink_bias=None if x["sink_bias"] is None else x["sink_bias"].cpu(),
                               scale=x["scale"], cache_chunk_size=c.C, return_lse=True)
        del rkt, rrc, P2
    o, lse = wa.wall_attn_decode(x["q"], x["v"], pc, kt, rc, sink_bias=x["sink_bias"],
                                 scale=x["scale"], cache_chunk_size=c.C)
    torch.cuda.synchronize()
    for b in rows:
        ro, rl = ref[b]
        check(o[b:b + 1].float().cpu().numpy(), ro, 2e-2, f"decode32k kernel b={b}")
        check(lse[b:b + 1].cpu().numpy(), rl, lse_tol(c.dtype, rl), f"decode32k kernel lse b={b}")
    # end to end against the forward's last row: measured and printed
    for b in rows:
        q = torch.zeros(1, c.T_kv, c.HQ, c.K, dtype=torch.float32)
        q[0, -1] = x["q"][b, 0].float().cpu()
        fo = oracle.wall_attn(q, x["k"][b:b + 1].cpu(), x["v"][b:b + 1].cpu(),
                              x["g"][b:b + 1].cpu(), scale=x["scale"],
                              sink_bias=None if x["sink_bias"] is None else x["sink_bias"].cpu(),
                              rows=[c.T_kv - 1])
        err = np.abs(o_e2e[b].float().cpu().numpy() - fo).max()
        print(f"decode32k end-to-end b={b}: max-abs err vs forward {err:.3e}", flush=True)
        assert np.isfinite(o_e2e[b].float().cpu().numpy()).all()


@pytest.mark.parametrize("B,T", [(4, 4096), (2, 2048)])
def test_decode_pipeline_full_heads_equals_forward(wa, B, T):
    """The decode workload's head layout (HQ=32, H=8, D=128) at T_kv where the problem is
    well conditioned: GPU prefix -> cache -> decode against the oracle forward's last row."""
    c = cfg("dec_full_heads", B, T, 32, 8, 128, 128, torch.bfloat16, seed=40 + T)
    x = W.make_prefill(c)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64)
    o, lse = wa.wall_attn_decode(d["q"][:, -1:].contiguous(), d["v"], P[:, -1:].contiguous(), kt,
                                 rc, scale=d["scale"])
    torch.cuda.synchronize()
    rows = [b * T + T - 1 for b in range(B)]
    ro, rl = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"], rows=rows,
                              return_lse=True)
    check(o[:, 0].float().cpu().numpy(), ro, 2e-2, f"decode heads32 T={T}")
    check(lse[:, 0].cpu().numpy(), rl, lse_tol(torch.bfloat16, rl), f"decode heads32 lse T={T}")
