"""GPU parity of the backward pass (wall_attn_bwd) against the fp64 gradient
oracle (oracle.wall_attn_bwd, pinned to central differences and to autograd
through SDPA in test_oracle_grad_pins.py).

The pages fix no tolerance for gradients; the output tolerance (2e-2 for bf16
inputs, 1e-4 for fp32) is applied relative to each gradient's own scale:
max-abs error <= tol * max(1, max |reference|).  dg is a reverse running sum
over the sequence and grows with its length, so an absolute bound would
measure the length, not the kernel.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_channel_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


@pytest.fixture(scope="module")
def wa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_channel_amd as lib
    lib.load_library()
    return lib


def cfg(name, B, T, HQ, H, K, V, dtype, **kw):
    return W.Prefill(name, B, T, HQ, H, K, V, dtype, **kw)


CASES = [
    cfg("bf16_T300_gqa2", 2, 300, 4, 2, 64, 64, torch.bfloat16, seed=81),
    cfg("bf16_T200_D128_gate_sink_window70", 1, 200, 4, 1, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=70, seed=82),
    cfg("bf16_T257_K64_V128_gqa4_sink", 1, 257, 8, 2, 64, 128, torch.bfloat16, sink=True, seed=83),
    cfg("bf16_T191_K128_V64_gate", 2, 191, 2, 2, 128, 64, torch.bfloat16, g_scalar_std=0.02,
        seed=84),
    cfg("bf16_varlen_window100_gate_sink", 1, 0, 4, 2, 64, 64, torch.bfloat16, nseq=7, len_lo=1,
        len_hi=300, window=100, g_scalar_std=0.01, sink=True, seed=85),
    cfg("bf16_T1_sink", 3, 1, 4, 2, 64, 64, torch.bfloat16, sink=True, seed=86),
    cfg("bf16_T512_strong_decay_gate", 1, 512, 4, 2, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.5, g_scalar_std=0.01, seed=87),
    cfg("bf16_T400_fast_channels_sink", 1, 400, 4, 2, 64, 64, torch.bfloat16, fast_ch=4,
        fast_g=-2.0, sink=True, seed=88),
    cfg("f32_T190_D128_V64_gate_sink_window", 1, 190, 4, 2, 128, 64, torch.float32,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, window=77, seed=89),
    cfg("f32_varlen_gqa2", 1, 0, 4, 2, 64, 64, torch.float32, nseq=5, len_lo=1, len_hi=200,
        seed=90),
    # random-walk decay whose chunk-end sums rise by more than 4 log2 units
    # between chunks in most heads: those heads leave the matrix-core kernels
    # for the float32 ones (see test_rising_decay_case_leaves_the_fast_range)
    cfg("bf16_T384_rising_decay_gate", 1, 384, 4, 2, 64, 64, torch.bfloat16, g_mode="normal",
        g_std=0.07, g_scalar_std=0.01, seed=93),
    # the README's usage shape (B=2, T=1024, HQ=8, H=4, D=64)
    cfg("bf16_usage_shape_T1024", 2, 1024, 8, 4, 64, 64, torch.bfloat16, seed=91),
    # the long-context workload's head layout and decay at T=2048
    cfg("bf16_T2048_HQ16_H4_D128_gate_sink", 1, 2048, 16, 4, 128, 128, torch.bfloat16,
        g_mode="neg_softplus", g_std=0.05, g_scalar_std=0.01, sink=True, seed=92),
]


def grads_gpu(wa, x, dO):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o, lse = wa.wall_attn(d["q"], d["k"], d["v"], d["g"], scale=d["scale"], g_scalar=d["g_scalar"],
                          sink_bias=d["sink_bias"], window_size=d["window_size"],
                          cu_seqlens=d["cu_seqlens"], return_lse=True)
    out = wa.wall_attn_bwd(d["q"], d["k"], d["v"], d["g"], o, lse, dO.to(DEV), scale=d["scale"],
                           g_scalar=d["g_scalar"], sink_bias=d["sink_bias"],
                           window_size=d["window_size"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dg", "dg_scalar", "dsink")
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in zip(names, out) if t is not None}


def check_grads(got, ref, tol, what):
    for name, r in ref.items():
        e = np.abs(got[name] - r)
        bound = tol * max(1.0, float(np.abs(r).max()))
        i = np.unravel_index(np.argmax(e), e.shape)
        print(f"{what} {name}: max-abs err {e.max():.3e} at {i}, max|ref| {np.abs(r).max():.3e} "
              f"(bound {bound:.3e})", flush=True)
        assert np.isfinite(got[name]).all(), (what, name)
        assert e.max() <= bound, (what, name, float(e.max()), bound)


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_backward_matches_oracle(wa, c):
    x = W.make_prefill(c)
    gen = torch.Generator().manual_seed(c.seed + 1000)
    dO = torch.randn(x["q"].shape[:3] + (c.V,), generator=gen).to(c.dtype)
    got = grads_gpu(wa, x, dO)
    ref = oracle.wall_attn_bwd(x["q"], x["k"], x["v"], x["g"], dO, scale=x["scale"],
                               g_scalar=x["g_scalar"], sink_bias=x["sink_bias"],
                               window_size=x["window_size"], cu_seqlens=x["cu_seqlens"])
    check_grads(got, ref, TOL[c.dtype], c.name)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_backward_varlen_with_empty_sequences(wa, dtype):
    """cu_seqlens with zero-length sequences first, in the middle and in a
    row, next to sequences of one to three 64-token chunks."""
    c = cfg("bwd_varlen_empty", 1, 0, 4, 2, 64, 64, dtype, nseq=9, len_lo=0, len_hi=90, window=33,
            g_scalar_std=0.01, sink=True, seed=41)
    x = W.make_prefill(c)
    assert x["q"].shape[1] == 350
    x["cu_seqlens"] = torch.tensor([0, 0, 13, 13, 13, 124, 141, 141, 292, 350], dtype=torch.int32)
    dO = torch.randn(x["q"].shape[:3] + (c.V,), generator=torch.Generator().manual_seed(1041)).to(dtype)
    got = grads_gpu(wa, x, dO)
    ref = oracle.wall_attn_bwd(x["q"], x["k"], x["v"], x["g"], dO, scale=x["scale"],
                               g_scalar=x["g_scalar"], sink_bias=x["sink_bias"],
                               window_size=x["window_size"], cu_seqlens=x["cu_seqlens"])
    check_grads(got, ref, TOL[dtype], "backward, varlen with empty sequences")


def test_backward_deterministic(wa):
    c = CASES[1]
    x = W.make_prefill(c)
    dO = torch.randn(x["q"].shape[:3] + (c.V,), generator=torch.Generator().manual_seed(5)).to(c.dtype)
    a = grads_gpu(wa, x, dO)
    b = grads_gpu(wa, x, dO)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_rising_decay_case_leaves_the_fast_range():
    """Precondition of the rising-decay case: its chunk-end decay sums (log2
    units, rounded as the anchors are) rise by more than 4 between an older
    and a newer chunk in some head, which the matrix-core kernels hand to the
    float32 kernels, while no chunk spans more than the operands' 8 log2
    units (so the forward's own range flags stay clear)."""
    c = [x for x in CASES if x.name == "bf16_T384_rising_decay_gate"][0]
    g = W.make_prefill(c)["g"][0].double()
    P2 = torch.cumsum(g, 0) * 1.4426950408889634
    T = P2.shape[0]
    ends = [min(64 * i + 63, T - 1) for i in range((T + 63) // 64)]
    A = torch.stack([torch.round(P2[e]) for e in ends])
    rise = max(float((A[i] - A[j]).max()) for i in range(len(ends)) for j in range(i + 1))
    assert rise > 4
    span = float((P2 - A.repeat_interleave(64, 0)[:T]).abs().max())
    assert span < 7
