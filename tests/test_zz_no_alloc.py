"""wall_attn_decode_noalloc (the decode without a workspace, for callers that
cannot allocate) against wall_attn_decode_ext through the C ABI: identical
outputs on two calls in a row, the second with a smaller input, and a
rejection, before any launch, of a call whose partials exceed the static
scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from exact_attention_channel_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_channel_amd as wa
    return wa.load_library()


def ptr(t):
    return None if t is None else t.data_ptr()


def case(wa, B, T, HQ, H, D, seed, lens=None, window=0, gate=False):
    c = W.Prefill("na", B, T, HQ, H, D, D, torch.bfloat16, sink=True, seed=seed,
                  g_scalar_std=0.02 if gate else 0.0)
    x = W.make_prefill(c)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    if gate:
        P, G = wa.wall_attn_prefix_log2(d["g"], g_scalar=d["g_scalar"])
    else:
        P, G = wa.wall_attn_prefix_log2(d["g"]), None
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64)
    L = lens if lens is not None else [T] * B
    q = torch.stack([d["q"][b, n - 1] for b, n in enumerate(L)])[:, None].contiguous()
    pc = torch.stack([P[b, n - 1] for b, n in enumerate(L)])[:, None].contiguous()
    gc = None if G is None else torch.stack([G[b, n - 1] for b, n in enumerate(L)])[:, None].contiguous()
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    return dict(x=x, d=d, P=P, G=G, kt=kt, rc=rc, q=q, pc=pc, gc=gc, sl=sl, B=B, T=T, HQ=HQ, H=H,
                D=D, window=window, L=L)


def run(lib, wa, cs, noalloc):
    B, T, HQ, H, D = cs["B"], cs["T"], cs["HQ"], cs["H"], cs["D"]
    d = cs["d"]
    o = torch.full((B, 1, HQ, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, 1, HQ), float("nan"), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    common = (ptr(cs["q"]), ptr(d["v"]), ptr(cs["pc"]), ptr(cs["kt"]), ptr(cs["rc"]),
              ptr(d["sink_bias"]), ptr(cs["G"]), ptr(cs["gc"]), ptr(o), ptr(lse), B, T, HQ, H, D,
              D, 64, float(d["scale"]), wa.WA_BF16, wa.WA_F32, ptr(cs["sl"]), cs["window"], None,
              0, 0, 0)
    if noalloc:
        rc = lib.wall_attn_decode_noalloc(*common, stream)
    else:
        need = lib.wall_attn_decode_workspace_bytes(B, T, HQ, H, D, D, 64)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        rc = lib.wall_attn_decode_ext(*common, ptr(ws), need, stream)
    assert rc == 0, lib.wall_attn_last_error().decode()
    torch.cuda.synchronize()
    return o, lse


def test_decode_noalloc_matches_decode_ext(lib):
    import exact_attention_channel_amd as wa
    first = case(wa, 8, 4096, 32, 8, 128, seed=70)
    second = case(wa, 3, 1000, 8, 2, 64, seed=71, lens=[1000, 1, 517], window=300, gate=True)
    for name, cs in (("first (B=8, T=4096)", first), ("second, smaller (B=3, T=1000)", second)):
        o_ref, l_ref = run(lib, wa, cs, noalloc=False)
        o, l = run(lib, wa, cs, noalloc=True)
        print(f"{name}: max-abs diff {float((o.float() - o_ref.float()).abs().max()):.3e}", flush=True)
        assert torch.isfinite(o).all() and torch.isfinite(l).all()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), name
        # and the oracle's decode over the same cache, to the parity bound
        x = cs["x"]
        ro = oracle.decode_ext(cs["q"].cpu(), x["v"], cs["pc"].cpu(), cs["kt"].cpu(), cs["rc"].cpu(),
                               sink_bias=x["sink_bias"], scale=x["scale"],
                               gate_cache=None if cs["G"] is None else cs["G"].cpu(),
                               gate_curr=None if cs["gc"] is None else cs["gc"].cpu(),
                               cache_seqlens=None if cs["sl"] is None else cs["L"],
                               window_size=cs["window"] or None)
        err = float(np.abs(o.float().cpu().numpy() - ro).max())
        print(f"{name}: max-abs err vs oracle {err:.3e}", flush=True)
        assert err <= 2e-2


def test_decode_noalloc_rejects_oversized_partials(lib):
    """B*HQ*splits*(V+2) floats beyond 32 MiB: rejected on the host, nothing
    launched (the pointers are never dereferenced)."""
    fake = 0x10000
    B, T, HQ, H, D = 4096, 65536, 64, 8, 128
    assert lib.wall_attn_decode_workspace_bytes(B, T, HQ, H, D, D, 64) > (32 << 20)
    rc = lib.wall_attn_decode_noalloc(fake, fake, fake, fake, fake, None, None, None, fake, None,
                                      B, T, HQ, H, D, D, 64, 0.0, 0, 1, None, 0, None, 0, 0, 0,
                                      None)
    assert rc == 2
    assert b"static scratch" in lib.wall_attn_last_error()
