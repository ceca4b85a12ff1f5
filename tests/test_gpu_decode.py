"""GPU parity of the decode path against the fp64 oracle (run on an MI355X).

Every test calls the HIP library through its C ABI (via the thin binding):
the running-sum kernel, the cache build in all three cache element types,
the decode over the cache (README "Decode") with and without the serving
options (per-row lengths, window, gate cache, paged cache), and the
streaming append (README "Tests": token by token generation reproduces the
forward).  Bounds:
  * outputs: max-abs 2e-2 for bf16 inputs, 1e-4 for fp32 inputs;
  * lse of a decode: 2e-2 + 2^-19 |lse| (bf16) or 1e-4 + 2^-19 |lse| (fp32):
    the float32 P2 / p_curr the API stores, and the float32 accumulation of
    the dot products, move a score by at most ~2^-20 of the sum of its terms'
    magnitudes; on the 32K-token workload |lse| reaches ~3e5.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_channel_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
CACHE_TYPES = [torch.float32, torch.float16, torch.bfloat16]
CT_IDS = ["kt_f32", "kt_f16", "kt_bf16"]


def dec_lse_tol(dtype, ref):
    return TOL[dtype] + 2.0 ** -19 * np.abs(ref)


@pytest.fixture(scope="module")
def wa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_channel_amd as lib
    lib.load_library()  # raises if the HIP library is missing
    return lib


def check(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err), err.shape)
    tol_a = np.broadcast_to(np.asarray(tol, dtype=np.float64), err.shape)
    print(f"{what}: max-abs err {err.max():.3e} at {i} (tol {tol_a[i]:.3g})", flush=True)
    assert np.isfinite(got).all(), what
    bad = err > tol_a
    assert not bad.any(), (f"{what}: {bad.sum()} elements over tolerance; max-abs error "
                           f"{err.max():.3e} at {i}")
    return float(err.max())


def npy(t):
    return t.float().cpu().numpy().astype(np.float64)


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def small(B=3, T=300, HQ=8, H=2, K=128, V=128, dtype=torch.bfloat16, seed=31, sink=True, gs=0.0):
    c = W.Prefill("dec", B, T, HQ, H, K, V, dtype, sink=sink, seed=seed, g_scalar_std=gs)
    return W.make_prefill(c)


# ----------------------------------------------------------------------------- prefix and cache

def test_prefix_log2_matches_oracle(wa):
    """The running sums are accumulated in double: every P2 / G2 is within one
    float32 ulp of the exact value."""
    x = small(T=333, gs=0.02)
    P2, G2 = wa.wall_attn_prefix_log2(x["g"].to(DEV), g_scalar=x["g_scalar"].to(DEV))
    ref = oracle.prefix_log2(x["g"])
    check(npy(P2), ref, 2.0 ** -23 * np.abs(ref) + 1e-12, "prefix_log2")
    gref = oracle.prefix_log2(x["g_scalar"][..., None])[..., 0]
    check(npy(G2), gref, 2.0 ** -23 * np.abs(gref) + 1e-12, "prefix_log2 gate")
    c = W.Prefill("dec_varlen", 1, 0, 4, 2, 64, 64, torch.bfloat16, nseq=5, len_lo=1, len_hi=200,
                  seed=32, g_scalar_std=0.02)
    y = W.make_prefill(c)
    P2, G2 = wa.wall_attn_prefix_log2(y["g"].to(DEV), cu_seqlens=y["cu_seqlens"].to(DEV),
                                      g_scalar=y["g_scalar"].to(DEV))
    ref = oracle.prefix_log2(y["g"], cu_seqlens=y["cu_seqlens"])
    check(npy(P2), ref, 2.0 ** -23 * np.abs(ref) + 1e-12, "prefix_log2 varlen")
    gref = oracle.prefix_log2(y["g_scalar"][..., None], cu_seqlens=y["cu_seqlens"])[..., 0]
    check(npy(G2), gref, 2.0 ** -23 * np.abs(gref) + 1e-12, "prefix_log2 varlen gate")


REL = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -24}


@pytest.mark.parametrize("ct", CACHE_TYPES, ids=CT_IDS)
@pytest.mark.parametrize("B,T", [(3, 300), (32, 1100)], ids=["chunk_order", "pair_order"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_build_cache_matches_oracle(wa, dtype, B, T, ct):
    # 32 x 18 chunks x 8 heads exceed the workgroups the GPU holds at once:
    # the cache build then runs its (key/value head, chunk) pair order
    x = small(B=B, T=T, dtype=dtype)
    P2 = torch.from_numpy(oracle.prefix_log2(x["g"]).astype(np.float32))
    kt, rc = wa.build_wall_kv_cache(x["k"].to(DEV), P2.to(DEV), chunk_size=64, cache_dtype=ct)
    rkt, rrc = oracle.build_kv_cache(x["k"], P2, chunk_size=64)
    assert np.array_equal(npy(rc), rrc), "anchors must copy P2"
    assert kt.dtype == ct
    # round-to-nearest of a float32 product whose exp2 and multiply add ~2^-22
    rel = REL[ct] + 2.0 ** -21
    # half subnormals (below 2^-14) round to a multiple of 2^-24
    absol = 2.0 ** -25 if ct == torch.float16 else 1e-30
    got = npy(kt)
    assert np.all(np.abs(got - rkt) <= rel * np.abs(rkt) + absol)


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("ct", CACHE_TYPES, ids=CT_IDS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_over_oracle_cache(wa, dtype, ct):
    """Kernel parity: the GPU decode and the oracle decode read the same cache
    (built and rounded on the CPU)."""
    x = small(T=300, dtype=dtype, B=2, HQ=8, H=2, K=64, V=128)
    P2 = oracle.prefix_log2(x["g"]).astype(np.float32)
    rkt, rrc = oracle.build_kv_cache(x["k"], P2, chunk_size=64)
    kt = torch.from_numpy(rkt).to(ct)
    rc = torch.from_numpy(rrc.astype(np.float32))
    pc = torch.from_numpy(P2[:, -1:].copy())
    q = x["q"][:, -1:].contiguous()
    o, lse = wa.wall_attn_decode(q.to(DEV), x["v"].to(DEV), pc.to(DEV), kt.to(DEV), rc.to(DEV),
                                 sink_bias=x["sink_bias"].to(DEV), scale=x["scale"])
    ro, rl = oracle.decode(q, x["v"], pc, kt, rc, sink_bias=x["sink_bias"], scale=x["scale"],
                           return_lse=True)
    check(npy(o), ro, TOL[dtype], f"decode over oracle cache ({ct})")
    check(lse.cpu().numpy(), rl, dec_lse_tol(dtype, rl), "decode lse")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 4096])
def test_decode_pipeline_equals_forward_last_row(wa, T):
    x = small(T=T, B=2)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64)
    o, lse = wa.wall_attn_decode(d["q"][:, -1:].contiguous(), d["v"], P[:, -1:].contiguous(), kt,
                                 rc, sink_bias=d["sink_bias"], scale=d["scale"])
    torch.cuda.synchronize()
    rows = [b * T + T - 1 for b in range(x["q"].shape[0])]
    ro, rl = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"],
                              sink_bias=x["sink_bias"], rows=rows, return_lse=True)
    check(npy(o[:, 0]), ro, 2e-2, f"decode T={T} vs oracle forward")
    check(lse[:, 0].cpu().numpy(), rl, dec_lse_tol(torch.bfloat16, rl), f"decode lse T={T}")
    # and the GPU prefill's last row
    of = wa.wall_attn(d["q"], d["k"], d["v"], d["g"], scale=d["scale"], sink_bias=d["sink_bias"])
    check(npy(o[:, 0]), npy(of[:, -1]), 2e-2, f"decode T={T} vs GPU prefill")


@pytest.mark.parametrize("ct", [torch.float32, torch.float16], ids=["kt_f32", "kt_f16"])
@pytest.mark.parametrize("B,T", [(4, 4096), (2, 2048)])
def test_decode_pipeline_full_heads_equals_forward(wa, B, T, ct):
    """The 32K decode workload's head layout (HQ=32, H=8, D=128): GPU prefix ->
    cache -> decode against the oracle forward's last row."""
    c = W.Prefill("dec_full_heads", B, T, 32, 8, 128, 128, torch.bfloat16, seed=40 + T)
    x = W.make_prefill(c)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64, cache_dtype=ct)
    o, lse = wa.wall_attn_decode(d["q"][:, -1:].contiguous(), d["v"], P[:, -1:].contiguous(), kt,
                                 rc, scale=d["scale"])
    torch.cuda.synchronize()
    rows = [b * T + T - 1 for b in range(B)]
    ro, rl = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"], rows=rows,
                              return_lse=True)
    check(npy(o[:, 0]), ro, 2e-2, f"decode heads32 T={T} {ct}")
    check(lse[:, 0].cpu().numpy(), rl, dec_lse_tol(torch.bfloat16, rl), f"decode heads32 lse T={T}")


# ----------------------------------------------------------------------------- 32K workload

E2E_ROWS = (0, 9, 18, 27, 41, 50, 59, 63)


def _record(lines):
    """Append result lines to gpurun_out/decode32k_parity.txt when that folder exists."""
    if os.path.isdir("gpurun_out"):
        with open(os.path.join("gpurun_out", "decode32k_parity.txt"), "a") as f:
            f.write("\n".join(lines) + "\n")


def test_config_decode_32k(wa):
    """The decode workload (B=64, T_kv=32768, HQ=32, H=8, D=128, C=64) in the
    benchmark's launch configuration, with the default float32 cache:
      * end to end (GPU running sum -> GPU cache -> GPU decode) against the
        oracle forward's last row, on 8 batch rows, at 2e-2 (README "Tests":
        decode reproduces the forward);
      * kernel parity: the oracle decoding the GPU's own cache (copied back)
        on the same rows;
      * two launches give identical bits.
    The half cache is built and decoded as well: its kernel parity (oracle over
    the same half cache) is asserted and its end-to-end error recorded (16-bit
    caches miss 2e-2 on this workload; the CPU conditioning test pins why)."""
    c = W.DECODE_T32768_BF16
    print("[decode32k] drawing inputs", flush=True)
    x = W.make_decode(c, device=DEV)
    P = wa.wall_attn_prefix_log2(x["g"])
    pc = P[:, -1:].contiguous()
    kt, rc = wa.build_wall_kv_cache(x["k"], P, chunk_size=c.C)
    kh, rch = wa.build_wall_kv_cache(x["k"], P, chunk_size=c.C, cache_dtype=torch.float16)
    del P
    torch.cuda.empty_cache()
    o, lse = wa.wall_attn_decode(x["q"], x["v"], pc, kt, rc, scale=x["scale"], cache_chunk_size=c.C)
    o2, lse2 = wa.wall_attn_decode(x["q"], x["v"], pc, kt, rc, scale=x["scale"], cache_chunk_size=c.C)
    oh, lseh = wa.wall_attn_decode(x["q"], x["v"], pc, kh, rch, scale=x["scale"], cache_chunk_size=c.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "decode is not deterministic"
    lines = []
    for b in E2E_ROWS:
        r = W.decode_row(c, b)
        assert torch.equal(r["q"].to(DEV), x["q"][b:b + 1]), "inputs differ from the row draw"
        q = torch.zeros(1, c.T_kv, c.HQ, c.K)
        q[0, -1] = r["q"][0, 0].float()
        fo, fl = oracle.wall_attn(q, r["k"], r["v"], r["g"], scale=x["scale"], rows=[c.T_kv - 1],
                                  return_lse=True)
        e = check(npy(o[b]), fo, 2e-2, f"decode32k f32 cache end to end b={b}")
        el = check(lse[b].cpu().numpy(), fl, dec_lse_tol(c.dtype, fl), f"decode32k f32 lse b={b}")
        od, ld = oracle.decode(r["q"], r["v"], pc[b:b + 1].cpu(), kt[b:b + 1].cpu(),
                               rc[b:b + 1].cpu(), scale=x["scale"], cache_chunk_size=c.C,
                               return_lse=True)
        ek = check(npy(o[b:b + 1]), od, 2e-2, f"decode32k f32 kernel b={b}")
        check(lse[b:b + 1].cpu().numpy(), ld, dec_lse_tol(c.dtype, ld), f"decode32k f32 kernel lse b={b}")
        eh = float(np.abs(npy(oh[b]) - fo).max())
        line = (f"b={b:2d} float32 cache: end-to-end {e:.3e} (lse {el:.3e}), kernel {ek:.3e}; "
                f"float16 cache: end-to-end {eh:.3e}")
        if b in (0, 41, 63):
            odh, ldh = oracle.decode(r["q"], r["v"], pc[b:b + 1].cpu(), kh[b:b + 1].cpu(),
                                     rch[b:b + 1].cpu(), scale=x["scale"], cache_chunk_size=c.C,
                                     return_lse=True)
            ekh = check(npy(oh[b:b + 1]), odh, 2e-2, f"decode32k f16 kernel b={b}")
            check(lseh[b:b + 1].cpu().numpy(), ldh, dec_lse_tol(c.dtype, ldh),
                  f"decode32k f16 kernel lse b={b}")
            line += f", kernel {ekh:.3e}"
        print(line, flush=True)
        lines.append(line)
        del r, od, ld
    _record(lines)


# ----------------------------------------------------------------------------- serving options

def _pages(x_contig, table, page_size, num_pages):
    """Scatter contiguous per-row caches [B, T, ...] into a page pool."""
    B, T = x_contig.shape[:2]
    pool = torch.zeros((num_pages, page_size) + tuple(x_contig.shape[2:]), dtype=x_contig.dtype,
                       device=x_contig.device)
    for b in range(B):
        for lp in range(table.shape[1]):
            t0 = lp * page_size
            if t0 >= T:
                break
            n = min(page_size, T - t0)
            pool[table[b, lp], :n] = x_contig[b, t0:t0 + n]
    return pool


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("ct", [torch.float32, torch.bfloat16], ids=["kt_f32", "kt_bf16"])
def test_decode_lengths_window_gate_paged(wa, ct, window):
    """Ragged per-row lengths, a window and the gate cache, with the cache
    contiguous and paged (pages of 128 tokens in a shuffled pool): the two
    layouts give identical bits; both match the oracle decoding the same cache
    and the oracle forward's row len_b - 1 with the same window and gate."""
    B, T, HQ, H, K, V, PS = 3, 384, 8, 2, 128, 64, 128
    x = small(B=B, T=T, HQ=HQ, H=H, K=K, V=V, seed=50, gs=0.02)
    d = to_dev(x)
    lens = [300, 1, 129]
    P, G = wa.wall_attn_prefix_log2(d["g"], g_scalar=d["g_scalar"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64, cache_dtype=ct)
    seql = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qi = torch.stack([d["q"][b, L - 1] for b, L in enumerate(lens)])[:, None].contiguous()
    pi = torch.stack([P[b, L - 1] for b, L in enumerate(lens)])[:, None].contiguous()
    gi = torch.stack([G[b, L - 1] for b, L in enumerate(lens)])[:, None].contiguous()
    W_ = window if window > 0 else None
    o, lse = wa.wall_attn_decode(qi, d["v"], pi, kt, rc, sink_bias=d["sink_bias"], scale=x["scale"],
                                 cache_seqlens=seql, window_size=W_, gate_cache=G, gate_curr=gi)
    gen = torch.Generator().manual_seed(51)
    npages = 12
    table = torch.randperm(npages, generator=gen)[:B * 3].reshape(B, 3).to(torch.int32)
    ktp = _pages(kt, table, PS, npages)
    vp = _pages(d["v"], table, PS, npages)
    gp = _pages(G, table, PS, npages)
    rcp = _pages(rc, table, PS // 64, npages)
    op, lsep = wa.wall_attn_decode(qi, vp, pi, ktp, rcp, sink_bias=d["sink_bias"], scale=x["scale"],
                                   cache_seqlens=seql, window_size=W_, gate_cache=gp, gate_curr=gi,
                                   block_table=table.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o, op) and torch.equal(lse, lsep), "paged and contiguous layouts differ"
    # kernel parity over the same cache
    od, ld = oracle.decode_ext(qi.cpu(), x["v"], pi.cpu(), kt.cpu(), rc.cpu(),
                               sink_bias=x["sink_bias"], scale=x["scale"], gate_cache=G.cpu(),
                               gate_curr=gi.cpu(), cache_seqlens=np.array(lens, np.int32),
                               window_size=W_, return_lse=True)
    check(npy(o), od, 2e-2, f"decode options kernel ({ct}, W={window})")
    check(lse.cpu().numpy(), ld, dec_lse_tol(torch.bfloat16, ld), "decode options kernel lse")
    # end to end: the oracle forward over each row's first len_b tokens
    for b, L in enumerate(lens):
        fo, fl = oracle.wall_attn(x["q"][b:b + 1, :L], x["k"][b:b + 1, :L], x["v"][b:b + 1, :L],
                                  x["g"][b:b + 1, :L], scale=x["scale"],
                                  g_scalar=x["g_scalar"][b:b + 1, :L], sink_bias=x["sink_bias"],
                                  window_size=W_, rows=[L - 1], return_lse=True)
        if ct == torch.float32:
            check(npy(o[b]), fo, 2e-2, f"decode options end to end b={b}")
            check(lse[b].cpu().numpy(), fl, dec_lse_tol(torch.bfloat16, fl), f"lse b={b}")


def test_decode_empty_row(wa):
    """A row with no cached token: o = 0, lse = the sink logit."""
    x = small(B=2, T=128, HQ=4, H=2, K=64, V=64, seed=52)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    kt, rc = wa.build_wall_kv_cache(d["k"], P, chunk_size=64)
    seql = torch.tensor([0, 128], dtype=torch.int32, device=DEV)
    o, lse = wa.wall_attn_decode(d["q"][:, -1:].contiguous(), d["v"], P[:, -1:].contiguous(), kt,
                                 rc, sink_bias=d["sink_bias"], scale=x["scale"], cache_seqlens=seql)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o[0]) == 0
    # lse = sink * log2(e) * ln 2 through the kernels' log2 units
    np.testing.assert_allclose(lse[0, 0].cpu().numpy(), x["sink_bias"].numpy(), rtol=1e-6, atol=1e-6)
    ro = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"],
                          sink_bias=x["sink_bias"], rows=[2 * 128 - 1])
    check(npy(o[1]), ro[0], 2e-2, "decode next to an empty row")


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("ct", [torch.float32, torch.float16], ids=["kt_f32", "kt_f16"])
def test_decode_streaming_append(wa, ct, paged):
    """The serving loop (README "Decode" and "Tests"): row 1 starts from a
    37-token prompt built with the cache build, row 0 from an empty cache; at
    every step each row appends its next token (wall_attn_cache_append) and
    decodes it.  Every step reproduces the oracle forward's row; the anchors
    the append leaves are integers within half a unit of P2 at each chunk's
    newest token, and k_tilde * 2^(P2 - anchor) gives back k."""
    B, T, HQ, H, K, V = 2, 200, 4, 2, 64, 64
    x = small(B=B, T=T, HQ=HQ, H=H, K=K, V=V, seed=33)
    d = to_dev(x)
    P = wa.wall_attn_prefix_log2(d["g"])
    cap, PS = 256, 128
    start = [0, 37]
    steps = 150
    kt = torch.zeros(B, cap, HQ, K, dtype=ct, device=DEV)
    vc = torch.zeros(B, cap, H, V, dtype=x["v"].dtype, device=DEV)
    rc = torch.zeros(B, cap // 64, HQ, K, dtype=torch.float32, device=DEV)
    kt1, rc1 = wa.build_wall_kv_cache(d["k"][1:2, :37].contiguous(), P[1:2, :37].contiguous(),
                                      cache_dtype=ct)
    kt[1, :37] = kt1[0]
    rc[1, :1] = rc1[0]
    vc[1, :37] = d["v"][1, :37]
    seql = torch.tensor(start, dtype=torch.int32, device=DEV)
    table = None
    if paged:
        table = torch.tensor([[3, 0], [1, 2]], dtype=torch.int32, device=DEV)
        kt, vc, rc = (_pages(kt, table.cpu(), PS, 4), _pages(vc, table.cpu(), PS, 4),
                      _pages(rc, table.cpu(), PS // 64, 4))
    outs = []
    for t in range(steps):
        pos = [start[0] + t, start[1] + t]
        sel = lambda a: torch.stack([a[b, p] for b, p in enumerate(pos)])[:, None].contiguous()
        p_new = sel(P)
        wa.wall_attn_cache_append(sel(d["k"]), sel(d["v"]), p_new, kt, vc, rc, seql,
                                  block_table=table)
        o, _ = wa.wall_attn_decode(sel(d["q"]), vc, p_new, kt, rc, sink_bias=d["sink_bias"],
                                   scale=x["scale"], cache_seqlens=seql, block_table=table)
        outs.append(o[:, 0].clone())
    torch.cuda.synchronize()
    assert seql.cpu().tolist() == [start[0] + steps, start[1] + steps]
    got = torch.stack(outs, 1).float().cpu().numpy()  # [B, steps, HQ, V]
    rows = [b * T + start[b] + t for b in range(B) for t in range(steps)]
    ro = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], scale=x["scale"],
                          sink_bias=x["sink_bias"], rows=rows)
    check(got.reshape(B * steps, HQ, V), ro, 2e-2, f"streaming append ({ct}, paged={paged})")
    if paged:
        return
    # the cache the appends left: integer anchors at each chunk's newest token
    P2 = oracle.prefix_log2(x["g"])
    rcn = npy(rc)
    ktn = npy(kt)
    for b in range(B):
        L = start[b] + steps
        for cix in range((L + 63) // 64):
            last = min(64 * cix + 64, L) - 1
            assert np.array_equal(rcn[b, cix], np.rint(rcn[b, cix])), "anchors must be integers"
            assert np.abs(rcn[b, cix] - P2[b, last]).max() <= 0.5 + 1e-6
            rows_c = np.arange(64 * cix, last + 1)
            back = ktn[b, rows_c] * np.exp2(P2[b, rows_c] - rcn[b, cix][None])
            kr = np.repeat(x["k"][b, rows_c].float().numpy().astype(np.float64), HQ // H, axis=1)
            assert np.all(np.abs(back - kr) <= (REL[ct] + 2.0 ** -20) * 2 * np.abs(kr) + 1e-6)
