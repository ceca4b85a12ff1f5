"""Python binding of libwallattn: exact causal Wall Attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libwallattn.so`` (built in-tree by
``python -m exact_attention_channel_amd.build``).  There is no CPU or PyTorch
fallback: if the library is missing, every call raises.

The call shapes follow the Wall Attention README ("Usage" and "Decode"):

    o = wall_attn(q, k, v, g, scale=K**-0.5, g_scalar=None, sink_bias=None,
                  window_size=None, cu_seqlens=None)
    P = wall_attn_prefix_log2(g)                    # cumsum(g) / ln 2
    k_tilde, r_cache = build_wall_kv_cache(k, P, chunk_size=64)
    o, lse = wall_attn_decode(q[:, -1:], v, P[:, -1:], k_tilde, r_cache,
                              sink_bias=None, scale=K**-0.5, cache_chunk_size=64)

Serving extensions (same kernels): ``wall_attn_decode(..., cache_seqlens=,
window_size=, gate_cache=, gate_curr=, block_table=)`` and
``wall_attn_cache_append`` for the token-by-token loop.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["wall_attn", "wall_attn_bwd", "wall_attn_prefix_log2", "build_wall_kv_cache", "wall_attn_decode",
           "wall_attn_cache_append", "cache_dtype", "library_path", "load_library",
           "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwallattn.so")
_lib = None

WA_BF16, WA_F32, WA_F16 = 0, 1, 2
_STATUS = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "HIP_ERROR", 4: "WORKSPACE_TOO_SMALL"}

EXPORTED_SYMBOLS = (
    "wall_attn_last_error", "wall_attn_fwd_workspace_bytes", "wall_attn_fwd",
    "wall_attn_fwd_prepare", "wall_attn_fwd_attend",
    "wall_attn_prefix_log2_workspace_bytes", "wall_attn_prefix_log2",
    "wall_attn_build_kv_cache", "wall_attn_decode_workspace_bytes", "wall_attn_decode",
    "wall_attn_decode_ext", "wall_attn_cache_append", "wall_attn_decode_noalloc",
    "wall_attn_bwd_workspace_bytes", "wall_attn_bwd",
)


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libwallattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_attention_channel_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, Z, F, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_int
    lib.wall_attn_last_error.restype = ctypes.c_char_p
    lib.wall_attn_last_error.argtypes = []
    lib.wall_attn_fwd_workspace_bytes.restype = Z
    lib.wall_attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, S]
    lib.wall_attn_fwd.restype = S
    lib.wall_attn_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, I, I, I, F, S, P, Z, P]
    lib.wall_attn_fwd_prepare.restype = S
    lib.wall_attn_fwd_prepare.argtypes = [P, P, P, P, I, I, I, I, I, I, P, I, I, F, S, P, Z, P]
    lib.wall_attn_fwd_attend.restype = S
    lib.wall_attn_fwd_attend.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, I, I, I, F, S, P, Z, P]
    lib.wall_attn_prefix_log2_workspace_bytes.restype = Z
    lib.wall_attn_prefix_log2_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.wall_attn_prefix_log2.restype = S
    lib.wall_attn_prefix_log2.argtypes = [P, P, P, P, I, I, I, I, P, I, I, S, P, Z, P]
    lib.wall_attn_build_kv_cache.restype = S
    lib.wall_attn_build_kv_cache.argtypes = [P, P, P, P, I, I, I, I, I, I, S, S, P]
    lib.wall_attn_decode_workspace_bytes.restype = Z
    lib.wall_attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.wall_attn_decode.restype = S
    lib.wall_attn_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, S, S, P, Z, P]
    lib.wall_attn_decode_ext.restype = S
    lib.wall_attn_decode_ext.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, S,
                                         S, P, I, P, I, I, I, P, Z, P]
    lib.wall_attn_decode_noalloc.restype = S
    lib.wall_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F,
                                             S, S, P, I, P, I, I, I, P]
    lib.wall_attn_bwd_workspace_bytes.restype = Z
    lib.wall_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, S]
    lib.wall_attn_bwd.restype = S
    lib.wall_attn_bwd.argtypes = [P] * 15 + [I] * 6 + [P, I, I, I, F, S, P, Z, P]
    lib.wall_attn_cache_append.restype = S
    lib.wall_attn_cache_append.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, S, S,
                                           P, I, I, I, P]
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().wall_attn_last_error().decode()
        err = RuntimeError if rc == 3 else ValueError
        raise err(f"{what}: {_STATUS.get(rc, rc)}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WA_BF16
    if t.dtype == torch.float32:
        return WA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("all tensors must be torch tensors on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _same_dtype(ref, *ts):
    for t in ts:
        if t is not None and t.dtype != ref.dtype:
            raise ValueError(f"expected {ref.dtype}, got {t.dtype}")


def _f32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise ValueError("sink_bias, P / p_curr and r_cache must be float32")


def _varlen(cu_seqlens, max_seqlen, check=True):
    """(num_seqs, max_seqlen) for the C ABI.  Without max_seqlen it is read
    back from cu_seqlens; a given one is checked against cu_seqlens (one small
    device-to-host read) unless ``check`` is False, in which case an
    understated max_seqlen leaves the rows past it unwritten (the library
    never reads or writes outside its workspace for it)."""
    if cu_seqlens is None:
        return 0, 0
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    nseq = cu_seqlens.shape[0] - 1
    if max_seqlen is None or check:
        true_max = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        if max_seqlen is not None and int(max_seqlen) < true_max:
            raise ValueError(f"max_seqlen {max_seqlen} is below the longest sequence ({true_max})")
        max_seqlen = true_max if max_seqlen is None else max_seqlen
    return nseq, int(max_seqlen)


def wall_attn(q, k, v, g, scale=None, g_scalar=None, sink_bias=None, window_size=None,
              cu_seqlens=None, max_seqlen=None, return_lse=False, workspace=None,
              check_max_seqlen=True):
    """Exact causal Wall Attention forward (README "Usage"): o [B,T,HQ,V].

    ``cu_seqlens`` (int32, B == 1) packs sequences; ``max_seqlen`` with
    ``check_max_seqlen=False`` avoids a device-to-host read of it.  ``workspace`` optionally supplies a uint8
    device buffer of at least ``fwd_workspace_bytes(...)`` bytes.
    """
    lib = load_library()
    dev = _dev(q, k, v, g, g_scalar, sink_bias, cu_seqlens, workspace)
    code = _dtype_code(q)
    _same_dtype(q, k, v, g, g_scalar)
    _f32(sink_bias)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, T, H, K) or tuple(v.shape) != (B, T, H, V) or tuple(g.shape) != (B, T, HQ, K):
        raise ValueError("shapes must be q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K]")
    if g_scalar is not None and tuple(g_scalar.shape) != (B, T, HQ):
        raise ValueError("g_scalar must be [B,T,HQ]")
    if sink_bias is not None and tuple(sink_bias.shape) != (HQ,):
        raise ValueError("sink_bias must be [HQ]")
    nseq, max_seqlen = _varlen(cu_seqlens, max_seqlen, check_max_seqlen)
    o = torch.empty(B, T, HQ, V, dtype=q.dtype, device=dev)
    lse = torch.empty(B, T, HQ, dtype=torch.float32, device=dev) if return_lse else None
    need = lib.wall_attn_fwd_workspace_bytes(B, T, HQ, H, K, V, nseq, max_seqlen, code)
    if need == 0:
        _check(lib.wall_attn_fwd(None, None, None, None, None, None, None, None, B, T, HQ, H, K, V,
                                 _ptr(cu_seqlens), nseq, max_seqlen, 0, 0.0, code, None, 0, None),
               "wall_attn")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    W = 0 if window_size is None else int(window_size)
    s = 0.0 if scale is None else float(scale)
    rc = lib.wall_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_scalar), _ptr(sink_bias),
                           _ptr(o), _ptr(lse), B, T, HQ, H, K, V, _ptr(cu_seqlens), nseq,
                           max_seqlen, W, s, code, _ptr(workspace), workspace.numel(),
                           _stream(dev))
    _check(rc, "wall_attn")
    return (o, lse) if return_lse else o


def wall_attn_bwd(q, k, v, g, o, lse, dO, scale=None, g_scalar=None, sink_bias=None,
                  window_size=None, cu_seqlens=None, max_seqlen=None, check_max_seqlen=True):
    """Gradients of wall_attn for dL/do = dO (README introduction: analytic
    gradients for q, k, v, g and the gate), from the forward's output o and
    its lse (``wall_attn(..., return_lse=True)``).

    Returns (dq, dk, dv, dg, dg_scalar, dsink): dg_scalar is None without
    g_scalar, dsink (float32 [HQ]) None without sink_bias."""
    lib = load_library()
    dev = _dev(q, k, v, g, o, lse, dO, g_scalar, sink_bias, cu_seqlens)
    code = _dtype_code(q)
    _same_dtype(q, k, v, g, o, dO, g_scalar)
    _f32(sink_bias, lse)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if (tuple(k.shape) != (B, T, H, K) or tuple(v.shape) != (B, T, H, V)
            or tuple(g.shape) != (B, T, HQ, K) or tuple(o.shape) != (B, T, HQ, V)
            or tuple(dO.shape) != (B, T, HQ, V) or tuple(lse.shape) != (B, T, HQ)):
        raise ValueError("shapes must be q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K], "
                         "o and dO [B,T,HQ,V], lse [B,T,HQ]")
    nseq, max_seqlen = _varlen(cu_seqlens, max_seqlen, check_max_seqlen)
    dq, dg = torch.empty_like(q), torch.empty_like(g)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    dgs = None if g_scalar is None else torch.empty_like(g_scalar)
    dsink = None if sink_bias is None else torch.empty_like(sink_bias)
    need = lib.wall_attn_bwd_workspace_bytes(B, T, HQ, H, K, V, nseq, max_seqlen, code)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    W = 0 if window_size is None else int(window_size)
    s = 0.0 if scale is None else float(scale)
    rc = lib.wall_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_scalar), _ptr(sink_bias),
                           _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                           _ptr(dgs), _ptr(dsink), B, T, HQ, H, K, V, _ptr(cu_seqlens), nseq,
                           max_seqlen, W, s, code, _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "wall_attn_bwd")
    return dq, dk, dv, dg, dgs, dsink


def fwd_workspace_bytes(B, T, HQ, H, K, V, num_seqs=0, max_seqlen=0, dtype=torch.bfloat16):
    code = WA_BF16 if dtype == torch.bfloat16 else WA_F32
    return int(load_library().wall_attn_fwd_workspace_bytes(B, T, HQ, H, K, V, num_seqs,
                                                             max_seqlen, code))


def wall_attn_prefix_log2(g, cu_seqlens=None, max_seqlen=None, g_scalar=None):
    """P2 = cumsum(g) / ln 2 along time, per sequence (README "Decode"); float32.

    With ``g_scalar`` [B,T,HQ] also returns G2 = cumsum(g_scalar) / ln 2 (the
    gate cache of the decode), as ``(P2, G2)``."""
    lib = load_library()
    dev = _dev(g, g_scalar)
    code = _dtype_code(g)
    _same_dtype(g, g_scalar)
    B, T, HQ, K = g.shape
    if g_scalar is not None and tuple(g_scalar.shape) != (B, T, HQ):
        raise ValueError("g_scalar must be [B,T,HQ]")
    nseq, max_seqlen = _varlen(cu_seqlens, max_seqlen)
    P2 = torch.empty(B, T, HQ, K, dtype=torch.float32, device=dev)
    G2 = None if g_scalar is None else torch.empty(B, T, HQ, dtype=torch.float32, device=dev)
    need = lib.wall_attn_prefix_log2_workspace_bytes(B, T, HQ, K, nseq, max_seqlen)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rc = lib.wall_attn_prefix_log2(_ptr(g), _ptr(g_scalar), _ptr(P2), _ptr(G2), B, T, HQ, K,
                                   _ptr(cu_seqlens), nseq, max_seqlen, code, _ptr(ws), ws.numel(),
                                   _stream(dev))
    _check(rc, "wall_attn_prefix_log2")
    return P2 if g_scalar is None else (P2, G2)


_CACHE_CODES = {torch.bfloat16: WA_BF16, torch.float16: WA_F16, torch.float32: WA_F32}


def cache_dtype(dtype=None):
    """Default element type of k_tilde: float32 for every input type (24
    mantissa bits hold the long random-walk decays whose decode scores reach
    ~1e5); bfloat16 (k's own type) and float16 caches are available by
    passing ``cache_dtype=`` to build_wall_kv_cache."""
    return torch.float32


def _cache_code(t):
    if t not in _CACHE_CODES:
        raise ValueError(f"k_tilde dtype {t} not supported (bfloat16, float16, float32)")
    return _CACHE_CODES[t]


def build_wall_kv_cache(k, P, chunk_size=64, cache_dtype=None):
    """(k_tilde [B,T,HQ,K], r_cache [B,ceil(T/C),HQ,K]) from k and P (README "Decode").

    k_tilde has ``cache_dtype`` (default float32); r_cache is float32."""
    lib = load_library()
    dev = _dev(k, P)
    code = _dtype_code(k)
    _f32(P)
    B, T, H, K = k.shape
    HQ = P.shape[2]
    if tuple(P.shape) != (B, T, HQ, K):
        raise ValueError("P must be [B,T,HQ,K]")
    ct = globals()["cache_dtype"]() if cache_dtype is None else cache_dtype
    nc = -(-T // chunk_size)
    kt = torch.empty(B, T, HQ, K, dtype=ct, device=dev)
    rc_ = torch.empty(B, nc, HQ, K, dtype=torch.float32, device=dev)
    rc = lib.wall_attn_build_kv_cache(_ptr(k), _ptr(P), _ptr(kt), _ptr(rc_), B, T, HQ, H, K,
                                      chunk_size, code, _cache_code(ct), _stream(dev))
    _check(rc, "build_wall_kv_cache")
    return kt, rc_


def wall_attn_decode(q, v, p_curr, k_tilde, r_cache, sink_bias=None, scale=None,
                     cache_chunk_size=64, workspace=None, out=None, lse_out=None,
                     cache_seqlens=None, window_size=None, gate_cache=None, gate_curr=None,
                     block_table=None, page_size=None):
    """One decode step over the cache (README "Decode"): (o [B,1,HQ,V], lse [B,1,HQ]).

    Contiguous caches: v [B,T_kv,H,V], k_tilde [B,T_kv,HQ,K], r_cache
    [B,ceil(T_kv/C),HQ,K].  Options: ``cache_seqlens`` int32 [B] (row b holds
    len_b tokens, its query at len_b - 1), ``window_size``, the gate cache
    ``gate_cache`` [B,T_kv,HQ] with ``gate_curr`` [B,1,HQ] (log2-unit running
    sums of g_scalar), and a paged cache: ``block_table`` int32 [B,max_blocks]
    with pools v [P,page_size,H,V], k_tilde [P,page_size,HQ,K], r_cache
    [P,page_size/C,HQ,K], gate_cache [P,page_size,HQ].
    """
    lib = load_library()
    dev = _dev(q, v, p_curr, k_tilde, r_cache, sink_bias, workspace, out, lse_out, cache_seqlens,
               gate_cache, gate_curr, block_table)
    code = _dtype_code(q)
    _same_dtype(q, v)
    ccode = _cache_code(k_tilde.dtype)
    _f32(p_curr, r_cache, sink_bias, gate_cache, gate_curr)
    B, _, HQ, K = q.shape
    H, V = v.shape[2], v.shape[3]
    if tuple(q.shape) != (B, 1, HQ, K) or tuple(p_curr.shape) != (B, 1, HQ, K):
        raise ValueError("q and p_curr must be [B,1,HQ,K]")
    C = cache_chunk_size
    if block_table is None:
        T = v.shape[1]
        if v.shape[0] != B:
            raise ValueError("v must be [B,T_kv,H,V]")
        if tuple(k_tilde.shape) != (B, T, HQ, K):
            raise ValueError("k_tilde must be [B,T_kv,HQ,K]")
        if tuple(r_cache.shape) != (B, -(-T // C), HQ, K):
            raise ValueError("r_cache must be [B,ceil(T_kv/C),HQ,K]")
        if gate_cache is not None and tuple(gate_cache.shape) != (B, T, HQ):
            raise ValueError("gate_cache must be [B,T_kv,HQ]")
        max_blocks = ps = npages = 0
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B,max_blocks]")
        npages, ps = v.shape[0], v.shape[1]
        if page_size is not None and page_size != ps:
            raise ValueError("page_size does not match the pools")
        max_blocks = block_table.shape[1]
        T = max_blocks * ps
        if tuple(k_tilde.shape) != (npages, ps, HQ, K) or ps % C:
            raise ValueError("k_tilde pool must be [num_pages,page_size,HQ,K], page_size % C == 0")
        if tuple(r_cache.shape) != (npages, ps // C, HQ, K):
            raise ValueError("r_cache pool must be [num_pages,page_size/C,HQ,K]")
        if gate_cache is not None and tuple(gate_cache.shape) != (npages, ps, HQ):
            raise ValueError("gate_cache pool must be [num_pages,page_size,HQ]")
    if cache_seqlens is not None and (cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,)):
        raise ValueError("cache_seqlens must be int32 [B]")
    if gate_curr is not None and tuple(gate_curr.shape) != (B, 1, HQ):
        raise ValueError("gate_curr must be [B,1,HQ]")
    o = out if out is not None else torch.empty(B, 1, HQ, V, dtype=q.dtype, device=dev)
    lse = lse_out if lse_out is not None else torch.empty(B, 1, HQ, dtype=torch.float32, device=dev)
    need = lib.wall_attn_decode_workspace_bytes(B, T, HQ, H, K, V, C)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    s = 0.0 if scale is None else float(scale)
    W = 0 if window_size is None else int(window_size)
    rc = lib.wall_attn_decode_ext(_ptr(q), _ptr(v), _ptr(p_curr), _ptr(k_tilde), _ptr(r_cache),
                                  _ptr(sink_bias), _ptr(gate_cache), _ptr(gate_curr), _ptr(o),
                                  _ptr(lse), B, T, HQ, H, K, V, C, s, code, ccode,
                                  _ptr(cache_seqlens), W, _ptr(block_table), max_blocks, ps,
                                  npages, _ptr(workspace), workspace.numel(), _stream(dev))
    _check(rc, "wall_attn_decode")
    return o, lse


def wall_attn_cache_append(k_new, v_new, p_new, k_tilde, v_cache, r_cache, cache_seqlens,
                           gate_new=None, gate_cache=None, block_table=None, cache_chunk_size=64):
    """Append one token per batch row to a decode cache, in place (README
    "Decode": the sequential-append serving loop).  k_new [B,1,H,K], v_new
    [B,1,H,V], p_new [B,1,HQ,K] float32 (P2 at the new token), gate_new
    [B,1,HQ] float32 (G2 at the new token) with gate_cache; caches laid out
    as for wall_attn_decode.  cache_seqlens (int32 [B]) is advanced by one on
    every row that had room."""
    lib = load_library()
    dev = _dev(k_new, v_new, p_new, k_tilde, v_cache, r_cache, cache_seqlens, gate_new,
               gate_cache, block_table)
    code = _dtype_code(k_new)
    _same_dtype(k_new, v_new, v_cache)
    ccode = _cache_code(k_tilde.dtype)
    _f32(p_new, r_cache, gate_new, gate_cache)
    B, _, H, K = k_new.shape
    HQ, V = p_new.shape[2], v_new.shape[3]
    C = cache_chunk_size
    if block_table is None:
        T = v_cache.shape[1]
        if tuple(k_tilde.shape) != (B, T, HQ, K) or tuple(r_cache.shape) != (B, -(-T // C), HQ, K):
            raise ValueError("caches must be k_tilde [B,T,HQ,K], r_cache [B,ceil(T/C),HQ,K]")
        max_blocks = ps = npages = 0
    else:
        npages, ps = v_cache.shape[0], v_cache.shape[1]
        max_blocks = block_table.shape[1]
        T = max_blocks * ps
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be int32 [B]")
    rc = lib.wall_attn_cache_append(_ptr(k_new), _ptr(v_new), _ptr(p_new), _ptr(gate_new),
                                    _ptr(k_tilde), _ptr(v_cache), _ptr(r_cache), _ptr(gate_cache),
                                    _ptr(cache_seqlens), B, T, HQ, H, K, V, C, code, ccode,
                                    _ptr(block_table), max_blocks, ps, npages, _stream(dev))
    _check(rc, "wall_attn_cache_append")


def decode_workspace_bytes(B, T, HQ, H, K, V, chunk_size=64):
    return int(load_library().wall_attn_decode_workspace_bytes(B, T, HQ, H, K, V, chunk_size))
