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
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["wall_attn", "wall_attn_prefix_log2", "build_wall_kv_cache", "wall_attn_decode",
           "cache_dtype", "library_path", "load_library", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwallattn.so")
_lib = None

WA_BF16, WA_F32 = 0, 1
_STATUS = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "HIP_ERROR", 4: "WORKSPACE_TOO_SMALL"}

EXPORTED_SYMBOLS = (
    "wall_attn_last_error", "wall_attn_fwd_workspace_bytes", "wall_attn_fwd",
    "wall_attn_fwd_prepare", "wall_attn_fwd_attend",
    "wall_attn_prefix_log2_workspace_bytes", "wall_attn_prefix_log2",
    "wall_attn_build_kv_cache", "wall_attn_decode_workspace_bytes", "wall_attn_decode",
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
    lib.wall_attn_prefix_log2.argtypes = [P, P, I, I, I, I, P, I, I, S, P, Z, P]
    lib.wall_attn_build_kv_cache.restype = S
    lib.wall_attn_build_kv_cache.argtypes = [P, P, P, P, I, I, I, I, I, I, S, P]
    lib.wall_attn_decode_workspace_bytes.restype = Z
    lib.wall_attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.wall_attn_decode.restype = S
    lib.wall_attn_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, S, P, Z, P]
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


def wall_attn(q, k, v, g, scale=None, g_scalar=None, sink_bias=None, window_size=None,
              cu_seqlens=None, max_seqlen=None, return_lse=False, workspace=None):
    """Exact causal Wall Attention forward (README "Usage"): o [B,T,HQ,V].

    ``cu_seqlens`` (int32, B == 1) packs sequences; ``max_seqlen`` avoids a
    device-to-host read of it.  ``workspace`` optionally supplies a uint8
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
    nseq = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        nseq = cu_seqlens.shape[0] - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
    else:
        max_seqlen = 0
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


def fwd_workspace_bytes(B, T, HQ, H, K, V, num_seqs=0, max_seqlen=0, dtype=torch.bfloat16):
    code = WA_BF16 if dtype == torch.bfloat16 else WA_F32
    return int(load_library().wall_attn_fwd_workspace_bytes(B, T, HQ, H, K, V, num_seqs,
                                                             max_seqlen, code))


def wall_attn_prefix_log2(g, cu_seqlens=None, max_seqlen=None):
    """P2 = cumsum(g) / ln 2 along time, per sequence (README "Decode"); float32."""
    lib = load_library()
    dev = _dev(g, cu_seqlens)
    code = _dtype_code(g)
    B, T, HQ, K = g.shape
    nseq = 0
    if cu_seqlens is not None:
        nseq = cu_seqlens.shape[0] - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
    else:
        max_seqlen = 0
    P2 = torch.empty(B, T, HQ, K, dtype=torch.float32, device=dev)
    need = lib.wall_attn_prefix_log2_workspace_bytes(B, T, HQ, K, nseq, max_seqlen)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rc = lib.wall_attn_prefix_log2(_ptr(g), _ptr(P2), B, T, HQ, K, _ptr(cu_seqlens), nseq,
                                   max_seqlen, code, _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "wall_attn_prefix_log2")
    return P2


def cache_dtype(dtype):
    """Element type of k_tilde for inputs of ``dtype``: float16 for bfloat16
    inputs (same bytes, 3 more mantissa bits), float32 for float32."""
    return torch.float16 if dtype == torch.bfloat16 else torch.float32


def build_wall_kv_cache(k, P, chunk_size=64):
    """(k_tilde [B,T,HQ,K], r_cache [B,ceil(T/C),HQ,K]) from k and P (README "Decode").

    k_tilde has ``cache_dtype(k.dtype)``; r_cache is float32."""
    lib = load_library()
    dev = _dev(k, P)
    code = _dtype_code(k)
    _f32(P)
    B, T, H, K = k.shape
    HQ = P.shape[2]
    if tuple(P.shape) != (B, T, HQ, K):
        raise ValueError("P must be [B,T,HQ,K]")
    nc = -(-T // chunk_size)
    kt = torch.empty(B, T, HQ, K, dtype=cache_dtype(k.dtype), device=dev)
    rc_ = torch.empty(B, nc, HQ, K, dtype=torch.float32, device=dev)
    rc = lib.wall_attn_build_kv_cache(_ptr(k), _ptr(P), _ptr(kt), _ptr(rc_), B, T, HQ, H, K,
                                      chunk_size, code, _stream(dev))
    _check(rc, "build_wall_kv_cache")
    return kt, rc_


def wall_attn_decode(q, v, p_curr, k_tilde, r_cache, sink_bias=None, scale=None,
                     cache_chunk_size=64, workspace=None, out=None, lse_out=None):
    """One decode step over the cache (README "Decode"): (o [B,1,HQ,V], lse [B,1,HQ])."""
    lib = load_library()
    dev = _dev(q, v, p_curr, k_tilde, r_cache, sink_bias, workspace, out, lse_out)
    code = _dtype_code(q)
    _same_dtype(q, v)
    if k_tilde.dtype != cache_dtype(q.dtype):
        raise ValueError(f"k_tilde must be {cache_dtype(q.dtype)} for {q.dtype} inputs")
    _f32(p_curr, r_cache, sink_bias)
    B, _, HQ, K = q.shape
    T, H, V = v.shape[1], v.shape[2], v.shape[3]
    if tuple(q.shape) != (B, 1, HQ, K) or tuple(p_curr.shape) != (B, 1, HQ, K):
        raise ValueError("q and p_curr must be [B,1,HQ,K]")
    if tuple(k_tilde.shape) != (B, T, HQ, K):
        raise ValueError("k_tilde must be [B,T_kv,HQ,K]")
    nc = -(-T // cache_chunk_size)
    if tuple(r_cache.shape) != (B, nc, HQ, K):
        raise ValueError("r_cache must be [B,ceil(T_kv/C),HQ,K]")
    o = out if out is not None else torch.empty(B, 1, HQ, V, dtype=q.dtype, device=dev)
    lse = lse_out if lse_out is not None else torch.empty(B, 1, HQ, dtype=torch.float32, device=dev)
    need = lib.wall_attn_decode_workspace_bytes(B, T, HQ, H, K, V, cache_chunk_size)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    s = 0.0 if scale is None else float(scale)
    rc = lib.wall_attn_decode(_ptr(q), _ptr(v), _ptr(p_curr), _ptr(k_tilde), _ptr(r_cache),
                              _ptr(sink_bias), _ptr(o), _ptr(lse), B, T, HQ, H, K, V,
                              cache_chunk_size, s, code, _ptr(workspace), workspace.numel(),
                              _stream(dev))
    _check(rc, "wall_attn_decode")
    return o, lse


def decode_workspace_bytes(B, T, HQ, H, K, V, chunk_size=64):
    return int(load_library().wall_attn_decode_workspace_bytes(B, T, HQ, H, K, V, chunk_size))
