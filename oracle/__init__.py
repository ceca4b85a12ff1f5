"""fp64 CPU oracle for Wall Attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and has
no fallback to it.  It shares no code with the HIP path: the arithmetic lives
in ``wall_oracle.c`` (plain C, double precision, OpenMP over independent
rows), built here with gcc.

The functions take CPU tensors or arrays holding the exact values of the
inputs (bf16 and fp32 values are exact in float32) and return float64 numpy
arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wall_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile wall_oracle.c into liboracle.so (gcc -O2 -fopenmp, no fast-math)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_wall_attn_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, I, I, D, P, I, P, P]
        lib.oracle_wall_attn_fwd.restype = ctypes.c_int
        lib.oracle_prefix_log2.argtypes = [P, I, I, I, I, P, I, P]
        lib.oracle_prefix_log2.restype = ctypes.c_int
        lib.oracle_build_kv_cache.argtypes = [P, P, I, I, I, I, I, I, P, P]
        lib.oracle_build_kv_cache.restype = ctypes.c_int
        lib.oracle_decode_cache.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P]
        lib.oracle_decode_cache.restype = ctypes.c_int
        lib.oracle_decode_cache_ext.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                                D, P, P]
        lib.oracle_decode_cache_ext.restype = ctypes.c_int
        lib.oracle_wall_attn_bwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, I, I, D,
                                             P, P, P, P, P, P]
        lib.oracle_wall_attn_bwd.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Threads of the oracle's OpenMP loops from now on; returns the count in force."""
    return int(_load().oracle_set_num_threads(int(n)))


def _f32(x):
    """Exact float32 numpy copy of a tensor/array (bf16 and fp32 values are exact)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.int32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def wall_attn(q, k, v, g, scale=None, g_scalar=None, sink_bias=None, window_size=None,
              cu_seqlens=None, rows=None, return_lse=False):
    """Exact Wall Attention forward (Wall Attention README, "Usage").

    Shapes follow the README: q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V],
    g [B,T,HQ,K], g_scalar [B,T,HQ], sink_bias [HQ], cu_seqlens [N+1] (B == 1).
    ``rows`` optionally selects global token indices (b*T + t, or packed
    indices with cu_seqlens); the result then has shape [len(rows),HQ,V].
    Without ``rows`` it has shape [B,T,HQ,V].
    """
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    gs, sink, cu = _f32(g_scalar), _f32(sink_bias), _i32(cu_seqlens)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if scale is None:
        scale = K ** -0.5
    nseq = 0 if cu is None else cu.shape[0] - 1
    W = 0 if window_size is None else int(window_size)
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_a.shape[0]
    else:
        rows_a = None
        nrows = B * T
    o = np.zeros((nrows, HQ, V), dtype=np.float64)
    lse = np.zeros((nrows, HQ), dtype=np.float64)
    rc = _load().oracle_wall_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gs), _ptr(sink),
                                      B, T, HQ, H, K, V, _ptr(cu), nseq, W, float(scale),
                                      _ptr(rows_a), nrows, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_wall_attn_fwd: bad arguments")
    if rows is None:
        o = o.reshape(B, T, HQ, V)
        lse = lse.reshape(B, T, HQ)
    return (o, lse) if return_lse else o


def prefix_log2(g, cu_seqlens=None):
    """P2 = cumsum(g) / ln 2 along time, restarted per segment (README "Decode")."""
    g = _f32(g)
    cu = _i32(cu_seqlens)
    B, T, HQ, K = g.shape
    nseq = 0 if cu is None else cu.shape[0] - 1
    out = np.zeros(g.shape, dtype=np.float64)
    _load().oracle_prefix_log2(_ptr(g), B, T, HQ, K, _ptr(cu), nseq, _ptr(out))
    return out


def build_kv_cache(k, P2, chunk_size=64):
    """(k_tilde, r_cache) in float64, unrounded (README "Decode")."""
    k, P2 = _f32(k), _f32(P2)
    B, T, H, K = k.shape
    HQ = P2.shape[2]
    nc = -(-T // chunk_size)
    kt = np.zeros((B, T, HQ, K), dtype=np.float64)
    rc = np.zeros((B, nc, HQ, K), dtype=np.float64)
    r = _load().oracle_build_kv_cache(_ptr(k), _ptr(P2), B, T, HQ, H, K, chunk_size,
                                      _ptr(kt), _ptr(rc))
    if r != 0:
        raise ValueError("oracle_build_kv_cache: bad arguments")
    return kt, rc


def decode(q, v, p_curr, k_tilde, r_cache, sink_bias=None, scale=None, cache_chunk_size=64,
           return_lse=False):
    """Single-step decode over the cache (README "Decode"): o [B,1,HQ,V]."""
    q, v, p_curr = _f32(q), _f32(v), _f32(p_curr)
    k_tilde, r_cache, sink = _f32(k_tilde), _f32(r_cache), _f32(sink_bias)
    B, T, H, V = v.shape
    HQ, K = q.shape[2], q.shape[3]
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, HQ, V), dtype=np.float64)
    lse = np.zeros((B, HQ), dtype=np.float64)
    r = _load().oracle_decode_cache(_ptr(q), _ptr(v), _ptr(p_curr), _ptr(k_tilde), _ptr(r_cache),
                                    _ptr(sink), B, T, HQ, H, K, V, cache_chunk_size, float(scale),
                                    _ptr(o), _ptr(lse))
    if r != 0:
        raise ValueError("oracle_decode_cache: bad arguments")
    o = o.reshape(B, 1, HQ, V)
    lse = lse.reshape(B, 1, HQ)
    return (o, lse) if return_lse else o


def decode_ext(q, v, p_curr, k_tilde, r_cache, sink_bias=None, scale=None, cache_chunk_size=64,
               gate_cache=None, gate_curr=None, cache_seqlens=None, window_size=None,
               return_lse=False):
    """Decode over the cache with per-row lengths, a window and the gate cache
    (README "Decode" formula, the FlexAttention window rule, the forward's
    gate term): o [B,1,HQ,V].  Caches are contiguous [B,T,...] arrays;
    gate_cache [B,T,HQ] and gate_curr [B,1,HQ] are running sums of g_scalar
    in log2 units; cache_seqlens int [B]."""
    q, v, p_curr = _f32(q), _f32(v), _f32(p_curr)
    k_tilde, r_cache, sink = _f32(k_tilde), _f32(r_cache), _f32(sink_bias)
    gc, gq, lens = _f32(gate_cache), _f32(gate_curr), _i32(cache_seqlens)
    B, T, H, V = v.shape
    HQ, K = q.shape[2], q.shape[3]
    if scale is None:
        scale = K ** -0.5
    W = 0 if window_size is None else int(window_size)
    o = np.zeros((B, HQ, V), dtype=np.float64)
    lse = np.zeros((B, HQ), dtype=np.float64)
    r = _load().oracle_decode_cache_ext(_ptr(q), _ptr(v), _ptr(p_curr), _ptr(k_tilde),
                                        _ptr(r_cache), _ptr(sink), _ptr(gc), _ptr(gq), _ptr(lens),
                                        W, B, T, HQ, H, K, V, cache_chunk_size, float(scale),
                                        _ptr(o), _ptr(lse))
    if r != 0:
        raise ValueError("oracle_decode_cache_ext: bad arguments")
    o = o.reshape(B, 1, HQ, V)
    lse = lse.reshape(B, 1, HQ)
    return (o, lse) if return_lse else o


def wall_attn_bwd(q, k, v, g, dO, scale=None, g_scalar=None, sink_bias=None, window_size=None,
                  cu_seqlens=None):
    """Gradients of the forward (README introduction: analytic gradients for q,
    k, v, g; and g_scalar, sink_bias) for dL/do = dO [B,T,HQ,V].

    Returns a dict of float64 arrays: dq [B,T,HQ,K], dk [B,T,H,K],
    dv [B,T,H,V], dg [B,T,HQ,K], dg_scalar [B,T,HQ] (if g_scalar is given),
    dsink [HQ] (if sink_bias is given)."""
    q, k, v, g, dO = _f32(q), _f32(k), _f32(v), _f32(g), _f32(dO)
    gs, sink, cu = _f32(g_scalar), _f32(sink_bias), _i32(cu_seqlens)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if scale is None:
        scale = K ** -0.5
    nseq = 0 if cu is None else cu.shape[0] - 1
    W = 0 if window_size is None else int(window_size)
    out = dict(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(v.shape),
               dg=np.zeros(g.shape))
    dgs = np.zeros((B, T, HQ)) if gs is not None else None
    dsk = np.zeros(HQ) if sink is not None else None
    r = _load().oracle_wall_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gs), _ptr(sink),
                                     _ptr(dO), B, T, HQ, H, K, V, _ptr(cu), nseq, W, float(scale),
                                     _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                     _ptr(out["dg"]), _ptr(dgs), _ptr(dsk))
    if r != 0:
        raise ValueError("oracle_wall_attn_bwd: bad arguments")
    if dgs is not None:
        out["dg_scalar"] = dgs
    if dsk is not None:
        out["dsink"] = dsk
    return out
