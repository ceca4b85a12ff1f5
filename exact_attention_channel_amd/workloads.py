"""Seeded synthetic inputs for Wall Attention workloads.

This module only draws random tensors; it holds none of the attention
arithmetic.  The GPU tests, the benchmark and the oracle tests all take their
inputs from here, so both sides of every parity check see identical values.

Recipe (shapes follow the Wall Attention README, "Usage" and "Decode"):
draw with ``torch.Generator(device).manual_seed(seed)`` in float32, in the
order lengths, q, k, v, g, g_scalar, sink; scale where stated; cast to the
working dtype with round-to-nearest-even.  ``sink_bias`` stays float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    T: int                       # per-batch length (ignored when lengths is given)
    HQ: int
    H: int
    K: int
    V: int
    dtype: torch.dtype
    g_mode: str = "normal"       # "normal": g = std*N(0,1); "neg_softplus": g = -std*softplus(N(0,1)); "zero"
    g_std: float = 0.02
    g_scalar_std: float = 0.0    # > 0: g_scalar = -std*softplus(N(0,1)) of shape [B,T,HQ]
    sink: bool = False           # sink_bias ~ N(0,1) of shape [HQ]
    window: int = 0              # <= 0: no sliding window
    nseq: int = 0                # > 0: packed varlen with this many sequences (B == 1)
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 0
    # > 0: channel 0 of g is set to this rise in log2 units per token (times
    # ln 2, as g is in nats) and channel 0 of k to zero, so the decay sum of
    # that channel climbs steadily without adding to any score
    rise_ch0_log2: float = 0.0
    # > 0: channels 0 .. fast_ch-1 of g are set to fast_g (natural-log decay
    # per token) in query heads 0 .. fast_heads-1 (every head if 0)
    fast_ch: int = 0
    fast_g: float = 0.0
    fast_heads: int = 0


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    T_kv: int
    HQ: int
    H: int
    K: int
    V: int
    C: int
    dtype: torch.dtype
    g_std: float = 0.02
    sink: bool = False
    seed: int = 0


# The five workloads: a tiny fp32 case, the README's usage shape, an 8K-token
# long-context case, a packed varlen case with a sliding window, and a
# single-token decode over a 32K-token cache.
PREFILL_T128_FP32 = Prefill("prefill_B1_T128_HQ2_H1_D64_fp32", 1, 128, 2, 1, 64, 64,
                            torch.float32, seed=1)
PREFILL_T1024_BF16 = Prefill("prefill_B2_T1024_HQ8_H4_D64_bf16", 2, 1024, 8, 4, 64, 64,
                             torch.bfloat16, seed=2)
PREFILL_T8192_BF16 = Prefill("prefill_B1_T8192_HQ16_H4_D128_bf16_gscalar_sink", 1, 8192, 16, 4,
                             128, 128, torch.bfloat16, g_mode="neg_softplus", g_std=0.05,
                             g_scalar_std=0.01, sink=True, seed=3)
VARLEN_W2048_BF16 = Prefill("varlen16_L512-4096_HQ32_H8_D128_W2048_bf16", 1, 0, 32, 8, 128, 128,
                            torch.bfloat16, window=2048, nseq=16, len_lo=512, len_hi=4096, seed=4)
DECODE_T32768_BF16 = Decode("decode_B64_Tkv32768_C64_HQ32_H8_D128_bf16", 64, 32768, 32, 8, 128,
                            128, 64, torch.bfloat16, seed=5)

PREFILL_CONFIGS = [PREFILL_T128_FP32, PREFILL_T1024_BF16, PREFILL_T8192_BF16, VARLEN_W2048_BF16]


def _gen(device, seed):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def varlen_lengths(cfg: Prefill) -> list:
    gen = _gen("cpu", cfg.seed)
    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.nseq,), generator=gen)
    return [int(x) for x in lens]


def make_prefill(cfg: Prefill, device="cpu", seed: Optional[int] = None) -> dict:
    """Inputs for a prefill workload as a dict of tensors on ``device``.

    Keys: q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K] in cfg.dtype;
    g_scalar [B,T,HQ] (cfg.dtype) or None; sink_bias [HQ] float32 or None;
    cu_seqlens int32 [nseq+1] or None; window_size; scale (= K^-0.5).
    Random draws happen on the CPU, so values do not depend on ``device``.
    """
    seed = cfg.seed if seed is None else seed
    gen = _gen("cpu", seed)
    if cfg.nseq > 0:
        lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.nseq,), generator=gen)
        cu = torch.zeros(cfg.nseq + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
        B, T = 1, int(cu[-1])
    else:
        cu = None
        B, T = cfg.B, cfg.T
    f32 = torch.float32
    q = torch.randn(B, T, cfg.HQ, cfg.K, generator=gen, dtype=f32)
    k = torch.randn(B, T, cfg.H, cfg.K, generator=gen, dtype=f32)
    v = torch.randn(B, T, cfg.H, cfg.V, generator=gen, dtype=f32)
    if cfg.g_mode == "zero":
        g = torch.zeros(B, T, cfg.HQ, cfg.K, dtype=f32)
    else:
        g = torch.randn(B, T, cfg.HQ, cfg.K, generator=gen, dtype=f32)
        if cfg.g_mode == "normal":
            g = g * cfg.g_std
        elif cfg.g_mode == "neg_softplus":
            g = -torch.nn.functional.softplus(g) * cfg.g_std
        else:
            raise ValueError(cfg.g_mode)
    gs = None
    if cfg.g_scalar_std > 0:
        gs = -torch.nn.functional.softplus(
            torch.randn(B, T, cfg.HQ, generator=gen, dtype=f32)) * cfg.g_scalar_std
    sink = torch.randn(cfg.HQ, generator=gen, dtype=f32) if cfg.sink else None
    if cfg.rise_ch0_log2 > 0:
        g[..., 0] = cfg.rise_ch0_log2 * 0.6931471805599453
        k[..., 0] = 0.0
    if cfg.fast_ch > 0:
        nh = cfg.fast_heads if cfg.fast_heads > 0 else cfg.HQ
        g[:, :, :nh, :cfg.fast_ch] = cfg.fast_g
    dt = cfg.dtype
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.to(dt),
               g_scalar=None if gs is None else gs.to(dt), sink_bias=sink,
               cu_seqlens=cu, window_size=cfg.window if cfg.window > 0 else None,
               scale=cfg.K ** -0.5)
    for key in ("q", "k", "v", "g", "g_scalar", "sink_bias", "cu_seqlens"):
        if out[key] is not None:
            out[key] = out[key].to(device)
    return out


def decode_row(cfg: Decode, b: int) -> dict:
    """Batch row b of a decode workload, drawn on the CPU with its own
    generator (seed * 100003 + b), in the order k, v, g, q: any row can be
    drawn alone, identically on every machine.

    Keys: k [1,T_kv,H,K], v [1,T_kv,H,V], g [1,T_kv,HQ,K], q [1,1,HQ,K] in
    cfg.dtype."""
    gen = _gen("cpu", cfg.seed * 100003 + b)
    f32, dt, T = torch.float32, cfg.dtype, cfg.T_kv
    k = torch.randn(1, T, cfg.H, cfg.K, generator=gen, dtype=f32).to(dt)
    v = torch.randn(1, T, cfg.H, cfg.V, generator=gen, dtype=f32).to(dt)
    g = (torch.randn(1, T, cfg.HQ, cfg.K, generator=gen, dtype=f32) * cfg.g_std).to(dt)
    q = torch.randn(1, 1, cfg.HQ, cfg.K, generator=gen, dtype=f32).to(dt)
    return dict(k=k, v=v, g=g, q=q)


def decode_sink(cfg: Decode):
    """sink_bias of a decode workload (float32 [HQ], seed * 100003 - 1), or None."""
    if not cfg.sink:
        return None
    return torch.randn(cfg.HQ, generator=_gen("cpu", cfg.seed * 100003 - 1), dtype=torch.float32)


def make_decode(cfg: Decode, device="cpu", threads: int = 16) -> dict:
    """Inputs for a decode workload: k, v, g over the cache and the newest query.

    Keys: k [B,T_kv,H,K], v [B,T_kv,H,V], g [B,T_kv,HQ,K], q [B,1,HQ,K]
    (cfg.dtype) on ``device``, sink_bias [HQ] float32 or None, scale.  Every
    batch row is ``decode_row(cfg, b)`` (rows are drawn in parallel host
    threads, each with its own generator, and copied to ``device`` as they
    finish).
    """
    from concurrent.futures import ThreadPoolExecutor
    B, T, dt = cfg.B, cfg.T_kv, cfg.dtype
    out = dict(k=torch.empty(B, T, cfg.H, cfg.K, dtype=dt, device=device),
               v=torch.empty(B, T, cfg.H, cfg.V, dtype=dt, device=device),
               g=torch.empty(B, T, cfg.HQ, cfg.K, dtype=dt, device=device),
               q=torch.empty(B, 1, cfg.HQ, cfg.K, dtype=dt, device=device))
    with ThreadPoolExecutor(max_workers=max(1, min(threads, B))) as ex:
        for b, row in enumerate(ex.map(lambda i: decode_row(cfg, i), range(B))):
            for key in ("k", "v", "g", "q"):
                out[key][b:b + 1].copy_(row[key])
    sink = decode_sink(cfg)
    out["sink_bias"] = None if sink is None else sink.to(device)
    out["scale"] = cfg.K ** -0.5
    return out
