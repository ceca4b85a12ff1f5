#!/usr/bin/env python3
"""Benchmark of libwallattn on one MI355X: Wall Attention prefill TFLOP/s at
T = 8K and single-step decode GB/s over a 32K-token cache.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100]

One "step" is one call of wall_attn_fwd (running-sum pre-pass + attention)
on the long-context workload B=1, T=8192, HQ=16, H=4, K=V=128, bf16, with
g = -0.05*softplus(N(0,1)), g_scalar and sink_bias (inputs resident in HBM
before timing starts).  After the warm-up steps, untimed steps run for
--settle seconds (the clocks ramp up over the first tens of milliseconds);
the timed steps are then interleaved in blocks with blocks of the
pre-pass alone and of the attention kernel alone, so the three figures see
the same clocks.  ``value`` is its throughput in algorithmic TFLOP/s:
2*HQ*(K+V) per visible (query, key) pair, only causal pairs counted.

Also reported on the same JSON line:
  roofline      the attention kernel alone (wall_attn_fwd_attend), timed with
                HIP events on the launch stream, against the MI355X dense
                fp16/bf16 MFMA peak;
  decode        wall_attn_decode on B=64, T_kv=32768, HQ=32, H=8, K=V=128,
                C=64, for each cache element type (float32 -- the format
                that reproduces the forward on this workload -- float16,
                bfloat16): algorithmic bytes (k_tilde, v, r_cache, q, p_curr,
                o, sink) per call over its event-timed duration, against HBM
                peak; the cache build is reported beside it;
  cpu_baseline  the fp64 CPU oracle timed on this host's cores over a row
                sample of the prefill workload, scaled to TFLOP/s; the two
                small workloads (tiny fp32, usage shape) are also timed in
                full on one host thread (all_configs[].cpu_oracle_1thread).
The roofline "traffic" fields are HBM bytes per launch measured with rocprof
counters (profiles/hbm_traffic.json); they are null when the kernel sources
no longer match the ones the counters were taken on.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "prefill TFLOP/s (% bf16 MFMA peak) at T=8K; decode GB/s (% HBM peak)"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU needs some tens of milliseconds of work to reach steady clocks:
    # with 5 warm-up steps (~2 ms) the first timed steps of the 8K prefill ran
    # ~15% slower than later ones
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed launches after the warm-up steps, before timing")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-row-stride", type=int, default=1,
                    help="oracle baseline evaluates every n-th query row")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (read) + 1 GiB (write), "
                         "three times: the calibration kernel for rocprof's FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "exact_attention_channel_amd", "csrc")
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.json")
# sources whose kernels the recorded counters describe
TRAFFIC_SOURCES = {
    "attend": ["attn_fwd.hip", "common.h", "launch.h"],
    "decode_split_float32": ["decode_kernels.h", "decode.hip", "common.h", "launch.h"],
    "decode_split_float16": ["decode_kernels.h", "decode.hip", "common.h", "launch.h"],
    "decode_split_bfloat16": ["decode_kernels.h", "decode.hip", "common.h", "launch.h"],
}


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(key):
    """HBM bytes per launch of kernel `key` from rocprof FETCH_SIZE + WRITE_SIZE
    (scaled by the copy-kernel calibration), or None when no counters were
    recorded or the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(TRAFFIC_SOURCES[key]):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe():
    import torch
    n = 1 << 28  # float32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 x elementwise copy of {n * 4} bytes read + {n * 4} bytes written")


def causal_pairs(lengths, window=0):
    tot = 0
    for L in lengths:
        if window <= 0 or window >= L:
            tot += L * (L + 1) // 2
        else:
            tot += window * (window + 1) // 2 + (L - window) * window
    return tot


def event_time_ms(fn, n, torch):
    """Average milliseconds of fn() over n back-to-back launches on the current stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def time_prefill(cfg, lib, wa, W, torch, dev, stream, steps, warmup):
    """Event-timed wall_attn_fwd on one prefill workload: (ms per call, algorithmic FLOPs)."""
    x = W.make_prefill(cfg, device=dev)
    B, T = int(x["q"].shape[0]), int(x["q"].shape[1])
    HQ, H, K, V = cfg.HQ, cfg.H, cfg.K, cfg.V
    dt = wa.WA_BF16 if cfg.dtype == torch.bfloat16 else wa.WA_F32
    cu = x["cu_seqlens"]
    if cu is None:
        nseq, maxlen, lengths = 0, 0, [T] * B
    else:
        lengths = (cu[1:] - cu[:-1]).tolist()
        nseq, maxlen = len(lengths), max(lengths)
    window = x["window_size"] or 0
    o = torch.empty(B, T, HQ, V, dtype=cfg.dtype, device=dev)
    wsb = lib.wall_attn_fwd_workspace_bytes(B, T, HQ, H, K, V, nseq, maxlen, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ptr = lambda t: None if t is None else t.data_ptr()

    def fwd():
        rc = lib.wall_attn_fwd(ptr(x["q"]), ptr(x["k"]), ptr(x["v"]), ptr(x["g"]),
                               ptr(x["g_scalar"]), ptr(x["sink_bias"]), ptr(o), None,
                               B, T, HQ, H, K, V, ptr(cu), nseq, maxlen, window,
                               float(x["scale"]), dt, ptr(ws), wsb, stream)
        if rc:
            raise RuntimeError(lib.wall_attn_last_error().decode())

    for _ in range(warmup):
        fwd()
    ms = event_time_ms(fwd, steps, torch)
    return ms, 2.0 * HQ * (K + V) * causal_pairs(lengths, window)


def settle_clocks(fn, seconds, torch):
    """Untimed launches of fn until `seconds` of wall time have passed (the
    GPU clocks ramp up over the first tens of milliseconds of work); returns
    the time spent."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def interleaved_ms(fns, steps, torch, blocks=5):
    """Average ms per launch of each fn: `steps` launches of each, in `blocks`
    rounds that cycle through the fns, every round's launches of one fn timed
    between two events on the current stream."""
    n = [steps // blocks + (1 if b < steps % blocks else 0) for b in range(blocks)]
    tot = [0.0] * len(fns)
    for nb in n:
        if nb == 0:
            continue
        for i, fn in enumerate(fns):
            tot[i] += event_time_ms(fn, nb, torch) * nb
    return [t / steps for t in tot]


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return

    import torch
    import exact_attention_channel_amd as wa
    from exact_attention_channel_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = wa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    # ------------------------------------------------------------------ prefill
    c = W.PREFILL_T8192_BF16
    log(f"[bench] prefill workload {c.name}: generating inputs")
    x = W.make_prefill(c, device=dev)
    B, T, HQ, H, K, V = c.B, c.T, c.HQ, c.H, c.K, c.V
    o = torch.empty(B, T, HQ, V, dtype=c.dtype, device=dev)
    lse = torch.empty(B, T, HQ, dtype=torch.float32, device=dev)
    wsb = lib.wall_attn_fwd_workspace_bytes(B, T, HQ, H, K, V, 0, 0, wa.WA_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    scale = float(x["scale"])

    def fwd():
        rc = lib.wall_attn_fwd(ptr(x["q"]), ptr(x["k"]), ptr(x["v"]), ptr(x["g"]),
                               ptr(x["g_scalar"]), ptr(x["sink_bias"]), ptr(o), ptr(lse),
                               B, T, HQ, H, K, V, None, 0, 0, 0, scale, wa.WA_BF16,
                               ptr(ws), wsb, stream)
        if rc:
            raise RuntimeError(lib.wall_attn_last_error().decode())

    def prepare():
        rc = lib.wall_attn_fwd_prepare(ptr(x["q"]), ptr(x["k"]), ptr(x["g"]), ptr(x["g_scalar"]),
                                       B, T, HQ, H, K, V, None, 0, 0, scale, wa.WA_BF16,
                                       ptr(ws), wsb, stream)
        if rc:
            raise RuntimeError(lib.wall_attn_last_error().decode())

    def attend():
        rc = lib.wall_attn_fwd_attend(ptr(x["q"]), ptr(x["v"]), ptr(x["g"]), ptr(x["g_scalar"]),
                                      ptr(x["sink_bias"]), ptr(o), ptr(lse), B, T, HQ, H, K, V,
                                      None, 0, 0, 0, scale, wa.WA_BF16, ptr(ws), wsb, stream)
        if rc:
            raise RuntimeError(lib.wall_attn_last_error().decode())

    flops = 2.0 * HQ * (K + V) * causal_pairs([T] * B)
    for _ in range(args.warmup):
        fwd()
    settle_s = settle_clocks(fwd, args.settle, torch)
    # timed region: exactly `steps` full forward passes, in blocks interleaved
    # with blocks of the two stages alone, so that all three see the same
    # clocks; each block is bracketed by synchronisations and events
    ms_step, ms_prep, ms_attn = interleaved_ms([fwd, prepare, attend], args.steps, torch)
    log(f"[bench] prefill step {ms_step:.4f} ms; prepare {ms_prep:.4f} ms, attend {ms_attn:.4f} ms "
        f"(after {args.warmup} warm-up steps and {settle_s:.2f} s of clock settling)")
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    del ws, o, lse, x
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": round(settle_s, 3),
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": c.name, "B": B, "T": T, "HQ": HQ, "H": H, "K": K, "V": V,
                   "causal": True, "g": "-0.05*softplus(N(0,1))", "g_scalar": True,
                   "sink_bias": True, "gflop_per_step": round(flops / 1e9, 3)},
        "roofline": {"kernel": "k_attn_fwd_bf16 (wall_attn_fwd_attend)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4),
                     "traffic": recorded_traffic("attend"), "kernel_ms": round(ms_attn, 4)},
        "prefill_breakdown_ms": {"prepare": round(ms_prep, 4), "attend": round(ms_attn, 4)},
    }

    # ------------------------------------------------------------------ backward
    if not args.no_backward:
        xb = W.make_prefill(c, device=dev)
        ob, lb = wa.wall_attn(xb["q"], xb["k"], xb["v"], xb["g"], scale=xb["scale"],
                              g_scalar=xb["g_scalar"], sink_bias=xb["sink_bias"], return_lse=True)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        dO = torch.randn(ob.shape, generator=gen, device=dev).to(ob.dtype)
        grads = [torch.empty_like(xb[n]) for n in ("q", "k", "v", "g", "g_scalar")]
        dsink = torch.empty_like(xb["sink_bias"])
        bwb = lib.wall_attn_bwd_workspace_bytes(B, T, HQ, H, K, V, 0, 0, wa.WA_BF16)
        bws = torch.empty(bwb, dtype=torch.uint8, device=dev)

        def bwd():
            rc = lib.wall_attn_bwd(ptr(xb["q"]), ptr(xb["k"]), ptr(xb["v"]), ptr(xb["g"]),
                                   ptr(xb["g_scalar"]), ptr(xb["sink_bias"]), ptr(ob), ptr(lb),
                                   ptr(dO), *[ptr(t) for t in grads[:4]], ptr(grads[4]),
                                   ptr(dsink), B, T, HQ, H, K, V, None, 0, 0, 0, scale,
                                   wa.WA_BF16, ptr(bws), bwb, stream)
            if rc:
                raise RuntimeError(lib.wall_attn_last_error().decode())

        bwd()
        nb = max(2, min(args.steps, 5))
        ms_bwd = event_time_ms(bwd, nb, torch)
        # per visible pair and head: scores 2K, dO.v 2V, dv 2V, dq 2K, dk 2K
        bflops = 2.0 * HQ * (3 * K + 2 * V) * causal_pairs([T] * B)
        btf = bflops / (ms_bwd * 1e-3) / 1e12
        log(f"[bench] backward {ms_bwd:.3f} ms, {btf:.1f} TFLOP/s")
        out["backward"] = {
            "workload": c.name, "call": "wall_attn_bwd", "ms": round(ms_bwd, 3),
            "gflop": round(bflops / 1e9, 3), "TFLOP/s": round(btf, 2), "launches_timed": nb,
            # the whole call (pre-pass, both matrix-core kernels, running sums)
            "roofline": {"kernel": "wall_attn_bwd (k_bwd_dkdv_w16 + k_bwd_dq_w16 + finishing)",
                         "bound": "mfma", "achieved": round(btf, 2), "peak": PEAK_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(btf / PEAK_MFMA_TFLOPS, 4),
                         "traffic": None},
        }
        del xb, ob, lb, dO, grads, dsink, bws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ other workloads
    # the remaining prefill workloads (tiny fp32, usage shape, packed varlen
    # with a window), same protocol; their outputs are checked by the GPU tests
    allc = []
    for cfg in W.PREFILL_CONFIGS:
        if cfg is c:
            ms_c, fl_c = ms_step, flops
        else:
            ms_c, fl_c = time_prefill(cfg, lib, wa, W, torch, dev, stream, args.steps,
                                      args.warmup)
            torch.cuda.empty_cache()
        tf = fl_c / (ms_c * 1e-3) / 1e12
        e = {"workload": cfg.name, "call": "wall_attn_fwd",
             "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
             "ms": round(ms_c, 4), "gflop": round(fl_c / 1e9, 3), "TFLOP/s": round(tf, 2)}
        if cfg.dtype == torch.bfloat16:
            e["frac_mfma_peak"] = round(tf / PEAK_MFMA_TFLOPS, 4)
        log(f"[bench] {cfg.name}: {ms_c:.4f} ms, {tf:.1f} TFLOP/s")
        allc.append(e)
    out["all_configs"] = allc

    # ------------------------------------------------------------------ decode
    if not args.no_decode:
        d = W.DECODE_T32768_BF16
        log(f"[bench] decode workload {d.name}: drawing inputs (one host thread per batch row)")
        y = W.make_decode(d, device=dev)
        P = wa.wall_attn_prefix_log2(y["g"])
        del y["g"]
        torch.cuda.empty_cache()
        pc = P[:, -1:].contiguous()
        do = torch.empty(d.B, 1, d.HQ, d.V, dtype=d.dtype, device=dev)
        dl = torch.empty(d.B, 1, d.HQ, dtype=torch.float32, device=dev)
        dwb = lib.wall_attn_decode_workspace_bytes(d.B, d.T_kv, d.HQ, d.H, d.K, d.V, d.C)
        dws = torch.empty(dwb, dtype=torch.uint8, device=dev)
        dscale = float(y["scale"])
        out["decode"] = {}
        # float32 cache first: the format that reproduces the forward on this
        # workload (the headline decode figure); the 16-bit caches for context
        for cname, ct, code in (("float32", torch.float32, wa.WA_F32),
                                ("float16", torch.float16, wa.WA_F16),
                                ("bfloat16", torch.bfloat16, wa.WA_BF16)):
            kt, rc_ = wa.build_wall_kv_cache(y["k"], P, chunk_size=d.C, cache_dtype=ct)

            def build():
                r = lib.wall_attn_build_kv_cache(ptr(y["k"]), ptr(P), ptr(kt), ptr(rc_), d.B,
                                                 d.T_kv, d.HQ, d.H, d.K, d.C, wa.WA_BF16, code,
                                                 stream)
                if r:
                    raise RuntimeError(lib.wall_attn_last_error().decode())

            def dec():
                r = lib.wall_attn_decode(ptr(y["q"]), ptr(y["v"]), ptr(pc), ptr(kt), ptr(rc_),
                                         ptr(y["sink_bias"]), ptr(do), ptr(dl), d.B, d.T_kv, d.HQ,
                                         d.H, d.K, d.V, d.C, dscale, wa.WA_BF16, code, ptr(dws),
                                         dwb, stream)
                if r:
                    raise RuntimeError(lib.wall_attn_last_error().decode())

            build_ms = event_time_ms(build, 3, torch)
            for _ in range(args.warmup):
                dec()
            dms = event_time_ms(dec, args.steps, torch)
            nc = -(-d.T_kv // d.C)
            assert rc_.shape[1] == nc
            dbytes = (kt.numel() * kt.element_size() + y["v"].numel() * 2 + rc_.numel() * 4
                      + y["q"].numel() * 2 + pc.numel() * 4 + do.numel() * 2
                      + (0 if y["sink_bias"] is None else d.HQ * 4))
            gbs = dbytes / (dms * 1e-3) / 1e9
            build_bytes = (y["k"].numel() * 2 + d.B * d.T_kv * d.HQ * d.K * 4
                           + kt.numel() * kt.element_size() + rc_.numel() * 4)
            log(f"[bench] decode ({cname} cache) {dms:.4f} ms, {gbs:.1f} GB/s; "
                f"cache build {build_ms:.3f} ms")
            out["decode"][cname + "_cache"] = {
                "workload": d.name, "cache_dtype": cname, "metric": "decode GB/s",
                "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(dms, 4),
                "bytes_per_call": dbytes,
                "roofline": {"kernel": "k_decode_split + k_decode_combine (wall_attn_decode)",
                             "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "traffic": recorded_traffic("decode_split_" + cname)},
                "cache_build": {"ms": round(build_ms, 3),
                                "GB/s": round(build_bytes / (build_ms * 1e-3) / 1e9, 1)},
            }
            out["all_configs"].append({"workload": d.name, "call": "wall_attn_decode",
                                       "dtype": "bf16", "cache_dtype": cname, "ms": round(dms, 4),
                                       "GB/s": round(gbs, 1),
                                       "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})
            del kt, rc_
            torch.cuda.empty_cache()
        del y, dws, do, dl, pc, P
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        import oracle
        cx = W.make_prefill(c)
        stride = max(1, args.cpu_row_stride)
        rows = list(range(stride - 1, T, stride))
        sample_flops = 2.0 * HQ * (K + V) * sum(r + 1 for r in rows)
        log(f"[bench] cpu baseline: oracle over {len(rows)} rows on {oracle.num_threads()} threads")
        t0 = time.perf_counter()
        oracle.wall_attn(cx["q"], cx["k"], cx["v"], cx["g"], scale=cx["scale"],
                         g_scalar=cx["g_scalar"], sink_bias=cx["sink_bias"], rows=rows)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"every {stride}th query row of {c.name} ({len(rows)} rows x {HQ} heads, "
                      f"{sample_flops / 1e9:.1f} GFLOP algorithmic) in {dt:.2f} s; "
                      "TFLOP/s = sample FLOPs / wall time",
        }
        # the two small workloads in full on one host thread as well
        n_all = oracle.num_threads()
        oracle.set_num_threads(1)
        try:
            for e in out["all_configs"]:
                cfg = next((p for p in (W.PREFILL_T128_FP32, W.PREFILL_T1024_BF16)
                            if p.name == e["workload"]), None)
                if cfg is None:
                    continue
                x1 = W.make_prefill(cfg)
                t0 = time.perf_counter()
                oracle.wall_attn(x1["q"], x1["k"], x1["v"], x1["g"], scale=x1["scale"],
                                 g_scalar=x1["g_scalar"], sink_bias=x1["sink_bias"],
                                 window_size=x1["window_size"], cu_seqlens=x1["cu_seqlens"])
                dt1 = time.perf_counter() - t0
                e["cpu_oracle_1thread"] = {"s": round(dt1, 4),
                                           "TFLOP/s": round(e["gflop"] * 1e9 / dt1 / 1e12, 6),
                                           "gpu_speedup": round(dt1 * 1e3 / e["ms"], 1)}
                log(f"[bench] oracle on one thread, {cfg.name}: {dt1:.3f} s")
        finally:
            oracle.set_num_threads(n_all)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
