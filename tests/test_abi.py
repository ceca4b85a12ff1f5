"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

The argument checks only exercise paths that return before the first HIP
call, so they run on a machine without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wallattn.h")


@pytest.fixture(scope="module")
def lib():
    import exact_attention_channel_amd as wa
    if not os.path.exists(wa.library_path()):
        from exact_attention_channel_amd import build
        build.build()
    return wa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wall_attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("wall_attn_fwd", "wall_attn_build_kv_cache", "wall_attn_decode",
              "wall_attn_prefix_log2", "wall_attn_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    import exact_attention_channel_amd as wa
    names = declared_functions()
    assert set(names) == set(wa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", wa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def fwd(lib, B=1, T=128, HQ=4, H=2, K=64, V=64, cu=None, nseq=0, maxlen=0, dtype=0,
        ws_bytes=1 << 40, q=FAKE, k=FAKE, v=FAKE, g=FAKE, o=FAKE, ws=FAKE, gs=None):
    return lib.wall_attn_fwd(q, k, v, g, gs, None, o, None, B, T, HQ, H, K, V, cu, nseq, maxlen,
                             0, 0.0, dtype, ws, ws_bytes, None)


def test_fwd_rejects_bad_shapes(lib):
    assert fwd(lib, HQ=6, H=4) == 1                       # HQ % H != 0
    assert b"multiple" in lib.wall_attn_last_error()
    assert fwd(lib, B=2, cu=FAKE, nseq=2, maxlen=64) == 1   # cu_seqlens needs B == 1
    assert fwd(lib, B=0) == 1
    assert fwd(lib, T=-5) == 1
    assert fwd(lib, K=96) == 2
    assert fwd(lib, V=256) == 2
    assert fwd(lib, dtype=7) == 2
    assert fwd(lib, cu=FAKE, nseq=0, maxlen=64) == 1
    assert fwd(lib, cu=FAKE, nseq=2, maxlen=500) == 1       # max_seqlen > T
    # bf16: one sequence's rescaled keys must fit 32-bit offsets
    assert fwd(lib, T=1 << 19, HQ=16, H=4, K=128, V=128) == 2
    assert b"too long" in lib.wall_attn_last_error()
    assert lib.wall_attn_fwd_workspace_bytes(1, (1 << 19) - 64, 16, 4, 128, 128, 0, 0, 0) > 0
    assert lib.wall_attn_fwd_workspace_bytes(1, 1 << 19, 16, 4, 128, 128, 0, 0, 1) > 0  # fp32: 64-bit
    # launch-grid limits: at most 65535 segments, HQ*(ceil(max_seqlen/64)+8)*segments < 2^31
    assert fwd(lib, B=1, T=70000, cu=FAKE, nseq=70000, maxlen=1, dtype=1) == 2
    assert b"launch grid" in lib.wall_attn_last_error()
    assert fwd(lib, B=65535, T=4096, HQ=1024, H=1024, dtype=1) == 2
    assert b"launch grid" in lib.wall_attn_last_error()
    assert lib.wall_attn_fwd_workspace_bytes(65535, 4096, 1024, 1024, 64, 64, 0, 0, 1) == 0


def test_fwd_rejects_bad_pointers_and_workspace(lib):
    assert fwd(lib, q=None) == 1
    assert fwd(lib, o=None) == 1
    assert fwd(lib, ws=None) == 1
    assert fwd(lib, k=FAKE + 2) == 1                        # misaligned
    assert fwd(lib, gs=FAKE + 8) == 1
    need = lib.wall_attn_fwd_workspace_bytes(1, 128, 4, 2, 64, 64, 0, 0, 0)
    assert need > 0
    assert fwd(lib, ws_bytes=need - 1) == 4
    assert b"workspace" in lib.wall_attn_last_error()


def test_workspace_sizes(lib):
    assert lib.wall_attn_fwd_workspace_bytes(1, 128, 4, 3, 64, 64, 0, 0, 0) == 0
    a = lib.wall_attn_fwd_workspace_bytes(1, 8192, 16, 4, 128, 128, 0, 0, 0)
    b = lib.wall_attn_fwd_workspace_bytes(1, 8192, 16, 4, 128, 128, 0, 0, 1)
    # the rescaled operands dominate: bf16 keeps half keys with 16 extra
    # channels per row (the queries are rescaled inside the attention kernel),
    # fp32 keeps float queries and keys
    assert a >= 8192 * 16 * (128 + 16) * 2 and b >= 2 * 8192 * 16 * 128 * 4 and b > a
    assert lib.wall_attn_decode_workspace_bytes(64, 32768, 32, 8, 128, 128, 64) > 0
    assert lib.wall_attn_decode_workspace_bytes(64, 32768, 32, 8, 128, 128, 32) == 0
    assert lib.wall_attn_prefix_log2_workspace_bytes(2, 100, 4, 64, 0, 0) > 0


def test_cache_and_decode_reject_bad_arguments(lib):
    bk = lib.wall_attn_build_kv_cache
    assert bk(FAKE, FAKE, FAKE, FAKE, 1, 128, 4, 2, 64, 32, 0, 1, None) == 2   # chunk_size
    assert bk(FAKE, FAKE, FAKE, FAKE, 1, 128, 4, 3, 64, 64, 0, 1, None) == 1   # HQ % H
    assert bk(None, FAKE, FAKE, FAKE, 1, 128, 4, 2, 64, 64, 0, 1, None) == 1
    assert bk(FAKE, FAKE, FAKE + 4, FAKE, 1, 128, 4, 2, 64, 64, 0, 1, None) == 1
    assert bk(FAKE, FAKE, FAKE, FAKE, 70000, 128, 4, 2, 64, 64, 1, 1, None) == 2      # B > 65535
    assert bk(FAKE, FAKE, FAKE, FAKE, 2, 1 << 26, 1024, 8, 64, 64, 1, 1, None) == 2   # grid x
    assert bk(FAKE, FAKE, FAKE, FAKE, 1, 128, 4, 2, 64, 64, 0, 5, None) == 2   # cache dtype
    dec = lib.wall_attn_decode

    def d(**kw):
        a = dict(q=FAKE, v=FAKE, p=FAKE, kt=FAKE, r=FAKE, s=None, o=FAKE, l=None, B=2, T=256,
                 HQ=8, H=2, K=128, V=128, C=64, scale=0.0, dt=0, ct=1, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return dec(a["q"], a["v"], a["p"], a["kt"], a["r"], a["s"], a["o"], a["l"], a["B"],
                   a["T"], a["HQ"], a["H"], a["K"], a["V"], a["C"], a["scale"], a["dt"], a["ct"],
                   a["ws"], a["wsb"], None)
    assert d(C=128) == 2
    assert d(HQ=6, H=4) == 1
    assert d(K=80) == 2
    assert d(kt=None) == 1
    assert d(o=FAKE + 2) == 1
    assert d(wsb=16) == 4
    assert d(dt=3) == 2
    assert d(ct=3) == 2
    assert d(T=1 << 31) == 2                  # 32-bit token positions
    assert d(HQ=65536 * 2, H=2) == 2          # launch grid / 32-bit chunk offsets


def test_decode_ext_and_append_reject_bad_arguments(lib):
    ext = lib.wall_attn_decode_ext

    def d(**kw):
        a = dict(q=FAKE, v=FAKE, p=FAKE, kt=FAKE, r=FAKE, s=None, gc=None, gq=None, o=FAKE,
                 l=None, B=2, T=256, HQ=8, H=2, K=128, V=128, C=64, scale=0.0, dt=0, ct=1,
                 lens=None, W=0, bt=None, mb=0, ps=0, np_=0, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return ext(a["q"], a["v"], a["p"], a["kt"], a["r"], a["s"], a["gc"], a["gq"], a["o"],
                   a["l"], a["B"], a["T"], a["HQ"], a["H"], a["K"], a["V"], a["C"], a["scale"],
                   a["dt"], a["ct"], a["lens"], a["W"], a["bt"], a["mb"], a["ps"], a["np_"],
                   a["ws"], a["wsb"], None)
    assert d(W=-1) == 1                                   # negative window
    assert d(gc=FAKE) == 1                                # gate cache without gate_curr
    assert d(gq=FAKE) == 1
    assert d(bt=FAKE, mb=4, ps=96, np_=8) == 1            # page size not a multiple of 64
    assert d(bt=FAKE, mb=0, ps=128, np_=8) == 1           # no blocks
    assert d(bt=FAKE, mb=4, ps=128, np_=0) == 1           # no pages
    assert d(bt=FAKE + 4, mb=4, ps=128, np_=8) == 1       # misaligned table
    assert d(lens=FAKE + 4) == 1
    # the paged capacity max_blocks*page_size sizes the workspace
    need = lib.wall_attn_decode_workspace_bytes(2, 4 * 128, 8, 2, 128, 128, 64)
    assert d(bt=FAKE, mb=4, ps=128, np_=8, wsb=need - 1) == 4
    app = lib.wall_attn_cache_append

    def a(**kw):
        x = dict(k=FAKE, v=FAKE, p=FAKE, gn=None, kt=FAKE, vc=FAKE, r=FAKE, gc=None, lens=FAKE,
                 B=2, T=256, HQ=8, H=2, K=128, V=128, C=64, dt=0, ct=1, bt=None, mb=0, ps=0, np_=0)
        x.update(kw)
        return app(x["k"], x["v"], x["p"], x["gn"], x["kt"], x["vc"], x["r"], x["gc"], x["lens"],
                   x["B"], x["T"], x["HQ"], x["H"], x["K"], x["V"], x["C"], x["dt"], x["ct"],
                   x["bt"], x["mb"], x["ps"], x["np_"], None)
    assert a(lens=None) == 1
    assert a(gn=FAKE) == 1
    assert a(C=32) == 2
    assert a(ct=9) == 2
    assert a(HQ=6, H=4) == 1
    assert a(bt=FAKE, mb=2, ps=100, np_=4) == 1


def test_python_binding_fails_loudly_without_gpu_tensors():
    import torch
    import exact_attention_channel_amd as wa
    x = torch.zeros(1, 64, 2, 64)
    with pytest.raises(ValueError):
        wa.wall_attn(x, x[:, :, :1], x[:, :, :1], x)
