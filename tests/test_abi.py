"""The C ABI of libfa: exports and argument validation (CPU only).

libfa validates every argument before any HIP call, so every error path is
reachable without a GPU.  Fake (but suitably aligned) device addresses are
passed where a pointer must merely be non-NULL; validation never
dereferences them and these calls fail before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

import exact_io_aware_31_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = ctypes.c_void_p(0x10000)        # aligned stand-in pointer, never dereferenced
P_ODD = ctypes.c_void_p(0x10002)    # 2-byte aligned only
NULL = ctypes.c_void_p(0)
ERR = {v: k for k, v in fa.STATUS_NAMES.items()}


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == {"fa_fwd", "fa_bwd", "fa_decode", "fa_fwd_ex", "fa_bwd_ex",
                          "fa_decode_ex", "fa_decode_varlen", "fa_decode_noalloc",
                          "fa_bwd_workspace_bytes", "fa_decode_workspace_bytes",
                          "fa_status_string", "fa_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/fa.h but not exported"


def test_status_strings_and_version(lib):
    for code, name in fa.STATUS_NAMES.items():
        assert fa.fa_status_string(code).startswith(name)
    assert "unknown" in fa.fa_status_string(99)
    assert re.fullmatch(r"\d+\.\d+\.\d+", fa.fa_version())


def test_workspace_sizes(lib):
    # fp32 row terms D, rounded up to 256 bytes
    assert fa.fa_bwd_workspace_bytes(2, 16, 4096, 128) == 2 * 16 * 4096 * 4
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 64) == 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 65, 128) == 512
    # fp32 partial outputs + fp32 partial lse
    assert fa.fa_decode_workspace_bytes(64, 32, 128, 16) == 64 * 32 * 16 * 128 * 4 + 64 * 32 * 16 * 4
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 3) == 768 + 256
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 0) == 0


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dt=1):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dt, NULL)


def test_fwd_validation(lib):
    for kw in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{kw: NULL}) == ERR["FA_ERR_NULL"]
    assert fwd(lib, dt=2) == ERR["FA_ERR_DTYPE"]
    for kw in ("B", "H", "N"):
        assert fwd(lib, **{kw: 0}) == ERR["FA_ERR_SHAPE"]
        assert fwd(lib, **{kw: -3}) == ERR["FA_ERR_SHAPE"]
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert fwd(lib, scale=bad) == ERR["FA_ERR_SHAPE"]
    for d in (32, 96, 256, 0):
        assert fwd(lib, d=d) == ERR["FA_ERR_UNSUPPORTED"]
    assert fwd(lib, B=1 << 20, H=1 << 10, N=1 << 20) == ERR["FA_ERR_SHAPE"]
    for kw in ("q", "k", "v", "o"):
        assert fwd(lib, **{kw: P_ODD}) == ERR["FA_ERR_ALIGN"]
    assert fwd(lib, lse=P_ODD) == ERR["FA_ERR_ALIGN"]


def bwd(lib, ws=P, ws_bytes=1 << 30, B=1, H=1, N=16, d=64, dt=0, scale=0.125, **ptrs):
    p = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P)
    p.update(ptrs)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"],
                      p["dv"], ws, ws_bytes, B, H, N, d, scale, 1, dt, NULL)


def test_bwd_validation(lib):
    for kw in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(lib, **{kw: NULL}) == ERR["FA_ERR_NULL"]
    assert bwd(lib, dt=7) == ERR["FA_ERR_DTYPE"]
    assert bwd(lib, N=0) == ERR["FA_ERR_SHAPE"]
    assert bwd(lib, d=80) == ERR["FA_ERR_UNSUPPORTED"]
    assert bwd(lib, ws=NULL) == ERR["FA_ERR_WORKSPACE"]
    need = fa.fa_bwd_workspace_bytes(1, 1, 16, 64)
    assert bwd(lib, ws_bytes=need - 1) == ERR["FA_ERR_WORKSPACE"]
    for kw in ("q", "dout", "dq", "dk", "dv"):
        assert bwd(lib, **{kw: P_ODD}) == ERR["FA_ERR_ALIGN"]
    assert bwd(lib, ws=P_ODD) == ERR["FA_ERR_ALIGN"]


def dec(lib, q=P, k=P, v=P, o=P, lse=P, B=2, H=3, Nkv=100, d=128, scale=0.1, splits=4, ws=P,
        ws_bytes=1 << 30, dt=1):
    return lib.fa_decode(q, k, v, o, lse, B, H, Nkv, d, scale, splits, ws, ws_bytes, dt, NULL)


def test_decode_validation(lib):
    for kw in ("q", "k", "v", "o"):
        assert dec(lib, **{kw: NULL}) == ERR["FA_ERR_NULL"]
    assert dec(lib, Nkv=0) == ERR["FA_ERR_SHAPE"]
    assert dec(lib, d=48) == ERR["FA_ERR_UNSUPPORTED"]
    assert dec(lib, dt=-1) == ERR["FA_ERR_DTYPE"]
    assert dec(lib, splits=0) == ERR["FA_ERR_SPLITS"]
    assert dec(lib, splits=fa.FA_MAX_SPLITS + 1) == ERR["FA_ERR_SPLITS"]
    assert dec(lib, ws=NULL) == ERR["FA_ERR_WORKSPACE"]
    need = fa.fa_decode_workspace_bytes(2, 3, 128, 4)
    assert dec(lib, ws_bytes=need - 4) == ERR["FA_ERR_WORKSPACE"]
    assert dec(lib, k=P_ODD) == ERR["FA_ERR_ALIGN"]
    assert dec(lib, lse=P_ODD) == ERR["FA_ERR_ALIGN"]


def fwd_ex(lib, B=1, H=4, H_kv=2, N=16, d=64, causal=1, window=0, **ptrs):
    p = dict(q=P, k=P, v=P, o=P, lse=P)
    p.update(ptrs)
    return lib.fa_fwd_ex(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, H_kv, N, d, 0.125,
                         causal, window, 1, NULL)


def bwd_ex(lib, B=1, H=4, H_kv=2, N=16, d=64, causal=1, window=0, ws_bytes=1 << 30, **ptrs):
    p = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P)
    p.update(ptrs)
    return lib.fa_bwd_ex(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"],
                         p["dv"], p["ws"], ws_bytes, B, H, H_kv, N, d, 0.125, causal, window, 0,
                         NULL)


def dec_ex(lib, B=2, H=8, H_kv=2, Nkv=100, d=128, splits=4, ws_bytes=1 << 30, **ptrs):
    p = dict(q=P, k=P, v=P, o=P, lse=P, ws=P)
    p.update(ptrs)
    return lib.fa_decode_ex(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, H_kv, Nkv, d, 0.1,
                            splits, p["ws"], ws_bytes, 1, NULL)


@pytest.mark.parametrize("call", [fwd_ex, bwd_ex, dec_ex], ids=["fwd_ex", "bwd_ex", "decode_ex"])
def test_grouped_head_validation(lib, call):
    for h_kv in (0, -2, 3, 5):  # 4 (or 8) query heads: not a divisor
        assert call(lib, H_kv=h_kv) == ERR["FA_ERR_SHAPE"]
    assert call(lib, q=NULL) == ERR["FA_ERR_NULL"]
    assert call(lib, k=P_ODD) == ERR["FA_ERR_ALIGN"]


@pytest.mark.parametrize("call", [fwd_ex, bwd_ex], ids=["fwd_ex", "bwd_ex"])
def test_window_validation(lib, call):
    assert call(lib, window=-1) == ERR["FA_ERR_SHAPE"]
    assert call(lib, window=4, causal=0) == ERR["FA_ERR_UNSUPPORTED"]
    assert call(lib, d=96, window=4) == ERR["FA_ERR_UNSUPPORTED"]


def test_decode_varlen_validation(lib):
    def call(kv_lens=P, **kw):
        a = dict(B=2, H=8, H_kv=2, Nkv=100, d=128, splits=4)
        a.update(kw)
        return lib.fa_decode_varlen(P, P, P, kv_lens, P, P, a["B"], a["H"], a["H_kv"], a["Nkv"],
                                    a["d"], 0.1, a["splits"], P, 1 << 30, 1, NULL)
    assert call(kv_lens=NULL) == ERR["FA_ERR_NULL"]
    assert call(kv_lens=P_ODD) == ERR["FA_ERR_ALIGN"]
    assert call(H_kv=3) == ERR["FA_ERR_SHAPE"]
    assert call(splits=0) == ERR["FA_ERR_SPLITS"]
    assert call(d=32) == ERR["FA_ERR_UNSUPPORTED"]


def test_decode_noalloc_validation(lib):
    """Checks run before any HIP call: a call needing more than the static scratch is refused
    with FA_ERR_SCRATCH; the other checks are fa_decode_ex's."""
    def call(q=P, k=P, v=P, o=P, lse=P, B=2, H=8, H_kv=2, Nkv=100, d=128, splits=4, dt=1):
        return lib.fa_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Nkv, d, 0.1, splits, dt, NULL)
    for kw in ("q", "k", "v", "o"):
        assert call(**{kw: NULL}) == ERR["FA_ERR_NULL"]
    assert call(H_kv=3) == ERR["FA_ERR_SHAPE"]
    assert call(splits=0) == ERR["FA_ERR_SPLITS"]
    assert call(d=80) == ERR["FA_ERR_UNSUPPORTED"]
    assert call(dt=5) == ERR["FA_ERR_DTYPE"]
    assert call(o=P_ODD) == ERR["FA_ERR_ALIGN"]
    # 64 x 64 heads x 32 chunks x (128 + 1) floats = 64.5 MiB > 32 MiB
    assert fa.fa_decode_workspace_bytes(64, 64, 128, 32) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert call(B=64, H=64, H_kv=64, splits=32) == ERR["FA_ERR_SCRATCH"]
    # the decode of the B64 H32 d128 16-chunk workload fits
    assert fa.fa_decode_workspace_bytes(64, 32, 128, 16) <= fa.FA_NOALLOC_SCRATCH_BYTES
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_probe_library_exports_every_declared_function():
    from exact_io_aware_31_amd import probe
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == ["fa_probe_mfma_bf16", "fa_probe_stream_read"]
    plib = probe.load_library()
    for n in names:
        assert hasattr(plib, n), f"{n} declared in include/fa_probe.h but not exported"
    # argument checks happen before any launch
    assert plib.fa_probe_mfma_bf16(NULL, P, 1, 1, NULL) == 1
    assert plib.fa_probe_mfma_bf16(P, P, 0, 1, NULL) == 2
    assert plib.fa_probe_stream_read(P, probe.READ_CHUNK + 16, P, 1, NULL) == 2
    assert plib.fa_probe_stream_read(P_ODD, probe.READ_CHUNK, P, 1, NULL) == 4


def test_bwd_ex_workspace_is_per_query_head(lib):
    need = fa.fa_bwd_workspace_bytes(1, 4, 16, 64)
    assert bwd_ex(lib, ws=NULL) == ERR["FA_ERR_WORKSPACE"]
    assert bwd_ex(lib, ws_bytes=need - 1) == ERR["FA_ERR_WORKSPACE"]
    need = fa.fa_decode_workspace_bytes(2, 8, 128, 4)
    assert dec_ex(lib, ws_bytes=need - 4) == ERR["FA_ERR_WORKSPACE"]


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)
    with pytest.raises(ValueError):
        fa.attention_fwd(q, q, q)
    with pytest.raises(ValueError):
        fa.fa_fwd(q.float(), q, q, q, torch.zeros(1, 1, 16), 0.1, False)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        fa.load_library(str(tmp_path / "libfa.so"))


def test_header_is_plain_c_and_callable_from_c(tmp_path):
    """include/fa.h compiles as strict C99 and the validation paths answer a C caller."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this machine")
    lib_dir = os.path.dirname(fa.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    build = subprocess.run(
        [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
         "-L", lib_dir, "-lfa", f"-Wl,-rpath,{lib_dir}", "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout
