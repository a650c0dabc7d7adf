"""The C ABI without a GPU: symbols, status strings and host-side validation.

Every call here is rejected (or sized) on the host before any HIP call, so
these tests run on a machine with no GPU.  No call here launches a kernel.
"""
import ctypes
import os
import re

import pytest

import exact_io_aware_65_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

# fake device addresses: never dereferenced, because validation rejects every call
A = 1 << 32
B_ = 2 << 32
C = 3 << 32
O = 4 << 32
L = 5 << 32
W = 6 << 32
DO_ = 7 << 32
GQ = 8 << 32
GK = 9 << 32
GV = 10 << 32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "fa_bwd", "fa_bwd_workspace_size", "fa_decode", "fa_decode_num_splits", "fa_decode_paged",
        "fa_decode_noalloc", "fa_decode_workspace_size", "fa_fwd", "fa_fwd_fp8", "fa_quantize_e4m3", "fa_last_error",
        "fa_status_str", "fa_version"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert hasattr(fa, name), f"binding lacks {name}"


def test_version_and_status_strings():
    assert fa.fa_version() == 5
    assert [fa.fa_status_str(s) for s in range(5)] == [
        "FA_OK", "FA_ERR_INVALID", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP"]
    assert fa.fa_status_str(99) == "FA_ERR_UNKNOWN"


def status_of(fn, *args):
    try:
        fn(*args)
    except fa.FaError as e:
        return e.status, fa.fa_last_error()
    return fa.FA_OK, ""


def fwd(q=A, k=B_, v=C, o=O, lse=L, B=1, H=2, Nq=64, Nkv=64, d=128, causal=0, scale=0.125, dtype=fa.FA_F16):
    return status_of(fa.fa_fwd, q, k, v, o, lse, B, H, Nq, Nkv, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(o=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED, "d=96"),
    (dict(d=0), fa.FA_ERR_INVALID, "positive"),
    (dict(dtype=3), fa.FA_ERR_INVALID, "dtype"),
    (dict(dtype=fa.FA_F16 | 0x200), fa.FA_ERR_INVALID, "dtype"),
    (dict(causal=1, Nq=65, Nkv=64), fa.FA_ERR_INVALID, "Nq <= Nkv"),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID, "finite"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID, "finite"),
    (dict(Nkv=0), fa.FA_ERR_INVALID, "no keys"),
    (dict(B=-1), fa.FA_ERR_INVALID, "negative"),
    (dict(q=A + 8), fa.FA_ERR_INVALID, "aligned"),
    (dict(lse=L + 2), fa.FA_ERR_INVALID, "aligned"),
    (dict(o=A), fa.FA_ERR_INVALID, "o overlaps q"),
    (dict(o=A + 1024 * 16), fa.FA_ERR_INVALID, "o overlaps q"),
    (dict(lse=C), fa.FA_ERR_INVALID, "lse overlaps v"),
    (dict(lse=O + 16), fa.FA_ERR_INVALID, "lse overlaps o"),
    (dict(B=1 << 20, H=1 << 20, Nq=1 << 20, Nkv=1 << 20), fa.FA_ERR_INVALID, "2^62"),
    (dict(B=1, H=1, Nq=64, Nkv=1 << 24, o=A + (1 << 31)), fa.FA_ERR_UNSUPPORTED, "4 GiB"),
])
def test_fwd_rejects(kw, status, needle):
    got, msg = fwd(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def fwd8(q=A, k=B_, v=C, o=O, lse=L, B=1, H=2, Nq=64, Nkv=64, d=128, causal=0, scale=0.125, dtype=fa.FA_F16):
    return status_of(fa.fa_fwd_fp8, q, k, v, o, lse, B, H, Nq, Nkv, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(k=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED, "d=32"),
    (dict(dtype=4), fa.FA_ERR_INVALID, "dtype"),
    (dict(causal=1, Nq=65, Nkv=64), fa.FA_ERR_INVALID, "Nq <= Nkv"),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID, "finite"),
    (dict(Nkv=0), fa.FA_ERR_INVALID, "no keys"),
    (dict(k=B_ + 8), fa.FA_ERR_INVALID, "aligned"),
    # k8 holds one byte per element: its last 16 of 2*64*128 bytes
    (dict(o=B_ + 2 * 64 * 128 - 16), fa.FA_ERR_INVALID, "o overlaps k"),
    (dict(lse=C + 64), fa.FA_ERR_INVALID, "lse overlaps v"),
])
def test_fwd_fp8_rejects(kw, status, needle):
    got, msg = fwd8(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def test_fwd_fp8_empty_is_noop():
    assert fwd8(Nq=0, q=None, k=None, v=None, o=None, lse=None)[0] == fa.FA_OK


@pytest.mark.parametrize("args,status,needle", [
    ((A, B_, 100, 3), fa.FA_ERR_INVALID, "dtype"),
    ((A, B_, 100, fa.FA_F16 | fa.FA_OUT_F32), fa.FA_ERR_INVALID, "dtype"),
    ((None, B_, 100, fa.FA_F16), fa.FA_ERR_INVALID, "non-NULL"),
    ((A, B_ + 8, 100, fa.FA_F16), fa.FA_ERR_INVALID, "aligned"),
    ((A, A + 192, 100, fa.FA_BF16), fa.FA_ERR_INVALID, "overlaps"),
])
def test_quantize_rejects(args, status, needle):
    got, msg = status_of(fa.fa_quantize_e4m3, *args, None)
    assert got == status, (got, msg)
    assert needle in msg, msg
    assert status_of(fa.fa_quantize_e4m3, None, None, 0, fa.FA_F16, None)[0] == fa.FA_OK


def test_fwd_empty_is_noop():
    # nothing to compute: OK without touching the (null) pointers or the GPU
    assert fwd(q=None, k=None, v=None, o=None, lse=None, Nq=0)[0] == fa.FA_OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, B=0)[0] == fa.FA_OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, H=0)[0] == fa.FA_OK


def dec(q=A, k=B_, v=C, o=O, lse=L, B=2, H=2, Nkv=1000, d=128, scale=0.1, dtype=fa.FA_F16, splits=0,
        ws=W, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = fa.fa_decode_workspace_size(B, H, Nkv, d, splits)
    return status_of(fa.fa_decode, q, k, v, o, lse, B, H, Nkv, d, scale, dtype, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(d=80), fa.FA_ERR_UNSUPPORTED, "d=80"),
    (dict(Nkv=0), fa.FA_ERR_INVALID, "no keys"),
    (dict(splits=-1), fa.FA_ERR_INVALID, "num_splits"),
    (dict(ws=None), fa.FA_ERR_WORKSPACE, "workspace"),
    (dict(ws=W + 4), fa.FA_ERR_WORKSPACE, "aligned"),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE, "hold"),
    (dict(ws=B_), fa.FA_ERR_WORKSPACE, "workspace overlaps k"),
    (dict(v=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(dtype=0), fa.FA_ERR_INVALID, "dtype"),
])
def test_decode_rejects(kw, status, needle):
    got, msg = dec(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def dec_noalloc(q=A, k=B_, v=C, o=O, lse=L, B=2, H=2, Nkv=1000, d=128, scale=0.1, dtype=fa.FA_F16, splits=0):
    return status_of(fa.fa_decode_noalloc, q, k, v, o, lse, B, H, Nkv, d, scale, dtype, splits, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(d=80), fa.FA_ERR_UNSUPPORTED, "d=80"),
    (dict(Nkv=0), fa.FA_ERR_INVALID, "no keys"),
    (dict(splits=-1), fa.FA_ERR_INVALID, "num_splits"),
    (dict(o=B_), fa.FA_ERR_INVALID, "o overlaps k"),
    (dict(dtype=0), fa.FA_ERR_INVALID, "dtype"),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID, "finite"),
    # 512 heads x 64 splits x (128 + 1) floats = 16.9 MB of partials > the 4 MiB scratch
    (dict(B=16, H=32, Nkv=32768, splits=64), fa.FA_ERR_WORKSPACE, "device scratch"),
])
def test_decode_noalloc_rejects(kw, status, needle):
    got, msg = dec_noalloc(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def test_decode_noalloc_scratch_bound():
    # every automatic split count up to 2048 heads fits the scratch at d = 128
    for bh in (1, 7, 64, 512, 513, 700, 1024, 2048):
        need = fa.fa_decode_workspace_size(1, bh, 1 << 20, 128, 0)
        assert 0 < need <= fa.FA_DECODE_NOALLOC_SCRATCH_BYTES, (bh, need)
    assert dec_noalloc(B=0, q=None, k=None, v=None, o=None, lse=None)[0] == fa.FA_OK


TB = 11 << 32
SL = 12 << 32


def paged(q=A, kp=B_, vp=C, table=TB, lens=SL, o=O, lse=L, B=2, H=2, d=128, num_pages=64, page_size=16,
          max_pages=32, layout=fa.FA_PAGED_HND, max_seq_len=None, scale=0.1, dtype=fa.FA_F16, splits=0, ws=W,
          ws_bytes=None):
    if max_seq_len is None:
        max_seq_len = max_pages * page_size
    if ws_bytes is None:
        ws_bytes = fa.fa_decode_workspace_size(B, H, max(max_seq_len, 1), d, splits)
    return status_of(fa.fa_decode_paged, q, kp, vp, table, lens, o, lse, B, H, d, num_pages, page_size, max_pages,
                     layout, max_seq_len, scale, dtype, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED, "d=96"),
    (dict(dtype=5), fa.FA_ERR_INVALID, "dtype"),
    (dict(page_size=0), fa.FA_ERR_INVALID, "page_size"),
    (dict(layout=2), fa.FA_ERR_INVALID, "layout"),
    (dict(num_pages=-1), fa.FA_ERR_INVALID, "negative"),
    (dict(num_pages=0), fa.FA_ERR_INVALID, "pool is empty"),
    (dict(max_seq_len=0), fa.FA_ERR_INVALID, "max_seq_len"),
    (dict(max_seq_len=32 * 16 + 1), fa.FA_ERR_INVALID, "max_seq_len"),
    (dict(max_pages=1 << 20, page_size=1 << 11, max_seq_len=100), fa.FA_ERR_INVALID, "2^31"),
    (dict(splits=-2), fa.FA_ERR_INVALID, "num_splits"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID, "finite"),
    (dict(table=None), fa.FA_ERR_INVALID, "block_table"),
    (dict(lens=SL + 2), fa.FA_ERR_INVALID, "4-byte"),
    (dict(kp=B_ + 8), fa.FA_ERR_INVALID, "16-byte"),
    (dict(o=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(lse=L + 1), fa.FA_ERR_INVALID, "aligned"),
    (dict(o=B_ + 4096), fa.FA_ERR_INVALID, "o overlaps k_pages"),
    (dict(lse=TB), fa.FA_ERR_INVALID, "lse overlaps block_table"),
    (dict(lse=O), fa.FA_ERR_INVALID, "lse overlaps o"),
    (dict(ws=None), fa.FA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=64), fa.FA_ERR_WORKSPACE, "hold"),
    (dict(ws=SL - 64), fa.FA_ERR_WORKSPACE, "workspace overlaps seq_lens"),
])
def test_decode_paged_rejects(kw, status, needle):
    got, msg = paged(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def test_decode_paged_empty_is_noop():
    assert paged(B=0, q=None, kp=None, vp=None, table=None, lens=None, o=None, lse=None, ws=None,
                 ws_bytes=0)[0] == fa.FA_OK
    assert paged(H=0, q=None, kp=None, vp=None, table=None, lens=None, o=None, lse=None, ws=None,
                 ws_bytes=0)[0] == fa.FA_OK


def test_decode_sizes():
    # workspace = B*H*splits*(d+1) fp32; splits clamp to Nkv and never leave a split empty
    assert fa.fa_decode_workspace_size(2, 3, 1000, 128, 4) == 2 * 3 * 4 * 129 * 4
    assert fa.fa_decode_workspace_size(1, 1, 5, 64, 16) == 1 * 1 * 5 * 65 * 4
    # 10 keys in 4 requested splits: chunks of 3 -> 4 splits (3,3,3,1)
    assert fa.fa_decode_workspace_size(1, 1, 10, 64, 4) == 4 * 65 * 4
    # 10 keys in 6 requested splits: chunks of 2 -> 5 splits
    assert fa.fa_decode_workspace_size(1, 1, 10, 64, 6) == 5 * 65 * 4
    assert fa.fa_decode_workspace_size(1, 1, 0, 64, 0) == 0
    assert fa.fa_decode_workspace_size(1, 1, 10, 96, 0) == 0
    s = fa.fa_decode_num_splits(16, 32, 32768, 128)
    assert 1 <= s <= 256
    assert fa.fa_decode_workspace_size(16, 32, 32768, 128, 0) == 16 * 32 * s * 129 * 4
    assert fa.fa_decode_num_splits(1, 1, 1, 128) == 1
    assert dec(B=0, q=None, k=None, v=None, o=None, lse=None, ws=None, ws_bytes=0)[0] == fa.FA_OK


def test_last_error_is_empty_in_a_new_thread():
    import threading
    fwd(d=96)
    seen = {}

    def other():
        seen["msg"] = fa.fa_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "d=96" in fa.fa_last_error()


def bwd(q=A, k=B_, v=C, o=O, dout=DO_, lse=L, dq=GQ, dk=GK, dv=GV, B=1, H=2, Nq=64, Nkv=96, d=128, causal=1,
        scale=0.125, dtype=fa.FA_F16, ws=W, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(B, H, Nq)
    return status_of(fa.fa_bwd, q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, causal, scale, dtype, ws,
                     ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dout=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(dk=None), fa.FA_ERR_INVALID, "non-NULL"),
    (dict(lse=None), fa.FA_ERR_INVALID, "lse"),
    (dict(o=O + 8), fa.FA_ERR_INVALID, "aligned"),
    (dict(dv=GV + 4), fa.FA_ERR_INVALID, "aligned"),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED, "d=32"),
    (dict(dtype=4), fa.FA_ERR_INVALID, "dtype"),
    (dict(causal=1, Nq=97), fa.FA_ERR_INVALID, "Nq <= Nkv"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID, "finite"),
    (dict(Nkv=0), fa.FA_ERR_INVALID, "no keys"),
    (dict(H=-2), fa.FA_ERR_INVALID, "negative"),
    (dict(dq=A), fa.FA_ERR_INVALID, "dq overlaps q"),
    (dict(dk=DO_ + 64), fa.FA_ERR_INVALID, "dk overlaps dout"),
    (dict(dv=GK + 128, dtype=fa.FA_F16 | fa.FA_OUT_F32), fa.FA_ERR_INVALID, "dk overlaps dv"),
    (dict(dq=L), fa.FA_ERR_INVALID, "dq overlaps lse"),
    (dict(ws=None), fa.FA_ERR_WORKSPACE, "workspace"),
    (dict(ws=W + 8), fa.FA_ERR_WORKSPACE, "aligned"),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE, "hold"),
    (dict(ws=GV), fa.FA_ERR_WORKSPACE, "workspace overlaps dv"),
    (dict(B=1, H=1, Nq=64, Nkv=1 << 24, dtype=fa.FA_F16 | fa.FA_OUT_F32), fa.FA_ERR_UNSUPPORTED, "4 GiB"),
])
def test_bwd_rejects(kw, status, needle):
    got, msg = bwd(**kw)
    assert got == status, (got, msg)
    assert needle in msg, msg


def test_bwd_sizes_and_empty():
    # two fp32 values per query row
    assert fa.fa_bwd_workspace_size(2, 3, 100) == 2 * 3 * 100 * 2 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 0) == 0
    assert fa.fa_bwd_workspace_size(-1, 1, 4) == 0
    assert bwd(B=0, q=None, k=None, v=None, o=None, dout=None, lse=None, dq=None, dk=None, dv=None, ws=None,
               ws_bytes=0)[0] == fa.FA_OK


def test_abi_from_c(tmp_path):
    # the header is plain C: a C99 program includes it, links the library and
    # makes the calls that need no GPU
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(fa.LIBRARY)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", libdir, "-lfa355",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_last_error_is_per_thread_under_contention():
    # each thread sees the message of its own last failing call
    import threading
    results = {}

    def worker(d):
        for _ in range(200):
            got, msg = fwd(d=d)
            if f"d={d}" not in msg:
                results[d] = msg
                return
        results[d] = "ok"

    threads = [threading.Thread(target=worker, args=(d,)) for d in (80, 96, 112, 160)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(v == "ok" for v in results.values()), results


def test_read_probe_library():
    # the streaming-read probe bench.py reports decode against: built beside
    # the library, exporting its two calls; bad arguments fail before any launch
    import ctypes

    from exact_io_aware_65_amd import build as libbuild
    lib = ctypes.CDLL(libbuild.PROBE_LIBRARY)
    lib.fa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.fa_probe_read_blocks() == 2048
    assert lib.fa_probe_read(None, 1 << 20, 0x1000, None) == 1
    assert lib.fa_probe_read(0x1000, 1000, 0x1000, None) == 1   # not a multiple of 16
    assert lib.fa_probe_read(0x1008, 1 << 20, 0x1000, None) == 1  # misaligned


def test_abi_validation_under_sanitizers(tmp_path):
    # the ABI layer (fa_abi.cpp) built for the host with g++ under
    # AddressSanitizer and UndefinedBehaviorSanitizer, against stub launchers:
    # every entry point, valid calls and each class of invalid argument,
    # including sizes at INT_MAX that exercise the overflow guards
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(os.path.dirname(here), "exact_io_aware_65_amd", "csrc")
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(os.path.dirname(here), "include"), "-I", csrc,
                    os.path.join(here, "c", "abi_sanitize.cpp"), os.path.join(here, "c", "abi_sanitize_stubs.cpp"),
                    os.path.join(csrc, "fa_abi.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ran clean" in r.stdout
