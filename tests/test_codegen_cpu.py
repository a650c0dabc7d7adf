"""Checks on the code hipcc emits for gfx950 (CPU only: cross-compilation, no GPU).

The half-wave exchange in the prefill kernel relies on both results of the
permlane32 swap; an earlier form of the helper (a bit cast applied directly to
a vector element) was lowered by clang as two reads of the first result.

The prefill ring relies on the kernel being spill-free: a scratch reload makes
the compiler wait for all outstanding vector-memory operations (vmcnt(0)),
which includes every in-flight K/V tile load.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_65_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def device_ir(src, tmp_path):
    out = tmp_path / "k.ll"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-x", "hip", "-S", "--cuda-device-only", "-emit-llvm",
                    os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def test_permlane_swap_uses_both_results(tmp_path):
    ir = device_ir("fa_fwd.hip", tmp_path)
    calls = re.findall(r"(%\d+) = tail call \{ i32, i32 \} @llvm\.amdgcn\.permlane32\.swap", ir)
    assert calls, "prefill kernel no longer uses permlane32.swap"
    for v in calls:
        assert re.search(rf"extractvalue \{{ i32, i32 \}} {v}, 0", ir), v
        assert re.search(rf"extractvalue \{{ i32, i32 \}} {v}, 1", ir), f"second result of {v} unused"


def test_no_packed_fp32_arithmetic(tmp_path):
    # packed fp32 add/mul/fma are kept out of the kernels
    asm = tmp_path / "k.s"
    for src in ("fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip"):
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-I", os.path.join(ROOT, "include"),
                        "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip",
                        "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", str(asm)],
                       check=True, capture_output=True)
        text = asm.read_text()
        for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
            assert op not in text, f"{op} in {src}"


def kernel_metadata(src, tmp_path):
    asm = tmp_path / (src + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip",
                    "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", str(asm)],
                   check=True, capture_output=True)
    text = asm.read_text().split("amdhsa.kernels:", 1)[1]
    kernels = []
    for block in re.split(r"\n\s+- \.", text)[1:]:
        fields = dict(re.findall(r"\.(\w+):\s+(\S+)", "." + block))
        if "name" in fields and "vgpr_spill_count" in fields:  # kernel entries, not argument entries
            kernels.append(fields)
    return kernels


# Every kernel leaves room for two waves per SIMD (256 of the 512 registers).


@pytest.mark.parametrize("src", ["fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip"])
def test_kernels_do_not_spill(src, tmp_path):
    kernels = kernel_metadata(src, tmp_path)
    assert kernels, f"no kernels found in {src}"
    for k in kernels:
        assert int(k["vgpr_spill_count"]) == 0, f"{k['name']} spills {k['vgpr_spill_count']} VGPRs"
        assert int(k["private_segment_fixed_size"]) == 0, f"{k['name']} uses scratch"
        assert int(k["vgpr_count"]) <= 256, f"{k['name']}: {k['vgpr_count']} registers"


def device_asm(src, tmp_path):
    asm = tmp_path / (src + ".hazard.s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip",
                    "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", str(asm)],
                   check=True, capture_output=True)
    return asm.read_text()


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("src", ["fa_fwd.hip", "fa_bwd.hip"])
def test_lds_dma_loads_are_padded_after_valu_sgpr_writes(src, tmp_path):
    # The direct-to-LDS loads are inline asm, which the compiler's hazard
    # pass does not look into.  When it runs short of SGPRs it reloads the
    # buffer descriptor from a spill lane with v_readlane right before such a
    # load, and a VMEM read of an SGPR written by VALU needs 5 wait states;
    # without them the load may use a stale descriptor (loads from the wrong
    # tensor or a wild address).  Every such load must be at least 5 wait
    # states after any VALU write of its SGPR operands.
    lines = [ln.split(";")[0].strip() for ln in device_asm(src, tmp_path).splitlines()]
    loads = bad = 0
    for n, ln in enumerate(lines):
        if not (ln.startswith("buffer_load") and " lds" in ln):
            continue
        loads += 1
        ops = [t.strip() for t in ln.split(None, 1)[1].split(",")]
        regs = _sgprs(ops[1]) | _sgprs(ops[2].split()[0])
        waits, k = 0, n - 1
        while k >= 0 and waits < 5:
            prev = lines[k]
            k -= 1
            if not prev or prev.startswith(".") or prev.endswith(":"):
                continue
            m = re.match(r"s_nop (\d+)", prev)
            if m:
                waits += int(m.group(1)) + 1
                continue
            w = re.match(r"v_(?:readlane|readfirstlane)_b32 (s\d+)|v_cmp\S* (s\[\d+:\d+\])", prev)
            if w and _sgprs(w.group(1) or w.group(2)) & regs:
                bad += 1
                break
            waits += 1
    assert loads > 0, f"no direct-to-LDS loads found in {src}"
    assert bad == 0, f"{bad} of {loads} direct-to-LDS loads in {src} follow a VALU write of their SGPRs too closely"
