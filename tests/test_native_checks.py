"""Native-code checks on the host (no GPU, no compute on a device).

1. Sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer):
   * the CPU oracle, built with gcc and driven by tests/sanitize/oracle_driver.c
     on exact-size buffers (ragged K and N, row subsets, the empty and
     degenerate cases, the argument errors), each result also compared with a
     direct per-element evaluation of the definition;
   * the library's host side — the selector, the plan and workspace
     arithmetic, the instance descriptions, the status strings and the
     argument checks of the entry points — built with the sanitizers on the
     host code only (`-Xarch_host -fsanitize=...`; the device code is compiled
     as for the library) and driven by tests/sanitize/api_driver.cpp.
2. The direct-to-LDS copies are written as inline asm, where the compiler
   inserts no wait states, so the asm pads its own.  The same compile keeps the
   gfx950 assembly of the kernels (-save-temps); every LDS-DMA instruction in it
   must come right after the m0 write that gives its LDS destination and an
   `s_nop 4`: one wait state is required between a scalar write of m0 and an
   LDS-DMA load reading it, five between a VALU write of an SGPR (the copies'
   buffer descriptors are built with v_readfirstlane) and a vector-memory
   instruction reading it.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from fp8_block_scaled_a8w8_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ("a8w8_api", "a8w8_kernels", "a8w8_quant", "a8w8_prepack")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _tool(path, name):
    for c in (path, shutil.which(name)):
        if c and os.path.exists(c):
            return c
    pytest.skip(f"{name} not available")


@pytest.fixture(scope="module")
def native_build():
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="a8w8_native_")
    flags = [f for f in build.HIPCC_FLAGS if f != "-shared"]
    procs = []
    for src in SOURCES:
        cmd = [hipcc, *flags, "-g", "-save-temps", *SAN_HOST, "-I", os.path.join(build.ROOT, "include"),
               "-I", os.path.join(build.HERE, "csrc"), "-c", os.path.join(build.HERE, "csrc", src + ".hip"),
               "-o", os.path.join(d, src + ".o")]
        procs.append((src, subprocess.Popen(cmd, cwd=d, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{src}: {out[-2000:]}"
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_under_sanitizers(tmp_path):
    gcc = _tool(None, "gcc")
    exe = str(tmp_path / "oracle_san")
    cmd = [gcc, "-g", "-O1", "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(build.ROOT, "oracle", "a8w8_oracle.c"),
           os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout


def test_host_api_under_sanitizers(native_build):
    clang = _tool("/opt/rocm/llvm/bin/clang++", "clang++")
    d = native_build
    drv = os.path.join(d, "api_driver.o")
    res = subprocess.run([clang, "-g", "-O1", "-std=c++17", "-fsanitize=address,undefined",
                          "-fno-sanitize-recover=all", "-I", os.path.join(build.ROOT, "include"), "-c",
                          os.path.join(HERE, "sanitize", "api_driver.cpp"), "-o", drv], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    exe = os.path.join(d, "api_san")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(build.hipcc())), "lib")
    res = subprocess.run([clang, "-fsanitize=address,undefined", *[os.path.join(d, s + ".o") for s in SOURCES], drv,
                          "-L", rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout


DMA = re.compile(r"^\s*(buffer_load_dword\w*\s.*\blds\b|global_load_lds_dword\w*\s)")


def _check_dma_padding(path, at_least):
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.strip() and not ln.strip().startswith(";")]
    n = 0
    for i, ln in enumerate(lines):
        if not DMA.match(ln):
            continue
        n += 1
        prev2, prev1 = lines[i - 2].strip(), lines[i - 1].strip()
        assert prev1 == "s_nop 4", (i, prev2, prev1, ln)
        assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", prev2), (i, prev2, prev1, ln)
    assert n >= at_least, f"only {n} LDS-DMA copies found"


def test_every_lds_dma_copy_is_padded_after_its_m0_write(native_build):
    _check_dma_padding(os.path.join(native_build, "a8w8_kernels-hip-amdgcn-amd-amdhsa-gfx950.s"), 1000)


def test_capacity_probe_copies_are_padded(tmp_path):
    """The per-CU capacity probe (a measurement aid the benchmark runs) uses the same copy form."""
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in build.HIPCC_FLAGS if f != "-shared"]
    cmd = [hipcc, *flags, "-save-temps", "-c", os.path.join(build.HERE, "csrc", "cu_capacity.hip"),
           "-o", str(tmp_path / "cu_capacity.o")]
    res = subprocess.run(cmd, cwd=tmp_path, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    _check_dma_padding(str(tmp_path / "cu_capacity-hip-amdgcn-amd-amdhsa-gfx950.s"), 8)
