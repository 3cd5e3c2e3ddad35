"""Bounds check of the 256x256 expert GEMM without a GPU.

The kernel source (top_routed_expert_amd/csrc/grouped_gemm_big8.hip) is
turned into host C++: HIP keywords and builtins become plain functions (tests/emul/
shim.h), the inline-asm LDS reads become checked reads, the kernel launches
become loops that run every lane of every block in turn. tests/emul/driver.cpp
builds the launch arguments the way the library does, with exact-size buffers,
and the whole thing runs under AddressSanitizer: any global load, store or
table read outside its buffer, or any LDS access outside its array, fails the
run. The matrix-core arithmetic is not emulated (the GPU parity tests cover the
values); this test covers the index arithmetic, at shapes that take the
multi-item hand-over, the chunked order of multi-tile groups, odd A-stage counts
and the shortest contraction the kernel accepts.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from emul_source import big8_source, clang as _clang, compile_cmd, internal_header, read


def host_source(kernel_src: str) -> str:
    return big8_source(kernel_src)


def kernel_source() -> str:
    return read("grouped_gemm_big8.hip")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cc = _clang()
    if cc is None:
        pytest.skip("clang++ with AddressSanitizer is needed")
    d = tmp_path_factory.mktemp("emul")
    open(d / "emul_internal.h", "w").write(internal_header())
    open(d / "emul_big.cpp", "w").write(host_source(kernel_source()))
    exe = d / "driver"
    r = subprocess.run(compile_cmd(cc, d, "driver.cpp", exe), capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("no AddressSanitizer runtime for the host compiler")
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


SHAPES = {
    # several items per block for gate/up, the shortest contraction (128) and three A stages (192)
    "multi_item_short_k": (32768, 8, 2, 128, 192, 192, 2, 0),
    # an odd number of A stages in the down projection (320 = 5 x 64)
    "odd_a_stages": (600, 8, 2, 512, 320, 320, 3, 0),
    # hot experts with many row tiles (chunked order), many experts
    "skewed": (4096, 64, 8, 512, 256, 256, 4, 1),
    # the decode/prefill widths with fewer tokens
    "wide": (512, 16, 8, 4096, 1280, 1280, 5, 0),
    # 141 mean rows per group: the form that skips the empty half of an item
    "sparse_items": (800, 16, 2, 256, 256, 256, 6, 0),
    "fp8_sparse_items": (800, 16, 2, 256, 256, 256, 6, 0, 1),
    # fp8 weights (64-element weight stages, per-column scales): short and odd contractions, several items
    "fp8_multi_item_short_k": (32768, 8, 2, 128, 192, 192, 2, 0, 1),
    "fp8_odd_stages_skewed": (4096, 64, 8, 512, 320, 320, 4, 1, 1),
    "fp8_wide": (512, 16, 8, 4096, 1280, 1280, 5, 0, 1),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_big_gemm_accesses_stay_in_bounds(driver, name):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([driver, *map(str, SHAPES[name])], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.count(" ok") == (2 if name.startswith("fp8") else 4), r.stdout


def test_planted_offset_is_caught(driver, tmp_path):
    """The check itself: an A row offset one row too far must be reported."""
    src = kernel_source()
    planted = src.replace("aoff[i] = (uint32_t)rows[i] * (uint32_t)(Kdim >> 3)",
                          "aoff[i] = (uint32_t)(rows[i] + 1) * (uint32_t)(Kdim >> 3)")
    assert planted != src
    d = os.path.dirname(driver)
    work = tmp_path / "planted"
    work.mkdir()
    shutil.copy(os.path.join(d, "emul_internal.h"), work / "emul_internal.h")
    open(work / "emul_big.cpp", "w").write(host_source(planted))
    exe = work / "driver"
    r = subprocess.run(compile_cmd(_clang(), work, "driver.cpp", exe), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(exe), "600", "8", "2", "512", "320", "320", "3"], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
