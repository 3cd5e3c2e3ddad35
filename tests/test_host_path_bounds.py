"""Bounds check of the library's own host path without a GPU.

tests/emul/host_path.cpp compiles the C ABI (csrc/api.hip) for the host, with
every kernel it launches turned into host C++ (tests/emul_source.py, runner in
tests/emul/runner.h), and calls the entry points with exact-size host buffers
under AddressSanitizer: the argument checks, workspace carving, tile schedules
and launch arguments are the library's own, and every lane of every block of
every kernel runs, so any access outside a caller buffer, the workspace or an
LDS array fails the run. Matrix-core results are not computed (bf16 logits
come out zero, so a router bias spreads the choices); fp32 layers compute real
values through the generic GEMM, so their routing is the real one.

Scenarios:
  halves  the standalone expert halves with the layer's arguments (E routed
          groups + the shared expert as one more group: offsets of E+2
          entries, gather of T*K rows, n_rows = T*K + T), preceded by the
          permutation kernels, and the grouped FFN over the routed rows and
          over the shared expert alone;
  layer   moe_layer_forward, moe_layer_forward_dynamic and
          moe_layer_forward_noalloc with weights converted by the library's
          own packer or fp8 quantiser.
The prefill-shaped halves (8192 tokens, d_model 4096, width 1280, 288
experts) take about twenty minutes of host time; they run when
MOE_EMUL_PREFILL=1 is set (see test_halves_at_the_prefill_shape).
"""
from __future__ import annotations

import os
import subprocess

import pytest

import emul_source as ES


@pytest.fixture(scope="module")
def host_path(tmp_path_factory):
    cc = ES.clang()
    if cc is None:
        pytest.skip("clang++ with AddressSanitizer is needed")
    d = tmp_path_factory.mktemp("host_path")
    ES.write_tree(str(d))
    exe = d / "host_path"
    r = subprocess.run(ES.compile_cmd(cc, d, "host_path.cpp", exe), capture_output=True, text=True, timeout=600)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("no AddressSanitizer runtime for the host compiler")
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


def calls_ok(out: str) -> int:
    """Entry-point calls reported ok by the driver."""
    return sum(1 for l in out.splitlines() if l.startswith("  moe_") and l.rstrip().endswith(" ok"))


def run(exe, *args, timeout=900):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-4000:])
    assert "all calls ok" in r.stdout, r.stdout
    return r.stdout


HALVES = {
    # the decode/prefill widths, 256-row tiles, permutation through its rank/place kernels
    "wide_256_row_tiles": (512, 16, 8, 4096, 1280, 5, 0, 1, 0),
    # hot experts spanning many 256-row tiles (chunked row-tile order), row-major weights
    "skewed_many_tiles_rows": (4096, 64, 8, 512, 256, 4, 1, 0, 0),
    # 141 mean rows per group: the 256x256 kernel's form that skips empty half items
    "sparse_items": (800, 16, 2, 256, 256, 6, 0, 1, 0),
    # few rows per expert: 32- and 64-row tiles of the other GEMM family
    "few_rows_small_tiles": (40, 32, 8, 512, 256, 7, 0, 1, 0),
}


@pytest.mark.parametrize("name", list(HALVES))
def test_halves_in_bounds(host_path, name):
    out = run(host_path, "halves", *HALVES[name])
    assert calls_ok(out) == 6, out


LAYERS = {
    # fp32: the generic GEMM computes real values, so the routing is the real one
    "tiny_fp32_real_routing": (64, 16, 4, 128, 64, 0, 0, 1),
    # decode-like: router split over 8 contraction slices (one top-k block per token), single-block
    # permutation writing the tile table, 32-row expert tiles, packed weights
    "decode_like_packed": (8, 32, 8, 512, 128, 1, 1, 0),
    # fp8 expert weights (quantised by the library), decode-like
    "decode_like_fp8": (8, 32, 8, 512, 128, 2, 2, 0),
    # rank/place permutation (T*K above 1024) and the 256x256 expert GEMM (its form that skips
    # empty half items: 147 mean rows per group), packed; router over 8 contraction slices
    "mid_packed_256_row_tiles": (264, 8, 4, 512, 256, 3, 1, 0),
    # router over 4 slices added by the one-wave-per-token top-k, packed
    "split_router_wave_topk": (100, 8, 2, 256, 64, 8, 1, 0),
    # row-major weights, ragged widths of the bf16 MFMA path
    "small_rows": (20, 16, 6, 256, 192, 4, 0, 0),
}


@pytest.mark.parametrize("name", list(LAYERS))
def test_layer_in_bounds(host_path, name):
    out = run(host_path, "layer", *LAYERS[name])
    assert calls_ok(out) >= 3 and "moe_layer_forward_noalloc" in out, out


@pytest.mark.skipif(os.environ.get("MOE_EMUL_PREFILL") != "1",
                    reason="about twenty minutes of host time: set MOE_EMUL_PREFILL=1 to run it")
def test_halves_at_the_prefill_shape(host_path):
    """The standalone halves at the prefill workload's full size (8192 tokens, 288 experts, d_model
    4096, width 1280), in the argument pattern of a timing script that once faulted the GPU.
    The permutation is made on the host (its barrier-heavy kernels are slow in the emulation and are
    covered at the smaller shapes above)."""
    out = run(host_path, "halves", 8192, 288, 8, 4096, 1280, 11, 0, 1, 1, timeout=7200)
    assert calls_ok(out) == 4, out


LIMIT_LAYERS = {
    # the largest expert count and K, split router, general permutation (T*K = 1024, E > 1022)
    "E1024_K64_T16": (16, 1024, 64, 256, 64, 1, 0, 0),
    # the same over more tokens (rank/place permutation), packed weights
    "E1024_K64_T40_packed": (40, 1024, 64, 256, 64, 2, 1, 0),
    # the single-block permutation at its expert limit and one past it
    "E1022_K64_T16": (16, 1022, 64, 256, 64, 3, 0, 0),
    "E1023_K64_T16": (16, 1023, 64, 256, 64, 4, 0, 0),
    # the fused router (6145 to 12288 tokens) at its expert limit and one past it
    "E320_K1_T6145": (6145, 320, 1, 128, 64, 5, 0, 0),
    "E321_K1_T6145_packed": (6145, 321, 1, 128, 64, 6, 1, 0),
    # fp32 with the largest expert count and K (real routing through the generic GEMM)
    "E1024_K64_T40_fp32": (40, 1024, 64, 128, 32, 7, 0, 1),
}


@pytest.mark.skipif(os.environ.get("MOE_EMUL_LIMITS") != "1",
                    reason="1.5 to 7 minutes of host time each: set MOE_EMUL_LIMITS=1 to run them")
@pytest.mark.parametrize("name", list(LIMIT_LAYERS))
def test_layer_at_the_limits_in_bounds(host_path, name):
    """The layer entry points at the edges of the accepted configuration (1024 experts, K = 64, the
    expert limits of the single-block permutation and of the fused router)."""
    out = run(host_path, "layer", *LIMIT_LAYERS[name], timeout=1800)
    assert calls_ok(out) >= 3 and "moe_layer_forward_noalloc" in out, out


def test_planted_workspace_mistake_is_caught(tmp_path):
    """The check itself: carving the SwiGLU activations one row short of the workspace must be reported."""
    cc = ES.clang()
    if cc is None:
        pytest.skip("clang++ with AddressSanitizer is needed")
    ES.write_tree(str(tmp_path))
    api = (tmp_path / "emul_api.cpp").read_text()
    planted = api.replace("w.h = a.take_bytes(n_rows * (int64_t)d_ff * (int64_t)elem_bytes(c->dtype));",
                          "w.h = a.take_bytes((n_rows - 1) * (int64_t)d_ff * (int64_t)elem_bytes(c->dtype));")
    assert planted != api
    (tmp_path / "emul_api.cpp").write_text(planted)
    exe = tmp_path / "host_path"
    r = subprocess.run(ES.compile_cmd(cc, tmp_path, "host_path.cpp", exe), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(exe), "halves", "40", "32", "8", "512", "256", "7", "0", "1", "0"],
                       capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout[-2000:], r.stderr[-2000:])
