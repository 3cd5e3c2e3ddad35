"""Rewriting of the library's HIP sources into host C++ for the bounds emulation (tests/emul).

HIP keywords and builtins become plain C++ (tests/emul/shim.h); the inline-asm
LDS reads of the 256x256 GEMM become checked reads; waits and barriers written
in asm disappear; every kernel launch becomes a call of the runner
(tests/emul/runner.h), which runs each lane of each block on the host. Kernels
that scan or count through LDS run with one OS thread per lane and real
barriers; the others lane by lane.
"""
from __future__ import annotations

import os
import re
import shutil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_routed_expert_amd", "csrc")
EMUL = os.path.join(ROOT, "tests", "emul")

# kernels whose lanes talk through LDS, shuffles or barriers: one OS thread per lane
# (the fp8 quantiser's row maximum goes through LDS too, but only into values, not addresses:
# it runs lane by lane, as the GEMMs do)
SYNC_KERNELS = {"build_tiles_kernel", "permute_rank_kernel", "permute_place_kernel", "permute_small_kernel",
                "ep_plan_kernel", "topk_kernel", "group_partials_kernel", "group_stats_kernel", "combine_kernel",
                "combine16_kernel",
                "gemm_generic",
                "router_topk_kernel"}


def clang() -> str | None:
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    return None


def read(name: str) -> str:
    return open(os.path.join(CSRC, name)).read()


def internal_header() -> str:
    return read("moe_internal.h").replace("#include <hip/hip_runtime.h>", '#include "shim.h"')


def _asm_to_host(s: str) -> tuple:
    """Inline asm of the LDS-staged kernels: LDS address spaces and bases, checked ds_read_b128 reads,
    waits and barriers dropped. Returns the source and the number of reads rewritten."""
    s, _ = re.subn(r"typedef __attribute__\(\(address_space\(3\)\)\) void (\w+);", r"typedef void \1;", s)
    s, _ = re.subn(r"\(uint32_t\)\(uintptr_t\)\(\w+\*\)&(\w+)\[0\]\[0\]",
                   lambda m: f"emul_lds_base((void*)&{m.group(1)}, sizeof({m.group(1)}))", s)
    s, _ = re.subn(r"\(uint32_t\)\(uintptr_t\)\(\w+\*\)&(\w+)\[0\]",
                   lambda m: f"emul_lds_base((void*)&{m.group(1)}, sizeof({m.group(1)}))", s)
    s, k1 = re.subn(r'asm volatile\("ds_read_b128 %0, %1 offset:%2" : "=v"\(([^)]*\]?)\) : "v"\((\w+)\), '
                    r'"n"\(([^)]*)\)\);',
                    lambda m: (f"{m.group(1)} = emul_ds_read<std::remove_reference_t<decltype({m.group(1)})>>"
                               f"({m.group(2)} + ({m.group(3)}));"), s)
    s, _ = re.subn(r'asm volatile\("s_waitcnt lgkmcnt\(%1\)" : "\+v"\([^)]*\) : "n"\([^)]*\)\);', ";", s)
    s, _ = re.subn(r'asm volatile\("s_waitcnt lgkmcnt\(\d+\)"(?: : "\+v"\([^;]*?\))+\);', ";", s, flags=re.S)
    s, _ = re.subn(r'asm volatile\("[^"]*" ::: "memory"\);', ";", s)
    return s, k1


def big8_source(kernel_src: str) -> str:
    """grouped_gemm_big8.hip for the host: asm LDS reads checked, asm waits dropped, launches emulated."""
    s = kernel_src.replace('#include "moe_internal.h"', '#include "emul_internal.h"')
    k0 = s.count("(uint32_t)(uintptr_t)(lds8_void_t*)&")
    s, k1 = _asm_to_host(s)
    s, k4 = re.subn(r"(gemm_bf16_big8?<[^>]*>)<<<\(unsigned\)blocks, (256|512), 0, s>>>\(g\);",
                    lambda m: f"emul_launch({m.group(1)}, (unsigned)blocks, {m.group(2)}, g);", s)
    left = re.findall(r"asm volatile.*|<<<.*>>>", s)
    assert k0 >= 1 and k1 >= 2 and k4 >= 4 and not left, (k0, k1, k4, left)
    return s


def _kernel_name_start(s: str, i: int) -> int:
    """Start of the kernel name (identifier plus template arguments) that ends at s[i]."""
    j = i
    if s[j - 1] == ">":  # template arguments, balanced
        depth = 0
        while True:
            j -= 1
            depth += s[j] == ">"
            depth -= s[j] == "<"
            if depth == 0:
                break
    while j > 0 and (s[j - 1].isalnum() or s[j - 1] == "_"):
        j -= 1
    return j


def launches_source(src: str) -> str:
    """A kernel source whose launches `k<<<grid, threads, shm, stream>>>(args)` all go through the runner."""
    s = src.replace('#include "moe_internal.h"', '#include "emul_internal.h"')
    s, _ = _asm_to_host(s)
    n = 0
    while True:
        i = s.find("<<<")
        if i < 0:
            break
        j = s.index(">>>", i)
        k = j + 3
        assert s[k] == "(", s[i - 40:k + 20]
        depth, e = 0, k
        while True:  # the balanced argument list
            depth += s[e] == "("
            depth -= s[e] == ")"
            if depth == 0:
                break
            e += 1
        start = _kernel_name_start(s, i)
        name = s[start:i]
        cfg = [c.strip() for c in s[i + 3:j].split(",")]
        assert len(cfg) == 4, cfg
        sync = "true" if name.split("<")[0] in SYNC_KERNELS else "false"
        s = s[:start] + f"emul_run({sync}, {name}, emul_grid({cfg[0]}), {cfg[1]}, {s[k + 1:e]})" + s[e + 1:]
        n += 1
    assert n >= 1 and "asm volatile" not in s, n
    return s


def api_source() -> str:
    """The C ABI for the host: only its include changes (the shim maps the runtime calls it makes)."""
    s = read("api.hip")
    assert s.count('#include "moe_internal.h"') == 1
    return s.replace('#include "moe_internal.h"', '#include "emul_internal.h"')


def write_tree(d, big8_src: str | None = None) -> None:
    """The rewritten sources of every file the host-path driver includes, into directory d."""
    open(os.path.join(d, "emul_internal.h"), "w").write(internal_header())
    open(os.path.join(d, "emul_big.cpp"), "w").write(big8_source(big8_src or read("grouped_gemm_big8.hip")))
    open(os.path.join(d, "emul_gemm.cpp"), "w").write(launches_source(read("grouped_gemm.hip")))
    open(os.path.join(d, "emul_permute.cpp"), "w").write(launches_source(read("permute.hip")))
    open(os.path.join(d, "emul_route.cpp"), "w").write(launches_source(read("route.hip")))
    open(os.path.join(d, "emul_router.cpp"), "w").write(launches_source(read("router.hip")))
    open(os.path.join(d, "emul_combine.cpp"), "w").write(launches_source(read("combine.hip")))
    open(os.path.join(d, "emul_pack.cpp"), "w").write(launches_source(read("pack.hip")))
    open(os.path.join(d, "emul_api.cpp"), "w").write(api_source())


def compile_cmd(cc: str, d, main: str, exe) -> list:
    return [cc, "-std=c++20", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-pthread",
            "-Wno-unused-lambda-capture", "-I", str(d), "-I", EMUL, "-I", os.path.join(ROOT, "include"),
            os.path.join(EMUL, main), "-o", str(exe)]
