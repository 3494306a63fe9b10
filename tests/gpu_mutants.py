"""Mutated builds of the HIP library, for the GPU mutant tier (tests/test_gpu_mutants.py).

TEST INFRASTRUCTURE ONLY.  Each mutant plants one plausible mistake in a copy of one translation unit
of the library -- a reduction schedule chosen from t, a reordered fold (of the slice sums, in one launch
or in the small-N fold launch, or of the logprob's block partials), a local instead of a global shift, a
different in-block tree, a row maximum taken over rows past the vocabulary -- and is linked with the product's other objects into
tests/mutant_libs/lib_<name>.so.  The GPU tests load each one beside the product library and check
that their invariance and parity checks catch it while the product passes them.  Every mutation keeps
all memory accesses and loop bounds of the code it replaces (no mutant can fault or hang).  The
product never loads these libraries.
"""
from __future__ import annotations

import contextlib
import os
import shutil
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_DIR = os.path.join(HERE, "mutant_libs")

# the slices of an equal 8-way plan (a different K plan), for the t-chosen-schedule mutant
_EQUAL = "2 * ((G / 2) * ({i}) / 8)"

MUTANTS = {
    # the K-slice plan of both projection kernels switches to 8 equal slices when t > 16
    "k_plan_from_t": ("w8inv_gemm.hip", [
        ("const int g_begin = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, wave));",
         "const int g_begin = __builtin_amdgcn_readfirstlane(t > 16 ? " + _EQUAL.format(i="wave")
         + " : (int)kslice_begin(G, wave));"),
        ("const int g_end = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, wave + 1));",
         "const int g_end = __builtin_amdgcn_readfirstlane(t > 16 ? (wave + 1 >= 8 ? G : "
         + _EQUAL.format(i="wave + 1") + ") : (int)kslice_begin(G, wave + 1));"),
        ("    int next_bound = (int)kslice_begin(G, 1);",
         "    int next_bound = t > 16 ? " + _EQUAL.format(i="1") + " : (int)kslice_begin(G, 1);"),
        ("        next_bound = (int)kslice_begin(G, slice + 1);",
         "        next_bound = t > 16 ? (slice + 1 >= 8 ? G : " + _EQUAL.format(i="slice + 1")
         + ") : (int)kslice_begin(G, slice + 1);"),
        ("                next_bound = (int)kslice_begin(G, 1);",
         "                next_bound = t > 16 ? " + _EQUAL.format(i="1") + " : (int)kslice_begin(G, 1);"),
    ]),
    # the split kernel folds the 8 slice sums right to left when t > 16
    "slice_fold_reversed_from_t": ("w8inv_gemm.hip", [
        ("        double sum = *part(0, V);\n#pragma unroll\n        for (int w = 1; w < kKSlices; ++w) sum = sum + *part(w, V);",
         "        double sum = *part(t > 16 ? kKSlices - 1 : 0, V);\n#pragma unroll\n"
         "        for (int w = 1; w < kKSlices; ++w) sum = sum + *part(t > 16 ? kKSlices - 1 - w : w, V);"),
    ]),
    # the K-slice path's fold launch folds the 8 slice sums from the last when t > 16
    "kslice_fold_reversed_from_t": ("w8inv_kslice.hip", [
        ("    double sum = p[0];\n#pragma unroll\n    for (int w = 1; w < kKSlices; ++w) sum = sum + p[w * stride];",
         "    double sum = p[t > 16 ? (kKSlices - 1) * stride : 0];\n#pragma unroll\n"
         "    for (int w = 1; w < kKSlices; ++w) sum = sum + p[(t > 16 ? kKSlices - 1 - w : w) * stride];"),
    ]),
    # the logprob's fold adds four block partials together before adding them to the running sum
    "block_fold_regrouped": ("w8inv_logprob.hip", [
        ("                S = S + p0;\n                S = S + p1;\n                S = S + p2;\n                S = S + p3;",
         "                S = S + ((p0 + p1) + (p2 + p3));"),
    ]),
    # each block's exps are shifted by the block's own maximum instead of the row's
    "block_local_max": ("w8inv_logprob.hip", [
        ("    const float m = row_max_from_blocks<kLpThreads>(M, nm, j, nan);\n    if (nan) {",
         "    float m = row_max_from_blocks<kLpThreads>(M, nm, j, nan);\n    m = nm == nb ? M[(int64_t)j * nm + b] : m;\n"
         "    if (nan) {"),
    ]),
    # the fused head's max epilogue counts every row of the last strip, the rows past V too
    "max_epilogue_counts_padding_rows": ("w8inv_gemm.hip", [
        ("key[tt][v] = mx_key(bv[tt][v], n < N);", "key[tt][v] = mx_key(bv[tt][v], true);"),
    ]),
    # the in-wave butterfly of a block's tree pairs lanes 32 apart first (strided halves)
    "in_block_tree_strided": ("w8inv_logprob.hip", [
        ("    for (int off = 1; off < 64; off <<= 1) s = s + __shfl_xor(s, off);",
         "    for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off);"),
    ]),
}


def lib_path(name: str) -> str:
    return os.path.join(LIB_DIR, f"lib_{name}.so")


@contextlib.contextmanager
def library(path: str):
    """Route the binding's calls to the library built at `path` while the block runs."""
    import invariant_quantized_decode_amd as w8

    saved = w8._lib
    w8._lib = w8._load(path)
    try:
        yield
    finally:
        w8._lib = saved


def build(hip_build) -> list:
    """Build the product library and every mutant library.  `hip_build` is the product's build module:
    the mutated translation units compile alongside the product's, and each mutant is linked with the
    product's other objects once those exist."""
    os.makedirs(LIB_DIR, exist_ok=True)
    os.makedirs(hip_build.BUILD, exist_ok=True)
    work = os.path.join(hip_build.BUILD, "mutants")

    def compile_mutant(item):
        name, (target, edits) = item
        src_dir = os.path.join(work, name)
        shutil.rmtree(src_dir, ignore_errors=True)
        shutil.copytree(hip_build.CSRC, src_dir)
        path = os.path.join(src_dir, target)
        text = open(path).read()
        for old, new in edits:
            assert text.count(old) == 1, f"{name}: mutation site not found once: {old[:60]!r}"
            text = text.replace(old, new)
        open(path, "w").write(text)
        return hip_build.compile_source(path, os.path.join(src_dir, target.replace(".hip", ".o")), include_dir=src_dir)

    with ThreadPoolExecutor(max_workers=len(MUTANTS) + 1) as ex:
        product = ex.submit(hip_build.build)
        objs = list(ex.map(compile_mutant, MUTANTS.items()))
        product.result()
    libs = []
    for (name, (target, _)), obj in zip(MUTANTS.items(), objs):
        others = [os.path.join(hip_build.BUILD, s.replace(".hip", ".o")) for s in hip_build.SOURCES if s != target]
        hip_build.link_objects([obj] + others, lib_path(name))
        libs.append(lib_path(name))
    return libs
