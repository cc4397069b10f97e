"""Host replay of the kernels' index arithmetic (tests/index_check.cpp over
long_context_exact_fwd_amd/csrc/attn_index.h, the header the kernels inline):
LDS tile copies and fragment reads in bounds, tiles filled exactly once, every
MFMA operand slot receiving the element the product needs, every read free of
bank conflicts under the LDS model stated in index_check.cpp, tile ranges and
key-split shares over a sweep of sequence shapes, workspace layouts and 32-bit
copy ranges up to the largest accepted sequence. Built with g++ under the host
address and undefined-behaviour sanitizers; no GPU needed.

The second test plants mistakes in a copy of the header and checks that the
replay catches each of them."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "index_check.cpp")
HEADER = os.path.join(ROOT, "long_context_exact_fwd_amd", "csrc", "attn_index.h")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def _build_and_run(tmp_path, header=None, sanitize=True):
    exe = str(tmp_path / "index_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-o", exe, SRC]
    if sanitize:
        cmd[4:4] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    if header is not None:
        cmd.append(f'-DATTN_INDEX_HEADER="{header}"')
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_index_arithmetic_in_bounds_and_layouts_exact(tmp_path):
    r = _build_and_run(tmp_path)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "index_check: OK" in r.stdout


MUTATIONS = [
    # (description, original text, planted mistake)
    ("perm_rows swaps bits 1 and 2", "((m & 4) << 1) | ((m & 8) >> 1)", "((m & 2) << 1) | ((m & 4) >> 1)"),
    ("B128 swizzle of D = 128 loses a row bit (bank conflicts only)", "const int f = (row & 3) | (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 3);",
     "const int f = (row & 3) | (((row >> 3) & 1) << 2);"),
    ("backward transposed fragment second half one row off",
     "return off_dual_unit<D>(8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * hi,",
     "return off_dual_unit<D>(8 * (lane >> 5) + ((lane & 15) >> 2) + 3 * hi,"),
    ("D = 64 dual swizzle without row bit 3 (bank conflicts only)",
     "return chunk ^ (((row >> 1) & 3) | ((((row >> 1) ^ (row >> 3)) & 1) << 2));",
     "return chunk ^ (((row >> 1) & 3) | (((row >> 1) & 1) << 2));"),
    ("tile copy destination stride of 256 elements", "return (i * waves + wave) * 512 + lane * 8;", "return (i * waves + wave) * 256 + lane * 8;"),
    ("fp8 K swizzle of the earlier, conflicting layout", "ATTN_HD int fp8_fk_swz(int row) { return (row >> 1) & 7; }",
     "ATTN_HD int fp8_fk_swz(int row) { return (row & 3) | ((row >> 1) & 4); }"),
    ("fp8 V swizzle from the wrong row bits (bank conflicts only)", "ATTN_HD int fp8_fv_swz(int row) { return row & 7; }",
     "ATTN_HD int fp8_fv_swz(int row) { return (row >> 1) & 7; }"),
    ("segment end not clamped", "end = imin(seqlen, imax(cu[hi], i + 1));", "end = imax(cu[hi], i + 1);"),
    ("workspace order offset overlaps the statistics", "return (size_t)8 * batch * hq * stat_stride_for(seqlen);",
     "return (size_t)4 * batch * hq * stat_stride_for(seqlen);"),
    ("few-key rows of a causal segment one too many", "return causal ? imin(kFewKeyLimit - 1, len)",
     "return causal ? imin(kFewKeyLimit, len)"),
    ("few-key rows of a non-causal segment up to length 64", "(len < kFewKeyLimit ? len : 0)",
     "(len <= kFewKeyLimit ? len : 0)"),
]


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(tmp_path, desc, old, new):
    text = open(HEADER, encoding="utf-8").read()
    assert text.count(old) == 1, desc
    bad = tmp_path / "attn_index_planted.h"
    bad.write_text(text.replace(old, new), encoding="utf-8")
    r = _build_and_run(tmp_path, header=str(bad), sanitize=False)
    assert r.returncode != 0, f"planted mistake not caught: {desc}"
