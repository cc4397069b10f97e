"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

import long_context_exact_fwd_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lca.LIB_PATH), reason="library not built")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    assert _declared() == sorted(lca.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = lca.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


@pytest.mark.skipif(not os.path.exists(lca.DEBUG_LIB_PATH), reason="debug library not built")
def test_debug_library_exports_and_checks_like_the_release_one():
    """libmi355attn_debug.so (the -DATTN_DEBUG build) has the same ABI and argument checks."""
    dbg = lca.load_library(lca.DEBUG_LIB_PATH)
    for name in _declared():
        assert hasattr(dbg, name), name
    assert dbg.attn_status_str(lca.ATTN_ERR_DEBUG_CHECK) == b"ATTN_ERR_DEBUG_CHECK"
    rel = lca.load_library()
    args = [NULL] * 6 + [1, 4, 2, 128, 128, 1, NULL, 0, 0.125, S0]
    assert dbg.attn_fwd(*args) == rel.attn_fwd(*args) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert dbg.attn_bwd_workspace_bytes(1, 28, 4, 32768, 128) == rel.attn_bwd_workspace_bytes(1, 28, 4, 32768, 128)


def test_status_strings():
    lib = lca.load_library()
    assert lib.attn_status_str(0) == b"ATTN_OK"
    assert lib.attn_status_str(1) == b"ATTN_ERR_INVALID_ARGUMENT"
    assert lib.attn_status_str(2) == b"ATTN_ERR_UNSUPPORTED"
    assert lib.attn_status_str(3) == b"ATTN_ERR_HIP"
    assert lib.attn_status_str(5) == b"ATTN_ERR_DEBUG_CHECK"
    assert lib.attn_status_str(77) == b"ATTN_ERR_UNKNOWN"
    assert lib.attn_last_hip_error() == 0


def _split(B, Hq, Hkv, S):
    units = B * Hkv * (-(-S // 128))
    return 1 if units >= 1024 else min(Hq // Hkv, -(-1024 // units))


def _ksplit(B, Hq, S):
    units = B * Hq * (-(-S // 128))
    return 1 if units >= 1024 else min(4, -(-1024 // units))


def _ws(B, Hq, Hkv, S, D):
    """Layout stated in include/attn.h: Delta + LSE*log2e, work order, partial dK/dV, partial dQ."""
    a256 = lambda x: -(-x // 256) * 256
    s64 = -(-S // 64) * 64
    nblk = -(-S // 128)
    ns, nk = _split(B, Hq, Hkv, S), _ksplit(B, Hq, S)
    end = a256(8 * B * Hq * s64 + 4 * nblk * (ns + nk))
    end = a256(end + (8 * ns * B * S * Hkv * D if ns > 1 else 0))
    return end + (4 * nk * B * S * Hq * D if nk > 1 else 0)


def test_workspace_bytes():
    lib = lca.load_library()
    # gqa32k: enough dK/dV and dQ workgroups, no split
    assert _split(1, 28, 4, 32768) == 1 and _ksplit(1, 28, 32768) == 1
    assert lib.attn_bwd_workspace_bytes(1, 28, 4, 32768, 128) == 8 * 28 * 32768 + 8 * 256
    # packed32k share: 512 key-block units, the 7 heads of a group split in 2
    assert _split(1, 14, 2, 32768) == 2
    assert lib.attn_bwd_workspace_bytes(1, 14, 2, 32768, 128) == _ws(1, 14, 2, 32768, 128)
    assert lib.attn_bwd_workspace_bytes(1, 14, 2, 32768, 128) > 8 * 2 * 32768 * 2 * 128
    # short sequences: split up to the group size (dK/dV) and up to 4 (dQ)
    assert _split(2, 3, 1, 5) == 3 and _ksplit(2, 3, 5) == 4
    for args in [(2, 3, 1, 5, 64), (1, 1, 1, 65, 128), (1, 1, 1, 129, 64), (1, 8, 1, 65536, 128),
                 (3, 12, 4, 1000, 64), (1, 7, 1, 32768, 128)]:
        assert lib.attn_bwd_workspace_bytes(*args) == _ws(*args), args
    assert lib.attn_bwd_workspace_bytes(0, 3, 1, 5, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, -1, 1, 5, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, 6, 4, 5, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, 4, 2, 5, 0) == 0


# fake, 16-byte aligned, never dereferenced: every case below must fail validation first
P = ctypes.c_void_p(1 << 20)
PM = ctypes.c_void_p((1 << 20) + 2)  # misaligned
NULL = ctypes.c_void_p(0)
S0 = ctypes.c_void_p(0)


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, ws=NULL, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, cu=NULL, n=0,
             scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["B"], a["Hq"],
                                       a["Hkv"], a["S"], a["D"], a["causal"], a["cu"], a["n"], a["scale"], S0)


def _fp8(**kw):
    a = dict(q=P, k=P, v=P, dq=P, dk=P, dv=P, o=P, lse=P, ws=NULL, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd_fp8(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"], a["lse"],
                                           a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"], a["cu"],
                                           a["n"], a["scale"], S0)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                       a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"], a["cu"],
                                       a["n"], a["scale"], S0)


def _fwd_merge(**kw):
    """attn_fwd_merge with o and lse standing for the running o_acc and lse_acc."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, out=NULL, acc=1, ws=NULL, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, cu=NULL,
             n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd_merge(a["q"], a["k"], a["v"], a["o"], a["lse"], a["out"], a["acc"], a["ws"],
                                             a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"], a["cu"],
                                             a["n"], a["scale"], S0)


def _fp8_merge(**kw):
    """attn_fwd_fp8_merge with o and lse standing for the running o_acc and lse_acc."""
    a = dict(q=P, k=P, v=P, dq=P, dk=P, dv=P, o=P, lse=P, out=NULL, acc=1, ws=NULL, B=1, Hq=4, Hkv=2, S=128, D=128,
             causal=1, cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd_fp8_merge(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"], a["lse"],
                                                 a["out"], a["acc"], a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"],
                                                 a["D"], a["causal"], a["cu"], a["n"], a["scale"], S0)


def _bwd_acc(**kw):
    """attn_bwd_accumulate with dq, dk, dv standing for the fp32 accumulators."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, acc=1, ws=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd_accumulate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                                  a["dv"], a["acc"], a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"],
                                                  a["D"], a["causal"], a["cu"], a["n"], a["scale"], S0)


BAD = [
    dict(q=NULL), dict(lse=NULL), dict(B=0), dict(Hq=0), dict(Hkv=0), dict(S=0), dict(S=-5), dict(D=0),
    dict(Hq=6, Hkv=4), dict(causal=2), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")),
    dict(scale=float("nan")), dict(cu=P, n=0), dict(cu=P, n=3, B=2), dict(cu=NULL, n=2), dict(cu=P, n=200),
    dict(q=PM), dict(o=PM), dict(cu=ctypes.c_void_p((1 << 20) + 2), n=2),
]


@pytest.mark.parametrize("kw", BAD)
def test_invalid_arguments_rejected(kw):
    assert _fwd(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _bwd(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _fp8(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _fwd_merge(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _fp8_merge(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _bwd_acc(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("fn,kw", [(_bwd_acc, dict(acc=2)), (_bwd_acc, dict(acc=-1)), (_bwd_acc, dict(ws=NULL)),
                                   (_bwd_acc, dict(dk=NULL)), (_bwd_acc, dict(dq=PM)), (_bwd_acc, dict(ws=PM)),(_fp8_merge, dict(out=PM)), (_fp8_merge, dict(acc=2)), (_fp8_merge, dict(dv=NULL)),
                                   (_fp8_merge, dict(lse=ctypes.c_void_p((1 << 20) + 2))),
                                   (_fp8_merge, dict(dq=ctypes.c_void_p((1 << 20) + 2))), (_fp8_merge, dict(ws=PM)),(_fwd_merge, dict(out=PM)), (_fwd_merge, dict(acc=2)), (_fwd_merge, dict(acc=-1)),
                                   (_fwd_merge, dict(lse=ctypes.c_void_p((1 << 20) + 2))),
                                   (_fwd_merge, dict(ws=PM)), (_fwd, dict(ws=PM)), (_bwd, dict(ws=NULL)), (_bwd, dict(do=NULL)),
                                   (_bwd, dict(ws=PM)), (_fp8, dict(dq=NULL)), (_fp8, dict(ws=PM)),
                                   (_fp8, dict(dv=ctypes.c_void_p((1 << 20) + 2)))])
def test_entry_specific_pointers(fn, kw):
    assert fn(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("D", [32, 80, 96, 256])
def test_unsupported_head_dims(D):
    assert _fwd(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8(D=64) == lca.ATTN_ERR_UNSUPPORTED
    assert _fwd_merge(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8_merge(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8_merge(D=64) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd_acc(D=D) == lca.ATTN_ERR_UNSUPPORTED


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(ImportError):
        lca.load_library(str(tmp_path / "missing.so"))


def _merge(**kw):
    a = dict(oa=P, la=P, op=P, lp=P, out=NULL, B=1, S=128, H=4, D=128, acc=1)
    a.update(kw)
    return lca.load_library().attn_merge(a["oa"], a["la"], a["op"], a["lp"], a["out"], a["B"], a["S"], a["H"],
                                         a["D"], a["acc"], S0)


@pytest.mark.parametrize("kw", [dict(oa=NULL), dict(la=NULL), dict(op=NULL), dict(lp=NULL), dict(oa=PM),
                                dict(op=PM), dict(out=PM), dict(la=ctypes.c_void_p((1 << 20) + 2)),
                                dict(B=0), dict(S=0), dict(H=-1), dict(D=0), dict(acc=2)])
def test_merge_invalid_arguments_rejected(kw):
    assert _merge(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("D", [32, 80, 256])
def test_merge_unsupported_head_dims(D):
    assert _merge(D=D) == lca.ATTN_ERR_UNSUPPORTED


def test_oversized_requests_unsupported():
    """seqlen * Hq * D beyond 2^31 - 1 is refused before any HIP call."""
    big = dict(S=1 << 20, Hq=16, Hkv=4, D=128)  # 2^31 elements per batch slice
    assert _fwd(**big) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd(**big) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8(**big) == lca.ATTN_ERR_UNSUPPORTED
    assert _fwd_merge(**big) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8_merge(**big) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd_acc(**big) == lca.ATTN_ERR_UNSUPPORTED
    lib = lca.load_library()
    assert lib.attn_bwd_workspace_bytes(1, 16, 4, 1 << 20, 128) == 0
    # merge: more than 2^40 elements in total
    assert _merge(B=1 << 10, S=1 << 20, H=1 << 10, D=128) == lca.ATTN_ERR_UNSUPPORTED


def _fwd_split(B, Hq, S):
    units = B * Hq * (-(-S // 128))
    if units >= 512:
        return 1
    return max(1, min(-(-512 // units), 8, (-(-S // 64)) // 32))


def test_fwd_workspace_bytes():
    """Layout stated in include/attn.h: fp32 partial O, then (256-byte aligned) the partial row statistics."""
    lib = lca.load_library()
    a256 = lambda x: -(-x // 256) * 256
    for args in [(1, 28, 4, 32768, 128), (2, 32, 32, 8192, 128), (1, 14, 2, 32768, 128), (1, 2, 1, 4032, 64),
                 (1, 2, 1, 4033, 64), (1, 1, 1, 32768, 128), (1, 2, 1, 32768, 128), (3, 3, 1, 9000, 64),
                 (1, 8, 1, 1000, 128), (1, 1, 1, 1, 128)]:
        B, Hq, Hkv, S, D = args
        ks = _fwd_split(B, Hq, S)
        want = 0 if ks == 1 else a256(4 * ks * B * S * Hq * D) + 4 * ks * B * Hq * S
        assert lib.attn_fwd_workspace_bytes(*args) == want, args
    assert _fwd_split(1, 28, 32768) == 1 and _fwd_split(1, 2, 32768) == 1 and _fwd_split(1, 1, 32768) == 2
    assert _fwd_split(1, 2, 4096) == 2 and _fwd_split(1, 1, 16384) == 4
    assert _fwd_split(1, 2, 4032) == 1 and _fwd_split(1, 2, 4033) == 2
    assert lib.attn_fwd_workspace_bytes(0, 1, 1, 32768, 128) == 0
    assert lib.attn_fwd_workspace_bytes(1, 3, 2, 32768, 128) == 0
    assert lib.attn_fwd_workspace_bytes(1, 16, 4, 1 << 20, 128) == 0


def _phases(ph, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd_phases(ph, a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                              a["dv"], a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"],
                                              a["cu"], a["n"], a["scale"], S0)


@pytest.mark.parametrize("ph", [0, 8, 9, 15, 0xFFFFFFFF])
def test_bwd_phases_bitmask_rejected(ph):
    assert _phases(ph) == lca.ATTN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", BAD[:8] + [dict(ws=NULL), dict(do=PM)])
def test_bwd_phases_arguments_checked_like_bwd(kw):
    for ph in (lca.BWD_DELTA, lca.BWD_DKDV, lca.BWD_DQ, lca.BWD_ALL):
        assert _phases(ph, **kw) == lca.ATTN_ERR_INVALID_ARGUMENT
    assert _phases(lca.BWD_ALL, D=96) == lca.ATTN_ERR_UNSUPPORTED


def _noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                               a["dv"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"],
                                               a["cu"], a["n"], a["scale"], S0)


@pytest.mark.parametrize("kw", BAD + [dict(do=NULL), dict(dk=PM)])
def test_noalloc_arguments_checked_like_bwd(kw):
    assert _noalloc(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


def test_noalloc_size_limits():
    """Requests whose per-row statistics alone (8 * B * Hq * S64 bytes) exceed the fixed scratch are
    refused with ATTN_ERR_SCRATCH_TOO_SMALL before any HIP call; head dims and the 2^31 limit as bwd."""
    lib = lca.load_library()
    assert lib.attn_status_str(lca.ATTN_ERR_SCRATCH_TOO_SMALL) == b"ATTN_ERR_SCRATCH_TOO_SMALL"
    assert _noalloc(B=1, Hq=64, Hkv=8, S=140000, D=128) == lca.ATTN_ERR_SCRATCH_TOO_SMALL
    assert _noalloc(B=8, Hq=32, Hkv=8, S=33000, D=64) == lca.ATTN_ERR_SCRATCH_TOO_SMALL
    assert 8 * 1 * 64 * 131072 >= lca.NOALLOC_SCRATCH_BYTES
    assert _noalloc(D=96) == lca.ATTN_ERR_UNSUPPORTED
    assert _noalloc(S=1 << 20, Hq=16, Hkv=4, D=128) == lca.ATTN_ERR_UNSUPPORTED


def _bwd8(**kw):
    a = dict(q=P, k=P, v=P, dq_s=P, dk_s=P, dv_s=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P, B=1, Hq=4, Hkv=2, S=128,
             D=128, causal=1, cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd_fp8(a["q"], a["k"], a["v"], a["dq_s"], a["dk_s"], a["dv_s"], a["o"], a["lse"],
                                           a["do"], a["dq"], a["dk"], a["dv"], a["ws"], a["B"], a["Hq"], a["Hkv"],
                                           a["S"], a["D"], a["causal"], a["cu"], a["n"], a["scale"], S0)


@pytest.mark.parametrize("kw", BAD + [dict(ws=NULL), dict(ws=PM), dict(dq_s=NULL), dict(dv_s=ctypes.c_void_p((1 << 20) + 2)),
                                      dict(do=PM)])
def test_bwd_fp8_arguments_rejected(kw):
    assert _bwd8(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


def test_bwd_fp8_workspace_and_head_dims():
    lib = lca.load_library()
    a256 = lambda x: -(-x // 256) * 256
    for (B, Hq, Hkv, S) in [(1, 8, 1, 65536), (2, 3, 1, 77), (1, 14, 2, 2048)]:
        want = a256(2 * B * S * Hq * 128) + 2 * a256(2 * B * S * Hkv * 128) + _ws(B, Hq, Hkv, S, 128)
        assert lib.attn_bwd_fp8_workspace_bytes(B, Hq, Hkv, S, 128) == want
    assert lib.attn_bwd_fp8_workspace_bytes(1, 4, 2, 128, 64) == 0
    assert _bwd8(D=64) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd8(S=1 << 20, Hq=16, Hkv=4) == lca.ATTN_ERR_UNSUPPORTED
