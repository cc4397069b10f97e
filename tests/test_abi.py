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


def test_status_strings():
    lib = lca.load_library()
    assert lib.attn_status_str(0) == b"ATTN_OK"
    assert lib.attn_status_str(1) == b"ATTN_ERR_INVALID_ARGUMENT"
    assert lib.attn_status_str(2) == b"ATTN_ERR_UNSUPPORTED"
    assert lib.attn_status_str(3) == b"ATTN_ERR_HIP"
    assert lib.attn_status_str(77) == b"ATTN_ERR_UNKNOWN"
    assert lib.attn_last_hip_error() == 0


def test_workspace_bytes():
    lib = lca.load_library()
    # two fp32 arrays [B, Hq, S rounded up to 64], two int32 arrays [ceil(S / 128)]
    assert lib.attn_bwd_workspace_bytes(1, 28, 32768) == 8 * 28 * 32768 + 8 * 256
    assert lib.attn_bwd_workspace_bytes(2, 3, 5) == 8 * 2 * 3 * 64 + 8
    assert lib.attn_bwd_workspace_bytes(1, 1, 65) == 8 * 128 + 8
    assert lib.attn_bwd_workspace_bytes(1, 1, 129) == 8 * 192 + 16
    assert lib.attn_bwd_workspace_bytes(0, 3, 5) == 0
    assert lib.attn_bwd_workspace_bytes(1, -1, 5) == 0


# fake, 16-byte aligned, never dereferenced: every case below must fail validation first
P = ctypes.c_void_p(1 << 20)
PM = ctypes.c_void_p((1 << 20) + 2)  # misaligned
NULL = ctypes.c_void_p(0)
S0 = ctypes.c_void_p(0)


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["S"],
                                       a["D"], a["causal"], a["cu"], a["n"], a["scale"], S0)


def _fp8(**kw):
    a = dict(q=P, k=P, v=P, dq=P, dk=P, dv=P, o=P, lse=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, cu=NULL, n=0,
             scale=0.088)
    a.update(kw)
    return lca.load_library().attn_fwd_fp8(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"], a["lse"],
                                           a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"], a["cu"], a["n"],
                                           a["scale"], S0)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1,
             cu=NULL, n=0, scale=0.088)
    a.update(kw)
    return lca.load_library().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                       a["ws"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["causal"], a["cu"],
                                       a["n"], a["scale"], S0)


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


@pytest.mark.parametrize("fn,kw", [(_fwd, dict(ws=None)), (_bwd, dict(ws=NULL)), (_bwd, dict(do=NULL)),
                                   (_bwd, dict(ws=PM)), (_fp8, dict(dq=NULL)),
                                   (_fp8, dict(dv=ctypes.c_void_p((1 << 20) + 2)))])
def test_entry_specific_pointers(fn, kw):
    kw = {k: v for k, v in kw.items() if v is not None}
    if not kw:
        pytest.skip("attn_fwd has no workspace")
    assert fn(**kw) == lca.ATTN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("D", [32, 80, 96, 256])
def test_unsupported_head_dims(D):
    assert _fwd(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _bwd(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8(D=D) == lca.ATTN_ERR_UNSUPPORTED
    assert _fp8(D=64) == lca.ATTN_ERR_UNSUPPORTED


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
