"""Shared helpers for the GPU parity tests: device upload and error metrics."""
import numpy as np


def dev_bf16(bits: np.ndarray):
    import long_context_exact_fwd_amd as lca
    return lca.bf16_from_bits(bits, "cuda")


def dev_u8(codes: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def dev_i32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm((x - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))


def max_abs(x, r) -> float:
    return float(np.max(np.abs(np.asarray(x, dtype=np.float64) - np.asarray(r, dtype=np.float64))))


# Tolerances against the fp64 oracle (bf16 outputs, fp32 LSE).
TOL_O_MAXABS = 1e-2
TOL_O_REL = 5e-3
TOL_LSE = 1e-3
TOL_GRAD_REL = 1e-2
TOL_ZERO_GRAD_ABS = 1e-3  # where the exact gradient is zero
TOL_FP8_REL = 5e-2


def delta_from_o_rows(S, causal, cu_seqlens=None) -> np.ndarray:
    """Rows [S] whose Delta the backward takes from the O it is given (Delta_i = dO_i . O_i): rows with at
    least 64 visible keys. The others (the first 63 rows of a causal segment, every row of a non-causal
    segment shorter than 64) get Delta_i = sum_j P_ij dP_ij from its definition, so the rounding of the
    given O does not reach their gradients."""
    edges = np.asarray(cu_seqlens if cu_seqlens is not None else [0, S], dtype=np.int64)
    out = np.zeros(S, dtype=bool)
    for a, b in zip(edges[:-1], edges[1:]):
        if causal:
            out[a + 63:b] = True
        elif b - a >= 64:
            out[a:b] = True
    return out


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bfloat16 values (8 significant bits) at |x|: 2^(floor(log2|x|) - 7)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7.0)


def o_bound(ro) -> np.ndarray:
    """Per-element O bound: 1e-2, or half a bf16 ulp of the exact value where even the correctly rounded
    bf16 output can be further than 1e-2 away (|ref| >= 4, where half an ulp is 2^-6)."""
    return np.maximum(TOL_O_MAXABS, 0.5 * bf16_ulp(ro))


def check_fwd(o, lse, ro, rl, tag="", rel_tol=TOL_O_REL, abs_factor=1.0):
    """O: |o - ref| <= max(1e-2, ulp_bf16(ref) / 2) and rel-L2 <= 5e-3 against the exact oracle; LSE max-abs <= 1e-3."""
    o = np.asarray(o, dtype=np.float64)
    raw = np.abs(o - ro)
    excess = raw / (abs_factor * o_bound(ro))
    at = np.unravel_index(int(np.argmax(raw)), raw.shape)
    worst = float(np.max(excess)) if excess.size else 0.0
    rr, rlse = rel_l2(o, ro), max_abs(lse, rl)
    msg = (f"{tag} O maxabs={raw[at]:.3e} at {tuple(int(i) for i in at)} (|ref|={abs(ro[at]):.3f}) "
           f"worst err/bound={worst:.3f} relL2={rr:.3e} LSE maxabs={rlse:.3e}")
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), msg
    assert worst <= 1.0 and rr <= rel_tol and rlse <= TOL_LSE, msg


def check_grads(pairs, tag=""):
    msgs = []
    ok = True
    for name, x, r in pairs:
        if np.any(np.asarray(r) != 0):
            e = rel_l2(x, r)
            msgs.append(f"{name} relL2={e:.3e}")
            ok = ok and np.all(np.isfinite(x)) and e <= TOL_GRAD_REL
        else:
            # exactly zero reference (e.g. dQ, dK when every row sees one key):
            # the kernel's dP - Delta is a difference of two fp32 dot products
            # of the same values summed in different orders, so it leaves
            # rounding noise of about 1e-6 instead of exact zeros
            e = max_abs(x, r)
            msgs.append(f"{name} maxabs={e:.3e} (zero reference)")
            ok = ok and np.all(np.isfinite(x)) and e <= TOL_ZERO_GRAD_ABS
    msg = tag + " " + " ".join(msgs)
    print(msg, flush=True)
    assert ok, msg
