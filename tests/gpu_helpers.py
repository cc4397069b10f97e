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


def rounding_o_bound(o, ro, abar) -> np.ndarray:
    """Per-element O bound from the tiled forward's arithmetic, for inputs outside the stated workloads.

    The kernel forms O = bf16(sum_j bf16(P_j) V_j / l) with P_j in fp32 and l = sum_j P_j unrounded. Rounding
    P_j to bf16 (8 significant bits) moves it by at most 2^-8 P_j, so the sum moves by at most
    2^-8 sum_j w_j |V_j| = 2^-8 abar (w the softmax weights; abar is the attention of the same scores over |V|);
    the output rounding adds half a bf16 ulp of the value rounded (taken at the larger of |o| and |ref|). The
    fp32 scores, exponentials and sums add relative errors of order 2^-20, covered by 2^-12 abar + 1e-6. With
    one key holding most of a row's weight nothing averages the first term out: 2^-8 |V| reaches 1.5e-2 at
    |V| = 4."""
    o = np.asarray(o, dtype=np.float64)
    abar = np.asarray(abar, dtype=np.float64)
    return (2.0 ** -8 + 2.0 ** -12) * abar + 0.5 * bf16_ulp(np.maximum(np.abs(o), np.abs(ro))) + 1e-6


def fp8_lse_bound(qv, kv, causal, scale, cu_seqlens=None) -> np.ndarray:
    """Per-row LSE bound [B, Hq, S] for the fp8 forward on inputs outside the stated workloads: 1e-3 plus
    2^-11 scale max_j sum_d |q_id k_jd| over the row's visible keys. The E4M3 MFMA does not add its 64
    products exactly but drops low-order bits against the largest (measured on MI355X: up to 2^-12.2 of the
    sum of |products|), which moves large scores, and through them the LSE, by more than 1e-3."""
    B, S, Hq, _ = qv.shape
    G = Hq // kv.shape[2]
    edges = np.asarray(cu_seqlens if cu_seqlens is not None else [0, S], dtype=np.int64)
    seg = np.searchsorted(edges, np.arange(S), side="right") - 1
    vis = seg[:, None] == seg[None, :]
    if causal:
        vis &= np.tri(S, dtype=bool)
    out = np.empty((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            dots = np.abs(qv[b, :, h]) @ np.abs(kv[b, :, h // G]).T
            out[b, h] = TOL_LSE + 2.0 ** -11 * scale * np.where(vis, dots, 0.0).max(axis=1)
    return out


def check_fwd(o, lse, ro, rl, tag="", rel_tol=TOL_O_REL, abs_factor=1.0, bound=None):
    """O: |o - ref| <= max(1e-2, ulp_bf16(ref) / 2) (or the given per-element bound) and rel-L2 <= 5e-3 against
    the exact oracle; LSE max-abs <= 1e-3."""
    o = np.asarray(o, dtype=np.float64)
    raw = np.abs(o - ro)
    excess = raw / (abs_factor * o_bound(ro) if bound is None else bound)
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
