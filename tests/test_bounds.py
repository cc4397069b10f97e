"""CPU: the stress-input O bound (rounding_o_bound) holds for a model of the tiled forward's arithmetic.

The model follows the kernel's order of operations for one query row: scores in fp32, the first 64-key
tile's maximum kept as the running maximum, P_j = 2^(s_j c - m) in fp32, l = sum_j P_j unrounded,
O = bf16(sum_j bf16(P_j) V_j / l). On peaky inputs (Q and K scaled by 2.5-4, the inputs of the stress
tests) every modelled element must stay within the bound derived from that arithmetic, with the exact O
and the weighted |V| taken from the oracle. The bound would fail if its P term were 2^-9 instead of 2^-8
(checked too: the 2^-9 version is exceeded on these inputs), so the test pins the figure the stress
tests rely on.
"""
import numpy as np

import oracle
import seeded_inputs as si
from tests.gpu_helpers import bf16_ulp, rounding_o_bound


def _bf16(x):
    """Round to bfloat16 (nearest even), returned as float64."""
    a = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((a + 0x7FFF + ((a >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _model_forward(qv, kv, vv, scale):
    """The tiled kernel's arithmetic for a causal, unpacked call (B = 1, Hq = Hkv)."""
    _, S, H, D = qv.shape
    c = np.float32(scale * np.log2(np.e))
    out = np.empty((1, S, H, D))
    for h in range(H):
        q32, k32 = qv[0, :, h].astype(np.float32), kv[0, :, h].astype(np.float32)
        s = q32 @ k32.T                                               # fp32 scores
        for i in range(S):
            row = s[i, : i + 1]
            m = np.float32(row[:64].max() * c)                        # first tile's maximum, log2 units
            p = np.exp2(row * c - m).astype(np.float32)
            l = np.float64(p.astype(np.float32).sum(dtype=np.float32))
            out[0, i, h] = _bf16((_bf16(p) @ vv[0, : i + 1, h]) / l)
    return out


def test_stress_bound_holds_for_the_kernel_arithmetic():
    S, H, D = 300, 4, 64
    worst, worst_9 = 0.0, 0.0
    for seed, std in ((401, 2.5), (402, 3.0), (403, 4.0)):
        x = si.make_inputs(1, H, H, S, D, seed, with_do=False, qk_std=std)
        qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
        scale = 1.0 / np.sqrt(D)
        ro, _ = oracle.attention_fwd(qv, kv, vv, causal=True, scale=scale, workers=None)
        abar, _ = oracle.attention_fwd(qv, kv, np.abs(vv), causal=True, scale=scale, workers=None)
        o = _model_forward(qv, kv, vv, scale)
        err = np.abs(o - ro)
        worst = max(worst, float(np.max(err / rounding_o_bound(o, ro, abar))))
        bound_9 = 2.0 ** -9 * abar + 0.5 * bf16_ulp(np.maximum(np.abs(o), np.abs(ro))) + 1e-6
        worst_9 = max(worst_9, float(np.max(err / bound_9)))
    print(f"modelled O error: {worst:.3f} of the bound, {worst_9:.3f} of a bound with a 2^-9 P term", flush=True)
    assert worst <= 1.0
    assert worst_9 > 1.0
