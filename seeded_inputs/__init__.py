"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This module draws random numbers and rounds them into the storage formats the
kernels consume (bf16, OCP FP8 E4M3FN with a per-tensor fp32 scale, int32
``cu_seqlens`` for packed sequences). It holds none of the attention
arithmetic: no scores, no softmax, no products of Q, K or V.

Workloads (shapes follow the long-context fine-tuning setups of the pages
"ms-swift长文本训练秘诀：Ulysses并行技术解析" §3/§5 (Qwen2.5-7B, 32K, packed
documents) and "ms-swift集成FlashAttention 2/3，长文本训练更高效" (FA-2/FA-3
table at 8K and 32K); the activations themselves are N(0, 1) stand-ins because
the pages' datasets and weights are not available):

  tiny       B=1 H=2        S=256   D=64   seed 1  causal and non-causal, fwd+bwd
  mid        B=2 H=32       S=8192  D=128  seed 2  causal, fwd
  gqa32k     B=1 Hq=28 Hkv=4 S=32768 D=128 seed 3  causal, fwd+bwd
  packed32k  B=1 Hq=14 Hkv=2 S=32768 D=128 seed 4  packed causal, fwd+bwd
  fp8_64k    B=1 Hq=8 Hkv=1 S=65536 D=128  seed 5  causal, fp8 fwd

Draw order for every workload: (packed only) the segment lengths, then Q, K,
V, dO, each ``standard_normal(shape, dtype=float32)`` in [B, S, H, D] order
from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# storage-format rounding (no attention arithmetic)
# ----------------------------------------------------------------------------


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def _e4m3_positive_table() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3FN codes 0x00..0x7E (index = code)."""
    vals = np.zeros(127, dtype=np.float64)
    for code in range(127):
        e = code >> 3
        m = code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as OCP FP8 E4M3FN codes (uint8).

    Round to nearest, ties to the even code; magnitudes beyond 448 saturate to
    448 (the format has no infinity). NaN maps to 0x7F.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.minimum(a, E4M3_MAX)
    # index of the largest table value <= a
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    vlo = _E4M3_POS[lo]
    vhi = _E4M3_POS[hi]
    dlo = a - vlo
    dhi = vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((lo & 1) == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    out = code | sign
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, np.uint8(0x7F), out)
    return out.astype(np.uint8)


def e4m3_quantize(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-tensor scaled E4M3 quantisation: descale = amax / 448 (fp32), codes = E4M3(x / descale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    descale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    codes = e4m3_encode((x / descale).astype(np.float32))
    return codes, descale


# ----------------------------------------------------------------------------
# packed sequence lengths
# ----------------------------------------------------------------------------


def packed_lengths(rng: np.random.Generator, total: int = 32768, lo: int = 512, hi: int = 8192) -> list[int]:
    """Random segment lengths, each in [lo, hi], summing to ``total``.

    Draw a length uniform in [lo, min(hi, R - lo)] while the remainder R
    exceeds hi; the remainder is the last segment.
    """
    out: list[int] = []
    rem = total
    while rem > hi:
        length = int(rng.integers(lo, min(hi, rem - lo) + 1))
        out.append(length)
        rem -= length
    out.append(rem)
    return out


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    c = np.zeros(len(lengths) + 1, dtype=np.int32)
    c[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return c


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    seqlen: int
    head_dim: int
    seed: int
    causal: bool
    packed: bool = False
    fp8: bool = False
    backward: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 256, 64, 1, causal=True),
    "mid": Workload("mid", 2, 32, 32, 8192, 128, 2, causal=True, backward=False),
    "gqa32k": Workload("gqa32k", 1, 28, 4, 32768, 128, 3, causal=True),
    "packed32k": Workload("packed32k", 1, 14, 2, 32768, 128, 4, causal=True, packed=True),
    "fp8_64k": Workload("fp8_64k", 1, 8, 1, 65536, 128, 5, causal=True, fp8=True, backward=False),
}


@dataclasses.dataclass
class Inputs:
    """Host-side inputs. ``*_bits`` are uint16 bf16 patterns or uint8 E4M3 codes."""

    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    do_bits: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    descale: Optional[tuple]  # (q, k, v) fp32 descales for fp8 inputs
    fp8: bool

    def values(self, name: str) -> np.ndarray:
        """Exact float64 value of an input as the kernels consume it."""
        bits = getattr(self, name + "_bits")
        if self.fp8 and name in ("q", "k", "v"):
            raise ValueError("fp8 inputs: decode with the oracle's own E4M3 decoder")
        return bf16_bits_to_f64(bits)


def make_inputs(batch: int, hq: int, hkv: int, seqlen: int, head_dim: int, seed: int,
                lengths=None, random_lengths: bool = False, fp8: bool = False,
                with_do: bool = True, qk_std: float = 1.0) -> Inputs:
    """Draw Q, K, V, dO ~ N(0, 1) in [B, S, H, D] and round them to the kernel formats.

    ``qk_std`` multiplies Q and K only (sharper softmax rows, V unchanged).
    """
    rng = np.random.default_rng(seed)
    cu = None
    if random_lengths:
        lengths = packed_lengths(rng, total=seqlen)
    if lengths is not None:
        if batch != 1:
            raise ValueError("packed sequences need batch == 1")
        cu = cu_seqlens_from_lengths(lengths)
        if int(cu[-1]) != seqlen:
            raise ValueError("lengths must sum to seqlen")
    q = rng.standard_normal((batch, seqlen, hq, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, seqlen, hkv, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, seqlen, hkv, head_dim), dtype=np.float32)
    if qk_std != 1.0:
        q *= np.float32(qk_std)
        k *= np.float32(qk_std)
    do = rng.standard_normal((batch, seqlen, hq, head_dim), dtype=np.float32) if with_do else None
    if fp8:
        q8, dq = e4m3_quantize(q)
        k8, dk = e4m3_quantize(k)
        v8, dv = e4m3_quantize(v)
        return Inputs(q8, k8, v8, None if do is None else bf16_bits_from_f32(do), cu, (dq, dk, dv), True)
    return Inputs(bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v),
                  None if do is None else bf16_bits_from_f32(do), cu, None, False)


def workload_inputs(w: Workload, with_do: Optional[bool] = None) -> Inputs:
    if with_do is None:
        with_do = w.backward
    return make_inputs(w.batch, w.hq, w.hkv, w.seqlen, w.head_dim, w.seed,
                       random_lengths=w.packed, fp8=w.fp8, with_do=with_do)


def sample_indices(seed: int, n: int, count: int, must=()) -> np.ndarray:
    """Sorted unique indices in [0, n): the ``must`` ones plus ``count`` seeded uniform draws."""
    rng = np.random.default_rng(seed + 1000003)
    s = set(int(i) for i in must if 0 <= int(i) < n)
    if count > 0 and n > 0:
        s.update(int(i) for i in rng.integers(0, n, size=count))
    return np.array(sorted(s), dtype=np.int64)
