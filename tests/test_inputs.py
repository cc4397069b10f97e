"""Pins for the seeded input generators (storage-format rounding, packed lengths)."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 8, 100000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf], dtype=np.float32),
        # exact ties: bf16 keeps 8 significant bits, these sit halfway between two bf16 values
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32),
    ]).astype(np.float32)
    ours = si.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    np.testing.assert_array_equal(si.bf16_bits_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_e4m3_encoder_matches_torch_cast_with_saturation():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(50.0),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000).astype(np.float32),  # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 464.0, 500.0, -1e6, 2.0 ** -10, 2.0 ** -9 * 1.5], dtype=np.float32),
    ])
    ours = si.e4m3_encode(x)
    ref = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = si.e4m3_encode(vals)
    # +0 and -0 both decode to zero; the encoder keeps the sign bit
    assert np.array_equal(back, codes)


def test_e4m3_quantize_scale_and_saturation():
    x = np.random.default_rng(2).standard_normal(10000).astype(np.float32)
    codes, descale = si.e4m3_quantize(x)
    assert descale == np.float32(np.max(np.abs(x)) / np.float32(448.0))
    deq = oracle.e4m3_decode(codes) * float(descale)
    assert np.max(np.abs(deq)) <= 448.0 * float(descale) * (1 + 1e-7)
    # relative error of E4M3 rounding is at most 2^-4 for normal values
    big = np.abs(x) > 2.0 ** -6 * float(descale)
    assert np.max(np.abs(deq[big] - x[big]) / np.abs(x[big])) <= 2.0 ** -4 + 1e-7


def test_packed_lengths_seed4():
    rng = np.random.default_rng(4)
    lengths = si.packed_lengths(rng)
    assert lengths == [6091, 7755, 7282, 4439, 7201]
    for seed in range(200):
        ls = si.packed_lengths(np.random.default_rng(seed))
        assert sum(ls) == 32768
        assert all(512 <= x <= 8192 for x in ls)
    cu = si.cu_seqlens_from_lengths(lengths)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 32768


def test_workload_draws_are_deterministic():
    a = si.make_inputs(1, 2, 1, 64, 16, seed=9)
    b = si.make_inputs(1, 2, 1, 64, 16, seed=9)
    for n in ("q_bits", "k_bits", "v_bits", "do_bits"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    w = si.WORKLOADS["packed32k"]
    assert (w.hq, w.hkv, w.seqlen, w.head_dim) == (14, 2, 32768, 128)
    idx = si.sample_indices(3, 100, 10, must=(0, 99))
    assert idx[0] == 0 and idx[-1] == 99 and np.all(np.diff(idx) > 0)
