"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, the
visible-pair counts behind every TFLOP/s figure, and the source lists the
HBM-traffic records are keyed on."""
import os

import numpy as np
import pytest

import bench
import seeded_inputs as si


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _brute_pairs(S, causal, lengths=None):
    seg = np.zeros(S, dtype=int) if lengths is None else np.repeat(np.arange(len(lengths)), lengths)
    i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    ok = seg[i] == seg[j]
    if causal:
        ok &= j <= i
    return int(ok.sum())


def test_visible_pairs_match_brute_force():
    for S, causal, lengths in [(1, True, None), (7, True, None), (7, False, None), (64, True, None),
                               (20, True, [5, 1, 14]), (20, False, [5, 1, 14]), (9, True, [1] * 9)]:
        cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        assert bench._pairs(S, causal, cu) == _brute_pairs(S, causal, lengths), (S, causal, lengths)


def test_headline_flop_count():
    # gqa32k: 14 D flops per visible pair (4 forward + 10 backward), 28 query heads
    w = si.WORKLOADS["gqa32k"]
    pairs = bench._pairs(w.seqlen, True) * w.batch * w.hq
    assert pairs == 28 * 32768 * 32769 / 2
    assert abs(14 * 128 * pairs - 2.694e13) / 2.694e13 < 1e-3


def test_kernel_sources_exist_and_hash_stably():
    csrc = os.path.join(bench.ROOT, "long_context_exact_fwd_amd", "csrc")
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), (kernel, f)
        h = bench.kernel_source_hash(kernel)
        assert h == bench.kernel_source_hash(kernel) and len(h) >= 16
    assert set(bench.KERNEL_OF_PHASE.values()) <= set(bench.KERNEL_SOURCES)


def test_build_info_names_the_compile_flags():
    info = bench.build_info()
    assert info["arch"] == "gfx950" and "--offload-arch=gfx950" in info["flags"] and "-packed-fp32-ops" in info["flags"]
    assert not any(tok.startswith("/") for tok in info["flags"].split())


def test_counter_record_hash_ignores_comments_only():
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n/* note */\n"
    assert bench.code_text(code) == bench.code_text(code.replace("one more", "plus one").replace("note", "x"))
    assert bench.code_text(code) == bench.code_text(code.replace("\n", "\n\n  "))
    assert bench.code_text(code) != bench.code_text(code.replace("a + 1", "a + 2"))


def test_cpu_baseline_fields_and_extrapolation():
    """The CPU baseline reports threads and host cores apart, the CPU model, a single-thread time, the
    flops the oracle executes (12 D per pair) and whole-workload times labelled as extrapolated."""
    w = si.WORKLOADS["tiny"]
    x = si.workload_inputs(w)
    r = bench.cpu_baseline(w, x, sample_len=128, single_len=64)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["cores"] == r["threads"] >= 1 and r["host_cores"] >= 1 and r["affinity_cores"] >= 1
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    g = w.hq // w.hkv
    pairs = bench._pairs(128, w.causal) * g
    assert abs(r["value"] - 12.0 * w.head_dim * pairs / r["seconds"] / 1e12) <= 0.01 * r["value"]
    assert abs(r["value_14d_convention"] / r["value"] - 14.0 / 12.0) < 1e-9
    full = bench._pairs(w.seqlen, w.causal) * w.batch * w.hq
    ex = r["extrapolated_full_workload_s"]
    assert "extrapolated" in ex["note"]
    assert abs(ex["threads"] - r["seconds"] * full / pairs) <= 0.01 + 0.01 * ex["threads"]
    assert r["single_thread"]["seconds"] > 0 and r["single_thread"]["value"] > 0


def test_mfma_ceiling_probe_library_exports():
    """The ceiling probe is its own library (not part of the attention ABI); its flop count is 8 waves x
    8 chains x 2*32*32*16 per workgroup and iteration."""
    import ctypes
    from long_context_exact_fwd_amd import build as bld
    if not os.path.exists(bld.PROBE_LIB):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(bld.PROBE_LIB)
    lib.mfma_ceiling_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mfma_ceiling_flops.restype = ctypes.c_double
    assert lib.mfma_ceiling_flops(1, 1) == 8 * 8 * 2 * 32 * 32 * 16
    assert lib.mfma_ceiling_flops(256, 1000) == 256 * 1000 * 8 * 8 * 2 * 32 * 32 * 16
    lib.mfma_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.mfma_ceiling_launch.restype = ctypes.c_int
    # argument checks run before any HIP call
    assert lib.mfma_ceiling_launch(None, None, 1, 1, 1, None) == -1
    assert lib.mfma_ceiling_launch(ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), 0, 1, 1, None) == -1


@pytest.mark.gpu
def test_mfma_ceiling_probe_runs():
    import torch
    r = bench.mfma_ceiling_case(torch.device("cuda"), iters=2000, reps=2)
    print("mfma ceiling (short run):", r, flush=True)
    for k in (r, r["low_entropy_operands"]):
        assert 100.0 < k["tflops"] < 1.05 * bench.PEAK_BF16_TFLOPS
        assert 0.5 < k["clock_ghz"] < 3.0
