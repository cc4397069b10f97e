"""Plausible oracle mistakes, planted on the CPU, must fail at least one pin.

Each case patches one step of the oracle, runs the pin that should catch it
and asserts that the pin now fails. The real oracle is restored afterwards
(monkeypatch), so nothing here changes what the other tests check.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests.test_oracle import _brute_fwd, _ev, _rand

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_fails():
    with open(os.path.join(GOLDEN, "hand_worked_s3.json"), encoding="utf-8") as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.array(g["k"], dtype=np.float64)[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    for kind in ("causal", "noncausal"):
        with np.errstate(all="ignore"):
            o, lse = oracle.attention_fwd(q, k, v, causal=(kind == "causal"), scale=g["scale"])
        want_o = np.array([[_ev(x) for x in row] for row in g[kind]["o"]])
        want_l = np.array([_ev(x) for x in g[kind]["lse"]])
        if not (np.allclose(o[0, :, 0], want_o, atol=1e-12) and np.allclose(lse[0, 0], want_l, atol=1e-12)):
            return True
    return False


def _brute_fails():
    S, D = 12, 3
    q, k, v = _rand((1, S, 4, D), 1), _rand((1, S, 2, D), 2), _rand((1, S, 2, D), 3)
    for causal in (True, False):
        with np.errstate(all="ignore"):
            o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=0.4)
        bo, bl = _brute_fwd(q, k, v, causal, 0.4, None)
        if not (np.allclose(o, bo, atol=1e-12) and np.allclose(lse, bl, atol=1e-12)):
            return True
    return False


def _fd_fails():
    S, D = 10, 3
    q, k, v, do = _rand((1, S, 2, D), 4), _rand((1, S, 1, D), 5), _rand((1, S, 1, D), 6), _rand((1, S, 2, D), 7)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.5)
    h = 1e-6
    rng = np.random.default_rng(8)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            args = {"q": q, "k": k, "v": v}
            xp = x.copy()
            xp[idx] += h
            args[name] = xp
            lp = float(np.sum(oracle.attention_fwd(args["q"], args["k"], args["v"], causal=True, scale=0.5)[0] * do))
            xm = x.copy()
            xm[idx] -= h
            args[name] = xm
            lm = float(np.sum(oracle.attention_fwd(args["q"], args["k"], args["v"], causal=True, scale=0.5)[0] * do))
            if abs((lp - lm) / (2 * h) - g[idx]) > 1e-6 * max(1.0, abs(g[idx])):
                return True
    return False


def _probs_variant(kind):
    real = A._block_probs

    def f(qb, kk, rows, klo, lo, hi, scale):
        if kind == "causal_off_by_one":  # j < i instead of j <= i (keeping at least one key per row)
            hi = np.where(hi == rows + 1, np.maximum(rows, lo + 1), hi)
        if kind == "double_scale":
            scale = scale * scale
        p, lse = real(qb, kk, rows, klo, lo, hi, scale)
        if kind == "log2_lse":
            lse = lse / math.log(2.0)
        if kind == "no_max_shift_in_lse":
            m = np.max(np.where(np.isfinite(p), scale * (qb @ kk.T), -np.inf), axis=1)
            lse = lse - m
        return p, lse
    return f


@pytest.mark.parametrize("kind", ["causal_off_by_one", "double_scale", "log2_lse", "no_max_shift_in_lse"])
def test_forward_mutations_are_caught(kind, monkeypatch):
    monkeypatch.setattr(A, "_block_probs", _probs_variant(kind))
    assert _golden_fails() or _brute_fails()


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    # interleaved grouping (h % G) instead of consecutive groups (h // G)
    monkeypatch.setattr(A, "_kv_head", lambda h, group: h % group)
    assert _brute_fails()


@pytest.mark.parametrize("kind", ["drop_delta", "dq_without_scale", "dv_from_dp", "dk_sign"])
def test_backward_mutations_are_caught(kind, monkeypatch):
    def mutated(qb, kk, vv, dob, rows, klo, lo, hi, scale):
        p, _ = A._block_probs(qb, kk, rows, klo, lo, hi, scale)
        ob = p @ vv
        delta = np.sum(dob * ob, axis=1)
        if kind == "drop_delta":
            delta = 0.0 * delta
        dp = dob @ vv.T
        ds = p * (dp - delta[:, None])
        dq = (1.0 if kind == "dq_without_scale" else scale) * (ds @ kk)
        dk = scale * (ds.T @ qb) * (-1.0 if kind == "dk_sign" else 1.0)
        dv = (dp.T if kind == "dv_from_dp" else p.T) @ dob
        return dq, dk, dv

    monkeypatch.setattr(A, "_bwd_rows_block", mutated)
    assert _fd_fails()


def _merge_pins_fail():
    from tests import test_oracle as T
    for fn, args in ((T.test_merge_of_key_chunks_equals_full_attention, (3, 2, 1)),
                     (T.test_ring_layout_causal, (4,)), (T.test_merge_brute_force_two_rows, ())):
        try:
            with np.errstate(all="ignore"):
                fn(*args)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("kind", ["unnormalised", "swapped_weights", "lse_is_max", "weight_sign"])
def test_merge_mutations_are_caught(kind, monkeypatch):
    real = A.merge_partials

    def mutated(o1, l1, o2, l2):
        o1, o2 = np.asarray(o1, dtype=np.float64), np.asarray(o2, dtype=np.float64)
        l1, l2 = np.asarray(l1, dtype=np.float64), np.asarray(l2, dtype=np.float64)
        if kind == "lse_is_max":
            o, _ = real(o1, l1, o2, l2)
            return o, np.maximum(l1, l2)
        m = np.maximum(l1, l2)
        sgn = -1.0 if kind == "weight_sign" else 1.0
        w1, w2 = np.exp(sgn * (l1 - m)), np.exp(sgn * (l2 - m))
        if kind == "swapped_weights":
            w1, w2 = w2, w1
        tot = w1 + w2
        norm = 1.0 if kind == "unnormalised" else tot
        a1 = np.transpose(w1 / norm, (0, 2, 1))[..., None]
        a2 = np.transpose(w2 / norm, (0, 2, 1))[..., None]
        return a1 * o1 + a2 * o2, m + np.log(tot)

    monkeypatch.setattr(oracle, "merge_partials", mutated)
    assert _merge_pins_fail()
