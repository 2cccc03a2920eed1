"""Pins for the oracle's gate + hard Top-K (CPU only).

Each test checks the oracle against something other than itself: scipy's
softmax, a brute-force full sort, closed forms (rows sum to one, shift
invariance) and hand-worked examples in tests/golden.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from trainable_block_sparse_gate_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def brute_topk(s, i, k):
    """Full sort by (score descending, index ascending); keep k, ascending."""
    order = sorted(range(i), key=lambda j: (-float(s[j]), j))
    return sorted(order[:k])


def rows_of(cu, blk):
    """(sequence, local block) for each global query block."""
    out = []
    for s in range(len(cu) - 1):
        nb = (cu[s + 1] - cu[s] + blk - 1) // blk
        out += [(s, i) for i in range(nb)]
    return out


def _case(lengths, hkv, ld_extra=0, seed=0, blk=4, sigma=2.0, kind="normal"):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    nb = [(n + blk - 1) // blk for n in lengths]
    QB, ld = sum(nb), max(nb) + ld_extra
    g = np.random.default_rng(seed)
    if kind == "normal":
        lg = g.normal(0, sigma, (hkv, QB, ld)).astype(np.float32)
    elif kind == "ties":
        lg = g.integers(-2, 3, (hkv, QB, ld)).astype(np.float32)
    elif kind == "zeros_signed":
        lg = np.where(g.random((hkv, QB, ld)) < 0.5, -0.0, 0.0).astype(np.float32)
        lg[g.random((hkv, QB, ld)) < 0.3] = 1.0
    elif kind == "neginf":
        lg = g.normal(0, sigma, (hkv, QB, ld)).astype(np.float32)
        lg[g.random((hkv, QB, ld)) < 0.4] = -np.inf
    return cu, lg, QB


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros_signed", "neginf"])
@pytest.mark.parametrize("Kb", [1, 2, 3, 5, 40])
@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL, oracle.GATE_SIGMOID,
                                  oracle.GATE_RAW, oracle.GATE_STE])
def test_topk_matches_brute_force(kind, Kb, mode):
    lengths = [37, 4, 64, 1, 23]
    blk = 4
    cu, lg, QB = _case(lengths, 2, ld_extra=3, seed=Kb * 7 + mode, blk=blk, kind=kind)
    if kind == "neginf" and mode == oracle.GATE_ALL:
        lg[np.isinf(lg)] = -30.0  # the all-softmax reading needs a finite current logit
    idx, _, _ = oracle.gate_topk(cu, lg, 2, Kb, mode, blk=blk)
    for g in range(2):
        for Q, (s, i) in enumerate(rows_of(cu, blk)):
            k = min(Kb - 1, i)
            want = brute_topk(lg[g, Q], i, k) + [i]
            want += [-1] * (Kb - len(want))
            assert idx[g, Q].tolist() == want, (g, Q, i)


@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL])
def test_gates_sum_to_one_when_everything_is_kept(mode):
    lengths = [50, 17]
    blk = 4
    cu, lg, QB = _case(lengths, 3, seed=3, blk=blk)
    idx, sl, lse = oracle.gate_topk(cu, lg, 3, Kb=64, mode=mode, blk=blk)
    for g in range(3):
        for Q, (s, i) in enumerate(rows_of(cu, blk)):
            n = i + 1
            gates = np.exp(sl[g, Q, :n])
            if mode == oracle.GATE_HIST:
                assert sl[g, Q, i] == 0.0  # current block keeps gate 1
                if i > 0:
                    assert abs(gates[:i].sum() - 1.0) < 1e-12
                else:
                    assert lse[g, Q] == -np.inf
            else:
                assert abs(gates.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL])
def test_kept_gates_match_scipy_softmax(mode):
    lengths = [64, 41]
    blk = 4
    cu, lg, QB = _case(lengths, 2, seed=11, blk=blk, sigma=3.0)
    Kb = 4
    idx, sl, lse = oracle.gate_topk(cu, lg, 2, Kb, mode, blk=blk)
    for g in range(2):
        for Q, (s, i) in enumerate(rows_of(cu, blk)):
            n = i + (1 if mode == oracle.GATE_ALL else 0)
            if n == 0:
                continue
            p = softmax(lg[g, Q, :n].astype(np.float64))
            for slot in range(Kb):
                j = idx[g, Q, slot]
                if j < 0:
                    assert sl[g, Q, slot] == -np.inf
                    continue
                if j == i and mode == oracle.GATE_HIST:
                    assert sl[g, Q, slot] == 0.0
                else:
                    assert abs(math.exp(sl[g, Q, slot]) - p[j]) < 1e-12


@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL])
def test_shift_invariance(mode):
    """The normalised gate is invariant to adding one constant to all of a
    row's scores (paper text, ablation results: the page titled "SAS: Simple Attention Sparsification via End-to-End Optimization of Context Ranking")."""
    lengths = [100, 30]
    blk = 4
    cu, lg, QB = _case(lengths, 2, seed=5, blk=blk)
    lg = (np.round(lg * 256) / 256).astype(np.float32)  # so that +c is exact
    shifted = (lg + np.float32(3.0)).astype(np.float32)
    assert np.all(shifted - np.float32(3.0) == lg)
    a = oracle.gate_topk(cu, lg, 2, 6, mode, blk=blk)
    b = oracle.gate_topk(cu, shifted, 2, 6, mode, blk=blk)
    assert np.array_equal(a[0], b[0])
    fin = np.isfinite(a[1])
    assert np.array_equal(fin, np.isfinite(b[1]))
    assert np.max(np.abs(a[1][fin] - b[1][fin])) < 1e-12


def test_all_minus_inf_history_gives_zero_gates():
    s = np.array([-np.inf, -np.inf, -np.inf, 0.0], np.float32)
    idx, sl, lse = oracle.gate_row(s, 3, 3)
    assert idx.tolist() == [0, 1, 3]
    assert sl[0] == -np.inf and sl[1] == -np.inf and sl[2] == 0.0
    assert lse == -np.inf


def test_golden_gate_examples():
    cases = json.load(open(GOLDEN))["gate"]
    for c in cases:
        if "logits_ln_of" in c:
            s = np.log(np.array(c["logits_ln_of"], np.float64)).astype(np.float32)
        else:
            s = np.array(c["logits"], np.float32)
        mode = oracle.GATE_ALL if c["mode"] == "all" else oracle.GATE_HIST
        idx, sl, lse = oracle.gate_row(s, c["i"], c["Kb"], mode)
        assert idx.tolist() == c["expect_idx"], c["name"]
        if "expect_gates" in c:
            assert np.allclose(np.exp(sl), c["expect_gates"], atol=1e-6), c["name"]
        if "expect_lse_exp" in c:
            assert abs(math.exp(lse) - c["expect_lse_exp"]) < 1e-5, c["name"]


def test_workload_logits_layout_and_boost():
    """The varlen workload's boosted columns are the same for every row of a
    (sequence, kv head); check that the generator did what it says."""
    case = wl.make_varlen("t", [256, 128], 4, 2, 8, 4, dtype="f32", logit_sigma=3.0,
                          workload_id=99, boost_frac=0.05, ld=4)
    assert case.logits.shape == (2, 6, 4)
    for s, per_head in enumerate(case.boosted):
        for cols in per_head:
            assert len(cols) == 1


@pytest.mark.parametrize("mode", [oracle.GATE_SIGMOID, oracle.GATE_RAW])
def test_independent_activations_match_closed_forms(mode):
    """The activation ablations (paper text section 4, review 3-3): kept
    history blocks get log sigmoid(s) or s itself, the current block log-gate
    0, padding -inf; there is no normaliser (gate_lse 0).  The expected values
    are written here from the definitions with the math module."""
    lengths = [37, 23]
    blk, Kb = 4, 4
    cu, lg, QB = _case(lengths, 2, ld_extra=2, seed=11 + mode, blk=blk)
    lg[0, 5, 1] = -np.inf  # an infinite logit: gate 0 (log -inf) in both modes
    idx, sl, lse = oracle.gate_topk(cu, lg, 2, Kb, mode, blk=blk)
    assert np.all(lse == 0.0)
    for g in range(2):
        for Q, (s, i) in enumerate(rows_of(cu, blk)):
            k = min(Kb - 1, i)
            for sl_i in range(Kb):
                j = int(idx[g, Q, sl_i])
                if sl_i < k:
                    x = float(lg[g, Q, j])
                    if mode == oracle.GATE_RAW:
                        want = x
                    elif x == -math.inf:
                        want = -math.inf
                    else:
                        want = -math.log(1.0 + math.exp(-x))
                    assert sl[g, Q, sl_i] == pytest.approx(want, rel=1e-14, abs=1e-14)
                elif sl_i == k:
                    assert j == i and sl[g, Q, sl_i] == 0.0
                else:
                    assert j == -1 and sl[g, Q, sl_i] == -math.inf
