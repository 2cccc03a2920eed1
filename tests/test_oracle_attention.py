"""Pins for the oracle's gated block-sparse forward and backward (CPU only).

Checks against torch's SDPA (a library routine, float64, additive mask),
dense causal attention, the softmax/log-gate identity, central finite
differences and exact invariants of the gradients.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.dense_reference import dlg_from_mask_grad, gate_mask, sdpa_sequence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def small_problem(lengths, hq, hkv, d, Kb, blk, seed, mode=oracle.GATE_HIST, sigma=2.0):
    g = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    nb = [(n + blk - 1) // blk for n in lengths]
    QB = sum(nb)
    q = g.normal(size=(T, hq, d))
    k = g.normal(size=(T, hkv, d))
    v = g.normal(size=(T, hkv, d))
    dO = g.normal(size=(T, hq, d))
    logits = g.normal(0, sigma, (hkv, QB, max(nb))).astype(np.float32)
    idx, sl, _ = oracle.gate_topk(cu, logits, hkv, Kb, mode, blk=blk)
    return dict(cu=cu, q=q, k=k, v=v, dO=dO, logits=logits, idx=idx, sl=sl, Kb=Kb, blk=blk,
                hq=hq, hkv=hkv, d=d, scale=1.0 / math.sqrt(d))


CASES = [
    # lengths, hq, hkv, d, Kb, blk
    ([29, 8, 17], 4, 2, 8, 3, 4),
    ([40], 2, 1, 8, 2, 4),
    ([33, 5], 8, 2, 8, 4, 4),
    ([24, 24], 4, 4, 16, 2, 8),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL])
def test_fwd_bwd_match_torch_sdpa_with_gate_mask(case, mode):
    lengths, hq, hkv, d, Kb, blk = CASES[case]
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=case, mode=mode)
    o, lse = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], P["sl"], Kb, P["scale"],
                        blk=blk)
    dq, dk, dv, dlg = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"], P["sl"],
                                 Kb, P["scale"], blk=blk)
    cu = P["cu"]
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        M = gate_mask(cu, P["idx"], P["sl"], hkv, blk, s)
        ref = sdpa_sequence(P["q"][a:b], P["k"][a:b], P["v"][a:b], M, P["scale"],
                            dO=P["dO"][a:b])
        assert np.max(np.abs(o[a:b] - ref["o"])) < 1e-12
        assert np.max(np.abs(lse[:, a:b] - ref["lse"])) < 1e-12
        assert np.max(np.abs(dq[a:b] - ref["dq"])) < 1e-11
        assert np.max(np.abs(dk[a:b] - ref["dk"])) < 1e-11
        assert np.max(np.abs(dv[a:b] - ref["dv"])) < 1e-11
        nb = (b - a + blk - 1) // blk
        qb0 = sum((cu[x + 1] - cu[x] + blk - 1) // blk for x in range(s))
        want = dlg_from_mask_grad(ref["dM"], cu, P["idx"], hkv, blk, s)
        assert np.max(np.abs(dlg[:, qb0:qb0 + nb] - want)) < 1e-11


def test_dense_special_case_equals_causal_attention():
    """Gates all 1 and a budget covering every block: plain causal attention
    (review section 1-1, dense attention equation)."""
    lengths, hq, hkv, d, blk = [45, 21], 4, 2, 8, 4
    P = small_problem(lengths, hq, hkv, d, 64, blk, seed=9)
    idx = P["idx"]
    assert np.all(idx[..., :1] >= 0)
    zero = np.where(idx >= 0, 0.0, -np.inf)
    o, lse = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], idx, zero, 64, P["scale"], blk=blk)
    cu = P["cu"]
    G = hq // hkv
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        qt = torch.tensor(P["q"][a:b]).permute(1, 0, 2)
        kt = torch.tensor(P["k"][a:b]).permute(1, 0, 2).repeat_interleave(G, 0)
        vt = torch.tensor(P["v"][a:b]).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[None], kt[None], vt[None], is_causal=True, scale=P["scale"])[0]
        assert np.max(np.abs(o[a:b] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_log_gate_equals_multiplicative_reweighting():
    """softmax(a + log g) = g e^a / sum_j g_j e^a_j (review section 2-2)."""
    lengths, hq, hkv, d, Kb, blk = [36], 2, 1, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=4)
    g = np.random.default_rng(1).uniform(0.05, 1.0, P["idx"].shape)
    lg = np.where(P["idx"] >= 0, np.log(g), -np.inf)
    o, _ = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], lg, Kb, P["scale"], blk=blk)
    for t in range(36):
        i = t // blk
        for h in range(hq):
            num = np.zeros(d)
            den = 0.0
            for slot in range(Kb):
                j = P["idx"][0, i, slot]
                if j < 0:
                    continue
                for u in range(j * blk, min(j * blk + blk, t + 1)):
                    w = g[0, i, slot] * math.exp(P["scale"] * P["q"][t, h] @ P["k"][u, 0])
                    num += w * P["v"][u, 0]
                    den += w
            assert np.max(np.abs(o[t, h] - num / den)) < 1e-12


def test_varlen_sequences_are_isolated():
    lengths, hq, hkv, d, Kb, blk = [23, 30], 2, 1, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=8)
    o, lse = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], P["sl"], Kb, P["scale"],
                        blk=blk)
    # second sequence alone
    a = 23
    nb0 = (23 + blk - 1) // blk
    o2, lse2 = oracle.fwd(np.array([0, 30], np.int32), P["q"][a:], P["k"][a:], P["v"][a:],
                          P["idx"][:, nb0:], P["sl"][:, nb0:], Kb, P["scale"], blk=blk)
    assert np.array_equal(o[a:], o2)
    assert np.array_equal(lse[:, a:], lse2)


def _loss(P, q, k, v, sl):
    o, _ = oracle.fwd(P["cu"], q, k, v, P["idx"], sl, P["Kb"], P["scale"], blk=P["blk"])
    return float(np.sum(o * P["dO"]))


def test_bwd_matches_central_finite_differences():
    lengths, hq, hkv, d, Kb, blk = [21, 10], 4, 2, 4, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=12)
    dq, dk, dv, dlg = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"], P["sl"],
                                 Kb, P["scale"], blk=blk)
    h = 1e-6
    g = np.random.default_rng(0)
    for name, arr, grad in (("q", P["q"], dq), ("k", P["k"], dk), ("v", P["v"], dv)):
        for _ in range(12):
            pos = tuple(int(g.integers(0, n)) for n in arr.shape)
            xp, xm = arr.copy(), arr.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = {"q": P["q"], "k": P["k"], "v": P["v"]}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (_loss(P, args_p["q"], args_p["k"], args_p["v"], P["sl"]) -
                  _loss(P, args_m["q"], args_m["k"], args_m["v"], P["sl"])) / (2 * h)
            assert abs(fd - grad[pos]) < 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    for pos in zip(*np.nonzero(P["idx"] >= 0)):
        sp, sm = P["sl"].copy(), P["sl"].copy()
        sp[pos] += h
        sm[pos] -= h
        fd = (_loss(P, P["q"], P["k"], P["v"], sp) - _loss(P, P["q"], P["k"], P["v"], sm)) / (2 * h)
        assert abs(fd - dlg[pos]) < 1e-7 * max(1.0, abs(fd)), (pos, fd, dlg[pos])


def test_bwd_invariants():
    """Per row the log-gate gradients sum to 0 (sum_u dS_tu = 0) and the value
    gradients of one (sequence, kv head) sum to the sum of dO over its query
    heads (every softmax row sums to one)."""
    lengths, hq, hkv, d, Kb, blk = [64, 40], 4, 2, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=2)
    dq, dk, dv, dlg = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"], P["sl"],
                                 Kb, P["scale"], blk=blk)
    assert np.max(np.abs(dlg.sum(-1))) < 1e-12
    cu = P["cu"]
    G = hq // hkv
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        for g in range(hkv):
            want = P["dO"][a:b, g * G:(g + 1) * G].sum(axis=(0, 1))
            assert np.max(np.abs(dv[a:b, g].sum(0) - want)) < 1e-10


def test_gradient_reaches_only_the_kept_blocks():
    """Sparse scope (review section 3-5): with dO nonzero on one query block
    only, dk and dv are nonzero exactly on that row's kept blocks."""
    lengths, hq, hkv, d, Kb, blk = [64], 4, 2, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=21)
    i = 13
    dO = np.zeros_like(P["dO"])
    dO[i * blk:(i + 1) * blk] = P["dO"][i * blk:(i + 1) * blk]
    _, dk, dv, _ = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], dO, P["idx"], P["sl"], Kb,
                              P["scale"], blk=blk)
    for g in range(hkv):
        kept = set(int(j) for j in P["idx"][g, i] if j >= 0)
        assert len(kept) == Kb
        for j in range(16):
            nz = np.any(dk[j * blk:(j + 1) * blk, g] != 0) or np.any(dv[j * blk:(j + 1) * blk, g] != 0)
            assert nz == (j in kept), (g, j)


def test_row_and_key_masks_select_outputs():
    lengths, hq, hkv, d, Kb, blk = [48, 20], 4, 2, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=6)
    full = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"], P["sl"], Kb,
                      P["scale"], blk=blk)
    QB = P["idx"].shape[1]
    rm = np.zeros((hkv, QB), np.uint8)
    km = np.zeros((hkv, QB), np.uint8)
    rm[1, 3] = rm[0, 13] = 1
    km[0, 0] = km[1, 12] = 1
    part = oracle.bwd(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"], P["sl"], Kb,
                      P["scale"], row_mask=rm, kblk_mask=km, blk=blk)
    assert np.array_equal(part[3][rm.astype(bool)], full[3][rm.astype(bool)])
    # key block 0 of sequence 0 (head 0) and key block 0 of sequence 1 (head 1, global block 12)
    assert np.array_equal(part[1][0:4, 0], full[1][0:4, 0])
    assert np.array_equal(part[2][48:52, 1], full[2][48:52, 1])
    o_full, _ = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], P["sl"], Kb, P["scale"],
                           blk=blk)
    o_part, _ = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], P["sl"], Kb, P["scale"],
                           row_mask=rm, blk=blk)
    assert np.array_equal(o_part[12:16, 2:4], o_full[12:16, 2:4])


def test_golden_attention_example():
    c = json.load(open(GOLDEN))["attention"][0]
    blk, d, Kb = c["block"], c["d"], c["Kb"]
    T = len(c["q"])
    q = np.array(c["q"]).reshape(T, 1, d)
    k = np.array(c["k"]).reshape(T, 1, d)
    v = np.array(c["v"]).reshape(T, 1, d)
    idx = np.array(c["row_sel"], np.int32)[None]
    gates = np.array(c["row_gates"])[None]
    with np.errstate(divide="ignore"):
        lg = np.where(idx >= 0, np.log(gates), -np.inf)
    o, lse = oracle.fwd(np.array([0, T], np.int32), q, k, v, idx, lg, Kb, 1.0, blk=blk)
    assert np.allclose(o[:, 0, 0], c["expect_o"], atol=1e-12)
    assert np.allclose(np.exp(lse[0]), c["expect_lse_exp"], atol=1e-12)


# ----------------------------------------------------------------- outer gate
def _outer_sdpa_reference(P, sl):
    """Outer gate through torch SDPA (float64): per query block, the keys'
    values scaled by the row's gates, the mask free of any gate (0 on the
    attended keys, -inf elsewhere)."""
    cu, blk, hkv, hq = P["cu"], P["blk"], P["hkv"], P["hq"]
    G = hq // hkv
    T, d = P["q"].shape[0], P["d"]
    o = np.zeros((T, hq, d))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        ones = np.where(P["idx"] >= 0, 0.0, -np.inf)
        M = gate_mask(cu, P["idx"], ones, hkv, blk, s)  # attended keys only, no gate
        qb0 = sum((int(cu[x + 1]) - int(cu[x]) + blk - 1) // blk for x in range(s))
        for i in range((L + blk - 1) // blk):
            t0, t1 = i * blk, min((i + 1) * blk, L)
            r = qb0 + i
            for g in range(hkv):
                gate = np.zeros(L)
                for slot in range(P["Kb"]):
                    j = int(P["idx"][g, r, slot])
                    if j >= 0:
                        gate[j * blk:min((j + 1) * blk, L)] = math.exp(sl[g, r, slot])
                vg = torch.tensor(P["v"][a:b, g] * gate[:, None])
                kg = torch.tensor(P["k"][a:b, g])
                for hh in range(G):
                    h = g * G + hh
                    qt = torch.tensor(P["q"][a + t0:a + t1, h])
                    mask = torch.tensor(M[g, t0:t1])
                    out = torch.nn.functional.scaled_dot_product_attention(
                        qt[None], kg[None], vg[None], attn_mask=mask[None], scale=P["scale"])[0]
                    o[a + t0:a + t1, h] = out.numpy()
    return o


@pytest.mark.parametrize("case", range(len(CASES)))
def test_outer_gate_fwd_matches_sdpa_with_scaled_values(case):
    """The gate-position ablation (review 3-2 outer-gate equation): softmax
    of the ungated logits times the gate-scaled values."""
    lengths, hq, hkv, d, Kb, blk = CASES[case]
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=40 + case)
    o, lse = oracle.fwd_outer(P["cu"], P["q"], P["k"], P["v"], P["idx"], P["sl"], Kb, P["scale"],
                              blk=blk)
    ref = _outer_sdpa_reference(P, P["sl"])
    assert np.max(np.abs(o - ref)) < 1e-12
    # lse is that of the ungated logits: the inner forward with zero gates
    zero = np.where(P["idx"] >= 0, 0.0, -np.inf)
    _, lse0 = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], zero, Kb, P["scale"], blk=blk)
    assert np.max(np.abs(lse - lse0)) < 1e-12


def test_outer_gate_with_unit_gates_equals_inner_gate():
    lengths, hq, hkv, d, Kb, blk = [29, 8, 17], 4, 2, 8, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=51)
    zero = np.where(P["idx"] >= 0, 0.0, -np.inf)
    o1, l1 = oracle.fwd_outer(P["cu"], P["q"], P["k"], P["v"], P["idx"], zero, Kb, P["scale"], blk=blk)
    o2, l2 = oracle.fwd(P["cu"], P["q"], P["k"], P["v"], P["idx"], zero, Kb, P["scale"], blk=blk)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


def test_outer_gate_bwd_matches_central_finite_differences():
    lengths, hq, hkv, d, Kb, blk = [21, 10], 4, 2, 4, 3, 4
    P = small_problem(lengths, hq, hkv, d, Kb, blk, seed=13)
    dq, dk, dv, dlg = oracle.bwd_outer(P["cu"], P["q"], P["k"], P["v"], P["dO"], P["idx"],
                                       P["sl"], Kb, P["scale"], blk=blk)

    def loss(q, k, v, sl):
        o, _ = oracle.fwd_outer(P["cu"], q, k, v, P["idx"], sl, Kb, P["scale"], blk=blk)
        return float(np.sum(o * P["dO"]))

    h = 1e-6
    g = np.random.default_rng(1)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(12):
            pos = tuple(int(g.integers(0, n)) for n in P[name].shape)
            args_p = {"q": P["q"], "k": P["k"], "v": P["v"]}
            args_m = dict(args_p)
            xp, xm = P[name].copy(), P[name].copy()
            xp[pos] += h
            xm[pos] -= h
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"], P["sl"]) -
                  loss(args_m["q"], args_m["k"], args_m["v"], P["sl"])) / (2 * h)
            assert abs(fd - grad[pos]) < 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    for pos in zip(*np.nonzero(P["idx"] >= 0)):
        sp, sm = P["sl"].copy(), P["sl"].copy()
        sp[pos] += h
        sm[pos] -= h
        fd = (loss(P["q"], P["k"], P["v"], sp) - loss(P["q"], P["k"], P["v"], sm)) / (2 * h)
        assert abs(fd - dlg[pos]) < 1e-7 * max(1.0, abs(fd)), (pos, fd, dlg[pos])
