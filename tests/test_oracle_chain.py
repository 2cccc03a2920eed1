"""The oracle's end-to-end chain, selector weights -> logits -> gate and
Top-K -> gated attention -> loss, with its analytic gradient (oracle
backward, oracle gate backward, then fp64 autograd through the stand-in
selector) pinned by central finite differences of the loss in the weights.
The GPU autograd test compares the library's gradients with this chain.
"""
import numpy as np
import pytest

import oracle
from tests.stand_in_selector import selector_logits
from trainable_block_sparse_gate_amd import workloads as wl


def _setup():
    import torch
    lengths, hq, hkv, d, Kb, f = [200, 130], 4, 2, 16, 2, 4
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cuq = np.concatenate([[0], np.cumsum([(n + 63) // 64 for n in lengths])]).astype(np.int32)
    QB, T, ld = int(cuq[-1]), int(cu[-1]), max((n + 63) // 64 for n in lengths)
    g = wl.rng(97, 0)
    q, k, v, R = (wl.normal(g, s) for s in ((T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)))
    qf, kf = wl.normal(g, (QB, f)), wl.normal(g, (QB, f))
    W = wl.normal(g, (hkv, f, f), sigma=0.7).astype(np.float64)
    scale = 1.0 / np.sqrt(d)
    t = {"qf": torch.from_numpy(qf).double(), "kf": torch.from_numpy(kf).double()}
    return dict(cu=cu, cuq=cuq, ld=ld, hkv=hkv, Kb=Kb, q=q, k=k, v=v, R=R, W=W, scale=scale,
                **t)


def _logits(s, W):
    import torch
    return selector_logits(s["qf"], s["kf"], torch.as_tensor(W), s["cuq"], s["ld"])


def _loss(s, W):
    lg32 = _logits(s, W).numpy().astype(np.float32)
    idx, sl, _ = oracle.gate_topk(s["cu"], lg32, s["hkv"], s["Kb"])
    o, _ = oracle.fwd(s["cu"], s["q"], s["k"], s["v"], idx, sl, s["Kb"], s["scale"])
    return float(np.sum(o * s["R"])), idx


def test_selector_weight_gradient_matches_finite_differences():
    import torch
    s = _setup()
    W = torch.from_numpy(s["W"]).double().requires_grad_()
    logits = _logits(s, W)
    lg32 = logits.detach().numpy().astype(np.float32)
    idx, sl, _ = oracle.gate_topk(s["cu"], lg32, s["hkv"], s["Kb"])
    # some rows must drop candidates, or the Top-K is not exercised
    assert np.any(idx[..., :-1] != np.arange(s["Kb"] - 1)), "every row kept all history"
    _, _, _, dlg = oracle.bwd(s["cu"], s["q"], s["k"], s["v"], s["R"], idx, sl, s["Kb"],
                              s["scale"])
    dz = oracle.gate_bwd(s["cu"], lg32, idx, dlg, s["hkv"], s["Kb"])
    logits.backward(torch.from_numpy(dz))
    dW = W.grad.numpy()
    assert np.max(np.abs(dW)) > 1e-3
    h = 1e-3
    checked = 0
    for flat in range(0, s["W"].size, 3):
        e = np.unravel_index(flat, s["W"].shape)
        Wp, Wm = s["W"].copy(), s["W"].copy()
        Wp[e] += h
        Wm[e] -= h
        lp, ip = _loss(s, Wp)
        lm, im = _loss(s, Wm)
        if not (np.array_equal(ip, idx) and np.array_equal(im, idx)):
            continue  # the kept set moved: no derivative there
        fd = (lp - lm) / (2 * h)
        assert abs(fd - dW[e]) <= 1e-4 + 2e-3 * abs(fd), (e, fd, dW[e])
        checked += 1
    assert checked >= 8


def test_selector_gradient_is_zero_when_every_candidate_is_kept_and_gates_are_uniform():
    """With a budget above every row's history and W = 0 the gates are the
    uniform softmax; the loss still has a nonzero weight gradient only
    through d logits, whose rows sum to zero (softmax Jacobian): check the
    row sums of the oracle's d logits vanish."""
    s = _setup()
    s["Kb"] = 8
    W0 = np.zeros_like(s["W"])
    lg32 = _logits(s, W0).numpy().astype(np.float32)
    idx, sl, _ = oracle.gate_topk(s["cu"], lg32, s["hkv"], s["Kb"])
    _, _, _, dlg = oracle.bwd(s["cu"], s["q"], s["k"], s["v"], s["R"], idx, sl, s["Kb"],
                              s["scale"])
    dz = oracle.gate_bwd(s["cu"], lg32, idx, dlg, s["hkv"], s["Kb"])
    assert np.max(np.abs(dz)) > 1e-6
    for sq in range(len(s["cuq"]) - 1):
        for Q in range(s["cuq"][sq], s["cuq"][sq + 1]):
            i = Q - s["cuq"][sq]
            np.testing.assert_allclose(dz[:, Q, :i].sum(axis=-1), 0.0, atol=1e-12)
