"""End-to-end gradient through the torch.autograd wrapper on the GPU: a
stand-in bilinear selector (torch, fp32) produces the logits, the wrapper
runs gate + Top-K, the gated forward, the fused backward and the gate
backward through the C ABI, and torch's autograd carries d logits back to
the selector weights.  The reference is the oracle's chain on the same
fp32 logits (its finite-difference pin is in test_oracle_chain.py).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, assert_close, dev_tensor, say
from tests.stand_in_selector import selector_logits
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [sas.GATE_HIST, sas.GATE_SIGMOID])
def test_loss_reaches_selector_weights(mode):
    import torch
    from trainable_block_sparse_gate_amd.autograd import GatedBlockSparseAttention
    lengths, hq, hkv, d, Kb, f = [300, 129, 700], 4, 2, 64, 4, 8
    say(f"[autograd selector mode={mode} lengths={lengths}]")
    case = wl.make_varlen("autograd", lengths, hq, hkv, d, Kb, workload_id=41)
    QB, ld = case.total_qblocks, max(case.qblocks)
    g = wl.rng(41, 9)
    qf, kf = wl.normal(g, (QB, f)), wl.normal(g, (QB, f))
    W = wl.normal(g, (hkv, f, f), sigma=0.5)
    prob = sas.Varlen(lengths, hq, hkv, d, Kb)
    q = dev_tensor(case.q, case.bits["q"], "bf16").requires_grad_()
    k = dev_tensor(case.k, case.bits["k"], "bf16").requires_grad_()
    v = dev_tensor(case.v, case.bits["v"], "bf16").requires_grad_()
    R = dev_tensor(case.dO, case.bits["dO"], "bf16")
    Wt = torch.tensor(W, device="cuda", requires_grad=True)
    logits = selector_logits(torch.tensor(qf, device="cuda"), torch.tensor(kf, device="cuda"),
                             Wt, case.cu_qblocks, ld)
    logits.retain_grad()
    o, sel, lg = GatedBlockSparseAttention.apply(q, k, v, logits, prob, mode)
    loss = (o.float() * R.float()).sum()
    loss.backward()
    torch.cuda.synchronize()

    lg32 = logits.detach().cpu().numpy()
    ridx, rlg, _ = oracle.gate_topk(case.cu_seqlens, lg32, hkv, Kb, mode)
    assert np.array_equal(sel.cpu().numpy(), ridx)
    ro, _ = oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, ridx, rlg, Kb, case.scale)
    assert_close("o", o.float().detach().cpu().numpy(), ro, TOL["bf16"])
    rdq, rdk, rdv, rdlg = oracle.bwd(case.cu_seqlens, case.q, case.k, case.v, case.dO, ridx,
                                     rlg, Kb, case.scale)
    # q/k/v are bf16 leaves: torch rounds the fp32 gradients to bf16
    for nm, t, ref in (("dq", q, rdq), ("dk", k, rdk), ("dv", v, rdv)):
        assert t.grad.dtype == torch.bfloat16
        assert_close(nm, t.grad.float().cpu().numpy(), ref,
                     TOL["bf16"] + np.max(np.abs(ref)) * 2.0 ** -8)
    rdz = oracle.gate_bwd(case.cu_seqlens, lg32, ridx, rdlg, hkv, Kb, mode)
    assert_close("d_logits", logits.grad.cpu().numpy(), rdz, TOL["bf16"])
    # the selector weights: fp64 autograd through the same selector
    W64 = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    z64 = selector_logits(torch.tensor(qf, dtype=torch.float64),
                          torch.tensor(kf, dtype=torch.float64), W64, case.cu_qblocks, ld)
    z64.backward(torch.from_numpy(rdz))
    ref = W64.grad.numpy()
    got = Wt.grad.cpu().numpy()
    rel = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    say(f"  dW: max rel err {rel:.3e} (max|ref| {np.max(np.abs(ref)):.3e})")
    # d logits is fp32 work (its error is ~1e-6 of its scale), so the
    # weights' gradient is held to 1e-3 relative, well inside the bf16 bar
    assert np.max(np.abs(ref)) > 1e-3 and rel <= 1e-3
