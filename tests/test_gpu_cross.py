"""Cross-kernel consistency on the GPU, through the C ABI.

- Decoding the last token of a sequence attends exactly the keys the
  forward's last row attends (the same kept blocks, the same log gates, the
  current block up to and including the token), so sas_decode must give the
  forward's output and lse for that token.  The two kernels round P to bf16
  for their products at different points (different running maxima), so the
  outputs agree to the bf16 bar, not bit for bit.
- The split of a decode row's kept blocks over workgroups (num_splits)
  changes only the order of the fp32 sums and where P is rounded, so every
  split count gives the same selection and the same output to the bf16 bar;
  with one split per row the output is the unsplit kernel's own.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, assert_close, dev_tensor, say
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,hq,hkv,d,Kb", [
    ([64 * 20 + 37, 64 * 9, 700], 8, 2, 128, 6),
    ([64 * 33 + 1, 129], 16, 2, 128, 16),
    ([1000], 4, 2, 64, 5),
])
def test_decode_of_last_token_equals_forward_row(lengths, hq, hkv, d, Kb):
    import torch
    say(f"[cross fwd/decode] lengths {lengths} heads {hq}/{hkv} d {d} Kb {Kb}")
    case = wl.make_varlen("cross", lengths, hq, hkv, d, Kb, dtype="bf16", workload_id=71)
    prob = sas.Varlen(lengths, hq, hkv, d, Kb, dtype="bf16", out_dtype="f32")
    q = dev_tensor(case.q, case.bits["q"], "bf16")
    k = dev_tensor(case.k, case.bits["k"], "bf16")
    v = dev_tensor(case.v, case.bits["v"], "bf16")
    logits = torch.from_numpy(case.logits).cuda()
    sel, lg, _ = sas.gate_topk(prob, logits)
    o, lse = sas.fwd(prob, q, k, v, sel, lg)
    # the same tokens as a batch of contiguous decode caches, query = last token
    B, L = len(lengths), max(lengths)
    cu = case.cu_seqlens
    kc = torch.zeros((B, hkv, L, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    qd = torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda")
    last_rows = []
    for b, n in enumerate(lengths):
        kc[b, :, :n] = k[cu[b]:cu[b + 1]].transpose(0, 1)
        vc[b, :, :n] = v[cu[b]:cu[b + 1]].transpose(0, 1)
        qd[b] = q[cu[b + 1] - 1]
        last_rows.append(case.cu_qblocks[b + 1] - 1)
    dsel = sel[:, last_rows, :].transpose(0, 1).reshape(B * hkv, Kb).contiguous()
    dlg = lg[:, last_rows, :].transpose(0, 1).reshape(B * hkv, Kb).contiguous()
    dp = sas.Decode(lengths, hq, hkv, d, Kb, False, L, out_dtype="f32")
    od, lsed = sas.decode(dp, qd, kc, vc, dsel, dlg)
    torch.cuda.synchronize()
    want_o = o[torch.as_tensor(cu[1:] - 1, device="cuda").long()]
    want_lse = lse[:, torch.as_tensor(cu[1:] - 1, device="cuda").long()].T
    assert_close("decode o vs forward row", od.cpu().numpy(), want_o.cpu().numpy(), TOL["bf16"])
    assert_close("decode lse vs forward row", lsed.cpu().numpy(), want_lse.cpu().numpy(), 1e-4)
    # and both against the oracle's decode of the same row
    G = hq // hkv
    for b, n in enumerate(lengths):
        for g in range(hkv):
            K = case.k[cu[b]:cu[b + 1], g]
            V = case.v[cu[b]:cu[b + 1], g]
            ridx = dsel[b * hkv + g].cpu().numpy()
            rlg = dlg[b * hkv + g].cpu().numpy().astype(np.float64)
            ro, rl = oracle.decode_row(case.q[cu[b + 1] - 1, g * G:(g + 1) * G], K, V, ridx,
                                       rlg, Kb, prob.scale)
            assert np.max(np.abs(od[b, g * G:(g + 1) * G].cpu().numpy() - ro)) <= TOL["bf16"]
            assert np.max(np.abs(lsed[b, g * G:(g + 1) * G].cpu().numpy() - rl)) <= 1e-4


@pytest.mark.parametrize("paged", [False, True])
def test_decode_split_count_does_not_change_the_result(paged):
    import torch
    seqlens, hq, hkv, d, Kb = [64 * 40 + 5, 64 * 70, 200, 1], 16, 2, 128, 24
    say(f"[cross splits] paged={paged} seqlens {seqlens} Kb {Kb}")
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, paged, seed=72)
    npages = host["k"].shape[0] if paged else 0
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    vc = dev_tensor(host["v"], host["v_bits"], "bf16")

    def run(num_splits):
        p = sas.Decode(seqlens, hq, hkv, d, Kb, paged, max(seqlens),
                       page_table=host["page_table"], num_pages=npages, out_dtype="f32",
                       num_splits=num_splits)
        ksum = sas.pool_keys(p, kc)
        sel, lg, _, _ = sas.decode_select(p, q, ksum)
        o, lse = sas.decode(p, q, kc, vc, sel, lg)
        torch.cuda.synchronize()
        return sel.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()

    sel0, o0, lse0 = run(1)
    G = hq // hkv
    for b, L in enumerate(seqlens):
        for g in range(hkv):
            K = wl.gather_row_cache(host["k"], host["page_table"], b, g, L)
            V = wl.gather_row_cache(host["v"], host["page_table"], b, g, L)
            qg = host["q"][b, g * G:(g + 1) * G]
            ridx, rlg, _, _ = oracle.decode_select_row(qg, K, Kb)
            assert np.array_equal(sel0[b * hkv + g], ridx)
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, Kb, 1.0 / np.sqrt(d))
            assert np.max(np.abs(o0[b, g * G:(g + 1) * G] - ro)) <= TOL["bf16"]
            assert np.max(np.abs(lse0[b, g * G:(g + 1) * G] - rl)) <= 1e-4
    again = run(1)
    assert np.array_equal(again[1], o0) and np.array_equal(again[2], lse0), "not deterministic"
    for n in (0, 2, 3, 5, 8, Kb):
        sel_n, o_n, lse_n = run(n)
        assert np.array_equal(sel_n, sel0), n
        say(f"  num_splits={n}: max |o - o(1 split)| {np.max(np.abs(o_n - o0)):.3e}, "
            f"max |lse diff| {np.max(np.abs(lse_n - lse0)):.3e}")
        assert np.max(np.abs(o_n - o0)) <= TOL["bf16"], n
        assert np.max(np.abs(lse_n - lse0)) <= 1e-4, n
