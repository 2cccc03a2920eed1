"""GPU parity of the decode step loop: a prefilled prefix handed over with
sas_pool_keys, then several steps of sas_decode_append (new token into the
cache, the finished block's summary when a block is crossed),
sas_decode_select and sas_decode.  After every step the caches and the
summaries must equal, bit for bit, the host cache and the oracle's
summaries of it, the selection must equal the oracle's, and the output
must be within the bf16 bar.  Paged and contiguous caches.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, say, summaries_f32
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


@pytest.mark.parametrize("paged,summary", [(False, "f32"), (True, "f32"), (True, "bf16"),
                                           (False, "fp8")])
def test_decode_step_loop(paged, summary):
    import torch
    L0 = [62, 128, 300, 1, 63, 191]   # steps cross 64, 128 (first step), 192, and none
    steps, hq, hkv, d, Kb = 4, 8, 2, 128, 3
    B, G = len(L0), hq // hkv
    Lfin = [n + steps for n in L0]
    cap = max(Lfin)
    say(f"[decode step loop paged={paged} summary={summary} L0={L0} steps={steps}]")
    g = wl.rng(43, 1)
    kb = wl.round_bf16(wl.normal(g, (B, hkv, cap, d)))
    vb = wl.round_bf16(wl.normal(g, (B, hkv, cap, d)))
    qb = wl.round_bf16(wl.normal(g, (steps, B, hq, d)))
    kf, vf, qf = wl.bf16_bits_to_f32(kb), wl.bf16_bits_to_f32(vb), wl.bf16_bits_to_f32(qb)
    npg = [(n + 63) // 64 for n in Lfin]
    maxp = max(npg)
    stride = -(-max(1, (cap - 1) // 64) // 64) * 64

    # the prefilled prefix (tokens < L0) in the chosen layout; the rest zero
    if paged:
        perm = wl.rng(43, 2).permutation(sum(npg)).astype(np.int32)
        pt = np.zeros((B, maxp), np.int32)
        o = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        kc_h = np.zeros((sum(npg), hkv, 64, d), np.uint16)
        vc_h = np.zeros_like(kc_h)
        for b in range(B):
            for t in range(L0[b]):
                kc_h[pt[b, t // 64], :, t % 64] = kb[b, :, t]
                vc_h[pt[b, t // 64], :, t % 64] = vb[b, :, t]
    else:
        pt = None
        kc_h = np.zeros((B, hkv, cap, d), np.uint16)
        vc_h = np.zeros_like(kc_h)
        for b in range(B):
            kc_h[b, :, :L0[b]] = kb[b, :, :L0[b]]
            vc_h[b, :, :L0[b]] = vb[b, :, :L0[b]]
    kc, vc = _bf16_dev(kc_h), _bf16_dev(vc_h)

    def problem(lens):
        return sas.Decode(lens, hq, hkv, d, Kb, paged, cap, page_table=pt,
                          num_pages=sum(npg) if paged else 0, nblk_stride=stride,
                          summary_dtype=summary)

    ksum = sas.pool_keys(problem(L0), kc)   # dense-prefill handoff
    for s in range(steps):
        lens = [n + s + 1 for n in L0]
        prob = problem(lens)
        t = np.array(lens) - 1
        k_new = _bf16_dev(kb[np.arange(B), :, t])
        v_new = _bf16_dev(vb[np.arange(B), :, t])
        sas.decode_append(prob, k_new, v_new, kc, vc, ksum)
        q = _bf16_dev(qb[s])
        sel, lg, glse, scores = sas.decode_select(prob, q, ksum)
        out, lse = sas.decode(prob, q, kc, vc, sel, lg)
        torch.cuda.synchronize()
        kc_d = kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vc_d = vc.view(torch.int16).cpu().numpy().view(np.uint16)
        ks_h, sel_h = summaries_f32(ksum), sel.cpu().numpy()
        o_h = out.float().cpu().numpy()
        for b in range(B):
            L = lens[b]
            if paged:
                pages = pt[b, :(L + 63) // 64]
                got_k = kc_d[pages].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
                got_v = vc_d[pages].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
            else:
                got_k, got_v = kc_d[b, :, :L], vc_d[b, :, :L]
            assert np.array_equal(got_k, kb[b, :, :L]), (s, b, "k cache")
            assert np.array_equal(got_v, vb[b, :, :L]), (s, b, "v cache")
            cur = (L - 1) // 64
            for h in range(hkv):
                K, V = kf[b, h, :L], vf[b, h, :L]
                assert np.array_equal(ks_h[b, h, :cur, :],
                                      oracle.pool_keys_row(K, summary=summary)), \
                    (s, b, h, "summaries")
                qg = qf[s, b, h * G:(h + 1) * G]
                ridx, rlg, _, _ = oracle.decode_select_row(qg, K, Kb, summary=summary)
                assert np.array_equal(sel_h[b * hkv + h], ridx), (s, b, h, "selection")
                ro, _ = oracle.decode_row(qg, K, V, ridx, rlg, Kb, prob.scale)
                err = float(np.max(np.abs(o_h[b, h * G:(h + 1) * G] - ro)))
                assert err <= TOL["bf16"], (s, b, h, err)
        say(f"  step {s}: lengths {lens} match")
