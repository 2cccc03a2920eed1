"""GPU parity of the hierarchical (coarse-to-fine) decode selection (review,
section 7-2) against the oracle, through the C ABI.

Super-block summaries and pooled scores are fixed-order fp32, so they, the
kept super-blocks' candidates and the selected index sets must match bit
for bit; log gates and gate_lse to 1e-5; the decode output with that
selection to the bf16 bar.  With every super-block kept the selection must
be the exact one.  In the step loop, sas_decode_append keeps the
super-block summaries equal to the oracle's after every step.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, dev_tensor, say, summaries_f32
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seqlens, hq, hkv, d, Kb, coarse_keep)
    "mixed_g4_d128": ([64 * 300 + 5, 64 * 90 + 1, 64 * 17, 70], 8, 2, 128, 16, 4),
    "keep1_g2_d64": ([64 * 200 + 40, 64 * 33 + 2, 1], 4, 2, 64, 6, 1),
    "keep127_g2_d64": ([64 * 1100 + 3], 2, 1, 64, 64, 127),
    "many_chunks_g8_d128": ([64 * 9000 + 9], 8, 1, 128, 32, 31),
}


# every layout and summary dtype for the short cases; for the long one, whose
# oracle pass takes most of the time, the contiguous layout with bf16 summaries
PARAMS = [(n, paged, s) for n in CASES if n != "many_chunks_g8_d128"
          for paged in (False, True) for s in ("f32", "bf16", "fp8")]
PARAMS.append(("many_chunks_g8_d128", False, "bf16"))


@pytest.mark.parametrize("name,paged,summary", PARAMS)
def test_hier_selection_matches_oracle(name, paged, summary):
    import torch
    seqlens, hq, hkv, d, Kb, C = CASES[name]
    say(f"[hier case {name} paged={paged} summary={summary} C={C}]")
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, paged, seed=31)
    prob = sas.Decode(seqlens, hq, hkv, d, Kb, paged, max(seqlens),
                      page_table=host["page_table"],
                      num_pages=host["k"].shape[0] if paged else 0, summary_dtype=summary)
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    vc = dev_tensor(host["v"], host["v_bits"], "bf16")
    ksum = sas.pool_keys(prob, kc)
    csum = sas.pool_coarse(prob, ksum)
    sel, lg, glse, scores = sas.decode_select_hier(prob, q, ksum, csum, C)
    o, lse = sas.decode(prob, q, kc, vc, sel, lg)
    torch.cuda.synchronize()
    G = hq // hkv
    cs_h, sc_h = summaries_f32(csum), scores.cpu().numpy()
    sel_h, lg_h, glse_h = sel.cpu().numpy(), lg.cpu().numpy(), glse.cpu().numpy()
    o_h = o.float().cpu().numpy()
    for b, L in enumerate(seqlens):
        for g in range(hkv):
            r = b * hkv + g
            K = wl.gather_row_cache(host["k"], host["page_table"], b, g, L)
            V = wl.gather_row_cache(host["v"], host["page_table"], b, g, L)
            qg = host["q"][b, g * G:(g + 1) * G]
            cbar = oracle.coarse_summaries_row(oracle.pool_keys_row(K, summary=summary), summary)
            assert np.array_equal(cs_h[b, g, :cbar.shape[0], :], cbar), (b, g, "coarse summaries")
            ridx, rlg, rlse, rs, cand = oracle.decode_select_row_hier(qg, K, Kb, C,
                                                                      summary=summary)
            assert np.array_equal(sc_h[b, g, cand], rs[cand]), (b, g, "candidate scores")
            assert np.array_equal(sel_h[r], ridx), (b, g, sel_h[r], ridx)
            fin = np.isfinite(rlg)
            assert np.array_equal(np.isfinite(lg_h[r]), fin)
            assert np.max(np.abs(lg_h[r][fin] - rlg[fin]), initial=0) < 1e-5
            if np.isfinite(rlse):
                assert abs(glse_h[r] - rlse) < 1e-5
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, Kb, prob.scale)
            assert float(np.max(np.abs(o_h[b, g * G:(g + 1) * G] - ro))) <= TOL["bf16"]
    say("  all rows match")


def test_hier_keeping_every_super_block_is_the_exact_selection():
    import torch
    seqlens, hq, hkv, d, Kb = [64 * 300 + 5, 64 * 90 + 1, 33], 8, 2, 128, 16
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, True, seed=32)
    prob = sas.Decode(seqlens, hq, hkv, d, Kb, True, max(seqlens),
                      page_table=host["page_table"], num_pages=host["k"].shape[0])
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    ksum = sas.pool_keys(prob, kc)
    csum = sas.pool_coarse(prob, ksum)
    want = sas.decode_select(prob, q, ksum)
    got = sas.decode_select_hier(prob, q, ksum, csum, 127)
    torch.cuda.synchronize()
    assert torch.equal(got[0], want[0])
    fin = torch.isfinite(want[1])
    assert torch.equal(torch.isfinite(got[1]), fin)
    assert float((got[1][fin] - want[1][fin]).abs().max()) < 1e-5
    for b, L in enumerate(seqlens):
        nh = (L - 1) // 64
        assert torch.equal(got[3][b, :, :nh], want[3][b, :, :nh])


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def test_hier_step_loop_keeps_super_block_summaries():
    """A contiguous cache prefilled to just below super-block boundaries;
    the appended tokens finish blocks that complete super-blocks."""
    import torch
    hq, hkv, d, Kb, C = 8, 2, 128, 8, 2
    L0 = [64 * 16 - 1, 64 * 24, 64 * 40 - 1, 5]  # steps finish blocks 15 and 39
    steps = 3
    B, G = len(L0), hq // hkv
    cap = max(L0) + steps
    g = wl.rng(44, 1)
    kb = wl.round_bf16(wl.normal(g, (B, hkv, cap, d)))
    qb = wl.round_bf16(wl.normal(g, (steps, B, hq, d)))
    kf, qf = wl.bf16_bits_to_f32(kb), wl.bf16_bits_to_f32(qb)
    kc_h = np.zeros((B, hkv, cap, d), np.uint16)
    for b in range(B):
        kc_h[b, :, :L0[b]] = kb[b, :, :L0[b]]
    kc, vc = _bf16_dev(kc_h), _bf16_dev(kc_h)
    stride = -(-max(1, (cap - 1) // 64) // 64) * 64

    def problem(lens):
        return sas.Decode(lens, hq, hkv, d, Kb, False, cap, nblk_stride=stride,
                          summary_dtype="bf16")

    ksum = sas.pool_keys(problem(L0), kc)
    csum = sas.pool_coarse(problem(L0), ksum)
    for s in range(steps):
        lens = [n + s + 1 for n in L0]
        prob = problem(lens)
        t = np.array(lens) - 1
        k_new = _bf16_dev(kb[np.arange(B), :, t])
        sas.decode_append(prob, k_new, k_new, kc, vc, ksum, csum)
        q = _bf16_dev(qb[s])
        sel, lg, glse, scores = sas.decode_select_hier(prob, q, ksum, csum, C)
        torch.cuda.synchronize()
        cs_h, sel_h = summaries_f32(csum), sel.cpu().numpy()
        for b in range(B):
            L = lens[b]
            for h in range(hkv):
                K = kf[b, h, :L]
                cbar = oracle.coarse_summaries_row(oracle.pool_keys_row(K, summary="bf16"),
                                                   "bf16")
                assert np.array_equal(cs_h[b, h, :cbar.shape[0], :], cbar), (s, b, h)
                qg = qf[s, b, h * G:(h + 1) * G]
                ridx = oracle.decode_select_row_hier(qg, K, Kb, C, summary="bf16")[0]
                assert np.array_equal(sel_h[b * hkv + h], ridx), (s, b, h, "selection")
        say(f"  step {s}: lengths {lens} match")
