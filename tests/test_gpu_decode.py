"""GPU parity of the decode path (block summaries, pooled selection, split-K
decode attention) against the oracle, through the C ABI.

Summaries and pooled scores are fixed-order fp32, so they and the selected
index sets must match bit for bit; gates to 1e-5; outputs to the bf16
tolerance.  Paged and contiguous caches holding the same tokens must give
bit-identical results.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, assert_close, dev_tensor, say
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seqlens, hq, hkv, d, Kb)
    "mixed_g4_d128": ([700, 640, 65, 1, 64 * 9 + 63], 8, 2, 128, 4),
    "g2_d64": ([1000, 333], 4, 2, 64, 6),
    "g8_d128_bigK": ([64 * 40 + 5], 16, 2, 128, 64),
    "g1_d128": ([500, 129], 2, 2, 128, 3),
}


def run_decode(name, paged, out_dtype="bf16", gated=True, seed=7, summary="f32"):
    import torch
    seqlens, hq, hkv, d, Kb = CASES[name]
    say(f"[decode case {name} paged={paged} out={out_dtype} gated={gated}]")
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, paged, seed=seed)
    B = len(seqlens)
    max_len = max(seqlens)
    npages = host["k"].shape[0] if paged else 0
    prob = sas.Decode(seqlens, hq, hkv, d, Kb, paged, max_len, page_table=host["page_table"],
                      num_pages=npages, out_dtype=out_dtype, summary_dtype=summary)
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    vc = dev_tensor(host["v"], host["v_bits"], "bf16")
    ksum = sas.pool_keys(prob, kc)
    sel, lg, glse, scores = sas.decode_select(prob, q, ksum)
    o, lse = sas.decode(prob, q, kc, vc, sel, lg if gated else None)
    torch.cuda.synchronize()
    G = hq // hkv
    assert ksum.dtype == (torch.bfloat16 if summary == "bf16" else torch.float32)
    ksum_h, scores_h = ksum.float().cpu().numpy(), scores.cpu().numpy()
    sel_h, lg_h, glse_h = sel.cpu().numpy(), lg.cpu().numpy(), glse.cpu().numpy()
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        L = seqlens[b]
        cur = (L - 1) // 64
        for g in range(hkv):
            r = b * hkv + g
            K = wl.gather_row_cache(host["k"], host["page_table"], b, g, L)
            V = wl.gather_row_cache(host["v"], host["page_table"], b, g, L)
            qg = host["q"][b, g * G:(g + 1) * G]
            kbar = oracle.pool_keys_row(K, summary=summary)
            assert np.array_equal(ksum_h[b, g, :, :cur].T, kbar), (b, g, "summaries")
            ridx, rlg, rlse, rs = oracle.decode_select_row(qg, K, Kb, summary=summary)
            assert np.array_equal(scores_h[b, g, :cur], rs), (b, g, "scores")
            assert np.array_equal(sel_h[r], ridx), (b, g, sel_h[r], ridx)
            fin = np.isfinite(rlg)
            assert np.array_equal(np.isfinite(lg_h[r]), fin)
            assert np.max(np.abs(lg_h[r][fin] - rlg[fin]), initial=0) < 1e-5
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg if gated else None, Kb, prob.scale)
            err = np.max(np.abs(o_h[b, g * G:(g + 1) * G] - ro))
            assert err <= TOL["bf16"], (b, g, err)
            assert np.max(np.abs(lse_h[b, g * G:(g + 1) * G] - rl)) <= 1e-4
    say("  all rows match")
    return (ksum, sel, lg, o, lse), host


@pytest.mark.parametrize("name", list(CASES))
def test_decode_contiguous(name):
    run_decode(name, paged=False)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_paged(name):
    run_decode(name, paged=True)


def test_decode_ungated_and_fp32_output():
    run_decode("mixed_g4_d128", paged=True, out_dtype="f32", gated=False)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("name", ["mixed_g4_d128", "g2_d64"])
def test_decode_bf16_summaries(name, paged):
    """Summaries stored as bf16 (the fp32 means rounded to nearest even):
    summaries, scores and selection bit-exact against the oracle's bf16
    reading, output at the bf16 bar."""
    run_decode(name, paged, summary="bf16")


def test_paged_equals_contiguous_bitwise():
    """The same tokens in a shuffled page pool and in a contiguous cache."""
    import torch
    seqlens, hq, hkv, d, Kb = CASES["mixed_g4_d128"]
    (ks_p, sel_p, lg_p, o_p, lse_p), host = run_decode("mixed_g4_d128", paged=True)
    B, max_len = len(seqlens), max(seqlens)
    cont = {}
    for nm in ("k", "v"):
        bits = np.zeros((B, hkv, max_len, d), np.uint16)
        for b, L in enumerate(seqlens):
            for g in range(hkv):
                rows = wl.gather_row_cache(host[nm + "_bits"], host["page_table"], b, g, L)
                bits[b, g, :L] = rows
        cont[nm] = dev_tensor(None, bits, "bf16")
    prob = sas.Decode(seqlens, hq, hkv, d, Kb, False, max_len)
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    ksum = sas.pool_keys(prob, cont["k"])
    sel, lg, glse, scores = sas.decode_select(prob, q, ksum)
    o, lse = sas.decode(prob, q, cont["k"], cont["v"], sel, lg)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_p) and torch.equal(lg, lg_p)
    assert torch.equal(o, o_p) and torch.equal(lse, lse_p)


def test_unaligned_summary_stride_bitwise():
    """A summary stride that is not a multiple of 4 takes the one-block
    scoring kernel; summaries, scores, selection and output are the same
    bits as with the padded stride."""
    import torch
    seqlens, hq, hkv, d, Kb = CASES["g8_d128_bigK"]
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, True, seed=11)
    res = []
    for stride in (None, 41):  # padded default (40), and 41: 40 history blocks
        prob = sas.Decode(seqlens, hq, hkv, d, Kb, True, max(seqlens),
                          page_table=host["page_table"], num_pages=host["k"].shape[0],
                          nblk_stride=stride)
        say(f"[decode stride {prob.nblk_stride}]")
        q = dev_tensor(host["q"], host["q_bits"], "bf16")
        kc = dev_tensor(host["k"], host["k_bits"], "bf16")
        vc = dev_tensor(host["v"], host["v_bits"], "bf16")
        ksum = sas.pool_keys(prob, kc)
        sel, lg, glse, scores = sas.decode_select(prob, q, ksum)
        o, lse = sas.decode(prob, q, kc, vc, sel, lg)
        torch.cuda.synchronize()
        nh = (max(seqlens) - 1) // 64
        res.append((ksum[..., :nh].cpu(), scores[..., :nh].cpu(), sel.cpu(), lg.cpu(), o.cpu(),
                    lse.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
