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
from tests.gpu_helpers import TOL, assert_close, dev_tensor, say, summaries_f32
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seqlens, hq, hkv, d, Kb)
    "mixed_g4_d128": ([700, 640, 65, 1, 64 * 9 + 63], 8, 2, 128, 4),
    "g2_d64": ([1000, 333], 4, 2, 64, 6),
    "g8_d128_bigK": ([64 * 40 + 5], 16, 2, 128, 64),
    "g1_d128": ([500, 129], 2, 2, 128, 3),
    # several chunks of 256 blocks per row: 6 x 63 candidates in the merge
    "chunks_g4_d128": ([64 * 1500 + 10, 64 * 700 + 1, 90], 8, 2, 128, 64),
    # 17 chunks x 63 = 1071 candidates: the merge takes 8 per thread
    "wide_merge_g2_d64": ([64 * 4300 + 7, 64 * 300 + 3], 2, 1, 64, 64),
    # 17 chunks x 127 = 2159 candidates: the merge takes 16 per thread
    "widest_merge_g2_d64": ([64 * 4300 + 7, 64 * 300 + 3], 2, 1, 64, 128),
    # 256-block chunks would give 17 x 255 candidates, more than the merge
    # takes: two blocks per scoring thread (9 chunks of 512)
    "two_per_thread_g2_d64": ([64 * 4200 + 1], 2, 1, 64, 256),
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
    assert ksum.dtype == {"bf16": torch.bfloat16, "fp8": torch.uint8, "f32": torch.float32}[summary]
    ksum_h, scores_h = summaries_f32(ksum), scores.cpu().numpy()
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
            assert np.array_equal(ksum_h[b, g, :cur, :], kbar), (b, g, "summaries")
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
@pytest.mark.parametrize("name", ["mixed_g4_d128", "g2_d64", "two_per_thread_g2_d64"])
@pytest.mark.parametrize("summary", ["bf16", "fp8"])
def test_decode_reduced_precision_summaries(name, paged, summary):
    """Summaries stored as bf16 or fp8 e4m3 (the fp32 means rounded to
    nearest, ties to even): summaries, scores and selection bit-exact
    against the oracle's reading, output at the bf16 bar."""
    run_decode(name, paged, summary=summary)


def test_fp8_summary_codes_for_every_rounding_case():
    """The stored e4m3 codes of summaries whose fp32 means land on chosen
    values: exact e4m3 values, midpoints between neighbours (ties go to the
    even code), the subnormal range, signed zeros, and means past the
    largest finite value (448) that round to it or overflow to NaN.  Keys
    of a block are all equal to the wanted mean, so the token-order sum is
    exact and the mean is that value (bf16 keys: the wanted means are the
    ones bf16 holds exactly)."""
    import torch
    g = np.random.default_rng(13)
    codes = [c for c in range(256) if (c & 0x7f) != 0x7f]
    vals = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    order = np.argsort(vals, kind="stable")
    v = vals[order]
    mids = ((v[1:] + v[:-1]) / 2)[np.diff(v) > 0]
    # bf16 keys: keep wanted means that bf16 represents exactly
    want = np.concatenate([v, mids, [464.0, 472.0, 480.0, 1000.0, -464.0, 2.0**-10,
                                     0.0]]).astype(np.float32)
    want = want[torch.from_numpy(want).to(torch.bfloat16).float().numpy() == want]
    # keys of -0 sum to +0 (the sum starts from +0), so -0 is no mean here
    want = want[~((want == 0) & np.signbit(want))]
    nblk = len(want)
    L = 64 * nblk + 1
    hq, hkv, d, Kb = 2, 1, 64, 4
    k = np.repeat(want[:, None], 64, axis=0)  # block j: 64 keys equal to want[j]
    kc = np.zeros((1, hkv, L, d), np.float32)
    kc[0, 0, :64 * nblk] = np.repeat(k, d, axis=1)[:, :d]
    prob = sas.Decode([L], hq, hkv, d, Kb, False, L, summary_dtype="fp8")
    kct = torch.from_numpy(kc).to(torch.bfloat16).cuda()
    ksum = sas.pool_keys(prob, kct)
    torch.cuda.synchronize()
    got = sas.summaries_by_block(ksum)[0, 0, :nblk, 0].cpu()
    ref = torch.from_numpy(want).to(torch.float8_e4m3fn).view(torch.uint8)
    # NaN has two codes (0x7f, 0xff) and torch writes 0x7f for either sign
    nan = (ref & 0x7f) == 0x7f
    assert torch.equal((got & 0x7f)[nan], ref[nan] & 0x7f)
    assert torch.equal(got[~nan], ref[~nan]), (want[~nan.numpy()][(got != ref)[~nan].numpy()])
    assert np.array_equal(summaries_f32(ksum)[0, 0, :nblk, 0][~nan.numpy()],
                          oracle.round_e4m3(want)[~nan.numpy()])
    # the selection decodes every code to the same value: pooled scores of
    # these summaries equal the oracle's bit for bit (NaN summaries: NaN)
    qh = wl.round_bf16(wl.normal(g, (1, hq, d)))
    q = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).cuda()
    scores = sas.decode_select(prob, q, ksum)[3]
    torch.cuda.synchronize()
    kbar = np.repeat(oracle.round_e4m3(want)[:, None], d, axis=1)
    rs = oracle.decode_scores_row(wl.bf16_bits_to_f32(qh)[0], kbar)
    gs = scores[0, 0, :nblk].cpu().numpy()
    fin = ~np.isnan(rs)
    assert np.array_equal(np.isnan(gs), ~fin)
    assert np.array_equal(gs[fin].view(np.uint32), rs[fin].view(np.uint32))
    say(f"  {nblk} summaries: codes equal torch's conversion, scores equal the oracle's")


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


def test_wider_summary_stride_bitwise():
    """A summary / score row stride of two tiles instead of one: summaries,
    scores, selection and output are the same bits."""
    import torch
    seqlens, hq, hkv, d, Kb = CASES["g8_d128_bigK"]
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, True, seed=11)
    res = []
    for stride in (None, 128):  # one tile (the default for 40 history blocks), two
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
        res.append((sas.summaries_by_block(ksum)[..., :nh, :].cpu(), scores[..., :nh].cpu(),
                    sel.cpu(), lg.cpu(), o.cpu(),
                    lse.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_select_workspace_reused_across_calls():
    """One workspace serves repeated selections and a smaller problem in
    between: every result equals that of a fresh workspace."""
    import torch
    seqlens, hq, hkv, d, Kb = CASES["chunks_g4_d128"]
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, True, seed=17)
    big = sas.Decode(seqlens, hq, hkv, d, Kb, True, max(seqlens),
                     page_table=host["page_table"], num_pages=host["k"].shape[0])
    small = sas.Decode(seqlens[1:], hq, hkv, d, Kb, True, max(seqlens),
                       page_table=host["page_table"][1:], num_pages=host["k"].shape[0])
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    ks_big, ks_small = sas.pool_keys(big, kc), sas.pool_keys(small, kc)
    q_small = q[1:].contiguous()
    fresh_big = [x.cpu() for x in sas.decode_select(big, q, ks_big)]
    fresh_small = [x.cpu() for x in sas.decode_select(small, q_small, ks_small)]
    ws = sas.decode_select_workspace(big)
    assert ws.numel() >= sas.decode_select_workspace_bytes(small)
    for prob, qq, ks, want in ((big, q, ks_big, fresh_big), (big, q, ks_big, fresh_big),
                               (small, q_small, ks_small, fresh_small),
                               (big, q, ks_big, fresh_big)):
        got = [x.cpu() for x in sas.decode_select(prob, qq, ks, workspace=ws)]
        for a, b in zip(got[:3], want[:3]):  # sel_idx, log gates, gate_lse
            assert torch.equal(a, b)
        for bi, L in enumerate(prob.seqlens):  # scores exist for history blocks only
            nh = (L - 1) // 64
            assert torch.equal(got[3][bi, :, :nh], want[3][bi, :, :nh])
    say("  four calls on one workspace equal fresh ones")
