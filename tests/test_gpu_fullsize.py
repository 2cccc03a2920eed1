"""GPU parity at the workloads' full sizes, through the C ABI, in the launch
configuration bench.py times.

Selected index sets and log gates are compared with the oracle on every row
of every workload.  Both training workloads are compared everywhere (every
row's o, lse, dq, d log-gate and d logits; every key block's dk and dv),
the 81,920-token packed one with its boosted key blocks, whose dk/dv the
kernel splits over several segments and sums in a second kernel.  Decode:
every (sequence,
kv head) row of both decode workloads (scores, selection, log gates,
output, lse).  Invariants that hold at any size are checked on every row:
each log-gate-gradient row sums to zero, selections are ascending with the
current block kept.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, assert_close, case_to_device, say
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu


def check_selection_structure(sel, cuq, hkv):
    """Every row: kept history ascending, then the current block, then -1."""
    QB = sel.shape[1]
    seq = np.searchsorted(cuq, np.arange(QB), side="right") - 1
    i_of = np.arange(QB) - cuq[seq]
    Kb = sel.shape[2]
    for g in range(hkv):
        for Q in range(QB):
            i = i_of[Q]
            k = min(Kb - 1, i)
            row = sel[g, Q]
            assert np.all(np.diff(row[:k]) > 0) and (k == 0 or row[k - 1] < i)
            assert row[k] == i and np.all(row[k + 1:] == -1)


def keep_counts(ridx, cuq, hkv):
    """[hkv][QB]: how many rows keep each key block (global query-block index)."""
    QB = ridx.shape[1]
    seq = np.searchsorted(cuq, np.arange(QB), side="right") - 1
    keep = np.zeros((hkv, QB), np.int64)
    for g in range(hkv):
        j = ridx[g]
        rows = np.broadcast_to(np.arange(QB)[:, None], j.shape)
        ok = j >= 0
        np.add.at(keep[g], (cuq[seq[rows]] + j)[ok], 1)
    return keep


def token_masks(case, rm, km):
    """Token x head masks of the rows in rm (query side) and the key blocks
    in km (key side)."""
    cu, cuq = case.cu_seqlens, case.cu_qblocks
    G = case.hq // case.hkv
    tok = np.zeros((case.T, case.hq), bool)
    ktok = np.zeros((case.T, case.hkv), bool)
    for gg in range(case.hkv):
        for Q in np.nonzero(rm[gg] | km[gg])[0]:
            s = np.searchsorted(cuq, Q, side="right") - 1
            a = cu[s] + 64 * (Q - cuq[s])
            b = min(cu[s + 1], a + 64)
            if rm[gg, Q]:
                tok[a:b, gg * G:(gg + 1) * G] = True
            if km[gg, Q]:
                ktok[a:b, gg] = True
    return tok, ktok


def run_training_workload(case, rm, km):
    """gate -> fwd -> bwd phases -> gate bwd on the GPU in the bench's launch
    configuration; selections and log gates compared on every row, the
    other outputs on the rows in rm ([hkv][QB] mask) and the key blocks in
    km (dk, dv: the oracle sums every row that keeps such a block)."""
    import torch
    prob = sas.Varlen(case.lengths, case.hq, case.hkv, case.d, case.budget_blocks,
                      dtype=case.dtype)
    dv = case_to_device(case)
    say(f"[full {case.name}] T={case.T} rows={case.hkv * case.total_qblocks} "
        f"checked rows={int(rm.sum())} key blocks={int(km.sum())}")
    sel, lg, glse = sas.gate_topk(prob, dv["logits"])
    o, lse = sas.fwd(prob, dv["q"], dv["k"], dv["v"], sel, lg)
    f32 = torch.float32
    dq = torch.empty((prob.T, prob.hq, prob.d), dtype=f32, device="cuda")
    dk = torch.empty((prob.T, prob.hkv, prob.d), dtype=f32, device="cuda")
    dvv = torch.empty_like(dk)
    dlg = torch.empty(sel.shape, dtype=f32, device="cuda")
    ws = torch.empty(sas.bwd_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    sas.bwd_phases(prob, dv["q"], dv["k"], dv["v"], o, dv["dO"], lse, sel, lg,
                   (dq, dk, dvv, dlg), ws)
    dz = sas.gate_bwd(prob, dv["logits"], sel, glse, dlg)
    torch.cuda.synchronize()
    Kb = case.budget_blocks
    ridx, rlg, rlse = oracle.gate_topk(case.cu_seqlens, case.logits, case.hkv, Kb)
    sel_h = sel.cpu().numpy()
    assert np.array_equal(sel_h, ridx), "selected index sets differ"
    check_selection_structure(sel_h, case.cu_qblocks, case.hkv)
    fin = np.isfinite(rlg)
    assert np.array_equal(np.isfinite(lg.cpu().numpy()), fin)
    assert_close("log_gate", lg.cpu().numpy()[fin], rlg[fin], 1e-5)
    # invariant on every row: the log-gate gradient of a row sums to zero
    dlg_h = dlg.cpu().numpy()
    row_sums = np.abs(dlg_h.sum(-1))
    say(f"  max |sum_slot dlg| over all rows = {row_sums.max():.3e}")
    assert row_sums.max() < TOL[case.dtype]
    every_row = bool(rm.all())
    say("  oracle forward ...")
    ro, rl = oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, ridx, rlg, Kb, case.scale,
                        row_mask=None if every_row else rm)
    say("  oracle backward ...")
    rdq, rdk, rdv, rdlg = oracle.bwd(case.cu_seqlens, case.q, case.k, case.v, case.dO, ridx,
                                     rlg, Kb, case.scale, row_mask=None if every_row else rm,
                                     kblk_mask=None if km.all() else km)
    say("  comparing")
    tok, ktok = token_masks(case, rm, km)
    o_h, lse_h, dq_h = o.float().cpu().numpy(), lse.cpu().numpy().T, dq.cpu().numpy()
    assert_close("o", o_h[tok], ro[tok], TOL[case.dtype])
    assert_close("lse", lse_h[tok], rl.T[tok], TOL[case.dtype])
    assert_close("dq", dq_h[tok], rdq[tok], TOL[case.dtype])
    rows = rm.astype(bool)
    assert_close("dlg", dlg_h[rows], rdlg[rows], TOL[case.dtype])
    assert_close("dk", dk.cpu().numpy()[ktok], rdk[ktok], TOL[case.dtype])
    assert_close("dv", dvv.cpu().numpy()[ktok], rdv[ktok], TOL[case.dtype])
    rdz = oracle.gate_bwd(case.cu_seqlens, case.logits, ridx, np.where(rm[..., None], rdlg, 0),
                          case.hkv, Kb)
    assert_close("d_logits", dz.cpu().numpy()[rows], rdz[rows], TOL[case.dtype])
    return ridx


def test_tiny_fp32_every_row():
    """1 x 512 tokens, 2/1 heads, d 64, fp32, budget 2 + current: all rows."""
    import torch
    case = wl.tiny()
    prob = sas.Varlen(case.lengths, case.hq, case.hkv, case.d, case.budget_blocks, dtype="f32")
    dv = case_to_device(case)
    sel, lg, glse = sas.gate_topk(prob, dv["logits"])
    o, lse = sas.fwd(prob, dv["q"], dv["k"], dv["v"], sel, lg)
    dq, dk, dvv, dlg = sas.bwd(prob, dv["q"], dv["k"], dv["v"], o, dv["dO"], lse, sel, lg)
    dz = sas.gate_bwd(prob, dv["logits"], sel, glse, dlg)
    torch.cuda.synchronize()
    Kb = case.budget_blocks
    ridx, rlg, _ = oracle.gate_topk(case.cu_seqlens, case.logits, case.hkv, Kb)
    assert np.array_equal(sel.cpu().numpy(), ridx)
    ro, rl = oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, ridx, rlg, Kb, case.scale)
    rdq, rdk, rdv, rdlg = oracle.bwd(case.cu_seqlens, case.q, case.k, case.v, case.dO, ridx,
                                     rlg, Kb, case.scale)
    rdz = oracle.gate_bwd(case.cu_seqlens, case.logits, ridx, rdlg, case.hkv, Kb)
    for name, got, want in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk),
                            ("dv", dvv, rdv), ("dlg", dlg, rdlg), ("d_logits", dz, rdz)):
        assert_close(name, got.cpu().numpy(), want, TOL["f32"])


def test_layer16k_full_size():
    """1 x 16384 tokens, 32/8 heads, d 128, bf16, budget 16 blocks: every
    row (o, lse, dq, d log-gate, d logits) and every key block (dk, dv)."""
    case = wl.layer16k()
    QB = case.total_qblocks
    everything = np.ones((case.hkv, QB), np.uint8)
    run_training_workload(case, everything, everything)


def test_varlen_full_size():
    """4 packed sequences (32768/24576/16384/8192), 32/8 heads, d 128, bf16,
    budget 32 blocks, logits N(0,3) with boosted key-block columns: every
    row (o, lse, dq, d log-gate, d logits) and every key block (dk, dv),
    the boosted ones included (kept by hundreds of rows: split over several
    dk/dv segments and summed by the reduce kernel)."""
    case = wl.varlen()
    Kb, QB, cuq = case.budget_blocks, case.total_qblocks, case.cu_qblocks
    ridx, _, _ = oracle.gate_topk(case.cu_seqlens, case.logits, case.hkv, Kb)
    keep = keep_counts(ridx, cuq, case.hkv)
    say(f"  {int((keep > 64).sum())} key blocks kept by more than 64 rows (most: "
        f"{int(keep.max())}); dk/dv segments hold at most 64")
    assert keep.max() > 64, "some key blocks must span several segments"
    everything = np.ones((case.hkv, QB), np.uint8)
    run_training_workload(case, everything, everything)


def host_cache(t, name):
    """The whole cache on the host as bf16 bit patterns (uint16)."""
    import torch
    return t[name].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode_rows_check(spec, t, prob, out_rows):
    """Selection (scores, index sets, log gates) on every (sequence, kv head)
    row against the oracle, the output and lse on the rows in out_rows."""
    import torch
    ksum = sas.pool_keys(prob, t["k"])
    sel, lg, glse, scores = sas.decode_select(prob, t["q"], ksum)
    o, lse = sas.decode(prob, t["q"], t["k"], t["v"], sel, lg)
    torch.cuda.synchronize()
    sel_h, lg_h, sc_h = sel.cpu().numpy(), lg.cpu().numpy(), scores.cpu().numpy()
    G = spec.hq // spec.hkv
    q_h = t["q"].float().cpu().numpy()
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    kb, vb = host_cache(t, "k"), host_cache(t, "v")
    worst, n_out = 0.0, 0
    for b, L in enumerate(spec.seqlens):
        cur = (L - 1) // 64
        for g in range(spec.hkv):
            K = bits_f32(wl.gather_row_cache(kb, t["page_table"], b, g, L))
            qg = q_h[b, g * G:(g + 1) * G]
            ridx, rlg, rlse, rs = oracle.decode_select_row(qg, K, spec.budget_blocks,
                                                           summary=prob.summary_dtype)
            r = b * spec.hkv + g
            assert np.array_equal(sc_h[b, g, :cur], rs), (b, g, "pooled scores")
            assert np.array_equal(sel_h[r], ridx), (b, g, "selection")
            fin = np.isfinite(rlg)
            assert np.array_equal(np.isfinite(lg_h[r]), fin)
            assert np.max(np.abs(lg_h[r][fin] - rlg[fin]), initial=0.0) < 1e-5
            if (b, g) not in out_rows:
                continue
            V = bits_f32(wl.gather_row_cache(vb, t["page_table"], b, g, L))
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, spec.budget_blocks, prob.scale)
            err = float(np.max(np.abs(o_h[b, g * G:(g + 1) * G] - ro)))
            worst = max(worst, err)
            n_out += 1
            assert err <= TOL["bf16"], (b, g, err)
            assert np.max(np.abs(lse_h[b, g * G:(g + 1) * G] - rl)) <= 1e-4
    say(f"  selection of all {spec.batch * spec.hkv} rows bit-exact; output of {n_out} rows, "
        f"max |o err| {worst:.3e}")


@pytest.mark.parametrize("context", [131072, 524288])
def test_decode_contiguous_full_size(context):
    """batch 1, 32/8 heads, d 128, contiguous bf16 cache, budget 32 blocks:
    every (sequence, kv head) row against the oracle."""
    import torch
    spec = wl.decode_spec(context)
    say(f"[full {spec.name}]")
    t = wl.draw_decode_device(spec)
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, False,
                      spec.max_len)
    decode_rows_check(spec, t, prob, {(0, g) for g in range(spec.hkv)})
    del t
    torch.cuda.empty_cache()


def test_decode_paged_full_size():
    """batch 32, lengths U[32768, 131072], paged bf16 cache, budget 64
    blocks: every (sequence, kv head) row's scores, selection, log gates,
    output and lse against the oracle."""
    import torch
    spec = wl.paged_spec()
    say(f"[full {spec.name}] lengths {min(spec.seqlens)}..{max(spec.seqlens)}")
    t = wl.draw_decode_device(spec)
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                      spec.max_len, page_table=t["page_table"], num_pages=t["k"].shape[0])
    every = {(b, g) for b in range(spec.batch) for g in range(spec.hkv)}
    decode_rows_check(spec, t, prob, every)
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("summary", ["bf16", "fp8"])
def test_decode_paged_full_size_reduced_summaries(summary):
    """The paged batch with bf16 / fp8 block summaries (its selection runs in
    512-thread chunks): every row's scores, selection and log gates against
    the oracle's reading of the rounded summaries, the output of 32 rows."""
    import torch
    spec = wl.paged_spec()
    say(f"[full {spec.name} summaries {summary}]")
    t = wl.draw_decode_device(spec)
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                      spec.max_len, page_table=t["page_table"], num_pages=t["k"].shape[0],
                      summary_dtype=summary)
    some = {(b, b % spec.hkv) for b in range(spec.batch)}
    decode_rows_check(spec, t, prob, some)
    del t
    torch.cuda.empty_cache()


def test_decode_step_loop_paged_full_size():
    """The paged batch as a step loop: each sequence prefilled to the largest
    multiple of 64 below its length minus one (summaries by sas_pool_keys),
    then two steps of sas_decode_append with new tokens, the first of which
    opens a block in every sequence, so the append summarises the block it
    closes.  After the steps: every row's summaries equal the oracle's of the
    updated cache bit for bit, every row's selection the oracle's, and the
    output of 32 rows is within the bf16 bar."""
    import torch
    from tests.gpu_helpers import summaries_f32
    spec = wl.paged_spec()
    t = wl.draw_decode_device(spec)
    L0 = [64 * ((L - 2) // 64) for L in spec.seqlens]
    say(f"[full {spec.name} step loop] prefix {min(L0)}..{max(L0)}, 2 steps")
    B, hkv, d, G = spec.batch, spec.hkv, spec.d, spec.hq // spec.hkv

    # one summary layout for every step (the stride of the longest history)
    stride = -(-max((L - 1) // 64 for L in spec.seqlens) // 64) * 64

    def problem(lens):
        return sas.Decode(lens, spec.hq, hkv, d, spec.budget_blocks, True, spec.max_len,
                          page_table=t["page_table"], num_pages=t["k"].shape[0],
                          nblk_stride=stride)

    ksum = sas.pool_keys(problem(L0), t["k"])
    g = np.random.Generator(np.random.PCG64(97))
    new = [{nm: wl.round_bf16(wl.normal(g, (B, hkv, d))) for nm in ("k", "v")}
           for _ in range(2)]
    for s in range(2):
        lens = [n + s + 1 for n in L0]
        k_new, v_new = (torch.from_numpy(new[s][nm].view(np.int16)).view(torch.bfloat16).cuda()
                        for nm in ("k", "v"))
        sas.decode_append(problem(lens), k_new, v_new, t["k"], t["v"], ksum)
    prob = problem(lens)
    sel, lg, _, _ = sas.decode_select(prob, t["q"], ksum)
    o, lse = sas.decode(prob, t["q"], t["k"], t["v"], sel, lg)
    torch.cuda.synchronize()
    ks_h, sel_h, lg_h = summaries_f32(ksum), sel.cpu().numpy(), lg.cpu().numpy()
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    q_h = t["q"].float().cpu().numpy()
    kb, vb = host_cache(t, "k"), host_cache(t, "v")
    pt = t["page_table"]
    for s in range(2):  # the host caches with the steps' tokens
        for b in range(B):
            pos = L0[b] + s
            kb[pt[b, pos // 64], :, pos % 64] = new[s]["k"][b]
            vb[pt[b, pos // 64], :, pos % 64] = new[s]["v"][b]
    worst = 0.0
    for b, L in enumerate(lens):
        cur = (L - 1) // 64
        for gg in range(hkv):
            K = bits_f32(wl.gather_row_cache(kb, pt, b, gg, L))
            assert np.array_equal(ks_h[b, gg, :cur], oracle.pool_keys_row(K)), (b, gg, "ksum")
            qg = q_h[b, gg * G:(gg + 1) * G]
            ridx, rlg, _, _ = oracle.decode_select_row(qg, K, spec.budget_blocks)
            r = b * hkv + gg
            assert np.array_equal(sel_h[r], ridx), (b, gg, "selection")
            fin = np.isfinite(rlg)
            assert np.max(np.abs(lg_h[r][fin] - rlg[fin]), initial=0.0) < 1e-5
            if gg != b % hkv:
                continue
            V = bits_f32(wl.gather_row_cache(vb, pt, b, gg, L))
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, spec.budget_blocks, prob.scale)
            err = float(np.max(np.abs(o_h[b, gg * G:(gg + 1) * G] - ro)))
            worst = max(worst, err)
            assert err <= TOL["bf16"], (b, gg, err)
            assert np.max(np.abs(lse_h[b, gg * G:(gg + 1) * G] - rl)) <= 1e-4
    say(f"  summaries and selection of all {B * hkv} rows bit-exact after the steps; "
        f"output of {B} rows, max |o err| {worst:.3e}")
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("summary", ["f32", "fp8"])
def test_hier_selection_paged_full_size(summary):
    """The hierarchical selection on the paged batch (coarse_keep = budget - 1
    super-blocks of 8 blocks): every row's super-block summaries, candidate
    scores and index sets bit-exact against the oracle, log gates to 1e-5."""
    import torch
    from tests.gpu_helpers import summaries_f32
    spec = wl.paged_spec()
    say(f"[full {spec.name} hierarchical selection, summaries {summary}]")
    t = wl.draw_decode_device(spec)
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                      spec.max_len, page_table=t["page_table"], num_pages=t["k"].shape[0],
                      summary_dtype=summary)
    C, Kb, hkv, G = spec.budget_blocks - 1, spec.budget_blocks, spec.hkv, spec.hq // spec.hkv
    ksum = sas.pool_keys(prob, t["k"])
    csum = sas.pool_coarse(prob, ksum)
    sel, lg, glse, scores = sas.decode_select_hier(prob, t["q"], ksum, csum, C)
    torch.cuda.synchronize()
    cs_h, sc_h = summaries_f32(csum), scores.cpu().numpy()
    sel_h, lg_h, glse_h = sel.cpu().numpy(), lg.cpu().numpy(), glse.cpu().numpy()
    q_h = t["q"].float().cpu().numpy()
    kb, pt = host_cache(t, "k"), t["page_table"]
    for b, L in enumerate(spec.seqlens):
        for gg in range(hkv):
            K = bits_f32(wl.gather_row_cache(kb, pt, b, gg, L))
            qg = q_h[b, gg * G:(gg + 1) * G]
            cbar = oracle.coarse_summaries_row(oracle.pool_keys_row(K, summary=summary), summary)
            assert np.array_equal(cs_h[b, gg, :cbar.shape[0]], cbar), (b, gg, "coarse summaries")
            ridx, rlg, rlse, rs, cand = oracle.decode_select_row_hier(qg, K, Kb, C,
                                                                      summary=summary)
            r = b * hkv + gg
            assert np.array_equal(sc_h[b, gg, cand], rs[cand]), (b, gg, "candidate scores")
            assert np.array_equal(sel_h[r], ridx), (b, gg, "selection")
            fin = np.isfinite(rlg)
            assert np.array_equal(np.isfinite(lg_h[r]), fin)
            assert np.max(np.abs(lg_h[r][fin] - rlg[fin]), initial=0.0) < 1e-5
            assert abs(glse_h[r] - rlse) < 1e-5
    say(f"  all {spec.batch * hkv} rows bit-exact")
    del t
    torch.cuda.empty_cache()
