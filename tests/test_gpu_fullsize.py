"""GPU parity at the workloads' full sizes, through the C ABI, in the launch
configuration bench.py times.

Selected index sets and log gates are compared on every row.  Outputs and
gradients are compared on sampled rows (dq, d log-gate, d logits, o, lse)
and sampled key blocks (dk, dv: every row that keeps the block is
recomputed by the oracle).  Invariants that hold at any size are checked on
every row: each log-gate-gradient row sums to zero, selections are
ascending with the current block kept, decode selections are valid.
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


def run_training_workload(case, n_rows=12, n_kblocks=8, seed=0, max_keepers=16):
    import torch
    prob = sas.Varlen(case.lengths, case.hq, case.hkv, case.d, case.budget_blocks,
                      dtype=case.dtype)
    dv = case_to_device(case)
    say(f"[full {case.name}] T={case.T} rows={case.hkv * case.total_qblocks}")
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
    assert_close("log_gate", lg.cpu().numpy()[fin], rlg[fin], 1e-5)
    # invariant on every row: the log-gate gradient of a row sums to zero
    dlg_h = dlg.cpu().numpy()
    row_sums = np.abs(dlg_h.sum(-1))
    say(f"  max |sum_slot dlg| over all rows = {row_sums.max():.3e}")
    assert row_sums.max() < TOL[case.dtype]

    g = np.random.default_rng(seed)
    QB = case.total_qblocks
    cu, cuq = case.cu_seqlens, case.cu_qblocks
    rm = np.zeros((case.hkv, QB), np.uint8)
    picks = set(g.integers(0, QB, n_rows - 2).tolist()) | {0, QB - 1}
    for Q in picks:
        rm[g.integers(0, case.hkv), Q] = 1
    # key blocks for dk/dv: the oracle recomputes every row that keeps one, so
    # pick blocks with at most `max_keepers` keeping rows (hot blocks split
    # over many segments have their own test at a smaller size)
    km = np.zeros((case.hkv, QB), np.uint8)
    for x in range(n_kblocks):
        gg = x % case.hkv
        keep = np.zeros(QB, int)
        for Q in range(QB):
            s = np.searchsorted(cuq, Q, side="right") - 1
            for j in ridx[gg, Q]:
                if j >= 0:
                    keep[cuq[s] + j] += 1
        cand = np.nonzero(keep <= max_keepers)[0]
        km[gg, int(g.choice(cand))] = 1
    ro, rl = oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, ridx, rlg, Kb, case.scale,
                        row_mask=rm)
    rdq, rdk, rdv, rdlg = oracle.bwd(case.cu_seqlens, case.q, case.k, case.v, case.dO, ridx,
                                     rlg, Kb, case.scale, row_mask=rm, kblk_mask=km)
    tok = np.zeros((case.T, case.hq), bool)
    ktok = np.zeros((case.T, case.hkv), bool)
    G = case.hq // case.hkv
    for gg in range(case.hkv):
        for Q in range(QB):
            s = np.searchsorted(cuq, Q, side="right") - 1
            i = Q - cuq[s]
            a = cu[s] + 64 * i
            b = min(cu[s + 1], a + 64)
            if rm[gg, Q]:
                tok[a:b, gg * G:(gg + 1) * G] = True
            if km[gg, Q]:
                ktok[a:b, gg] = True
    assert_close("o (sampled rows)", o.float().cpu().numpy()[tok], ro[tok], TOL[case.dtype])
    assert_close("lse (sampled rows)", lse.cpu().numpy().T[tok], rl.T[tok], TOL[case.dtype])
    assert_close("dq (sampled rows)", dq.cpu().numpy()[tok], rdq[tok], TOL[case.dtype])
    rows = rm.astype(bool)
    assert_close("dlg (sampled rows)", dlg_h[rows], rdlg[rows], TOL[case.dtype])
    assert_close("dk (sampled key blocks)", dk.cpu().numpy()[ktok], rdk[ktok], TOL[case.dtype])
    assert_close("dv (sampled key blocks)", dvv.cpu().numpy()[ktok], rdv[ktok], TOL[case.dtype])
    rdz = oracle.gate_bwd(case.cu_seqlens, case.logits, ridx, np.where(rm[..., None], rdlg, 0),
                          case.hkv, Kb)
    assert_close("d_logits (sampled rows)", dz.cpu().numpy()[rows], rdz[rows], TOL[case.dtype])


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
    """1 x 16384 tokens, 32/8 heads, d 128, bf16, budget 16 blocks."""
    run_training_workload(wl.layer16k(), n_rows=12, n_kblocks=8, seed=2)


def test_varlen_full_size():
    """4 packed sequences (32768/24576/16384/8192), 32/8 heads, d 128, bf16,
    budget 32 blocks, logits N(0,3) with boosted key-block columns."""
    run_training_workload(wl.varlen(), n_rows=12, n_kblocks=8, seed=3, max_keepers=8)


def decode_rows_check(spec, t, prob, rows):
    import torch
    ksum = sas.pool_keys(prob, t["k"])
    sel, lg, glse, scores = sas.decode_select(prob, t["q"], ksum)
    o, lse = sas.decode(prob, t["q"], t["k"], t["v"], sel, lg)
    torch.cuda.synchronize()
    sel_h, lg_h = sel.cpu().numpy(), lg.cpu().numpy()
    # validity on every row
    for b, L in enumerate(spec.seqlens):
        cur = (L - 1) // 64
        for g in range(spec.hkv):
            r = sel_h[b * spec.hkv + g]
            k = min(spec.budget_blocks - 1, cur)
            assert np.all(np.diff(r[:k]) > 0) and r[k] == cur and np.all(r[k + 1:] == -1)
    G = spec.hq // spec.hkv
    q_h = t["q"].float().cpu().numpy()
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for (b, g) in rows:
        L = spec.seqlens[b]
        if t["page_table"] is None:
            K = t["k"][b, g, :L].float().cpu().numpy()
            V = t["v"][b, g, :L].float().cpu().numpy()
        else:
            nb = (L + 63) // 64
            pages = torch.from_numpy(t["page_table"][b, :nb]).long().cuda()
            K = t["k"][pages, g].reshape(-1, spec.d)[:L].float().cpu().numpy()
            V = t["v"][pages, g].reshape(-1, spec.d)[:L].float().cpu().numpy()
        qg = q_h[b, g * G:(g + 1) * G]
        ridx, rlg, rlse, rs = oracle.decode_select_row(qg, K, spec.budget_blocks)
        r = b * spec.hkv + g
        assert np.array_equal(sel_h[r], ridx), (b, g)
        fin = np.isfinite(rlg)
        assert np.max(np.abs(lg_h[r][fin] - rlg[fin])) < 1e-5
        ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, spec.budget_blocks, prob.scale)
        err = float(np.max(np.abs(o_h[b, g * G:(g + 1) * G] - ro)))
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, g, err)
        assert np.max(np.abs(lse_h[b, g * G:(g + 1) * G] - rl)) <= 1e-4
    say(f"  {len(rows)} rows checked against the oracle, max |o err| {worst:.3e}")


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
    decode_rows_check(spec, t, prob, [(0, g) for g in range(spec.hkv)])
    del t
    torch.cuda.empty_cache()


def test_decode_paged_full_size():
    """batch 32, lengths U[32768, 131072], paged bf16 cache, budget 64
    blocks: every row's selection is valid, 16 sampled rows against the
    oracle."""
    import torch
    spec = wl.paged_spec()
    say(f"[full {spec.name}] lengths {min(spec.seqlens)}..{max(spec.seqlens)}")
    t = wl.draw_decode_device(spec)
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                      spec.max_len, page_table=t["page_table"], num_pages=t["k"].shape[0])
    g = np.random.default_rng(5)
    rows = sorted({(int(b), int(h)) for b, h in zip(g.integers(0, spec.batch, 16),
                                                    g.integers(0, spec.hkv, 16))})
    decode_rows_check(spec, t, prob, rows)
    del t
    torch.cuda.empty_cache()
