"""One decode step (cache append, selection, attention), and one training
step (gate, forward, backward, gate backward), captured in a HIP graph and
replayed, through the C ABI.

Once its outputs and workspaces are given, every entry point of the step only
launches kernels on the caller's stream (no allocation, copy, fill or
synchronisation), so the step can be captured whole.  Each replay, with eager
work and a synchronisation between replays, must give the bits of the same
step run eagerly.  The step is idempotent (the lengths already count the new
token, which is written at the same place each time), so the caches and
summaries must also come out unchanged.  The eager step itself is held to the
oracle: selection bit-exact, output at the bf16 bar.  Both decode entry
points are captured: the one with a workspace and the one that allocates
nothing.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, dev_tensor, say
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl

pytestmark = pytest.mark.gpu

# the first and third lengths make their new token open a block (L - 1 a
# multiple of 64), so the append also summarises the block it closes
SEQLENS = [64 * 40 + 1, 64 * 17 + 30, 64 * 5 + 1, 200]


def _garbage(ts):
    import torch
    for t in ts:
        t.fill_(-7 if t.dtype == torch.int32 else float("nan"))


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_step_graph_replays_match_eager(paged, noalloc):
    import torch
    hq, hkv, d, Kb = 8, 2, 128, 12
    say(f"[graph step paged={paged} noalloc={noalloc}]")
    host = wl.draw_decode_host_small(SEQLENS, hq, hkv, d, Kb, paged, seed=91)
    prob = sas.Decode(SEQLENS, hq, hkv, d, Kb, paged, max(SEQLENS),
                      page_table=host["page_table"],
                      num_pages=host["k"].shape[0] if paged else 0)
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    vc = dev_tensor(host["v"], host["v_bits"], "bf16")
    ksum = sas.pool_keys(prob, kc)
    g = np.random.Generator(np.random.PCG64(92))
    new_bits = {nm: wl.round_bf16(wl.normal(g, (len(SEQLENS), hkv, d))) for nm in ("k", "v")}
    k_new = dev_tensor(wl.bf16_bits_to_f32(new_bits["k"]), new_bits["k"], "bf16")
    v_new = dev_tensor(wl.bf16_bits_to_f32(new_bits["v"]), new_bits["v"], "bf16")
    sws = sas.decode_select_workspace(prob)
    ws = torch.empty(max(1, sas.decode_workspace_bytes(prob)), dtype=torch.uint8, device="cuda")

    def alloc():
        sel_out = sas.decode_select(prob, q, ksum, workspace=sws)
        return sel_out, sas.decode(prob, q, kc, vc, sel_out[0], sel_out[1], workspace=ws)

    def step(sel_out, dec_out):
        sas.decode_append(prob, k_new, v_new, kc, vc, ksum)
        sas.decode_select(prob, q, ksum, out=sel_out, workspace=sws)
        if noalloc:
            sas.decode_noalloc(prob, q, kc, vc, sel_out[0], sel_out[1], out=dec_out)
        else:
            sas.decode(prob, q, kc, vc, sel_out[0], sel_out[1], workspace=ws, out=dec_out)

    # the eager step, its results kept
    ref_sel, ref_dec = alloc()
    step(ref_sel, ref_dec)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*ref_sel, *ref_dec, kc, vc, ksum)]

    # warm-up on a side stream, then capture into a graph
    g_sel, g_dec = alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(g_sel, g_dec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_sel, g_dec)
    names = ["sel_idx", "sel_lg", "gate_lse", "scores", "o", "lse", "k_cache", "v_cache", "ksum"]
    for r in range(3):
        _garbage((*g_sel, *g_dec))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (*g_sel, *g_dec, kc, vc, ksum)
        for nm, a, b in zip(names, got, ref):
            if nm == "scores":  # past each row's history the scores are padding
                for bi, L in enumerate(SEQLENS):
                    cur = (L - 1) // 64
                    assert torch.equal(a[bi, :, :cur], b[bi, :, :cur]), (r, nm, bi)
            else:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, nm)
    say("  3 replays: the eager step's bits")

    # the eager step against the oracle, on the caches with the new token
    G = hq // hkv
    sel_h, lg_h = ref_sel[0].cpu().numpy(), ref_sel[1].cpu().numpy().astype(np.float64)
    o_h, lse_h = ref_dec[0].float().cpu().numpy(), ref_dec[1].cpu().numpy()
    kh, vh = host["k"].copy(), host["v"].copy()
    kn, vn = wl.bf16_bits_to_f32(new_bits["k"]), wl.bf16_bits_to_f32(new_bits["v"])
    for b, L in enumerate(SEQLENS):
        t = L - 1
        for gg in range(hkv):
            if paged:
                page = host["page_table"][b, t // 64]
                kh[page, gg, t % 64], vh[page, gg, t % 64] = kn[b, gg], vn[b, gg]
            else:
                kh[b, gg, t], vh[b, gg, t] = kn[b, gg], vn[b, gg]
    for b, L in enumerate(SEQLENS):
        for gg in range(hkv):
            K = wl.gather_row_cache(kh, host["page_table"], b, gg, L)
            V = wl.gather_row_cache(vh, host["page_table"], b, gg, L)
            qg = host["q"][b, gg * G:(gg + 1) * G]
            ridx, rlg, _, _ = oracle.decode_select_row(qg, K, Kb)
            r = b * hkv + gg
            assert np.array_equal(sel_h[r], ridx), (b, gg, "selection")
            ro, rl = oracle.decode_row(qg, K, V, ridx, rlg, Kb, prob.scale)
            assert np.max(np.abs(o_h[b, gg * G:(gg + 1) * G] - ro)) <= TOL["bf16"]
            assert np.max(np.abs(lse_h[b, gg * G:(gg + 1) * G] - rl)) <= 1e-4
    say("  eager step: selection bit-exact, output at the bf16 bar")


def test_training_step_graph_replays_match_eager():
    """Gate + Top-K, forward, backward and gate backward captured in one
    graph (outputs allocated once, inside the capture, from the graph's
    pool): every replay gives the eager step's bits, the kernels being
    deterministic; the eager selection and forward are held to the oracle."""
    import torch
    from tests.gpu_helpers import assert_close, case_to_device
    lengths, hq, hkv, d, Kb = [700, 64 * 9 + 5, 300], 8, 2, 128, 4
    say("[graph training step]")
    case = wl.make_varlen("graph", lengths, hq, hkv, d, Kb, dtype="bf16", logit_sigma=2.0,
                          workload_id=95)
    prob = sas.Varlen(lengths, hq, hkv, d, Kb)
    dv = case_to_device(case)
    ws = torch.empty(max(1, sas.bwd_workspace_bytes(prob)), dtype=torch.uint8, device="cuda")

    def step():
        sel, lg, glse = sas.gate_topk(prob, dv["logits"])
        o, lse = sas.fwd(prob, dv["q"], dv["k"], dv["v"], sel, lg)
        dq, dk, dvv, dlg = sas.bwd(prob, dv["q"], dv["k"], dv["v"], o, dv["dO"], lse, sel, lg,
                                   workspace=ws)
        dz = sas.gate_bwd(prob, dv["logits"], sel, glse, dlg)
        return sel, lg, glse, o, lse, dq, dk, dvv, dlg, dz

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    names = ["sel_idx", "sel_lg", "gate_lse", "o", "lse", "dq", "dk", "dv", "dlg", "d_logits"]
    for r in range(3):
        _garbage(outs)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for nm, a, b in zip(names, outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, nm)
    say("  3 replays: the eager step's bits")
    ridx, rlg, _ = oracle.gate_topk(case.cu_seqlens, case.logits, hkv, Kb)
    assert np.array_equal(ref[0].cpu().numpy(), ridx)
    ro, rl = oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, ridx, rlg, Kb, case.scale)
    assert_close("o", ref[3].float().cpu().numpy(), ro, TOL["bf16"])
    assert_close("lse", ref[4].cpu().numpy(), rl, TOL["bf16"])
