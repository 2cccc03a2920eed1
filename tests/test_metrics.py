"""CPU checks of the algorithmic work counts behind the benchmark's figures:
the attended (query, key) pairs are counted token by token from the oracle's
own selections, and the decode byte counts block by block from its decode
selections, then compared with the closed forms in metrics.py."""
import numpy as np

import oracle
from trainable_block_sparse_gate_amd import metrics
from trainable_block_sparse_gate_amd import workloads as wl


def test_attended_pairs_match_a_token_by_token_count():
    lengths, hq, hkv, d, Kb = [1, 63, 64, 65, 700, 64 * 9], 4, 2, 64, 5
    case = wl.make_varlen("pairs", lengths, hq, hkv, d, Kb, dtype="f32", logit_sigma=2.0,
                          workload_id=97, with_dO=False)
    idx, _, _ = oracle.gate_topk(case.cu_seqlens, case.logits, hkv, Kb)
    cuq = case.cu_qblocks
    for g in range(hkv):
        count = 0
        for s, n in enumerate(lengths):
            nb = (n + 63) // 64
            for i in range(nb):
                kept = [int(j) for j in idx[g, cuq[s] + i] if j >= 0]
                assert kept[-1] == i  # the current block, last
                for t in range(64 * i, min(64 * i + 64, n)):
                    count += 64 * (len(kept) - 1) + (t - 64 * i + 1)
        assert count == metrics.pairs_per_head(lengths, Kb)
    f = metrics.train_flops(lengths, hq, d, Kb)
    assert f["pairs"] == hq * metrics.pairs_per_head(lengths, Kb)
    assert (f["fwd"], f["bwd"]) == (4 * d * f["pairs"], 10 * d * f["pairs"])
    assert f["dq_kernel"] + f["dkdv_kernel"] == f["bwd"]


def test_decode_bytes_match_a_block_by_block_count():
    seqlens, hq, hkv, d, Kb = [1, 64, 65, 64 * 7 + 3, 64 * 40], 4, 2, 64, 6
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, False, seed=98)
    G = hq // hkv
    kv = scan = 0
    for b, L in enumerate(seqlens):
        cur = (L - 1) // 64
        for g in range(hkv):
            K = host["k"][b, g, :L]
            idx, _, _, _ = oracle.decode_select_row(host["q"][b, g * G:(g + 1) * G], K, Kb)
            for j in idx[idx >= 0]:
                tokens = 64 if j < cur else L - 64 * cur
                kv += tokens * d * 2 * 2  # K and V rows, bf16
            scan += cur * d * 4  # fp32 summaries of the history blocks
    assert kv == metrics.decode_kv_bytes(seqlens, hkv, d, Kb)
    assert scan == metrics.decode_scan_bytes(seqlens, hkv, d)
    assert metrics.decode_scan_bytes(seqlens, hkv, d, 1) * 4 == scan
