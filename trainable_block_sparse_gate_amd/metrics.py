"""Algorithmic work of the SAS hot path, for throughput and roofline figures.

Attended (query, key) pairs per query head: a row (query block i with nq
tokens) keeps k = min(Kb - 1, i) history blocks, each whole (64 keys), and
its own block causally (nq (nq + 1) / 2 pairs).  History blocks are always
full, so the count depends only on the sequence lengths and the budget.

FLOPs per pair and head (multiply-add = 2):
  forward            4 d   (q.k, p.v)
  backward          10 d   (recompute q.k, dO.v, dV, dQ, dK)
The backward runs as two kernels, each recomputing q.k and dO.v (the dq
kernel also forms dS.K, the dk/dv kernel P^T dO and dS^T Q), so they
execute 6 d and 8 d.  Roofline figures credit each kernel only with
algorithmic work: its own products plus half of the shared recomputation,
  dq kernel          4 d   (dS.K 2d + half of q.k and dO.v)
  dk/dv kernel       6 d   (P^T dO, dS^T Q 4d + half of q.k and dO.v)
which adds up to the backward's 10 d.
Decode bytes: every kept block's K and V rows actually read (history blocks
whole, the current block's present tokens), bf16.
"""
import numpy as np

BLOCK = 64

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # fp32 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E


def pairs_per_head(lengths, budget_blocks):
    total = 0
    for n in lengths:
        nb = (n + BLOCK - 1) // BLOCK
        for i in range(nb):
            nq = min(BLOCK, n - i * BLOCK)
            k = min(budget_blocks - 1, i)
            total += k * BLOCK * nq + nq * (nq + 1) // 2
    return total


def train_flops(lengths, hq, d, budget_blocks):
    pairs = pairs_per_head(lengths, budget_blocks) * hq
    return {"pairs": pairs, "fwd": 4 * d * pairs, "bwd": 10 * d * pairs,
            "dq_kernel": 4 * d * pairs, "dkdv_kernel": 6 * d * pairs,
            "dq_kernel_executed": 6 * d * pairs, "dkdv_kernel_executed": 8 * d * pairs}


def decode_kv_bytes(seqlens, hkv, d, budget_blocks, elem_bytes=2):
    """K+V bytes read by the decode kernel over all (sequence, kv head) rows."""
    total = 0
    for L in seqlens:
        cur = (L - 1) // BLOCK
        hist = min(budget_blocks - 1, cur)
        tokens = hist * BLOCK + (L - cur * BLOCK)
        total += tokens * d * elem_bytes * 2 * hkv
    return total


def decode_scan_bytes(seqlens, hkv, d, elem_bytes=4):
    """Block-summary bytes the pooled selector scans (4 per value for fp32
    summaries, 2 for bf16)."""
    return sum((L - 1) // BLOCK for L in seqlens) * hkv * d * elem_bytes


def decode_q_bytes(batch, hq, d):
    return batch * hq * d * 2
