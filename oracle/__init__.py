"""Plain fp64 CPU oracle for SAS gated block-sparse attention (ctypes + numpy).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may import this; the product library and its binding never do.
The arithmetic lives in ``sas_oracle.c`` (see its header for the passages of
the SAS pages each step follows and the readings taken where they are
silent).  This module only marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force, finite differences and library routines.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

GATE_HIST = 0     # softmax over the history blocks; current block log-gate 0
GATE_ALL = 1      # softmax over history and current block
GATE_SIGMOID = 2  # independent gates sigmoid(s); current block log-gate 0
GATE_RAW = 3      # the raw logit as the log-gate; current block log-gate 0
GATE_STE = 4      # hard gate 1 forward, soft-softmax straight-through backward

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = ctypes.CDLL(LIB)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u8(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.uint8)


def num_qblocks(cu_seqlens, blk=64):
    cu = _i32(cu_seqlens)
    lib = _load()
    lib.sas_oracle_num_qblocks.restype = ctypes.c_int
    return lib.sas_oracle_num_qblocks(len(cu) - 1, _p(cu), blk)


def gate_topk(cu_seqlens, logits, hkv, Kb, mode=GATE_HIST, blk=64):
    """Gate + hard Top-K for every (kv head, query block) row.

    logits: [hkv][QB][ld] float32.  Returns (sel_idx int32 [hkv,QB,Kb],
    sel_lg float64 [hkv,QB,Kb], gate_lse float64 [hkv,QB]).
    """
    cu = _i32(cu_seqlens)
    lg = _f32(logits)
    QB = num_qblocks(cu, blk)
    ld = lg.shape[-1]
    assert lg.size == hkv * QB * ld
    idx = np.empty((hkv, QB, Kb), np.int32)
    sl = np.empty((hkv, QB, Kb), np.float64)
    lse = np.empty((hkv, QB), np.float64)
    rc = _load().sas_oracle_gate_topk(
        len(cu) - 1, _p(cu), blk, hkv, Kb, mode, _p(lg), ctypes.c_int64(ld),
        _p(idx), _p(sl), _p(lse))
    if rc:
        raise ValueError(f"oracle gate_topk failed: {rc}")
    return idx, sl, lse


def gate_row(scores, i, Kb, mode=GATE_HIST):
    """Gate + Top-K of one row whose scores are given directly (decode)."""
    s = _f32(scores)
    assert s.size >= i + (1 if mode == GATE_ALL else 0)
    if s.size == 0:
        s = np.zeros(1, np.float32)
    idx = np.empty(Kb, np.int32)
    sl = np.empty(Kb, np.float64)
    lse = ctypes.c_double()
    _load().sas_oracle_gate_row(_p(s), i, Kb, mode, _p(idx), _p(sl), ctypes.byref(lse))
    return idx, sl, lse.value


def fwd(cu_seqlens, q, k, v, sel_idx, sel_lg, Kb, scale, row_mask=None, blk=64):
    """Gated block-sparse forward.  q [T,hq,d], k/v [T,hkv,d] (taken as float64).

    Returns (o float64 [T,hq,d], lse float64 [hq,T]); rows skipped by row_mask
    are left as NaN.
    """
    cu = _i32(cu_seqlens)
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    idx, sl = _i32(sel_idx), _f64(sel_lg)
    o = np.full((T, hq, d), np.nan)
    lse = np.full((hq, T), np.nan)
    rm = _u8(row_mask)
    rc = _load().sas_oracle_fwd(
        len(cu) - 1, _p(cu), blk, hq, hkv, d, Kb, ctypes.c_double(scale),
        _p(q), _p(k), _p(v), _p(idx), _p(sl), _p(rm), _p(o), _p(lse))
    if rc:
        raise ValueError(f"oracle fwd failed: {rc}")
    return o, lse


def bwd(cu_seqlens, q, k, v, dO, sel_idx, sel_lg, Kb, scale, row_mask=None,
        kblk_mask=None, blk=64):
    """Gradients of the gated forward: (dq, dk, dv, dlg), all float64."""
    cu = _i32(cu_seqlens)
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    T, hq, d = q.shape
    hkv = k.shape[1]
    idx, sl = _i32(sel_idx), _f64(sel_lg)
    dq = np.empty((T, hq, d))
    dk = np.empty((T, hkv, d))
    dv = np.empty((T, hkv, d))
    dlg = np.empty(idx.shape)
    rc = _load().sas_oracle_bwd(
        len(cu) - 1, _p(cu), blk, hq, hkv, d, Kb, ctypes.c_double(scale),
        _p(q), _p(k), _p(v), _p(dO), _p(idx), _p(sl), _p(_u8(row_mask)),
        _p(_u8(kblk_mask)), _p(dq), _p(dk), _p(dv), _p(dlg))
    if rc:
        raise ValueError(f"oracle bwd failed: {rc}")
    return dq, dk, dv, dlg


def fwd_outer(cu_seqlens, q, k, v, sel_idx, sel_lg, Kb, scale, blk=64):
    """Outer-gate forward (the gate-position ablation): softmax of the
    ungated logits, each key's value scaled by its block's gate.  Returns
    (o, lse) float64; lse is that of the ungated logits."""
    cu = _i32(cu_seqlens)
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    idx, sl = _i32(sel_idx), _f64(sel_lg)
    o = np.full((T, hq, d), np.nan)
    lse = np.full((hq, T), np.nan)
    rc = _load().sas_oracle_fwd_outer(
        len(cu) - 1, _p(cu), blk, hq, hkv, d, Kb, ctypes.c_double(scale),
        _p(q), _p(k), _p(v), _p(idx), _p(sl), _p(o), _p(lse))
    if rc:
        raise ValueError(f"oracle fwd_outer failed: {rc}")
    return o, lse


def bwd_outer(cu_seqlens, q, k, v, dO, sel_idx, sel_lg, Kb, scale, blk=64):
    """Gradients of the outer-gate forward: (dq, dk, dv, dlg), float64."""
    cu = _i32(cu_seqlens)
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    T, hq, d = q.shape
    hkv = k.shape[1]
    idx, sl = _i32(sel_idx), _f64(sel_lg)
    dq = np.empty((T, hq, d))
    dk = np.empty((T, hkv, d))
    dv = np.empty((T, hkv, d))
    dlg = np.empty(idx.shape)
    rc = _load().sas_oracle_bwd_outer(
        len(cu) - 1, _p(cu), blk, hq, hkv, d, Kb, ctypes.c_double(scale),
        _p(q), _p(k), _p(v), _p(dO), _p(idx), _p(sl), _p(dq), _p(dk), _p(dv), _p(dlg))
    if rc:
        raise ValueError(f"oracle bwd_outer failed: {rc}")
    return dq, dk, dv, dlg


def gate_bwd(cu_seqlens, logits, sel_idx, dlg, hkv, Kb, mode=GATE_HIST, blk=64):
    """d logits [hkv,QB,ld] from d log-gate through the gate softmax."""
    cu = _i32(cu_seqlens)
    lg = _f32(logits)
    ld = lg.shape[-1]
    out = np.empty(lg.shape, np.float64)
    _load().sas_oracle_gate_bwd(
        len(cu) - 1, _p(cu), blk, hkv, Kb, mode, _p(lg), ctypes.c_int64(ld),
        _p(_i32(sel_idx)), _p(_f64(dlg)), _p(out))
    return out


def round_bf16(x):
    """Nearest bf16 value (ties to even) of every fp32 entry, as fp32."""
    x = _f32(x)
    out = np.empty_like(x)
    _load().sas_oracle_round_bf16(ctypes.c_int64(x.size), _p(x), _p(out))
    return out


def round_e4m3(x):
    """Nearest fp8 e4m3 value (ties to even; 480 and beyond, infinities and
    NaN give NaN) of every fp32 entry, as fp32."""
    x = _f32(x)
    out = np.empty_like(x)
    _load().sas_oracle_round_e4m3(ctypes.c_int64(x.size), _p(x), _p(out))
    return out


def pool_keys_row(K, blk=64, summary="f32"):
    """Block summaries [nhist, d] of one (sequence, kv head) cache K [L, d]:
    the fp32 means, or those rounded to bf16 (summary="bf16") or to fp8 e4m3
    (summary="fp8"), as fp32."""
    K = _f32(K)
    L, d = K.shape
    nhist = (L - 1) // blk
    out = np.empty((max(nhist, 1), d), np.float32)
    _load().sas_oracle_pool_keys_row(L, blk, d, _p(K), _p(out))
    out = out[:nhist]
    if summary == "bf16":
        return round_bf16(out)
    if summary == "fp8":
        return round_e4m3(out)
    return out


def decode_scores_row(q, kbar):
    """fp32 pooled scores [nhist] from the group's queries q [G, d]."""
    q, kb = _f32(q), _f32(kbar)
    G, d = q.shape
    nhist = kb.shape[0]
    out = np.empty(max(nhist, 1), np.float32)
    if nhist:
        _load().sas_oracle_decode_scores_row(nhist, d, G, _p(q), _p(kb), _p(out))
    return out[:nhist]


def decode_select_row(q, K, Kb, mode=GATE_HIST, blk=64, summary="f32"):
    """Summaries -> pooled scores -> gate + Top-K for one decode row."""
    L = K.shape[0]
    cur = (L - 1) // blk
    kbar = pool_keys_row(K, blk, summary)
    s = decode_scores_row(q, kbar)
    idx, sl, lse = gate_row(s, cur, Kb, mode)
    return idx, sl, lse, s


COARSE_BLOCKS = 8  # history blocks per super-block of the hierarchical selection


def coarse_summaries_row(kbar, summary="f32", F=COARSE_BLOCKS):
    """Super-block summaries [nhist // F, d] from the stored block summaries
    kbar [nhist, d]: the fp32 mean of each F consecutive blocks (summed in
    block order), rounded like the block summaries (bf16 / fp8 e4m3)."""
    kb = _f32(kbar)
    nhist, d = kb.shape
    nsup = nhist // F
    out = np.empty((max(nsup, 1), d), np.float32)
    _load().sas_oracle_coarse_summaries(nhist, d, F, _p(kb), _p(out))
    out = out[:nsup]
    if summary == "bf16":
        return round_bf16(out)
    if summary == "fp8":
        return round_e4m3(out)
    return out


def decode_select_row_hier(q, K, Kb, coarse_keep, blk=64, summary="f32", F=COARSE_BLOCKS):
    """Hierarchical (coarse-to-fine) selection of one decode row (review
    7-2): score the super-block summaries, keep the coarse_keep best
    super-blocks (earlier on ties), then take the gate + Top-K over the
    candidate blocks only: every block of a kept super-block and the
    trailing history blocks that form no complete super-block, in block
    order.  The gates are normalised over the candidates.  Returns
    (sel_idx, log gates, gate lse, fine scores of every history block,
    candidate blocks)."""
    L = K.shape[0]
    cur = (L - 1) // blk
    kbar = pool_keys_row(K, blk, summary)
    nhist = kbar.shape[0]
    cbar = coarse_summaries_row(kbar, summary, F)
    nsup = cbar.shape[0]
    S = decode_scores_row(q, cbar)
    cidx, _, _ = gate_row(S, nsup, coarse_keep + 1)  # the coarse_keep best, ascending
    kept = cidx[:min(coarse_keep, nsup)]
    parts = [F * int(J) + np.arange(F) for J in kept] + [np.arange(F * nsup, nhist)]
    cand = np.concatenate(parts).astype(np.int32)
    s = decode_scores_row(q, kbar)
    n = cand.size
    idx_c, lg, lse = gate_row(s[cand], n, Kb)
    idx = idx_c.copy()
    hist = (idx_c >= 0) & (idx_c < n)
    idx[hist] = cand[idx_c[hist]]
    idx[idx_c == n] = cur
    return idx, lg, lse, s, cand


def decode_row(q, K, V, sel_idx, sel_lg, Kb, scale, blk=64):
    """Decode attention of one row: (o float64 [G,d], lse float64 [G])."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    G, d = q.shape
    L = K.shape[0]
    o = np.empty((G, d))
    lse = np.empty(G)
    _load().sas_oracle_decode_row(
        L, blk, d, G, Kb, ctypes.c_double(scale), _p(q), _p(K), _p(V),
        _p(_i32(sel_idx)), _p(None if sel_lg is None else _f64(sel_lg)), _p(o), _p(lse))
    return o, lse
