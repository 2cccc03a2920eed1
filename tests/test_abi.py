"""The C-ABI library on the host (no GPU): it loads, exports every entry
point include/sas.h declares, and rejects bad arguments with the documented
status before launching anything (so these calls never reach a device)."""
import ctypes
import os
import re

import numpy as np
import pytest

from trainable_block_sparse_gate_amd import sas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")

FAKE = 0x10000  # a 16-byte-aligned stand-in for a device pointer (never touched)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sas.LIB_PATH):
        from trainable_block_sparse_gate_amd import build
        build.build()
    return sas.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sas.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert lib.sas_abi_version() == sas.ABI_VERSION == 6
    assert lib.sas_status_string(0) == b"ok"
    assert b"unsupported" in lib.sas_status_string(-5)


def problem(lengths=(200, 64), hq=8, hkv=2, d=128, Kb=4, dtype=0, out=0, block=64,
            bad_cuq=False):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    nb = [(n + 63) // 64 for n in lengths]
    cuq = np.concatenate([[0], np.cumsum(nb)]).astype(np.int32)
    if bad_cuq:
        cuq[-1] += 1
    p = sas.Problem(len(lengths), int(cu[-1]), int(cuq[-1]), hq, hkv, d, block, Kb, dtype, out,
                    1.0 / np.sqrt(d), FAKE, FAKE, cu.ctypes.data, cuq.ctypes.data)
    p._keep = (cu, cuq)
    return p


def call_fwd(lib, p, q=FAKE):
    return lib.sas_fwd(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(d=96), -5), (dict(block=32), -5), (dict(hq=6, hkv=4), -2), (dict(Kb=0), -5),
    (dict(Kb=300), -5), (dict(dtype=7), -3), (dict(dtype=1, out=0), -5), (dict(bad_cuq=True), -2),
    (dict(hq=16384, hkv=16384), -5),  # hq * head_dim above 2^20
])
def test_fwd_rejects_bad_problems(lib, kwargs, status):
    assert call_fwd(lib, problem(**kwargs)) == status
    assert lib.sas_last_error() != b""


def test_null_and_alignment_checks(lib):
    assert lib.sas_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert call_fwd(lib, problem(), q=None) == -1
    assert call_fwd(lib, problem(), q=FAKE + 2) == -4
    assert b"aligned" in lib.sas_last_error()


def test_gate_topk_checks(lib):
    p = problem(lengths=(640,))
    # ld smaller than the 10 blocks of the sequence
    assert lib.sas_gate_topk(ctypes.byref(p), FAKE, 9, 0, FAKE, FAKE, FAKE, None) == -2
    assert lib.sas_gate_topk(ctypes.byref(p), FAKE, 10, 5, FAKE, FAKE, FAKE, None) == -2
    assert lib.sas_gate_topk(ctypes.byref(p), None, 10, 0, FAKE, FAKE, FAKE, None) == -1


def test_bwd_workspace_checks(lib):
    p = problem()
    need = lib.sas_bwd_workspace_size(ctypes.byref(p))
    assert need > 0
    args = [FAKE] * 12
    assert lib.sas_bwd(ctypes.byref(p), *args, None, need, None) == -6
    assert lib.sas_bwd(ctypes.byref(p), *args, FAKE, need - 1, None) == -6
    for fn, n in (("sas_bwd_prepare", 1), ("sas_bwd_dq", 10), ("sas_bwd_dkdv", 8)):
        f = getattr(lib, fn)
        assert f(ctypes.byref(p), *([FAKE] * n), FAKE, 16, None) == -6, fn
    # an invalid problem has no workspace size
    assert lib.sas_bwd_workspace_size(ctypes.byref(problem(d=96))) == 0


def decode_problem(seqlens=(700, 129), hq=8, hkv=2, d=128, Kb=4, paged=True, max_pages=None,
                   nblk=None, max_seqlen=None, page_table_host=None, num_splits=0,
                   num_pages=32):
    sl = np.array(seqlens, np.int32)
    mp = max_pages if max_pages is not None else (max(seqlens) + 63) // 64
    nb = nblk if nblk is not None else -(-max(1, (max(seqlens) - 1) // 64) // 64) * 64
    pth = None if page_table_host is None else np.ascontiguousarray(page_table_host, np.int32)
    p = sas.DecodeProblem(len(seqlens), hq, hkv, d, 64, Kb, 0, 0, 1 if paged else 0,
                          max_seqlen if max_seqlen is not None else max(seqlens), mp, num_pages,
                          nb, 1.0 / np.sqrt(d), FAKE, sl.ctypes.data, FAKE if paged else None, 0,
                          None if pth is None else pth.ctypes.data, num_splits)
    p._keep = (sl, pth)
    return p


def test_decode_checks(lib):
    ws = [FAKE, 1 << 20]
    good = decode_problem()
    assert lib.sas_decode_workspace_size(ctypes.byref(good)) > 0
    bad = [decode_problem(hq=6, hkv=2),          # group of 3 heads
           decode_problem(max_pages=5),          # page table too short for 700 tokens
           decode_problem(nblk=3),               # summary stride too short
           decode_problem(nblk=70),              # not whole 64-block summary tiles
           decode_problem(paged=False, max_seqlen=600)]
    want = [-5, -2, -2, -2, -2]
    for p, w in zip(bad, want):
        assert lib.sas_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, *ws,
                              None) == w
    p = decode_problem()
    p.page_table = None
    assert lib.sas_pool_keys(ctypes.byref(p), FAKE, FAKE, None) == -1
    assert lib.sas_decode(ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                          None) == -6


def test_binding_raises_on_rejected_calls(lib):
    with pytest.raises(sas.SasError) as e:
        sas._check(lib.sas_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None))
    assert e.value.status == -1
    assert "problem is NULL" in str(e.value)


def test_decode_page_table_host_checked(lib):
    """With a host copy of the page table, every page a sequence uses must
    lie in [0, num_pages); unused entries (past a sequence's pages) are free."""
    ws = [FAKE, 1 << 20]
    seqlens = (700, 129)  # 11 and 3 pages
    table = np.full((2, 11), -1, np.int32)
    table[0, :11] = np.arange(11)
    table[1, :3] = [11, 12, 13]
    good = decode_problem(seqlens, page_table_host=table, num_pages=14)
    assert lib.sas_decode_workspace_size(ctypes.byref(good)) > 0
    for b, c, val in ((0, 4, 14), (1, 2, -1), (0, 10, 1 << 20)):
        bad_table = table.copy()
        bad_table[b, c] = val
        p = decode_problem(seqlens, page_table_host=bad_table, num_pages=14)
        assert lib.sas_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, *ws,
                              None) == -2
        assert b"page_table" in lib.sas_last_error()
        assert lib.sas_decode_append(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                     None) == -2
        assert lib.sas_pool_keys(ctypes.byref(p), FAKE, FAKE, None) == -2


def test_decode_num_splits_checked_and_sized(lib):
    """num_splits in [0, budget_blocks]; the workspace follows the split."""
    sizes = {}
    for n in (0, 1, 2, 4, 64):
        p = decode_problem(Kb=64, num_splits=n)
        sizes[n] = lib.sas_decode_workspace_size(ctypes.byref(p))
    rows_g_d = 2 * 2 * 4 * (128 + 2) * 4  # (batch x hkv) x G x (d + 2) fp32
    assert sizes[1] == rows_g_d and sizes[2] == 2 * rows_g_d and sizes[64] == 64 * rows_g_d
    assert sizes[0] == 16 * rows_g_d  # automatic: at most ceil(64 / 4) splits
    for n in (-1, 65):
        p = decode_problem(Kb=64, num_splits=n)
        assert lib.sas_decode_workspace_size(ctypes.byref(p)) == 0
        assert lib.sas_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              1 << 30, None) == -2


def test_binding_checks_tensors_before_calling():
    """The binding checks dtype, shape and contiguity of every tensor
    against the problem before the library sees a pointer (CPU tensors: the
    device check comes last, so each earlier mistake is what is reported)."""
    import torch
    prob = sas.Varlen([200, 64], 8, 2, 128, 4, device="cpu")
    T, QB = prob.T, prob.QB
    bf = torch.bfloat16
    q = torch.zeros(T, 8, 128, dtype=bf)
    k = torch.zeros(T, 2, 128, dtype=bf)
    sel = torch.zeros(2, QB, 4, dtype=torch.int32)
    lg = torch.zeros(2, QB, 4)
    cases = [
        (lambda: sas.gate_topk(prob, torch.zeros(2, QB, 4, dtype=bf)), -3),  # bf16 logits
        (lambda: sas.gate_topk(prob, torch.zeros(2, QB, 3)), -2),  # row shorter than 4 blocks
        (lambda: sas.gate_topk(prob, torch.zeros(2, QB + 1, 4)), -2),
        (lambda: sas.gate_topk(prob, torch.zeros(2, QB, 4)), -2),  # CPU tensor
        (lambda: sas.fwd(prob, q.float(), k, k, sel, lg), -3),
        (lambda: sas.fwd(prob, q, k[:T - 1], k, sel, lg), -2),
        (lambda: sas.fwd(prob, q.transpose(0, 1).contiguous().transpose(0, 1), k, k, sel, lg),
         -2),  # not contiguous
        (lambda: sas.fwd(prob, q, k, k, sel.long(), lg), -3),
        (lambda: sas.fwd(prob, q, k, k, sel, lg[:, :, :3]), -2),
        (lambda: sas.fwd(prob, None, k, k, sel, lg), -1),
    ]
    for fn, status in cases:
        with pytest.raises(sas.SasError) as e:
            fn()
        assert e.value.status == status, (str(e.value), status)


def test_binding_checks_decode_tensors():
    import torch
    table = np.arange(14, dtype=np.int32).reshape(1, 14)
    prob = sas.Decode([700], 8, 2, 128, 4, True, 896, page_table=table, num_pages=14,
                      device="cpu")
    bf = torch.bfloat16
    with pytest.raises(sas.SasError) as e:
        sas.pool_keys(prob, torch.zeros(14, 2, 32, 128, dtype=bf))  # pages of 32 rows
    assert e.value.status == -2
    with pytest.raises(sas.SasError) as e:
        sas.pool_keys(prob, torch.zeros(14, 2, 64, 128))  # fp32 cache
    assert e.value.status == -3
    q = torch.zeros(1, 8, 128, dtype=bf)
    cache = torch.zeros(14, 2, 64, 128, dtype=bf)
    with pytest.raises(sas.SasError) as e:
        sas.decode(prob, q, cache, cache, torch.zeros(2, 5, dtype=torch.int32), None,
                   workspace=torch.zeros(16, dtype=torch.uint8))
    assert e.value.status == -2
    # summaries: the tiled layout [batch][hkv][tiles][pieces][64][channels per piece]
    ksum = torch.zeros(prob.summary_shape())
    assert prob.summary_shape() == (1, 2, 1, 32, 64, 4)
    with pytest.raises(sas.SasError) as e:
        sas.decode_select(prob, q, ksum.view(1, 2, 64, 128))  # block-major, not tiled
    assert e.value.status == -2
    with pytest.raises(sas.SasError) as e:
        sas.pool_coarse(prob, ksum.to(bf))  # bf16 summaries for an fp32 problem
    assert e.value.status == -3
    csum = torch.zeros(prob.coarse_shape())
    assert prob.coarse_shape() == (1, 2, 1, 32, 64, 4)
    with pytest.raises(sas.SasError) as e:
        sas.decode_select_hier(prob, q, ksum, csum[:, :1], 4)  # one kv head short
    assert e.value.status == -2
    with pytest.raises(sas.SasError) as e:
        sas.decode_append(prob, torch.zeros(1, 2, 128, dtype=bf), torch.zeros(1, 2, 128, dtype=bf),
                          cache, cache, ksum, csum.to(bf))
    assert e.value.status == -3


def test_decode_select_workspace_and_limits(lib):
    """The selection's workspace follows its chunking: more chunks for few
    long rows than for many short ones; too many candidates is unsupported;
    a short workspace is rejected before any launch."""
    ws = lib.sas_decode_select_workspace_size
    one_long = decode_problem(seqlens=(524288,), hq=32, hkv=8, Kb=32, paged=False)
    many = decode_problem(seqlens=(131072,) * 32, hq=32, hkv=8, Kb=64, paged=False)
    n_long = ws(ctypes.byref(one_long))
    n_many = ws(ctypes.byref(many))
    # one row of 8191 blocks over 8 kv heads: 32 chunks of 256 blocks, 31 candidates each
    assert n_long >= 8 * 32 * 31 * 8 + 8 * 32 * 8
    assert n_many >= 256 * 63 * 8  # at least one chunk per row
    assert lib.sas_decode_select(ctypes.byref(one_long), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 n_long - 1, None) == -6
    assert lib.sas_decode_select(ctypes.byref(one_long), FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, n_long, None) == -4  # summaries not 16-byte aligned
    huge = decode_problem(seqlens=(64 * 70000,), hq=8, hkv=2, Kb=256, paged=False)
    assert lib.sas_decode_select(ctypes.byref(huge), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 40, None) == -5
