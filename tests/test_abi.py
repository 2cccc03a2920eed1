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
    assert lib.sas_abi_version() == sas.ABI_VERSION == 2
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
                   nblk=None, max_seqlen=None, G_override=None):
    sl = np.array(seqlens, np.int32)
    mp = max_pages if max_pages is not None else (max(seqlens) + 63) // 64
    nb = nblk if nblk is not None else max(1, (max(seqlens) - 1) // 64)
    p = sas.DecodeProblem(len(seqlens), hq, hkv, d, 64, Kb, 0, 0, 1 if paged else 0,
                          max_seqlen if max_seqlen is not None else max(seqlens), mp, 32, nb,
                          1.0 / np.sqrt(d), FAKE, sl.ctypes.data, FAKE if paged else None)
    p._keep = sl
    return p


def test_decode_checks(lib):
    ws = [FAKE, 1 << 20]
    good = decode_problem()
    assert lib.sas_decode_workspace_size(ctypes.byref(good)) > 0
    bad = [decode_problem(hq=6, hkv=2),          # group of 3 heads
           decode_problem(max_pages=5),          # page table too short for 700 tokens
           decode_problem(nblk=3),               # summary stride too short
           decode_problem(paged=False, max_seqlen=600)]
    want = [-5, -2, -2, -2]
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
