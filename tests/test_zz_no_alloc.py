"""sas_decode_noalloc (the decode entry point that takes no workspace and
allocates nothing) against sas_decode, through the C ABI.

Both run the same kernels with the same split, so the outputs must be the
same bits; they are also held to the oracle at the bf16 bar.  Two calls in a
row, the second on a smaller problem, so the second finds the first call's
partials in the shared scratch and must not depend on them.
"""
import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, dev_tensor, say
from trainable_block_sparse_gate_amd import sas
from trainable_block_sparse_gate_amd import workloads as wl


def _case(seqlens, hq, hkv, d, Kb, paged, seed, num_splits=0):
    import torch
    say(f"[noalloc] seqlens {seqlens} heads {hq}/{hkv} d {d} Kb {Kb} paged {paged} "
        f"num_splits {num_splits}")
    host = wl.draw_decode_host_small(seqlens, hq, hkv, d, Kb, paged, seed=seed)
    npages = host["k"].shape[0] if paged else 0
    prob = sas.Decode(seqlens, hq, hkv, d, Kb, paged, max(seqlens),
                      page_table=host["page_table"], num_pages=npages, out_dtype="f32",
                      num_splits=num_splits)
    q = dev_tensor(host["q"], host["q_bits"], "bf16")
    kc = dev_tensor(host["k"], host["k_bits"], "bf16")
    vc = dev_tensor(host["v"], host["v_bits"], "bf16")
    ksum = sas.pool_keys(prob, kc)
    sel, lg, _, _ = sas.decode_select(prob, q, ksum)
    o_ref, lse_ref = sas.decode(prob, q, kc, vc, sel, lg)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    sas.decode_noalloc(prob, q, kc, vc, sel, lg, out=(o, lse))
    torch.cuda.synchronize()
    o_h, lse_h = o.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(o_h, o_ref.cpu().numpy()), "o differs from sas_decode"
    assert np.array_equal(lse_h, lse_ref.cpu().numpy()), "lse differs from sas_decode"
    G = hq // hkv
    sel_h, lg_h = sel.cpu().numpy(), lg.cpu().numpy().astype(np.float64)
    for b, L in enumerate(seqlens):
        for g in range(hkv):
            K = wl.gather_row_cache(host["k"], host["page_table"], b, g, L)
            V = wl.gather_row_cache(host["v"], host["page_table"], b, g, L)
            qg = host["q"][b, g * G:(g + 1) * G]
            ro, rl = oracle.decode_row(qg, K, V, sel_h[b * hkv + g], lg_h[b * hkv + g], Kb,
                                       prob.scale)
            assert np.max(np.abs(o_h[b, g * G:(g + 1) * G] - ro)) <= TOL["bf16"]
            assert np.max(np.abs(lse_h[b, g * G:(g + 1) * G] - rl)) <= 1e-4
    say("  same bits as sas_decode; oracle bar met")


@pytest.mark.gpu
def test_noalloc_decode_matches_decode_on_two_calls():
    # first: 3 sequences x 2 kv heads, 64 kept blocks -> split rows (scratch used)
    _case([64 * 70 + 3, 64 * 40, 900], 8, 2, 128, 64, True, seed=81)
    # second, smaller: one sequence; its partials land over the first call's
    _case([64 * 30 + 17], 8, 2, 128, 32, False, seed=82)
    # a forced split count, and head_dim 64
    _case([2000, 1500], 4, 2, 64, 16, True, seed=83, num_splits=3)


def test_noalloc_rejects_partials_beyond_the_scratch():
    """Host check, before any launch: batch 32 x 8 kv heads, 64 forced splits
    of 4 query heads x (128 + 2) floats = 34 MB of partials > 4 MiB."""
    lib = sas.lib()
    FAKE = 0x10000
    sl = np.full(32, 64 * 100, np.int32)
    p = sas.DecodeProblem(32, 32, 8, 128, 64, 64, 0, 0, 0, 64 * 100, 0, 0, 128,
                          1.0 / np.sqrt(128), FAKE, sl.ctypes.data, None, 0, None, 64)
    assert lib.sas_decode_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None) == -6
    assert b"scratch" in lib.sas_last_error()
