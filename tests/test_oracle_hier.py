"""Pins of the oracle's hierarchical (coarse-to-fine) decode selection
(review, section 7-2: a coarse retrieval narrows the candidate blocks, the
selector's Top-K then picks among them).

The pins: with every super-block kept the selection is the exact one; the
super-block summaries are exact means on integer inputs; on dyadic inputs
(every score exact in fp32, ties frequent) the whole selection equals a
float64 brute force that sorts coarse and fine scores with the tie rule;
a block outside the kept super-blocks is never selected, however high its
own score.
"""
import numpy as np
import pytest

import oracle

F = oracle.COARSE_BLOCKS


def _rand(L, d, G, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((G, d)).astype(np.float32),
            rng.standard_normal((L, d)).astype(np.float32))


@pytest.mark.parametrize("summary", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("L", [64 * 9 + 1, 64 * 77 + 30, 64 * 200 + 64])
def test_hier_equals_exact_when_every_super_block_is_kept(L, summary):
    q, K = _rand(L, 64, 4, L)
    nsup = ((L - 1) // 64) // F
    want = oracle.decode_select_row(q, K, 6, summary=summary)
    got = oracle.decode_select_row_hier(q, K, 6, max(nsup, 1), summary=summary)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    assert got[2] == want[2]
    assert np.array_equal(got[4], np.arange((L - 1) // 64))


def test_coarse_summaries_are_exact_means_on_integer_inputs():
    rng = np.random.default_rng(3)
    kbar = rng.integers(-50, 50, (8 * 13 + 5, 32)).astype(np.float32)
    c = oracle.coarse_summaries_row(kbar)
    assert c.shape == (13, 32)
    want = kbar[:8 * 13].astype(np.float64).reshape(13, 8, 32).mean(axis=1)
    assert np.array_equal(c.astype(np.float64), want)


def _brute(q, K, Kb, C):
    """float64 brute force; exact on dyadic inputs (d = 64, G = 4)."""
    L, d = K.shape
    nhist = (L - 1) // 64
    qbar = q.astype(np.float64).mean(axis=0)
    kbar = K[:64 * nhist].astype(np.float64).reshape(nhist, 64, d).mean(axis=1)
    nsup = nhist // F
    cbar = kbar[:F * nsup].reshape(nsup, F, d).mean(axis=1)
    S = cbar @ qbar / np.sqrt(d)
    kept = sorted(sorted(range(nsup), key=lambda J: (-S[J], J))[:C])
    cand = [F * J + b for J in kept for b in range(F)] + list(range(F * nsup, nhist))
    s = kbar @ qbar / np.sqrt(d)
    top = sorted(sorted(cand, key=lambda j: (-s[j], j))[:min(Kb - 1, len(cand))])
    lse = np.log(np.sum(np.exp(s[cand]))) if cand else -np.inf
    return top, [s[j] - lse for j in top], lse, cand


@pytest.mark.parametrize("seed", range(6))
def test_hier_matches_brute_force_on_dyadic_inputs(seed):
    rng = np.random.default_rng(100 + seed)
    L = 64 * int(rng.integers(20, 120)) + int(rng.integers(1, 64))
    # small integers: block means, super-block means, the mean query and every
    # product and partial sum are exact in fp32; many scores tie
    K = rng.integers(-2, 3, (L, 64)).astype(np.float32)
    q = rng.integers(-3, 4, (4, 64)).astype(np.float32)
    Kb, C = int(rng.integers(2, 12)), int(rng.integers(1, 6))
    idx, lg, lse, s, cand = oracle.decode_select_row_hier(q, K, Kb, C)
    top, tlg, tlse, tcand = _brute(q, K, Kb, C)
    cur = (L - 1) // 64
    assert list(cand) == tcand
    k = len(top)
    assert list(idx[:k]) == top and idx[k] == cur and np.all(idx[k + 1:] == -1)
    assert abs(lse - tlse) < 1e-9
    assert np.allclose(lg[:k], tlg, rtol=0, atol=1e-9) and lg[k] == 0.0


def test_block_outside_the_kept_super_blocks_is_never_selected():
    d, G = 64, 4
    nhist = 3 * F + 2  # three super-blocks and two trailing blocks
    L = 64 * nhist + 1
    q = np.ones((G, d), np.float32)
    K = np.zeros((L, d), np.float32)

    def blk(j, v):
        K[64 * j:64 * j + 64] = v

    for j in range(nhist):
        blk(j, 0.1)
    blk(3, 5.0)                # the best single block, in super-block 0 ...
    for j in (0, 1, 2, 4, 5, 6, 7):
        blk(j, -2.0)           # ... whose mean is the lowest
    for j in range(F, 2 * F):
        blk(j, 0.5)            # super-block 1: the best mean
    exact = oracle.decode_select_row(q, K, 4)
    assert 3 in exact[0]
    idx, lg, lse, s, cand = oracle.decode_select_row_hier(q, K, 4, 1)
    assert list(cand) == list(range(F, 2 * F)) + [3 * F, 3 * F + 1]
    assert 3 not in idx and set(idx[:3]) <= set(cand)
