"""Pins for the oracle's gate backward and decode path (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle

H = 2.0 ** -12  # logits live on a 2^-12 grid, so s +- H is exact in fp32


def grid_logits(shape, seed, sigma=2.0):
    g = np.random.default_rng(seed)
    x = np.clip(g.normal(0, sigma, shape), -7.5, 7.5)
    return (np.round(x / H) * H).astype(np.float32)


@pytest.mark.parametrize("mode", [oracle.GATE_HIST, oracle.GATE_ALL, oracle.GATE_SIGMOID,
                                  oracle.GATE_RAW])
def test_gate_bwd_matches_finite_differences(mode):
    blk, hkv, Kb = 4, 2, 3
    lengths = [30, 13]
    cu = np.array([0, 30, 43], np.int32)
    QB = 8 + 4
    lg = grid_logits((hkv, QB, 8), 1)
    idx, sl, _ = oracle.gate_topk(cu, lg, hkv, Kb, mode, blk=blk)
    W = np.random.default_rng(2).normal(size=idx.shape)
    W[idx < 0] = 0.0
    fin = np.isfinite(sl)
    d_logits = oracle.gate_bwd(cu, lg, idx, W, hkv, Kb, mode, blk=blk)

    def L(x):
        i2, s2, _ = oracle.gate_topk(cu, x, hkv, Kb, mode, blk=blk)
        assert np.array_equal(i2, idx)  # the selection must not move
        return float(np.sum(np.where(fin, W * np.where(fin, s2, 0.0), 0.0)))

    rows = []
    for s in range(2):
        nb = (lengths[s] + blk - 1) // blk
        rows += [(s, i) for i in range(nb)]
    for g in range(hkv):
        for Q, (s, i) in enumerate(rows):
            ncols = i + 1 if mode == oracle.GATE_ALL else i
            kept = set(int(j) for j in idx[g, Q] if 0 <= j < i)
            for m in range(8):
                xp, xm = lg.copy(), lg.copy()
                xp[g, Q, m] += np.float32(H)
                xm[g, Q, m] -= np.float32(H)
                fd = (L(xp) - L(xm)) / (2 * H)
                assert abs(fd - d_logits[g, Q, m]) < 2e-6, (g, Q, m, fd, d_logits[g, Q, m])
                if m >= ncols:
                    assert d_logits[g, Q, m] == 0.0
                if mode in (oracle.GATE_SIGMOID, oracle.GATE_RAW) and m not in kept:
                    assert d_logits[g, Q, m] == 0.0  # independent gates: kept blocks only
    if mode in (oracle.GATE_HIST, oracle.GATE_ALL):
        # shift invariance of the gate => the gradient of every row sums to zero
        assert np.max(np.abs(d_logits.sum(-1))) < 1e-12


def test_end_to_end_logit_gradient_through_attention():
    """d loss / d logits through gate -> gated attention: oracle bwd (dlg)
    followed by gate bwd, against finite differences of the whole chain."""
    blk, hq, hkv, d, Kb = 4, 2, 1, 4, 3
    T = 24
    cu = np.array([0, T], np.int32)
    g = np.random.default_rng(5)
    q, k, v, dO = (g.normal(size=(T, n, d)) for n in (hq, hkv, hkv, hq))
    lg = grid_logits((hkv, 6, 6), 7)
    scale = 1.0 / math.sqrt(d)
    idx, sl, _ = oracle.gate_topk(cu, lg, hkv, Kb, blk=blk)
    _, _, _, dlg = oracle.bwd(cu, q, k, v, dO, idx, sl, Kb, scale, blk=blk)
    dz = oracle.gate_bwd(cu, lg, idx, dlg, hkv, Kb, blk=blk)

    def L(x):
        i2, s2, _ = oracle.gate_topk(cu, x, hkv, Kb, blk=blk)
        assert np.array_equal(i2, idx)
        o, _ = oracle.fwd(cu, q, k, v, i2, s2, Kb, scale, blk=blk)
        return float(np.sum(o * dO))

    for Q in range(6):
        for m in range(Q):
            xp, xm = lg.copy(), lg.copy()
            xp[0, Q, m] += np.float32(H)
            xm[0, Q, m] -= np.float32(H)
            fd = (L(xp) - L(xm)) / (2 * H)
            assert abs(fd - dz[0, Q, m]) < 1e-6 * max(1, abs(fd)), (Q, m, fd, dz[0, Q, m])


def test_pooled_summaries_are_exact_means_on_integer_keys():
    g = np.random.default_rng(0)
    K = g.integers(-8, 9, (64 * 5 + 17, 16)).astype(np.float32)
    kbar = oracle.pool_keys_row(K)
    assert kbar.shape == (5, 16)
    want = K[:320].reshape(5, 64, 16).astype(np.float64).mean(1)
    assert np.array_equal(kbar.astype(np.float64), want)


def test_pooled_summaries_within_sequential_sum_bound():
    g = np.random.default_rng(1)
    K = g.normal(size=(64 * 9, 32)).astype(np.float32)
    kbar = oracle.pool_keys_row(K)[:8]
    blocks = K[:512].reshape(8, 64, 32).astype(np.float64)
    exact = blocks.mean(1)
    bound = 64 * 2.0 ** -24 * np.abs(blocks).sum(1) / 64 + 2.0 ** -24 * np.abs(exact)
    assert np.all(np.abs(kbar - exact) <= bound)


def test_pooled_scores_exact_on_dyadic_inputs_and_bounded_otherwise():
    g = np.random.default_rng(2)
    d, G = 64, 4
    # dyadic values with few bits: every fp32 step is exact, sqrt(64) = 8
    q = g.integers(-4, 5, (G, d)).astype(np.float32)
    kbar = (g.integers(-16, 17, (10, d)) / 64.0).astype(np.float32)
    s = oracle.decode_scores_row(q, kbar)
    qbar = q.astype(np.float64).sum(0) / G
    exact = (kbar.astype(np.float64) @ qbar) / 8.0
    assert np.array_equal(s.astype(np.float64), exact)
    # random values: within the fp32 dot-product error bound of the exact score
    q = g.normal(size=(G, 128)).astype(np.float32)
    kbar = g.normal(size=(50, 128)).astype(np.float32) / 8
    s = oracle.decode_scores_row(q, kbar).astype(np.float64)
    qbar64 = q.astype(np.float64).sum(0) / G
    exact = (kbar.astype(np.float64) @ qbar64) / math.sqrt(128)
    u = 2.0 ** -24
    mag = (np.abs(kbar.astype(np.float64)) @ (np.abs(q.astype(np.float64)).sum(0) / G))
    bound = (128 + G + 4) * u * mag / math.sqrt(128) + 4 * u * np.abs(exact)
    assert np.all(np.abs(s - exact) <= bound)


@pytest.mark.parametrize("L", [64 * 20 + 1, 64 * 21, 64 * 7 + 33, 65])
def test_decode_row_equals_forward_last_token(L):
    """The decode path on the newest token equals the training forward's row
    for the same selection and gates (review section 3-7)."""
    G, d, Kb = 4, 16, 5
    g = np.random.default_rng(L)
    q_all = g.normal(size=(L, G, d))
    K = g.normal(size=(L, d)).astype(np.float32)
    V = g.normal(size=(L, d))
    qlast = q_all[-1].astype(np.float32)
    idx, sl, lse_gate, _ = oracle.decode_select_row(qlast, K, Kb)
    cur = (L - 1) // 64
    assert idx[min(Kb - 1, cur)] == cur
    o, lse = oracle.decode_row(qlast, K, V, idx, sl, Kb, 0.25)
    nb = cur + 1
    sel_all = np.full((1, nb, Kb), -1, np.int32)
    lg_all = np.full((1, nb, Kb), -np.inf)
    sel_all[0, cur], lg_all[0, cur] = idx, sl
    for i in range(cur):
        sel_all[0, i, 0], lg_all[0, i, 0] = i, 0.0
    q_all[-1] = qlast
    rm = np.zeros((1, nb), np.uint8)
    rm[0, cur] = 1
    of, lf = oracle.fwd(np.array([0, L], np.int32), q_all, K[:, None].astype(np.float64),
                        V[:, None], sel_all, lg_all, Kb, 0.25, row_mask=rm)
    assert np.max(np.abs(of[-1] - o)) < 1e-12
    assert np.max(np.abs(lf[:, -1] - lse)) < 1e-12


def test_decode_all_blocks_ungated_is_dense_single_query_attention():
    G, d, L = 4, 32, 64 * 6 + 10
    g = np.random.default_rng(3)
    q = g.normal(size=(G, d))
    K = g.normal(size=(L, d))
    V = g.normal(size=(L, d))
    idx = np.array(list(range(7)) + [-1], np.int32)
    o, lse = oracle.decode_row(q, K, V, idx, None, 8, 1 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, None], torch.tensor(K)[None].expand(G, L, d),
        torch.tensor(V)[None].expand(G, L, d), scale=1 / math.sqrt(d))[:, 0]
    assert np.max(np.abs(o - ref.numpy())) < 1e-12


def test_ste_gate_matches_torch_straight_through_autograd():
    """The ranking-preservation ablation (paper text section 4): hard Top-K
    gates in the forward, the soft softmax gate's gradient in the backward.
    The oracle's gate backward against torch autograd of
    g = g_hard + g_soft - g_soft.detach() (float64), with dL/dg = the given
    d log g on the kept history blocks (the hard gate is 1)."""
    blk, hkv, Kb = 4, 2, 3
    lengths = [30, 13]
    cu = np.array([0, 30, 43], np.int32)
    QB = 8 + 4
    lg = grid_logits((hkv, QB, 8), 5)
    idx, sl, glse = oracle.gate_topk(cu, lg, hkv, Kb, oracle.GATE_STE, blk=blk)
    W = np.random.default_rng(6).normal(size=idx.shape)
    W[idx < 0] = 0.0
    d_logits = oracle.gate_bwd(cu, lg, idx, W, hkv, Kb, oracle.GATE_STE, blk=blk)
    rows = []
    for s in range(2):
        nb = (lengths[s] + blk - 1) // blk
        rows += [(s, i) for i in range(nb)]
    for g in range(hkv):
        for Q, (s, i) in enumerate(rows):
            k = min(Kb - 1, i)
            # forward: hard gate 1 on every kept block, the soft normaliser in gate_lse
            assert np.all(sl[g, Q, :k + 1] == 0.0)
            if i > 0:
                assert glse[g, Q] == pytest.approx(
                    float(torch.logsumexp(torch.tensor(lg[g, Q, :i], dtype=torch.float64), 0)),
                    abs=1e-12)
            x = torch.tensor(lg[g, Q, :8], dtype=torch.float64, requires_grad=True)
            loss = torch.zeros((), dtype=torch.float64)
            if i > 0:
                soft = torch.softmax(x[:i], 0)
                for slot in range(k):
                    j = int(idx[g, Q, slot])
                    gste = 1.0 + soft[j] - soft[j].detach()
                    loss = loss + float(W[g, Q, slot]) * gste
            if loss.requires_grad:
                loss.backward()
                want = x.grad.numpy()
            else:
                want = np.zeros(8)
            assert np.max(np.abs(d_logits[g, Q] - want)) < 1e-12, (g, Q)


def test_bf16_summary_rounding_matches_torch_conversion():
    """The oracle's bf16 summary storage is round-to-nearest-even: the same
    values as torch's fp32 -> bf16 conversion, on random values, exact
    halfway cases (which must go to the even neighbour), signed zeros,
    infinities, overflow and subnormals."""
    import torch
    g = np.random.default_rng(3)
    x = np.concatenate([
        g.standard_normal(4096).astype(np.float32) * np.float32(3.0),
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-9, 0.0, -0.0, np.inf, -np.inf,
                  3.3961e38, 1e-40, -1e-41, 2**-126], np.float32)])
    got = oracle.round_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # the ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to 1
    assert got[4096] == 1.0 and got[4097] == np.float32(1 + 2**-6)


def test_bf16_summaries_are_the_rounded_fp32_means():
    g = np.random.default_rng(4)
    K = g.standard_normal((64 * 5 + 7, 32)).astype(np.float32)
    f32 = oracle.pool_keys_row(K)
    b16 = oracle.pool_keys_row(K, summary="bf16")
    assert b16.shape == f32.shape == (5, 32)
    assert np.array_equal(b16, oracle.round_bf16(f32))
    assert np.max(np.abs(b16 - f32)) <= np.max(np.abs(f32)) * 2.0 ** -8
    q = g.standard_normal((4, 32)).astype(np.float32)
    idx, lg, lse, s = oracle.decode_select_row(q, K, 3, summary="bf16")
    assert np.array_equal(s, oracle.decode_scores_row(q, b16))


def _e4m3_values():
    """Every finite fp8 e4m3 value, from its bit fields (sign, 4-bit
    exponent with bias 7, 3-bit mantissa; 0x7f / 0xff are NaN)."""
    vals = []
    for code in range(256):
        sgn, ef, m = code >> 7, (code >> 3) & 15, code & 7
        if ef == 15 and m == 7:
            continue
        v = m * 2.0 ** -9 if ef == 0 else (8 + m) * 2.0 ** (ef - 10)
        vals.append(-v if sgn else v)
    return np.array(sorted(set(vals)), np.float64)


def test_e4m3_summary_rounding_matches_torch_conversion():
    """The oracle's fp8 summary storage rounds to nearest, ties to even, with
    no saturation: the same values as torch's fp32 -> float8_e4m3fn
    conversion, on random values over the whole range, every e4m3 value,
    every midpoint between neighbours (ties), the overflow boundary,
    subnormals, signed zeros, infinities and NaN."""
    import torch
    g = np.random.default_rng(11)
    v = _e4m3_values()
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    x = np.concatenate([
        g.standard_normal(8192).astype(np.float32) * np.float32(0.125),
        (g.standard_normal(4096) * 100).astype(np.float32),
        v.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
        np.nextafter(mids, np.float32(-np.inf)),
        np.array([448, 464, 472, 479.9, 480, 1e4, -464, -480, 2**-9, 2**-10, 3 * 2**-11, 2**-11,
                  0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)])
    got = oracle.round_e4m3(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    # e4m3 values are fixed points; 464 (halfway to the NaN pattern) goes to
    # 448; the half-spacing subnormal 2^-10 goes to 0 (even)
    assert np.array_equal(oracle.round_e4m3(v.astype(np.float32)), v.astype(np.float32))
    r = oracle.round_e4m3(np.array([464, 480, 2**-10, 3 * 2**-10], np.float32))
    assert r[0] == 448 and np.isnan(r[1]) and r[2] == 0.0 and r[3] == 2**-8


def test_fp8_summaries_are_the_rounded_fp32_means():
    g = np.random.default_rng(12)
    K = g.standard_normal((64 * 5 + 7, 32)).astype(np.float32)
    f32 = oracle.pool_keys_row(K)
    f8 = oracle.pool_keys_row(K, summary="fp8")
    assert f8.shape == f32.shape == (5, 32)
    assert np.array_equal(f8, oracle.round_e4m3(f32))
    # relative error of e4m3 is at most 2^-4 for normal values, and the
    # absolute error at most 2^-10 in the subnormal range
    assert np.all(np.abs(f8 - f32) <= np.maximum(np.abs(f32) * 2.0 ** -4, 2.0 ** -10))
    q = g.standard_normal((4, 32)).astype(np.float32)
    idx, lg, lse, s = oracle.decode_select_row(q, K, 3, summary="fp8")
    assert np.array_equal(s, oracle.decode_scores_row(q, f8))
