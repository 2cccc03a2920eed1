"""Library-routine cross-checks for the oracle: torch's CPU scaled-dot-product
attention in float64 with an additive mask that carries the log gates.

The additive mask is what the gated formulation adds to the logits
(the page titled "SAS: Simple Attention Sparsification via End-to-End Optimization of Context Ranking Review", section 2-2: softmax(q K_S^T + log g_S) V_S):
log g of the key's block where the block is attended (causal inside the
current block), -inf elsewhere.  Building it is pure indexing; the attention
arithmetic is torch's.
"""
import numpy as np
import torch


def gate_mask(cu, sel_idx, sel_lg, hkv, blk, s):
    """[hkv][L][L] float64 additive mask for sequence s."""
    start, end = int(cu[s]), int(cu[s + 1])
    L = end - start
    nb = (L + blk - 1) // blk
    qb0 = sum((int(cu[x + 1]) - int(cu[x]) + blk - 1) // blk for x in range(s))
    QB = sel_idx.shape[1]
    M = np.full((hkv, L, L), -np.inf)
    for g in range(hkv):
        for i in range(nb):
            r = qb0 + i
            t0, t1 = i * blk, min((i + 1) * blk, L)
            for slot in range(sel_idx.shape[2]):
                j = int(sel_idx[g, r, slot])
                if j < 0:
                    continue
                u0, u1 = j * blk, min((j + 1) * blk, L)
                M[g, t0:t1, u0:u1] = sel_lg[g, r, slot]
        tri = np.triu(np.ones((L, L), bool), 1)
        M[g][tri] = -np.inf
    assert QB >= qb0 + nb
    return M


def sdpa_sequence(q, k, v, M, scale, dO=None):
    """Gated attention of one sequence through torch SDPA (float64, CPU).

    q [L,hq,d], k/v [L,hkv,d], M [hkv,L,L].  Returns o [L,hq,d], lse [hq,L]
    and, when dO is given, (dq, dk, dv, dM) from autograd of sum(dO * o).
    """
    L, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    qt = torch.tensor(np.asarray(q, np.float64)).permute(1, 0, 2).contiguous().requires_grad_(True)
    kt = torch.tensor(np.asarray(k, np.float64)).permute(1, 0, 2).contiguous().requires_grad_(True)
    vt = torch.tensor(np.asarray(v, np.float64)).permute(1, 0, 2).contiguous().requires_grad_(True)
    Mt = torch.tensor(M).requires_grad_(True)
    ke = kt.repeat_interleave(G, 0)
    ve = vt.repeat_interleave(G, 0)
    Me = Mt.repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(0), ke.unsqueeze(0), ve.unsqueeze(0), attn_mask=Me.unsqueeze(0),
        scale=scale)[0]
    logits = torch.matmul(qt, ke.transpose(1, 2)) * scale + Me
    lse = torch.logsumexp(logits, dim=-1)
    out = {"o": o.permute(1, 0, 2).detach().numpy(), "lse": lse.detach().numpy()}
    if dO is not None:
        dOt = torch.tensor(np.asarray(dO, np.float64)).permute(1, 0, 2)
        (o * dOt).sum().backward()
        out["dq"] = qt.grad.permute(1, 0, 2).numpy()
        out["dk"] = kt.grad.permute(1, 0, 2).numpy()
        out["dv"] = vt.grad.permute(1, 0, 2).numpy()
        dM = Mt.grad.numpy().copy()
        dM[~np.isfinite(M)] = 0.0
        out["dM"] = dM
    return out


def dlg_from_mask_grad(dM, cu, sel_idx, hkv, blk, s):
    """Sum the mask gradient over each (row, kept block) tile -> [hkv][nb][Kb]."""
    start, end = int(cu[s]), int(cu[s + 1])
    L = end - start
    nb = (L + blk - 1) // blk
    qb0 = sum((int(cu[x + 1]) - int(cu[x]) + blk - 1) // blk for x in range(s))
    Kb = sel_idx.shape[2]
    out = np.zeros((hkv, nb, Kb))
    for g in range(hkv):
        for i in range(nb):
            t0, t1 = i * blk, min((i + 1) * blk, L)
            for slot in range(Kb):
                j = int(sel_idx[g, qb0 + i, slot])
                if j < 0:
                    continue
                u0, u1 = j * blk, min((j + 1) * blk, L)
                out[g, i, slot] = dM[g, t0:t1, u0:u1].sum()
    return out
