"""torch.autograd bridge over the C ABI (argument marshalling only).

``forward`` runs the gate and hard Top-K on the selector's logits
(``sas_gate_topk``) and the gated block-sparse forward (``sas_fwd``);
``backward`` runs the fused backward (``sas_bwd``: dQ, dK, dV and the
per-block log-gate gradient) and the gate backward (``sas_gate_bwd``),
so the language-model loss reaches the selector's logits, and through
them whatever produced the logits: SAS trains its selector end to end by
putting the kept blocks' log gates inside the attention softmax (review
section 1, summary; p3's overview flowchart, where the loss flows back
through the gate to the selector).  The hard Top-K itself has no gradient:
the selected index set is a constant of the backward.

Every step runs in the library's HIP kernels; this module only calls the
binding in :mod:`trainable_block_sparse_gate_amd.sas`.
"""
import torch

from . import sas


class GatedBlockSparseAttention(torch.autograd.Function):
    """o = gated block-sparse attention(q, k, v; Top-K of gate(logits)).

    q [T, hq, d], k / v [T, hkv, d] in the problem's dtype; logits fp32
    [hkv, QB, ld] (column = key block of the row's own sequence; other
    dtypes or shapes raise SasError before anything runs).  Returns
    (o, sel_idx, sel_loggate); only o is differentiable.  Gradients come
    back in fp32, and torch casts them to each input's dtype.
    """

    @staticmethod
    def forward(ctx, q, k, v, logits, prob, mode=sas.GATE_HIST):
        q, k, v, logits = q.contiguous(), k.contiguous(), v.contiguous(), logits.contiguous()
        sel, lg, glse = sas.gate_topk(prob, logits, mode)
        o, lse = sas.fwd(prob, q, k, v, sel, lg)
        ctx.save_for_backward(q, k, v, o, lse, logits, sel, lg, glse)
        ctx.prob, ctx.mode = prob, mode
        ctx.mark_non_differentiable(sel, lg)
        return o, sel, lg

    @staticmethod
    def backward(ctx, dO, _dsel, _dlg):
        q, k, v, o, lse, logits, sel, lg, glse = ctx.saved_tensors
        prob = ctx.prob
        dO = dO.to(prob.torch_dtype("out")).contiguous()
        dq, dk, dv, dlg = sas.bwd(prob, q, k, v, o, dO, lse, sel, lg)
        dlogits = sas.gate_bwd(prob, logits, sel, glse, dlg, ctx.mode)
        return dq, dk, dv, dlogits, None, None


def gated_block_sparse_attention(q, k, v, logits, prob, mode=sas.GATE_HIST):
    """Functional form: returns o (see :class:`GatedBlockSparseAttention`)."""
    return GatedBlockSparseAttention.apply(q, k, v, logits, prob, mode)[0]
