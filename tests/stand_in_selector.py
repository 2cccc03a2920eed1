"""A stand-in trainable selector for the end-to-end gradient tests.

The pages do not fix the selector network, only that its block scores
enter the attention softmax as log gates and are trained by the loss.  Any
differentiable map from weights to logits exercises that path; this one is
a bilinear score between per-block query and key features,

    logits[g, Q, j] = qf[Q] . W[g] . kf[c_s + j]

for the key blocks j of query block Q's own sequence s (c_s its first
block), and 0 in the padding columns.  Random weights, plain torch ops
(test code: runs wherever its tensors live).
"""


def selector_logits(qf, kf, W, cu_qblocks, ld):
    """qf, kf [QB, f]; W [hkv, f, f] -> logits [hkv, QB, ld]."""
    import torch
    rows = []
    for s in range(len(cu_qblocks) - 1):
        a, b = int(cu_qblocks[s]), int(cu_qblocks[s + 1])
        A = torch.matmul(torch.matmul(qf[a:b].unsqueeze(0), W), kf[a:b].t().contiguous())
        rows.append(torch.nn.functional.pad(A, (0, ld - (b - a))))
    return torch.cat(rows, dim=1).contiguous()
