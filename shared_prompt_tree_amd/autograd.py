"""Tree attention as one differentiable torch op.

Forward runs the prompt prefill and the response replay, with the prompt
column and the own-branch part merged per row.  Backward runs the replay
backward. Its float32 prompt seeds (the sum over branches, AugTree paper
section 3.2, Eq. 2) go into the prefill backward, so the prompt K/V get
their whole gradient.  The page's "Exact many-to-one backward" describes
this step: the seeds flow back through the prompt's own prefill.  Used
inside a model, the prompt K/V gradient then reaches the projections that
produced them.

All arithmetic runs in the HIP library; this module only passes tensors.
"""

from __future__ import annotations

import torch

from . import ops


class TreeAttention(torch.autograd.Function):
    """(o_p, o_r) = tree attention of (q_p, k_p, v_p) and (q_r, k_r, v_r).

    Shapes follow the C ABI: prompt tensors [sum P_g, H, d], response
    tensors [sum r_i, H, d], with H = Hq for q/o and Hkv for k/v.  All six
    inputs share the problem's dtype and device.
    """

    @staticmethod
    def forward(ctx, problem, q_p, k_p, v_p, q_r, k_r, v_r):
        q_p, k_p, v_p, q_r, k_r, v_r = (x.contiguous() for x in (q_p, k_p, v_p, q_r, k_r, v_r))
        o_p, lse_p = ops.tree_attn_prefill(problem, q_p, k_p, v_p)
        o_r, lse_r = ops.tree_attn_replay_fwd(problem, k_p, v_p, q_r, k_r, v_r)
        ctx.problem = problem
        ctx.save_for_backward(q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r)
        return o_p, o_r

    @staticmethod
    def backward(ctx, do_p, do_r):
        q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r = ctx.saved_tensors
        pr = ctx.problem
        do_p = torch.zeros_like(o_p) if do_p is None else do_p.contiguous()
        do_r = torch.zeros_like(o_r) if do_r is None else do_r.contiguous()
        dq_r, dk_r, dv_r, dks, dvs = ops.tree_attn_replay_bwd(pr, k_p, v_p, q_r, k_r, v_r, o_r,
                                                              lse_r, do_r)
        dq_p, dk_p, dv_p = ops.tree_attn_prefill_bwd(pr, q_p, k_p, v_p, o_p, lse_p, do_p, dks,
                                                     dvs)
        return None, dq_p, dk_p, dv_p, dq_r, dk_r, dv_r


def tree_attention(problem, q_p, k_p, v_p, q_r, k_r, v_r):
    """Differentiable tree attention; returns (o_p, o_r)."""
    return TreeAttention.apply(problem, q_p, k_p, v_p, q_r, k_r, v_r)
