"""Test helpers: random small trees and a dense tree-mask reference.

The dense reference is a second formulation, independent of the oracle: it
packs the prompt and every branch of a group into one sequence and applies
the tree mask of Eq. 1 of the AugTree paper (section 3.2: a response token
sees the prompt and its own prefix, never a sibling branch; prompt tokens see
the prompt causally).  Gradients come from torch float64 autograd on the loss
sum(dO * O).
"""

import numpy as np
import torch

from shared_prompt_tree_amd.workloads import Tree, offsets, tensor_shapes


def rand_inputs(seed, prompt_lens, resp_lens, hq, hkv, d):
    """Random float64 inputs for a small tree (numpy arrays + offsets)."""
    tree = Tree(list(prompt_lens), [list(r) for r in resp_lens], hq, hkv, d, "f32")
    rng = np.random.default_rng(seed)
    t = {k: rng.standard_normal(s) for k, s in tensor_shapes(tree).items()}
    t.update(offsets(tree))
    return tree, t


def tree_mask(plen, rlens):
    """Boolean visibility matrix of one group, rows = queries, cols = keys."""
    n = plen + sum(rlens)
    m = np.zeros((n, n), dtype=bool)
    for t in range(plen):
        m[t, :t + 1] = True
    start = plen
    for r in rlens:
        for u in range(r):
            m[start + u, :plen] = True
            m[start + u, start:start + u + 1] = True
        start += r
    return m


def dense_reference(tree, t, scale):
    """Forward + backward of the packed tree under the dense Eq. 1 mask."""
    hq, hkv = tree.hq, tree.hkv
    rep = hq // hkv
    res = {
        "o_p": np.zeros(t["q_p"].shape), "o_r": np.zeros(t["q_r"].shape),
        "lse_p": np.zeros((hq, t["q_p"].shape[0])), "lse_r": np.zeros((hq, t["q_r"].shape[0])),
        "dq_p": np.zeros(t["q_p"].shape), "dq_r": np.zeros(t["q_r"].shape),
        "dk_p": np.zeros(t["k_p"].shape), "dk_r": np.zeros(t["k_r"].shape),
        "dv_p": np.zeros(t["v_p"].shape), "dv_r": np.zeros(t["v_r"].shape),
    }
    for g in range(tree.n_groups):
        p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
        b0, b1 = int(tree.group_branch_cu[g]), int(tree.group_branch_cu[g + 1])
        r0, r1 = int(tree.resp_cu[b0]), int(tree.resp_cu[b1])
        rl = [int(tree.resp_cu[i + 1] - tree.resp_cu[i]) for i in range(b0, b1)]
        cat = lambda a, b: torch.tensor(np.concatenate([t[a][p0:p1], t[b][r0:r1]]),
                                        dtype=torch.float64)
        q = cat("q_p", "q_r").requires_grad_(True)
        k = cat("k_p", "k_r").requires_grad_(True)
        v = cat("v_p", "v_r").requires_grad_(True)
        do = cat("do_p", "do_r")
        mask = torch.tensor(tree_mask(p1 - p0, rl))
        n = q.shape[0]
        if n == 0:
            continue
        kv_of_head = torch.arange(hq) // rep
        kh = k[:, kv_of_head]  # [n, hq, d]
        vh = v[:, kv_of_head]
        s = scale * torch.einsum("thd,jhd->htj", q, kh)
        s = s.masked_fill(~mask[None], float("-inf"))
        lse = torch.logsumexp(s, dim=-1)
        p = torch.softmax(s, dim=-1)
        o = torch.einsum("htj,jhd->thd", p, vh)
        (o * do).sum().backward()
        plen = p1 - p0
        o_n, lse_n = o.detach().numpy(), lse.detach().numpy()
        res["o_p"][p0:p1], res["o_r"][r0:r1] = o_n[:plen], o_n[plen:]
        res["lse_p"][:, p0:p1], res["lse_r"][:, r0:r1] = lse_n[:, :plen], lse_n[:, plen:]
        for name, grad in (("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
            gn = grad.numpy()
            res[name + "_p"][p0:p1] = gn[:plen]
            res[name + "_r"][r0:r1] = gn[plen:]
    return res


OUTPUTS = ("o_p", "lse_p", "o_r", "lse_r", "dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nrm = np.linalg.norm(ref)
    err = np.linalg.norm(x - ref)
    return err / nrm if nrm > 0 else err
