"""Multi-layer exactness of the differentiable tree attention (GPU).

A small random-weight decoder (learned positions, RMSNorm, GQA attention,
SiLU MLP, LM head) is run two ways with the same weights:

* tree: each prompt once and each branch replayed against the prompt's
  per-layer K/V through ``autograd.tree_attention`` (the HIP library) on
  the GPU;
* flattened: every (prompt, branch) pair as one ordinary causal sequence,
  plain torch float64 on the CPU (the baseline the AugTree paper compares
  against, section 2.1, whose result the tree execution must reproduce,
  section 3.2).

Loss: cross entropy on random targets, with the prompt positions counted
once per group, one "first token" target per branch at the last prompt
position, and every response position.  In the flattened run the prompt
positions count only in the group's first sequence.  Every parameter
gradient must agree (relative L2), which requires the prompt K/V gradient
summed over branches to flow back through the prefill into the K/V
projections of every layer.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from shared_prompt_tree_amd import ops
from shared_prompt_tree_amd.autograd import tree_attention
from tests._gpu import rel_l2, say

pytestmark = pytest.mark.gpu

VOCAB, LAYERS, HQ, HKV, D, HIDDEN = 61, 2, 4, 2, 64, 384
DM = HQ * D


def _params(seed, max_pos):
    g = torch.Generator().manual_seed(seed)

    def rnd(*shape, scale):
        return (torch.randn(*shape, generator=g, dtype=torch.float64) * scale)

    p = {"emb": rnd(VOCAB, DM, scale=1.0), "pos": rnd(max_pos, DM, scale=0.5),
         "norm_f": 1.0 + rnd(DM, scale=0.1), "out": rnd(DM, VOCAB, scale=DM ** -0.5)}
    for layer in range(LAYERS):
        p[f"n1_{layer}"] = 1.0 + rnd(DM, scale=0.1)
        p[f"n2_{layer}"] = 1.0 + rnd(DM, scale=0.1)
        p[f"wq_{layer}"] = rnd(DM, HQ * D, scale=DM ** -0.5)
        p[f"wk_{layer}"] = rnd(DM, HKV * D, scale=DM ** -0.5)
        p[f"wv_{layer}"] = rnd(DM, HKV * D, scale=DM ** -0.5)
        p[f"wo_{layer}"] = rnd(HQ * D, DM, scale=(HQ * D) ** -0.5)
        p[f"w1_{layer}"] = rnd(DM, HIDDEN, scale=DM ** -0.5)
        p[f"w2_{layer}"] = rnd(HIDDEN, DM, scale=HIDDEN ** -0.5)
    return p


def _rms(x, w):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-6) * w


def _block_tail(p, layer, x, attn):
    x = x + attn.reshape(x.shape[0], HQ * D) @ p[f"wo_{layer}"]
    h = _rms(x, p[f"n2_{layer}"])
    return x + F.silu(h @ p[f"w1_{layer}"]) @ p[f"w2_{layer}"]


def _qkv(p, layer, x):
    h = _rms(x, p[f"n1_{layer}"])
    n = x.shape[0]
    return ((h @ p[f"wq_{layer}"]).reshape(n, HQ, D), (h @ p[f"wk_{layer}"]).reshape(n, HKV, D),
            (h @ p[f"wv_{layer}"]).reshape(n, HKV, D))


def _causal_attention(q, k, v):
    """Plain causal attention (diagonal included), GQA by contiguous groups."""
    rep = HQ // HKV
    k = k.repeat_interleave(rep, dim=1)
    v = v.repeat_interleave(rep, dim=1)
    s = torch.einsum("thd,jhd->htj", q, k) / math.sqrt(D)
    n = q.shape[0]
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    return torch.einsum("htj,jhd->thd", torch.softmax(s, -1), v)


def _make_batch(prompt_lens, resp_lens, seed):
    rng = np.random.default_rng(seed)
    b = {"p_tok": [rng.integers(0, VOCAB, n) for n in prompt_lens],
         "p_tgt": [rng.integers(0, VOCAB, n) for n in prompt_lens],
         "r_tok": [[rng.integers(0, VOCAB, r) for r in rs] for rs in resp_lens],
         "r_tgt": [[rng.integers(0, VOCAB, r) for r in rs] for rs in resp_lens],
         "first": [[int(rng.integers(0, VOCAB)) for _ in rs] for rs in resp_lens]}
    return b


def _flattened_loss(p, prompt_lens, resp_lens, b):
    """float64 CPU, one causal sequence per (prompt, branch)."""
    total = 0.0
    for g, plen in enumerate(prompt_lens):
        seqs = [(i, r) for i, r in enumerate(resp_lens[g])] or [(None, 0)]
        for k, (i, r) in enumerate(seqs):
            tok = np.concatenate([b["p_tok"][g]] + ([b["r_tok"][g][i]] if i is not None else []))
            n = plen + r
            x = p["emb"][torch.as_tensor(tok)] + p["pos"][:n]
            for layer in range(LAYERS):
                q, kk, v = _qkv(p, layer, x)
                x = _block_tail(p, layer, x, _causal_attention(q, kk, v))
            logits = _rms(x, p["norm_f"]) @ p["out"]
            if k == 0 and plen > 0:
                total = total + F.cross_entropy(logits[:plen], torch.as_tensor(b["p_tgt"][g]),
                                                reduction="sum")
            if i is not None:
                if plen > 0:
                    total = total + F.cross_entropy(logits[plen - 1:plen],
                                                    torch.as_tensor([b["first"][g][i]]),
                                                    reduction="sum")
                if r > 0:
                    total = total + F.cross_entropy(logits[plen:],
                                                    torch.as_tensor(b["r_tgt"][g][i]),
                                                    reduction="sum")
    return total


def _tree_loss(p, prompt_lens, resp_lens, b, problem, dev, op_dtype):
    """The same model over the tree: prompts once, branches replayed.  The
    attention op runs in op_dtype; everything else in the parameters' dtype
    (Q, K, V are rounded to op_dtype on the way in, O converted back)."""
    p_tok = torch.as_tensor(np.concatenate(b["p_tok"]), device=dev)
    p_pos = torch.as_tensor(np.concatenate([np.arange(n) for n in prompt_lens]), device=dev)
    r_tok = torch.as_tensor(np.concatenate([t for rs in b["r_tok"] for t in rs] or [[]]),
                            dtype=torch.long, device=dev)
    r_pos = torch.as_tensor(np.concatenate(
        [np.arange(plen, plen + r) for plen, rs in zip(prompt_lens, resp_lens) for r in rs] or [[]]),
        dtype=torch.long, device=dev)
    xp = p["emb"][p_tok] + p["pos"][p_pos]
    xr = p["emb"][r_tok] + p["pos"][r_pos]
    for layer in range(LAYERS):
        qp, kp, vp = _qkv(p, layer, xp)
        qr, kr, vr = _qkv(p, layer, xr)
        op, orr = tree_attention(problem, *(x.to(op_dtype) for x in (qp, kp, vp, qr, kr, vr)))
        xp = _block_tail(p, layer, xp, op.to(xp.dtype))
        xr = _block_tail(p, layer, xr, orr.to(xr.dtype))
    lp = _rms(xp, p["norm_f"]) @ p["out"]
    lr = _rms(xr, p["norm_f"]) @ p["out"]
    total = F.cross_entropy(lp.float(), torch.as_tensor(np.concatenate(b["p_tgt"]), device=dev),
                            reduction="sum")
    if xr.shape[0] > 0:
        total = total + F.cross_entropy(
            lr.float(), torch.as_tensor(np.concatenate([t for rs in b["r_tgt"] for t in rs]),
                                        device=dev), reduction="sum")
    last = np.cumsum(prompt_lens) - 1
    rows = [int(last[g]) for g, rs in enumerate(resp_lens) for _ in rs if prompt_lens[g] > 0]
    tg = [b["first"][g][i] for g, rs in enumerate(resp_lens) for i in range(len(rs))
          if prompt_lens[g] > 0]
    if rows:
        total = total + F.cross_entropy(lp[rows].float(), torch.as_tensor(tg, device=dev),
                                        reduction="sum")
    return total


# (attention op dtype, model dtype, tolerance).  In the bf16 case the rest of
# the model runs in float32, so the comparison measures the op's own bf16
# rounding (its inputs rounded to bf16, its float32-accumulated result
# rounded to bf16) against the float64 flattened run, at the op's bf16
# tolerance.
CASES = {
    "f32": (torch.float32, torch.float32, 1e-5),
    "bf16": (torch.bfloat16, torch.float32, 1e-2),
}


@pytest.mark.parametrize("dtype_name", list(CASES))
def test_multilayer_gradients_match_flattened(dtype_name):
    dtype, model_dtype, tol = CASES[dtype_name]
    dev = torch.device("cuda:0")
    prompt_lens = [70, 33]
    resp_lens = [[20, 50, 1], [0, 40, 7]]
    say(f"[autograd] {dtype_name}: prompts {prompt_lens}, branches {resp_lens}")
    master = _params(1, max(pl + max(rs, default=0) for pl, rs in zip(prompt_lens, resp_lens)))
    b = _make_batch(prompt_lens, resp_lens, 2)

    ref = {k: v.clone().requires_grad_(True) for k, v in master.items()}
    ref_loss = _flattened_loss(ref, prompt_lens, resp_lens, b)
    ref_loss.backward()

    gcu = np.concatenate([[0], np.cumsum([len(rs) for rs in resp_lens])])
    resp_flat = [r for rs in resp_lens for r in rs]
    problem = ops.TreeProblem(np.concatenate([[0], np.cumsum(prompt_lens)]), gcu,
                              np.concatenate([[0], np.cumsum(resp_flat)]), HQ, HKV, D, dtype,
                              device=dev)
    gp = {k: v.to(dev, model_dtype).requires_grad_(True) for k, v in master.items()}
    loss = _tree_loss(gp, prompt_lens, resp_lens, b, problem, dev, dtype)
    loss.backward()
    torch.cuda.synchronize()

    lv, rv = float(loss.detach()), float(ref_loss.detach())
    lerr = abs(lv - rv) / abs(rv)
    say(f"[autograd] {dtype_name}: loss {lv:.6f} vs {rv:.6f} "
        f"(rel {lerr:.2e})")
    assert lerr <= tol
    worst = 0.0
    for k in master:
        a = gp[k].grad.detach().to("cpu", torch.float64).numpy()
        e = rel_l2(a, ref[k].grad.numpy())
        worst = max(worst, e)
        assert e <= tol, (k, e)
    say(f"[autograd] {dtype_name}: worst parameter-gradient rel L2 {worst:.2e}")
