"""Helpers for the GPU parity tests: run the HIP library, run the oracle on
the same inputs, compare by relative L2."""

import math
import os
import sys

import numpy as np
import torch

import oracle
from shared_prompt_tree_amd import ops
from shared_prompt_tree_amd import workloads as wl

OUT_NAMES = ("o_p", "lse_p", "o_r", "lse_r", "dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")
TOL = {"f32": 1e-5, "bf16": 1e-2}
WORKERS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def make_case(tree, seed, value_scale=1.0, zero_do_p=False, dq_strategy=ops.DQ_SEPARATE):
    """Inputs on the GPU plus the problem descriptor."""
    dev = device()
    t = wl.make_tensors(tree, seed, device=dev, value_scale=value_scale)
    if zero_do_p:
        t["do_p"].zero_()
    prob = ops.TreeProblem.from_tree(tree, device=dev, dq_strategy=dq_strategy)
    return prob, t


def fused_ok(tree):
    """The fused dQ strategy covers bf16 with head_dim 128."""
    return tree.dtype == "bf16" and tree.d == 128


def strategies(tree):
    """The dQ strategies a parity case runs: both where the fused one applies."""
    return (ops.DQ_SEPARATE, ops.DQ_FUSED) if fused_ok(tree) else (ops.DQ_SEPARATE,)


STRATEGY_NAME = {ops.DQ_SEPARATE: "separate dQ", ops.DQ_FUSED: "fused dQ"}


def run_library(prob, t, seeds=True):
    out = ops.tree_attention_forward_backward(prob, t, seeds=seeds)
    torch.cuda.synchronize()
    return out


def host64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def oracle_inputs(tree, t):
    d = {k: host64(v) for k, v in t.items()}
    d.update(wl.offsets(tree))
    return d


def run_oracle(tree, t):
    o, _ = oracle.tree_attention_parallel(oracle_inputs(tree, t), 1.0 / math.sqrt(tree.d),
                                          fast=True, workers=WORKERS)
    return o


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    e = np.linalg.norm(x - ref)
    return e / n if n > 0 else e


def _segments(tree, name):
    """Row ranges of an output tensor that the per-segment check gates: the
    prompt of each group for prompt tensors, each branch for response
    tensors.  Returns (token axis, [(start, stop), ...])."""
    cu = tree.prompt_cu if name.endswith("_p") else tree.resp_cu
    axis = 1 if name.startswith("lse") else 0
    return axis, [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]


# A segment whose reference norm is below this fraction of its share of the
# whole tensor's norm (the tensor norm scaled by sqrt(segment size / tensor
# size)) is compared against that share instead: its own norm is then a
# cancellation residue, not a scale.
SEG_FLOOR = 1e-2


def segment_errors(x, ref, tree, name):
    """Relative L2 of every (segment, head) block of one output tensor:
    ||x - ref|| / max(||ref||, SEG_FLOOR * share), per group prompt or per
    branch and per head.  Returns the worst value and where it occurred."""
    axis, segs = _segments(tree, name)
    n_tok = ref.shape[axis]
    total = np.linalg.norm(ref)
    worst, where = 0.0, None
    heads = ref.shape[0] if axis == 1 else ref.shape[1]
    for a, b in segs:
        for h in range(heads):
            if axis == 1:
                xs, rs = x[h, a:b], ref[h, a:b]
            else:
                xs, rs = x[a:b, h], ref[a:b, h]
            share = total * math.sqrt((b - a) / max(n_tok, 1) / heads)
            den = max(np.linalg.norm(rs), SEG_FLOOR * share)
            e = np.linalg.norm(xs - rs) / den if den > 0 else np.linalg.norm(xs)
            if e > worst:
                worst, where = e, (a, b, h)
    return worst, where


def compare(lib, ref, tol, names=OUT_NAMES, label="", tree=None):
    """Relative L2 per output tensor, and (given the tree) per group prompt or
    branch and head, so that a large-norm row cannot hide errors elsewhere.
    Both must be within tol."""
    errs, seg = {}, {}
    for k in names:
        a = host64(lib[k])
        if a.size == 0:
            errs[k] = 0.0
            continue
        assert np.all(np.isfinite(a)), f"{label} {k}: non-finite values"
        errs[k] = rel_l2(a, ref[k])
        if tree is not None:
            seg[k] = segment_errors(a, np.asarray(ref[k], np.float64), tree, k)
    say(label, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    if seg:
        say(label, "worst segment:", " ".join(f"{k}={v[0]:.2e}" for k, v in seg.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: rel L2 above {tol}: {bad}"
    bad = {k: v for k, v in seg.items() if not v[0] <= tol}
    assert not bad, f"{label}: per-segment rel L2 above {tol} (start, stop, head): {bad}"
    return errs
