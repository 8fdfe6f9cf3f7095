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


def make_case(tree, seed, value_scale=1.0, zero_do_p=False):
    """Inputs on the GPU plus the problem descriptor."""
    dev = device()
    t = wl.make_tensors(tree, seed, device=dev, value_scale=value_scale)
    if zero_do_p:
        t["do_p"].zero_()
    prob = ops.TreeProblem.from_tree(tree, device=dev)
    return prob, t


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


def compare(lib, ref, tol, names=OUT_NAMES, label=""):
    errs = {}
    for k in names:
        a = host64(lib[k])
        if a.size == 0:
            errs[k] = 0.0
            continue
        assert np.all(np.isfinite(a)), f"{label} {k}: non-finite values"
        errs[k] = rel_l2(a, ref[k])
    say(label, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: rel L2 above {tol}: {bad}"
    return errs
