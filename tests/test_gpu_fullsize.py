"""Full-size workloads on the GPU, checked against the oracle on sampled
outputs it can compute one by one, and against sum rules over everything.

Sampled checks (float64 oracle, ``oracle.causal_unit`` on the flattened
(P, R_i) sequence of the sampled branch):
* forward outputs O, LSE and the query gradient dQ of sampled rows: each
  depends on its own row only;
* dK, dV of the last keys of sampled branches: only rows of that branch at
  or after the key read it, so the rows [k0, L) give the exact gradient;
* (prompt-heavy shape) dK_P, dV_P of the last prompt keys: the prompt rows
  after them plus every response row of every branch.
Sum rules over all outputs: per group and kv head, sum_j dK_j = 0 and
sum_j dV_j = sum of dO over the rows of the query heads that read it.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from shared_prompt_tree_amd import workloads as wl
from tests._gpu import TOL, host64, make_case, rel_l2, run_library, say

pytestmark = pytest.mark.gpu

FULL = ["prompt_heavy", "response_heavy", "long_mixed"]


def _flat(tree, t, g, i, h, with_branch=True):
    """Float64 flattened sequence (prompt of group g, then branch i) for
    query head h and its kv head."""
    kv = h * tree.hkv // tree.hq
    p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
    parts = {"q": [], "k": [], "v": [], "do": []}
    first = i == int(tree.group_branch_cu[g])
    for name, hh in (("q", h), ("k", kv), ("v", kv), ("do", h)):
        x = t[name + "_p"][p0:p1, hh]
        if name == "do" and not first:
            x = torch.zeros_like(x)
        parts[name].append(x)
        if with_branch:
            r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
            parts[name].append(t[name + "_r"][r0:r1, hh])
    return {k: host64(torch.cat(v)) for k, v in parts.items()}


def _sample_branches(tree, rng):
    picks = set()
    for g in range(tree.n_groups):
        b0, b1 = int(tree.group_branch_cu[g]), int(tree.group_branch_cu[g + 1])
        if b1 > b0:
            picks.update({b0, b1 - 1, int(rng.integers(b0, b1))})
    return sorted(picks)[:6]


def _group_of(tree, i):
    return int(np.searchsorted(tree.group_branch_cu, i, side="right") - 1)


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    spec = wl.SPECS[name]
    tree = wl.make_tree(spec)
    scale = 1.0 / math.sqrt(tree.d)
    say(f"[full] {name}: {tree.prompt_tokens} prompt + {tree.resp_tokens} response tokens")
    prob, t = make_case(tree, spec.seed)
    lib = run_library(prob, t)
    for k, v in lib.items():
        if v is not None:
            assert bool(torch.isfinite(v).all()), k
    say("[full] library done")
    rng = np.random.default_rng(spec.seed)
    got = {k: [] for k in ("o", "lse", "dq", "dk", "dv")}
    want = {k: [] for k in got}

    # sampled response rows and prompt rows
    for i in _sample_branches(tree, rng):
        g = _group_of(tree, i)
        P = int(tree.prompt_cu[g + 1] - tree.prompt_cu[g])
        r = int(tree.resp_cu[i + 1] - tree.resp_cu[i])
        if r == 0:
            continue
        for h in sorted({0, tree.hq - 1, int(rng.integers(0, tree.hq))}):
            f = _flat(tree, t, g, i, h)
            loc = sorted({0, r - 1, r // 2, *rng.integers(0, r, size=5).tolist()})
            rows = np.array([P + u for u in loc])
            o, lse, dq, _, _ = oracle.causal_unit(f["q"], f["k"], f["v"], f["do"], scale, rows=rows)
            tok = [int(tree.resp_cu[i]) + u for u in loc]
            got["o"].append(host64(lib["o_r"][tok, h]))
            got["lse"].append(host64(lib["lse_r"][h, tok]))
            got["dq"].append(host64(lib["dq_r"][tok, h]))
            want["o"].append(o)
            want["lse"].append(lse)
            want["dq"].append(dq)
    for g in range(tree.n_groups):
        P = int(tree.prompt_cu[g + 1] - tree.prompt_cu[g])
        h = int(rng.integers(0, tree.hq))
        f = _flat(tree, t, g, int(tree.group_branch_cu[g]), h, with_branch=False)
        loc = np.array(sorted({0, P - 1, P // 3, *rng.integers(0, P, size=5).tolist()}))
        o, lse, dq, _, _ = oracle.causal_unit(f["q"], f["k"], f["v"], f["do"], scale, rows=loc)
        tok = (int(tree.prompt_cu[g]) + loc).tolist()
        got["o"].append(host64(lib["o_p"][tok, h]))
        got["lse"].append(host64(lib["lse_p"][h, tok]))
        got["dq"].append(host64(lib["dq_p"][tok, h]))
        want["o"].append(o)
        want["lse"].append(lse)
        want["dq"].append(dq)

    # dK_R, dV_R of the last keys of sampled branches
    rep = tree.hq // tree.hkv
    for i in _sample_branches(tree, rng)[:3]:
        g = _group_of(tree, i)
        P = int(tree.prompt_cu[g + 1] - tree.prompt_cu[g])
        r = int(tree.resp_cu[i + 1] - tree.resp_cu[i])
        n = min(r, 48)
        if n == 0:
            continue
        kv = int(rng.integers(0, tree.hkv))
        dk = 0
        dv = 0
        for h in range(kv * rep, (kv + 1) * rep):
            f = _flat(tree, t, g, i, h)
            rows = np.arange(P + r - n, P + r)
            _, _, _, dk_h, dv_h = oracle.causal_unit(f["q"], f["k"], f["v"], f["do"], scale,
                                                     rows=rows)
            dk = dk + dk_h[P + r - n:]
            dv = dv + dv_h[P + r - n:]
        r1 = int(tree.resp_cu[i + 1])
        got["dk"].append(host64(lib["dk_r"][r1 - n:r1, kv]))
        got["dv"].append(host64(lib["dv_r"][r1 - n:r1, kv]))
        want["dk"].append(dk)
        want["dv"].append(dv)

    if name == "prompt_heavy":
        # last prompt keys: prompt rows after them and every response row
        g, kv, n = 0, int(rng.integers(0, tree.hkv)), 32
        P = int(tree.prompt_cu[1])
        b0, b1 = int(tree.group_branch_cu[0]), int(tree.group_branch_cu[1])
        dk = 0
        dv = 0
        for h in range(kv * rep, (kv + 1) * rep):
            for i in range(b0, b1):
                f = _flat(tree, t, g, i, h)
                L = f["q"].shape[0]
                rows = np.arange(P - n if i == b0 else P, L)
                _, _, _, dk_h, dv_h = oracle.causal_unit(f["q"], f["k"], f["v"], f["do"], scale,
                                                         rows=rows)
                dk = dk + dk_h[P - n:P]
                dv = dv + dv_h[P - n:P]
        got["dk"].append(host64(lib["dk_p"][P - n:P, kv]))
        got["dv"].append(host64(lib["dv_p"][P - n:P, kv]))
        want["dk"].append(dk)
        want["dv"].append(dv)

    for k in got:
        if not got[k]:
            continue
        a = np.concatenate([x.ravel() for x in got[k]])
        b = np.concatenate([x.ravel() for x in want[k]])
        err = rel_l2(a, b)
        say(f"[full] {name} sampled {k}: {len(a)} values, rel L2 {err:.2e}")
        assert err <= TOL["bf16"], (k, err)

    # sum rules over every output, float64 on the GPU
    worst_k = worst_v = 0.0
    for g in range(tree.n_groups):
        p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
        b0, b1 = int(tree.group_branch_cu[g]), int(tree.group_branch_cu[g + 1])
        r0, r1 = int(tree.resp_cu[b0]), int(tree.resp_cu[b1])
        for kv in range(tree.hkv):
            hs = slice(kv * rep, (kv + 1) * rep)
            dk = torch.cat([lib["dk_p"][p0:p1, kv], lib["dk_r"][r0:r1, kv]]).double()
            dv = torch.cat([lib["dv_p"][p0:p1, kv], lib["dv_r"][r0:r1, kv]]).double()
            do_sum = (t["do_p"][p0:p1, hs].double().sum((0, 1))
                      + t["do_r"][r0:r1, hs].double().sum((0, 1)))
            ek = float(dk.sum(0).norm() / dk.norm())
            ev = float((dv.sum(0) - do_sum).norm() / do_sum.norm())
            worst_k, worst_v = max(worst_k, ek), max(worst_v, ev)
    say(f"[full] {name} sum rules: |sum dK|/|dK| {worst_k:.2e}, "
        f"|sum dV - sum dO|/|sum dO| {worst_v:.2e}")
    assert worst_k <= TOL["bf16"] and worst_v <= TOL["bf16"]


def test_wide_forward_tiles():
    """Prefill large enough for the 12-wave forward kernel (384-row tiles:
    6144 tokens x 16 packed heads / 384 = 256 tiles per head group, 4 head
    groups): sampled prompt rows of O, LSE and dQ against the oracle, and
    the sum rules."""
    tree = wl.Tree([6144], [[700]], 64, 4, 64, "bf16")
    scale = 1.0 / math.sqrt(tree.d)
    say("[wide] prefill 6144 tokens, 64/4 heads, d 64")
    prob, t = make_case(tree, 21)
    lib = run_library(prob, t)
    rng = np.random.default_rng(21)
    P = 6144
    got = {k: [] for k in ("o", "lse", "dq")}
    want = {k: [] for k in got}
    for h in (0, 17, 63):
        f = _flat(tree, t, 0, 0, h, with_branch=False)
        loc = np.array(sorted({0, 383, 384, P - 1, *rng.integers(0, P, size=12).tolist()}))
        o, lse, dq, _, _ = oracle.causal_unit(f["q"], f["k"], f["v"], f["do"], scale, rows=loc)
        got["o"].append(host64(lib["o_p"][loc, h]))
        got["lse"].append(host64(lib["lse_p"][h, loc]))
        got["dq"].append(host64(lib["dq_p"][loc, h]))
        want["o"].append(o)
        want["lse"].append(lse)
        want["dq"].append(dq)
    for k in got:
        a = np.concatenate([x.ravel() for x in got[k]])
        b = np.concatenate([x.ravel() for x in want[k]])
        err = rel_l2(a, b)
        say(f"[wide] sampled {k}: {len(a)} values, rel L2 {err:.2e}")
        assert err <= TOL["bf16"], (k, err)
