"""Full-size workloads on the GPU, checked against the oracle on sampled
outputs it can compute one by one, and against sum rules over everything.

Sampled checks (float64 oracle, ``oracle.causal_unit`` on the flattened
(P, R_i) sequence of a branch), each gated per row as well as over the
sample, so that rows with a large norm cannot hide errors on others:
* forward outputs O, LSE and the query gradient dQ of sampled rows: each
  depends on its own row only;
* dK, dV of the last keys of sampled branches: only rows of that branch at
  or after the key read it, so the rows [k0, L) give the exact gradient;
* prompt dK_P, dV_P of chosen prompt keys of one group and kv head
  (``oracle.causal_key_grads``): the prompt rows at or after the key plus
  every response row of every branch of the group, for every query head of
  the kv head (the sum over branches
  of the AugTree paper, section 3.2, Eq. 2).  Prompt-heavy: the first 64 and
  the last 32 prompt keys; response-heavy: all 256 prompt keys (the launch
  cuts each group's prompt tiles into branch ranges, so this also covers the
  partial seeds and their ordered sum); long-mixed: the last 64 prompt keys.
Sum rules over all outputs: per group and kv head, sum_j dK_j = 0 and
sum_j dV_j = sum of dO over the rows of the query heads that read it.

Each workload runs with both dQ strategies (the separate dQ pass and the
fused dK/dV/dQ kernel) on the same inputs; the automatic choice that the
benchmark uses is one of the two, so its launch configuration is covered.
"""

import math
import multiprocessing as mp

import numpy as np
import pytest
import torch

import oracle
from shared_prompt_tree_amd import ops
from shared_prompt_tree_amd import workloads as wl
from tests._gpu import STRATEGY_NAME, TOL, WORKERS, host64, make_case, rel_l2, run_library, say

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


# ------------------------------------------------------------ prompt keys
#
# The rows that read a prompt key are spread over every branch of its group,
# so the oracle's share is cut into units of rows (bounded work each) and run
# in forked workers; the inputs of the one group and kv head are float64
# host copies inherited by the workers.

_KEYS = None
_PAIRS_PER_UNIT = 200_000_000


def _key_unit(args):
    """dK, dV of the chosen prompt keys from one query head of one branch,
    over the flattened rows [a, b) of that branch."""
    from threadpoolctl import threadpool_limits

    i, j, a, b, scale = args
    d = _KEYS
    first = i == d["b0"]
    xq = np.concatenate([d["qp"][:, j], d["qr"][i][:, j]])
    xk = np.concatenate([d["kp"], d["kr"][i]])
    xv = np.concatenate([d["vp"], d["vr"][i]])
    dop = d["dop"][:, j] if first else np.zeros_like(d["dop"][:, j])
    xdo = np.concatenate([dop, d["dor"][i][:, j]])
    with threadpool_limits(1):
        return oracle.causal_key_grads(xq, xk, xv, xdo, scale, np.arange(a, b), d["keys"],
                                       chunk=512)


def prompt_key_grads(tree, t, g, kv, keys):
    """Oracle dK_P, dV_P [len(keys), d] of prompt keys ``keys`` (positions in
    group g's prompt) for kv head kv: every query head of kv, every branch of
    g.  The prompt rows carry their upstream gradient in the group's first
    branch only (exact: the backward is linear in dO), so later branches
    contribute through their response rows alone."""
    global _KEYS
    rep = tree.hq // tree.hkv
    hs = slice(kv * rep, (kv + 1) * rep)
    p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
    b0, b1 = int(tree.group_branch_cu[g]), int(tree.group_branch_cu[g + 1])
    P = p1 - p0
    keys = np.asarray(keys)
    data = {"b0": b0, "keys": keys, "qp": host64(t["q_p"][p0:p1, hs]),
            "kp": host64(t["k_p"][p0:p1, kv]), "vp": host64(t["v_p"][p0:p1, kv]),
            "dop": host64(t["do_p"][p0:p1, hs]), "qr": {}, "kr": {}, "vr": {}, "dor": {}}
    units = []
    scale = 1.0 / math.sqrt(tree.d)
    for i in range(b0, b1):
        r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
        data["qr"][i] = host64(t["q_r"][r0:r1, hs])
        data["kr"][i] = host64(t["k_r"][r0:r1, kv])
        data["vr"][i] = host64(t["v_r"][r0:r1, kv])
        data["dor"][i] = host64(t["do_r"][r0:r1, hs])
        L = P + r1 - r0
        start = int(keys.min()) if i == b0 else P  # first row that can read a chosen key
        for j in range(rep):
            a = start
            while a < L:  # rows [a, b) with about _PAIRS_PER_UNIT (row, key) pairs
                b = min(L, a + max(1, _PAIRS_PER_UNIT // (a + 1)))
                units.append((i, j, a, b, scale))
                a = b
    _KEYS = data
    try:
        with mp.get_context("fork").Pool(min(WORKERS, len(units))) as pool:
            parts = pool.map(_key_unit, units, chunksize=1)
    finally:
        _KEYS = None
    dk = sum(x[0] for x in parts)
    dv = sum(x[1] for x in parts)
    say(f"[full] prompt keys of group {g}, kv head {kv}: {len(keys)} keys, {len(units)} "
        f"oracle units over {b1 - b0} branches x {rep} query heads")
    return dk, dv


# A sampled row whose reference norm is below this fraction of the sample's
# median row norm is measured against that fraction instead: prompt row 0,
# with a single visible key, has dQ = 0 exactly (its one dS is dP - D with
# D = dP), and the GPU's value is the float32 rounding residue of that
# difference, about 1.5e-5 of the median row on the prompt-heavy workload.
ROW_FLOOR = 1e-2


def _row_errors(a, b, kind):
    """Error of each row of a sampled block: relative L2 of a (token, head)
    vector of head_dim values, floored at ROW_FLOOR times the median row
    norm; for LSE (one value per row, a logarithm) |x - x*| / max(1, |x*|)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if kind == "lse":
        return np.abs(a - b).ravel() / np.maximum(1.0, np.abs(b).ravel())
    a = a.reshape(-1, a.shape[-1])
    b = b.reshape(a.shape)
    den = np.linalg.norm(b, axis=1)
    den = np.maximum(den, ROW_FLOOR * np.median(den))
    return np.linalg.norm(a - b, axis=1) / den


def _check_sampled(label, got, want):
    for k in got:
        if not got[k]:
            continue
        a = np.concatenate([x.ravel() for x in got[k]])
        b = np.concatenate([x.ravel() for x in want[k]])
        err = rel_l2(a, b)
        kind = "lse" if k == "lse" else "vec"
        rows = np.concatenate([_row_errors(x, y, kind) for x, y in zip(got[k], want[k])])
        worst = int(np.argmax(rows))
        say(f"[full] {label} sampled {k}: {len(a)} values, rel L2 {err:.2e}; "
            f"{len(rows)} rows, worst row {rows[worst]:.2e}, median row "
            f"{float(np.median(rows)):.2e}")
        assert err <= TOL["bf16"], (k, err)
        assert rows[worst] <= TOL["bf16"], (k, worst, rows[worst])


PROMPT_KEYS = {
    # (first keys, last keys) of group 0's prompt, one kv head
    "prompt_heavy": (64, 32),
    "response_heavy": (256, 0),
    "long_mixed": (0, 64),
}


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    spec = wl.SPECS[name]
    tree = wl.make_tree(spec)
    scale = 1.0 / math.sqrt(tree.d)
    say(f"[full] {name}: {tree.prompt_tokens} prompt + {tree.resp_tokens} response tokens")
    prob, t = make_case(tree, spec.seed)
    libs = {}
    for st in (ops.DQ_SEPARATE, ops.DQ_FUSED):
        prob.dq_strategy = st
        libs[st] = run_library(prob, t)
        for k, v in libs[st].items():
            if v is not None:
                assert bool(torch.isfinite(v).all()), (STRATEGY_NAME[st], k)
    say("[full] library done (both dQ strategies)")
    rng = np.random.default_rng(spec.seed)
    want = {k: [] for k in ("o", "lse", "dq", "dk", "dv")}
    got = {st: {k: [] for k in want} for st in libs}

    def take(k, f):
        for st, lib in libs.items():
            got[st][k].append(host64(f(lib)))

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
            take("o", lambda lib: lib["o_r"][tok, h])
            take("lse", lambda lib: lib["lse_r"][h, tok])
            take("dq", lambda lib: lib["dq_r"][tok, h])
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
        take("o", lambda lib: lib["o_p"][tok, h])
        take("lse", lambda lib: lib["lse_p"][h, tok])
        take("dq", lambda lib: lib["dq_p"][tok, h])
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
        take("dk", lambda lib: lib["dk_r"][r1 - n:r1, kv])
        take("dv", lambda lib: lib["dv_r"][r1 - n:r1, kv])
        want["dk"].append(dk)
        want["dv"].append(dv)

    # prompt dK_P, dV_P of chosen prompt keys of group 0, summed over every
    # branch of the group and every query head of the kv head
    n_first, n_last = PROMPT_KEYS[name]
    P = int(tree.prompt_cu[1])
    keys = np.array(sorted(set(range(min(n_first, P))) | set(range(max(0, P - n_last), P))))
    kv = int(rng.integers(0, tree.hkv))
    dk, dv = prompt_key_grads(tree, t, 0, kv, keys)
    for st, lib in libs.items():
        got[st]["dk_p"] = [host64(lib["dk_p"][keys, kv])]
        got[st]["dv_p"] = [host64(lib["dv_p"][keys, kv])]
    want["dk_p"] = [dk]
    want["dv_p"] = [dv]

    for st in libs:
        _check_sampled(f"{name} [{STRATEGY_NAME[st]}]", got[st], want)
    for st, lib in libs.items():
        _sum_rules(f"{name} [{STRATEGY_NAME[st]}]", tree, t, lib)


def _sum_rules(name, tree, t, lib):
    """sum rules over every output, float64 on the GPU"""
    rep = tree.hq // tree.hkv
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
    _check_sampled("wide prefill", got, want)
