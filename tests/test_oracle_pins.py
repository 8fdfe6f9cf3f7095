"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names the fact it relies on.  Paper = "Splitting Prompt Prefill
from Response Replay for Context-Parallel Long-Context LLM Post-Training".
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from shared_prompt_tree_amd import workloads as wl
from tests._dense import OUTPUTS, dense_reference, rand_inputs, rel_l2, tree_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (prompt_lens, resp_lens, hq, hkv, d): ragged lengths, an empty branch, a
# one-token prompt, G = 1, a prompt with no branch, MHA, GQA and MQA.
CASES = [
    ([7], [[5, 3, 4]], 2, 1, 4),
    ([5, 1], [[4, 0, 6], [3]], 4, 2, 8),
    ([6, 4], [[2, 5], []], 3, 3, 5),
    ([9], [[1]], 4, 4, 3),
    ([1], [[7, 2]], 2, 2, 6),
    ([0], [[4, 3]], 2, 1, 4),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("fast", [False, True])
def test_matches_dense_tree_mask_autograd(case, fast):
    """Flattened per-branch causal attention == dense Eq. 1 tree mask.

    Paper section 3.3 ("Common tile semantics") and section 4.5
    ("Correctness"): prompt-once replay computes the same attention as the
    flattened pairs, and section 3.2 Eq. 2: prompt gradients are the sum over
    branches.  The reference here is a different formulation (one dense
    masked softmax per group) with gradients from torch autograd.
    """
    pl, rl, hq, hkv, d = CASES[case]
    tree, t = rand_inputs(100 + case, pl, rl, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    got = oracle.tree_attention(t, scale, fast=fast, chunk=3)
    ref = dense_reference(tree, t, scale)
    for k in OUTPUTS:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-10, atol=1e-11, err_msg=k)


def test_parallel_driver_matches_serial():
    tree, t = rand_inputs(7, [12, 5], [[4, 9, 1], [6]], 4, 2, 8)
    a = oracle.tree_attention(t, 0.3, fast=False)
    b, used = oracle.tree_attention_parallel(t, 0.3, fast=True, workers=3)
    assert used == 3
    for k in OUTPUTS:
        np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-13, err_msg=k)


def _loss(t, scale, do_p, do_r):
    o = oracle.tree_attention(t, scale, fast=True)
    return float((o["o_p"] * do_p).sum() + (o["o_r"] * do_r).sum())


def test_finite_differences():
    """Central differences of L = sum(dO * O) agree with the oracle's
    gradients (calculus; no attention formula is reused)."""
    tree, t = rand_inputs(11, [4], [[3, 2]], 2, 1, 3)
    scale = 0.7
    g = oracle.tree_attention(t, scale, fast=False)
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, gname in (("q_p", "dq_p"), ("k_p", "dk_p"), ("v_p", "dv_p"),
                        ("q_r", "dq_r"), ("k_r", "dk_r"), ("v_r", "dv_r")):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in t[name].shape)
            tp = dict(t)
            tp[name] = t[name].copy()
            tp[name][idx] += h
            lp = _loss(tp, scale, t["do_p"], t["do_r"])
            tp[name][idx] -= 2 * h
            lm = _loss(tp, scale, t["do_p"], t["do_r"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[gname][idx]) < 1e-7 * max(1.0, abs(fd)), (name, idx)


def _subset_state(q, k, v, scale):
    """Partial attention state (O, LSE) of rows q over the key subset k/v."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    s = scale * q @ k.T
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=1, keepdims=True)
    return e @ v / ell, m[:, 0] + np.log(ell[:, 0])


@pytest.mark.parametrize("nshards", [2, 3, 7])
def test_prompt_split_and_merge_is_exact(nshards):
    """Sharding the prompt K/V, computing a partial state per shard plus the
    own-branch partial, and merging them in any order gives the unsplit
    replay output (paper section 3.3 and Fig. 8: partial online-softmax
    states along a query row are merged associatively)."""
    tree, t = rand_inputs(20 + nshards, [23], [[5, 8, 3]], 2, 1, 4)
    scale = 0.5
    full = oracle.tree_attention(t, scale, fast=True)
    rng = np.random.default_rng(nshards)
    plen = 23
    cuts = np.sort(rng.choice(np.arange(1, plen), size=nshards - 1, replace=False))
    bounds = [0, *cuts.tolist(), plen]
    bounds.insert(1, 0)  # one empty shard: the identity of the merge
    for h in range(tree.hq):
        kv = h * tree.hkv // tree.hq
        for i in range(tree.n_branches):
            r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
            q = t["q_r"][r0:r1, h]
            parts_o, parts_l = [], []
            for a, b in zip(bounds[:-1], bounds[1:]):
                o, lse = _subset_state(q, t["k_p"][a:b, kv], t["v_p"][a:b, kv], scale)
                parts_o.append(o)
                parts_l.append(lse)
            # own branch, causal with diagonal: row u sees keys r0 .. r0+u
            own_o, own_l = [], []
            for u in range(r1 - r0):
                o, lse = _subset_state(q[u:u + 1], t["k_r"][r0:r0 + u + 1, kv],
                                       t["v_r"][r0:r0 + u + 1, kv], scale)
                own_o.append(o[0])
                own_l.append(lse[0])
            parts_o.append(np.array(own_o))
            parts_l.append(np.array(own_l))
            po = np.stack(parts_o)[:, :, None, :]  # [S, rows, 1, d]
            pl = np.stack(parts_l)[:, None, :]     # [S, 1, rows]
            perm = rng.permutation(len(parts_o))
            o1, l1 = oracle.lse_merge(po[perm], pl[perm])
            # a different bracketing: merge the first half, then the rest
            half = len(perm) // 2
            oa, la = oracle.lse_merge(po[perm[:half]], pl[perm[:half]])
            o2, l2 = oracle.lse_merge(np.stack([oa, *po[perm[half:]]]),
                                      np.stack([la, *pl[perm[half:]]]))
            for o_m, l_m in ((o1, l1), (o2, l2)):
                np.testing.assert_allclose(o_m[:, 0], full["o_r"][r0:r1, h], atol=1e-13)
                np.testing.assert_allclose(l_m[0], full["lse_r"][h, r0:r1], atol=1e-13)


def test_lse_merge_special_cases():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 5, 2, 3))
    lse = rng.standard_normal((1, 2, 5))
    # one part is itself
    o1, l1 = oracle.lse_merge(o, lse)
    np.testing.assert_allclose(o1, o[0], atol=0)
    np.testing.assert_allclose(l1, lse[0], atol=0)
    # two equal parts: same output, normaliser doubled
    o2, l2 = oracle.lse_merge(np.concatenate([o, o]), np.concatenate([lse, lse]))
    np.testing.assert_allclose(o2, o[0], atol=1e-15)
    np.testing.assert_allclose(l2, lse[0] + math.log(2.0), atol=1e-14)
    # an empty part (LSE = -inf, any finite O) is the identity
    junk = rng.standard_normal(o.shape) * 1e6
    o3, l3 = oracle.lse_merge(np.concatenate([junk, o]),
                              np.concatenate([np.full(lse.shape, -np.inf), lse]))
    np.testing.assert_allclose(o3, o[0], atol=1e-15)
    np.testing.assert_allclose(l3, lse[0], atol=0)
    # every part empty: LSE = -inf and O = 0
    o4, l4 = oracle.lse_merge(junk, np.full(lse.shape, -np.inf))
    assert np.all(np.isneginf(l4)) and np.all(o4 == 0)
    # weights: a part 30 nats larger dominates
    o5, l5 = oracle.lse_merge(np.concatenate([o, junk]),
                              np.concatenate([lse + 30.0, lse]))
    np.testing.assert_allclose(o5, o[0], atol=1e-6 * 1e6)


def test_zero_queries_closed_form():
    """Q = 0: every visible key has score 0, so LSE = ln(#visible keys) and O
    is the mean of the visible V rows (prompt row t sees t+1 keys; response
    row u sees P + u + 1 keys)."""
    tree, t = rand_inputs(5, [6], [[4, 3]], 2, 1, 3)
    t["q_p"][:] = 0
    t["q_r"][:] = 0
    r = oracle.tree_attention(t, 0.9, fast=False)
    for h in range(2):
        for u in range(6):
            assert r["lse_p"][h, u] == pytest.approx(math.log(u + 1), abs=1e-14)
            np.testing.assert_allclose(r["o_p"][u, h], t["v_p"][:u + 1, 0].mean(0), atol=1e-14)
        for i in range(2):
            r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
            for u in range(r1 - r0):
                assert r["lse_r"][h, r0 + u] == pytest.approx(math.log(6 + u + 1), abs=1e-14)
                vis = np.concatenate([t["v_p"][:, 0], t["v_r"][r0:r0 + u + 1, 0]])
                np.testing.assert_allclose(r["o_r"][r0 + u, h], vis.mean(0), atol=1e-14)


def test_constant_values_closed_form():
    """All V rows equal c: O = c, and dP_tj = dO_t . c = D_t so dS = 0,
    dQ = 0 and dK = 0."""
    tree, t = rand_inputs(6, [5, 3], [[4, 2], [3]], 4, 2, 3)
    c = np.array([0.3, -1.2, 2.0])
    t["v_p"][:] = c
    t["v_r"][:] = c
    r = oracle.tree_attention(t, 0.8, fast=False)
    for k in ("o_p", "o_r"):
        np.testing.assert_allclose(r[k], np.broadcast_to(c, r[k].shape), atol=1e-14)
    for k in ("dq_p", "dq_r", "dk_p", "dk_r"):
        np.testing.assert_allclose(r[k], 0, atol=1e-13)


def test_single_branch_is_plain_causal_attention():
    """G = 1: the tree is one causal sequence [P; R_1]; compare with torch's
    float64 scaled_dot_product_attention (is_causal=True) and autograd."""
    tree, t = rand_inputs(8, [10], [[7]], 4, 2, 8)
    scale = 1 / math.sqrt(8)
    r = oracle.tree_attention(t, scale, fast=False)
    q = torch.tensor(np.concatenate([t["q_p"], t["q_r"]]).transpose(1, 0, 2), requires_grad=True)
    k = torch.tensor(np.concatenate([t["k_p"], t["k_r"]]).transpose(1, 0, 2), requires_grad=True)
    v = torch.tensor(np.concatenate([t["v_p"], t["v_r"]]).transpose(1, 0, 2), requires_grad=True)
    kk = k.repeat_interleave(2, dim=0)
    vv = v.repeat_interleave(2, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=scale)
    do = torch.tensor(np.concatenate([t["do_p"], t["do_r"]]).transpose(1, 0, 2))
    (o * do).sum().backward()
    o = o.detach().numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(r["o_p"], o[:10], atol=1e-12)
    np.testing.assert_allclose(r["o_r"], o[10:], atol=1e-12)
    dq = q.grad.numpy().transpose(1, 0, 2)
    dk = k.grad.numpy().transpose(1, 0, 2)
    dv = v.grad.numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(r["dq_p"], dq[:10], atol=1e-12)
    np.testing.assert_allclose(r["dq_r"], dq[10:], atol=1e-12)
    np.testing.assert_allclose(r["dk_p"], dk[:10], atol=1e-12)
    np.testing.assert_allclose(r["dk_r"], dk[10:], atol=1e-12)
    np.testing.assert_allclose(r["dv_p"], dv[:10], atol=1e-12)
    np.testing.assert_allclose(r["dv_r"], dv[10:], atol=1e-12)


def _sdpa_key_grads(q, k, v, do, scale, rows, keys):
    """dK, dV of the chosen keys from torch float64 causal
    scaled_dot_product_attention and autograd, with the upstream gradient
    zeroed outside the chosen rows (the loss is linear in dO)."""
    tq, tk, tv = (torch.tensor(x[None], requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    g = np.zeros_like(do)
    g[rows] = do[rows]
    (o * torch.tensor(g[None])).sum().backward()
    return tk.grad[0].numpy()[keys], tv.grad[0].numpy()[keys]


@pytest.mark.parametrize("rows,keys,chunk", [
    (np.arange(90), np.arange(90), 17),                          # every row and key
    (np.arange(40, 90), np.array([0, 3, 39, 40, 41, 89]), 8),    # keys on both sides of row 40
    (np.array([5, 6, 50, 89]), np.array([6, 50, 60, 2]), 3),     # sparse rows, a key no row sees
])
def test_key_gradients_match_sdpa_autograd(rows, keys, chunk):
    """oracle.causal_key_grads (prompt-key gradients from a subset of rows,
    used by the full-size GPU checks) against torch's causal
    scaled_dot_product_attention with autograd, float64."""
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal((90, 16)) for _ in range(4))
    dk, dv = oracle.causal_key_grads(q, k, v, do, 0.3, rows, keys, chunk=chunk)
    rk, rv = _sdpa_key_grads(q, k, v, do, 0.3, rows, keys)
    np.testing.assert_allclose(dk, rk, atol=1e-12)
    np.testing.assert_allclose(dv, rv, atol=1e-12)


def sum_rules(tree, t, r):
    """Per group and kv head: sum_j dK_j = 0 and sum_j dV_j = sum of dO over
    the rows of the q-heads that read that kv head.  Each softmax row's dS
    sums to zero and each row of P sums to one."""
    rep = tree.hq // tree.hkv
    worst = 0.0
    for g in range(tree.n_groups):
        p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
        b0, b1 = int(tree.group_branch_cu[g]), int(tree.group_branch_cu[g + 1])
        r0, r1 = int(tree.resp_cu[b0]), int(tree.resp_cu[b1])
        for kv in range(tree.hkv):
            hs = slice(kv * rep, (kv + 1) * rep)
            sk = r["dk_p"][p0:p1, kv].sum(0) + r["dk_r"][r0:r1, kv].sum(0)
            sv = r["dv_p"][p0:p1, kv].sum(0) + r["dv_r"][r0:r1, kv].sum(0)
            want = t["do_p"][p0:p1, hs].sum((0, 1)) + t["do_r"][r0:r1, hs].sum((0, 1))
            worst = max(worst, np.abs(sk).max(), np.abs(sv - want).max())
    return worst


def test_sum_rules():
    tree, t = rand_inputs(9, [8, 5], [[6, 0, 3], [4]], 4, 2, 5)
    r = oracle.tree_attention(t, 0.6, fast=True)
    assert sum_rules(tree, t, r) < 1e-12


def test_branch_permutation_and_duplication():
    """Permuting branches permutes their outputs and leaves the prompt
    gradients unchanged; G identical branches with dO_P = 0 give G times the
    single-branch prompt gradient (Eq. 2's sum over branches)."""
    tree, t = rand_inputs(12, [7], [[3, 5, 2]], 2, 1, 4)
    r = oracle.tree_attention(t, 0.5, fast=True)
    perm = [2, 0, 1]
    lens = [3, 5, 2]
    segs = [(int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])) for i in range(3)]
    tp = dict(t)
    for k in ("q_r", "k_r", "v_r", "do_r"):
        tp[k] = np.concatenate([t[k][segs[i][0]:segs[i][1]] for i in perm])
    tree2 = wl.Tree([7], [[lens[i] for i in perm]], 2, 1, 4, "f32")
    tp.update(wl.offsets(tree2))
    r2 = oracle.tree_attention(tp, 0.5, fast=True)
    for k in ("dk_p", "dv_p", "dq_p", "o_p", "lse_p"):
        np.testing.assert_allclose(r2[k], r[k], atol=1e-12, err_msg=k)
    for k in ("o_r", "dq_r", "dk_r", "dv_r"):
        np.testing.assert_allclose(r2[k], np.concatenate([r[k][segs[i][0]:segs[i][1]] for i in perm]),
                                   atol=1e-12, err_msg=k)
    # duplication
    one, t1 = rand_inputs(13, [6], [[4]], 2, 2, 3)
    t1["do_p"][:] = 0
    r1 = oracle.tree_attention(t1, 0.5)
    G = 5
    tg = dict(t1)
    for k in ("q_r", "k_r", "v_r", "do_r"):
        tg[k] = np.concatenate([t1[k]] * G)
    treeg = wl.Tree([6], [[4] * G], 2, 2, 3, "f32")
    tg.update(wl.offsets(treeg))
    rg = oracle.tree_attention(tg, 0.5, fast=True)
    np.testing.assert_allclose(rg["dk_p"], G * r1["dk_p"], atol=1e-12)
    np.testing.assert_allclose(rg["dv_p"], G * r1["dv_p"], atol=1e-12)


def test_prompt_gradient_is_sum_over_single_branch_trees():
    """Eq. 2: the prompt gradient of a G-branch tree equals the sum of the
    prompt gradients of the G one-branch trees (P, R_i), with dO_P counted
    once."""
    tree, t = rand_inputs(14, [9], [[4, 6, 2, 5]], 4, 2, 4)
    r = oracle.tree_attention(t, 0.4, fast=True)
    acc_k = np.zeros_like(r["dk_p"])
    acc_v = np.zeros_like(r["dv_p"])
    for i in range(4):
        r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
        ti = dict(t)
        for k in ("q_r", "k_r", "v_r", "do_r"):
            ti[k] = t[k][r0:r1]
        ti["do_p"] = t["do_p"] if i == 0 else np.zeros_like(t["do_p"])
        ti.update(wl.offsets(wl.Tree([9], [[r1 - r0]], 4, 2, 4, "f32")))
        ri = oracle.tree_attention(ti, 0.4)
        acc_k += ri["dk_p"]
        acc_v += ri["dv_p"]
        np.testing.assert_allclose(ri["o_r"], r["o_r"][r0:r1], atol=1e-13)
    np.testing.assert_allclose(acc_k, r["dk_p"], atol=1e-12)
    np.testing.assert_allclose(acc_v, r["dv_p"], atol=1e-12)


def test_pair_counter_matches_mask_and_redundancy():
    """The pair counter equals the number of visible entries of the dense
    Eq. 1 mask, and the flattened layout repeats the prompt rows once per
    branch: redundancy (G-1)/G, printed by the paper as 87.5% for G=8 and
    98.4% for G=64 (section 1)."""
    for pl, rl in (([7], [[5, 3, 4]]), ([5, 1], [[4, 0, 6], [3]]), ([6, 4], [[2, 5], []])):
        tree = wl.Tree(pl, rl, 1, 1, 1, "f32")
        c = wl.pair_counts(tree)
        assert c["tree"] == sum(int(tree_mask(p, r).sum()) for p, r in zip(pl, rl))
        flat = wl.flattened_tree(tree)
        assert wl.pair_counts(flat)["tree"] == c["flattened"]
    golden = {}
    with open(os.path.join(GOLDEN, "prompt_redundancy.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                g, pct = line.split()
                golden[int(g)] = float(pct)
    for G, pct in golden.items():
        tree = wl.Tree([4096], [[100] * G], 1, 1, 1, "f32")
        c = wl.pair_counts(tree)
        assert c["flattened_prompt"] == G * c["prefill"]
        red = 1 - c["prefill"] / c["flattened_prompt"]
        assert round(100 * red, 1) == pct


def test_useful_flops_of_the_configs():
    """4d forward + 10d backward FLOPs per valid pair and query head; the
    prompt-heavy config has fixed lengths, so its count is exact."""
    tree = wl.make_tree(wl.SPECS["prompt_heavy"])
    P, r, G = 32768, 512, 8
    pairs = P * (P + 1) // 2 + G * (r * P + r * (r + 1) // 2)
    assert wl.useful_flops(tree) == pairs * 32 * 128 * 14
    assert wl.useful_flops(tree, "fwd") == pairs * 32 * 128 * 4
