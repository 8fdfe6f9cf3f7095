"""HIP library vs the float64 oracle, element by element (GPU).

Every case runs the whole path (prefill, replay forward, replay backward
with seeds, prefill backward) through the C ABI and compares all ten outputs
by relative L2: 1e-5 for float32, 1e-2 for bf16.
"""

import numpy as np
import pytest
import torch

from shared_prompt_tree_amd import ops
from shared_prompt_tree_amd import workloads as wl
from tests._gpu import (STRATEGY_NAME, TOL, compare, host64, make_case, oracle_inputs, rel_l2,
                        run_library, run_oracle, say, strategies)

pytestmark = pytest.mark.gpu


def _case(tree, seed, value_scale=1.0, label="", zero_do_p=False):
    """Runs the library with each applicable dQ strategy (separate pass, and
    for bf16 / head_dim 128 also fused) and the oracle once.  Returns the
    problem, the inputs, {strategy: outputs} and the oracle's outputs."""
    say(f"[case] {label} groups={tree.n_groups} hq={tree.hq} hkv={tree.hkv} d={tree.d} "
        f"dtype={tree.dtype} P={tree.prompt_lens} r={tree.resp_lens}")
    prob, t = make_case(tree, seed, value_scale, zero_do_p)
    libs = {}
    for st in strategies(tree):
        prob.dq_strategy = st
        libs[st] = run_library(prob, t)
    ref = run_oracle(tree, t)
    return prob, t, libs, ref


def _compare_all(libs, ref, tol, label, tree, names=None):
    for st, lib in libs.items():
        kw = {} if names is None else {"names": names}
        compare(lib, ref, tol, label=f"{label} [{STRATEGY_NAME[st]}]", tree=tree, **kw)


def test_tiny_f32_full():
    spec = wl.SPECS["tiny"]
    tree = wl.make_tree(spec)
    _, _, libs, ref = _case(tree, spec.seed, spec.value_scale, "tiny")
    _compare_all(libs, ref, TOL["f32"], "tiny", tree)


def test_small_bf16_full():
    spec = wl.SPECS["small"]
    tree = wl.make_tree(spec)
    _, _, libs, ref = _case(tree, spec.seed, 1.0, "small")
    _compare_all(libs, ref, TOL["bf16"], "small", tree)


# Oracle-sized versions of the large shapes: the same heads, head_dim and
# length mix, fewer and shorter sequences, lengths that are not tile
# multiples.
REDUCED = {
    "prompt_heavy": wl.Tree([4097], [[300, 511, 64, 1]], 32, 8, 128, "bf16"),
    "response_heavy": wl.Tree([256, 130], [[1500, 777, 2049], [1030, 3]], 32, 8, 128, "bf16"),
    "long_mixed": wl.Tree([6000], [[1024, 1900, 3500]], 32, 8, 128, "bf16"),
}


# Replay launches of at least 1024 workgroups with 384-row tiles take the
# 12-wave forward kernel, which the large configs use for their whole replay
# forward: 64 branches of 200 tokens (3 tiles of 96 tokens x 4 packed heads
# each) x 8 head groups = 1536 workgroups; and a longer prompt with 48
# branches of 300 (4 tiles each) = 1536.  Prompts under 1024 keys are not
# cut into chunks, so the prompt column runs inside the 12-wave kernel too.
REDUCED["response_heavy 12-wave"] = wl.Tree([256], [[200] * 64], 32, 8, 128, "bf16")
REDUCED["prompt column 12-wave"] = wl.Tree([1000], [[300] * 47 + [61]], 32, 8, 128, "bf16")


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_reduced_shapes_full(name):
    tree = REDUCED[name]
    _, _, libs, ref = _case(tree, 7, 1.0, name)
    _compare_all(libs, ref, TOL["bf16"], name, tree)


EDGE = {
    "one-token prompt": wl.Tree([1], [[70, 5]], 4, 2, 128, "bf16"),
    "single branch": wl.Tree([333], [[129]], 8, 2, 128, "bf16"),
    "empty branches": wl.Tree([200, 77], [[0, 65, 0], [0]], 4, 1, 128, "bf16"),
    "group without branches": wl.Tree([90, 150], [[], [40, 300]], 4, 4, 128, "bf16"),
    "empty prompt": wl.Tree([0, 64], [[31, 200], [7]], 4, 2, 128, "bf16"),
    # no branch anywhere: replay is empty and the seeds are zero
    "no branches at all": wl.Tree([100, 64], [[], []], 4, 2, 128, "bf16"),
    # every prompt empty: replay is plain causal attention per branch
    "all prompts empty": wl.Tree([0, 0], [[10, 70], [33]], 4, 2, 64, "bf16"),
    "MHA head_dim 64": wl.Tree([300], [[100, 257]], 3, 3, 64, "bf16"),
    "GQA 7:1 (Qwen2.5-7B grouping)": wl.Tree([260], [[90, 130]], 14, 2, 128, "bf16"),
    "MQA": wl.Tree([129], [[64, 65]], 8, 1, 128, "bf16"),
    # 16 query heads packed per kv head in a 32-row block (2 tokens a block),
    # the largest packing; 12:1 packs 4 and leaves 3 head sub-groups.
    "GQA 16:1": wl.Tree([300], [[100, 65]], 32, 2, 128, "bf16"),
    "GQA 12:1 head_dim 64": wl.Tree([200], [[64, 90]], 24, 2, 64, "bf16"),
    "GQA 32:1": wl.Tree([150, 70], [[33], [0, 9]], 32, 1, 128, "bf16"),
    "f32 head_dim 128": wl.Tree([150], [[40, 90]], 2, 1, 128, "f32"),
    "f32 GQA ragged": wl.Tree([70, 33], [[5, 64, 1], [100]], 4, 2, 64, "f32"),
    # Prompt tiles split over branch ranges (partial seeds + ordered sum).
    # Split rule: target = max(longest branch, ceil(rows read by all key
    # tiles * Hkv / 512)); a group's prompt tiles get min(G, ceil(R_g /
    # target)) splits.  Here: 6 splits of one branch each.
    "split prompt tiles": wl.Tree([64], [[128] * 6], 2, 1, 64, "bf16"),
    # Group 0 (R = 669 rows, target 300): 3 splits with an empty and a 5-row
    # branch inside; group 1 is not split.
    "split uneven groups": wl.Tree([300, 40], [[100, 5, 300, 0, 64, 200], [50, 60]], 4, 2, 128,
                                   "bf16"),
    "split f32": wl.Tree([64], [[64] * 5], 2, 1, 64, "f32"),
    # Few response rows behind a long prompt: the replay query lists cut the
    # prompt column into chunks of >= 1024 keys, as many as a makespan model
    # finds worth their merge; forward partials merged by lse_merge, dQ
    # partials summed.  4 workgroups -> 8 chunks of 1024 keys here.
    "split prompt column": wl.Tree([8192], [[40, 33]], 8, 2, 128, "bf16"),
    # 264 workgroups: one more than a full round of 256 CUs; the dQ launch
    # cuts the 2048-key prompt into 2 chunks (3 rounds of half-length items
    # instead of 2 rounds of whole ones), the forward, with its larger
    # per-workgroup overhead, does not: the two launches differ.
    "split prompt column past a full round": wl.Tree([2048], [[150] * 11], 32, 8, 128, "bf16"),
    # 6 workgroups -> 4 chunks; prompts of 47 and 79 tiles, an empty branch.
    "split prompt column, two groups": wl.Tree([3000, 5000], [[17, 0, 64], [100]], 4, 2, 64,
                                               "bf16"),
    # 1 workgroup -> 4 chunks of 1024 keys, float32.
    "split prompt column f32": wl.Tree([4096], [[20]], 2, 1, 64, "f32"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    tree = EDGE[name]
    vs = 0.125 if tree.dtype == "f32" else 1.0
    _, _, libs, ref = _case(tree, 11, vs, name)
    _compare_all(libs, ref, TOL[tree.dtype], name, tree)


@pytest.mark.parametrize("dtype,scale", [("bf16", 3.0), ("f32", 3.0)])
def test_peaked_scores(dtype, scale):
    """Inputs scaled up so that scores spread over tens of log2 units: the
    running row maximum keeps growing from tile to tile, which drives the
    forward's rescaling of O and the normaliser (taken only when a row's
    maximum grows by more than 2^8)."""
    tree = wl.Tree([700, 90], [[300, 129], [260]], 8, 2, 128 if dtype == "bf16" else 64, dtype)
    _, _, libs, ref = _case(tree, 13, scale, f"peaked x{scale}")
    _compare_all(libs, ref, TOL[dtype], f"peaked {dtype}", tree)


def _key_ramp(tree, t, rising, span=0.75, qa=4.0):
    """Queries carry qa * u and keys f_j * u for one direction u per kv head,
    where key j of a row's key sequence (the prompt, then its own branch) has
    f_j rising from 0 to `span` over the longest sequence, or falling from
    it.  Rising, a row's scores grow by about qa * span * |u|^2 / sqrt(d)
    (~49 log2 units at head_dim 128) from its first keys to its last, so the
    forward's running maximum keeps growing past its lazy-rescale threshold;
    falling, later probabilities underflow instead.  The softmax still
    spreads over dozens of keys."""
    gen = torch.Generator().manual_seed(29)
    dev = t["q_p"].device
    grp = tree.hq // tree.hkv
    u = torch.randn(tree.hkv, tree.d, generator=gen).to(dev)
    longest = max(p + max(rs, default=0) for p, rs in zip(tree.prompt_lens, tree.resp_lens))

    def weight(pos):
        f = torch.tensor(pos, dtype=torch.float32, device=dev) / max(longest - 1, 1) * span
        return f if rising else span - f

    pos_p, pos_r = [], []
    for p, rs in zip(tree.prompt_lens, tree.resp_lens):
        pos_p += list(range(p))
        for r in rs:
            pos_r += [p + j for j in range(r)]
    for name, pos in (("k_p", pos_p), ("k_r", pos_r)):
        k = t[name]
        if k.shape[0]:
            k.copy_((weight(pos)[:, None, None] * u[None] + 0.5 * k.float()).to(k.dtype))
    uq = u.repeat_interleave(grp, dim=0)
    for name in ("q_p", "q_r"):
        q = t[name]
        if q.shape[0]:
            q.copy_((qa * uq[None] + 0.5 * q.float()).to(q.dtype))


@pytest.mark.parametrize("dtype,rising", [("bf16", True), ("bf16", False), ("f32", True)])
def test_key_ramp_scores(dtype, rising):
    """Scores that rise (or fall) steadily along every row's keys: the rising
    case drives the forward's rescale of O and the normaliser many times per
    row (its running maximum grows by more than 2^8 again and again), on
    prompt rows and on response rows behind the prompt column.

    Gated: the forward outputs and dV.  dQ and dK are not: with keys sharing
    one large direction, dS summing to zero along each row cancels that
    direction in dQ (and the queries' in dK), so bf16 rounding of dS - the
    operand every bf16 backward multiplies with - stands in front of a small
    remainder.  Their error here (up to ~3e-2 on a segment) is that input's
    conditioning, not a rescale path: the backward kernels have none, they
    use the final LSE.  Backward parity under peaked scores is covered by
    test_peaked_scores."""
    tree = wl.Tree([700, 90], [[300, 129], [260]], 8, 2, 128 if dtype == "bf16" else 64, dtype)
    label = f"key ramp {'rising' if rising else 'falling'} {dtype}"
    say(f"[case] {label}")
    prob, t = make_case(tree, 17, 0.25 if dtype == "f32" else 1.0)
    _key_ramp(tree, t, rising)
    libs = {}
    for st in strategies(tree):
        prob.dq_strategy = st
        libs[st] = run_library(prob, t)
    ref = run_oracle(tree, t)
    _compare_all(libs, ref, TOL[dtype], label, tree,
                 names=("o_p", "lse_p", "o_r", "lse_r", "dv_p", "dv_r"))


def _random_tree(seed):
    """A small random batch of trees: 1-3 groups, 0-6 branches each,
    prompts of 0-300 tokens and branches of 0-260 (zero-length ones
    included), a random GQA ratio, head_dim and dtype."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 3]))
    hq = hkv * int(rng.choice([1, 2, 3, 4, 6, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    ng = int(rng.integers(1, 4))
    prompts = [0 if rng.random() < 0.15 else int(x) for x in rng.integers(1, 301, ng)]
    branches = []
    for _ in range(ng):
        nb = int(rng.integers(0, 7))
        lens = rng.integers(0, 261, nb)
        lens[rng.random(nb) < 0.15] = 0
        branches.append([int(x) for x in lens])
    return wl.Tree(prompts, branches, hq, hkv, d, dtype)


@pytest.mark.parametrize("seed", range(12))
def test_random_trees(seed):
    tree = _random_tree(1000 + seed)
    vs = 0.125 if tree.dtype == "f32" else 1.0
    _, _, libs, ref = _case(tree, 50 + seed, vs, f"random {seed}")
    _compare_all(libs, ref, TOL[tree.dtype], f"random {seed}", tree)


def _random_split_tree(seed):
    """Random trees that take the split paths: a long prompt (2048-4096
    tokens) with a few short branches cuts the replay prompt column into
    chunks; a short prompt (16-128) with many branches splits the prompt
    key tiles over branch ranges."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    if seed % 2 == 0:
        prompts = [int(rng.integers(2048, 4097))]
        branches = [[int(x) for x in rng.integers(1, 101, int(rng.integers(1, 4)))]]
    else:
        prompts = [int(x) for x in rng.integers(16, 129, int(rng.integers(1, 3)))]
        branches = [[int(x) for x in rng.integers(64, 301, int(rng.integers(6, 13)))]
                    for _ in prompts]
    return wl.Tree(prompts, branches, hq, hkv, d, "bf16")


@pytest.mark.parametrize("seed", range(4))
def test_random_split_trees(seed):
    tree = _random_split_tree(2000 + seed)
    _, _, libs, ref = _case(tree, 70 + seed, 1.0, f"random split {seed}")
    _compare_all(libs, ref, TOL["bf16"], f"random split {seed}", tree)


@pytest.mark.parametrize("splits", [2, 5, 64])
def test_forced_prompt_col_splits(splits):
    """Forced prompt-column chunk counts, up to more chunks than the 47
    prompt tiles (the extra chunks hold no prompt key: empty partial states,
    the identity of the merge)."""
    tree = wl.Tree([3000], [[100, 37]], 8, 2, 128, "bf16")
    prob, t = make_case(tree, 17)
    prob.prompt_col_splits = splits
    lib = run_library(prob, t)
    ref = run_oracle(tree, t)
    compare(lib, ref, TOL["bf16"], label=f"forced S={splits}", tree=tree)


@pytest.mark.parametrize("rows", [1, 150, 10 ** 6])
def test_forced_prompt_tile_split_rows(rows):
    """Forced prompt-tile split targets: one branch per range (1), ranges of
    a few branches (150), no split (10^6); uneven branches with an empty one,
    two groups."""
    tree = wl.Tree([300, 40], [[100, 5, 300, 0, 64, 200], [50, 60]], 4, 2, 128, "bf16")
    prob, t = make_case(tree, 19)
    prob.prompt_tile_split_rows = rows
    lib = run_library(prob, t)
    ref = run_oracle(tree, t)
    compare(lib, ref, TOL["bf16"], label=f"forced split rows {rows}", tree=tree)


def test_zero_prompt_upstream_gradient():
    """dO_P = 0: dQ_P must be exactly zero; everything else still matches."""
    tree = wl.Tree([500], [[200, 64]], 8, 2, 128, "bf16")
    _, _, libs, ref = _case(tree, 5, 1.0, "dO_P=0", zero_do_p=True)
    for lib in libs.values():
        assert float(lib["dq_p"].abs().max()) == 0.0
    names = [n for n in ("o_p", "lse_p", "o_r", "lse_r", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")]
    _compare_all(libs, ref, TOL["bf16"], "dO_P=0", tree, names=names)


@pytest.mark.parametrize("strategy", [ops.DQ_SEPARATE, ops.DQ_FUSED])
def test_detached_prompt_seeds(strategy):
    """With no seeds, prefill backward returns only the prompt rows' own
    term, i.e. the gradients of a tree whose groups have no branch; the
    response rows' dQ still includes their prompt column (the fused kernel
    walks the prompt tiles for it without writing seeds)."""
    tree = wl.Tree([300, 129], [[100, 64], [50]], 4, 2, 128, "bf16")
    prob, t = make_case(tree, 9, dq_strategy=strategy)
    lib = run_library(prob, t, seeds=False)
    prompt_only = wl.Tree(tree.prompt_lens, [[] for _ in tree.prompt_lens], 4, 2, 128, "bf16")
    ti = {k: v for k, v in t.items() if k.endswith("_p")}
    for k in ("q_r", "k_r", "v_r", "do_r"):
        ti[k] = t[k][:0]
    ref = run_oracle(prompt_only, ti)
    label = f"detached [{STRATEGY_NAME[strategy]}]"
    compare(lib, ref, TOL["bf16"], names=("dq_p", "dk_p", "dv_p"), label=label, tree=tree)
    full = run_oracle(tree, t)
    compare(lib, full, TOL["bf16"], names=("o_r", "lse_r", "dq_r", "dk_r", "dv_r"),
            label=label, tree=tree)


def test_detached_prompt_seeds_split():
    """Detached prompt where the prompt tiles would be split."""
    tree = wl.Tree([64], [[128] * 6], 2, 1, 64, "bf16")
    prob, t = make_case(tree, 10)
    lib = run_library(prob, t, seeds=False)
    prompt_only = wl.Tree(tree.prompt_lens, [[]], 2, 1, 64, "bf16")
    ti = {k: v for k, v in t.items() if k.endswith("_p")}
    for k in ("q_r", "k_r", "v_r", "do_r"):
        ti[k] = t[k][:0]
    ref = run_oracle(prompt_only, ti)
    compare(lib, ref, TOL["bf16"], names=("dq_p", "dk_p", "dv_p"), label="detached split",
            tree=tree)


def test_deterministic():
    """Separate dQ pass, no atomics on any output: two runs are
    bit-identical."""
    for tree in (wl.Tree([700], [[300, 129, 64]], 8, 2, 128, "bf16"),
                 wl.Tree([64], [[128] * 6], 2, 1, 64, "bf16"),  # split prompt tiles
                 wl.Tree([8192], [[40, 33]], 8, 2, 128, "bf16")):  # split prompt column
        prob, t = make_case(tree, 3, dq_strategy=ops.DQ_SEPARATE)
        a = run_library(prob, t)
        b = run_library(prob, t)
        for k, v in a.items():
            if v is not None:
                assert torch.equal(v, b[k]), k


def test_deterministic_fused_except_dq():
    """Fused dQ: dQ is summed with atomics (rounding may differ between
    runs); every other output stays bit-identical."""
    for tree in (wl.Tree([700], [[300, 129, 64]], 8, 2, 128, "bf16"),
                 wl.Tree([64], [[128] * 6], 2, 1, 128, "bf16")):  # split prompt tiles
        prob, t = make_case(tree, 3, dq_strategy=ops.DQ_FUSED)
        a = run_library(prob, t)
        b = run_library(prob, t)
        for k, v in a.items():
            if v is not None and not k.startswith("dq"):
                assert torch.equal(v, b[k]), k
            elif v is not None:
                assert rel_l2(host64(v), host64(b[k])) < 1e-3, k


def test_lse_merge_matches_oracle():
    import oracle
    g = torch.Generator(device="cuda").manual_seed(4)
    S, rows, H, d = 5, 333, 6, 128
    o = torch.randn(S, rows, H, d, device="cuda", generator=g)
    lse = torch.randn(S, H, rows, device="cuda", generator=g) * 4
    lse[1, :, :50] = float("-inf")  # empty parts
    lse[:, 2, 7] = float("-inf")    # a row where every part is empty
    for dt, tol in ((torch.float32, 1e-6), (torch.bfloat16, 1e-2)):
        mo, ml = ops.lse_merge(o, lse, out_dtype=dt)
        torch.cuda.synchronize()
        ro, rl = oracle.lse_merge(host64(o), host64(lse))
        assert float(mo[7, 2].abs().max()) == 0.0 and float(ml[2, 7]) == float("-inf")
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(host64(ml)), fin)
        assert rel_l2(host64(ml)[fin], rl[fin]) < 1e-6
        assert rel_l2(host64(mo), ro) < tol
