"""Seeded synthetic replay trees and the valid-pair counter.

This module holds no attention arithmetic.  It draws response lengths and
input tensors, packs them, and counts the (query row, key) pairs that the
tree mask leaves visible.  Tests feed the same tensors to the float64 oracle
and to the HIP library; the benchmark uses the pair counts for its useful
FLOP numerator.

Workload shapes follow the AugTree paper ("Splitting Prompt Prefill from
Response Replay for Context-Parallel Long-Context LLM Post-Training"): a group
is one prompt with G sampled responses (section 2.1), prompt/response ratios
range from prompt-heavy long-document QA to response-heavy creative writing
(section 1, property (2); Fig. 1), and the attention shape is 32 query / 8 kv
heads of width 128 as in the Llama-3.1-8B runs (section 4.1).  The paper's
datasets are not used: values are i.i.d. normal draws.

Recipe:
* lengths: ``numpy.random.default_rng(seed)``; uniform lengths are
  ``integers(lo, hi + 1)``, log-uniform lengths are
  ``rint(exp(uniform(ln lo, ln hi)))`` clipped to [lo, hi], drawn group-major.
* tensors: one ``torch.Generator(device).manual_seed(seed)``; the packed
  tensors q_p, k_p, v_p, q_r, k_r, v_r, do_p, do_r are drawn in that order as
  float32 standard normals, in slices of at most ``DRAW_CHUNK`` elements along
  the token axis, times the value scale, then rounded to the I/O dtype
  (round to nearest even for bf16).  The same seed gives the same tensors on
  the same device type; CPU and GPU draws differ.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

DRAW_CHUNK = 1 << 26  # elements per generator call


@dataclass(frozen=True)
class Spec:
    """A workload recipe: shapes, length distribution, dtype and seed."""

    name: str
    n_groups: int
    hq: int
    hkv: int
    d: int
    prompt_len: int
    g: int
    resp: tuple  # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    dtype: str  # "f32" | "bf16"
    value_scale: float
    seed: int
    note: str = ""


SPECS = {
    "tiny": Spec("tiny", 1, 1, 1, 64, 128, 4, ("fixed", 64), "f32", 1.0 / 8.0,
                 20261203, "correctness only"),
    "small": Spec("small", 2, 8, 2, 128, 2048, 8, ("uniform", 256, 1024), "bf16", 1.0,
                  20261204),
    "prompt_heavy": Spec("prompt_heavy", 1, 32, 8, 128, 32768, 8, ("fixed", 512), "bf16",
                         1.0, 20261205, "long-document QA shape, prompt/response = 64"),
    "response_heavy": Spec("response_heavy", 4, 32, 8, 128, 256, 64,
                           ("uniform", 2048, 8192), "bf16", 1.0, 20261206,
                           "creative-writing shape, prompt/response ~ 0.05"),
    "long_mixed": Spec("long_mixed", 1, 32, 8, 128, 131072, 16,
                       ("loguniform", 1024, 16384), "bf16", 1.0, 20261207,
                       "one GPU's share of a long prompt"),
}
ORDER = ["tiny", "small", "prompt_heavy", "response_heavy", "long_mixed"]


@dataclass
class Tree:
    """Packed lengths of a batch of replay trees and their offset arrays."""

    prompt_lens: list
    resp_lens: list  # one list of branch lengths per group
    hq: int
    hkv: int
    d: int
    dtype: str
    prompt_cu: np.ndarray = field(init=False)
    group_branch_cu: np.ndarray = field(init=False)
    resp_cu: np.ndarray = field(init=False)

    def __post_init__(self):
        assert len(self.prompt_lens) == len(self.resp_lens)
        self.prompt_cu = np.concatenate([[0], np.cumsum(self.prompt_lens)]).astype(np.int32)
        counts = [len(r) for r in self.resp_lens]
        self.group_branch_cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        flat = [x for r in self.resp_lens for x in r]
        self.resp_cu = np.concatenate([[0], np.cumsum(flat)]).astype(np.int32)

    @property
    def n_groups(self):
        return len(self.prompt_lens)

    @property
    def n_branches(self):
        return int(self.group_branch_cu[-1])

    @property
    def prompt_tokens(self):
        return int(self.prompt_cu[-1])

    @property
    def resp_tokens(self):
        return int(self.resp_cu[-1])

    @property
    def max_prompt_len(self):
        return max(self.prompt_lens) if self.prompt_lens else 0

    @property
    def max_resp_len(self):
        flat = [x for r in self.resp_lens for x in r]
        return max(flat) if flat else 0


def draw_lengths(spec: Spec):
    rng = np.random.default_rng(spec.seed)
    resp = []
    for _ in range(spec.n_groups):
        kind = spec.resp[0]
        if kind == "fixed":
            r = [int(spec.resp[1])] * spec.g
        elif kind == "uniform":
            r = [int(x) for x in rng.integers(spec.resp[1], spec.resp[2] + 1, size=spec.g)]
        elif kind == "loguniform":
            lo, hi = spec.resp[1], spec.resp[2]
            x = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=spec.g)))
            r = [int(v) for v in np.clip(x, lo, hi)]
        else:
            raise ValueError(kind)
        resp.append(r)
    return [spec.prompt_len] * spec.n_groups, resp


def make_tree(spec: Spec) -> Tree:
    p, r = draw_lengths(spec)
    return Tree(p, r, spec.hq, spec.hkv, spec.d, spec.dtype)


def shrink(spec: Spec, **kw) -> Spec:
    """A smaller variant of a recipe (for oracle-sized parity cases)."""
    return replace(spec, **kw)


TENSOR_ORDER = ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r")


def tensor_shapes(tree: Tree):
    tp, tr = tree.prompt_tokens, tree.resp_tokens
    return {
        "q_p": (tp, tree.hq, tree.d), "k_p": (tp, tree.hkv, tree.d),
        "v_p": (tp, tree.hkv, tree.d), "q_r": (tr, tree.hq, tree.d),
        "k_r": (tr, tree.hkv, tree.d), "v_r": (tr, tree.hkv, tree.d),
        "do_p": (tp, tree.hq, tree.d), "do_r": (tr, tree.hq, tree.d),
    }


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_tensors(tree: Tree, seed: int, device="cpu", value_scale=1.0):
    """Draw the eight packed input tensors on ``device`` (see module recipe)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = {}
    dt = torch_dtype(tree.dtype)
    for name in TENSOR_ORDER:
        shape = tensor_shapes(tree)[name]
        dst = torch.empty(shape, dtype=dt, device=device)
        row = max(1, shape[1] * shape[2])
        step = max(1, DRAW_CHUNK // row)
        for a in range(0, shape[0], step):
            b = min(shape[0], a + step)
            x = torch.randn((b - a,) + shape[1:], generator=gen, dtype=torch.float32,
                            device=device)
            if value_scale != 1.0:
                x.mul_(value_scale)
            dst[a:b].copy_(x)
        out[name] = dst
    return out


def offsets(tree: Tree):
    return {"prompt_cu": tree.prompt_cu, "group_branch_cu": tree.group_branch_cu,
            "resp_cu": tree.resp_cu}


# ---------------------------------------------------------------- pair counts

def pair_counts(tree: Tree):
    """Valid (query row, key) pairs per query head under the tree mask.

    prefill: prompt rows over the prompt, causal with diagonal, P(P+1)/2.
    replay_prompt: every response row sees the whole prompt, r_i * P.
    replay_own: response rows over their own branch, r_i(r_i+1)/2.
    flattened: the same work when each (P, R_i) pair is its own causal
    sequence, (P + r_i)(P + r_i + 1)/2 per branch (P(P+1)/2 for a group with
    no branch); flattened_prompt counts its prompt-row part, G * P(P+1)/2.
    """
    c = dict(prefill=0, replay_prompt=0, replay_own=0, flattened=0, flattened_prompt=0)
    for p, rs in zip(tree.prompt_lens, tree.resp_lens):
        c["prefill"] += p * (p + 1) // 2
        if not rs:
            c["flattened"] += p * (p + 1) // 2
            c["flattened_prompt"] += p * (p + 1) // 2
        for r in rs:
            c["replay_prompt"] += r * p
            c["replay_own"] += r * (r + 1) // 2
            c["flattened"] += (p + r) * (p + r + 1) // 2
            c["flattened_prompt"] += p * (p + 1) // 2
    c["tree"] = c["prefill"] + c["replay_prompt"] + c["replay_own"]
    return c


FWD_FLOPS_PER_PAIR_PER_DIM = 4   # S = Q K^T and O = P V
BWD_FLOPS_PER_PAIR_PER_DIM = 10  # S recompute, dP, dV, dK, dQ


def useful_flops(tree: Tree, part="fwdbwd"):
    """Tree-masked useful FLOPs over all query heads (4d fwd, 10d bwd)."""
    per = {"fwd": FWD_FLOPS_PER_PAIR_PER_DIM, "bwd": BWD_FLOPS_PER_PAIR_PER_DIM,
           "fwdbwd": FWD_FLOPS_PER_PAIR_PER_DIM + BWD_FLOPS_PER_PAIR_PER_DIM,
           "fwdbwd_norecompute": 12}[part]
    return pair_counts(tree)["tree"] * tree.hq * tree.d * per


def flattened_tree(tree: Tree) -> Tree:
    """The per-branch flattened layout: one prompt-only group per (P, R_i)."""
    plens = []
    for p, rs in zip(tree.prompt_lens, tree.resp_lens):
        if not rs:
            plens.append(p)
        for r in rs:
            plens.append(p + r)
    return Tree(plens, [[] for _ in plens], tree.hq, tree.hkv, tree.d, tree.dtype)


def flatten_tensors(tree: Tree, t):
    """Pack [P; R_i] for every branch into prompt-side tensors of
    ``flattened_tree(tree)`` (pure data movement)."""
    import torch

    parts = {k: [] for k in ("q", "k", "v", "do")}
    for g, rs in enumerate(tree.resp_lens):
        p0, p1 = int(tree.prompt_cu[g]), int(tree.prompt_cu[g + 1])
        b0 = int(tree.group_branch_cu[g])
        if not rs:
            for k in parts:
                parts[k].append(t[k + "_p"][p0:p1])
        for j in range(len(rs)):
            r0, r1 = int(tree.resp_cu[b0 + j]), int(tree.resp_cu[b0 + j + 1])
            for k in parts:
                parts[k].append(t[k + "_p"][p0:p1])
                parts[k].append(t[k + "_r"][r0:r1])
    return {k + "_p": torch.cat(v) for k, v in parts.items()}


# ------------------------------------------------------------ work balance
#
# Replay units and grid assignment (AugTree paper, section 3.4, Eq. 6): the
# planner places units on lanes so as to minimise the largest lane load,
# exactly for few units and by largest-first greedy balancing otherwise.  On
# one GPU the lanes are compute units and the units are the workgroup items
# of a launch; the device work lists are ordered largest first, and the
# hardware dispatcher hands the next item to the next free compute unit,
# which is that greedy rule applied online.  These helpers evaluate the
# greedy placement on the host from item costs, to measure how far a launch
# is from perfect balance.

def assign_grid(costs, lanes):
    """Largest-first greedy placement of units with the given costs onto
    `lanes` lanes: each unit, in order of decreasing cost, goes to the lane
    with the smallest load.  Returns the lane loads."""
    import heapq

    loads = [(0.0, j) for j in range(lanes)]
    out = [0.0] * lanes
    for c in sorted(costs, reverse=True):
        load, j = heapq.heappop(loads)
        out[j] = load + c
        heapq.heappush(loads, (out[j], j))
    return out


def replay_items(tree: Tree, kind: str, hp: int):
    """Costs of the replay work items of one head group (query-stationary
    "dq": 64-key steps of each 256-row query tile, prompt column plus the
    causal part of its branch) or one kv head (key-stationary "dkv": 32-row
    query blocks each 256-key tile reads; a prompt tile reads every response
    row of its group).  Unsplit launches."""
    rows_tile = 256 // hp  # tokens per 256-row query tile
    out = []
    for p, rs in zip(tree.prompt_lens, tree.resp_lens):
        if kind == "dkv":
            rows = sum(rs)
            out += [rows * hp / 32] * (-(-p // 256))
            for r in rs:
                out += [(r - 256 * t) * hp / 32 for t in range(-(-r // 256))]
        else:
            for r in rs:
                for q0 in range(0, r, rows_tile):
                    out.append(-(-p // 64) + -(-min(r, q0 + rows_tile) // 64))
    return out


def schedule_balance(tree: Tree, kind: str, lanes: int = 32):
    """Largest-first makespan of the replay items of one head group or kv
    head on the `lanes` compute units of one XCD, over their mean load (1 is
    perfect balance; no placement can beat max(1, longest item / mean))."""
    hp = 1
    while hp < 16 and (tree.hq // tree.hkv) % (2 * hp) == 0:
        hp *= 2
    items = replay_items(tree, kind, hp)
    if not items:
        return 1.0
    loads = assign_grid(items, lanes)
    return max(loads) / (sum(items) / lanes)
