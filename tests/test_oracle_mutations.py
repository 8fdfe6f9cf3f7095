"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only; the real oracle is never modified)."""

import math
import os
import types

import numpy as np
import pytest

from tests._dense import OUTPUTS, dense_reference, rand_inputs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "tree_attention.py")

MUTATIONS = {
    "diagonal excluded": ("invisible = np.arange(kmax)[None, :] > r[:, None]",
                          "invisible = np.arange(kmax)[None, :] >= r[:, None]"),
    "scale dropped from scores": ("s = scale * (xq[r] @ xk[:kmax].T)",
                                  "s = (xq[r] @ xk[:kmax].T)"),
    "scale dropped from dK": ("dk[:kmax] += scale * (ds.T @ xq[r])",
                              "dk[:kmax] += (ds.T @ xq[r])"),
    "scale dropped from dQ": ("dq[a:a + len(r)] = scale * (ds @ xk[:kmax])",
                              "dq[a:a + len(r)] = (ds @ xk[:kmax])"),
    "sign of D in dS": ("ds = p * (dp - dd)", "ds = p * (dp + dd)"),
    "D term dropped": ("ds = p * (dp - dd)", "ds = p * dp"),
    "max dropped from LSE": ("lse[a:a + len(r)] = m[:, 0] + np.log(ell[:, 0])",
                             "lse[a:a + len(r)] = np.log(ell[:, 0])"),
    "GQA head mapping": ("return (h * hkv) // hq", "return h % hkv"),
    "dO_P given to every branch": ("dop if first else np.zeros_like(dop)", "dop"),
    "later branches overwrite the prompt gradient": ('res["dk_p"] += dk[:plen]',
                                                     'res["dk_p"] = dk[:plen]'),
    "response dV not summed over q-heads": ('out["dv_r"][r0:r1, kv] += dv',
                                            'out["dv_r"][r0:r1, kv] = dv'),
    "merge weight sign": ("w = np.exp(lse_parts - lse[None])",
                          "w = np.exp(lse[None] - lse_parts)"),
    "merge normaliser": ("lse = np.logaddexp.reduce(lse_parts, axis=0)",
                         "lse = np.max(lse_parts, axis=0)"),
    # causal_key_grads (prompt-key gradients from a subset of rows)
    "key grads: diagonal excluded": (
        "tail[np.arange(int(r[0]) + 1, kmax)[None, :] > r[:, None]] = -np.inf",
        "tail[np.arange(int(r[0]) + 1, kmax)[None, :] >= r[:, None]] = -np.inf"),
    "key grads: D term dropped": ("dsk = pk * (g @ xv[keys].T - dd)",
                                  "dsk = pk * (g @ xv[keys].T)"),
    "key grads: scale dropped from dK": ("dk += scale * (dsk.T @ xq[r])",
                                         "dk += (dsk.T @ xq[r])"),
    "key grads: scores not scaled": ("s *= scale", "s *= 1.0"),
    "key grads: wrong key column": ("pk[:, seen] = s[:, keys[seen]]",
                                    "pk[:, seen] = s[:, keys[seen] - 1]"),
}


def load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pins_hold(mod):
    """The dense-mask comparison and an LSE-merge split check."""
    for seed, (pl, rl, hq, hkv, d) in enumerate(
            [([5, 1], [[4, 0, 6], [3]], 4, 2, 8), ([7], [[5, 3, 4]], 2, 1, 4)]):
        tree, t = rand_inputs(300 + seed, pl, rl, hq, hkv, d)
        scale = 1 / math.sqrt(d)
        ref = dense_reference(tree, t, scale)
        for fast in (False, True):
            with np.errstate(all="ignore"):
                try:
                    got = mod.tree_attention(t, scale, fast=fast)
                except (AssertionError, ValueError, FloatingPointError):
                    return False
            for k in OUTPUTS:
                if not np.allclose(got[k], ref[k], rtol=1e-9, atol=1e-10):
                    return False
    # prompt-key gradients from a subset of rows against torch autograd
    from tests.test_oracle_pins import _sdpa_key_grads
    rng = np.random.default_rng(2)
    q, k, v, do = (rng.standard_normal((30, 4)) for _ in range(4))
    rows, keys = np.arange(9, 30), np.array([0, 8, 9, 10, 29])
    with np.errstate(all="ignore"):
        dk, dv = mod.causal_key_grads(q, k, v, do, 0.7, rows, keys, chunk=4)
    rk, rv = _sdpa_key_grads(q, k, v, do, 0.7, rows, keys)
    if not (np.allclose(dk, rk, atol=1e-10) and np.allclose(dv, rv, atol=1e-10)):
        return False
    # merge check: two halves of a key set merge to the whole
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((6, 4)) for _ in range(3))
    s = q @ k.T
    full_l = np.log(np.exp(s).sum(1))
    full_o = (np.exp(s) / np.exp(s).sum(1, keepdims=True)) @ v
    parts_o, parts_l = [], []
    for sl in (slice(0, 2), slice(2, 6)):
        e = np.exp(s[:, sl])
        parts_o.append((e / e.sum(1, keepdims=True)) @ v[sl])
        parts_l.append(np.log(e.sum(1)))
    o, lse = mod.lse_merge(np.stack(parts_o)[:, :, None], np.stack(parts_l)[:, None])
    return np.allclose(o[:, 0], full_o, atol=1e-12) and np.allclose(lse[0], full_l, atol=1e-12)


def test_unmutated_copy_passes():
    src = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert pins_hold(mod)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    old, new = MUTATIONS[name]
    assert not pins_hold(load_mutant(old, new)), f"pins missed: {name}"
