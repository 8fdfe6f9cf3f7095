"""Plain float64 oracle of shared-prompt tree attention, forward and backward.

TEST INFRASTRUCTURE.  This module is the checker that the HIP library is
compared against.  It is imported only by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``.  It
shares no code, tables or constants with the HIP path.

What it computes (source: "Splitting Prompt Prefill from Response Replay for
Context-Parallel Long-Context LLM Post-Training", the AugTree paper):

* Attention is O = softmax(Q K^T / sqrt(D_h) + M) V per head, with M marking
  invalid query/key positions (section 2.2, "Attention as block
  interactions").
* A replay tree is one shared prompt P and G response branches R_i
  (section 3.1).  Token t of branch i sees the whole prompt plus its own
  prefix and never a sibling branch (section 3.2, Eq. 1).
* Standard context parallelism flattens each (P, R_i) pair into one
  independent causal sequence (section 2.1, "Replay tree"; section 4.1,
  baseline MegaN).  The paper states that its prompt-once execution computes
  the same attention result (section 3.3, "Common tile semantics"; section
  4.5, "Correctness") with exact gradients (section 3.2, "Exact many-to-one
  backward", Eq. 2).  So the oracle is that plain definition: every (P, R_i)
  pair is run as one causal sequence, and the results are scattered back to
  the tree tensors.  Prompt-side gradients are the sum over all branches,
  which is Eq. 2 plus the prompt rows' own term.

Readings where the paper is silent (all listed with reasons in the design
notes of the repository):

* The causal mask includes the diagonal: the fallback plan runs each
  (P, R_i) pair under the standard causal mask (section 3.4, "Plan space").
* Query head h uses kv head floor(h * Hkv / Hq) (contiguous GQA grouping).
* The upstream gradient of the prompt rows, dO_P, is given to the first
  branch of the group only.  The backward pass is linear in dO, so this is
  the same as any split of dO_P over the branches.
* LSE is the natural log of sum_j exp(scale * q . k_j) over visible keys.

Layout: packed, token-major.  Prompt tensors are [sum P_g, H, d], response
tensors are [sum T_g, H, d], LSE arrays are [Hq, tokens].
"""

from __future__ import annotations

import os

import numpy as np

__all__ = [
    "causal_key_grads",
    "causal_unit",
    "lse_merge",
    "tree_attention",
    "tree_attention_parallel",
]


def causal_unit(xq, xk, xv, do, scale, rows=None, chunk=512):
    """Causal attention forward and backward over one flattened sequence.

    xq, xk, xv, do: float64 arrays of shape [L, d] (one query head and the kv
    head it reads).  Row t sees keys 0..t, diagonal included.

    rows: sorted int array of the query rows to evaluate (default: all).  The
    returned dK/dV are sums over those rows only, so dK[j] and dV[j] are the
    full gradient only when ``rows`` holds every row t >= j.

    Returns (o [n, d], lse [n], dq [n, d], dk [L, d], dv [L, d]) for the n
    selected rows.  Each chunk of rows sees its whole key range at once:
    there is no online softmax here.

    Backward of O = P V with P = softmax(S), S = scale * Q K^T, for the loss
    sum(dO * O): D = rowsum(dO * O), dP = dO V^T, dS = P * (dP - D),
    dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO.
    """
    L, d = xq.shape
    if rows is None:
        rows = np.arange(L)
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    o = np.zeros((n, d))
    lse = np.zeros(n)
    dq = np.zeros((n, d))
    dk = np.zeros((L, d))
    dv = np.zeros((L, d))
    for a in range(0, n, chunk):
        r = rows[a:a + chunk]
        kmax = int(r[-1]) + 1
        s = scale * (xq[r] @ xk[:kmax].T)
        invisible = np.arange(kmax)[None, :] > r[:, None]
        s[invisible] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        ell = e.sum(axis=1, keepdims=True)
        p = e / ell
        o_c = p @ xv[:kmax]
        o[a:a + len(r)] = o_c
        lse[a:a + len(r)] = m[:, 0] + np.log(ell[:, 0])
        g = do[r]
        dd = (g * o_c).sum(axis=1, keepdims=True)
        dp = g @ xv[:kmax].T
        ds = p * (dp - dd)
        dq[a:a + len(r)] = scale * (ds @ xk[:kmax])
        dk[:kmax] += scale * (ds.T @ xq[r])
        dv[:kmax] += p.T @ g
    return o, lse, dq, dk, dv


def causal_key_grads(xq, xk, xv, do, scale, rows, keys, chunk=256):
    """Gradient of sum(dO * O) with respect to chosen keys and values of one
    flattened causal sequence, from chosen query rows.

    The definitions are those of ``causal_unit``: row t sees keys 0..t
    (diagonal included), P = softmax(scale * Q K^T) over that whole range,
    O = P V, D = rowsum(dO * O), dS = P * (dO V^T - D).  Only the columns in
    ``keys`` of dP and dS are formed:
        dK[j] = scale * sum_{t in rows} dS[t, j] q_t,
        dV[j] = sum_{t in rows} P[t, j] dO_t.
    Each chunk of rows still evaluates every row's softmax over its whole key
    range (the normaliser and D need all of it); there is no online softmax.

    xq, xk, xv, do: float64 [L, d]; rows: sorted query rows; keys: key
    indices.  Returns (dk [len(keys), d], dv [len(keys), d]), sums over
    ``rows`` only (the full gradient of key j when rows holds every t >= j).
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    d = xq.shape[1]
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        kmax = int(r[-1]) + 1
        s = xq[r] @ xk[:kmax].T
        s *= scale
        # keys after a row are hidden; only columns past the chunk's first
        # row can be
        tail = s[:, int(r[0]) + 1:]
        tail[np.arange(int(r[0]) + 1, kmax)[None, :] > r[:, None]] = -np.inf
        m = s.max(axis=1, keepdims=True)
        s -= m
        np.exp(s, out=s)
        s /= s.sum(axis=1, keepdims=True)  # s now holds P
        g = do[r]
        dd = (g * (s @ xv[:kmax])).sum(axis=1, keepdims=True)  # D = rowsum(dO * O)
        seen = keys < kmax
        pk = np.zeros((len(r), len(keys)))
        pk[:, seen] = s[:, keys[seen]]
        dsk = pk * (g @ xv[keys].T - dd)
        dk += scale * (dsk.T @ xq[r])
        dv += pk.T @ g
    return dk, dv


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h, hq, hkv):
    """Contiguous GQA grouping: query head h reads kv head floor(h*Hkv/Hq)."""
    return (h * hkv) // hq


def _group_head_unit(t, g, h, scale, fast, chunk, check_prompt_rows):
    """All branches of group g for query head h.  Returns partial outputs."""
    hq = t["q_p"].shape[1]
    hkv = t["k_p"].shape[1]
    kv = kv_head_of(h, hq, hkv)
    p0, p1 = int(t["prompt_cu"][g]), int(t["prompt_cu"][g + 1])
    plen = p1 - p0
    b0, b1 = int(t["group_branch_cu"][g]), int(t["group_branch_cu"][g + 1])
    d = t["q_p"].shape[2]
    qp = _as64(t["q_p"][p0:p1, h])
    kp = _as64(t["k_p"][p0:p1, kv])
    vp = _as64(t["v_p"][p0:p1, kv])
    dop = _as64(t["do_p"][p0:p1, h])
    res = {
        "o_p": np.zeros((plen, d)), "lse_p": np.zeros(plen), "dq_p": np.zeros((plen, d)),
        "dk_p": np.zeros((plen, d)), "dv_p": np.zeros((plen, d)),
        "branches": [],
    }
    if b1 == b0:
        # A prompt with no branch still has its prefill and prefill backward.
        o, lse, dq, dk, dv = causal_unit(qp, kp, vp, dop, scale, chunk=chunk)
        res.update(o_p=o, lse_p=lse, dq_p=dq, dk_p=dk, dv_p=dv)
        return res
    for n, i in enumerate(range(b0, b1)):
        r0, r1 = int(t["resp_cu"][i]), int(t["resp_cu"][i + 1])
        xq = np.concatenate([qp, _as64(t["q_r"][r0:r1, h])])
        xk = np.concatenate([kp, _as64(t["k_r"][r0:r1, kv])])
        xv = np.concatenate([vp, _as64(t["v_r"][r0:r1, kv])])
        dor = _as64(t["do_r"][r0:r1, h])
        first = n == 0
        xdo = np.concatenate([dop if first else np.zeros_like(dop), dor])
        L = plen + (r1 - r0)
        if first or not fast:
            rows = np.arange(L)
        else:
            # Exact shortcut: a later branch's prompt rows give the same output
            # as the first branch's and carry a zero upstream gradient, so they
            # add nothing to any gradient.
            rows = np.arange(plen, L)
        o, lse, dq, dk, dv = causal_unit(xq, xk, xv, xdo, scale, rows=rows, chunk=chunk)
        off = L - len(rows)  # index of rows[0]
        if first:
            res["o_p"] = o[:plen]
            res["lse_p"] = lse[:plen]
            res["dq_p"] = dq[:plen]
        elif not fast and plen > 0:
            if check_prompt_rows:
                # Every branch computes the same prompt rows.
                np.testing.assert_allclose(o[:plen], res["o_p"], rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[:plen], res["lse_p"], rtol=0, atol=1e-12)
            res["dq_p"] += dq[:plen]
        res["dk_p"] += dk[:plen]
        res["dv_p"] += dv[:plen]
        res["branches"].append(
            (i, o[plen - off:], lse[plen - off:], dq[plen - off:], dk[plen:], dv[plen:]))
    return res


def _empty_outputs(t):
    tp, hq, d = t["q_p"].shape
    tr = t["q_r"].shape[0]
    hkv = t["k_p"].shape[1]
    return {
        "o_p": np.zeros((tp, hq, d)), "lse_p": np.zeros((hq, tp)),
        "o_r": np.zeros((tr, hq, d)), "lse_r": np.zeros((hq, tr)),
        "dq_p": np.zeros((tp, hq, d)), "dk_p": np.zeros((tp, hkv, d)),
        "dv_p": np.zeros((tp, hkv, d)),
        "dq_r": np.zeros((tr, hq, d)), "dk_r": np.zeros((tr, hkv, d)),
        "dv_r": np.zeros((tr, hkv, d)),
    }


def _scatter(out, t, g, h, res):
    hq = t["q_p"].shape[1]
    hkv = t["k_p"].shape[1]
    kv = kv_head_of(h, hq, hkv)
    p0, p1 = int(t["prompt_cu"][g]), int(t["prompt_cu"][g + 1])
    out["o_p"][p0:p1, h] = res["o_p"]
    out["lse_p"][h, p0:p1] = res["lse_p"]
    out["dq_p"][p0:p1, h] = res["dq_p"]
    out["dk_p"][p0:p1, kv] += res["dk_p"]
    out["dv_p"][p0:p1, kv] += res["dv_p"]
    for i, o, lse, dq, dk, dv in res["branches"]:
        r0, r1 = int(t["resp_cu"][i]), int(t["resp_cu"][i + 1])
        out["o_r"][r0:r1, h] = o
        out["lse_r"][h, r0:r1] = lse
        out["dq_r"][r0:r1, h] = dq
        out["dk_r"][r0:r1, kv] += dk
        out["dv_r"][r0:r1, kv] += dv


def tree_attention(t, scale, fast=False, chunk=512, groups=None, heads=None):
    """Forward and backward of the whole tree, one flattened pair at a time.

    ``t`` maps names to arrays: q_p, k_p, v_p, do_p (prompt, [sum P, H, d]),
    q_r, k_r, v_r, do_r (responses, [sum T, H, d]) and the int offset arrays
    prompt_cu [n_g+1], group_branch_cu [n_g+1], resp_cu [n_branches+1].  Values
    are upcast exactly to float64.

    fast=False evaluates every row of every flattened pair and checks that all
    branches agree on the prompt rows.  fast=True skips the prompt rows of
    every branch after the first; the result is the same (see
    ``_group_head_unit``).

    groups / heads restrict the work to a subset (other entries stay zero).

    Returns a dict of float64 arrays: o_p, lse_p, o_r, lse_r, dq_p, dk_p,
    dv_p, dq_r, dk_r, dv_r.  dk_p / dv_p are the total prompt gradients: the
    prompt rows' own term plus the sum over every branch (Eq. 2).
    """
    out = _empty_outputs(t)
    n_g = len(t["prompt_cu"]) - 1
    hq = t["q_p"].shape[1]
    for g in (range(n_g) if groups is None else groups):
        for h in (range(hq) if heads is None else heads):
            _scatter(out, t, g, h, _group_head_unit(t, g, h, scale, fast, chunk, True))
    return out


_FORK_INPUTS = None


def _worker(args):
    g, h, scale, fast, chunk = args
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            return g, h, _group_head_unit(_FORK_INPUTS, g, h, scale, fast, chunk, False)
    except ImportError:  # pragma: no cover - threadpoolctl is present here
        return g, h, _group_head_unit(_FORK_INPUTS, g, h, scale, fast, chunk, False)


def tree_attention_parallel(t, scale, fast=True, chunk=512, workers=None,
                            groups=None, heads=None):
    """Same result as ``tree_attention``, with one process per (group, head).

    Workers are forked with one BLAS thread each and inherit the inputs.
    Returns (outputs, workers_used).
    """
    global _FORK_INPUTS
    import multiprocessing as mp

    workers = workers or os.cpu_count() or 1
    n_g = len(t["prompt_cu"]) - 1
    hq = t["q_p"].shape[1]
    units = [(g, h, scale, fast, chunk)
             for g in (range(n_g) if groups is None else groups)
             for h in (range(hq) if heads is None else heads)]
    out = _empty_outputs(t)
    workers = max(1, min(workers, len(units)))
    _FORK_INPUTS = t
    try:
        if workers == 1:
            results = [_worker(u) for u in units]
        else:
            with mp.get_context("fork").Pool(workers) as pool:
                results = pool.map(_worker, units, chunksize=1)
    finally:
        _FORK_INPUTS = None
    for g, h, res in results:
        _scatter(out, t, g, h, res)
    return out, workers


def lse_merge(o_parts, lse_parts):
    """Merge S partial attention states for the same query rows.

    o_parts [S, rows, H, d] are normalised partial outputs, lse_parts
    [S, H, rows] their natural-log normalisers.  A partial state with
    LSE = -inf (no visible key) is the identity.  Definition: with
    LSE = ln sum_k exp(LSE_k), the merged output is
    O = sum_k exp(LSE_k - LSE) O_k.  Keeping the normaliser with each part is
    what makes the merge exact (section 3.3, MoveQ, and Fig. 8: partial
    online-softmax states (m, l, O_acc) are merged, not normalised outputs;
    (O, LSE) carries the same information as O_acc = l O, m = LSE - ln l).
    Returns (o [rows, H, d], lse [H, rows]).
    """
    o_parts = _as64(o_parts)
    lse_parts = _as64(lse_parts)
    lse = np.logaddexp.reduce(lse_parts, axis=0)
    with np.errstate(invalid="ignore"):
        w = np.exp(lse_parts - lse[None])
    w = np.where(np.isneginf(lse_parts), 0.0, w)  # empty part, or every part empty
    o = np.einsum("shr,srhd->rhd", w, o_parts)
    return o, lse
