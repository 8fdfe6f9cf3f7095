"""The C ABI library without a GPU: it loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments on the host
before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from shared_prompt_tree_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH),
                                reason="libtreeattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"tree_attn_prefill", "tree_attn_replay_fwd", "tree_attn_replay_bwd",
            "tree_attn_prefill_bwd", "lse_merge", "tree_attn_workspace_size",
            "tree_attn_error_string"} <= set(names)
    lib = ops.library()
    for n in names:
        assert hasattr(lib, n), n


def test_error_strings():
    lib = ops.library()
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert lib.tree_attn_error_string(code)


def small_problem(**kw):
    args = dict(prompt_cu=[0, 5, 9], group_branch_cu=[0, 2, 3], resp_cu=[0, 3, 3, 7],
                num_q_heads=4, num_kv_heads=2, head_dim=128, dtype=torch.bfloat16)
    args.update(kw)
    return ops.TreeProblem(**args)


def test_workspace_sizes_grow_with_tokens():
    a = small_problem()
    b = small_problem(prompt_cu=[0, 500, 900], resp_cu=[0, 300, 300, 700])
    for op in range(4):
        assert 0 < ops.tree_attn_workspace_size(a, op) < ops.tree_attn_workspace_size(b, op)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -2),
    (dict(dtype=torch.float16), -2),
    (dict(num_kv_heads=3), -1),
    (dict(prompt_cu=[1, 5, 9]), -1),
    (dict(prompt_cu=[0, 5, 4]), -1),
    (dict(group_branch_cu=[0, 2, 2]), -1),
    (dict(resp_cu=[0, 3, 2, 7]), -1),
    (dict(softmax_scale=0.0), -1),
    (dict(softmax_scale=float("nan")), -1),
])
def test_invalid_problem_rejected(kw, code):
    p = small_problem(**kw)
    with pytest.raises(ops.TreeAttnError) as e:
        ops.tree_attn_workspace_size(p, ops.OP_PREFILL)
    assert e.value.code == code


@pytest.mark.parametrize("prompt,resp,heads", [
    (2 ** 31 - 1, 0, 1),          # padding the prompt to 64 tokens passes int32
    (2 ** 30, 2 ** 30, 1),        # prompt + response tokens reach 2^31
    (2 ** 27, 0, 16),             # tokens x query heads reach 2^31
])
def test_token_totals_beyond_int32_rejected(prompt, resp, heads):
    """Indices the kernels form must fit in int32; such problems are
    rejected on the host, before any per-length arithmetic can overflow."""
    kw = dict(prompt_cu=[0, prompt], num_q_heads=heads, num_kv_heads=1, head_dim=64)
    if resp:
        kw.update(group_branch_cu=[0, 1], resp_cu=[0, resp])
    else:
        kw.update(group_branch_cu=[0, 0], resp_cu=[0])
    for op in range(4):
        with pytest.raises(ops.TreeAttnError) as e:
            ops.tree_attn_workspace_size(small_problem(**kw), op)
        assert e.value.code == -1


def test_attention_launch_dispatch_limit():
    """A launch is one dispatch of at most 2^32 - 1 work-items.  MHA with 64
    heads (64 head groups) and a prompt of 2^25 - 128 tokens passes every
    other size check (tokens x Hq < 2^31, the transposed copy < 4 GiB) but its
    prefill forward would need 64 x 131072 workgroups of 512 threads: it is
    rejected on the host.  Half the heads fits."""
    P = 2 ** 25 - 128
    too_big = small_problem(prompt_cu=[0, P], group_branch_cu=[0, 0], resp_cu=[0],
                            num_q_heads=64, num_kv_heads=64, head_dim=64)
    with pytest.raises(ops.TreeAttnError) as e:
        ops.tree_attn_workspace_size(too_big, ops.OP_PREFILL)
    assert e.value.code == -1
    fits = small_problem(prompt_cu=[0, P], group_branch_cu=[0, 0], resp_cu=[0],
                         num_q_heads=32, num_kv_heads=32, head_dim=64)
    assert ops.tree_attn_workspace_size(fits, ops.OP_PREFILL) > 0


def test_aux_launch_math_at_the_largest_problem(tmp_path):
    """The element-wise kernels (row dot, merge, seed and chunk sums,
    transposed copies) launch a capped grid and walk their elements with a
    64-bit grid-stride loop.  A host build of that geometry (grid_math.h, the
    header the kernels use) checks it at tokens x Hq = 2^31 - 1 rows of 16
    lanes each: the grid fits a dispatch, every element is visited, and the
    16 lanes of a row stay in one pass."""
    import shutil
    import subprocess

    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "grid_math_check"
    subprocess.run([gxx, "-std=c++17", "-O1", "-I",
                    os.path.join(ROOT, "shared_prompt_tree_amd", "csrc"),
                    os.path.join(ROOT, "tests", "grid_math_check.cpp"), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_transposed_copy_offset_limit():
    """A head group's slice of a transposed copy is addressed with 32-bit
    byte offsets: head_dim * padded tokens * packed heads * element size must
    stay below 4 GiB (16 packed heads here: 64 query heads on 4 kv heads)."""
    d, hp, esz = 64, 16, 2
    ok = (2 ** 32 - 1) // (d * hp * esz) // 64 * 64   # largest padded prompt that fits
    p = small_problem(prompt_cu=[0, ok], group_branch_cu=[0, 0], resp_cu=[0],
                      num_q_heads=64, num_kv_heads=4, head_dim=d)
    assert ops.tree_attn_workspace_size(p, ops.OP_PREFILL) > 0
    p = small_problem(prompt_cu=[0, ok + 64], group_branch_cu=[0, 0], resp_cu=[0],
                      num_q_heads=64, num_kv_heads=4, head_dim=d)
    with pytest.raises(ops.TreeAttnError) as e:
        ops.tree_attn_workspace_size(p, ops.OP_PREFILL)
    assert e.value.code == -1


def test_replay_workspace_holds_split_partial_seeds():
    """A short prompt read by many long branches is split over branch ranges
    (one split per branch here: 6 branches of 128 rows, target = the longest
    branch), so the replay-backward workspace holds float32 partial seeds for
    6 x 64 prompt rows (dK and dV); a single branch of the same total length
    is never split."""
    kw = dict(prompt_cu=[0, 64], group_branch_cu=[0, 6], resp_cu=[0, 128, 256, 384, 512, 640, 768],
              num_q_heads=2, num_kv_heads=1, head_dim=64)
    split = ops.tree_attn_workspace_size(small_problem(**kw), ops.OP_REPLAY_BWD)
    kw.update(group_branch_cu=[0, 1], resp_cu=[0, 768])
    single = ops.tree_attn_workspace_size(small_problem(**kw), ops.OP_REPLAY_BWD)
    partial = 2 * 6 * 64 * 1 * 64 * 4
    assert partial <= split - single < partial + 64 * 1024


def test_replay_workspace_holds_prompt_column_partials():
    """Few response rows behind a long prompt: 4 query workgroups (8 heads
    packed 4 per kv head, 2 branches of one tile) fit one round however the
    128-tile prompt column is cut, so the longest item decides and the
    column is cut into the most chunks of >= 1024 keys, 8192 // 1024 = 8;
    the replay-forward workspace holds their float32 partial O (and LSE)."""
    kw = dict(prompt_cu=[0, 8192], group_branch_cu=[0, 2], resp_cu=[0, 40, 73],
              num_q_heads=8, num_kv_heads=2, head_dim=128)
    split = ops.tree_attn_workspace_size(small_problem(**kw), ops.OP_REPLAY_FWD)
    kw.update(prompt_cu=[0, 1000])  # too short to cut
    whole = ops.tree_attn_workspace_size(small_problem(**kw), ops.OP_REPLAY_FWD)
    partial = 8 * 73 * 8 * 128 * 4 + 8 * 8 * 73 * 4
    assert split - whole >= partial


def _column_chunks(prompt, branches, op, hq=32, hkv=8, d=128):
    """Prompt-column chunks of the replay forward (op 1) or dQ (op 2) launch."""
    p = small_problem(prompt_cu=[0, prompt], group_branch_cu=[0, len(branches)],
                      resp_cu=np.concatenate([[0], np.cumsum(branches)]).tolist(),
                      num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      dq_strategy=ops.DQ_SEPARATE)
    return ops.tree_attn_prompt_col_splits_of(p, op)


def _split_ws(prompt, branches, op, forced):
    p = small_problem(prompt_cu=[0, prompt], group_branch_cu=[0, len(branches)],
                      resp_cu=np.concatenate([[0], np.cumsum(branches)]).tolist(),
                      num_q_heads=32, num_kv_heads=8, head_dim=128,
                      dq_strategy=ops.DQ_SEPARATE, prompt_col_splits=forced)
    return ops.tree_attn_workspace_size(p, op)


def test_column_split_model():
    """The prompt-column split follows the makespan model, priced separately
    for the forward and the dQ launch with constants fitted to measured
    sweeps (bench.py --split-sweep).  On those sweeps the choices below were
    the fastest measured S or within 2.5% of it: 512 workgroups (8 branches
    of 512, 32/8 heads) fill two rounds of the 256 CUs and are not cut; 520
    (13 of 260) are cut into 4 (forward) and 6 (dQ) chunks; a few rows
    behind a 131072-token prompt into 4; 264 workgroups behind a 2048-token
    prompt only in the dQ pass."""
    assert _column_chunks(32768, [512] * 8, 1) == 1 and _column_chunks(32768, [512] * 8, 2) == 1
    assert _column_chunks(32768, [260] * 13, 1) == 4 and _column_chunks(32768, [260] * 13, 2) == 6
    assert _column_chunks(131072, [64] * 8, 1) == 4 and _column_chunks(131072, [64] * 8, 2) == 4
    assert _column_chunks(2048, [150] * 11, 1) == 1 and _column_chunks(2048, [150] * 11, 2) == 2


def test_forced_column_splits():
    """prompt_col_splits forces the chunk count of both launches (the
    workspace grows by the float32 partials); beyond 64 it is invalid; the
    query reports 1 for the dQ launch of the fused strategy, which has none."""
    base = _split_ws(32768, [512] * 8, ops.OP_REPLAY_FWD, 1)
    assert _split_ws(32768, [512] * 8, ops.OP_REPLAY_FWD, 3) > base
    assert (_split_ws(32768, [512] * 8, ops.OP_REPLAY_BWD, 3)
            > _split_ws(32768, [512] * 8, ops.OP_REPLAY_BWD, 1))
    p = small_problem(prompt_col_splits=5)
    assert ops.tree_attn_prompt_col_splits_of(p, ops.OP_REPLAY_FWD) == 5
    assert ops.tree_attn_prompt_col_splits_of(p, ops.OP_REPLAY_BWD) == 5
    p.dq_strategy = ops.DQ_FUSED
    assert ops.tree_attn_prompt_col_splits_of(p, ops.OP_REPLAY_BWD) == 1
    for bad in (-1, 65):
        with pytest.raises(ops.TreeAttnError):
            ops.tree_attn_workspace_size(small_problem(prompt_col_splits=bad), ops.OP_REPLAY_FWD)
    with pytest.raises(ops.TreeAttnError):
        ops.tree_attn_prompt_col_splits_of(small_problem(), ops.OP_PREFILL)


def test_bad_op_and_null_out_pointer():
    lib = ops.library()
    p = small_problem()
    n = ctypes.c_size_t(0)
    assert lib.tree_attn_workspace_size(ctypes.byref(p.c), 9, ctypes.byref(n)) == -1
    assert lib.tree_attn_workspace_size(ctypes.byref(p.c), 0, None) == -1
    assert lib.tree_attn_workspace_size(None, 0, ctypes.byref(n)) == -1


def test_entry_points_reject_before_any_hip_call():
    """Missing device offsets, null tensors, misaligned tensors, a single
    seed pointer and a short workspace are all refused on the host."""
    lib = ops.library()
    p = small_problem()  # no device arrays
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: validation fails first
    assert lib.tree_attn_prefill(ctypes.byref(p.c), fake, fake, fake, fake, fake, fake,
                                 1 << 30, None) == -1
    # device offsets present (fake addresses), null q
    p.c.prompt_cu_d = p.c.group_branch_cu_d = p.c.resp_cu_d = 1 << 20
    assert lib.tree_attn_prefill(ctypes.byref(p.c), None, fake, fake, fake, fake, fake,
                                 1 << 30, None) == -1
    # misaligned tensor
    assert lib.tree_attn_prefill(ctypes.byref(p.c), vp((1 << 20) + 2), fake, fake, fake, fake,
                                 fake, 1 << 30, None) == -1
    # workspace too small
    assert lib.tree_attn_prefill(ctypes.byref(p.c), fake, fake, fake, fake, fake, fake, 16,
                                 None) == -3
    # exactly one seed pointer
    assert lib.tree_attn_replay_bwd(ctypes.byref(p.c), *([fake] * 11), fake, None, fake,
                                    1 << 30, None) == -1
    assert lib.tree_attn_prefill_bwd(ctypes.byref(p.c), *([fake] * 6), None, fake, fake, fake,
                                     fake, fake, 1 << 30, None) == -1
    # lse_merge argument checks
    assert lib.lse_merge(0, 4, 2, 128, 1, fake, fake, fake, fake, None) == -1
    assert lib.lse_merge(2, 4, 2, 80, 1, fake, fake, fake, fake, None) == -2
    assert lib.lse_merge(2, 4, 2, 128, 5, fake, fake, fake, fake, None) == -2
    assert lib.lse_merge(2, 4, 2, 128, 1, None, fake, fake, fake, None) == -1
    assert lib.lse_merge(2, 0, 2, 128, 1, None, None, None, None, None) == 0


def test_noalloc_replay_rejects_problems_beyond_the_static_scratch():
    """tree_attn_replay_fwd_noalloc refuses, on the host and before any HIP
    call, a problem whose replay scratch (the size tree_attn_workspace_size
    reports) exceeds TREE_ATTN_STATIC_SCRATCH_BYTES, and invalid arguments as
    the workspace form does."""
    lib = ops.library()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: the call fails first
    # response-heavy-sized replay: ~2.7 GB of transposed V copies
    big = small_problem(prompt_cu=[0, 256], group_branch_cu=[0, 256],
                        resp_cu=np.arange(257) * 5000, num_q_heads=32, num_kv_heads=8)
    assert ops.tree_attn_workspace_size(big, ops.OP_REPLAY_FWD) > ops.STATIC_SCRATCH_BYTES
    big.c.prompt_cu_d = big.c.group_branch_cu_d = big.c.resp_cu_d = 1 << 20
    assert lib.tree_attn_replay_fwd_noalloc(ctypes.byref(big.c), *([fake] * 7), None) == -5
    assert b"static scratch" in lib.tree_attn_error_string(-5)
    p = small_problem()
    assert ops.tree_attn_workspace_size(p, ops.OP_REPLAY_FWD) <= ops.STATIC_SCRATCH_BYTES
    # no device offsets, then a null tensor
    assert lib.tree_attn_replay_fwd_noalloc(ctypes.byref(p.c), *([fake] * 7), None) == -1
    p.c.prompt_cu_d = p.c.group_branch_cu_d = p.c.resp_cu_d = 1 << 20
    assert lib.tree_attn_replay_fwd_noalloc(ctypes.byref(p.c), fake, fake, None, fake, fake,
                                            fake, fake, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        ops.library()


def test_dq_strategy_validation():
    """dq_strategy outside the enum is invalid; the fused strategy covers
    bf16 with head_dim 128 only."""
    for bad in (-1, 3):
        p = small_problem(dq_strategy=bad)
        n = ctypes.c_size_t(0)
        assert ops.library().tree_attn_workspace_size(ctypes.byref(p.c), 2, ctypes.byref(n)) == -1
    for kw in (dict(head_dim=64), dict(dtype=torch.float32)):
        p = small_problem(dq_strategy=ops.DQ_FUSED, **kw)
        with pytest.raises(ops.TreeAttnError) as e:
            ops.tree_attn_workspace_size(p, ops.OP_REPLAY_BWD)
        assert e.value.code == -2
    # automatic choice outside the fused strategy's domain: the separate pass
    p = small_problem(head_dim=64)
    assert ops.tree_attn_dq_strategy_of(p, ops.OP_REPLAY_BWD) == ops.DQ_SEPARATE


def test_dq_strategy_workspaces():
    """The fused strategy needs a float32 dQ accumulator instead of the
    query-stationary work list and the K^T copies; each backward op reports
    the strategy it uses, and the forward ops are not affected."""
    sep = small_problem(prompt_cu=[0, 500, 900], resp_cu=[0, 300, 300, 700],
                        dq_strategy=ops.DQ_SEPARATE)
    fus = small_problem(prompt_cu=[0, 500, 900], resp_cu=[0, 300, 300, 700],
                        dq_strategy=ops.DQ_FUSED)
    for op in (ops.OP_PREFILL, ops.OP_REPLAY_FWD):
        assert ops.tree_attn_workspace_size(sep, op) == ops.tree_attn_workspace_size(fus, op)
    for op in (ops.OP_REPLAY_BWD, ops.OP_PREFILL_BWD):
        assert ops.tree_attn_workspace_size(sep, op) != ops.tree_attn_workspace_size(fus, op)
        assert ops.tree_attn_dq_strategy_of(sep, op) == ops.DQ_SEPARATE
        assert ops.tree_attn_dq_strategy_of(fus, op) == ops.DQ_FUSED
    with pytest.raises(ops.TreeAttnError):
        ops.tree_attn_dq_strategy_of(sep, ops.OP_PREFILL)


@pytest.mark.parametrize("name", ["prompt_heavy", "response_heavy", "long_mixed"])
def test_dq_cost_model_prefers_separate_pass(name):
    """Calibrated on same-box runs of both strategies: the fused kernel adds
    2 bytes of float32 atomics per (row, key) pair at head_dim 128, which at
    the measured ~0.95 TB/s takes longer than the separate pass's extra
    matrix products, so the automatic choice is the separate pass on the
    three large workloads."""
    from shared_prompt_tree_amd import workloads as wl
    tree = wl.make_tree(wl.SPECS[name])
    p = ops.TreeProblem.from_tree(tree)
    for op in (ops.OP_REPLAY_BWD, ops.OP_PREFILL_BWD):
        assert ops.tree_attn_dq_strategy_of(p, op) == ops.DQ_SEPARATE


def test_forced_prompt_tile_split_rows():
    """prompt_tile_split_rows sets the split target: one branch per range at
    1 row, the group unsplit at or above its rows; negative is invalid."""
    kw = dict(prompt_cu=[0, 64], group_branch_cu=[0, 6], resp_cu=[0, 128, 256, 384, 512, 640, 768],
              num_q_heads=2, num_kv_heads=1, head_dim=64)
    assert ops.tree_attn_prompt_tile_splits_of(small_problem(prompt_tile_split_rows=1, **kw)) == 6
    assert ops.tree_attn_prompt_tile_splits_of(small_problem(prompt_tile_split_rows=768, **kw)) == 1
    assert ops.tree_attn_prompt_tile_splits_of(small_problem(prompt_tile_split_rows=300, **kw)) == 3
    with pytest.raises(ops.TreeAttnError):
        ops.tree_attn_workspace_size(small_problem(prompt_tile_split_rows=-1), ops.OP_REPLAY_BWD)
