"""The replay forward without allocation (tree_attn_replay_fwd_noalloc,
static per-GPU scratch) against the workspace entry point, through the C ABI
(GPU).

Calls in a row on one GPU, each smaller than the one before, so every call
runs over what the previous one left in the shared scratch: the prompt-heavy
replay at full size (32768 prompt keys, 8 x 512 response rows, about 75 MB of
scratch), a reduced ragged shape, and a float32 tree whose prompt column is
cut into chunks (merge partials in the scratch too).  Each output must equal
the workspace entry point's (same kernels, deterministic), which is within
the bf16 / float32 tolerances of the parity tests.
"""

import pytest
import torch

from shared_prompt_tree_amd import ops
from shared_prompt_tree_amd import workloads as wl
from tests._gpu import TOL, host64, make_case, rel_l2, say

pytestmark = pytest.mark.gpu

CALLS = [
    ("prompt-heavy replay", wl.make_tree(wl.SPECS["prompt_heavy"]), 1.0),
    ("reduced ragged", wl.Tree([4097, 300], [[300, 511, 64, 1], [0, 77]], 32, 8, 128, "bf16"),
     1.0),
    ("f32 split prompt column", wl.Tree([4096], [[20, 3]], 2, 1, 64, "f32"), 0.125),
]


def test_noalloc_replay_matches_workspace_entry_point():
    for label, tree, vs in CALLS:
        prob, t = make_case(tree, 31, value_scale=vs)
        need = ops.tree_attn_workspace_size(prob, ops.OP_REPLAY_FWD)
        say(f"[noalloc] {label}: {tree.prompt_tokens} prompt + {tree.resp_tokens} response "
            f"tokens, scratch {need / 2**20:.1f} MiB of {ops.STATIC_SCRATCH_BYTES / 2**20:.0f}")
        assert need <= ops.STATIC_SCRATCH_BYTES
        o_ws, lse_ws = ops.tree_attn_replay_fwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                                t["v_r"])
        # outputs start as garbage so that nothing is inherited
        o_na = torch.full_like(o_ws, float("nan"))
        lse_na = torch.full_like(lse_ws, float("nan"))
        ops.tree_attn_replay_fwd_noalloc(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                         o_na, lse_na)
        torch.cuda.synchronize()
        eo = rel_l2(host64(o_na), host64(o_ws))
        el = rel_l2(host64(lse_na), host64(lse_ws))
        say(f"[noalloc] {label}: rel L2 O {eo:.2e}, LSE {el:.2e}")
        assert eo <= TOL[tree.dtype] and el <= TOL[tree.dtype]
        assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws)
