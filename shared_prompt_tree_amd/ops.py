"""ctypes binding of libtreeattn.so, with the entry-point names of the C ABI.

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the HIP library.  Loading
fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libtreeattn.so")

F32, BF16 = 0, 1
OP_PREFILL, OP_REPLAY_FWD, OP_REPLAY_BWD, OP_PREFILL_BWD = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16}


class TreeAttnError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_groups", ctypes.c_int32),
        ("num_branches", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("prompt_cu_h", ctypes.c_void_p),
        ("prompt_cu_d", ctypes.c_void_p),
        ("group_branch_cu_h", ctypes.c_void_p),
        ("group_branch_cu_d", ctypes.c_void_p),
        ("resp_cu_h", ctypes.c_void_p),
        ("resp_cu_d", ctypes.c_void_p),
        ("dq_strategy", ctypes.c_int32),
        ("prompt_col_splits", ctypes.c_int32),
        ("prompt_tile_split_rows", ctypes.c_int32),
    ]


# tree_attn_dq_strategy
DQ_AUTO, DQ_SEPARATE, DQ_FUSED = 0, 1, 2


_lib = None


def library():
    """Load libtreeattn.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libtreeattn.so not found at {LIB_PATH}; build it with "
            "`python -m shared_prompt_tree_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.tree_attn_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    lib.tree_attn_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tree_attn_replay_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tree_attn_replay_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.tree_attn_replay_bwd.argtypes = [P] + [vp] * 14 + [sz, vp]
    lib.tree_attn_prefill_bwd.argtypes = [P] + [vp] * 12 + [sz, vp]
    lib.lse_merge.argtypes = [ctypes.c_int32] * 5 + [vp] * 4 + [vp]
    lib.tree_attn_error_string.argtypes = [ctypes.c_int]
    lib.tree_attn_error_string.restype = ctypes.c_char_p
    lib.tree_attn_last_hip_error.argtypes = []
    lib.tree_attn_set_kernel_events.argtypes = [ctypes.c_int, vp, vp]
    lib.tree_attn_dq_strategy_of.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.tree_attn_prompt_col_splits_of.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.tree_attn_prompt_tile_splits_of.argtypes = [P, ctypes.POINTER(ctypes.c_int)]
    for name in ("tree_attn_workspace_size", "tree_attn_prefill", "tree_attn_replay_fwd",
                 "tree_attn_replay_fwd_noalloc",
                 "tree_attn_replay_bwd", "tree_attn_prefill_bwd", "lse_merge",
                 "tree_attn_last_hip_error", "tree_attn_set_kernel_events",
                 "tree_attn_dq_strategy_of", "tree_attn_prompt_col_splits_of",
                 "tree_attn_prompt_tile_splits_of"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn, code):
    if code != 0:
        lib = library()
        msg = lib.tree_attn_error_string(code).decode()
        if code == -4:
            msg += f" (hipError {lib.tree_attn_last_hip_error()})"
        raise TreeAttnError(fn, code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _used_on(stream, *tensors):
    """Tensors allocated here come from torch's caching allocator on the
    current stream.  When the library runs on another stream, mark them as
    used there, so their memory is not handed out again before that stream's
    work has finished."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


class TreeProblem:
    """Offsets and shapes of a batch of replay trees, on host and device.

    prompt_cu [n_g+1], group_branch_cu [n_g+1], resp_cu [n_branches+1] are
    int sequences; they are copied to int32 host arrays and, when ``device``
    is given, to int32 device tensors.
    """

    def __init__(self, prompt_cu, group_branch_cu, resp_cu, num_q_heads, num_kv_heads,
                 head_dim, dtype, softmax_scale=None, device=None, dq_strategy=DQ_AUTO,
                 prompt_col_splits=0, prompt_tile_split_rows=0):
        self.prompt_cu = np.ascontiguousarray(prompt_cu, dtype=np.int32)
        self.group_branch_cu = np.ascontiguousarray(group_branch_cu, dtype=np.int32)
        self.resp_cu = np.ascontiguousarray(resp_cu, dtype=np.int32)
        self.dtype = dtype
        self.hq, self.hkv, self.d = int(num_q_heads), int(num_kv_heads), int(head_dim)
        self.scale = float(softmax_scale if softmax_scale is not None else head_dim ** -0.5)
        self.device = device
        if device is not None:
            self.prompt_cu_d = torch.from_numpy(self.prompt_cu).to(device)
            self.group_branch_cu_d = torch.from_numpy(self.group_branch_cu).to(device)
            self.resp_cu_d = torch.from_numpy(self.resp_cu).to(device)
        else:
            self.prompt_cu_d = self.group_branch_cu_d = self.resp_cu_d = None
        self.c = Problem(
            num_groups=len(self.prompt_cu) - 1,
            num_branches=len(self.resp_cu) - 1,
            num_q_heads=self.hq, num_kv_heads=self.hkv, head_dim=self.d,
            dtype=_DTYPE_CODE.get(dtype, -1) if isinstance(dtype, torch.dtype) else int(dtype),
            softmax_scale=self.scale,
            prompt_cu_h=self.prompt_cu.ctypes.data,
            prompt_cu_d=None if self.prompt_cu_d is None else self.prompt_cu_d.data_ptr(),
            group_branch_cu_h=self.group_branch_cu.ctypes.data,
            group_branch_cu_d=(None if self.group_branch_cu_d is None
                               else self.group_branch_cu_d.data_ptr()),
            resp_cu_h=self.resp_cu.ctypes.data,
            resp_cu_d=None if self.resp_cu_d is None else self.resp_cu_d.data_ptr(),
            dq_strategy=int(dq_strategy),
            prompt_col_splits=int(prompt_col_splits),
            prompt_tile_split_rows=int(prompt_tile_split_rows),
        )

    @property
    def dq_strategy(self):
        return self.c.dq_strategy

    @dq_strategy.setter
    def dq_strategy(self, value):
        self.c.dq_strategy = int(value)

    @property
    def prompt_col_splits(self):
        return self.c.prompt_col_splits

    @prompt_col_splits.setter
    def prompt_col_splits(self, value):
        self.c.prompt_col_splits = int(value)

    @property
    def prompt_tile_split_rows(self):
        return self.c.prompt_tile_split_rows

    @prompt_tile_split_rows.setter
    def prompt_tile_split_rows(self, value):
        self.c.prompt_tile_split_rows = int(value)

    @classmethod
    def from_tree(cls, tree, device=None, softmax_scale=None, dq_strategy=DQ_AUTO):
        from .workloads import torch_dtype
        return cls(tree.prompt_cu, tree.group_branch_cu, tree.resp_cu, tree.hq, tree.hkv, tree.d,
                   torch_dtype(tree.dtype), softmax_scale, device, dq_strategy)

    @property
    def prompt_tokens(self):
        return int(self.prompt_cu[-1])

    @property
    def resp_tokens(self):
        return int(self.resp_cu[-1])


KERNEL_FWD, KERNEL_DQ, KERNEL_DKV = 0, 1, 2


def tree_attn_set_kernel_events(kind, start=None, stop=None):
    """Record torch.cuda.Event ``start``/``stop`` around every launch of a
    main kernel (KERNEL_FWD, KERNEL_DQ, KERNEL_DKV) from this thread; call
    with no events to clear."""
    s = None if start is None else ctypes.c_void_p(start.cuda_event)
    e = None if stop is None else ctypes.c_void_p(stop.cuda_event)
    _check("tree_attn_set_kernel_events", library().tree_attn_set_kernel_events(kind, s, e))


def tree_attn_dq_strategy_of(problem: TreeProblem, op: int) -> int:
    """DQ_SEPARATE or DQ_FUSED: the dQ strategy backward call ``op``
    (OP_REPLAY_BWD or OP_PREFILL_BWD) uses for this problem."""
    v = ctypes.c_int(-1)
    _check("tree_attn_dq_strategy_of",
           library().tree_attn_dq_strategy_of(ctypes.byref(problem.c), op, ctypes.byref(v)))
    return v.value


def tree_attn_prompt_col_splits_of(problem: TreeProblem, op: int) -> int:
    """Chunks per prompt column of the replay query launch of ``op``
    (OP_REPLAY_FWD: the forward; OP_REPLAY_BWD: the dQ pass); 1 = not split."""
    v = ctypes.c_int(-1)
    _check("tree_attn_prompt_col_splits_of",
           library().tree_attn_prompt_col_splits_of(ctypes.byref(problem.c), op,
                                                    ctypes.byref(v)))
    return v.value


def tree_attn_prompt_tile_splits_of(problem: TreeProblem) -> int:
    """Prompt key-tile work items per tile position, summed over groups
    (n_g when no group's prompt tiles are split over branch ranges)."""
    v = ctypes.c_int(-1)
    _check("tree_attn_prompt_tile_splits_of",
           library().tree_attn_prompt_tile_splits_of(ctypes.byref(problem.c), ctypes.byref(v)))
    return v.value


def tree_attn_workspace_size(problem: TreeProblem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("tree_attn_workspace_size",
           library().tree_attn_workspace_size(ctypes.byref(problem.c), op, ctypes.byref(n)))
    return n.value


def _req(name, t, shape, dtype, device=None):
    """A tensor argument must match the problem exactly: the library reads
    raw pointers and cannot check sizes itself."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the problem's GPU")


def _check_tensors(problem, **named):
    tp, tr = problem.prompt_tokens, problem.resp_tokens
    hq, hkv, d, dt = problem.hq, problem.hkv, problem.d, problem.dtype
    shapes = {
        "q_p": (tp, hq, d), "k_p": (tp, hkv, d), "v_p": (tp, hkv, d), "o_p": (tp, hq, d),
        "do_p": (tp, hq, d), "dq_p": (tp, hq, d), "dk_p": (tp, hkv, d), "dv_p": (tp, hkv, d),
        "q_r": (tr, hq, d), "k_r": (tr, hkv, d), "v_r": (tr, hkv, d), "o_r": (tr, hq, d),
        "do_r": (tr, hq, d), "dq_r": (tr, hq, d), "dk_r": (tr, hkv, d), "dv_r": (tr, hkv, d),
        "lse_p": (hq, tp), "lse_r": (hq, tr),
        "dk_p_seed": (tp, hkv, d), "dv_p_seed": (tp, hkv, d),
    }
    f32 = {"lse_p", "lse_r", "dk_p_seed", "dv_p_seed"}
    dev = problem.prompt_cu_d.device if problem.prompt_cu_d is not None else None
    if dev is None:
        raise ValueError("the problem has no device offset arrays (pass device=...)")
    for name, t in named.items():
        if t is None and name in ("dk_p_seed", "dv_p_seed"):
            continue
        _req(name, t, shapes[name], torch.float32 if name in f32 else dt, dev)


def _workspace(problem, op, device):
    n = tree_attn_workspace_size(problem, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def tree_attn_prefill(problem, q_p, k_p, v_p, o_p=None, lse_p=None, stream=None):
    """Causal prompt prefill.  Returns (o_p, lse_p)."""
    dev = q_p.device
    made = []
    if o_p is None:
        o_p = torch.empty_like(q_p)
        made.append(o_p)
    if lse_p is None:
        lse_p = torch.empty(problem.hq, problem.prompt_tokens, dtype=torch.float32, device=dev)
        made.append(lse_p)
    _check_tensors(problem, q_p=q_p, k_p=k_p, v_p=v_p, o_p=o_p, lse_p=lse_p)
    ws, n = _workspace(problem, OP_PREFILL, dev)
    _check("tree_attn_prefill", library().tree_attn_prefill(
        ctypes.byref(problem.c), _ptr(q_p), _ptr(k_p), _ptr(v_p), _ptr(o_p), _ptr(lse_p),
        _ptr(ws), n, _stream(stream)))
    _used_on(stream, ws, *made)
    return o_p, lse_p


def tree_attn_replay_fwd(problem, k_p, v_p, q_r, k_r, v_r, o_r=None, lse_r=None, stream=None):
    """Response replay forward.  Returns (o_r, lse_r)."""
    dev = q_r.device
    made = []
    if o_r is None:
        o_r = torch.empty_like(q_r)
        made.append(o_r)
    if lse_r is None:
        lse_r = torch.empty(problem.hq, problem.resp_tokens, dtype=torch.float32, device=dev)
        made.append(lse_r)
    _check_tensors(problem, k_p=k_p, v_p=v_p, q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r, lse_r=lse_r)
    ws, n = _workspace(problem, OP_REPLAY_FWD, dev)
    _check("tree_attn_replay_fwd", library().tree_attn_replay_fwd(
        ctypes.byref(problem.c), _ptr(k_p), _ptr(v_p), _ptr(q_r), _ptr(k_r), _ptr(v_r),
        _ptr(o_r), _ptr(lse_r), _ptr(ws), n, _stream(stream)))
    _used_on(stream, ws, *made)
    return o_r, lse_r


STATIC_SCRATCH_BYTES = 128 << 20


def tree_attn_replay_fwd_noalloc(problem, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, stream=None):
    """Response replay forward into caller-provided o_r / lse_r, with the
    library's static scratch instead of a workspace: no device memory is
    allocated here or in the library.  Returns (o_r, lse_r)."""
    _check_tensors(problem, k_p=k_p, v_p=v_p, q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r, lse_r=lse_r)
    _check("tree_attn_replay_fwd_noalloc", library().tree_attn_replay_fwd_noalloc(
        ctypes.byref(problem.c), _ptr(k_p), _ptr(v_p), _ptr(q_r), _ptr(k_r), _ptr(v_r),
        _ptr(o_r), _ptr(lse_r), _stream(stream)))
    return o_r, lse_r


def tree_attn_replay_bwd(problem, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, do_r, seeds=True,
                         out=None, stream=None):
    """Replay backward.  Returns (dq_r, dk_r, dv_r, dk_p_seed, dv_p_seed);
    the seeds are None when ``seeds`` is False (detached prompt)."""
    dev = q_r.device
    made = ()
    if out is None:
        out = (torch.empty_like(q_r), torch.empty_like(k_r), torch.empty_like(v_r),
               torch.empty(k_p.shape, dtype=torch.float32, device=dev) if seeds else None,
               torch.empty(v_p.shape, dtype=torch.float32, device=dev) if seeds else None)
        made = out
    dq_r, dk_r, dv_r, dks, dvs = out
    _check_tensors(problem, k_p=k_p, v_p=v_p, q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r, lse_r=lse_r,
                   do_r=do_r, dq_r=dq_r, dk_r=dk_r, dv_r=dv_r, dk_p_seed=dks, dv_p_seed=dvs)
    ws, n = _workspace(problem, OP_REPLAY_BWD, dev)
    _check("tree_attn_replay_bwd", library().tree_attn_replay_bwd(
        ctypes.byref(problem.c), _ptr(k_p), _ptr(v_p), _ptr(q_r), _ptr(k_r), _ptr(v_r),
        _ptr(o_r), _ptr(lse_r), _ptr(do_r), _ptr(dq_r), _ptr(dk_r), _ptr(dv_r), _ptr(dks),
        _ptr(dvs), _ptr(ws), n, _stream(stream)))
    _used_on(stream, ws, *made)
    return dq_r, dk_r, dv_r, dks, dvs


def tree_attn_prefill_bwd(problem, q_p, k_p, v_p, o_p, lse_p, do_p, dk_p_seed=None,
                          dv_p_seed=None, out=None, stream=None):
    """Prefill backward with the replay seeds.  Returns (dq_p, dk_p, dv_p)."""
    dev = q_p.device
    made = ()
    if out is None:
        out = (torch.empty_like(q_p), torch.empty_like(k_p), torch.empty_like(v_p))
        made = out
    dq_p, dk_p, dv_p = out
    _check_tensors(problem, q_p=q_p, k_p=k_p, v_p=v_p, o_p=o_p, lse_p=lse_p, do_p=do_p,
                   dk_p_seed=dk_p_seed, dv_p_seed=dv_p_seed, dq_p=dq_p, dk_p=dk_p, dv_p=dv_p)
    ws, n = _workspace(problem, OP_PREFILL_BWD, dev)
    _check("tree_attn_prefill_bwd", library().tree_attn_prefill_bwd(
        ctypes.byref(problem.c), _ptr(q_p), _ptr(k_p), _ptr(v_p), _ptr(o_p), _ptr(lse_p),
        _ptr(do_p), _ptr(dk_p_seed), _ptr(dv_p_seed), _ptr(dq_p), _ptr(dk_p), _ptr(dv_p),
        _ptr(ws), n, _stream(stream)))
    _used_on(stream, ws, *made)
    return dq_p, dk_p, dv_p


def lse_merge(o_parts, lse_parts, out_dtype=torch.float32, o_out=None, lse_out=None,
              stream=None):
    """Merge partial states o_parts [S, rows, H, d] / lse_parts [S, H, rows]."""
    s, rows, heads, d = o_parts.shape
    dev = o_parts.device
    _req("o_parts", o_parts, (s, rows, heads, d), torch.float32, dev)
    _req("lse_parts", lse_parts, (s, heads, rows), torch.float32, dev)
    made = []
    if o_out is None:
        o_out = torch.empty(rows, heads, d, dtype=out_dtype, device=dev)
        made.append(o_out)
    if lse_out is None:
        lse_out = torch.empty(heads, rows, dtype=torch.float32, device=dev)
        made.append(lse_out)
    _req("o_out", o_out, (rows, heads, d), o_out.dtype, dev)
    _req("lse_out", lse_out, (heads, rows), torch.float32, dev)
    _check("lse_merge", library().lse_merge(
        s, rows, heads, d, _DTYPE_CODE[o_out.dtype], _ptr(o_parts), _ptr(lse_parts),
        _ptr(o_out), _ptr(lse_out), _stream(stream)))
    _used_on(stream, *made)
    return o_out, lse_out


def tree_attention_forward_backward(problem, t, seeds=True, stream=None):
    """One pass of the whole path: prefill, replay forward, replay backward,
    prefill backward.  ``t`` holds q_p, k_p, v_p, q_r, k_r, v_r, do_p, do_r.
    Returns a dict with every output."""
    o_p, lse_p = tree_attn_prefill(problem, t["q_p"], t["k_p"], t["v_p"], stream=stream)
    o_r, lse_r = tree_attn_replay_fwd(problem, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                      stream=stream)
    dq_r, dk_r, dv_r, dks, dvs = tree_attn_replay_bwd(
        problem, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_r, lse_r, t["do_r"],
        seeds=seeds, stream=stream)
    dq_p, dk_p, dv_p = tree_attn_prefill_bwd(problem, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p,
                                             t["do_p"], dks, dvs, stream=stream)
    return dict(o_p=o_p, lse_p=lse_p, o_r=o_r, lse_r=lse_r, dq_r=dq_r, dk_r=dk_r, dv_r=dv_r,
                dk_p_seed=dks, dv_p_seed=dvs, dq_p=dq_p, dk_p=dk_p, dv_p=dv_p)
