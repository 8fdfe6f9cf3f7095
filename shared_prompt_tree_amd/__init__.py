"""Shared-prompt tree attention on MI355X (gfx950).

The compute path is the HIP library ``libtreeattn.so`` (C ABI declared in
``include/tree_attn.h``).  ``shared_prompt_tree_amd.ops`` is a thin ctypes
binding with the same entry-point names; it raises if the library is missing.
``workloads`` draws seeded synthetic replay trees.
"""

__all__ = ["ops", "workloads"]
