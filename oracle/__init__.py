"""Float64 CPU oracle for shared-prompt tree attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  The HIP library never calls it and shares no code
with it.
"""

from .tree_attention import (  # noqa: F401
    causal_key_grads,
    causal_unit,
    lse_merge,
    tree_attention,
    tree_attention_parallel,
)
