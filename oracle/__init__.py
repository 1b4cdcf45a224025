"""fp64 CPU oracle for the multi-head attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

* ``mha_oracle``  -- the forward pass written out from its definition, fp64 numpy.
* ``brute``       -- the same quantities from scalar formulas in Python floats,
                     for tiny inputs; used to pin ``mha_oracle``.

Every function in ``mha_oracle`` is pinned by the CPU tests (brute force,
torch.nn.MultiheadAttention in float64, closed forms and the invariants the
pages state); none is "parity unpinned".
"""

from .mha_oracle import (  # noqa: F401
    linear, split_heads, concat_heads, masked_scores, softmax_rows,
    attention, mha_forward, mha_forward_rows, mha_forward_blocked, param_count,
    sigmoid, head_gates, apply_gates,
)
