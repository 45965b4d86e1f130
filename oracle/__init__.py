"""fp64 CPU oracle for exact attention (forward and gradient).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The product
path (the HIP library and its Python binding) never does, and shares no code with it.

The method reaches exactly the plain attention result, only with fewer HBM accesses
(FlashAttention-NeurIPS22 digest, "一句话总结" and "设计取舍": exact dense attention
semantics are kept), so this oracle *is* the plain definition, written out in float64:
it materialises S and P per head, the way the digest's "问题与动机" describes the
standard implementation.  Every function here is pinned by tests in
``tests/test_oracle.py`` against brute force, a library routine, closed forms,
invariants and finite differences.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    head_forward,
    head_backward,
    forward,
    backward,
    forward_rows,
)
from .dropout import (  # noqa: F401
    philox4x32_10,
    drop_threshold,
    draw_halves,
    keep_mask,
    head_forward_dropout,
    head_backward_dropout,
    forward_dropout,
    backward_dropout,
)
from .fp8 import (  # noqa: F401
    e4m3_value,
    dequantize,
    head_forward_fp8,
)
