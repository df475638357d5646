"""CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The HIP library never calls it, and no
product code path falls back to it.

The oracle shares no code with the GPU path: it does its own arithmetic with
numpy (fp64) and, for the long shapes, plain torch CPU matrix products (fp32).
"""

from .attention import (  # noqa: F401
    scores,
    softmax_rows,
    attention_probs,
    attention_fwd,
    attention_bwd,
    attention_fwd_rows,
    attention_fwd_f32,
    attention_bwd_f32,
    exp2_exact,
)
