"""CPU oracle for the scaled-dot-product-attention backward pass.

Test infrastructure only: the GPU library never imports this package, and this package never
imports the GPU library.  Only the tests, the smoke check of ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may call it.
"""
from .sdpa_oracle import (  # noqa: F401
    visible_mask,
    forward,
    backward,
    dsink,
    backward_dq_rows,
    backward_dkdv_rows,
    attention_flops,
)
from .nvfp4_qat import (  # noqa: F401
    e4m3_round,
    e2m1_round,
    fake_nvfp4,
    qat_forward,
    qat_backward,
)
