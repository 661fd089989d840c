"""fp64 CPU oracle for exact attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the library never does.
"""
from .attention import (  # noqa: F401
    fp32_scale, visible_mask, head_forward, head_backward, forward, backward,
    forward_rows, online_softmax, blockwise_attention_row, decode_visible_mask,
    decode_head_forward, decode_forward,
)
from . import block_sparse, dropout, fp8  # noqa: F401
