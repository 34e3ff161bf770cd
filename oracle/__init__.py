"""fp64 CPU oracle for the fused attention forward pass (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package. The product path never does.
"""
from .attention import (MASK_BLOCK_K, MASK_BLOCK_Q, attention, attention_backward,
                        attention_rows, block_visible, visible_count, visible_mask)

__all__ = ["attention", "attention_backward", "attention_rows", "visible_count", "visible_mask", "block_visible",
           "MASK_BLOCK_Q", "MASK_BLOCK_K"]
