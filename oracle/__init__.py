"""fp64 CPU oracle for BigBird block-sparse attention -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product (the HIP library and its Python binding)
never does.
"""
from .bigbird_oracle import (  # noqa: F401
    MASK_OFFSET,
    attention_backward,
    attention_backward_unit,
    attention_forward,
    attention_lse,
    attention_probs,
    attention_rows,
    block_adjacency,
    check_rand_idx,
    layer_forward,
    layer_rows,
    layer_stack_forward,
    num_blocks,
    token_mask,
)
