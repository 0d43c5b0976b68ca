"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
import this package.  The library never does.
"""

from .exact_attention import (  # noqa: F401
    attention_head,
    attention_ref,
    attention_ref_gqa,
    attention_ref_window,
    attention_head_window,
    attention_rows,
    finalize,
    merge_stats,
    partial_stats,
    probabilities,
    scores,
    softmax_stats,
    tiled_online_attention,
    kv_head_of,
    visible,
    visible_window,
    probabilities_window,
    visible_block_sparse,
    layout_index,
    attention_head_block_sparse,
    attention_ref_block_sparse,
    gather_pages,
    visible_decode,
    decode_paged_ref,
)
from .attention_grad import (  # noqa: F401
    attention_grad_head,
    attention_grad_ref,
    attention_grad_ref_gqa,
    delta_rows,
    grad_magnitudes_head,
)
from . import fp8_attention  # noqa: F401
