"""FP64 CPU oracle for selected-key and split-K flash attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

attention.py  vectorised FP64 definition (NumPy), the one the tests compare to.
brute.py      an independent scalar twin in pure Python for tiny shapes.

Parity status of each function is stated in the header of attention.py.
"""

from .attention import (  # noqa: F401
    kv_to_f64,
    tree_path,
    visible_decode_row,
    visible_mask_row,
    visible_selection,
    scores,
    attend_scores,
    partial_scores,
    combine_partials,
    decode,
    decode_split,
    prefill,
    prefill_split,
    visited_decode,
    visited_prefill,
)
