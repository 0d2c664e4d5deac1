"""Independent fp64 CPU oracle for verification attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library never does,
and this package imports nothing from the product. Every function cites the
passage of SpecStream ("Resource-Efficient Speculative Decoding for
Long-Context LLM Serving", section 4.2) or of the Speculative Streaming post it
follows.

`tiering` follows section 4.1 of the same paper (Eq. 4-5: which committed
history migrates to the host, and when). `sparse` reads the block importance
statistics and block-sparse verification of the SparseSpec-L and Dustin
abstracts on the same pages.

Pins: every function here is checked by tests that do not reuse its code
(pure-Python brute force, a library SDPA cross-check, the worked mask example
printed in the Speculative Streaming post, closed forms and invariants).
"""

from . import sparse, tiering  # noqa: F401
from .verify_attention import (  # noqa: F401
    NEG_INF,
    attention_reference,
    attention_slice,
    candidate_state,
    chain_mask,
    chunk_list,
    chunk_slot_states,
    chunked_attention,
    empty_state,
    finalize,
    local_state,
    mask_to_bits,
    merge_slots,
    merge_states,
    tree_depths,
    tree_mask,
    visibility,
)
