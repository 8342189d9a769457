"""CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product path (the HIP
library and its binding) never imports, links or calls it, and the two share
no code.

Parity unpinned: nothing.  Every function here is tied to a passage of the
pages by a CPU test (worked examples, closed forms, a library routine, or a
second, independent formulation from the pages).
"""
from .oracle import (  # noqa: F401
    ORC_BF16,
    ORC_F32,
    blocks_needed,
    capacity,
    copy_blocks,
    decode,
    fragmentation_ratio,
    gather,
    gather_flat_index,
    gather_loop_cat,
    last_block_fill,
    library_path,
    prefill,
    scatter,
    scatter_index_put,
    slot_mapping,
    swap_in,
    swap_out,
)
from .block_manager import BlockManagerOracle  # noqa: F401
from . import quant  # noqa: F401
