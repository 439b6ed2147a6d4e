"""fp64 CPU oracle for memory-efficient exact attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``memory_efficient_exact_tiled_amd``) never imports
it, shares no code with it and has no CPU fallback.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against library routines, closed forms and the
invariants the pages fix. Two readings are parity unpinned by the pages: the
form of ALiBi without a causal mask, and the block-sparse mask (64 x 64
blocks ANDed with the causal rule; the pages name a block-sparse variant
without defining it). Both are tested against the stated reading only (the
block mask against torch SDPA with the element mask the blocks expand to).
"""
from .attention import (  # noqa: F401
    BLOCK,
    attend,
    attend_grad,
    bwd,
    decode,
    decode_bits,
    fwd,
    fwd_kvcache,
    fwd_rows,
    kv_append,
    kv_head,
)
