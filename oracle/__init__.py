"""fp64 CPU oracle for memory-efficient exact attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``memory_efficient_exact_tiled_amd``) never imports
it, shares no code with it and has no CPU fallback.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against library routines, closed forms and the
invariants the pages fix. One reading is parity unpinned by the pages: the
form of ALiBi without a causal mask (it is tested against the stated reading
only).
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
