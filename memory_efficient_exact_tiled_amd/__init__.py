"""Memory-efficient exact attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``libmea.so`` (``include/mea.h``); this package is its thin Python binding:

* :func:`fwd` - tiled exact attention forward (causal, packed block-diagonal,
  grouped-query, ALiBi);
* :func:`fwd_blocksparse` - the forward over a 64 x 64 block-sparse pattern;
* :func:`bwd` - its backward (dq, dk, dv with the scores recomputed);
* :func:`decode` - one KV-cache decode step (split-KV partials + combine);
* :func:`decode_noalloc` - the same step with the library's static per-device
  scratch, for callers that cannot allocate;
* :func:`fwd_kvcache` - chunked prefill / multi-token decode over a KV cache;
* :func:`kv_append` - append new key/value rows to a KV cache.

Import fails if the library has not been built
(``python memory_efficient_exact_tiled_amd/build.py``).
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MEA_BF16,
    MEA_BIAS_ALIBI,
    MEA_DECODE_NOALLOC_SCRATCH_BYTES,
    MEA_EHIP,
    MEA_EINVAL,
    MEA_ESCRATCH,
    MEA_EUNSUPPORTED,
    MEA_EWORKSPACE,
    MEA_FP16,
    MEA_MASK_BLOCKDIAG,
    MEA_MASK_CAUSAL,
    MEA_OK,
    MeaError,
    bwd,
    block_sparse_block,
    bwd_workspace_bytes,
    decode,
    decode_chunk,
    decode_noalloc,
    decode_workspace_bytes,
    fwd,
    fwd_blocksparse,
    fwd_kvcache,
    kv_append,
    lib,
    strerror,
    supported,
)
