"""Seeded synthetic inputs for the attention workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no attention arithmetic. It only

* draws N(0,1) float32 samples from numpy's PCG64 generator (one independent
  stream per tensor, derived from the seed with ``numpy.random.SeedSequence``),
* rounds them once, round-to-nearest-even, to fp16 or bf16 and returns the raw
  16-bit patterns as ``uint16`` arrays, and
* draws the integer lengths (packed segment lengths, decode context lengths).

Both sides receive identical bits: the oracle decodes them to float64 itself,
the GPU path hands them to the kernels as fp16/bf16 device tensors.

The workloads follow the pages' own examples: N(0,1) q/k/v in the
``[B, M, H, K]`` layout of the xFormers tutorial (chipsbuilder.com page,
"Applicare Attenzione Causale" and GQA snippets), head dim 64 or 128.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("fp16", "bf16")

# Tensor ids for SeedSequence spawning; fixed so that a tensor's values do not
# depend on which other tensors a caller asks for.
_Q, _K, _V, _LEN, _KC, _VC = 0, 1, 2, 3, 4, 5


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> uint16 bit patterns of fp16 or bf16, round-to-nearest-even.

    Inputs must be finite (they are N(0,1) draws)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        b = x.view(np.uint32)
        rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return rounded.astype(np.uint16)
    raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


def normal_bits(seed: int, shape, dtype: str, *stream: int) -> np.ndarray:
    """N(0,1) float32 draws of ``shape`` rounded to ``dtype`` bits."""
    g = _rng(seed, *stream)
    return round_bits(g.standard_normal(size=tuple(shape), dtype=np.float32), dtype)


def dense_case(seed: int, B: int, M: int, N: int, Hq: int, Hkv: int, D: int, dtype: str) -> dict:
    """q ``[B,M,Hq,D]``, k and v ``[B,N,Hkv,D]`` as uint16 bit patterns."""
    return {
        "q": normal_bits(seed, (B, M, Hq, D), dtype, _Q),
        "k": normal_bits(seed, (B, N, Hkv, D), dtype, _K),
        "v": normal_bits(seed, (B, N, Hkv, D), dtype, _V),
        "dtype": dtype,
    }


def segment_lengths(seed: int, nseq: int, lo: int, hi: int) -> np.ndarray:
    """``nseq`` lengths uniform on the integers ``[lo, hi]`` (both ends included)."""
    return _rng(seed, _LEN).integers(lo, hi + 1, size=nseq).astype(np.int64)


def seqstart(lengths) -> np.ndarray:
    """Prefix sums ``[0, L0, L0+L1, ...]`` as int32 (the packed-batch boundaries)."""
    s = np.zeros(len(lengths) + 1, dtype=np.int64)
    s[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if s[-1] > np.iinfo(np.int32).max:
        raise ValueError("packed length exceeds int32")
    return s.astype(np.int32)


def varlen_case(seed: int, lengths, Hq: int, Hkv: int, D: int, dtype: str) -> dict:
    """Segments of the given lengths packed with no padding: q ``[1,T,Hq,D]``,
    k and v ``[1,T,Hkv,D]`` with ``T = sum(lengths)``; ``seqstart`` int32 ``[nseq+1]``."""
    st = seqstart(lengths)
    T = int(st[-1])
    return {
        "q": normal_bits(seed, (1, T, Hq, D), dtype, _Q),
        "k": normal_bits(seed, (1, T, Hkv, D), dtype, _K),
        "v": normal_bits(seed, (1, T, Hkv, D), dtype, _V),
        "seqstart": st,
        "lengths": np.asarray(lengths, dtype=np.int64),
        "dtype": dtype,
    }


def varlen_cross_case(seed: int, q_lengths, k_lengths, Hq: int, Hkv: int, D: int, dtype: str) -> dict:
    """Packed batch whose query and key segments differ in length (segment s
    of q attends to segment s of k): q ``[1,Tq,Hq,D]``, k and v ``[1,Tk,Hkv,D]``,
    ``seqstart_q`` and ``seqstart_k`` int32 ``[nseq+1]``."""
    sq, sk = seqstart(q_lengths), seqstart(k_lengths)
    return {
        "q": normal_bits(seed, (1, int(sq[-1]), Hq, D), dtype, _Q),
        "k": normal_bits(seed, (1, int(sk[-1]), Hkv, D), dtype, _K),
        "v": normal_bits(seed, (1, int(sk[-1]), Hkv, D), dtype, _V),
        "seqstart_q": sq,
        "seqstart_k": sk,
        "dtype": dtype,
    }


def alibi_slopes(Hq: int) -> np.ndarray:
    """Per-query-head ALiBi slopes ``2^(-8(h+1)/Hq)``, h = 0..Hq-1, as float32."""
    h = np.arange(Hq, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / Hq).astype(np.float32)


# Bit pattern written into KV-cache slots at or beyond a sequence's context
# length: a quiet NaN. No correct decode may read these slots.
POISON = {"fp16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def context_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence decode context lengths uniform on ``[lo, hi]``, int32."""
    return _rng(seed, _LEN).integers(lo, hi + 1, size=B).astype(np.int32)


def decode_case(seed: int, ctx_lens, S_max: int, Hq: int, Hkv: int, D: int, dtype: str,
                batches=None) -> dict:
    """One decode step: q ``[B,Hq,D]``; caches ``[B,S_max,Hkv,D]`` whose slots
    ``>= ctx_lens[b]`` hold NaN bit patterns.

    Row ``b`` of each cache is drawn from its own stream, so ``batches`` (a list
    of batch indices) may restrict generation to a few rows: the other rows are
    then left poisoned in full. ``q`` is always drawn in full."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    B = len(ctx)
    if np.any(ctx < 0) or np.any(ctx > S_max):
        raise ValueError("context lengths must lie in [0, S_max]")
    kc = np.full((B, S_max, Hkv, D), POISON[dtype], dtype=np.uint16)
    vc = np.full((B, S_max, Hkv, D), POISON[dtype], dtype=np.uint16)
    for b in (range(B) if batches is None else batches):
        n = int(ctx[b])
        kc[b, :n] = normal_bits(seed, (n, Hkv, D), dtype, _KC, b)
        vc[b, :n] = normal_bits(seed, (n, Hkv, D), dtype, _VC, b)
    return {
        "q": normal_bits(seed, (B, Hq, D), dtype, _Q),
        "kcache": kc,
        "vcache": vc,
        "ctx_lens": ctx.astype(np.int32),
        "dtype": dtype,
    }


def decode_cache_rows(seed: int, b: int, n: int, Hkv: int, D: int, dtype: str):
    """The first ``n`` rows of batch row ``b`` of (kcache, vcache), as drawn by
    :func:`decode_case`. Lets a caller fill a large device cache row by row."""
    return (normal_bits(seed, (n, Hkv, D), dtype, _KC, b),
            normal_bits(seed, (n, Hkv, D), dtype, _VC, b))


def random_block_mask(seed: int, n_qblocks: int, n_kblocks: int, density: float, keep_diagonal: bool = True):
    """Seeded boolean block mask ``[n_qblocks, n_kblocks]`` (uint8 0/1): each
    block on with probability ``density``; ``keep_diagonal`` also turns on
    block (r, r) so no query block of a square case is left without keys."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7, 7])))
    m = (rng.random((n_qblocks, n_kblocks)) < density)
    if keep_diagonal:
        r = np.arange(min(n_qblocks, n_kblocks))
        m[r, r] = True
    return m.astype(np.uint8)


def band_global_block_mask(n_qblocks: int, n_kblocks: int, half_width: int, n_global: int):
    """Sliding-window block pattern: query block r sees key blocks
    r - half_width .. r + half_width, plus the first ``n_global`` key blocks
    (global tokens), as uint8 ``[n_qblocks, n_kblocks]``."""
    r = np.arange(n_qblocks)[:, None]
    c = np.arange(n_kblocks)[None, :]
    return ((np.abs(r - c) <= half_width) | (c < n_global)).astype(np.uint8)
