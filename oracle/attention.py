"""fp64 CPU oracle: exact scaled-dot-product attention written as its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What it computes, and where the pages fix it
--------------------------------------------
The memory-efficient method is exact: it reaches the same result as standard
attention, only without storing the score matrix ("FlashAttention (2022):
l'attenzione che non satura la memoria", section "L'idea: non scrivere mai la
matrice intera"; the xFormers tutorial "Come costruire Transformer efficienti
in memoria con xFormers...", section "Impostare xFormers e Validare
l'Attenzione Memory-Efficient", which validates it against a standard
implementation up to fp16 rounding). So this oracle is the plain definition,
in float64, with the full score block of one (segment, head) held at once:

  scores  = scale * q k^T                      (briefia.fr page "Transformer :
                                                 comprendre l'entrainement et
                                                 l'inference", class SelfAttention)
  scores += ALiBi bias                          (xFormers tutorial, section
                                                 "Utilizzare SwiGLU e ALiBi")
  masked  -> -inf                               (causal: the same code's lower-
                                                 triangular mask, shifted by the
                                                 number of cached tokens)
  p       = softmax over the allowed keys
  o       = p v ;  lse = log sum exp(scores)

Readings taken where the pages are silent (each also listed in the design doc):

* scale is the caller's float32 value, widened exactly to float64;
* causal alignment is bottom-right: query i of a segment with M queries and N
  keys sees key j iff ``j <= i + (N - M)``. The KV-cache code of the
  briefia.fr page builds its causal mask as a lower triangle shifted right by
  the number of cached tokens, which is this rule; for M == N it is the usual
  lower triangle;
* ALiBi adds ``-slope[h] * |(i + N - M) - j|`` (segment-local positions,
  query head ``h``, slope as the caller's float32) after scaling and before
  masking; the pages name ALiBi but print no formula;
* grouped-query attention maps query head ``h`` to KV head
  ``h // (Hq // Hkv)``: the tutorial's GQA snippet lays q out as
  ``[B, M, G, Hq/G, K]`` against k, v ``[B, M, G, 1, K]``, so consecutive
  query heads share one KV head;
* a query row with no allowed key returns o = 0 and lse = -inf;
* decode: the newest token's k/v is already in the cache (briefia.fr page,
  section "Pre-remplissage et decodage"); its query, at position ctx-1,
  attends to cache rows 0..ctx-1;
* block-sparse attention (the FlashAttention page, section on what the
  numbers showed, names a block-sparse variant without defining it): a
  boolean mask over blocks of ``BLOCK`` x ``BLOCK`` (query row, key) index
  pairs, the same for every batch row and head; a pair is allowed only if its
  block is on, and under a causal mask only if the causal rule allows it too.
  Positions are the dense row and key indices (block (i // BLOCK, j // BLOCK));
* backward: the gradients of the loss sum(dO * o) with respect to q, k and v
  (not the slopes, not the scale), for an upstream gradient dO. The
  FlashAttention page (section on the softmax that needs not see the whole
  row) says only that the backward recomputes the scores instead of storing
  them; the gradient itself is the derivative of the definition above, written
  out with the softmax Jacobian: dP = dO v^T, dS = P * (dP - rowsum(P * dP)),
  dq = scale dS k, dk = scale dS^T q, dv = P^T dO. A KV head shared by several
  query heads (GQA) receives the sum over them; rows with no allowed key
  contribute nothing.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64   # block edge of block-sparse masks (query rows and keys)


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of fp16/bf16 -> exactly equal float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head used by query head ``h`` (tutorial GQA snippet: q ``[.., G, Hq/G, K]``
    against k, v ``[.., G, 1, K]``)."""
    return h // (Hq // Hkv)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
           slopes=None, rows=None, block_mask=None):
    """Attention of one segment, float64 throughout.

    q ``[M, Hq, D]``, k and v ``[N, Hkv, D]`` (float64). ``rows`` optionally
    selects which query rows to compute (default all). ``block_mask``
    (``[ceil(M/BLOCK), ceil(N/BLOCK)]`` booleans) keeps only the pairs whose
    block is on. Returns ``(o [len(rows), Hq, D], lse [Hq, len(rows)])``.
    """
    M, Hq, D = q.shape
    N, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    sc = float(np.float32(scale))
    i = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(N)
    pos_i = i + (N - M)                       # bottom-right aligned query position
    if causal:
        allowed = j[None, :] <= pos_i[:, None]
    else:
        allowed = np.ones((len(i), N), dtype=bool)
    if block_mask is not None:
        allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // BLOCK, j[None, :] // BLOCK]
    any_allowed = allowed.any(axis=1)

    o = np.zeros((len(i), Hq, D), dtype=np.float64)
    lse = np.full((Hq, len(i)), -np.inf, dtype=np.float64)
    if N == 0 or len(i) == 0:
        return o, lse
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        s = sc * (q[i, h, :] @ k[:, g, :].T)
        if slopes is not None:
            slope = float(np.float32(slopes[h]))
            s = s - slope * np.abs(pos_i[:, None] - j[None, :]).astype(np.float64)
        s = np.where(allowed, s, -np.inf)
        m = np.where(any_allowed, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        l = e.sum(axis=1)
        safe_l = np.where(l > 0, l, 1.0)
        o[:, h, :] = np.where(any_allowed[:, None], (e @ v[:, g, :]) / safe_l[:, None], 0.0)
        lse[h] = np.where(any_allowed, m + np.log(safe_l), -np.inf)
    return o, lse


def _segments(B, M, N, seqstart_q, seqstart_k):
    if seqstart_q is None:
        return [(b, 0, M, 0, N) for b in range(B)]
    sq = np.asarray(seqstart_q, dtype=np.int64)
    sk = np.asarray(seqstart_k if seqstart_k is not None else seqstart_q, dtype=np.int64)
    return [(0, int(sq[s]), int(sq[s + 1]), int(sk[s]), int(sk[s + 1])) for s in range(len(sq) - 1)]


def fwd(q_bits, k_bits, v_bits, dtype: str, scale: float, causal: bool = False,
        seqstart_q=None, seqstart_k=None, alibi_slopes=None, block_mask=None):
    """Forward attention over bit-pattern inputs.

    Dense: q ``[B,M,Hq,D]``, k/v ``[B,N,Hkv,D]``. Packed (block-diagonal): q
    ``[1,T_q,Hq,D]``, k/v ``[1,T_k,Hkv,D]`` and int prefix sums ``seqstart_q``
    (``seqstart_k`` defaults to it): query segment s sees only key segment s
    (tutorial section "Utilizzare Sequenze di Lunghezza Variabile",
    BlockDiagonalMask / BlockDiagonalCausalMask).

    ``block_mask`` (dense only): see :func:`attend`.

    Returns ``(o, lse)``: o float64 shaped like q, lse ``[B, Hq, M]`` (dense)
    or ``[1, Hq, T_q]`` (packed).
    """
    if block_mask is not None and seqstart_q is not None:
        raise ValueError("block-sparse masks are defined for dense batches")
    q = decode_bits(q_bits, dtype)
    k = decode_bits(k_bits, dtype)
    v = decode_bits(v_bits, dtype)
    B, M, Hq, D = q.shape
    N = k.shape[1]
    o = np.zeros_like(q)
    lse = np.full((B, Hq, M), -np.inf)
    for b, q0, q1, k0, k1 in _segments(B, M, N, seqstart_q, seqstart_k):
        ob, lb = attend(q[b, q0:q1], k[b, k0:k1], v[b, k0:k1], scale, causal, alibi_slopes, block_mask=block_mask)
        o[b, q0:q1] = ob
        lse[b, :, q0:q1] = lb
    return o, lse


def fwd_rows(q_bits, k_bits, v_bits, dtype: str, scale: float, b: int, rows, causal: bool = False,
             seqstart_q=None, seqstart_k=None, segment: int | None = None, alibi_slopes=None, block_mask=None):
    """Selected query rows of :func:`fwd` for one batch row ``b`` (dense) or one
    packed ``segment`` (then ``rows`` are segment-local). Only that batch row
    or segment is decoded, so this stays cheap at full workload sizes."""
    if seqstart_q is None:
        q = decode_bits(q_bits[b], dtype)
        k = decode_bits(k_bits[b], dtype)
        v = decode_bits(v_bits[b], dtype)
    else:
        sq = np.asarray(seqstart_q, dtype=np.int64)
        sk = np.asarray(seqstart_k if seqstart_k is not None else seqstart_q, dtype=np.int64)
        q = decode_bits(q_bits[0, sq[segment]:sq[segment + 1]], dtype)
        k = decode_bits(k_bits[0, sk[segment]:sk[segment + 1]], dtype)
        v = decode_bits(v_bits[0, sk[segment]:sk[segment + 1]], dtype)
    return attend(q, k, v, scale, causal, alibi_slopes, rows=rows, block_mask=block_mask)


def decode(q_bits, kcache_bits, vcache_bits, ctx_lens, dtype: str, scale: float,
           alibi_slopes=None, batches=None):
    """One KV-cache decode step.

    q ``[B,Hq,D]``; caches ``[B,S_max,Hkv,D]``; the query of batch row b sits at
    position ``ctx_lens[b]-1`` and attends to cache rows ``0..ctx_lens[b]-1``
    (its own k/v already appended). Rows not in ``batches`` are left NaN.
    Returns o float64 ``[B,Hq,D]``.
    """
    B, Hq, D = q_bits.shape
    o = np.full((B, Hq, D), np.nan)
    for b in (range(B) if batches is None else batches):
        n = int(ctx_lens[b])
        qb = decode_bits(q_bits[b], dtype)[None]
        kb = decode_bits(kcache_bits[b, :n], dtype)
        vb = decode_bits(vcache_bits[b, :n], dtype)
        ob, _ = attend(qb, kb, vb, scale, causal=True, slopes=alibi_slopes)
        o[b] = ob[0]
    return o


def fwd_kvcache(q_bits, kcache_bits, vcache_bits, ctx_lens, dtype: str, scale: float, causal: bool = True,
                alibi_slopes=None, batches=None):
    """The M newest queries of each sequence against its KV cache (chunked
    prefill / multi-token decode).

    q ``[B,M,Hq,D]`` holds the queries of positions ``ctx-M .. ctx-1`` of
    sequence b, whose keys and values are already in the cache
    ``[B,S_max,Hkv,D]``; they attend to cache rows ``0..ctx-1`` with the
    bottom-right causal alignment of the briefia.fr KV-cache code (row i sees
    keys j <= i + ctx - M). Returns ``(o [B,M,Hq,D], lse [B,Hq,M])``; rows of
    batch entries not in ``batches`` are NaN.
    """
    B, M, Hq, D = q_bits.shape
    o = np.full((B, M, Hq, D), np.nan)
    lse = np.full((B, Hq, M), np.nan)
    for b in (range(B) if batches is None else batches):
        n = int(ctx_lens[b])
        ob, lb = attend(decode_bits(q_bits[b], dtype), decode_bits(kcache_bits[b, :n], dtype),
                        decode_bits(vcache_bits[b, :n], dtype), scale, causal, alibi_slopes)
        o[b], lse[b] = ob, lb
    return o, lse


def kv_append(kcache_bits, vcache_bits, k_new_bits, v_new_bits, ctx_lens):
    """Cache after appending T new rows per sequence at positions ctx..ctx+T-1
    (rows that would fall past S_max are dropped). Bit patterns in, bit
    patterns out: appending is a copy (briefia.fr page, section on the simple
    KV cache: each decode step concatenates the new key and value)."""
    kc, vc = np.array(kcache_bits, copy=True), np.array(vcache_bits, copy=True)
    B, S_max = kc.shape[:2]
    T = k_new_bits.shape[1]
    for b in range(B):
        c = int(ctx_lens[b])
        n = max(0, min(T, S_max - c))
        kc[b, c:c + n] = k_new_bits[b, :n]
        vc[b, c:c + n] = v_new_bits[b, :n]
    return kc, vc


def attend_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                causal: bool = False, slopes=None, block_mask=None):
    """Gradients of sum(do * attend(q, k, v)[0]) for one segment, float64.

    q, do ``[M, Hq, D]``; k, v ``[N, Hkv, D]``. The attention weights are
    recomputed from q and k (nothing from the forward is reused). Returns
    ``(dq [M,Hq,D], dk [N,Hkv,D], dv [N,Hkv,D])``.
    """
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    if do.shape != q.shape or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    sc = float(np.float32(scale))
    dq = np.zeros((M, Hq, D))
    dk = np.zeros((N, Hkv, D))
    dv = np.zeros((N, Hkv, D))
    if M == 0 or N == 0:
        return dq, dk, dv
    i = np.arange(M)
    j = np.arange(N)
    pos = i + (N - M)
    allowed = (j[None, :] <= pos[:, None]) if causal else np.ones((M, N), dtype=bool)
    if block_mask is not None:
        allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // BLOCK, j[None, :] // BLOCK]
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        s = sc * (q[:, h, :] @ k[:, g, :].T)
        if slopes is not None:
            s = s - float(np.float32(slopes[h])) * np.abs(pos[:, None] - j[None, :]).astype(np.float64)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, initial=-np.inf)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        tot = e.sum(axis=1, keepdims=True)
        p = e / np.where(tot > 0, tot, 1.0)             # rows with no key: p = 0
        dp = do[:, h, :] @ v[:, g, :].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[:, h, :] = sc * (ds @ k[:, g, :])
        dk[:, g, :] += sc * (ds.T @ q[:, h, :])
        dv[:, g, :] += p.T @ do[:, h, :]
    return dq, dk, dv


def bwd(q_bits, k_bits, v_bits, do_bits, dtype: str, scale: float, causal: bool = False,
        seqstart_q=None, seqstart_k=None, alibi_slopes=None, batches=None, block_mask=None):
    """Backward of :func:`fwd` over bit-pattern inputs (same layouts; ``do``
    shaped like q). Returns float64 ``(dq, dk, dv)`` shaped like q, k, v.
    Dense batch rows not in ``batches`` are left NaN (packed inputs are one row)."""
    if block_mask is not None and seqstart_q is not None:
        raise ValueError("block-sparse masks are defined for dense batches")
    q = decode_bits(q_bits, dtype)
    k = decode_bits(k_bits, dtype)
    v = decode_bits(v_bits, dtype)
    do = decode_bits(do_bits, dtype)
    B, M = q.shape[:2]
    N = k.shape[1]
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    keep = set(range(B) if batches is None else batches)
    for b in keep:
        dk[b] = 0.0
        dv[b] = 0.0
        dq[b] = 0.0
    for b, q0, q1, k0, k1 in _segments(B, M, N, seqstart_q, seqstart_k):
        if b not in keep:
            continue
        g = attend_grad(q[b, q0:q1], k[b, k0:k1], v[b, k0:k1], do[b, q0:q1], scale, causal, alibi_slopes,
                        block_mask=block_mask)
        dq[b, q0:q1] = g[0]
        dk[b, k0:k1] = g[1]
        dv[b, k0:k1] = g[2]
    return dq, dk, dv
