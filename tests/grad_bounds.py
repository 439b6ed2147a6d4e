"""Per-element error bounds of the backward kernels' gradients (test infrastructure).

Every gradient element is a sum of products; its rounding error is bounded by
a small multiple of the unit roundoff u of the input type (2^-8 bf16, 2^-11
fp16) times the sum of the MAGNITUDES of its own terms, not by the largest
gradient of the tensor. With P the softmax weights, dP = dO v^T, the row
term Delta_i = sum_d dO_id o_id and dS = P (dP - Delta) (the derivative of the
definition, as the oracle writes it), the kernels compute

  dv_j = sum_i P_ij dO_i          dq_i = scale sum_j dS_ij k_j
  dk_j = scale sum_i dS_ij q_i

with these roundings, each relative to the quantity it touches:
  * P is recomputed from the forward's lse, whose error is at most 1.25 u, and
    P is rounded to the input type before its product (u);
  * Delta is formed from the forward's stored output, whose elements are off
    by at most 3 u sum_j P_ij |v_jd| (the rounded weights of the forward's P.V,
    2 u, and the output's own rounding, u), so
    |d Delta_i| <= 3 u A_i with A_i = sum_d |dO_id| (P |v|)_id;
  * dP and Delta are fp32 dot products of D terms, each within gamma_D =
    D 2^-24 of the sum of its terms' magnitudes, B_ij = sum_d |dO_id| (|v_jd| +
    |o_id|) for their difference;
  * dS is rounded to the input type before its products (u), and each stored
    gradient once more (u).
Values too small for the format are an absolute error: rounding P or dS to
fp16 below its normal range moves them by up to eta = 2^-25 (half the
subnormal spacing 2^-24), and for bf16 the fp32 exponentials and products
underflow below 2^-126 (eta = 2^-126 covers flushing them to zero). Summed to
first order, over the allowed pairs only:
  |err dv_jd| <= 3.25 u sum_i P_ij |dO_id| + eta (sum_i |dO_id| + 1)
  |err dq_id| <= scale sum_j |k_jd| (3.25 u |dS_ij| + 3 u P_ij A_i + 2 gamma_D P_ij B_ij + eta) + eta
and dk like dq with q in place of k. ``grad_terms`` returns the bracketed
magnitude sums T with the u factors taken out (E_ij = P_ij (3 A_i +
2 gamma_D / u B_ij) + eta / u beside |dS_ij|), so that the bar of every
element is ``C * u * T`` with C = 4 (3.25 to first order, the rest for fp32
accumulation over up to a few thousand keys, whose random-walk error is far
below u).

``grad_terms`` also returns the gradients summed from the same P and dS, which
a CPU test compares with the oracle's backward to 1e-12: the terms bounded
here are the terms of the oracle's gradients.
"""
from __future__ import annotations

import numpy as np

import oracle.attention as orc

U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
ETA = {"fp16": 2.0 ** -25, "bf16": 2.0 ** -126}
C = 4.0


def _segments(B, M, N, seqstart_q, seqstart_k):
    if seqstart_q is None:
        return [(b, 0, M, 0, N) for b in range(B)]
    sq = np.asarray(seqstart_q, dtype=np.int64)
    sk = np.asarray(seqstart_k if seqstart_k is not None else seqstart_q, dtype=np.int64)
    return [(0, int(sq[s]), int(sq[s + 1]), int(sk[s]), int(sk[s + 1])) for s in range(len(sq) - 1)]


def _segment_terms(q, k, v, do, scale, u, eta, causal, slopes, block_mask):
    """(dq, dk, dv, Tdq, Tdk, Tdv) of one segment, float64."""
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    out = [np.zeros((M, Hq, D)), np.zeros((N, Hkv, D)), np.zeros((N, Hkv, D)),
           np.zeros((M, Hq, D)), np.zeros((N, Hkv, D)), np.zeros((N, Hkv, D))]
    if M == 0 or N == 0:
        return out
    dq, dk, dv, tq, tk, tv = out
    sc = float(np.float32(scale))
    gamma = D * 2.0 ** -24
    i = np.arange(M)
    j = np.arange(N)
    pos = i + (N - M)
    allowed = (j[None, :] <= pos[:, None]) if causal else np.ones((M, N), dtype=bool)
    if block_mask is not None:
        allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // orc.BLOCK, j[None, :] // orc.BLOCK]
    for h in range(Hq):
        g = orc.kv_head(h, Hq, Hkv)
        s = sc * (q[:, h, :] @ k[:, g, :].T)
        if slopes is not None:
            s = s - float(np.float32(slopes[h])) * np.abs(pos[:, None] - j[None, :]).astype(np.float64)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, initial=-np.inf)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        tot = e.sum(axis=1, keepdims=True)
        p = e / np.where(tot > 0, tot, 1.0)
        dp = do[:, h, :] @ v[:, g, :].T
        o = p @ v[:, g, :]
        delta = np.sum(do[:, h, :] * o, axis=1, keepdims=True)
        ds = p * (dp - delta)
        a = np.sum(np.abs(do[:, h, :]) * (p @ np.abs(v[:, g, :])), axis=1, keepdims=True)
        bm = np.abs(do[:, h, :]) @ np.abs(v[:, g, :]).T + np.sum(np.abs(do[:, h, :] * o), axis=1, keepdims=True)
        fl = (eta / u) * allowed
        w = np.abs(ds) + p * (3.0 * a + (2.0 * gamma / u) * bm) + fl
        dq[:, h, :] = sc * (ds @ k[:, g, :])
        dk[:, g, :] += sc * (ds.T @ q[:, h, :])
        dv[:, g, :] += p.T @ do[:, h, :]
        tq[:, h, :] = sc * (w @ np.abs(k[:, g, :]))
        tk[:, g, :] += sc * (w.T @ np.abs(q[:, h, :]))
        tv[:, g, :] += (p + fl).T @ np.abs(do[:, h, :])
    for t in (tq, tk, tv):
        t += eta / u          # the stored gradient's own rounding
    return out


def grad_terms(q_bits, k_bits, v_bits, do_bits, dtype: str, scale: float, causal: bool = False,
               seqstart_q=None, seqstart_k=None, alibi_slopes=None, block_mask=None, batches=None):
    """``(grads, terms)``: the gradients (dq, dk, dv) summed from P and dS, and
    their per-element magnitude sums (Tdq, Tdk, Tdv) as described in the
    module docstring. Layouts as the oracle's ``bwd``; dense batch rows not in
    ``batches`` are NaN."""
    u, eta = U[dtype], ETA[dtype]
    q = orc.decode_bits(q_bits, dtype)
    k = orc.decode_bits(k_bits, dtype)
    v = orc.decode_bits(v_bits, dtype)
    do = orc.decode_bits(do_bits, dtype)
    B, M = q.shape[:2]
    N = k.shape[1]
    res = [np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan),
           np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan)]
    keep = set(range(B) if batches is None else batches)
    for b in keep:
        for r in res:
            r[b] = 0.0
    for b, q0, q1, k0, k1 in _segments(B, M, N, seqstart_q, seqstart_k):
        if b not in keep:
            continue
        seg = _segment_terms(q[b, q0:q1], k[b, k0:k1], v[b, k0:k1], do[b, q0:q1], scale, u, eta, causal,
                             alibi_slopes, block_mask)
        for idx, (r, x) in enumerate(zip(res, seg)):
            sl = slice(q0, q1) if idx in (0, 3) else slice(k0, k1)
            r[b, sl] = x
    return tuple(res[:3]), tuple(res[3:])


def check_grads(name, got, want, terms, dtype, say=print):
    """Element-wise bar: |got - want| <= C u T for every element (NaN entries of
    ``want`` are not compared). ``got`` are float64 host arrays. Returns the
    largest error/bar ratio; raises AssertionError naming the worst element."""
    u = U[dtype]
    worst = 0.0
    for label, g, w, t in zip(("dq", "dk", "dv"), got, want, terms):
        sel = ~np.isnan(w)
        err = np.where(sel, np.abs(g - np.where(sel, w, 0.0)), 0.0)
        bar = C * u * np.where(sel, t, 0.0)
        ratio = np.where(bar > 0, err / np.where(bar > 0, bar, 1.0), np.where(err > 0, np.inf, 0.0))
        at = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
        r = float(ratio[at]) if ratio.size else 0.0
        say(f"[{name} {label}] max err/bar={r:.3f} (err={float(err[at]) if ratio.size else 0:.3e}, "
            f"bar={float(bar[at]) if ratio.size else 0:.3e} at {at}); max_abs_err={float(err.max(initial=0)):.3e}")
        assert r <= 1.0, (name, label, at, r)
        worst = max(worst, r)
    return worst
