"""Pins of the fp64 oracle to things other than itself.

Each ``check_*`` takes the oracle module (``oracle.attention`` or a mutated
copy of it) and raises ``AssertionError`` when the oracle disagrees with

* a library routine computing the same quantity (torch's float64
  ``scaled_dot_product_attention`` on the CPU, which also decodes fp16/bf16
  bits on its own, and ``torch.logsumexp``),
* a closed form (uniform weights for q = 0, geometric ALiBi weights, the first
  causal row), or
* an invariant the pages fix (block-diagonal == per-segment, GQA == repeated
  K/V, decode == last row of full causal attention, rows summing to one).

``tests/test_oracle_pins.py`` runs them on the oracle; ``tests/test_oracle_mutants.py``
plants mistakes in copies of the oracle and checks that some pin catches each.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import mea_inputs as inp

TOL = 1e-12


def _torch_decode(bits, dtype):
    """fp16/bf16 bits -> float64 torch tensor, using torch's own conversion."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.double()


def _sdpa(q, k, v, scale, causal=False, mask=None, gqa=False):
    """q [B,M,H,D] -> torch SDPA in [B,H,M,D] -> back to [B,M,H,D] (float64, CPU)."""
    out = F.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3),
        attn_mask=mask, is_causal=causal, scale=scale, enable_gqa=gqa)
    return out.permute(0, 2, 1, 3).numpy()


def _maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def _ones_bits(shape, dtype):
    return inp.round_bits(np.ones(shape, np.float32), dtype)


def _bits(x, dtype):
    return inp.round_bits(np.asarray(x, np.float32), dtype)


# --- library routine -------------------------------------------------------

def check_sdpa_nomask(orc):
    for seed, (B, M, N, H, D), dt in [(1, (2, 7, 11, 3, 8), "fp16"), (2, (1, 33, 17, 2, 16), "bf16")]:
        c = inp.dense_case(seed, B, M, N, H, H, D, dt)
        scale = float(np.float32(1.0 / np.sqrt(D)))
        o, _ = orc.fwd(c["q"], c["k"], c["v"], dt, scale)
        ref = _sdpa(_torch_decode(c["q"], dt), _torch_decode(c["k"], dt), _torch_decode(c["v"], dt), scale)
        assert _maxerr(o, ref) < TOL, ("sdpa nomask", _maxerr(o, ref))


def check_sdpa_causal_square(orc):
    for seed, (B, M, H, D), dt in [(3, (2, 19, 2, 8), "fp16"), (4, (1, 40, 3, 16), "bf16")]:
        c = inp.dense_case(seed, B, M, M, H, H, D, dt)
        scale = 0.3
        o, _ = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=True)
        ref = _sdpa(_torch_decode(c["q"], dt), _torch_decode(c["k"], dt), _torch_decode(c["v"], dt),
                    float(np.float32(scale)), causal=True)
        assert _maxerr(o, ref) < TOL, ("sdpa causal", _maxerr(o, ref))


def check_sdpa_gqa(orc):
    # torch's enable_gqa repeats each KV head over a contiguous run of query heads.
    c = inp.dense_case(5, 2, 13, 21, 8, 2, 16, "bf16")
    scale = 0.25
    o, _ = orc.fwd(c["q"], c["k"], c["v"], "bf16", scale)
    ref = _sdpa(_torch_decode(c["q"], "bf16"), _torch_decode(c["k"], "bf16"),
                _torch_decode(c["v"], "bf16"), scale, gqa=True)
    assert _maxerr(o, ref) < TOL, ("sdpa gqa", _maxerr(o, ref))


def check_sdpa_alibi_causal_as_key_bias(orc):
    """Under a causal mask the bias -slope*|i - j| differs from +slope*j by a
    per-row constant, which softmax ignores; torch SDPA with the additive float
    mask slope*j (a form with no |.| and no query index) must agree."""
    B, M, H, D = 1, 24, 4, 8
    c = inp.dense_case(6, B, M, M, H, H, D, "fp16")
    slopes = inp.alibi_slopes(H)
    scale = 0.35
    o, _ = orc.fwd(c["q"], c["k"], c["v"], "fp16", scale, causal=True, alibi_slopes=slopes)
    j = torch.arange(M, dtype=torch.float64)
    causal = torch.ones(M, M, dtype=torch.bool).tril()
    mask = torch.where(causal[None], torch.from_numpy(slopes.astype(np.float64))[:, None, None] * j[None, None, :],
                       torch.tensor(-float("inf"), dtype=torch.float64))
    ref = _sdpa(_torch_decode(c["q"], "fp16"), _torch_decode(c["k"], "fp16"), _torch_decode(c["v"], "fp16"),
                float(np.float32(scale)), mask=mask[None])
    assert _maxerr(o, ref) < TOL, ("alibi as key bias", _maxerr(o, ref))


def check_lse_logsumexp(orc):
    c = inp.dense_case(7, 1, 9, 14, 2, 2, 8, "bf16")
    scale = 0.5
    _, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", scale)
    q = _torch_decode(c["q"], "bf16")[0].permute(1, 0, 2)
    k = _torch_decode(c["k"], "bf16")[0].permute(1, 0, 2)
    ref = torch.logsumexp(torch.matmul(q, k.transpose(1, 2)) * scale, dim=-1).numpy()
    assert _maxerr(lse[0], ref) < TOL, ("lse", _maxerr(lse[0], ref))


# --- closed forms ------------------------------------------------------------

def check_rows_sum_to_one(orc):
    """V = 1 everywhere: every row with an allowed key returns exactly 1 (the
    softmax weights sum to one)."""
    for causal, slopes in [(False, None), (True, None), (True, inp.alibi_slopes(4)), (False, inp.alibi_slopes(4))]:
        c = inp.dense_case(8, 2, 12, 12, 4, 2, 8, "bf16")
        v1 = _ones_bits(c["v"].shape, "bf16")
        o, _ = orc.fwd(c["q"], c["k"], v1, "bf16", 0.7, causal=causal, alibi_slopes=slopes)
        assert _maxerr(o, 1.0) < TOL, ("rows sum", causal, _maxerr(o, 1.0))


def check_first_causal_row_is_v0(orc):
    c = inp.dense_case(9, 2, 10, 10, 4, 2, 8, "fp16")
    o, _ = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.4, causal=True, alibi_slopes=inp.alibi_slopes(4))
    v = orc.decode_bits(c["v"], "fp16")
    for h in range(4):
        assert np.array_equal(o[:, 0, h, :], v[:, 0, h // 2, :]), "first causal row"


def check_single_key(orc):
    c = inp.dense_case(10, 1, 5, 1, 2, 1, 8, "bf16")
    o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.9)
    v = orc.decode_bits(c["v"], "bf16")
    assert np.array_equal(o[0, :, 0, :], np.broadcast_to(v[0, 0, 0], (5, 8))), "N=1"
    assert np.array_equal(o[0, :, 1, :], np.broadcast_to(v[0, 0, 0], (5, 8))), "N=1"


def check_zero_query_uniform(orc):
    """q = 0: all scores are 0, so each row is the plain mean of v over the
    allowed keys. With v_j = j the mean exposes the exact allowed index set."""
    for M, N, causal in [(6, 6, True), (4, 9, True), (5, 7, False)]:
        q = np.zeros((1, M, 2, 4), np.uint16)
        k = inp.dense_case(11, 1, M, N, 2, 2, 4, "fp16")["k"]
        vj = np.broadcast_to(np.arange(N, dtype=np.float32)[None, :, None, None], (1, N, 2, 4))
        o, lse = orc.fwd(q, k, _bits(vj, "fp16"), "fp16", 0.5, causal=causal)
        for i in range(M):
            n_allowed = (i + N - M + 1) if causal else N
            assert abs(o[0, i, 0, 0] - (n_allowed - 1) / 2.0) < TOL, ("uniform", M, N, causal, i)
            assert abs(lse[0, 0, i] - np.log(n_allowed)) < TOL, ("uniform lse", i)


def check_zero_query_alibi_geometric(orc):
    """q = 0, causal, ALiBi: weights on key j are r^(i-j) with r = e^-slope, so
    with v_j = j the row mean is the arithmetico-geometric ratio
    i - sum t r^t / sum r^t over t = 0..i (closed forms of both series)."""
    M, H, Hkv = 9, 4, 2           # GQA too: slopes follow the query head
    slopes = inp.alibi_slopes(H)
    q = np.zeros((1, M, H, 4), np.uint16)
    k = inp.dense_case(12, 1, M, M, H, Hkv, 4, "bf16")["k"]
    vj = np.broadcast_to(np.arange(M, dtype=np.float32)[None, :, None, None], (1, M, Hkv, 4))
    o, _ = orc.fwd(q, k, _bits(vj, "bf16"), "bf16", 1.0, causal=True, alibi_slopes=slopes)
    for h in range(H):
        r = np.exp(-float(slopes[h]))
        for i in range(M):
            s0 = (1 - r ** (i + 1)) / (1 - r)
            s1 = r * (1 - (i + 1) * r ** i + i * r ** (i + 1)) / (1 - r) ** 2
            assert abs(o[0, i, h, 0] - (i - s1 / s0)) < 1e-10, ("alibi geometric", h, i)


def check_zero_query_alibi_two_sided(orc):
    """q = 0, no mask, ALiBi: weights r^|i-j|; with v = 1 rows are 1 and with
    v_j = j the mean follows from the two one-sided series (reading of ALiBi
    without a causal mask: the pages give no formula for it)."""
    N, H = 8, 2
    slopes = np.array([0.5, 0.25], np.float32)
    q = np.zeros((1, N, H, 4), np.uint16)
    k = inp.dense_case(13, 1, N, N, H, H, 4, "bf16")["k"]
    vj = np.broadcast_to(np.arange(N, dtype=np.float32)[None, :, None, None], (1, N, H, 4))
    o, _ = orc.fwd(q, k, _bits(vj, "bf16"), "bf16", 1.0, alibi_slopes=slopes)
    for h in range(H):
        r = np.exp(-float(slopes[h]))
        for i in range(N):
            def geo(n):  # sum_{t=0}^{n} r^t and sum t r^t
                s0 = (1 - r ** (n + 1)) / (1 - r)
                s1 = r * (1 - (n + 1) * r ** n + n * r ** (n + 1)) / (1 - r) ** 2
                return s0, s1
            a0, a1 = geo(i)              # keys j = i - t, t = 0..i
            b0, b1 = geo(N - 1 - i)      # keys j = i + t, t = 0..N-1-i
            num = (i * a0 - a1) + (i * b0 + b1) - i   # key i counted twice
            den = a0 + b0 - 1
            assert abs(o[0, i, h, 0] - num / den) < 1e-10, ("alibi two-sided", h, i)


def check_empty_rows(orc):
    """Rows with no allowed key (causal with fewer keys than queries): o = 0,
    lse = -inf (reading for fully masked rows)."""
    c = inp.dense_case(14, 1, 6, 2, 2, 2, 4, "fp16")
    o, lse = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.5, causal=True)
    assert np.all(o[0, :4] == 0) and np.all(np.isneginf(lse[0, :, :4])), "empty rows"
    assert np.all(np.isfinite(o[0, 4:])), "rows after the empty ones"


# --- invariants ----------------------------------------------------------------

def check_blockdiag_equals_per_segment(orc):
    for causal, slopes in [(False, None), (True, inp.alibi_slopes(4))]:
        lengths = [5, 1, 9, 3]
        c = inp.varlen_case(15, lengths, 4, 2, 8, "bf16")
        st = c["seqstart"]
        o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.3, causal=causal,
                         seqstart_q=st, seqstart_k=st, alibi_slopes=slopes)
        for s in range(len(lengths)):
            a, b = st[s], st[s + 1]
            os_, ls_ = orc.fwd(c["q"][:, a:b], c["k"][:, a:b], c["v"][:, a:b], "bf16", 0.3,
                               causal=causal, alibi_slopes=slopes)
            assert np.array_equal(o[:, a:b], os_), ("blockdiag", causal, s)
            assert np.array_equal(lse[:, :, a:b], ls_), ("blockdiag lse", s)


def check_gqa_equals_repeated_kv(orc):
    c = inp.dense_case(16, 2, 11, 11, 6, 2, 8, "fp16")
    rep = {"k": np.repeat(c["k"], 3, axis=2), "v": np.repeat(c["v"], 3, axis=2)}
    for causal in (False, True):
        o, _ = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.3, causal=causal)
        o2, _ = orc.fwd(c["q"], rep["k"], rep["v"], "fp16", 0.3, causal=causal)
        assert np.array_equal(o, o2), ("gqa repeat", causal)


def check_decode_is_last_causal_row(orc):
    """The scrapbox.io page's check (section "KV Cache"): attending with only
    the newest query row over the cached keys reproduces the last row of full
    attention; here with softmax and the causal mask, per batch row."""
    B, S, Hq, Hkv, D = 3, 40, 4, 2, 8
    ctx = np.array([40, 17, 1], np.int32)
    dec = inp.decode_case(17, ctx, S, Hq, Hkv, D, "bf16")
    slopes = inp.alibi_slopes(Hq)
    od = orc.decode(dec["q"], dec["kcache"], dec["vcache"], ctx, "bf16", 0.35, alibi_slopes=slopes)
    for b in range(B):
        n = int(ctx[b])
        qfull = inp.normal_bits(99, (1, n, Hq, D), "bf16", b)
        qfull[0, n - 1] = dec["q"][b]
        of, _ = orc.fwd(qfull, dec["kcache"][b:b + 1, :n], dec["vcache"][b:b + 1, :n], "bf16", 0.35,
                        causal=True, alibi_slopes=slopes)
        assert _maxerr(od[b], of[0, n - 1]) < TOL, ("decode last row", b)


def check_chunked_prefill_is_suffix(orc):
    """Bottom-right causal with M < N equals the last M rows of the square causal case."""
    N, M = 15, 4
    c = inp.dense_case(18, 1, N, N, 2, 1, 8, "fp16")
    full, lf = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.3, causal=True, alibi_slopes=np.float32([0.3, 0.1]))
    part, lp = orc.fwd(c["q"][:, N - M:], c["k"], c["v"], "fp16", 0.3, causal=True,
                       alibi_slopes=np.float32([0.3, 0.1]))
    assert np.array_equal(part, full[:, N - M:]), "chunked prefill"
    assert np.allclose(lp, lf[:, :, N - M:], rtol=0, atol=TOL), "chunked prefill lse"


def check_lse_merge(orc):
    """Splitting the keys in two and merging the halves by their lse gives the
    whole (the block update of the online softmax in the FlashAttention page,
    section on the softmax that needs not see the whole row)."""
    c = inp.dense_case(19, 1, 7, 20, 2, 2, 8, "bf16")
    o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.6)
    o1, l1 = orc.fwd(c["q"], c["k"][:, :8], c["v"][:, :8], "bf16", 0.6)
    o2, l2 = orc.fwd(c["q"], c["k"][:, 8:], c["v"][:, 8:], "bf16", 0.6)
    w1 = np.exp(l1[0] - lse[0]).T[:, :, None]
    w2 = np.exp(l2[0] - lse[0]).T[:, :, None]
    assert _maxerr(o[0], w1 * o1[0] + w2 * o2[0]) < TOL, "lse merge"
    assert _maxerr(np.logaddexp(l1, l2), lse) < TOL, "lse merge lse"


def check_fwd_rows_matches_fwd(orc):
    c = inp.dense_case(20, 2, 16, 16, 4, 2, 8, "bf16")
    o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.3, causal=True)
    rows = [0, 7, 15]
    orow, lrow = orc.fwd_rows(c["q"], c["k"], c["v"], "bf16", 0.3, 1, rows, causal=True)
    assert np.array_equal(orow, o[1, rows]) and np.array_equal(lrow, lse[1][:, rows]), "fwd_rows dense"
    v = inp.varlen_case(21, [6, 11], 4, 2, 8, "bf16")
    o, _ = orc.fwd(v["q"], v["k"], v["v"], "bf16", 0.3, causal=True, seqstart_q=v["seqstart"])
    orow, _ = orc.fwd_rows(v["q"], v["k"], v["v"], "bf16", 0.3, 0, [0, 10], causal=True,
                           seqstart_q=v["seqstart"], segment=1)
    assert np.array_equal(orow, o[0, [6, 16]]), "fwd_rows segment"


def check_kvcache_prefill(orc):
    """Multi-token decode over a cache: with one query it is the decode step;
    with M queries it is the last M rows of full causal attention over the
    sequence (positions ctx-M..ctx-1), per batch row."""
    B, S, Hq, Hkv, D, M = 3, 30, 4, 2, 8, 5
    ctx = np.array([30, 12, 5], np.int32)
    dec = inp.decode_case(23, ctx, S, Hq, Hkv, D, "bf16")
    slopes = inp.alibi_slopes(Hq)
    o1, _ = orc.fwd_kvcache(dec["q"][:, None], dec["kcache"], dec["vcache"], ctx, "bf16", 0.3, alibi_slopes=slopes)
    od = orc.decode(dec["q"], dec["kcache"], dec["vcache"], ctx, "bf16", 0.3, alibi_slopes=slopes)
    assert _maxerr(o1[:, 0], od) < TOL, "kvcache M=1 == decode"
    for b in range(B):
        n = int(ctx[b])
        qfull = inp.normal_bits(31, (1, n, Hq, D), "bf16", b)
        om, lm = orc.fwd_kvcache(qfull[:, n - M:], dec["kcache"][b:b + 1], dec["vcache"][b:b + 1], ctx[b:b + 1],
                                 "bf16", 0.3, alibi_slopes=slopes)
        of, lf = orc.fwd(qfull, dec["kcache"][b:b + 1, :n], dec["vcache"][b:b + 1, :n], "bf16", 0.3, causal=True,
                         alibi_slopes=slopes)
        assert _maxerr(om[0], of[0, n - M:]) < TOL, ("kvcache suffix rows", b)


def check_kv_append(orc):
    """Appending T rows then reading the first ctx+T rows == concatenation."""
    B, S, Hkv, D, T = 3, 16, 2, 4, 5
    ctx = np.array([0, 9, 14], np.int32)
    kc = inp.normal_bits(40, (B, S, Hkv, D), "fp16", 0)
    vc = inp.normal_bits(40, (B, S, Hkv, D), "fp16", 1)
    kn = inp.normal_bits(41, (B, T, Hkv, D), "fp16", 0)
    vn = inp.normal_bits(41, (B, T, Hkv, D), "fp16", 1)
    k2, v2 = orc.kv_append(kc, vc, kn, vn, ctx)
    for b in range(B):
        c = int(ctx[b])
        n = min(T, S - c)
        assert np.array_equal(k2[b, :c + n], np.concatenate([kc[b, :c], kn[b, :n]])), "append k"
        assert np.array_equal(v2[b, c + n:], vc[b, c + n:]), "append leaves the rest"



# --- backward ----------------------------------------------------------------

def _autograd_sdpa(q, k, v, do, scale, causal=False, mask=None, gqa=False):
    """torch float64 autograd through SDPA on the CPU; tensors [B,M,H,D]."""
    qt, kt, vt = (x.permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, is_causal=causal, scale=scale, enable_gqa=gqa)
    out.backward(do.permute(0, 2, 1, 3))
    return [x.grad.permute(0, 2, 1, 3).numpy() for x in (qt, kt, vt)]


def check_bwd_autograd_sdpa(orc):
    """Gradients against torch's own autograd of SDPA in float64 (no mask,
    causal, GQA with the KV gradient summed over each group)."""
    cases = [(31, (2, 9, 13, 3, 3, 8), "fp16", False), (32, (1, 17, 17, 2, 2, 16), "bf16", True),
             (33, (2, 12, 12, 6, 2, 8), "bf16", True), (34, (1, 7, 15, 4, 1, 8), "fp16", False)]
    for seed, (B, M, N, Hq, Hkv, D), dt, causal in cases:
        c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
        do = inp.normal_bits(seed + 100, (B, M, Hq, D), dt, 0)
        scale = 0.37
        g = orc.bwd(c["q"], c["k"], c["v"], do, dt, scale, causal=causal)
        ref = _autograd_sdpa(*(_torch_decode(x, dt) for x in (c["q"], c["k"], c["v"], do)),
                             float(np.float32(scale)), causal=causal, gqa=Hq != Hkv)
        for name, a, r in zip("qkv", g, ref):
            assert _maxerr(a, r) < TOL, ("bwd autograd", seed, name, _maxerr(a, r))


def check_bwd_autograd_alibi_causal(orc):
    """ALiBi under the causal mask: autograd of SDPA with the key-only float
    bias slope*j (a different but softmax-equivalent bias) gives the same
    gradients; the bias depends on no input, so it only enters through P."""
    B, M, H, D = 1, 14, 3, 8
    c = inp.dense_case(35, B, M, M, H, H, D, "bf16")
    do = inp.normal_bits(135, (B, M, H, D), "bf16", 0)
    slopes = inp.alibi_slopes(H)
    g = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", 0.3, causal=True, alibi_slopes=slopes)
    j = torch.arange(M, dtype=torch.float64)
    causal = torch.ones(M, M, dtype=torch.bool).tril()
    mask = torch.where(causal[None], torch.from_numpy(slopes.astype(np.float64))[:, None, None] * j[None, None, :],
                       torch.tensor(-float("inf"), dtype=torch.float64))
    ref = _autograd_sdpa(*(_torch_decode(x, "bf16") for x in (c["q"], c["k"], c["v"], do)),
                         float(np.float32(0.3)), mask=mask[None])
    for name, a, r in zip("qkv", g, ref):
        assert _maxerr(a, r) < TOL, ("bwd alibi", name, _maxerr(a, r))


def check_bwd_finite_difference(orc):
    """Directional derivatives of the forward (central differences of
    ``attend``) against <grad, direction>, in the cases no library covers:
    ALiBi without a mask, bottom-right causal with M > N (rows with no key)
    and M < N, GQA."""
    rng = np.random.default_rng(36)
    for M, N, Hq, Hkv, causal, slopes in [(5, 8, 4, 2, False, np.float32([0.5, 0.25, 0.125, 0.0625])),
                                          (7, 4, 2, 1, True, np.float32([0.3, 0.7])),
                                          (3, 9, 2, 2, True, None)]:
        D = 4
        q, do = rng.standard_normal((2, M, Hq, D))
        k, v = rng.standard_normal((2, N, Hkv, D))
        scale = 0.6
        grads = orc.attend_grad(q, k, v, do, scale, causal, slopes)
        eps = 1e-5
        for idx, x in enumerate((q, k, v)):
            d = rng.standard_normal(x.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx] = x + eps * d
            args_m[idx] = x - eps * d
            fp = np.sum(do * orc.attend(*args_p, scale, causal, slopes)[0])
            fm = np.sum(do * orc.attend(*args_m, scale, causal, slopes)[0])
            fd = (fp - fm) / (2 * eps)
            an = float(np.sum(grads[idx] * d))
            assert abs(fd - an) < 1e-7 * max(1.0, abs(an)), ("finite difference", "qkv"[idx], M, N, fd, an)


def check_bwd_zero_query_closed_form(orc):
    """q = 0, causal, dO = 1: P is uniform over keys 0..i, so
    dv_j = sum_{i >= j} 1/(i+1) = H_M - H_j (harmonic numbers), dk = 0 (every
    term carries q), and dq_i = scale * sum_{j<=i} (w_j - mean w) k_j / (i+1)
    with w_j = sum_d v_j (the covariance of w and k over the allowed keys)."""
    M, D = 8, 4
    q = np.zeros((1, M, 1, D), np.uint16)
    c = inp.dense_case(37, 1, M, M, 1, 1, D, "fp16")
    do = _ones_bits((1, M, 1, D), "fp16")
    dq, dk, dv = orc.bwd(q, c["k"], c["v"], do, "fp16", 0.5, causal=True)
    harmonic = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, M + 1))])
    for jj in range(M):
        assert abs(dv[0, jj, 0, 0] - (harmonic[M] - harmonic[jj])) < TOL, ("dv harmonic", jj)
    assert np.all(dk == 0), "dk with q = 0"
    k = orc.decode_bits(c["k"], "fp16")[0, :, 0]
    w = orc.decode_bits(c["v"], "fp16")[0, :, 0].sum(axis=1)
    for i in range(M):
        cov = ((w[:i + 1] - w[:i + 1].mean())[:, None] * k[:i + 1]).sum(axis=0) / (i + 1)
        assert _maxerr(dq[0, i, 0], 0.5 * cov) < TOL, ("dq covariance", i)


def check_bwd_constant_v(orc):
    """v constant across keys: the output no longer depends on q or k, so
    dq = dk = 0; and every row's weights sum to one, so the dv rows add up
    to the sum of dO over the rows that see any key."""
    B, M, N, Hq, Hkv, D = 1, 6, 9, 4, 2, 8
    c = inp.dense_case(38, B, M, N, Hq, Hkv, D, "bf16")
    row = c["v"][:, :1]
    vconst = np.repeat(row, N, axis=1)
    do = inp.normal_bits(138, (B, M, Hq, D), "bf16", 0)
    for causal, slopes in [(False, None), (True, inp.alibi_slopes(Hq))]:
        dq, dk, dv = orc.bwd(c["q"], c["k"], vconst, do, "bf16", 0.4, causal=causal, alibi_slopes=slopes)
        assert _maxerr(dq, 0.0) < TOL and _maxerr(dk, 0.0) < TOL, ("constant v", causal)
    dof = orc.decode_bits(do, "bf16")
    dq, dk, dv = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", 0.4, causal=True)
    for g in range(Hkv):
        want = dof[0, :, g * 2:(g + 1) * 2].sum(axis=(0, 1))
        assert _maxerr(dv[0, :, g].sum(axis=0), want) < 1e-10, ("dv column sums", g)
        assert _maxerr(dk[0, :, g].sum(axis=0), 0.0) < 1e-10, ("dk sums to zero", g)


def check_bwd_blockdiag_and_gqa(orc):
    """Packed backward == each segment's own backward; GQA backward == K/V
    repeated per query head with the repeats' gradients summed."""
    lengths = [4, 0, 7, 2]
    vc = inp.varlen_case(39, lengths, 4, 2, 8, "fp16")
    do = inp.normal_bits(139, vc["q"].shape, "fp16", 0)
    st = vc["seqstart"]
    for causal, slopes in [(False, None), (True, inp.alibi_slopes(4))]:
        dq, dk, dv = orc.bwd(vc["q"], vc["k"], vc["v"], do, "fp16", 0.3, causal=causal,
                             seqstart_q=st, alibi_slopes=slopes)
        for s_ in range(len(lengths)):
            a, b = st[s_], st[s_ + 1]
            g = orc.bwd(vc["q"][:, a:b], vc["k"][:, a:b], vc["v"][:, a:b], do[:, a:b], "fp16", 0.3,
                        causal=causal, alibi_slopes=slopes)
            assert np.array_equal(dq[:, a:b], g[0]) and np.array_equal(dk[:, a:b], g[1]) \
                and np.array_equal(dv[:, a:b], g[2]), ("bwd blockdiag", causal, s_)
    c = inp.dense_case(40, 2, 9, 9, 6, 2, 8, "bf16")
    do = inp.normal_bits(140, (2, 9, 6, 8), "bf16", 0)
    for causal in (False, True):
        g = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", 0.3, causal=causal)
        r = orc.bwd(c["q"], np.repeat(c["k"], 3, axis=2), np.repeat(c["v"], 3, axis=2), do, "bf16", 0.3,
                    causal=causal)
        assert np.array_equal(g[0], r[0]), ("bwd gqa dq", causal)
        for a, rr in zip(g[1:], r[1:]):
            summed = rr.reshape(2, 9, 2, 3, 8).sum(axis=3)
            assert _maxerr(a, summed) < TOL, ("bwd gqa dk/dv", causal)


# --- block-sparse ----------------------------------------------------------------

def _expand_blocks(bm, M, N, B=64):
    """Block mask -> per-element boolean mask [M, N] (np.kron, independent of the oracle's indexing)."""
    full = np.kron(np.asarray(bm, dtype=bool), np.ones((B, B), dtype=bool))
    return full[:M, :N]


def check_blocksparse_sdpa_bool_mask(orc):
    """Block-sparse attention == torch SDPA with the element-level boolean
    mask the blocks expand to (np.kron), alone and ANDed with the causal
    rule; forward and backward (torch autograd)."""
    for seed, (B, M, N, Hq, Hkv, D), causal in [(41, (2, 150, 200, 4, 2, 8), False), (42, (1, 190, 190, 2, 2, 8), True)]:
        c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, "bf16")
        nq, nk = -(-M // 64), -(-N // 64)
        bm = inp.random_block_mask(seed, nq, nk, 0.5)
        el = _expand_blocks(bm, M, N)
        if causal:
            el = el & np.tril(np.ones((M, N), dtype=bool), N - M)
        assert el.any(axis=1).all()
        mask = torch.from_numpy(el)[None, None]
        scale = 0.3
        o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", scale, causal=causal, block_mask=bm)
        tq, tk, tv = (_torch_decode(c[x], "bf16") for x in ("q", "k", "v"))
        ref = _sdpa(tq, tk, tv, float(np.float32(scale)), mask=mask, gqa=Hq != Hkv)
        assert _maxerr(o, ref) < TOL, ("blocksparse fwd", seed, _maxerr(o, ref))
        do = inp.normal_bits(seed + 100, (B, M, Hq, D), "bf16", 0)
        g = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", scale, causal=causal, block_mask=bm)
        gr = _autograd_sdpa(tq, tk, tv, _torch_decode(do, "bf16"), float(np.float32(scale)), mask=mask,
                            gqa=Hq != Hkv)
        for name, a, r in zip("qkv", g, gr):
            assert _maxerr(a, r) < TOL, ("blocksparse bwd", seed, name, _maxerr(a, r))


def check_blocksparse_all_on_is_dense(orc):
    c = inp.dense_case(43, 1, 130, 70, 2, 1, 8, "fp16")
    ones = np.ones((3, 2), np.uint8)
    for causal in (False, True):
        a = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.4, causal=causal)
        b = orc.fwd(c["q"], c["k"], c["v"], "fp16", 0.4, causal=causal, block_mask=ones)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), ("all-on mask", causal)


def check_blocksparse_masked_blocks_do_not_matter(orc):
    """Rows never read K/V of blocks that are off for them; a query block with
    every block off returns 0 and lse -inf."""
    c = inp.dense_case(44, 1, 192, 256, 2, 2, 8, "bf16")
    bm = np.array([[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1]], np.uint8)
    o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.5, block_mask=bm)
    k2, v2 = c["k"].copy(), c["v"].copy()
    k2[:, 64:128] = inp.normal_bits(45, k2[:, 64:128].shape, "bf16", 0)    # key block 1: off for query block 0
    v2[:, 192:256] = inp.normal_bits(45, v2[:, 192:256].shape, "bf16", 1)  # key block 3: off for query block 0
    o2, _ = orc.fwd(c["q"], k2, v2, "bf16", 0.5, block_mask=bm)
    assert np.array_equal(o[:, :64], o2[:, :64]), "masked blocks leak"
    assert not np.array_equal(o[:, 128:], o2[:, 128:]), "query block 2 must see key blocks 1 and 3"
    assert np.all(o[:, 64:128] == 0) and np.all(np.isneginf(lse[:, :, 64:128])), "empty query block"


def check_blockdiag_cross_segments(orc):
    """Packed cross-attention (query segment s sees key segment s, lengths
    differ, some empty) == each segment's own dense attention, forward and
    backward, with the bottom-right causal alignment per segment."""
    ql, kl = [5, 9, 0, 4, 3], [8, 3, 6, 4, 0]
    c = inp.varlen_cross_case(50, ql, kl, 4, 2, 8, "bf16")
    sq, sk = c["seqstart_q"], c["seqstart_k"]
    do = inp.normal_bits(150, c["q"].shape, "bf16", 0)
    for causal, slopes in [(False, None), (True, inp.alibi_slopes(4))]:
        o, lse = orc.fwd(c["q"], c["k"], c["v"], "bf16", 0.3, causal=causal, seqstart_q=sq, seqstart_k=sk,
                         alibi_slopes=slopes)
        g = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", 0.3, causal=causal, seqstart_q=sq, seqstart_k=sk,
                    alibi_slopes=slopes)
        for s_ in range(len(ql)):
            a, b, e, f = sq[s_], sq[s_ + 1], sk[s_], sk[s_ + 1]
            if b > a and f > e:
                os_, ls_ = orc.fwd(c["q"][:, a:b], c["k"][:, e:f], c["v"][:, e:f], "bf16", 0.3, causal=causal,
                                   alibi_slopes=slopes)
                gs = orc.bwd(c["q"][:, a:b], c["k"][:, e:f], c["v"][:, e:f], do[:, a:b], "bf16", 0.3,
                             causal=causal, alibi_slopes=slopes)
                assert np.array_equal(o[:, a:b], os_) and np.array_equal(lse[:, :, a:b], ls_), ("cross fwd", s_)
                assert np.array_equal(g[0][:, a:b], gs[0]) and np.array_equal(g[1][:, e:f], gs[1]) \
                    and np.array_equal(g[2][:, e:f], gs[2]), ("cross bwd", s_)
            else:   # no keys or no queries: zero output / zero gradients
                assert np.all(o[:, a:b] == 0) and np.all(g[0][:, a:b] == 0), ("cross empty q", s_)
                assert np.all(g[1][:, e:f] == 0) and np.all(g[2][:, e:f] == 0), ("cross empty k", s_)

ALL_CHECKS = [
    check_sdpa_nomask,
    check_sdpa_causal_square,
    check_sdpa_gqa,
    check_sdpa_alibi_causal_as_key_bias,
    check_lse_logsumexp,
    check_rows_sum_to_one,
    check_first_causal_row_is_v0,
    check_single_key,
    check_zero_query_uniform,
    check_zero_query_alibi_geometric,
    check_zero_query_alibi_two_sided,
    check_empty_rows,
    check_blockdiag_equals_per_segment,
    check_gqa_equals_repeated_kv,
    check_decode_is_last_causal_row,
    check_chunked_prefill_is_suffix,
    check_lse_merge,
    check_fwd_rows_matches_fwd,
    check_kvcache_prefill,
    check_kv_append,
    check_bwd_autograd_sdpa,
    check_bwd_autograd_alibi_causal,
    check_bwd_finite_difference,
    check_bwd_zero_query_closed_form,
    check_bwd_constant_v,
    check_bwd_blockdiag_and_gqa,
    check_blocksparse_sdpa_bool_mask,
    check_blocksparse_all_on_is_dense,
    check_blocksparse_masked_blocks_do_not_matter,
    check_blockdiag_cross_segments,
]
