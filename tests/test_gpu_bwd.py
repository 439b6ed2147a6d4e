"""Parity of the HIP backward kernels (through the C ABI) with the fp64 oracle, on the GPU.

The forward runs first (``mea_fwd`` with its lse), then ``mea_bwd``; the oracle
computes the gradients from q, k, v and dO alone, in float64.

Tolerance (element-wise): every gradient element is checked against its own
bar, C u T, u the unit roundoff of the input type (2^-8 bf16, 2^-11 fp16), C = 4
and T the sum of the magnitudes of that element's own terms (P, dS and their
error sources, evaluated in float64 from the definition: tests/grad_bounds.py
derives the bar and checks, on the CPU, that its terms sum to the oracle's
gradients).

Where the exact dq and dk vanish (one key, or v equal on every key: the
output no longer depends on q or k), the stored output is exactly v, and
dS = P (dP - Delta) is the difference of two fp32 dot products of the same
D-vectors summed in different orders, each within gamma_D = D 2^-24 of
A_i = sum_d |dO_id v_d|. Those cases are also checked against that tighter
bound: |dq_i| <= 2 gamma_D scale A_i |(P k)_i| and |dk_j| <= 2 gamma_D scale
sum_i P_ij A_i |q_i|, both evaluated with the oracle (P k is the forward with
v := k; P^T W is the dv of the backward with dO := W).
"""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import dev, f32, host_f64, i32, report, say
from grad_bounds import check_grads, grad_terms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _fwd_bwd(mea, q, k, v, do, dt, causal=False, slopes=None, st=None, scale=None):
    qd, kd, vd, dod = dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt)
    D = q.shape[-1]
    scale = float(np.float32(1.0 / np.sqrt(D))) if scale is None else scale
    B, M, Hq, _ = q.shape
    lse = torch.empty((B, Hq, M) if st is None else (Hq, M), dtype=torch.float32, device="cuda")
    sl = None if slopes is None else f32(slopes)
    sq = None if st is None else i32(st)
    out = mea.fwd(qd, kd, vd, causal=causal, scale=scale, alibi_slopes=sl, seqstart_q=sq, lse=lse)
    dq, dk, dv = mea.bwd(qd, kd, vd, out, dod, lse, causal=causal, scale=scale, alibi_slopes=sl, seqstart_q=sq)
    torch.cuda.synchronize()
    return (dq, dk, dv), scale


def _delta_terms(q, k, v, do, dt, scale, **kw):
    """Largest dq and dk shifts per unit relative error of Delta (module docstring)."""
    o, _ = orc.fwd(q, k, v, dt, scale, **kw)
    a = np.sum(np.abs(orc.decode_bits(do, dt) * o), axis=-1, keepdims=True)     # A_i per (row, head)
    pk, _ = orc.fwd(q, k, k, dt, scale, **kw)
    f_dq = scale * float(np.max(a * np.abs(pk), initial=0.0))
    w = inp.round_bits((a * np.abs(orc.decode_bits(q, dt))).astype(np.float32), dt)
    _, _, ptw = orc.bwd(q, k, v, w, dt, scale, **kw)
    f_dk = scale * float(np.nanmax(np.abs(ptw), initial=0.0))
    return f_dq, f_dk


def _want(q, k, v, do, dt, scale, **kw):
    """The oracle's gradients and the per-element magnitude sums of their terms."""
    return orc.bwd(q, k, v, do, dt, scale, **kw), grad_terms(q, k, v, do, dt, scale, **kw)[1]


def _check(name, got, want, terms, dt):
    check_grads(name, [host_f64(g) for g in got], want, terms, dt, say=say)


DENSE = [
    # name, seed, B, M, N, Hq, Hkv, D, dtype, causal
    ("b1_m128_h2_d64_fp16", 0, 1, 128, 128, 2, 2, 64, "fp16", False),
    ("b2_m256_h8_d64_fp16_causal", 1, 2, 256, 256, 8, 8, 64, "fp16", True),
    ("b4_m512_h16_d64_bf16", 2, 4, 512, 512, 16, 16, 64, "bf16", False),
    ("b4_m512_h16_d64_bf16_causal", 2, 4, 512, 512, 16, 16, 64, "bf16", True),
    ("ragged_m300_n177_d128_bf16_gqa", 4, 2, 300, 177, 4, 2, 128, "bf16", False),
    ("ragged_causal_m333_d128_fp16_gqa", 5, 1, 333, 333, 8, 2, 128, "fp16", True),
    ("chunked_prefill_m70_n500_causal", 6, 2, 70, 500, 4, 4, 64, "bf16", True),
    ("more_queries_than_keys_causal", 7, 1, 200, 90, 2, 1, 128, "bf16", True),
    ("single_query_n777_gqa", 9, 2, 1, 777, 4, 1, 128, "bf16", True),
    ("gqa_b2_m256_hq8_hkv2_d64_fp16", 10, 2, 256, 256, 8, 2, 64, "fp16", False),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: c[0])
def test_dense_bwd_parity(mea, case):
    name, seed, B, M, N, Hq, Hkv, D, dt, causal = case
    say(f"case bwd {name}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    do = inp.normal_bits(seed + 500, (B, M, Hq, D), dt, 0)
    got, scale = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, dt, causal=causal)
    want, terms = _want(c["q"], c["k"], c["v"], do, dt, scale, causal=causal)
    _check(name, got, want, terms, dt)


VARLEN = [
    # name, seed, lengths, Hq, Hkv, D, dtype, causal, alibi
    ("c4_like_causal_alibi_gqa_d128", 20, [497, 64, 1, 300, 0, 131], 8, 2, 128, "bf16", True, True),
    ("varlen_noncausal_alibi_d64_fp16", 21, [129, 3, 256, 77], 4, 4, 64, "fp16", False, True),
    ("varlen_causal_d64_bf16", 22, [200, 128, 5, 333], 4, 1, 64, "bf16", True, False),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: c[0])
def test_varlen_bwd_parity(mea, case):
    name, seed, lengths, Hq, Hkv, D, dt, causal, alibi = case
    say(f"case bwd {name}")
    c = inp.varlen_case(seed, lengths, Hq, Hkv, D, dt)
    do = inp.normal_bits(seed + 500, c["q"].shape, dt, 0)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    got, scale = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, dt, causal=causal, slopes=slopes, st=c["seqstart"])
    kw = dict(causal=causal, seqstart_q=c["seqstart"], alibi_slopes=slopes)
    want, terms = _want(c["q"], c["k"], c["v"], do, dt, scale, **kw)
    _check(name, got, want, terms, dt)


DEGENERATE = [
    # name, seed, B, M, N, Hq, Hkv, D, dtype, causal, alibi, constant v
    ("single_key_m1", 8, 3, 1, 1, 2, 2, 64, "fp16", False, False, False),
    ("single_key_m3_gqa_d128", 9, 2, 3, 1, 4, 2, 128, "bf16", False, False, False),
    ("constant_v_noncausal_m200", 10, 2, 200, 300, 4, 2, 64, "bf16", False, False, True),
    ("constant_v_causal_alibi_m260", 11, 1, 260, 260, 4, 4, 128, "fp16", True, True, True),
]


@pytest.mark.parametrize("case", DEGENERATE, ids=lambda c: c[0])
def test_bwd_vanishing_dq_dk(mea, case):
    """One key, or v equal on every key: dq = dk = 0 exactly, dv from the oracle."""
    name, seed, B, M, N, Hq, Hkv, D, dt, causal, alibi, const_v = case
    say(f"case bwd degenerate {name}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    v = np.repeat(c["v"][:, :1], N, axis=1) if const_v else c["v"]
    do = inp.normal_bits(seed + 500, (B, M, Hq, D), dt, 0)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    (dq, dk, dv), scale = _fwd_bwd(mea, c["q"], c["k"], v, do, dt, causal=causal, slopes=slopes)
    kw = dict(causal=causal, alibi_slopes=slopes)
    want, terms = _want(c["q"], c["k"], v, do, dt, scale, **kw)
    assert np.all(want[0] == 0) or const_v
    gamma = D * 2.0 ** -24
    e_dq, e_dk = _delta_terms(c["q"], c["k"], v, do, dt, scale, **kw)
    report(f"{name} dq", host_f64(dq), 0 * want[0], 2 * gamma * e_dq)
    report(f"{name} dk", host_f64(dk), 0 * want[1], 2 * gamma * e_dk)
    assert float(np.max(np.abs(host_f64(dq)))) <= 2 * gamma * e_dq + 1e-30
    assert float(np.max(np.abs(host_f64(dk)))) <= 2 * gamma * e_dk + 1e-30
    _check(name, (dq, dk, dv), want, terms, dt)


def test_varlen_bwd_thousands_of_short_segments(mea):
    """4096 packed segments of 1 to 64 tokens (some empty), causal with GQA:
    both backward kernels find their segment by binary search (query tiles
    over seqstart_q, key tiles over seqstart_k)."""
    lengths = [int(x) for x in np.random.default_rng(13).integers(0, 65, 4096)]
    c = inp.varlen_case(14, lengths, 4, 2, 64, "bf16")
    say(f"case bwd packed 4096 short segments, T={int(c['seqstart'][-1])}")
    do = inp.normal_bits(514, c["q"].shape, "bf16", 0)
    got, scale = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, "bf16", causal=True, st=c["seqstart"])
    want, terms = _want(c["q"], c["k"], c["v"], do, "bf16", scale, causal=True, seqstart_q=c["seqstart"])
    _check("bwd 4096 short segments", got, want, terms, "bf16")


def test_varlen_bwd_equals_per_segment_bitwise(mea):
    """Tiles start at segment starts, so the packed backward of each segment
    is the same arithmetic as that segment run alone: bitwise equal."""
    say("case bwd packed == per segment")
    lengths = [70, 129, 1, 200]
    c = inp.varlen_case(23, lengths, 4, 2, 64, "bf16")
    do = inp.normal_bits(523, c["q"].shape, "bf16", 0)
    st = c["seqstart"]
    slopes = inp.alibi_slopes(4)
    (dq, dk, dv), _ = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, "bf16", causal=True, slopes=slopes, st=st)
    for s in range(len(lengths)):
        a, b = st[s], st[s + 1]
        (sq, sk, sv), _ = _fwd_bwd(mea, c["q"][:, a:b], c["k"][:, a:b], c["v"][:, a:b], do[:, a:b], "bf16",
                                   causal=True, slopes=slopes)
        assert torch.equal(dq[:, a:b], sq) and torch.equal(dk[:, a:b], sk) and torch.equal(dv[:, a:b], sv), s


def test_bwd_deterministic(mea):
    say("case bwd deterministic")
    c = inp.dense_case(24, 2, 384, 384, 8, 2, 64, "bf16")
    do = inp.normal_bits(524, (2, 384, 8, 64), "bf16", 0)
    a, _ = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, "bf16", causal=True)
    b, _ = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, "bf16", causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_full_size_sampled_heads(mea, causal):
    """B=4, M=N=4096, H=16, D=64, bf16 (the forward's benchmark shape): the
    kernels run on the whole problem; the oracle checks every gradient of two
    (batch row, head) pairs (heads are independent without GQA)."""
    name = f"bwd_b4_m4096_h16_{'causal' if causal else 'noncausal'}"
    say(f"case {name}")
    B, M, H, D = 4, 4096, 16, 64
    c = inp.dense_case(31 + causal, B, M, M, H, H, D, "bf16")
    do = inp.normal_bits(531, (B, M, H, D), "bf16", 0)
    got, scale = _fwd_bwd(mea, c["q"], c["k"], c["v"], do, "bf16", causal=causal)
    for b, h in [(0, 0), (3, 13)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        args = (c["q"][sl], c["k"][sl], c["v"][sl], do[sl], "bf16", scale)
        want, terms = _want(*args, causal=causal)
        _check(f"{name} b{b} h{h}", [g[sl] for g in got], want, terms, "bf16")


def test_bwd_rejects_bad_workspace(mea):
    c = inp.dense_case(25, 1, 64, 64, 2, 2, 64, "fp16")
    q, k, v = dev(c["q"], "fp16"), dev(c["k"], "fp16"), dev(c["v"], "fp16")
    lse = torch.empty((1, 2, 64), dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, lse=lse)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mea.MeaError) as e:
        mea.bwd(q, k, v, out, out, lse, workspace=small)
    assert e.value.status == mea.MEA_EWORKSPACE


def test_varlen_cross_segments_bwd(mea):
    """Backward of packed cross-attention (seqstart_k != seqstart_q), causal
    with ALiBi and GQA; key segments no query sees get dk = dv = 0."""
    say("case bwd cross segments")
    ql, kl = [130, 64, 0, 300, 7, 200], [200, 64, 50, 129, 7, 0]
    c = inp.varlen_cross_case(41, ql, kl, 8, 2, 128, "bf16")
    do = inp.normal_bits(541, c["q"].shape, "bf16", 0)
    dt, Hq = "bf16", 8
    q, k, v, dod = (dev(x, dt) for x in (c["q"], c["k"], c["v"], do))
    scale = float(np.float32(1.0 / np.sqrt(128)))
    slopes = inp.alibi_slopes(Hq)
    sq, sk = i32(c["seqstart_q"]), i32(c["seqstart_k"])
    lse = torch.empty((Hq, int(c["seqstart_q"][-1])), dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=True, scale=scale, seqstart_q=sq, seqstart_k=sk, alibi_slopes=f32(slopes), lse=lse)
    got = mea.bwd(q, k, v, out, dod, lse, causal=True, scale=scale, seqstart_q=sq, seqstart_k=sk,
                  alibi_slopes=f32(slopes))
    torch.cuda.synchronize()
    want, terms = _want(c["q"], c["k"], c["v"], do, dt, scale, causal=True, seqstart_q=c["seqstart_q"],
                        seqstart_k=c["seqstart_k"], alibi_slopes=slopes)
    _check("bwd cross segments", got, want, terms, dt)
    e, f = int(c["seqstart_k"][2]), int(c["seqstart_k"][3])      # key segment 2: its query segment is empty
    assert np.all(host_f64(got[1])[:, e:f] == 0) and np.all(host_f64(got[2])[:, e:f] == 0)
