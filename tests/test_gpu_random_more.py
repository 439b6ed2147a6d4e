"""Seeded random configurations of the decode step, block-sparse forward and
backward, packed cross-attention and multi-token decode over a cache, each
against the fp64 oracle.

Each case draws its shapes, dtype, head dimension, GQA ratio, mask and ALiBi
from a fixed seed (so every run checks the same cases), including empty and
full contexts, query blocks with no key block and segments of length 0.
"""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, dev, f32, host_f64, i32, say
from grad_bounds import check_grads, grad_terms

pytestmark = pytest.mark.gpu

SEEDS = range(16)


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _common(rng):
    dt = ["fp16", "bf16"][rng.integers(2)]
    D = [64, 128][rng.integers(2)]
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 5]))
    alibi = bool(rng.integers(2))
    return dt, D, Hq, Hkv, (inp.alibi_slopes(Hq) if alibi else None), float(np.float32(1.0 / np.sqrt(D)))


def _check_lse(got, want, dt):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), "lse -inf pattern"
    assert np.max(np.abs(got[fin] - want[fin]), initial=0.0) <= LSE_TOL[dt], "lse"


@pytest.mark.parametrize("seed", SEEDS)
def test_random_decode(mea, seed):
    rng = np.random.default_rng(7100 + seed)
    dt, D, Hq, Hkv, slopes, scale = _common(rng)
    B = int(rng.integers(1, 40))
    S = int(rng.integers(1, 3000))
    ctx = [int(x) for x in rng.integers(0, S + 1, B)]
    ctx[0] = S if rng.integers(2) else 0
    say(f"case random decode {seed}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} alibi={slopes is not None}")
    d = inp.decode_case(seed, ctx, S, Hq, Hkv, D, dt)
    out = mea.decode(dev(d["q"], dt), dev(d["kcache"], dt), dev(d["vcache"], dt), i32(d["ctx_lens"]), scale=scale,
                     alibi_slopes=None if slopes is None else f32(slopes))
    torch.cuda.synchronize()
    want = orc.decode(d["q"], d["kcache"], d["vcache"], d["ctx_lens"], dt, scale, alibi_slopes=slopes)
    assert float(np.max(np.abs(host_f64(out) - want))) <= TOL[dt]


@pytest.mark.parametrize("seed", SEEDS)
def test_random_blocksparse_fwd_bwd(mea, seed):
    rng = np.random.default_rng(7200 + seed)
    dt, D, Hq, Hkv, slopes, scale = _common(rng)
    B = int(rng.integers(1, 3))
    M = int(rng.integers(1, 400))
    N = int(rng.integers(1, 400))
    causal = bool(rng.integers(2))
    bm = inp.random_block_mask(seed, -(-M // 64), -(-N // 64), float(rng.uniform(0.1, 0.9)),
                               keep_diagonal=bool(rng.integers(2)))
    say(f"case random blocksparse {seed}: B={B} M={M} N={N} Hq={Hq} Hkv={Hkv} D={D} {dt} causal={causal} "
        f"alibi={slopes is not None}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    do = inp.normal_bits(seed + 900, (B, M, Hq, D), dt, 0)
    q, k, v, dod = (dev(x, dt) for x in (c["q"], c["k"], c["v"], do))
    m = torch.from_numpy(np.ascontiguousarray(bm).astype(np.uint8)).cuda()
    sl = None if slopes is None else f32(slopes)
    lse = torch.empty((B, Hq, M), dtype=torch.float32, device="cuda")
    out = mea.fwd_blocksparse(q, k, v, m, causal=causal, scale=scale, alibi_slopes=sl, lse=lse)
    grads = mea.bwd(q, k, v, out, dod, lse, causal=causal, scale=scale, alibi_slopes=sl, block_mask=m)
    torch.cuda.synchronize()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, alibi_slopes=slopes, block_mask=bm)
    assert float(np.max(np.abs(host_f64(out) - want), initial=0.0)) <= TOL[dt], "out"
    _check_lse(lse.cpu().numpy(), wlse, dt)
    wg = orc.bwd(c["q"], c["k"], c["v"], do, dt, scale, causal=causal, alibi_slopes=slopes, block_mask=bm)
    terms = grad_terms(c["q"], c["k"], c["v"], do, dt, scale, causal=causal, alibi_slopes=slopes,
                       block_mask=bm)[1]
    check_grads(f"random blocksparse {seed}", [host_f64(g) for g in grads], wg, terms, dt, say=say)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_packed_cross(mea, seed):
    rng = np.random.default_rng(7300 + seed)
    dt, D, Hq, Hkv, slopes, scale = _common(rng)
    causal = bool(rng.integers(2))
    ns = int(rng.integers(1, 6))
    lq = [int(x) for x in rng.integers(0, 300, ns)]
    lk = [int(x) for x in rng.integers(0, 300, ns)]
    lq[0] = max(lq[0], 1)
    lk[-1] = max(lk[-1], 1)
    say(f"case random cross {seed}: lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} D={D} {dt} causal={causal} "
        f"alibi={slopes is not None}")
    c = inp.varlen_cross_case(seed, lq, lk, Hq, Hkv, D, dt)
    T = int(c["seqstart_q"][-1])
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    out = mea.fwd(dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt), causal=causal, scale=scale,
                  seqstart_q=i32(c["seqstart_q"]), seqstart_k=i32(c["seqstart_k"]),
                  alibi_slopes=None if slopes is None else f32(slopes), lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, seqstart_q=c["seqstart_q"],
                         seqstart_k=c["seqstart_k"], alibi_slopes=slopes)
    assert float(np.max(np.abs(host_f64(out) - want), initial=0.0)) <= TOL[dt], "out"
    _check_lse(lse.cpu().numpy(), wlse[0], dt)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_kvcache(mea, seed):
    rng = np.random.default_rng(7400 + seed)
    dt, D, Hq, Hkv, slopes, scale = _common(rng)
    causal = bool(rng.integers(2))
    B = int(rng.integers(1, 6))
    Mn = int(rng.integers(1, 40))
    S = int(rng.integers(Mn, 600))
    ctx = [int(x) for x in rng.integers(1, S + 1, B)]
    say(f"case random kvcache {seed}: B={B} M={Mn} S={S} ctx={ctx} Hq={Hq} Hkv={Hkv} D={D} {dt} causal={causal} "
        f"alibi={slopes is not None}")
    d = inp.decode_case(seed, ctx, S, Hq, Hkv, D, dt)
    q = inp.normal_bits(seed + 77, (B, Mn, Hq, D), dt, 0)
    lse = torch.empty((B, Hq, Mn), dtype=torch.float32, device="cuda")
    out = mea.fwd_kvcache(dev(q, dt), dev(d["kcache"], dt), dev(d["vcache"], dt), i32(d["ctx_lens"]), causal=causal,
                          alibi_slopes=None if slopes is None else f32(slopes), scale=scale, lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd_kvcache(q, d["kcache"], d["vcache"], d["ctx_lens"], dt, scale, causal=causal,
                                 alibi_slopes=slopes)
    assert float(np.max(np.abs(host_f64(out) - want), initial=0.0)) <= TOL[dt], "out"
    _check_lse(lse.cpu().numpy(), wlse, dt)
