"""Parity of the block-sparse forward and backward (``mea_fwd_blocksparse``, ``mea_bwd_blocksparse``) with the fp64 oracle, on the GPU."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, dev, f32, host_f64, report, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _mask(bm):
    return torch.from_numpy(np.ascontiguousarray(bm, dtype=np.uint8)).cuda()


def _run(mea, c, dt, bm, causal=False, slopes=None):
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    B, M, Hq, D = c["q"].shape
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((B, Hq, M), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd_blocksparse(q, k, v, _mask(bm), causal=causal, scale=scale,
                              alibi_slopes=None if slopes is None else f32(slopes), lse=lse)
    torch.cuda.synchronize()
    return out, lse, scale


CASES = [
    # name, seed, B, M, N, Hq, Hkv, D, dtype, causal, alibi, density
    ("ragged_m300_n260_d64_bf16_gqa", 0, 2, 300, 260, 4, 2, 64, "bf16", False, False, 0.4),
    ("causal_alibi_m333_d128_fp16", 1, 1, 333, 333, 4, 4, 128, "fp16", True, True, 0.5),
    ("causal_m512_d64_bf16_sparse", 2, 2, 512, 512, 8, 2, 64, "bf16", True, False, 0.25),
    ("noncausal_alibi_m200_n700_d128_bf16", 3, 1, 200, 700, 2, 1, 128, "bf16", False, True, 0.3),
    # 300 key blocks: the skip list moves to its second 256-block window
    ("causal_alibi_two_windows_m128_n19200_d64_bf16", 5, 1, 128, 19200, 2, 1, 64, "bf16", True, True, 0.3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_blocksparse_parity(mea, case):
    name, seed, B, M, N, Hq, Hkv, D, dt, causal, alibi, dens = case
    say(f"case blocksparse {name}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    bm = inp.random_block_mask(seed, -(-M // 64), -(-N // 64), dens)
    bm[-1, :] = 0                      # one query block with no key at all
    slopes = inp.alibi_slopes(Hq) if alibi else None
    out, lse, scale = _run(mea, c, dt, bm, causal=causal, slopes=slopes)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, alibi_slopes=slopes, block_mask=bm)
    err = report(name, host_f64(out), want, TOL[dt])
    assert err <= TOL[dt]
    got_lse = lse.cpu().numpy()
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(got_lse), fin), "lse -inf pattern"
    assert np.max(np.abs(got_lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dt], "lse"
    assert np.all(host_f64(out)[:, (bm.shape[0] - 1) * 64:] == 0), "query block with every block off"


def test_lse_rows_dominated_by_few_keys(mea):
    """Non-causal ALiBi with 32 heads: the steep heads give rows whose weight
    sits on a handful of keys, so the rounding of those few P values to bf16
    does not average out and the lse error approaches ln(1 + 2^-8). Output
    and lse against the oracle at the tolerances derived from that bound."""
    B, M, N, Hq, Hkv, D, dt = 2, 260, 325, 32, 4, 128, "bf16"
    say("case blocksparse steep-alibi lse")
    c = inp.dense_case(16, B, M, N, Hq, Hkv, D, dt)
    bm = inp.random_block_mask(16, -(-M // 64), -(-N // 64), 0.59, keep_diagonal=False)
    slopes = inp.alibi_slopes(Hq)
    out, lse, scale = _run(mea, c, dt, bm, slopes=slopes)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, alibi_slopes=slopes, block_mask=bm)
    assert report("steep alibi", host_f64(out), want, TOL[dt]) <= TOL[dt]
    got_lse = lse.cpu().numpy()
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(got_lse), fin), "lse -inf pattern"
    assert np.max(np.abs(got_lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dt], "lse"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_all_on_mask_is_the_dense_kernel_bitwise(mea, D, causal):
    """With every block on, the skip list visits every key block in order:
    the same arithmetic as the dense forward (no ALiBi: the dense causal
    ALiBi launch walks the blocks in reverse)."""
    say(f"case blocksparse all-on D={D} causal={causal}")
    c = inp.dense_case(4 + D, 2, 257, 300, 4, 2, D, "bf16")
    q, k, v = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16")
    ones = torch.ones((-(-257 // 64), -(-300 // 64)), dtype=torch.uint8, device="cuda")
    a = mea.fwd(q, k, v, causal=causal)
    b = mea.fwd_blocksparse(q, k, v, ones, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_band_global_full_size_sampled(mea):
    """B=1, M=N=16384, H=16, D=64, bf16 with a sliding window of 3 blocks on
    each side plus one global key block, causal: sampled rows of two heads
    against the oracle."""
    say("case blocksparse band_global m16384")
    B, M, H, D = 1, 16384, 16, 64
    c = inp.dense_case(40, B, M, M, H, H, D, "bf16")
    bm = inp.band_global_block_mask(M // 64, M // 64, 3, 1)
    out, lse, scale = _run(mea, c, "bf16", bm, causal=True)
    got = host_f64(out)
    rng = np.random.default_rng(16384)
    rows = np.unique(np.concatenate([[0, 63, 64, 200, 4095, 8191, M - 1], rng.integers(0, M, 25)]))
    for h in (0, 11):
        sl = (slice(0, 1), slice(None), slice(h, h + 1))
        want, wlse = orc.fwd_rows(c["q"][sl], c["k"][sl], c["v"][sl], "bf16", scale, 0, rows, causal=True,
                                  block_mask=bm)
        err = report(f"band_global h{h}", got[0, rows, h:h + 1], want, TOL["bf16"])
        assert err <= TOL["bf16"]
        assert np.max(np.abs(lse[0, h, rows].cpu().numpy() - wlse[0])) <= LSE_TOL["bf16"]


def test_band_global_whole_output(mea):
    """The benchmark's block-sparse item (its own inputs: B=1, M=N=16384, H=16,
    D=64, bf16, causal, a window of 3 blocks on each side plus one global key
    block): every output element and every row's lse against the oracle,
    evaluated 512 query rows at a time."""
    say("case blocksparse band_global m16384 whole output")
    B, M, H, D = 1, 16384, 16, 64
    c = inp.dense_case(12, B, M, M, H, H, D, "bf16")
    bm = inp.band_global_block_mask(M // 64, M // 64, 3, 1)
    out, lse, scale = _run(mea, c, "bf16", bm, causal=True)
    got, got_lse = host_f64(out)[0], lse.cpu().numpy()[0]
    q, k, v = (orc.decode_bits(c[x][0], "bf16") for x in ("q", "k", "v"))
    want = np.empty_like(got)
    wlse = np.empty_like(got_lse, dtype=np.float64)

    def one(r0):
        rows = np.arange(r0, min(r0 + 512, M))
        return rows, orc.attend(q, k, v, scale, True, rows=rows, block_mask=bm)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for rows, (w, wl) in ex.map(one, range(0, M, 512)):
            want[rows] = w
            wlse[:, rows] = wl
    assert report("band_global all rows", got, want, TOL["bf16"]) <= TOL["bf16"]
    err = float(np.max(np.abs(got_lse - wlse)))
    say(f"[band_global all rows lse] max_abs_err={err:.3e} tol={LSE_TOL['bf16']:.2e}")
    assert err <= LSE_TOL["bf16"]


BWD_CASES = [
    # name, seed, B, M, N, Hq, Hkv, D, dtype, causal, alibi, density
    ("bwd_ragged_m300_n260_d64_bf16_gqa", 5, 2, 300, 260, 4, 2, 64, "bf16", False, False, 0.4),
    ("bwd_causal_alibi_m333_d128_fp16", 6, 1, 333, 333, 4, 4, 128, "fp16", True, True, 0.5),
    ("bwd_causal_m512_d64_bf16", 7, 1, 512, 512, 4, 1, 64, "bf16", True, False, 0.3),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: c[0])
def test_blocksparse_bwd_parity(mea, case):
    """Backward over a block-sparse mask (mea_bwd_blocksparse) against the
    oracle, with the backward tests' tolerance; one query block and one key
    block are fully off (their dq, resp. dk and dv, are exactly 0)."""
    from grad_bounds import check_grads, grad_terms
    name, seed, B, M, N, Hq, Hkv, D, dt, causal, alibi, dens = case
    say(f"case blocksparse {name}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    bm = inp.random_block_mask(seed, -(-M // 64), -(-N // 64), dens)
    bm[1, :] = 0
    bm[:, 2] = 0
    do = inp.normal_bits(seed + 500, (B, M, Hq, D), dt, 0)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    q, k, v, dod = (dev(x, dt) for x in (c["q"], c["k"], c["v"], do))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.empty((B, Hq, M), dtype=torch.float32, device="cuda")
    sl = None if slopes is None else f32(slopes)
    m = _mask(bm)
    out = mea.fwd_blocksparse(q, k, v, m, causal=causal, scale=scale, alibi_slopes=sl, lse=lse)
    got = mea.bwd(q, k, v, out, dod, lse, causal=causal, scale=scale, alibi_slopes=sl, block_mask=m)
    torch.cuda.synchronize()
    want = orc.bwd(c["q"], c["k"], c["v"], do, dt, scale, causal=causal, alibi_slopes=slopes, block_mask=bm)
    terms = grad_terms(c["q"], c["k"], c["v"], do, dt, scale, causal=causal, alibi_slopes=slopes,
                       block_mask=bm)[1]
    check_grads(name, [host_f64(g) for g in got], want, terms, dt, say=say)
    assert np.all(host_f64(got[0])[:, 64:128] == 0), "dq of a query block with every block off"
    assert np.all(host_f64(got[1])[:, 128:192] == 0) and np.all(host_f64(got[2])[:, 128:192] == 0), \
        "dk, dv of a key block no query sees"
