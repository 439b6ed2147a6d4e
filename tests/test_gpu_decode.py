"""Parity of the HIP decode step (split-KV + combine, through the C ABI) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import TOL, TORCH_DTYPE, dev, f32, host_f64, i32, report, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


SMALL = [
    # name, seed, ctx_lens, S_max, Hq, Hkv, D, dtype, alibi
    ("chunk_edges_d128_bf16", 1, [1, 511, 512, 513, 1500, 2000], 2000, 8, 2, 128, "bf16", False),
    ("chunk_edges_d64_fp16_alibi", 2, [1024, 3, 1537, 64], 1600, 4, 4, 64, "fp16", True),
    ("empty_context", 3, [0, 5, 0], 64, 4, 1, 128, "bf16", False),
    ("group_20_two_head_blocks", 4, [700, 33], 800, 40, 2, 64, "bf16", True),
    ("mha_group_1", 5, [900, 1], 1000, 6, 6, 128, "fp16", False),
    # many short sequences (some empty) share one split work-group's span
    ("many_short_in_one_span", 6, [int(x) for x in np.random.default_rng(6).integers(0, 100, 40)] + [3000],
     3000, 8, 2, 64, "bf16", True),
    # more than 256 sequences: the context prefix sums carry across the
    # plan's 256-wide scan steps
    ("batch_300_scan_carry", 8, [int(x) for x in np.random.default_rng(8).integers(0, 60, 300)], 64, 2, 1, 64,
     "fp16", False),
    # more than 512 sequences: planned by the separate plan kernel
    ("batch_600_plan_kernel", 9, [int(x) for x in np.random.default_rng(9).integers(0, 20, 600)], 32, 2, 1, 64,
     "bf16", False),
    # more keys than 512 per compute unit: spans longer than the chunk,
    # crossing sequence boundaries mid-span
    ("long_spans", 7, [70000, 70001, 1, 9000], 70001, 4, 1, 64, "fp16", True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_decode_parity_small(mea, case):
    name, seed, ctx, S, Hq, Hkv, D, dt, alibi = case
    say(f"case {name}")
    d = inp.decode_case(seed, ctx, S, Hq, Hkv, D, dt)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = mea.decode(dev(d["q"], dt), dev(d["kcache"], dt), dev(d["vcache"], dt), i32(d["ctx_lens"]),
                     scale=scale, alibi_slopes=None if slopes is None else f32(slopes))
    torch.cuda.synchronize()
    want = orc.decode(d["q"], d["kcache"], d["vcache"], d["ctx_lens"], dt, scale, alibi_slopes=slopes)
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    assert report(name, got, want, TOL[dt]) <= TOL[dt]


def test_decode_equals_last_row_of_causal_fwd(mea):
    """The scrapbox.io page's check: the newest query alone against the cache
    reproduces the last row of full causal attention (here both on the GPU)."""
    B, N, Hq, Hkv, D = 2, 1200, 8, 2, 128
    c = inp.dense_case(40, B, N, N, Hq, Hkv, D, "bf16")
    q, k, v = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16")
    full = mea.fwd(q, k, v, causal=True)
    dec = mea.decode(q[:, N - 1].contiguous(), k, v, i32([N] * B))
    torch.cuda.synchronize()
    a, b = host_f64(full[:, N - 1]), host_f64(dec)
    assert report("decode vs fwd last row", b, a, 2 * TOL["bf16"]) <= 2 * TOL["bf16"]


def test_decode_full_config_sampled(mea):
    """B=32, context lengths uniform in [1024, 32768] (seeded), Hq=32, Hkv=8,
    D=128, bf16, S_max=32768: caches of 4 sampled sequences hold data; every
    other slot holds NaN, which must stay confined to those sequences' rows."""
    B, S, Hq, Hkv, D = 32, 32768, 32, 8, 128
    ctx = inp.context_lengths(5, B, 1024, 32768)
    sample = [0, 7, int(np.argmax(ctx)), int(np.argmin(ctx))]
    say(f"case cfg5 sampled batches={sample} ctx={[int(ctx[b]) for b in sample]}")
    q_bits = inp.normal_bits(5, (B, Hq, D), "bf16", 0)
    kc = torch.full((B, S, Hkv, D), 0, dtype=torch.int16, device="cuda")
    kc.fill_(int(np.int16(inp.POISON["bf16"].view(np.int16))))
    vc = kc.clone()
    host = {}
    for b in sample:
        kb, vb = inp.decode_cache_rows(5, b, int(ctx[b]), Hkv, D, "bf16")
        host[b] = (kb, vb)
        kc[b, :ctx[b]] = torch.from_numpy(kb.view(np.int16)).cuda()
        vc[b, :ctx[b]] = torch.from_numpy(vb.view(np.int16)).cuda()
    kc, vc = kc.view(torch.bfloat16), vc.view(torch.bfloat16)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = mea.decode(dev(q_bits, "bf16"), kc, vc, i32(ctx), scale=scale)
    torch.cuda.synchronize()
    got = host_f64(out)
    for b in sample:
        n = int(ctx[b])
        kcb = host[b][0][None]
        vcb = host[b][1][None]
        want = orc.decode(q_bits[b:b + 1], kcb, vcb, np.array([n], np.int32), "bf16", scale)
        assert report(f"cfg5 b{b} ctx={n}", got[b], want[0], TOL["bf16"]) <= TOL["bf16"]
    others = [b for b in range(B) if b not in sample]
    assert np.all(np.isnan(got[others]))
