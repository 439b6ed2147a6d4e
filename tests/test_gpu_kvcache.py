"""KV-cache append (bit-exact) and multi-token decode over a cache, against the fp64 oracle, on the GPU."""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, dev, f32, host_bits, host_f64, i32, report, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64)])
def test_kv_append_bitexact(mea, dt, D):
    B, S, Hkv, T = 4, 300, 2, 37
    ctx = np.array([0, 100, 280, 300], np.int32)        # the last two overflow S_max
    kc = inp.normal_bits(50, (B, S, Hkv, D), dt, 0)
    vc = inp.normal_bits(50, (B, S, Hkv, D), dt, 1)
    kn = inp.normal_bits(51, (B, T, Hkv, D), dt, 0)
    vn = inp.normal_bits(51, (B, T, Hkv, D), dt, 1)
    dkc, dvc = dev(kc, dt), dev(vc, dt)
    mea.kv_append(dkc, dvc, dev(kn, dt), dev(vn, dt), i32(ctx))
    torch.cuda.synchronize()
    wk, wv = orc.kv_append(kc, vc, kn, vn, ctx)
    assert np.array_equal(host_bits(dkc), wk) and np.array_equal(host_bits(dvc), wv)


CASES = [
    # name, seed, ctx, S_max, M, Hq, Hkv, D, dtype, causal, alibi
    ("chunk7_d128_bf16_alibi", 1, [700, 64, 7, 3], 800, 7, 8, 2, 128, "bf16", True, True),
    ("chunk130_d64_fp16", 2, [130, 1000, 257], 1024, 130, 4, 4, 64, "fp16", True, False),
    ("single_query_d128", 3, [1, 513, 2000], 2048, 1, 16, 2, 128, "bf16", True, False),
    ("noncausal_chunk", 4, [90, 300], 300, 33, 4, 1, 64, "bf16", False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fwd_kvcache_parity(mea, case):
    name, seed, ctx, S, M, Hq, Hkv, D, dt, causal, alibi = case
    say(f"case {name}")
    d = inp.decode_case(seed, ctx, S, Hq, Hkv, D, dt)          # slots >= ctx hold NaN
    q = inp.normal_bits(seed + 100, (len(ctx), M, Hq, D), dt, 0)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((len(ctx), Hq, M), 5.0, dtype=torch.float32, device="cuda")
    out = mea.fwd_kvcache(dev(q, dt), dev(d["kcache"], dt), dev(d["vcache"], dt), i32(d["ctx_lens"]), causal=causal,
                          scale=scale, alibi_slopes=None if slopes is None else f32(slopes), lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd_kvcache(q, d["kcache"], d["vcache"], d["ctx_lens"], dt, scale, causal=causal,
                                 alibi_slopes=slopes)
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    assert report(name, got, want, TOL[dt]) <= TOL[dt]
    gl = lse.cpu().numpy()
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.max(np.abs(gl[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dt]


def test_append_then_attend_matches_full_causal(mea):
    """Prefill a cache, append a chunk of 40 new tokens, attend the chunk over
    the cache: equals the last 40 rows of causal attention over the whole
    sequence (all on the GPU, within twice the tolerance)."""
    B, S, Hq, Hkv, D, P, T = 2, 512, 8, 2, 128, 300, 40
    full = inp.dense_case(60, B, P + T, P + T, Hq, Hkv, D, "bf16")
    kc = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :P] = dev(full["k"][:, :P], "bf16")
    vc[:, :P] = dev(full["v"][:, :P], "bf16")
    mea.kv_append(kc, vc, dev(full["k"][:, P:], "bf16"), dev(full["v"][:, P:], "bf16"), i32([P] * B))
    q = dev(full["q"], "bf16")
    chunk = mea.fwd_kvcache(q[:, P:].contiguous(), kc, vc, i32([P + T] * B))
    ref = mea.fwd(q, dev(full["k"], "bf16"), dev(full["v"], "bf16"), causal=True)
    torch.cuda.synchronize()
    assert report("append+attend", host_f64(chunk), host_f64(ref[:, P:]), 2 * TOL["bf16"]) <= 2 * TOL["bf16"]
