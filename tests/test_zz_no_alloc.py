"""mea_decode_noalloc (the decode step with the library's static per-device
scratch instead of a caller workspace) against mea_decode, on the GPU.

Both entry points run the same kernels over the same split of the keys, so
their outputs must be bitwise equal; both are also held to the fp64 oracle's
bar (max-abs 1.6e-2 bf16, 2e-3 fp16). Two calls in a row, the second with a
smaller batch, check that what the first call leaves in the shared scratch
does not leak into the second. Calls go through the C ABI with ctypes.
"""
import ctypes

import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import TOL, dev, host_f64, i32, report, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(mea, q, kc, vc, ctx, out, scale, slopes, dtype_code):
    B, Hq, D = q.shape
    S_max, Hkv = kc.shape[1], kc.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return mea.lib().mea_decode_noalloc(_ptr(q), _ptr(kc), _ptr(vc), _ptr(ctx), _ptr(out), B, Hq, Hkv, D, S_max,
                                        ctypes.c_float(scale), _ptr(slopes), dtype_code, stream)


CASES = [
    # name, seed, ctx lengths, S_max, Hq, Hkv, D, dtype, alibi
    ("bf16_b12_then_b3", 61, [5000, 1, 0, 777, 4096, 300, 64, 65, 12000, 2, 999, 3333], 12288, 8, 2, 128, "bf16",
     False),
    ("fp16_alibi_d64_b9_then_b3", 62, [100, 2000, 1, 513, 0, 3000, 63, 64, 700], 4096, 16, 4, 64, "fp16", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_noalloc_matches_decode_twice(mea, case):
    name, seed, ctx, S_max, Hq, Hkv, D, dt, alibi = case
    code = mea.MEA_BF16 if dt == "bf16" else mea.MEA_FP16
    scale = float(np.float32(1.0 / np.sqrt(D)))
    slopes = inp.alibi_slopes(Hq) if alibi else None
    sl = None if slopes is None else torch.from_numpy(slopes).cuda()
    first = inp.decode_case(seed, ctx, S_max, Hq, Hkv, D, dt)
    # The second call: a smaller batch (the last three sequences of a new draw).
    second = inp.decode_case(seed + 1, ctx[-3:], S_max, Hq, Hkv, D, dt)
    for label, c in (("first", first), ("second, smaller", second)):
        say(f"case noalloc {name} {label}: B={len(c['ctx_lens'])}")
        q, kc, vc = dev(c["q"], dt), dev(c["kcache"], dt), dev(c["vcache"], dt)
        ctx_d = i32(c["ctx_lens"])
        ref = mea.decode(q, kc, vc, ctx_d, scale=scale, alibi_slopes=sl)
        out = torch.full_like(q, float("nan"))
        rc = _noalloc(mea, q, kc, vc, ctx_d, out, scale, sl, code)
        torch.cuda.synchronize()
        assert rc == mea.MEA_OK, mea.strerror(rc)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{label}: not bitwise equal to mea_decode"
        want = orc.decode(c["q"], c["kcache"], c["vcache"], c["ctx_lens"], dt, scale, alibi_slopes=slopes)
        assert report(f"noalloc {name} {label}", host_f64(out), want, TOL[dt]) <= TOL[dt]


def test_noalloc_binding_and_limit(mea):
    """The Python binding reaches the same entry point; a step too large for
    the scratch is refused with MEA_ESCRATCH before anything is launched."""
    say("case noalloc binding and limit")
    c = inp.decode_case(63, [300, 1, 64], 512, 4, 1, 128, "bf16")
    q, kc, vc = dev(c["q"], "bf16"), dev(c["kcache"], "bf16"), dev(c["vcache"], "bf16")
    ctx_d = i32(c["ctx_lens"])
    out = torch.empty_like(q)
    mea.decode_noalloc(q, kc, vc, ctx_d, out)
    ref = mea.decode(q, kc, vc, ctx_d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # B=4096, Hq=64, D=128: (256 + 4096) * 64 * 130 * 4 bytes, well above 32 MiB.
    B, Hq, D = 4096, 64, 128
    qb = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((B, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    ctx_big = torch.ones(B, dtype=torch.int32, device="cuda")
    outb = torch.empty_like(qb)
    rc = _noalloc(mea, qb, cache, cache, ctx_big, outb, 0.1, None, mea.MEA_BF16)
    assert rc == mea.MEA_ESCRATCH
    assert "scratch" in mea.strerror(rc)


def test_noalloc_inside_a_captured_graph(mea):
    """The callers the entry point is for: a decode step captured in a HIP
    graph with no workspace allocated. Three replays, with eager work and
    synchronisations between them, each bitwise equal to mea_decode."""
    say("case noalloc graph capture")
    dt, Hq, Hkv, D = "bf16", 16, 4, 128
    c = inp.decode_case(64, [900, 1, 4096, 0, 513, 77], 4096, Hq, Hkv, D, dt)
    q, kc, vc = dev(c["q"], dt), dev(c["kcache"], dt), dev(c["vcache"], dt)
    ctx_d = i32(c["ctx_lens"])
    want = mea.decode(q, kc, vc, ctx_d)
    out = torch.empty_like(q)
    mea.decode_noalloc(q, kc, vc, ctx_d, out)          # first call on this device: resolves the scratch
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mea.decode_noalloc(q, kc, vc, ctx_d, out)      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mea.decode_noalloc(q, kc, vc, ctx_d, out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
