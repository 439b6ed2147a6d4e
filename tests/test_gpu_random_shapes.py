"""Seeded random small configurations through forward and backward, against the fp64 oracle.

Each case draws (dense or packed, M, N or segment lengths, Hq, Hkv, D, dtype,
causal, ALiBi) from a fixed seed, so every run checks the same 36 cases; the
hand-written parity tests pick the shapes that matter, these cover the
combinations between them.
"""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, dev, f32, host_f64, i32, say
from grad_bounds import check_grads, grad_terms

pytestmark = pytest.mark.gpu



def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dt = ["fp16", "bf16"][rng.integers(2)]
    D = [64, 128][rng.integers(2)]
    Hkv = int(rng.choice([1, 2, 3]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    causal = bool(rng.integers(2))
    alibi = bool(rng.integers(2))
    if rng.integers(3) == 0:
        lengths = [int(x) for x in rng.integers(0, 200, int(rng.integers(1, 6)))]
        return dict(dt=dt, D=D, Hq=Hq, Hkv=Hkv, causal=causal, alibi=alibi, lengths=lengths)
    B = int(rng.integers(1, 4))
    M = int(rng.integers(1, 300))
    N = int(rng.integers(1, 300))
    return dict(dt=dt, D=D, Hq=Hq, Hkv=Hkv, causal=causal, alibi=alibi, B=B, M=M, N=N)


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


@pytest.mark.parametrize("seed", range(36))
def test_random_shape(mea, seed):
    cfg = _draw(seed)
    say(f"case random {seed}: {cfg}")
    dt, D, Hq, Hkv = cfg["dt"], cfg["D"], cfg["Hq"], cfg["Hkv"]
    slopes = inp.alibi_slopes(Hq) if cfg["alibi"] else None
    if "lengths" in cfg:
        c = inp.varlen_case(seed, cfg["lengths"], Hq, Hkv, D, dt)
        st = c["seqstart"]
        T = int(st[-1])
        if T == 0:
            pytest.skip("all segments empty")
        kw_dev = dict(seqstart_q=i32(st))
        kw_orc = dict(seqstart_q=st)
        lse_shape = (Hq, T)
    else:
        c = inp.dense_case(seed, cfg["B"], cfg["M"], cfg["N"], Hq, Hkv, D, dt)
        kw_dev, kw_orc = {}, {}
        lse_shape = (cfg["B"], Hq, cfg["M"])
    do = inp.normal_bits(seed + 900, c["q"].shape, dt, 0)
    q, k, v, dod = (dev(x, dt) for x in (c["q"], c["k"], c["v"], do))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    sl = None if slopes is None else f32(slopes)
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=cfg["causal"], scale=scale, alibi_slopes=sl, lse=lse, **kw_dev)
    grads = mea.bwd(q, k, v, out, dod, lse, causal=cfg["causal"], scale=scale, alibi_slopes=sl, **kw_dev)
    torch.cuda.synchronize()

    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=cfg["causal"], alibi_slopes=slopes, **kw_orc)
    assert float(np.max(np.abs(host_f64(out) - want))) <= TOL[dt], "out"
    wl = wlse[0] if "lengths" in cfg else wlse
    gl = lse.cpu().numpy()
    fin = np.isfinite(wl)
    assert np.array_equal(np.isfinite(gl), fin), "lse -inf pattern"
    assert np.max(np.abs(gl[fin] - wl[fin]), initial=0.0) <= LSE_TOL[dt], "lse"

    wg = orc.bwd(c["q"], c["k"], c["v"], do, dt, scale, causal=cfg["causal"], alibi_slopes=slopes, **kw_orc)
    # the backward tests' element-wise bar (C u times the magnitude sum of each
    # element's own terms)
    terms = grad_terms(c["q"], c["k"], c["v"], do, dt, scale, causal=cfg["causal"], alibi_slopes=slopes,
                       **kw_orc)[1]
    check_grads(f"random {seed}", [host_f64(g) for g in grads], wg, terms, dt, say=say)
