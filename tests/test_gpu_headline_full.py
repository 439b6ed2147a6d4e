"""Whole-output parity at the full workload sizes, on the GPU.

The xFormers tutorial validates the memory-efficient kernel by comparing its
whole output with a standard implementation ("Come costruire Transformer
efficienti in memoria con xFormers...", chipsbuilder.com, section "Impostare
xFormers e Validare l'Attenzione Memory-Efficient"). These tests do the same at
the sizes the benchmark times, element by element against the fp64 oracle:

* the sequence-length sweep at M = N = 2048 and 4096 (B=4, H=16, D=64, bf16),
  without mask and causal: every output element and every row's lse; the
  same at M = 4096 in fp16 (its tighter bar, other kernel instances);
* the packed batch of 8 segments with lengths uniform in [64, 2048], Hq=32,
  Hkv=8, D=128, bf16, block-diagonal causal + ALiBi: every row of every
  segment, output and lse;
* the decode step, B=32, contexts uniform in [1024, 32768], Hq=32, Hkv=8,
  D=128, bf16, S_max=32768, with every sequence's cache filled: every output
  element (slots past each context hold NaN and must not be read);
* the backward at the size the benchmark times it (B=4, M=N=4096, H=16, D=64,
  bf16, without mask and causal): every element of dq, dk and dv of every
  (batch row, head), each against its own element-wise bar (the magnitudes of
  its terms, grad_bounds.py).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, dev, f32, host_f64, i32, report, say
from grad_bounds import check_grads, grad_terms

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _check_lse(name, got, want, dt):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: lse -inf pattern"
    err = float(np.max(np.abs(got[fin] - want[fin]), initial=0.0))
    say(f"[{name} lse] max_abs_err={err:.3e} tol={LSE_TOL[dt]:.2e}")
    assert err <= LSE_TOL[dt], name


@pytest.mark.parametrize("M,dt", [(2048, "bf16"), (4096, "bf16"), (4096, "fp16")])
@pytest.mark.parametrize("causal", [False, True])
def test_seqlen_sweep_whole_output(mea, M, dt, causal):
    B, H, D = 4, 16, 64
    name = f"cfg3_m{M}_{dt}_{'causal' if causal else 'noncausal'}_whole"
    say(f"case {name}")
    c = inp.dense_case(3, B, M, M, H, H, D, dt)       # the benchmark's inputs at M=4096
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((B, H, M), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=causal, scale=scale, lse=lse)
    torch.cuda.synchronize()
    got, got_lse = host_f64(out), lse.cpu().numpy()

    def one(b):
        return orc.fwd_rows(c["q"], c["k"], c["v"], dt, scale, b, np.arange(M), causal=causal)

    with ThreadPoolExecutor(max_workers=2) as ex:
        res = list(ex.map(one, range(B)))
    want = np.stack([r[0] for r in res])
    wlse = np.stack([r[1] for r in res])
    assert report(name, got, want, TOL[dt]) <= TOL[dt]
    _check_lse(name, got_lse, wlse, dt)


def test_packed_gqa_alibi_whole_output(mea):
    lengths = inp.segment_lengths(4, 8, 64, 2048)     # the benchmark's packed batch
    say(f"case cfg4 whole lengths={lengths.tolist()}")
    dt, Hq, Hkv, D = "bf16", 32, 8, 128
    c = inp.varlen_case(4, lengths, Hq, Hkv, D, dt)
    slopes = inp.alibi_slopes(Hq)
    T = int(c["seqstart"][-1])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((Hq, T), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt), causal=True, scale=scale,
                  seqstart_q=i32(c["seqstart"]), alibi_slopes=f32(slopes), lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=True, seqstart_q=c["seqstart"],
                         alibi_slopes=slopes)
    assert report(f"cfg4 all {T} rows", host_f64(out), want, TOL[dt]) <= TOL[dt]
    _check_lse("cfg4", lse.cpu().numpy(), wlse[0], dt)


def test_decode_every_sequence(mea):
    B, S, Hq, Hkv, D, dt = 32, 32768, 32, 8, 128, "bf16"
    ctx = inp.context_lengths(5, B, 1024, 32768)      # the benchmark's decode batch
    say(f"case cfg5 all {B} sequences, sum(ctx)={int(ctx.sum())}")
    q_bits = inp.normal_bits(5, (B, Hq, D), dt, 0)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    kc = torch.empty((B, S, Hkv, D), dtype=torch.int16, device="cuda")
    kc.fill_(int(inp.POISON[dt].view(np.int16)))
    vc = kc.clone()

    def one(b):
        n = int(ctx[b])
        kb, vb = inp.decode_cache_rows(5, b, n, Hkv, D, dt)
        want = orc.decode(q_bits[b:b + 1], kb[None], vb[None], ctx[b:b + 1], dt, scale)[0]
        return b, kb, vb, want

    want = np.empty((B, Hq, D))
    with ThreadPoolExecutor(max_workers=WORKERS) as ex:
        for b, kb, vb, w in ex.map(one, range(B)):
            kc[b, :ctx[b]] = torch.from_numpy(kb.view(np.int16)).cuda()
            vc[b, :ctx[b]] = torch.from_numpy(vb.view(np.int16)).cuda()
            want[b] = w
    say("cfg5 caches filled, oracle done")
    out = mea.decode(dev(q_bits, dt), kc.view(torch.bfloat16), vc.view(torch.bfloat16), i32(ctx), scale=scale)
    torch.cuda.synchronize()
    assert report("cfg5 all sequences", host_f64(out), want, TOL[dt]) <= TOL[dt]


def _bwd_head(args):
    """Oracle gradients and their bar terms for one (batch row, head)."""
    q, k, v, do, scale, causal = args
    want = orc.bwd(q, k, v, do, "bf16", scale, causal=causal)
    return want, grad_terms(q, k, v, do, "bf16", scale, causal=causal)[1]


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_whole_output(mea, causal):
    B, M, H, D, dt = 4, 4096, 16, 64, "bf16"
    name = f"bwd_b4_m4096_h16_{'causal' if causal else 'noncausal'}_whole"
    say(f"case {name}")
    c = inp.dense_case(31 + causal, B, M, M, H, H, D, dt)
    do = inp.normal_bits(531, (B, M, H, D), dt, 0)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qd, kd, vd, dod = (dev(x, dt) for x in (c["q"], c["k"], c["v"], do))
    lse = torch.empty((B, H, M), dtype=torch.float32, device="cuda")
    out = mea.fwd(qd, kd, vd, causal=causal, scale=scale, lse=lse)
    grads = mea.bwd(qd, kd, vd, out, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = [host_f64(g) for g in grads]
    want = [np.empty_like(g) for g in got]
    terms = [np.empty_like(g) for g in got]
    jobs = []
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            jobs.append(((b, h), (c["q"][sl], c["k"][sl], c["v"][sl], do[sl], scale, causal)))
    # Each job holds a few 4096 x 4096 float64 matrices (about 1.5 GB).
    with ThreadPoolExecutor(max_workers=min(WORKERS, 8)) as ex:
        for (b, h), (w, t) in zip((j[0] for j in jobs), ex.map(_bwd_head, (j[1] for j in jobs))):
            for arr, x in zip(want, w):
                arr[b, :, h] = x[0, :, 0]
            for arr, x in zip(terms, t):
                arr[b, :, h] = x[0, :, 0]
    say(f"{name}: oracle done for {B * H} (batch row, head) pairs")
    check_grads(name, got, want, terms, dt, say=say)
