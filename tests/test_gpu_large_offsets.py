"""Element offsets past 2^31 on the GPU: packed forward and backward batches
whose q, k, v, output and gradient tensors hold more than 2^31 elements each,
and a decode step whose caches hold 2^32 elements per tensor.

Offsets of whole tensors are 64-bit in the kernels (row strides and per-row
offsets within a segment or sequence are 32-bit); these tests place seeded
segments and sequences behind the 2^31-element mark and compare them with
the fp64 oracle. The rest of each tensor is filler: zeros for the packed
batches (their segments attend to zeros), and NaN bit patterns in every cache
slot a context does not cover (a read of one would surface as NaN).
"""
import numpy as np
import pytest
import torch

import mea_inputs as inp
import oracle.attention as orc
from gpu_util import LSE_TOL, TOL, TORCH_DTYPE, dev, f32, host_f64, i32, report, say
from grad_bounds import check_grads, grad_terms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


PACKED = [
    # name, seed, H (= Hq = Hkv), D, causal, alibi
    ("causal_alibi_d128", 60, 16, 128, True, True),
    ("noncausal_d64", 61, 32, 64, False, False),
]


@pytest.mark.parametrize("case", PACKED, ids=lambda c: c[0])
def test_packed_forward_past_2g_elements(mea, case):
    name, seed, H, D, causal, alibi = case
    dt = "bf16"
    n_fill, fill_len = 4100, 256
    t0 = n_fill * fill_len                     # first token of the checked segments
    assert t0 * H * D > 2 ** 31
    test_lengths = [300, 1, 0, 700, 64]
    c = inp.varlen_case(seed, test_lengths, H, H, D, dt)
    T = t0 + int(c["seqstart"][-1])
    say(f"case large packed {name}: T={T} tokens, {T * H * D / 2 ** 31:.2f} x 2^31 elements per tensor")
    st = np.concatenate([np.arange(n_fill, dtype=np.int64) * fill_len, t0 + c["seqstart"]]).astype(np.int32)
    tdt = TORCH_DTYPE[dt]
    q = torch.zeros((1, T, H, D), dtype=tdt, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    q[0, t0:] = dev(c["q"], dt)[0]
    k[0, t0:] = dev(c["k"], dt)[0]
    v[0, t0:] = dev(c["v"], dt)[0]
    slopes = inp.alibi_slopes(H) if alibi else None
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=causal, scale=scale, seqstart_q=i32(st),
                  alibi_slopes=None if slopes is None else f32(slopes), lse=lse)
    torch.cuda.synchronize()
    got = host_f64(out[0, t0:])
    got_lse = lse[:, t0:].cpu().numpy()
    fill_out = float(out[0, :t0].abs().max().item())
    del q, k, v, out
    torch.cuda.empty_cache()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, seqstart_q=c["seqstart"],
                         alibi_slopes=slopes)
    assert report(f"large packed {name}", got, want[0], TOL[dt]) <= TOL[dt]
    fin = np.isfinite(wlse[0])
    assert np.array_equal(np.isfinite(got_lse), fin), "lse -inf pattern"
    assert float(np.max(np.abs(got_lse[fin] - wlse[0][fin]))) <= LSE_TOL[dt]
    assert fill_out == 0.0, "filler segments attend to zeros"


def test_packed_backward_past_2g_elements(mea):
    dt, H, D, seed = "bf16", 16, 128, 63
    n_fill, fill_len = 4100, 256
    t0 = n_fill * fill_len
    assert t0 * H * D > 2 ** 31
    test_lengths = [300, 1, 0, 700, 64]
    c = inp.varlen_case(seed, test_lengths, H, H, D, dt)
    do_bits = inp.normal_bits(seed + 1, c["q"].shape, dt, 0)
    T = t0 + int(c["seqstart"][-1])
    say(f"case large packed backward: T={T} tokens, causal ALiBi, H={H}, D={D}")
    st = np.concatenate([np.arange(n_fill, dtype=np.int64) * fill_len, t0 + c["seqstart"]]).astype(np.int32)
    tdt = TORCH_DTYPE[dt]
    q = torch.zeros((1, T, H, D), dtype=tdt, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    do = torch.zeros_like(q)
    q[0, t0:] = dev(c["q"], dt)[0]
    k[0, t0:] = dev(c["k"], dt)[0]
    v[0, t0:] = dev(c["v"], dt)[0]
    do[0, t0:] = dev(do_bits, dt)[0]
    slopes = inp.alibi_slopes(H)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    sq, sl = i32(st), f32(slopes)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=True, scale=scale, seqstart_q=sq, alibi_slopes=sl, lse=lse)
    dq, dk, dv = mea.bwd(q, k, v, out, do, lse, causal=True, scale=scale, alibi_slopes=sl, seqstart_q=sq)
    torch.cuda.synchronize()
    got = [host_f64(g[0, t0:])[None] for g in (dq, dk, dv)]
    fill = max(float(g[0, :t0].abs().max().item()) for g in (dq, dk, dv))
    del q, k, v, do, out, dq, dk, dv
    torch.cuda.empty_cache()
    kw = dict(causal=True, seqstart_q=c["seqstart"], alibi_slopes=slopes)
    want = orc.bwd(c["q"], c["k"], c["v"], do_bits, dt, scale, **kw)
    terms = grad_terms(c["q"], c["k"], c["v"], do_bits, dt, scale, **kw)[1]
    check_grads("large packed backward", got, want, terms, dt, say=say)
    assert fill == 0.0, "filler segments have zero gradients"


def test_decode_past_2g_elements(mea):
    dt, B, S, Hq, Hkv, D = "bf16", 64, 65536, 32, 8, 128
    assert B * S * Hkv * D > 2 ** 31
    ctx = inp.context_lengths(62, B, 1, 64)
    ctx[-3:] = [40000, S, 12345]                # the last sequences start past 2^31 elements
    checked = [0, 30, B - 3, B - 2, B - 1]
    say(f"case large decode: caches of {B * S * Hkv * D / 2 ** 31:.1f} x 2^31 elements, ctx tail={ctx[-3:].tolist()}")
    kc = torch.empty((B, S, Hkv, D), dtype=torch.int16, device="cuda")
    kc.fill_(int(inp.POISON[dt].view(np.int16)))
    vc = kc.clone()
    rows = {}
    for b in range(B):
        kb, vb = inp.decode_cache_rows(62, b, int(ctx[b]), Hkv, D, dt)
        kc[b, :ctx[b]] = torch.from_numpy(kb.view(np.int16)).cuda()
        vc[b, :ctx[b]] = torch.from_numpy(vb.view(np.int16)).cuda()
        if b in checked:
            rows[b] = (kb, vb)
    q_bits = inp.normal_bits(62, (B, Hq, D), dt, 0)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = mea.decode(dev(q_bits, dt), kc.view(TORCH_DTYPE[dt]), vc.view(TORCH_DTYPE[dt]), i32(ctx), scale=scale)
    torch.cuda.synchronize()
    got = host_f64(out)
    del kc, vc
    torch.cuda.empty_cache()
    for b in checked:
        kb, vb = rows[b]
        want = orc.decode(q_bits[b:b + 1], kb[None], vb[None], ctx[b:b + 1], dt, scale)[0]
        assert report(f"large decode b{b} ctx={int(ctx[b])}", got[b], want, TOL[dt]) <= TOL[dt]
