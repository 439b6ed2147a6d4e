"""The entry points inside a captured HIP graph.

The library allocates nothing and issues no memset, so a caller can capture
a forward, its backward and a decode step on one stream and replay them
(serving loops, launch-bound inner loops). Each replay, with eager work and
synchronisations between replays, must reproduce the eager results bit for
bit: every kernel is deterministic.
"""
import numpy as np
import pytest
import torch

import mea_inputs as inp
from gpu_util import dev, f32, i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_exact_tiled_amd as m
    return m


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_fwd_bwd_decode_graph_replays_are_bitwise_eager(mea):
    say("case graph capture: packed causal ALiBi GQA fwd + bwd, decode")
    dt, Hq, Hkv, D = "bf16", 8, 2, 128
    c = inp.varlen_case(31, [37, 200, 64, 129], Hq, Hkv, D, dt)
    T = int(c["seqstart"][-1])
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    do = dev(inp.normal_bits(32, c["q"].shape, dt, 0), dt)
    st = i32(c["seqstart"])
    sl = f32(inp.alibi_slopes(Hq))
    d = inp.decode_case(33, [700, 1, 0, 513], 1024, Hq, Hkv, D, dt)
    dq_, dk_, dv_ = dev(d["q"], dt), dev(d["kcache"], dt), dev(d["vcache"], dt)
    ctx = i32(d["ctx_lens"])

    # Every buffer the captured calls touch is allocated before capture.
    out = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(mea.bwd_workspace_bytes(1, T, Hq, mea.MEA_MASK_CAUSAL | mea.MEA_MASK_BLOCKDIAG | mea.MEA_BIAS_ALIBI),
                      dtype=torch.uint8, device="cuda")
    dout = torch.empty_like(dq_)
    dws = torch.empty(mea.decode_workspace_bytes(4, Hq, D, 1024), dtype=torch.uint8, device="cuda")

    def step():
        mea.fwd(q, k, v, causal=True, seqstart_q=st, alibi_slopes=sl, out=out, lse=lse)
        mea.bwd(q, k, v, out, do, lse, causal=True, seqstart_q=st, alibi_slopes=sl, dq=gq, dk=gk, dv=gv,
                workspace=bws)
        mea.decode(dq_, dk_, dv_, ctx, out=dout, workspace=dws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, gq, gk, gv, dout)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (out, lse, gq, gk, gv, dout):
            t.fill_(0)              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("out", "lse", "dq", "dk", "dv", "decode"), (out, lse, gq, gk, gv, dout), eager):
            assert torch.equal(_bits(t), _bits(e)), (rep, name)
