"""The Python binding's argument checks, on the CPU.

The C ABI takes plain pointers, so an output or side array smaller than the
sizes passed would be written or read past its end by the kernels. The
binding derives every size from q/k (or the caches) and rejects any other
array whose shape, length or dtype disagrees, before it touches the device.
The tensors here are CPU tensors: each call must fail on its shape check,
not on the later device check.
"""
import pytest
import torch

mea = pytest.importorskip("memory_efficient_exact_tiled_amd")

BF = torch.bfloat16
F32 = torch.float32
I32 = torch.int32


def _raises(fn, match):
    with pytest.raises((ValueError, TypeError), match=match):
        fn()


def test_fwd_rejects_mis_sized_arrays():
    q = torch.zeros(2, 64, 4, 64, dtype=BF)
    k = torch.zeros(2, 80, 2, 64, dtype=BF)
    _raises(lambda: mea.fwd(q, k, k, out=torch.zeros(2, 64, 4, 32, dtype=BF)), "out must be")
    _raises(lambda: mea.fwd(q, k, k, out=torch.zeros(2, 64, 4, 64, dtype=torch.float16)), "out must be")
    _raises(lambda: mea.fwd(q, k, k, lse=torch.zeros(2, 4, 63, dtype=F32)), "lse must hold 512")
    _raises(lambda: mea.fwd(q, k, k, lse=torch.zeros(2, 4, 64, dtype=BF)), "lse must hold")
    _raises(lambda: mea.fwd(q, k, k, alibi_slopes=torch.zeros(3, dtype=F32)), "alibi_slopes must hold 4")
    _raises(lambda: mea.fwd(q[0], k[0], k[0]), "dense q/k")
    _raises(lambda: mea.fwd(q, k, k, seqstart_k=torch.zeros(3, dtype=I32)), "seqstart_k needs seqstart_q")


def test_packed_fwd_rejects_bad_seqstart():
    q = torch.zeros(1, 100, 4, 64, dtype=BF)
    k = torch.zeros(1, 100, 4, 64, dtype=BF)
    st = torch.tensor([0, 40, 100], dtype=I32)
    _raises(lambda: mea.fwd(q, k, k, seqstart_q=st.to(torch.int64)), "1-D int32")
    _raises(lambda: mea.fwd(q, k, k, seqstart_q=st.reshape(1, 3)), "1-D int32")
    _raises(lambda: mea.fwd(q, k, k, seqstart_q=st, seqstart_k=torch.tensor([0, 100], dtype=I32)),
            "as many entries")
    _raises(lambda: mea.fwd(q, k, k, seqstart_q=torch.tensor([0], dtype=I32)), "at least two entries")
    _raises(lambda: mea.fwd(q, k, k, seqstart_q=st, lse=torch.zeros(4, 99, dtype=F32)), "lse must hold 400")
    _raises(lambda: mea.fwd(torch.zeros(2, 100, 4, 64, dtype=BF), k, k, seqstart_q=st), r"\[1,T,H,D\]")


def test_blocksparse_rejects_mis_sized_arrays():
    q = torch.zeros(1, 128, 4, 64, dtype=BF)
    bm = torch.ones(2, 2, dtype=torch.uint8)
    _raises(lambda: mea.fwd_blocksparse(q, q, q, bm, out=torch.zeros(1, 127, 4, 64, dtype=BF)), "out must be")
    _raises(lambda: mea.fwd_blocksparse(q, q, q, bm, lse=torch.zeros(1, 4, 120, dtype=F32)), "lse must hold")
    _raises(lambda: mea.fwd_blocksparse(q, q, q, bm, alibi_slopes=torch.zeros(8, dtype=F32)), "alibi_slopes")
    _raises(lambda: mea.fwd_blocksparse(q, q, q, torch.ones(2, 3, dtype=torch.uint8)), "block_mask must be")


def test_bwd_rejects_mis_sized_arrays():
    q = torch.zeros(2, 64, 4, 64, dtype=BF)
    k = torch.zeros(2, 80, 2, 64, dtype=BF)
    lse = torch.zeros(2, 4, 64, dtype=F32)
    _raises(lambda: mea.bwd(q, k, k, q, q, lse, dq=torch.zeros(2, 64, 4, 63, dtype=BF)), "dq must be")
    _raises(lambda: mea.bwd(q, k, k, q, q, lse, dk=torch.zeros(2, 80, 4, 64, dtype=BF)), "dk must be")
    _raises(lambda: mea.bwd(q, k, k, q, q, lse, dv=torch.zeros(2, 80, 2, 64, dtype=F32)), "dv must be")
    _raises(lambda: mea.bwd(q, k, k, q, q, lse, alibi_slopes=torch.zeros(2, dtype=F32)), "alibi_slopes")
    _raises(lambda: mea.bwd(q, k, k, q, q, lse[:, :, :32]), "lse must be")
    _raises(lambda: mea.bwd(q, k, k, q[:, :32], q, lse), "out and dout must match q")


def test_decode_and_cache_calls_reject_mis_sized_arrays():
    q = torch.zeros(3, 8, 128, dtype=BF)
    kc = torch.zeros(3, 50, 2, 128, dtype=BF)
    ctx = torch.tensor([1, 2, 3], dtype=I32)
    _raises(lambda: mea.decode(q, kc, kc, ctx, out=torch.zeros(3, 8, 64, dtype=BF)), "out must be")
    _raises(lambda: mea.decode(q, kc, kc, ctx, alibi_slopes=torch.zeros(2, dtype=F32)), "alibi_slopes")
    _raises(lambda: mea.decode(q, kc, kc, ctx[:2]), "B entries")
    _raises(lambda: mea.decode_noalloc(q, kc, kc, ctx, torch.zeros(3, 8, 128, dtype=BF),
                                       alibi_slopes=torch.zeros(9, dtype=F32)), "alibi_slopes")
    _raises(lambda: mea.decode_noalloc(q, kc, kc, ctx, torch.zeros(3, 7, 128, dtype=BF)), "out is shaped like q")
    qm = torch.zeros(3, 5, 8, 128, dtype=BF)
    _raises(lambda: mea.fwd_kvcache(qm, kc, kc, ctx, out=torch.zeros(3, 5, 8, 64, dtype=BF)), "out must be")
    _raises(lambda: mea.fwd_kvcache(qm, kc, kc, ctx, lse=torch.zeros(3, 8, 4, dtype=F32)), "lse must hold 120")
    _raises(lambda: mea.fwd_kvcache(qm, kc, kc, ctx, alibi_slopes=torch.zeros(2, dtype=F32)), "alibi_slopes")
    _raises(lambda: mea.kv_append(kc, kc, torch.zeros(3, 4, 2, 64, dtype=BF), torch.zeros(3, 4, 2, 64, dtype=BF),
                                  ctx), "shapes disagree")
