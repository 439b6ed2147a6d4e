"""The C-ABI library loads, exports every symbol include/mea.h declares, and
rejects invalid calls on the host before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

import memory_efficient_exact_tiled_amd as mea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mea.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mea_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(mea.LIB_PATH)
    names = _declared()
    assert set(names) == set(mea.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_and_supported():
    assert mea.strerror(0) == "success"
    for s in range(1, 6):
        assert mea.strerror(s) and mea.strerror(s) != "unknown status"
    assert mea.strerror(99) == "unknown status"
    for dt in (mea.MEA_FP16, mea.MEA_BF16):
        assert mea.supported(dt, 64) and mea.supported(dt, 128)
        assert not mea.supported(dt, 96) and not mea.supported(dt, 256)
    assert not mea.supported(7, 64)


def test_workspace_bytes():
    assert mea.decode_chunk() == 64
    # plan header [B + 2] int32, then partials [1024 + B][Hq][D] and their
    # (max, sum) pairs, each part 256-byte aligned; independent of S_max
    rows = 1024 + 32
    o = rows * 32 * 128 * 4
    head = ((32 + 2) * 4 + 255) // 256 * 256
    want = head + ((o + 255) // 256) * 256 + rows * 32 * 2 * 4
    assert mea.decode_workspace_bytes(32, 32, 128, 32768) == want
    assert mea.decode_workspace_bytes(32, 32, 128, 1) == want
    assert mea.decode_workspace_bytes(0, 32, 128, 32768) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, M=8, N=8, Hq=2, Hkv=1, D=64, scale=0.125, kind=0,
             sq=None, sk=None, sl=None, dtype=mea.MEA_BF16, lse=None, stream=None)
    a.update(kw)
    return mea.lib().mea_fwd(a["q"], a["k"], a["v"], a["out"], a["B"], a["M"], a["N"], a["Hq"], a["Hkv"], a["D"],
                             a["scale"], a["kind"], a["sq"], a["sk"], a["sl"], a["dtype"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mea.MEA_EINVAL),
    (dict(out=None), mea.MEA_EINVAL),
    (dict(B=0), mea.MEA_EINVAL),
    (dict(M=-1), mea.MEA_EINVAL),
    (dict(N=0), mea.MEA_EINVAL),
    (dict(Hq=3, Hkv=2), mea.MEA_EINVAL),
    (dict(scale=0.0), mea.MEA_EINVAL),
    (dict(scale=-0.5), mea.MEA_EINVAL),
    (dict(scale=float("nan")), mea.MEA_EINVAL),
    (dict(scale=float("inf")), mea.MEA_EINVAL),
    (dict(kind=8), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_BIAS_ALIBI), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_MASK_BLOCKDIAG), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_MASK_BLOCKDIAG, sq=FAKE, M=8, N=9), mea.MEA_EINVAL),
    (dict(D=96), mea.MEA_EUNSUPPORTED),
    (dict(dtype=5), mea.MEA_EUNSUPPORTED),
])
def test_fwd_rejects(kw, status):
    assert _fwd(**kw) == status


def _dec(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ctx=FAKE, out=FAKE, B=2, Hq=4, Hkv=2, D=128, S=1024, scale=0.1, sl=None,
             dtype=mea.MEA_FP16, ws=ctypes.c_void_p(0x100000), wsb=1 << 30, stream=None)
    a.update(kw)
    return mea.lib().mea_decode(a["q"], a["kc"], a["vc"], a["ctx"], a["out"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                a["S"], a["scale"], a["sl"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ctx=None), mea.MEA_EINVAL),
    (dict(kc=None), mea.MEA_EINVAL),
    (dict(B=0), mea.MEA_EINVAL),
    (dict(S=0), mea.MEA_EINVAL),
    (dict(Hq=6, Hkv=4), mea.MEA_EINVAL),
    (dict(scale=-1.0), mea.MEA_EINVAL),
    (dict(D=32), mea.MEA_EUNSUPPORTED),
    (dict(B=4, S=1 << 29), mea.MEA_EINVAL),    # context prefix sums overflow int32
    (dict(ws=None), mea.MEA_EWORKSPACE),
    (dict(wsb=16), mea.MEA_EWORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), mea.MEA_EWORKSPACE),
])
def test_decode_rejects(kw, status):
    assert _dec(**kw) == status


def _dec_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ctx=FAKE, out=FAKE, B=2, Hq=4, Hkv=2, D=128, S=1024, scale=0.1, sl=None,
             dtype=mea.MEA_FP16, stream=None)
    a.update(kw)
    return mea.lib().mea_decode_noalloc(a["q"], a["kc"], a["vc"], a["ctx"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                        a["D"], a["S"], a["scale"], a["sl"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ctx=None), mea.MEA_EINVAL),
    (dict(out=None), mea.MEA_EINVAL),
    (dict(B=0), mea.MEA_EINVAL),
    (dict(Hq=6, Hkv=4), mea.MEA_EINVAL),
    (dict(scale=float("nan")), mea.MEA_EINVAL),
    (dict(D=32), mea.MEA_EUNSUPPORTED),
    (dict(B=4, S=1 << 29), mea.MEA_EINVAL),
    # (256 + 4096) * 64 * (128 + 2) * 4 bytes of partials: more than the scratch
    (dict(B=4096, Hq=64, Hkv=8, S=8), mea.MEA_ESCRATCH),
])
def test_decode_noalloc_rejects(kw, status):
    """Refused on the host before any HIP call, including a step larger than
    the static scratch (MEA_DECODE_NOALLOC_SCRATCH_BYTES)."""
    assert _dec_noalloc(**kw) == status
    assert "scratch" in mea.strerror(mea.MEA_ESCRATCH)


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=2, M=64, N=80, Hq=4,
             Hkv=2, D=64, scale=0.125, kind=mea.MEA_MASK_CAUSAL, sq=None, sk=None, sl=None, dtype=mea.MEA_BF16,
             ws=ctypes.c_void_p(0x100000), wsb=1 << 20, stream=None)
    a.update(kw)
    return mea.lib().mea_bwd(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                             a["B"], a["M"], a["N"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["kind"], a["sq"],
                             a["sk"], a["sl"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), mea.MEA_EINVAL),
    (dict(out=None), mea.MEA_EINVAL),
    (dict(do=None), mea.MEA_EINVAL),
    (dict(dk=None), mea.MEA_EINVAL),
    (dict(N=0), mea.MEA_EINVAL),
    (dict(Hq=3), mea.MEA_EINVAL),
    (dict(scale=float("nan")), mea.MEA_EINVAL),
    (dict(kind=16), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_BIAS_ALIBI), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_MASK_BLOCKDIAG), mea.MEA_EINVAL),
    (dict(kind=mea.MEA_MASK_BLOCKDIAG, sq=FAKE), mea.MEA_EINVAL),   # M != N needs seqstart_k
    (dict(D=256), mea.MEA_EUNSUPPORTED),
    (dict(ws=None), mea.MEA_EWORKSPACE),
    (dict(wsb=1024), mea.MEA_EWORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100040)), mea.MEA_EWORKSPACE),
])
def test_bwd_rejects(kw, status):
    assert _bwd(**kw) == status


def test_bwd_workspace_bytes():
    one = ((2 * 64 * 4 * 4 + 255) // 256) * 256
    assert mea.bwd_workspace_bytes(2, 64, 4, mea.MEA_MASK_CAUSAL) == 2 * one
    packed = ((64 * 4 * 4 + 255) // 256) * 256          # packed: one physical batch row
    assert mea.bwd_workspace_bytes(2, 64, 4, mea.MEA_MASK_BLOCKDIAG) == 2 * packed
    assert mea.bwd_workspace_bytes(0, 64, 4, 0) == 0


def test_blocksparse_rejects():
    lib = mea.lib()
    args = [FAKE, FAKE, FAKE, FAKE, 2, 128, 128, 4, 2, 64, 0.125, 0, FAKE, None, mea.MEA_BF16, None, None]
    assert mea.block_sparse_block() == 64
    a = list(args); a[12] = None                       # no mask
    assert lib.mea_fwd_blocksparse(*a) == mea.MEA_EINVAL
    a = list(args); a[11] = mea.MEA_MASK_BLOCKDIAG     # packed batches have no block-sparse form
    assert lib.mea_fwd_blocksparse(*a) == mea.MEA_EINVAL
    a = list(args); a[11] = mea.MEA_BIAS_ALIBI         # ALiBi without slopes
    assert lib.mea_fwd_blocksparse(*a) == mea.MEA_EINVAL
    a = list(args); a[9] = 80
    assert lib.mea_fwd_blocksparse(*a) == mea.MEA_EUNSUPPORTED


def test_product_package_does_not_reach_the_oracle():
    """The product package neither imports nor names the oracle."""
    pkg = os.path.join(ROOT, "memory_efficient_exact_tiled_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_single_hip_runtime_in_process():
    """The library binds to the HIP runtime torch already loaded (one copy of
    libamdhip64 in the process, whatever the import order)."""
    import subprocess
    import sys
    code = ("import memory_efficient_exact_tiled_amd, torch;"
            "m=open('/proc/self/maps').read();"
            "print(len(set(l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l)))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_kvcache_entry_points_reject():
    lib = mea.lib()
    # mea_fwd_kvcache: missing ctx_lens, block-diagonal flag, bad D
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 2, 128, 1024, 0.1, 1, None, 1, None, None]
    a = list(args); a[3] = None
    assert lib.mea_fwd_kvcache(*a) == mea.MEA_EINVAL
    a = list(args); a[12] = mea.MEA_MASK_BLOCKDIAG
    assert lib.mea_fwd_kvcache(*a) == mea.MEA_EINVAL
    a = list(args); a[3] = None; a[9] = 96
    assert lib.mea_fwd_kvcache(*a) == mea.MEA_EINVAL
    a = list(args); a[9] = 96
    assert lib.mea_fwd_kvcache(*a) == mea.MEA_EUNSUPPORTED
    # mea_kv_append: negative T, null cache, bad dtype
    ap = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1024, 2, 128, 4, 1, None]
    a = list(ap); a[9] = -1
    assert lib.mea_kv_append(*a) == mea.MEA_EINVAL
    a = list(ap); a[0] = None
    assert lib.mea_kv_append(*a) == mea.MEA_EINVAL
    a = list(ap); a[10] = 9
    assert lib.mea_kv_append(*a) == mea.MEA_EUNSUPPORTED
