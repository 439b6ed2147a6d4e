"""Parity of the HIP forward kernel (through the C ABI) with the fp64 oracle, on the GPU."""
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


def _run(mea, c, dt, causal=False, slopes=None, st=None, scale=None, with_lse=False):
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    D = c["q"].shape[-1]
    scale = float(np.float32(1.0 / np.sqrt(D))) if scale is None else scale
    lse = None
    if with_lse:
        B, M, Hq, _ = c["q"].shape
        lse = torch.full((B, Hq, M) if st is None else (Hq, M), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=causal, scale=scale,
                  alibi_slopes=None if slopes is None else f32(slopes),
                  seqstart_q=None if st is None else i32(st), lse=lse)
    torch.cuda.synchronize()
    return out, lse, scale


DENSE = [
    # name, seed, B, M, N, Hq, Hkv, D, dtype, causal
    ("cfg1_b1_m128_h2_d64_fp16", 0, 1, 128, 128, 2, 2, 64, "fp16", False),
    ("cfg2_b2_m256_h8_d64_fp16_causal", 1, 2, 256, 256, 8, 8, 64, "fp16", True),
    ("cfg3_m512_noncausal", 2, 4, 512, 512, 16, 16, 64, "bf16", False),
    ("cfg3_m512_causal", 2, 4, 512, 512, 16, 16, 64, "bf16", True),
    ("cfg3_m1024_noncausal", 3, 4, 1024, 1024, 16, 16, 64, "bf16", False),
    ("cfg3_m1024_causal", 3, 4, 1024, 1024, 16, 16, 64, "bf16", True),
    ("ragged_m300_n177_d128_bf16", 4, 2, 300, 177, 4, 2, 128, "bf16", False),
    ("ragged_causal_m333_d128_fp16_gqa", 5, 1, 333, 333, 8, 2, 128, "fp16", True),
    ("chunked_prefill_m70_n500_causal", 6, 2, 70, 500, 4, 4, 64, "bf16", True),
    ("more_queries_than_keys_causal", 7, 1, 200, 90, 2, 1, 128, "bf16", True),
    ("tiny_m1_n1", 8, 3, 1, 1, 2, 2, 64, "fp16", False),
    ("single_query_n777", 9, 2, 1, 777, 4, 1, 128, "bf16", True),
    ("gqa_tutorial_b2_m256_hq8_hkv2_d64_fp16", 10, 2, 256, 256, 8, 2, 64, "fp16", False),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: c[0])
def test_dense_parity(mea, case):
    name, seed, B, M, N, Hq, Hkv, D, dt, causal = case
    say(f"case {name}")
    c = inp.dense_case(seed, B, M, N, Hq, Hkv, D, dt)
    out, lse, scale = _run(mea, c, dt, causal=causal, with_lse=True)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal)
    err = report(name, host_f64(out), want, TOL[dt])
    assert err <= TOL[dt]
    got_lse = lse.cpu().numpy()
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(got_lse), fin), "lse -inf pattern"
    assert np.max(np.abs(got_lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dt], "lse"


@pytest.mark.parametrize("M", [2048, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_seqlen_sweep_sampled(mea, M, causal):
    """Sequence-length sweep at full size (B=4, H=16, D=64, bf16): the oracle
    checks a sample of rows of two batch rows, all heads."""
    name = f"cfg3_m{M}_{'causal' if causal else 'noncausal'}"
    say(f"case {name}")
    c = inp.dense_case(11 + M, 4, M, M, 16, 16, 64, "bf16")
    out, _, scale = _run(mea, c, "bf16", causal=causal)
    got = host_f64(out)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 255, 256, M - 1], rng.integers(0, M, 40)]))
    for b in (0, 3):
        want, _ = orc.fwd_rows(c["q"], c["k"], c["v"], "bf16", scale, b, rows, causal=causal)
        assert report(f"{name} b{b}", got[b, rows], want, TOL["bf16"]) <= TOL["bf16"]


@pytest.mark.parametrize("dt,alibi", [("bf16", False), ("fp16", True)])
def test_dense_wide_tiles_ragged(mea, dt, alibi):
    """Dense D=64 without mask at a size that takes the 256-row work-groups
    (B*Hq*ceil(M/256) >= 512), with M and N off the tile grid and M != N;
    sampled rows at the tile edges against the oracle."""
    B, M, N, Hq, Hkv = 8, 1000, 1100, 16, 4
    name = f"wide_{dt}{'_alibi' if alibi else ''}"
    say(f"case {name}")
    c = inp.dense_case(77, B, M, N, Hq, Hkv, 64, dt)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    out, _, scale = _run(mea, c, dt, slopes=slopes)
    got = host_f64(out)
    rows = np.array([0, 1, 31, 32, 63, 64, 255, 256, 511, 512, 767, 768, 998, 999])
    for b in (0, 7):
        want, _ = orc.fwd_rows(c["q"], c["k"], c["v"], dt, scale, b, rows, alibi_slopes=slopes)
        assert report(f"{name} b{b}", got[b, rows], want, TOL[dt]) <= TOL[dt]


@pytest.mark.parametrize("N", [1, 64, 65, 128, 129, 192, 193])
@pytest.mark.parametrize("dt,alibi", [("bf16", False), ("fp16", True)])
def test_dense_wide_tiles_few_key_blocks(mea, N, dt, alibi):
    """The 256-row work-groups (B*Hq*ceil(M/256) >= 512) walk their key blocks
    in pairs with a single-block tail; 1 to 4 blocks, full and ragged, cover
    an empty pair loop, one pair, a pair plus tail and two pairs."""
    B, M, Hq, Hkv = 8, 1000, 16, 4
    name = f"wide_few_blocks_n{N}_{dt}{'_alibi' if alibi else ''}"
    say(f"case {name}")
    c = inp.dense_case(78, B, M, N, Hq, Hkv, 64, dt)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    out, _, scale = _run(mea, c, dt, slopes=slopes)
    got = host_f64(out)
    rows = np.array([0, 63, 64, 255, 256, 600, 999])
    for b in (0, 5):
        want, _ = orc.fwd_rows(c["q"], c["k"], c["v"], dt, scale, b, rows, alibi_slopes=slopes)
        assert report(f"{name} b{b}", got[b, rows], want, TOL[dt]) <= TOL[dt]


def test_varlen_gqa_alibi_full_config(mea):
    """8 packed segments, lengths uniform in [64, 2048] (seeded), Hq=32, Hkv=8,
    D=128, bf16, block-diagonal causal + ALiBi: sampled rows of every segment."""
    lengths = inp.segment_lengths(4, 8, 64, 2048)
    say(f"case cfg4 lengths={lengths.tolist()}")
    c = inp.varlen_case(4, lengths, 32, 8, 128, "bf16")
    slopes = inp.alibi_slopes(32)
    out, _, scale = _run(mea, c, "bf16", causal=True, slopes=slopes, st=c["seqstart"])
    got = host_f64(out)
    st = c["seqstart"]
    rng = np.random.default_rng(5)
    for s, L in enumerate(lengths):
        rows = np.unique(np.concatenate([[0, 1, L - 1], rng.integers(0, L, 12)]))
        want, _ = orc.fwd_rows(c["q"], c["k"], c["v"], "bf16", scale, 0, rows, causal=True,
                               seqstart_q=st, segment=s, alibi_slopes=slopes)
        assert report(f"cfg4 seg{s} L={L}", got[0, st[s] + rows], want, TOL["bf16"]) <= TOL["bf16"]


def test_varlen_thousands_of_short_segments(mea):
    """4096 packed segments of 1 to 64 tokens (some empty), causal + ALiBi with
    GQA: every work-group finds its segment by a binary search over the
    segments' tile ranges. Whole output and lse against the oracle; the
    launch is timed on its own."""
    lengths = [int(x) for x in np.random.default_rng(11).integers(0, 65, 4096)]
    dt, Hq, Hkv, D = "bf16", 8, 2, 64
    c = inp.varlen_case(12, lengths, Hq, Hkv, D, dt)
    T = int(c["seqstart"][-1])
    say(f"case packed 4096 short segments, T={T}")
    slopes = inp.alibi_slopes(Hq)
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    st, sl = i32(c["seqstart"]), f32(slopes)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    lse = torch.full((Hq, T), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=True, scale=scale, seqstart_q=st, alibi_slopes=sl, lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=True, seqstart_q=c["seqstart"],
                         alibi_slopes=slopes)
    assert report("4096 short segments", host_f64(out), want, TOL[dt]) <= TOL[dt]
    fin = np.isfinite(wlse[0])
    got_lse = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.max(np.abs(got_lse[fin] - wlse[0][fin])) <= LSE_TOL[dt]
    for _ in range(3):
        mea.fwd(q, k, v, causal=True, scale=scale, seqstart_q=st, alibi_slopes=sl, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        mea.fwd(q, k, v, causal=True, scale=scale, seqstart_q=st, alibi_slopes=sl, out=out)
    e1.record()
    torch.cuda.synchronize()
    say(f"4096 short segments (T={T}, Hq=8, D=64, causal ALiBi): {e0.elapsed_time(e1) / 20 * 1e3:.1f} us per launch")


VARLEN = [
    # name, lengths, Hq, Hkv, D, dtype, causal, alibi
    ("ragged_segments_causal_alibi_d128", [1, 63, 64, 65, 130, 7, 256, 257], 8, 2, 128, "bf16", True, True),
    ("ragged_segments_noncausal_d64_fp16", [5, 300, 1, 129], 4, 4, 64, "fp16", False, False),
    ("ragged_segments_noncausal_alibi", [40, 100, 3], 4, 1, 64, "bf16", False, True),
    ("one_segment", [513], 2, 1, 128, "fp16", True, False),
    # packed batches: work-groups find their segment by a binary search over
    # the segments' tile ranges (64 and 70 segments, some empty, cover odd and
    # even search depths), and the causal launch order pins each KV head to
    # one XCD only when the KV heads split evenly over the 8 XCDs (not for Hq=6)
    ("segments_64_causal_hq8", [0, 3] + [int(x) for x in np.random.default_rng(5).integers(1, 150, 61)] + [0],
     8, 2, 64, "bf16", True, False),
    ("segments_70_causal_alibi", [int(x) for x in np.random.default_rng(6).integers(0, 120, 70)],
     8, 4, 128, "bf16", True, True),
    ("segments_hq6_noncausal", [77, 0, 200, 31, 129], 6, 2, 64, "fp16", False, False),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: c[0])
def test_varlen_parity_full(mea, case):
    name, lengths, Hq, Hkv, D, dt, causal, alibi = case
    say(f"case {name}")
    c = inp.varlen_case(21, lengths, Hq, Hkv, D, dt)
    slopes = inp.alibi_slopes(Hq) if alibi else None
    out, lse, scale = _run(mea, c, dt, causal=causal, slopes=slopes, st=c["seqstart"], with_lse=True)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, seqstart_q=c["seqstart"],
                         alibi_slopes=slopes)
    assert report(name, host_f64(out), want, TOL[dt]) <= TOL[dt]
    assert np.max(np.abs(lse.cpu().numpy() - wlse[0])) <= LSE_TOL[dt]


def test_varlen_equals_per_segment_bitwise(mea):
    """Block-diagonal output equals per-segment calls bit for bit (tiles start
    at segment starts, so the arithmetic is the same)."""
    lengths = [70, 1, 300, 129]
    c = inp.varlen_case(31, lengths, 8, 2, 128, "bf16")
    slopes = inp.alibi_slopes(8)
    out, _, _ = _run(mea, c, "bf16", causal=True, slopes=slopes, st=c["seqstart"])
    got = host_bits(out)
    st = c["seqstart"]
    for s in range(len(lengths)):
        a, b = st[s], st[s + 1]
        seg = {key: c[key][:, a:b] for key in ("q", "k", "v")}
        o2, _, _ = _run(mea, seg, "bf16", causal=True, slopes=slopes)
        assert np.array_equal(host_bits(o2), got[:, a:b]), f"segment {s}"


def test_gqa_equals_repeated_kv_bitwise(mea):
    c = inp.dense_case(32, 2, 200, 200, 8, 2, 64, "fp16")
    rep = dict(c, k=np.repeat(c["k"], 4, axis=2), v=np.repeat(c["v"], 4, axis=2))
    for causal in (False, True):
        o1, _, _ = _run(mea, c, "fp16", causal=causal)
        o2, _, _ = _run(mea, rep, "fp16", causal=causal)
        assert np.array_equal(host_bits(o1), host_bits(o2)), causal


@pytest.mark.parametrize("D,dt,alibi,Hq,Hkv,packed", [
    (64, "bf16", False, 8, 2, False), (128, "fp16", True, 8, 2, False), (64, "fp16", True, 16, 2, True),
    (128, "bf16", True, 32, 8, True), (128, "bf16", False, 4, 1, False)])
def test_grouped_query_workgroups_bitwise(mea, D, dt, alibi, Hq, Hkv, packed):
    """Causal launches whose KV heads serve a multiple of 4 query heads run
    32-row work-groups of 4 query heads (one per wave); with K/V repeated per
    query head they run the per-head 128-row work-groups. Every row goes
    through the same arithmetic either way: output and lse bitwise equal, and
    within the oracle's bar. Ragged sizes, M < N (bottom-right), packed
    segments of 0..300 tokens."""
    name = f"gq D={D} {dt} alibi={alibi} Hq={Hq} Hkv={Hkv} packed={packed}"
    say(f"case {name}")
    slopes = inp.alibi_slopes(Hq) if alibi else None
    if packed:
        c = inp.varlen_case(90, [300, 0, 37, 129, 1, 64, 255], Hq, Hkv, D, dt)
        st = c["seqstart"]
    else:
        c = inp.dense_case(91, 2, 301, 333, Hq, Hkv, D, dt)
        st = None
    rep = dict(c, k=np.repeat(c["k"], Hq // Hkv, axis=2), v=np.repeat(c["v"], Hq // Hkv, axis=2))
    o1, l1, scale = _run(mea, c, dt, causal=True, slopes=slopes, st=st, with_lse=True)
    o2, l2, _ = _run(mea, rep, dt, causal=True, slopes=slopes, st=st, with_lse=True)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert torch.equal(l1, l2)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=True, seqstart_q=st, alibi_slopes=slopes)
    assert report(name, host_f64(o1), want, TOL[dt]) <= TOL[dt]
    gl = l1.cpu().numpy()
    wl = wlse[0] if packed else wlse
    fin = np.isfinite(wl)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.max(np.abs(gl[fin] - wl[fin]), initial=0.0) <= LSE_TOL[dt]


def test_first_causal_row_is_v0_bitwise(mea):
    c = inp.dense_case(33, 2, 130, 130, 4, 2, 128, "bf16")
    out, _, _ = _run(mea, c, "bf16", causal=True, slopes=inp.alibi_slopes(4))
    got = host_bits(out)
    for h in range(4):
        assert np.array_equal(got[:, 0, h], c["v"][:, 0, h // 2])


def test_rows_sum_to_one(mea):
    """V = 1: every output is 1 up to the rounding of P to bf16 before P.V."""
    c = inp.dense_case(34, 2, 300, 300, 4, 4, 64, "bf16")
    c["v"] = inp.round_bits(np.ones(c["v"].shape, np.float32), "bf16")
    for causal in (False, True):
        out, _, _ = _run(mea, c, "bf16", causal=causal, slopes=inp.alibi_slopes(4))
        assert report(f"ones causal={causal}", host_f64(out), np.ones(out.shape), TOL["bf16"]) <= TOL["bf16"]


def test_deterministic(mea):
    c = inp.dense_case(35, 2, 1024, 1024, 8, 8, 128, "bf16")
    o1, _, _ = _run(mea, c, "bf16", causal=True)
    for _ in range(3):
        o2, _, _ = _run(mea, c, "bf16", causal=True)
        assert torch.equal(o1, o2)


def test_no_nan_from_neighbours(mea):
    """Packed rows beyond the last segment end are never read: NaN there
    (inside the buffer) does not reach the output."""
    lengths = [100, 60]
    c = inp.varlen_case(36, lengths, 2, 2, 64, "bf16")
    T = int(c["seqstart"][-1])
    pad = 50
    for key in ("q", "k", "v"):
        x = np.full((1, T + pad) + c[key].shape[2:], inp.POISON["bf16"], np.uint16)
        x[:, :T] = c[key]
        c[key] = x
    st = np.append(c["seqstart"], T + pad).astype(np.int32)   # a third segment of NaN rows
    q, k, v = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16")
    out = mea.fwd(q, k, v, causal=True, seqstart_q=i32(st))
    torch.cuda.synchronize()
    got = host_f64(out)[0, :T]
    assert np.all(np.isfinite(got))
    want, _ = orc.fwd(c["q"][:, :T], c["k"][:, :T], c["v"][:, :T], "bf16", 0.125, causal=True,
                      seqstart_q=st[:3])
    assert report("nan neighbours", got, want[0], TOL["bf16"]) <= TOL["bf16"]


CROSS = [
    # name, q lengths, k lengths, Hq, Hkv, D, dtype, causal, alibi
    ("cross_causal_alibi_d128", [130, 64, 0, 300, 7, 200], [200, 64, 50, 129, 7, 0], 8, 2, 128, "bf16", True, True),
    ("cross_noncausal_d64_fp16", [1, 257, 90], [333, 5, 0], 4, 4, 64, "fp16", False, False),
]


@pytest.mark.parametrize("case", CROSS, ids=lambda c: c[0])
def test_varlen_cross_segments(mea, case):
    """Packed cross-attention: query segment s attends to key segment s of a
    different length (seqstart_k != seqstart_q), bottom-right causal per
    segment, empty query or key segments."""
    name, ql, kl, Hq, Hkv, D, dt, causal, alibi = case
    say(f"case {name}")
    c = inp.varlen_cross_case(40, ql, kl, Hq, Hkv, D, dt)
    q, k, v = dev(c["q"], dt), dev(c["k"], dt), dev(c["v"], dt)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    slopes = inp.alibi_slopes(Hq) if alibi else None
    lse = torch.full((Hq, int(c["seqstart_q"][-1])), 7.0, dtype=torch.float32, device="cuda")
    out = mea.fwd(q, k, v, causal=causal, scale=scale, seqstart_q=i32(c["seqstart_q"]),
                  seqstart_k=i32(c["seqstart_k"]), alibi_slopes=None if slopes is None else f32(slopes), lse=lse)
    torch.cuda.synchronize()
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=causal, seqstart_q=c["seqstart_q"],
                         seqstart_k=c["seqstart_k"], alibi_slopes=slopes)
    assert report(name, host_f64(out), want, TOL[dt]) <= TOL[dt]
    got_lse = lse.cpu().numpy()
    fin = np.isfinite(wlse[0])
    assert np.array_equal(np.isfinite(got_lse), fin), "lse -inf pattern"
    assert np.max(np.abs(got_lse[fin] - wlse[0][fin]), initial=0.0) <= LSE_TOL[dt]


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_causal_alibi_extreme_slopes(mea, dt):
    """Causal ALiBi with slope / scale from 0.4 to 1e7: the bias the score
    MFMA adds must stay finite and exact enough in either 16-bit type."""
    say(f"case causal alibi extreme slopes {dt}")
    c = inp.dense_case(77, 2, 200, 200, 4, 2, 64, dt)
    slopes = np.float32([2.0 ** -8, 1.0, 300.0, 1.0e5])
    scale = 0.01
    out, lse, _ = _run(mea, c, dt, causal=True, slopes=slopes, scale=scale, with_lse=True)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, scale, causal=True, alibi_slopes=slopes)
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    assert report(f"extreme slopes {dt}", got, want, TOL[dt]) <= TOL[dt]
    assert np.max(np.abs(lse.cpu().numpy() - wlse)) <= LSE_TOL[dt] * max(1.0, float(np.max(np.abs(wlse))) * 2 ** -11)


def _bits_to_f32(bits, dt):
    b = np.ascontiguousarray(bits)
    if dt == "fp16":
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _lazy_max_outcomes(s):
    """The forward's per-block choice for D=64 without ALiBi, replayed in fp64.

    s: scores in log2 units [heads, rows, keys] (masked keys -inf). Rows go in
    groups of 32 (one wave's query block), keys in blocks of 64, each row's
    keys split into two halves of 32 (the two lanes holding a row). Per
    group and block the kernel takes P with its running max as the offset
    (outcome "fast") when every row of the group has a running max and every
    half-row sum of P stays below 2^7; otherwise it runs the full step
    ("first" while some row has no running max yet, else "full"), which
    raises the running maxima to the block maxima when any row's block max
    exceeds its running max by more than 2^8. Returns the outcome counts."""
    H, M, N = s.shape
    counts = {"first": 0, "fast": 0, "full": 0}
    for g0 in range(0, M, 32):
        blk = s[:, g0:g0 + 32]
        m = np.full(blk.shape[:2], -np.inf)
        for j in range((N + 63) // 64):
            x = blk[..., j * 64:(j + 1) * 64]
            for hd in range(H):
                mh = m[hd]
                if not np.all(np.isfinite(mh)):
                    kind = "first"
                else:
                    p = np.exp2(x[hd] - mh[:, None])
                    halves = [p[:, :32].sum(-1), p[:, 32:].sum(-1)]
                    kind = "fast" if all(np.all(h < 128.0) for h in halves) else "full"
                counts[kind] += 1
                if kind != "fast":
                    bm = x[hd].max(-1)
                    if np.any(bm > mh + 8.0):
                        m[hd] = np.maximum(mh, bm)
    return counts


@pytest.mark.parametrize("dt,mode", [("bf16", "rising"), ("fp16", "rising"), ("bf16", "wide")])
def test_causal_running_max_jumps(mea, dt, mode):
    """Causal D=64 rows whose running max often jumps by more than 2^7 in P
    from one key block to the next ("rising": key norms grow along the
    sequence; "wide": scale 1, scores spread over tens of log2 units), next
    to blocks where it does not. The forward takes P with the old running
    max as the offset only when no half-row sum of P in a wave's 32 rows
    reaches 2^7; both outcomes occur in these inputs, per wave and block
    (replayed below in fp64 with the kernel's own rule), and must agree with
    the oracle.""" 
    say(f"case causal running max jumps {dt} {mode}")
    B, M, H, D = 2, 1000, 4, 64
    c = inp.dense_case(91, B, M, M, H, H, D, dt)
    scale = None
    if mode == "rising":
        grow = np.float32(1.0) + np.float32(8.0) * np.arange(M, dtype=np.float32) / np.float32(M)
        c["k"] = inp.round_bits(_bits_to_f32(c["k"], dt) * grow[None, :, None, None], dt)
    else:
        scale = 1.0
    sc = float(np.float32(1.0 / np.sqrt(D))) if scale is None else scale
    # fp64 scores in log2 units; per (row, key block) the block max against
    # the max over the earlier allowed keys.
    q, k = _bits_to_f32(c["q"], dt).astype(np.float64), _bits_to_f32(c["k"], dt).astype(np.float64)
    s = np.einsum("bmhd,bnhd->bhmn", q, k) * sc / np.log(2.0)
    s = np.where(np.tril(np.ones((M, M), dtype=bool)), s, -np.inf)
    nkb = (M + 63) // 64
    bmax = np.stack([s[..., j * 64:(j + 1) * 64].max(-1) for j in range(nkb)], -1)
    run = np.maximum.accumulate(bmax, -1)
    jump = bmax[..., 1:] - run[..., :-1]
    live = np.isfinite(bmax[..., 1:]) & np.isfinite(run[..., :-1])
    assert np.any(live & (jump > 7.5)) and np.any(live & (jump < 0.0))
    counts = _lazy_max_outcomes(s[0])
    say(f"lazy max outcomes per (wave, block), batch row 0: {counts}")
    assert counts["fast"] > 0 and counts["full"] > 0
    out, lse, sc = _run(mea, c, dt, causal=True, scale=scale, with_lse=True)
    want, wlse = orc.fwd(c["q"], c["k"], c["v"], dt, sc, causal=True)
    assert report(f"running max jumps {dt} {mode}", host_f64(out), want, TOL[dt]) <= TOL[dt]
    assert np.max(np.abs(lse.cpu().numpy() - wlse)) <= LSE_TOL[dt] * max(1.0, float(np.max(np.abs(wlse))) * 2 ** -11)


@pytest.mark.parametrize("dt,mode", [("bf16", "rising"), ("fp16", "wide")])
def test_dense_wide_running_max_jumps(mea, dt, mode):
    """The same jumps of the running max in the dense D=64 launch with
    256-row work-groups (B*Hq*ceil(M/256) >= 512): sampled rows against the
    oracle, after checking in fp64 that jumps above 2^7 and blocks below the
    running max both occur."""
    say(f"case dense wide running max jumps {dt} {mode}")
    B, M, N, Hq, Hkv, D = 8, 1000, 1100, 16, 4, 64
    c = inp.dense_case(92, B, M, N, Hq, Hkv, D, dt)
    scale = None
    if mode == "rising":
        grow = np.float32(1.0) + np.float32(8.0) * np.arange(N, dtype=np.float32) / np.float32(N)
        c["k"] = inp.round_bits(_bits_to_f32(c["k"], dt) * grow[None, :, None, None], dt)
    else:
        scale = 1.0
    sc = float(np.float32(1.0 / np.sqrt(D))) if scale is None else scale
    q = _bits_to_f32(c["q"][0], dt).astype(np.float64)
    k = np.repeat(_bits_to_f32(c["k"][0], dt).astype(np.float64), Hq // Hkv, axis=1)
    s = np.einsum("mhd,nhd->hmn", q, k) * sc / np.log(2.0)
    bmax = np.stack([s[..., j * 64:(j + 1) * 64].max(-1) for j in range((N + 63) // 64)], -1)
    jump = bmax[..., 1:] - np.maximum.accumulate(bmax, -1)[..., :-1]
    assert np.any(jump > 7.5) and np.any(jump < 0.0)
    counts = _lazy_max_outcomes(s)
    say(f"lazy max outcomes per (wave, block), batch row 0: {counts}")
    assert counts["fast"] > 0 and counts["full"] > 0
    out, lse, sc = _run(mea, c, dt, scale=scale, with_lse=True)
    got = host_f64(out)
    got_lse = lse.cpu().numpy()
    rows = np.array([0, 1, 31, 32, 63, 64, 255, 256, 511, 512, 767, 768, 998, 999])
    for b in (0, 7):
        want, wlse = orc.fwd_rows(c["q"], c["k"], c["v"], dt, sc, b, rows)
        assert report(f"dense jumps {dt} {mode} b{b}", got[b, rows], want, TOL[dt]) <= TOL[dt]
        assert np.max(np.abs(got_lse[b][:, rows] - wlse)) <= LSE_TOL[dt], f"lse b{b}"
