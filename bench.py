#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM:

  1. forward, B=4, M=N=4096, H=16, D=64, bf16, no mask   (the headline)
  2. forward, same shapes, causal mask
  3. forward, 8 packed segments (lengths uniform in [64, 2048]), Hq=32,
     Hkv=8, D=128, bf16, block-diagonal causal mask + ALiBi
  4. decode step, B=32, contexts uniform in [1024, 32768], Hq=32, Hkv=8,
     D=128, bf16 KV cache of 32768 slots per sequence
  5. block-sparse forward, B=1, M=N=16384, H=16, D=64, bf16, causal, 64x64
     blocks: a sliding window of 3 blocks on each side plus one global key
     block (4*D flops per allowed query-key pair)
  6. backward (dq, dk, dv) of items 1 and 2, from their stored output and
     lse and a seeded upstream gradient (10*D algorithmic flops per allowed
     query-key pair: S recomputed, dP, dV, dK, dQ)

Prints ONE JSON line on stdout. ``value`` is the headline forward throughput
(algorithmic TFLOP/s of item 1: 4*B*H*M*N*D flops over its average launch
time, measured with HIP events on the stream the kernel runs on); the other
items are reported beside it, decode as algorithmic HBM GB/s (K and V bytes
of every sequence's context plus q and out). Each item's ``per_item`` entry
also carries its algorithmic bytes (inputs read once, outputs written once),
its arithmetic intensity and the fraction of its own roofline: the longer of
the MFMA time and the HBM time at peak, over the measured time (the
block-sparse item, at about 143 flop/B, sits below MI355X's ridge point of
315 flop/B and is HBM-bound). Progress goes to stderr.

The roofline objects of items 1 and 4 also carry ``alone``: the same kernel
timed over ALONE consecutive launches on its own (its sustained throughput
outside the mixed step). Runs need tens of milliseconds of warmup before the
GPU clock settles; --warmup steps provide it.

``cpu_baseline`` times the fp64 oracle (test infrastructure) on the host's
cores over a bounded sample of item 1 (rows of the first batch row, all
heads, until about --cpu-seconds have passed); ``cpu_baseline_decode`` does
the same for item 4 (whole sequences).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ALONE = 100                   # back-to-back launches of the headline items timed on their own


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_code_hash(text):
    """sha256[:16] of a kernel source with comments and blank lines removed: the
    fingerprint of the code the counters were taken on (a comment edit keeps it)."""
    import hashlib
    import re
    t = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    t = re.sub(r"//[^\n]*", "", t)
    lines = [ln.rstrip() for ln in t.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


# Sources whose code decides what the counted kernels do (kernels, launch
# shapes, host-side kernel and tile choices), and the compiler flags: the
# stored traffic counts only while all of them are unchanged.
TRAFFIC_SOURCES = ("api.hip", "fwd.hip", "bwd.hip", "decode.hip", "kvcache.hip", "common.hpp", "launch.hpp")


def code_fingerprints(root=None):
    """{source: kernel_code_hash} over TRAFFIC_SOURCES plus the build flags."""
    import hashlib
    root = ROOT if root is None else root
    csrc = os.path.join(root, "memory_efficient_exact_tiled_amd", "csrc")
    out = {name: kernel_code_hash(open(os.path.join(csrc, name)).read()) for name in TRAFFIC_SOURCES}
    build_py = open(os.path.join(root, "memory_efficient_exact_tiled_amd", "build.py")).read()
    flags = build_py[build_py.index("FLAGS = ["):]
    flags = flags[:flags.index("]") + 1]
    out["build.py FLAGS"] = hashlib.sha256(flags.encode()).hexdigest()[:16]
    return out


def measured_traffic():
    """HBM bytes per launch from profiles/hbm_traffic.json (rocprofv3 FETCH_SIZE
    and WRITE_SIZE, calibrated against a plain 1 GiB copy), or None for every
    kernel once a source in TRAFFIC_SOURCES or the build flags differ from the
    ones the counters were taken with."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("code_sha256_16") != code_fingerprints():
        return None
    out = {}
    for k, v in t["kernels"].items():
        out[k] = v["fetch_bytes"] + v["write_bytes"]
    return out


def traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_path):
    """Writes profiles/hbm_traffic.json from four rocprofv3 --pmc counter
    collections (FETCH_SIZE and WRITE_SIZE of a bench run, then of
    --copy-calibration): per kernel, the mean KiB per dispatch scaled by what
    the same counter reads for the 1 GiB copy, with the code fingerprints."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    def copy_kib(path, counter):
        vals = [v for k, (v, _) in per_kernel(path, counter).items() if "copyBuffer" in k]
        return max(vals)

    gib_kib = float(1 << 20)
    ff = gib_kib / copy_kib(copy_fetch_csv, "FETCH_SIZE")
    wf = gib_kib / copy_kib(copy_write_csv, "WRITE_SIZE")
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if "mea" not in k:
            continue
        kernels[k] = {"fetch_bytes": fetch[k][0] * ff * 1024, "write_bytes": write[k][0] * wf * 1024,
                      "dispatches": fetch[k][1]}
    res = {"code_sha256_16": code_fingerprints(), "fetch_factor": ff, "write_factor": wf, "kernels": kernels}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    return res


def traffic_for(traffic, *needles):
    if traffic is None:
        return None
    total = 0.0
    for nd in needles:
        hits = [v for k, v in traffic.items() if nd in k]
        if len(hits) != 1:
            return None
        total += hits[0]
    return round(total)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def build_inputs(torch, inp, with_decode=True):
    t0 = time.time()
    x = {}
    c = inp.dense_case(3, 4, 4096, 4096, 16, 16, 64, "bf16")
    x["dense"] = {k: to_dev(c[k], torch) for k in ("q", "k", "v")}
    x["dense_host"] = c
    lengths = inp.segment_lengths(4, 8, 64, 2048)
    v = inp.varlen_case(4, lengths, 32, 8, 128, "bf16")
    x["varlen"] = {k: to_dev(v[k], torch) for k in ("q", "k", "v")}
    x["varlen"]["seqstart"] = torch.from_numpy(v["seqstart"]).cuda()
    x["varlen"]["slopes"] = torch.from_numpy(inp.alibi_slopes(32)).cuda()
    x["lengths"] = lengths
    log(f"[bench] forward inputs ready ({time.time() - t0:.1f}s); packed lengths {lengths.tolist()}")

    B, S, Hq, Hkv, D = 32, 32768, 32, 8, 128
    ctx = inp.context_lengths(5, B, 1024, 32768)
    if not with_decode:
        # Decode is not among the items run: its 4.3 GB cache is not built.
        x["decode"] = {"ctx_host": ctx}
        return x
    kc = torch.empty((B, S, Hkv, D), dtype=torch.int16, device="cuda")
    vc = torch.empty_like(kc)
    poison = int(np.uint16(inp.POISON["bf16"]).view(np.int16))
    kc.fill_(poison)
    vc.fill_(poison)

    def rows(b):
        return b, inp.decode_cache_rows(5, b, int(ctx[b]), Hkv, D, "bf16")

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        for b, (kb, vb) in ex.map(rows, range(B)):
            kc[b, :ctx[b]] = torch.from_numpy(kb.view(np.int16)).cuda()
            vc[b, :ctx[b]] = torch.from_numpy(vb.view(np.int16)).cuda()
    x["decode"] = {
        "q": to_dev(inp.normal_bits(5, (B, Hq, D), "bf16", 0), torch),
        "kc": kc.view(torch.bfloat16), "vc": vc.view(torch.bfloat16),
        "ctx": torch.from_numpy(ctx).cuda(), "ctx_host": ctx,
    }
    log(f"[bench] decode cache ready ({time.time() - t0:.1f}s); sum(ctx)={int(ctx.sum())}")
    return x


def host_description():
    """The host the oracle runs on: logical CPUs, those this process may use,
    and the CPU model (from /proc/cpuinfo)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": usable, "logical_cpus": os.cpu_count(), "cpu_model": model}


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def _fwd_sample(c, seconds, max_rows):
    """fp64 oracle over blocks of 512 query rows (all 16 heads, all 4096 keys),
    batch row by batch row, until about ``seconds`` have passed or max_rows
    rows are done. Returns (rows, seconds)."""
    import oracle.attention as orc
    rows_done, t0 = 0, time.time()
    scale = float(np.float32(1.0 / 8.0))
    while rows_done < max_rows and time.time() - t0 < seconds:
        b, r0 = divmod(rows_done, 4096)
        orc.fwd_rows(c["q"], c["k"], c["v"], "bf16", scale, b, np.arange(r0, r0 + 512))
        rows_done += 512
    return rows_done, time.time() - t0


def cpu_baseline_fwd(c, seconds):
    """The oracle on the headline workload with every BLAS thread it gets (the
    reported value), then one thread on a smaller sample."""
    from threadpoolctl import threadpool_limits
    threads = _blas_threads()
    rows, dt = _fwd_sample(c, seconds, 4 * 4096)
    flops = 4.0 * 16 * rows * 4096 * 64
    with threadpool_limits(limits=1):
        rows1, dt1 = _fwd_sample(c, seconds / 3, 4 * 4096)
    flops1 = 4.0 * 16 * rows1 * 4096 * 64
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of 16384 query rows (batch-major) x 16 heads x 4096 keys, no mask, "
                      f"{flops / 1e9:.2f} GFLOP in {dt:.1f} s on {threads} BLAS threads",
            "single_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s",
                              "sample": f"{rows1} query rows x 16 heads x 4096 keys, {flops1 / 1e9:.2f} GFLOP "
                                        f"in {dt1:.1f} s"},
            "host": host_description()}


def cpu_baseline_decode(ctx, seconds):
    """fp64 oracle decode of whole sequences (all 32 heads) until the time is up."""
    import mea_inputs as inp
    import oracle.attention as orc
    B, Hq, Hkv, D = 32, 32, 8, 128
    q = inp.normal_bits(5, (B, Hq, D), "bf16", 0)
    done, nbytes, busy = [], 0, 0.0
    for b in range(B):
        kb, vb = inp.decode_cache_rows(5, b, int(ctx[b]), Hkv, D, "bf16")
        t0 = time.time()
        orc.decode(q[b:b + 1], kb[None], vb[None], ctx[b:b + 1], "bf16", float(np.float32(1 / np.sqrt(D))))
        busy += time.time() - t0
        done.append(b)
        nbytes += int(ctx[b]) * Hkv * D * 2 * 2 + Hq * D * 2 * 2
        if busy >= seconds:
            break
    threads = _blas_threads()
    return {"value": nbytes / busy / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} whole sequences (ctx {[int(ctx[b]) for b in done]}), "
                      f"{nbytes / 1e9:.3f} GB of K/V in {busy:.1f} s on {threads} BLAS threads",
            "host": host_description()}


def naive_vs_mea_table(torch, inp, mea, B=4, H=16, D=64, seqlens=(512, 1024, 2048, 4096)):
    """The xFormers tutorial's benchmark (chipsbuilder.com page, "Benchmark
    Memoria e Velocita dell'Attenzione Classica"): time and peak memory of a
    naive attention (the score matrix materialised: matmul, softmax, matmul in
    torch) against the memory-efficient kernel, over sequence lengths. Timing
    follows the page's method: 5 warmup calls, then the mean of 20 calls
    between two events; peak memory is torch's max_memory_allocated after
    resetting the peak. Shapes: B=4, H=16, D=64, bf16, no mask (the page does
    not state its own)."""
    def cuda_time(fn, iters=20, warmup=5):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / iters

    def peak_mb(fn):
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() / 1e6

    rows = []
    for M in seqlens:
        c = inp.dense_case(3, B, M, M, H, H, D, "bf16")
        q, k, v = (to_dev(c[x], torch) for x in ("q", "k", "v"))
        # [B,H,M,D] copies for the naive path; the key operand is transposed
        # into a contiguous tensor before the batched product.
        qh = q.permute(0, 2, 1, 3).contiguous()
        kt = k.permute(0, 2, 3, 1).contiguous()
        vh = v.permute(0, 2, 1, 3).contiguous()
        scale = 1.0 / np.sqrt(D)

        def naive():
            sc = torch.matmul(qh, kt) * scale
            p = torch.softmax(sc.float(), dim=-1).to(torch.bfloat16)
            return torch.matmul(p, vh)

        def memeff():
            return mea.fwd(q, k, v, scale=scale)

        o_n = naive().permute(0, 2, 1, 3).float()
        o_m = memeff().float()
        diff = float((o_n - o_m).abs().max())
        row = {"seqlen": M, "naive_mb": round(peak_mb(naive), 1), "mea_mb": round(peak_mb(memeff), 1),
               "naive_ms": round(cuda_time(naive), 3), "mea_ms": round(cuda_time(memeff), 3),
               "max_abs_diff": diff}
        row["speedup"] = round(row["naive_ms"] / row["mea_ms"], 2)
        rows.append(row)
        log(f"[table] {row}")
        del q, k, v, qh, kt, vh
    print(json.dumps({"table": "naive vs memory-efficient attention forward", "shape": {"B": B, "H": H, "D": D},
                      "dtype": "bf16", "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU clock takes tens of milliseconds to settle after start-up (the
    # headline launch runs 10-15 % slower in its first ~10 ms): 20 warmup
    # steps are about 50 ms.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--items", default="fwd_noncausal,fwd_causal,fwd_varlen,decode,fwd_blocksparse,"
                                       "bwd_noncausal,bwd_causal",
                    help="comma-separated subset of the step to run (for profiling one kernel)")
    ap.add_argument("--table", action="store_true",
                    help="reproduce the tutorial's naive-vs-memory-efficient table (ms, peak MB) for seqlen 512..4096")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, 5 times (reference for HBM counters)")
    ap.add_argument("--traffic-summary", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                            "COPY_WRITE_CSV", "OUT_JSON"),
                    help="write the per-kernel HBM traffic file from rocprofv3 counter collections and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mea_inputs as inp
    import memory_efficient_exact_tiled_amd as mea

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.table:
        naive_vs_mea_table(torch, inp, mea)
        return
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "copy_calibration_bytes_written": 1 << 30,
                          "launches": 5}), flush=True)
        return
    wanted = set(args.items.split(","))
    x = build_inputs(torch, inp, with_decode="decode" in wanted)
    d, vl, dc = x["dense"], x["varlen"], x["decode"]
    ws = torch.empty(mea.decode_workspace_bytes(32, 32, 128, 32768), dtype=torch.uint8, device="cuda")
    out_d = torch.empty_like(d["q"])
    out_c = torch.empty_like(d["q"])
    out_v = torch.empty_like(vl["q"])
    out_dec = torch.empty_like(dc["q"]) if "q" in dc else None
    # Backward inputs: the forward's output and lse (computed once, untimed)
    # and a seeded upstream gradient.
    B_, M_, H_ = d["q"].shape[:3]
    dout = to_dev(inp.normal_bits(7, tuple(d["q"].shape), "bf16", 0), torch)
    fb = {}
    for cz in (False, True):
        lse_ = torch.empty((B_, H_, M_), dtype=torch.float32, device="cuda")
        o_ = mea.fwd(d["q"], d["k"], d["v"], causal=cz, lse=lse_)
        fb[cz] = (o_, lse_, torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
                  torch.empty(mea.bwd_workspace_bytes(B_, M_, H_, int(cz)), dtype=torch.uint8, device="cuda"))

    # Block-sparse item: its own inputs (16K tokens) and mask.
    MS = 16384
    bs_host = inp.dense_case(12, 1, MS, MS, 16, 16, 64, "bf16")
    bs = {k_: to_dev(bs_host[k_], torch) for k_ in ("q", "k", "v")}
    bmask_host = inp.band_global_block_mask(MS // 64, MS // 64, 3, 1)
    bmask = torch.from_numpy(bmask_host).cuda()
    out_bs = torch.empty_like(bs["q"])
    r_, c_ = np.nonzero(bmask_host)
    bs_pairs = float(np.sum(np.where(c_ < r_, 64 * 64, np.where(c_ == r_, 64 * 65 // 2, 0))))

    def bwd_item(cz):
        o_, lse_, gq, gk, gv, wsb = fb[cz]
        return lambda: mea.bwd(d["q"], d["k"], d["v"], o_, dout, lse_, causal=cz, dq=gq, dk=gk, dv=gv, workspace=wsb)

    items = [
        ("fwd_noncausal", lambda: mea.fwd(d["q"], d["k"], d["v"], out=out_d)),
        ("fwd_causal", lambda: mea.fwd(d["q"], d["k"], d["v"], causal=True, out=out_c)),
        ("fwd_varlen", lambda: mea.fwd(vl["q"], vl["k"], vl["v"], causal=True, seqstart_q=vl["seqstart"],
                                       alibi_slopes=vl["slopes"], out=out_v)),
        ("decode", lambda: mea.decode(dc["q"], dc["kc"], dc["vc"], dc["ctx"], out=out_dec, workspace=ws)),
        ("fwd_blocksparse", lambda: mea.fwd_blocksparse(bs["q"], bs["k"], bs["v"], bmask, causal=True, out=out_bs)),
        ("bwd_noncausal", bwd_item(False)),
        ("bwd_causal", bwd_item(True)),
    ]
    unknown = wanted - {n for n, _ in items}
    if unknown:
        print(f"unknown items {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    items = [(n, fn) for n, fn in items if n in wanted]
    events = {name: [] for name, _ in items}

    def step(record):
        for name, fn in items:
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                events[name].append((e0, e1))
            else:
                fn()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f}s")

    ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev])) for n, ev in events.items()}

    # The headline forward and the decode are also timed on their own, outside
    # the mixed step: ALONE launches in a row between two events.
    alone = {}
    for name, fn in items:
        if name not in ("fwd_noncausal", "decode"):
            continue
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(ALONE):
            fn()
        e1.record()
        torch.cuda.synchronize()
        alone[name] = e0.elapsed_time(e1) / ALONE
    L = x["lengths"].astype(np.int64)
    flops_all = {
        "fwd_noncausal": 4.0 * 4 * 16 * 4096 * 4096 * 64,
        "fwd_causal": 4.0 * 4 * 16 * 64 * (4096 * 4097 / 2),
        "fwd_varlen": 4.0 * 128 * 32 * float(np.sum(L * (L + 1) // 2)),
        "fwd_blocksparse": 4.0 * 64 * 16 * bs_pairs,
        "bwd_noncausal": 10.0 * 4 * 16 * 4096 * 4096 * 64,
        "bwd_causal": 10.0 * 4 * 16 * 64 * (4096 * 4097 / 2),
    }
    ctx = x["decode"]["ctx_host"].astype(np.int64)
    dec_bytes = float(ctx.sum() * 8 * 128 * 2 * 2 + 32 * 32 * 128 * 2 * 2)
    # Algorithmic HBM bytes per item (every input read once, every output
    # written once), for each item's own roofline: the bound is whichever of
    # MFMA time and HBM time is longer at peak.
    dense_bytes = 4.0 * 4 * 4096 * 16 * 64 * 2                   # q, k, v, out
    bytes_all = {
        "fwd_noncausal": dense_bytes,
        "fwd_causal": dense_bytes,
        "fwd_varlen": float(L.sum()) * (2 * 32 + 2 * 8) * 128 * 2,  # q, out (Hq); k, v (Hkv)
        "fwd_blocksparse": 4.0 * MS * 16 * 64 * 2,
        "bwd_noncausal": 8.0 * 4 * 4096 * 16 * 64 * 2 + 4 * 16 * 4096 * 4,   # q k v out dout, dq dk dv; lse
        "bwd_causal": 8.0 * 4 * 4096 * 16 * 64 * 2 + 4 * 16 * 4096 * 4,
    }
    tflops = {n: flops_all[n] / (ms[n] * 1e-3) / 1e12 for n in flops_all if n in ms}
    dec_gbs = dec_bytes / (ms["decode"] * 1e-3) / 1e9 if "decode" in ms else None
    per_item = {}
    for n in ms:
        if n in tflops:
            log(f"[bench] {n}: {ms[n] * 1e3:.1f} us  {tflops[n]:.1f} TFLOP/s "
                f"({tflops[n] / PEAK_MFMA_TFLOPS:.1%} of MFMA peak; {flops_all[n] / bytes_all[n]:.0f} flop/B, "
                f"{max(flops_all[n] / (PEAK_MFMA_TFLOPS * 1e12), bytes_all[n] / (PEAK_HBM_GBS * 1e9)) / (ms[n] * 1e-3):.1%} "
                f"of its roofline)")
            t_mfma = flops_all[n] / (PEAK_MFMA_TFLOPS * 1e12)
            t_hbm = bytes_all[n] / (PEAK_HBM_GBS * 1e9)
            per_item[n] = {"avg_launch_us": round(ms[n] * 1e3, 2), "tflops": round(tflops[n], 2),
                           "frac_mfma_peak": round(tflops[n] / PEAK_MFMA_TFLOPS, 4),
                           "algorithmic_bytes": bytes_all[n],
                           "intensity_flop_per_byte": round(flops_all[n] / bytes_all[n], 1),
                           "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                           "frac_roofline": round(max(t_mfma, t_hbm) / (ms[n] * 1e-3), 4)}
        else:
            log(f"[bench] decode: {ms[n] * 1e3:.1f} us  {dec_gbs:.1f} GB/s ({dec_gbs / PEAK_HBM_GBS:.1%} of HBM peak)")
            per_item[n] = {"avg_launch_us": round(ms[n] * 1e3, 2), "gbs": round(dec_gbs, 1),
                           "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": dec_bytes}
    for n, t in alone.items():
        if n in tflops:
            log(f"[bench] {n} alone ({ALONE} back to back): {t * 1e3:.1f} us  "
                f"{flops_all[n] / (t * 1e-3) / 1e12:.1f} TFLOP/s")
        else:
            log(f"[bench] {n} alone ({ALONE} back to back): {t * 1e3:.1f} us  {dec_bytes / (t * 1e-3) / 1e9:.1f} GB/s")
    head = tflops.get("fwd_noncausal")
    traffic = measured_traffic()

    res = {
        "metric": "attn fwd TFLOP/s (bf16, M=4096, % MFMA peak); decode HBM GB/s",
        "value": round(head, 2) if head is not None else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "attention forward B=4 M=N=4096 H=16 D=64 bf16 (no mask; causal beside it) "
                        "+ packed 8x[64,2048] Hq=32 Hkv=8 D=128 block-diag causal ALiBi "
                        "+ decode B=32 ctx[1024,32768] Hq=32 Hkv=8 D=128 "
                        "+ block-sparse causal B=1 M=16384 H=16 D=64 (window 3 blocks + 1 global, 64x64) "
                        "+ backward of the two B=4 M=4096 forwards",
            "items": sorted(ms),
            "global_batch": 4, "seq_len": 4096, "parallelism": "none (1 GPU)",
        },
        "roofline": None if head is None else {
            "bound": "mfma", "achieved": round(head, 2), "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": round(head / PEAK_MFMA_TFLOPS, 4),
            "traffic": traffic_for(traffic, "fwd_kernelIDF16bLi64ELi2ELi2ELi2"),
            "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
            "kernel": "fwd_kernel<bf16,64,QB=2>", "avg_launch_us": round(ms["fwd_noncausal"] * 1e3, 2),
            "algorithmic_flops": flops_all["fwd_noncausal"],
            "alone": None if "fwd_noncausal" not in alone else {
                "launches_back_to_back": ALONE, "avg_launch_us": round(alone["fwd_noncausal"] * 1e3, 2),
                "achieved": round(flops_all["fwd_noncausal"] / (alone["fwd_noncausal"] * 1e-3) / 1e12, 2),
                "frac": round(flops_all["fwd_noncausal"] / (alone["fwd_noncausal"] * 1e-3) / 1e12
                              / PEAK_MFMA_TFLOPS, 4)},
        },
        "roofline_decode": None if dec_gbs is None else {
            "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            # At B=32 the plan runs inside the split kernel (no plan launch).
            "traffic": traffic_for(traffic, "decode_split_kernelIDF16bLi128", "decode_combine_kernelIDF16bLi128"),
            "kernel": "decode_split_kernel<bf16,128> (plan inside) + decode_combine_kernel<bf16,128>",
            "avg_launch_us": round(ms["decode"] * 1e3, 2), "algorithmic_bytes": dec_bytes,
            "alone": None if "decode" not in alone else {
                "launches_back_to_back": ALONE, "avg_launch_us": round(alone["decode"] * 1e3, 2),
                "achieved": round(dec_bytes / (alone["decode"] * 1e-3) / 1e9, 1),
                "frac": round(dec_bytes / (alone["decode"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        },
        "roofline_bwd": None if "bwd_noncausal" not in tflops else {
            "bound": "mfma", "achieved": round(tflops["bwd_noncausal"], 2), "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops["bwd_noncausal"] / PEAK_MFMA_TFLOPS, 4),
            "kernel": "bwd_prep + bwd_dkdv + bwd_dq <bf16,64> (non-causal)",
            "traffic": traffic_for(traffic, "bwd_prep_kernelIDF16bLi64", "bwd_dkdv_kernelIDF16bLi64ELi0ELi2ELi0",
                                   "bwd_dq_kernelIDF16bLi64ELi0ELi2ELi0"),
            "avg_launch_us": round(ms["bwd_noncausal"] * 1e3, 2),
            "algorithmic_flops": flops_all["bwd_noncausal"],
        },
        "per_item": per_item,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host (bounded sample)")
        res["cpu_baseline"] = cpu_baseline_fwd(x["dense_host"], args.cpu_seconds)
        res["cpu_baseline_decode"] = cpu_baseline_decode(x["decode"]["ctx_host"], args.cpu_seconds / 2)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
