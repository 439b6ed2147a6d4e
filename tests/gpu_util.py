"""Helpers of the GPU parity tests: move seeded bit patterns to the device and back."""
import sys

import numpy as np
import torch

TOL = {"fp16": 2e-3, "bf16": 1.6e-2}   # max-abs error against the fp64 oracle (fp32 accumulation)
# Row log-sum-exp: the normaliser l sums P after P is rounded to the input type
# (the weights P.V really uses), so |dl/l| <= u, the unit roundoff of that type
# (bf16: 8-bit significand, u = 2^-8; fp16: 11-bit, u = 2^-11), and
# |d lse| <= ln(1 + u) < u. The bound is reached when a few weights dominate a
# row and round the same way (a steep ALiBi slope); the margin covers fp32
# accumulation and the final log.
LSE_TOL = {"fp16": 2.0 ** -11 * 1.25, "bf16": 2.0 ** -8 * 1.25}
TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


def dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DTYPE[dtype]).cuda()


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def f32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).cuda()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def report(name, got, want, tol):
    err = np.abs(got - want)
    worst = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else ()
    me = float(err.max()) if err.size else 0.0
    say(f"[{name}] max_abs_err={me:.3e} tol={tol:.1e} worst_at={worst}"
        + (f" |o|={abs(float(want[worst])):.3f}" if err.size else ""))
    return me
