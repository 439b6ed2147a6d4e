"""The per-element gradient bars of the GPU backward tests (tests/grad_bounds.py), on the CPU.

The bars are only as good as the terms they sum: these checks pin those terms
to the oracle's backward (the gradients summed from the same P and dS agree
with ``oracle.attention.bwd`` to 1e-12) and check the properties a magnitude
sum must have (it dominates the sum; where no term exists only the floor of
the stored gradient's rounding is left).
"""
import numpy as np
import pytest

import mea_inputs as inp
import oracle.attention as orc
from grad_bounds import C, U, check_grads, grad_terms

CASES = [
    # name, kind, kwargs
    ("dense_nomask_fp16", dict(seed=1, B=2, M=37, N=50, Hq=2, Hkv=2, D=16, dt="fp16"), {}),
    ("dense_causal_alibi_gqa_bf16", dict(seed=2, B=1, M=70, N=70, Hq=4, Hkv=2, D=32, dt="bf16"),
     dict(causal=True, alibi=True)),
    ("dense_more_queries_than_keys_causal", dict(seed=3, B=1, M=40, N=9, Hq=2, Hkv=1, D=8, dt="bf16"),
     dict(causal=True)),
    ("blocksparse_causal", dict(seed=4, B=1, M=150, N=140, Hq=2, Hkv=2, D=8, dt="bf16"),
     dict(causal=True, block=0.5)),
]


def _case(spec, opts):
    c = inp.dense_case(spec["seed"], spec["B"], spec["M"], spec["N"], spec["Hq"], spec["Hkv"], spec["D"], spec["dt"])
    do = inp.normal_bits(spec["seed"] + 7, c["q"].shape, spec["dt"], 0)
    kw = dict(causal=opts.get("causal", False))
    if opts.get("alibi"):
        kw["alibi_slopes"] = inp.alibi_slopes(spec["Hq"])
    if opts.get("block"):
        kw["block_mask"] = inp.random_block_mask(spec["seed"], -(-spec["M"] // 64), -(-spec["N"] // 64),
                                                 opts["block"], keep_diagonal=False)
    scale = float(np.float32(1.0 / np.sqrt(spec["D"])))
    return c, do, scale, kw


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_terms_sum_to_the_oracle_gradients(case):
    _, spec, opts = case
    c, do, scale, kw = _case(spec, opts)
    want = orc.bwd(c["q"], c["k"], c["v"], do, spec["dt"], scale, **kw)
    grads, terms = grad_terms(c["q"], c["k"], c["v"], do, spec["dt"], scale, **kw)
    for w, g, t in zip(want, grads, terms):
        assert np.max(np.abs(w - g), initial=0.0) <= 1e-12 * max(1.0, float(np.max(np.abs(w), initial=0.0)))
        assert np.all(t >= np.abs(g) - 1e-12)      # a magnitude sum dominates its sum
        assert np.all(t[g != 0] > 0)


def test_packed_terms_match_the_oracle():
    c = inp.varlen_case(5, [33, 0, 70, 1], 4, 2, 16, "bf16")
    do = inp.normal_bits(12, c["q"].shape, "bf16", 0)
    kw = dict(causal=True, seqstart_q=c["seqstart"], alibi_slopes=inp.alibi_slopes(4))
    want = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", 0.25, **kw)
    grads, terms = grad_terms(c["q"], c["k"], c["v"], do, "bf16", 0.25, **kw)
    for w, g in zip(want, grads):
        assert np.max(np.abs(w - g)) <= 1e-12 * max(1.0, float(np.max(np.abs(w))))
    # row 0 of every causal segment has one key: its dq vanishes exactly, but
    # the bar does not (the Delta error terms stay).
    assert np.all(grads[0][0, 0] == 0) and np.all(terms[0][0, 0] > 0)


def test_rows_without_keys_get_only_the_rounding_floor():
    from grad_bounds import ETA
    c = inp.dense_case(6, 1, 12, 5, 2, 2, 8, "fp16")
    do = inp.normal_bits(13, c["q"].shape, "fp16", 0)
    _, terms = grad_terms(c["q"], c["k"], c["v"], do, "fp16", 0.3, causal=True)
    floor = ETA["fp16"] / U["fp16"]
    # M=12, N=5, bottom-right: rows 0..6 see no key
    assert np.all(terms[0][0, :7] == floor) and np.all(terms[0][0, 7:] > 10 * floor)


def test_check_grads_flags_one_wrong_element():
    """A gradient one bar off in one small element fails the check, although
    it is far inside a bar scaled by the tensor's largest gradient."""
    c, do, scale, kw = _case(*CASES[1][1:])
    want = orc.bwd(c["q"], c["k"], c["v"], do, "bf16", scale, **kw)
    _, terms = grad_terms(c["q"], c["k"], c["v"], do, "bf16", scale, **kw)
    got = [w.copy() for w in want]
    check_grads("exact", got, want, terms, "bf16", say=lambda *a: None)
    t = terms[2]
    at = np.unravel_index(int(np.argmin(np.where(t > 0, t, np.inf))), t.shape)
    got[2][at] += 2 * C * U["bf16"] * t[at]
    assert 2 * C * U["bf16"] * t[at] < C * U["bf16"] * float(np.max(np.abs(want[2])))
    with pytest.raises(AssertionError):
        check_grads("planted", got, want, terms, "bf16", say=lambda *a: None)
