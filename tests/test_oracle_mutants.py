"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

A pin set that a dropped term, a wrong sign or index, or a transposed operand
can slip through does not pin anything. Each mutant below is the oracle's own
source with one textual change; the test asserts that at least one check in
``oracle_checks.ALL_CHECKS`` fails on it. Mutants live only in memory, on the CPU.
"""
import inspect
import types

import pytest

import oracle.attention as orc
from oracle_checks import ALL_CHECKS

MUTANTS = {
    "causal_off_by_one": ("allowed = j[None, :] <= pos_i[:, None]", "allowed = j[None, :] < pos_i[:, None]"),
    "top_left_alignment": ("pos_i = i + (N - M)", "pos_i = i + 0"),
    "dropped_scale": ("s = sc * (q[i, h, :] @ k[:, g, :].T)", "s = (q[i, h, :] @ k[:, g, :].T)"),
    "alibi_sign": ("s = s - slope * np.abs", "s = s + slope * np.abs"),
    "alibi_without_abs": ("np.abs(pos_i[:, None] - j[None, :])", "(pos_i[:, None] - j[None, :])"),
    "alibi_slope_by_kv_head": ("slope = float(np.float32(slopes[h]))", "slope = float(np.float32(slopes[g]))"),
    "gqa_modulo_mapping": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "pv_uses_k": ("(e @ v[:, g, :])", "(e @ k[:, g, :])"),
    "lse_drops_max": ("lse[h] = np.where(any_allowed, m + np.log(safe_l), -np.inf)",
                      "lse[h] = np.where(any_allowed, np.log(safe_l), -np.inf)"),
    "unnormalised": ("(e @ v[:, g, :]) / safe_l[:, None]", "(e @ v[:, g, :])"),
    "decode_drops_new_token": ("kb = decode_bits(kcache_bits[b, :n], dtype)",
                               "kb = decode_bits(kcache_bits[b, :max(n - 1, 1)], dtype)"),
    "decode_wrong_batch_row": ("vb = decode_bits(vcache_bits[b, :n], dtype)",
                               "vb = decode_bits(vcache_bits[0, :n], dtype)"),
    "bf16_decode_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "transposed_p": ("(e @ v[:, g, :]) / safe_l[:, None]",
                     "((e.T if e.shape[0] == e.shape[1] else e) @ v[:, g, :]) / safe_l[:, None]"),
    "kvcache_drops_last_row": ("ob, lb = attend(decode_bits(q_bits[b], dtype), decode_bits(kcache_bits[b, :n], dtype),",
                               "ob, lb = attend(decode_bits(q_bits[b], dtype), decode_bits(kcache_bits[b, :n - 1], dtype),"),
    "kv_append_short": ("n = max(0, min(T, S_max - c))", "n = max(0, min(T, S_max - c - 1))"),
    "blockdiag_ignores_k_segments": ("return [(0, int(sq[s]), int(sq[s + 1]), int(sk[s]), int(sk[s + 1]))",
                                     "return [(0, int(sq[s]), int(sq[s + 1]), 0, int(sk[-1]))"),
    "bwd_drops_delta": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "bwd_delta_wrong_axis": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                             "ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))"),
    "bwd_dq_no_scale": ("dq[:, h, :] = sc * (ds @ k[:, g, :])", "dq[:, h, :] = (ds @ k[:, g, :])"),
    "bwd_dk_ds_untransposed": ("dk[:, g, :] += sc * (ds.T @ q[:, h, :])",
                               "dk[:, g, :] += sc * ((ds if M == N else ds.T) @ q[:, h, :])"),
    "bwd_dv_p_untransposed": ("dv[:, g, :] += p.T @ do[:, h, :]", "dv[:, g, :] += (p if M == N else p.T) @ do[:, h, :]"),
    "bwd_gqa_overwrites": ("dv[:, g, :] += p.T @ do[:, h, :]", "dv[:, g, :] = p.T @ do[:, h, :]"),
    "bwd_dp_uses_k": ("dp = do[:, h, :] @ v[:, g, :].T", "dp = do[:, h, :] @ k[:, g, :].T"),
    "bwd_dk_uses_k": ("dk[:, g, :] += sc * (ds.T @ q[:, h, :])", "dk[:, g, :] += sc * (ds.T @ k[:, g, :][:M] if M <= N else ds.T @ q[:, h, :])"),
    "bwd_unmasked": ("allowed = (j[None, :] <= pos[:, None]) if causal else np.ones((M, N), dtype=bool)",
                     "allowed = np.ones((M, N), dtype=bool)"),
    "bwd_top_left": ("pos = i + (N - M)", "pos = i"),
    "bwd_alibi_sign": ("s = s - float(np.float32(slopes[h])) * np.abs", "s = s + float(np.float32(slopes[h])) * np.abs"),
    "bwd_unnormalised_p": ("p = e / np.where(tot > 0, tot, 1.0)", "p = e"),
    "blocksparse_transposed": ("allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // BLOCK, j[None, :] // BLOCK]\n    any_allowed",
                               "allowed = allowed & np.asarray(block_mask, dtype=bool).T[j[None, :] // BLOCK, i[:, None] // BLOCK].T\n    any_allowed"),
    "blocksparse_block_32": ("BLOCK = 64", "BLOCK = 32"),
    "blocksparse_ignored_fwd": ("allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // BLOCK, j[None, :] // BLOCK]\n    any_allowed",
                                "pass\n    any_allowed"),
    "blocksparse_ignored_bwd": ("allowed = allowed & np.asarray(block_mask, dtype=bool)[i[:, None] // BLOCK, j[None, :] // BLOCK]\n    for h",
                                "pass\n    for h"),
}


def _mutant(old, new):
    src = inspect.getsource(orc)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin catches mutant {name}"
