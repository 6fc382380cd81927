"""Plausible mistakes planted in copies of the float64 checker (on the CPU)
must each be caught by at least one pin; the real checker is untouched."""

import os
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "gqa_modulo_map": ("kvh = h // group", "kvh = h % num_kv_heads"),
    "causal_off_by_one": ("min(start_pos + i + 1, kv_len)", "min(start_pos + i, kv_len)"),
    "start_pos_ignored": ("min(start_pos + i + 1, kv_len)", "min(i + 1, kv_len)"),
    "scale_dropped": ("s = scale * (qb @ kb.T)", "s = (qb @ kb.T)"),
    "scale_inverted": ("s = scale * (qb @ kb.T)", "s = (qb @ kb.T) / scale if scale else qb @ kb.T"),
    "wrong_value_operand": ("o = (e @ vb)", "o = (e @ kb)"),
    "max_sign_flip": ("np.exp(s - m_safe[:, None])", "np.exp(s + m_safe[:, None])"),
    "full_lse_not_pair": ("np.where(nonempty, np.log(z_safe), EMPTY_SENTINEL)",
                          "np.where(nonempty, np.log(z_safe) + m_safe, EMPTY_SENTINEL)"),
    "no_normalisation": ("o = (e @ vb) / z_safe[:, None]", "o = (e @ vb)"),
    "mask_inclusive": ("np.arange(wmax)[None, :] < w[:, None]",
                       "np.arange(wmax)[None, :] <= w[:, None] - 2"),
    "empty_sentinel_zero": ("EMPTY_SENTINEL = -1e30", "EMPTY_SENTINEL = 0.0"),
    "decode_window_short": ("min(int(kv_pos) + 1, max_seq)", "min(int(kv_pos), max_seq)"),
    "decode_gqa_modulo": ("        kvh = h // group\n        qv", "        kvh = h % num_kv_heads\n        qv"),
    "decode_no_scale": ("s = scale * (kw @ qv)", "s = (kw @ qv)"),
    "q_head_offset": ("qh = q[:, h * d:(h + 1) * d]", "qh = q[:, kvh * d:(kvh + 1) * d]"),
    "rope_sign_flip": ("lo * c - hi * s, hi * c + lo * s", "lo * c + hi * s, hi * c - lo * s"),
    "rope_interleaved_pairing": ("lo = xh[..., :half]\n    hi = xh[..., half:]",
                                 "lo = xh[..., 0::2]\n    hi = xh[..., 1::2]"),
    "rope_frequency_exponent": ("(-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)",
                                "(-(np.arange(half, dtype=np.float64)) / head_dim)"),
    "rope_cos_sin_swapped": ("np.stack([np.cos(ang), np.sin(ang)], axis=-1)",
                             "np.stack([np.sin(ang), np.cos(ang)], axis=-1)"),
    "rope_query_position_no_start": ("apply_rope(q[rows], start_pos + rows,",
                                     "apply_rope(q[rows], rows,"),
    "rope_key_position_shift": ("np.arange(kv_len), rope, num_kv_heads",
                                "np.arange(kv_len) // 2, rope, num_kv_heads"),
    "bwd_delta_sign": ("ds = p * (dp - dd[:, None])", "ds = p * (dp + dd[:, None])"),
    "bwd_delta_unweighted": ("dd = (p * dp).sum(axis=1)", "dd = dp.sum(axis=1)"),
    "bwd_dk_unscaled": ("+= scale * (ds[:, keys].T @ qb)", "+= (ds[:, keys].T @ qb)"),
    "bwd_dv_from_ds": ("+= p[:, keys].T @ gb", "+= ds[:, keys].T @ gb"),
    "bwd_dq_from_v": ("scale * (ds[sel] @ kc)", "scale * (ds[sel] @ vc)"),
    "bwd_dk_overwritten": ("dk[:, c * d:(c + 1) * d] += scale", "dk[:, c * d:(c + 1) * d] = scale"),
    "bwd_dv_not_summed_over_group": ("dv[:, c * d:(c + 1) * d] += p", "dv[:, c * d:(c + 1) * d] = p"),
    "bwd_magnitude_term_inflated": ("em = np.abs(ds) + p * (np.abs(dp) + np.abs(dd)[:, None])",
                                    "em = np.abs(ds) + 2.0 * p * (np.abs(dp) + np.abs(dd)[:, None])"),
    "bwd_magnitude_delta_dropped": ("em = np.abs(ds) + p * (np.abs(dp) + np.abs(dd)[:, None])",
                                    "em = np.abs(ds) + p * np.abs(dp)"),
    "bwd_magnitude_dv_inflated": ("dv_m[:, c * d:(c + 1) * d] += p[:, keys].T @ np.abs(gb)",
                                  "dv_m[:, c * d:(c + 1) * d] += 3.0 * p[:, keys].T @ np.abs(gb)"),
    "bwd_magnitude_dq_unscaled": ("scale * (em[sel] @ np.abs(kc))", "(em[sel] @ np.abs(kc))"),
    "rope_keys_unrotated": ("        k = apply_rope(k[:kv_len]", "        k = 1.0 * (k[:kv_len]"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # an assertion or a crash both count
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches mutant {name}"
