"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutant replaces one step of ``oracle.attention`` with a wrong variant:
a dropped or misplaced term, a wrong sign or index, a transposed operand.
The test passes when at least one pin from ``oracle_pins`` fails for the
mutant, i.e. the pins would have exposed that mistake in the real oracle.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import attention as A

_orig = {n: getattr(A, n) for n in ("scores", "causal_allowed", "softmax_rows", "attention_head",
                                    "kv_head_of", "e4m3fn_to_float", "gather_pages", "lse_merge")}


def _scores_no_scale(q, k, scale):
    return q @ k.T


def _scores_sqrt_scale(q, k, scale):
    return np.sqrt(scale) * (q @ k.T)


def _scores_transposed(q, k, scale):
    return float(scale) * (k @ q.T).T[:, ::-1]


def _causal_flipped(rows, Sq, Sk):
    return np.arange(Sk)[None, :] >= np.asarray(rows)[:, None] + (Sk - Sq)


def _causal_wrong_offset(rows, Sq, Sk):
    return np.arange(Sk)[None, :] <= np.asarray(rows)[:, None] + (Sq - Sk)


def _causal_strict(rows, Sq, Sk):
    return np.arange(Sk)[None, :] < np.asarray(rows)[:, None] + (Sk - Sq)


def _softmax_no_norm(s):
    P, m, l = _orig["softmax_rows"](s)
    return P * np.where(l > 0, l, 1)[:, None], m, l


def _softmax_linear(s):
    m = s.max(axis=1)
    e = np.where(np.isfinite(s), s - m[:, None] + 1.0, 0.0)
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def _head_lse_no_max(q, k, v, scale, causal=False, rows=None):
    o, lse = _orig["attention_head"](q, k, v, scale, causal, rows)
    Sq = q.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    s = _orig["scores"](q[rows], k, scale)
    return o, lse - s.max(axis=1) if s.shape[1] else lse


def _head_lse_log2(q, k, v, scale, causal=False, rows=None):
    o, lse = _orig["attention_head"](q, k, v, scale, causal, rows)
    return o, lse / np.log(2.0)


def _kv_head_modulo(h, Hq, Hkv, kv_head_map=None):
    if kv_head_map is not None:
        return int(kv_head_map[h])
    return h % Hkv


def _kv_head_ignores_map(h, Hq, Hkv, kv_head_map=None):
    return h // (Hq // Hkv)


def _fp8_bias8(codes):
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _fp8_no_subnormal(codes):
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _fp8_nan_as_480(codes):
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return sign * mag


def _gather_reversed(pool, table_row, L, g, scale=None):
    n = (L + 63) // 64
    return _orig["gather_pages"](pool, np.asarray(table_row)[:n][::-1], L, g, scale)


def _gather_untruncated(pool, table_row, L, g, scale=None):
    n = (L + 63) // 64
    return _orig["gather_pages"](pool, table_row, n * 64, g, scale)


def _gather_wrong_scale_index(pool, table_row, L, g, scale=None):
    if scale is None:
        return _orig["gather_pages"](pool, table_row, L, g, None)
    return _orig["gather_pages"](pool, table_row, L, g, np.asarray(scale)[::-1])


def _merge_plain_mean(po, pl):
    o, lse = _orig["lse_merge"](po, pl)
    fin = np.isfinite(np.asarray(pl, dtype=float))
    return np.asarray(po)[fin].mean(axis=0), lse


def _merge_max_lse(po, pl):
    o, _ = _orig["lse_merge"](po, pl)
    pl = np.asarray(pl, dtype=float)
    return o, pl[np.isfinite(pl)].max()


MUTANTS = {
    "scores_no_scale": ("scores", _scores_no_scale),
    "scores_sqrt_scale": ("scores", _scores_sqrt_scale),
    "scores_transposed": ("scores", _scores_transposed),
    "causal_flipped": ("causal_allowed", _causal_flipped),
    "causal_wrong_offset": ("causal_allowed", _causal_wrong_offset),
    "causal_strict": ("causal_allowed", _causal_strict),
    "softmax_unnormalised": ("softmax_rows", _softmax_no_norm),
    "softmax_linear": ("softmax_rows", _softmax_linear),
    "lse_without_max": ("attention_head", _head_lse_no_max),
    "lse_base2": ("attention_head", _head_lse_log2),
    "gqa_modulo": ("kv_head_of", _kv_head_modulo),
    "gqa_ignores_map": ("kv_head_of", _kv_head_ignores_map),
    "fp8_bias8": ("e4m3fn_to_float", _fp8_bias8),
    "fp8_no_subnormal": ("e4m3fn_to_float", _fp8_no_subnormal),
    "fp8_nan_as_finite": ("e4m3fn_to_float", _fp8_nan_as_480),
    "gather_reversed": ("gather_pages", _gather_reversed),
    "gather_untruncated": ("gather_pages", _gather_untruncated),
    "gather_wrong_scale": ("gather_pages", _gather_wrong_scale_index),
    "merge_plain_mean": ("lse_merge", _merge_plain_mean),
    "merge_max_lse": ("lse_merge", _merge_max_lse),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # an assertion or a crash both expose the mutant
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin catches mutant {name}"
