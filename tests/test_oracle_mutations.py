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
                                    "kv_head_of", "e4m3fn_to_float", "gather_pages", "lse_merge",
                                    "kv_append", "paged_prefill_request", "paged_prefill", "prefill",
                                    "paged_decode",
                                    "attention_head_backward", "prefill_backward")}


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


def _append_at(k_pages, v_pages, page_table, seqlens, cu, k_new, v_new, where):
    kp, vp = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    for b in range(len(seqlens)):
        L, n = int(seqlens[b]), int(cu[b + 1] - cu[b])
        for i in range(n):
            t = where(L, n, i, b, cu)
            kp[int(page_table[b][t // 64]), :, t % 64] = k_new[cu[b] + i]
            vp[int(page_table[b][t // 64]), :, t % 64] = v_new[cu[b] + i]
    return kp, vp


def _append_ignores_prefix(*a):
    return _append_at(*a, where=lambda L, n, i, b, cu: i)


def _append_prefix_from_offsets(*a):
    # prefix taken as L - cu[b+1] (a packed offset) instead of L - n
    return _append_at(*a, where=lambda L, n, i, b, cu: max(L - int(cu[b + 1]), 0) + i)


def _append_k_only(k_pages, v_pages, page_table, seqlens, cu, k_new, v_new):
    kp, _ = _orig["kv_append"](k_pages, v_pages, page_table, seqlens, cu, k_new, v_new)
    return kp, np.array(v_pages, copy=True)


def _ragged_top_left(q_b, k_pages, v_pages, table_row, L, scale, rows=None):
    # causal mask aligned top-left (key j <= new-token index i), ignoring the prefix
    q_b = np.asarray(q_b, dtype=np.float64)
    n, Hq, _ = q_b.shape
    Hkv = k_pages.shape[1]
    O, LSE = np.zeros((n, Hq, v_pages.shape[3])), np.zeros((n, Hq))
    for h in range(Hq):
        g = A.kv_head_of(h, Hq, Hkv)
        kb = A.gather_pages(k_pages, table_row, L, g)
        vb = A.gather_pages(v_pages, table_row, L, g)
        s = A.scores(q_b[:, h], kb, scale)
        s = np.where(np.arange(L)[None, :] <= np.arange(n)[:, None], s, -np.inf)
        P, m, l = A.softmax_rows(s)
        O[:, h] = P @ vb
        LSE[:, h] = m + np.log(l)
    return O, LSE


def _ragged_non_causal(q_b, k_pages, v_pages, table_row, L, scale, rows=None):
    q_b = np.asarray(q_b, dtype=np.float64)
    n, Hq, _ = q_b.shape
    Hkv = k_pages.shape[1]
    O, LSE = np.zeros((n, Hq, v_pages.shape[3])), np.zeros((n, Hq))
    for h in range(Hq):
        g = A.kv_head_of(h, Hq, Hkv)
        O[:, h], LSE[:, h] = A.attention_head(q_b[:, h], A.gather_pages(k_pages, table_row, L, g),
                                              A.gather_pages(v_pages, table_row, L, g), scale, False)
    return O, LSE


def _ragged_prefix_keys_only(q, k_pages, v_pages, page_table, seqlens, cu, scale):
    # keys limited to the cached prefix (length L - n): the new tokens are left out
    cu = np.asarray(cu)
    O = np.zeros((q.shape[0], q.shape[1], v_pages.shape[3]))
    LSE = np.zeros((q.shape[0], q.shape[1]))
    for b in range(len(seqlens)):
        s, e = int(cu[b]), int(cu[b + 1])
        O[s:e], LSE[s:e] = A.paged_prefill_request(q[s:e], k_pages, v_pages, page_table[b],
                                                   int(seqlens[b]) - (e - s), scale)
    return O, LSE


def _bwd_variant(kind):
    def f(q, k, v, do, scale, causal=False):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        Sq, Sk = q.shape[0], k.shape[0]
        s = A.scores(q, k, scale)
        if causal:
            s = np.where(A.causal_allowed(np.arange(Sq), Sq, Sk), s, -np.inf)
        P, _, _ = A.softmax_rows(s)
        o = P @ v
        dv = P.T @ do
        dp = do @ v.T
        Di = np.sum(do * o, axis=1)
        ds = P * (dp - Di[:, None]) if kind != "no_rowsum" else P * dp
        sc = float(scale) if kind != "no_scale" else 1.0
        dk = sc * (ds.T @ q) if kind != "dk_from_p" else sc * (P.T @ q)
        return sc * (ds @ k), dk, dv
    return f


def _bwd_gqa_first_head(q, k, v, do, scale, causal):
    # KV gradient taken from the first query head of each group only
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dq = np.zeros((B, Hq, Sq, D)); dk = np.zeros((B, Hkv, Sk, D)); dv = np.zeros((B, Hkv, Sk, D))
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head_of(h, Hq, Hkv)
            a, bb, c = A.attention_head_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[b, h] = a
            if h % (Hq // Hkv) == 0:
                dk[b, g] = bb
                dv[b, g] = c
    return dq, dk, dv


def _head_rows_reindexed(q, k, v, scale, causal=False, rows=None):
    # the mask built from the positions 0..R-1 of the selected rows, not the rows themselves
    Sq, Sk = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    s = A.scores(q[rows], k, scale)
    if causal:
        s = np.where(A.causal_allowed(np.arange(len(rows)), Sq, Sk), s, -np.inf)
    P, m, l = A.softmax_rows(s)
    o = P @ v
    lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def _prefill_block_positions(q, k, v, scale, causal, kv_head_map=None, row_block=512, heads=None, rows=None):
    # each row block computes the rows at its positions r0.. instead of the requested rows there
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    O = np.zeros((len(pairs), len(rows), v.shape[3]))
    LSE = np.zeros((len(pairs), len(rows)))
    for n, (b, h) in enumerate(pairs):
        g = A.kv_head_of(h, Hq, Hkv, kv_head_map)
        for r0 in range(0, len(rows), row_block):
            rr = np.arange(r0, min(r0 + row_block, len(rows)))
            O[n, r0:r0 + len(rr)], LSE[n, r0:r0 + len(rr)] = A.attention_head(q[b, h], k[b, g], v[b, g], scale,
                                                                               causal, rr)
    if heads is None:
        O, LSE = O.reshape(B, Hq, len(rows), -1), LSE.reshape(B, Hq, len(rows))
    return O, LSE


def _prefill_heads_sorted(q, k, v, scale, causal, kv_head_map=None, row_block=512, heads=None, rows=None):
    # the requested (b, h) pairs computed in sorted order instead of the order given
    return _orig["prefill"](q, k, v, scale, causal, kv_head_map, row_block,
                            None if heads is None else sorted(heads), rows)


def _prefill_last_block_dropped(q, k, v, scale, causal, kv_head_map=None, row_block=512, heads=None, rows=None):
    # the row-block loop stops one block early when the rows do not fill whole blocks
    B, Hq, Sq, D = q.shape
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    O, LSE = _orig["prefill"](q, k, v, scale, causal, kv_head_map, row_block, heads, rows)
    cut = (len(rows) // row_block) * row_block
    if 0 < cut < len(rows):
        O[..., cut:, :] = 0.0
        LSE[..., cut:] = 0.0
    return O, LSE


def _decode_len_by_slot(q, k_pages, v_pages, page_table, seqlens, scale, k_scale=None, v_scale=None,
                        requests=None):
    # the n-th requested request read with the length of request n
    reqs = range(len(seqlens)) if requests is None else list(requests)
    mixed = np.array(seqlens, copy=True)
    for n, b in enumerate(reqs):
        mixed[b] = seqlens[n]
    return _orig["paged_decode"](q, k_pages, v_pages, page_table, mixed, scale, k_scale, v_scale, requests)


def _ragged_rows_before_mask(q_b, k_pages, v_pages, table_row, L, scale, rows=None):
    # the rows selected from q first, then masked as if they were new tokens 0..R-1
    q_b = np.asarray(q_b, dtype=np.float64)
    rows = np.arange(q_b.shape[0]) if rows is None else np.asarray(rows)
    n = q_b.shape[0]
    sub = q_b[rows]
    Hq, Hkv = q_b.shape[1], k_pages.shape[1]
    O, LSE = np.zeros((len(rows), Hq, v_pages.shape[3])), np.zeros((len(rows), Hq))
    for h in range(Hq):
        g = A.kv_head_of(h, Hq, Hkv)
        kb = A.gather_pages(k_pages, table_row, L, g)
        vb = A.gather_pages(v_pages, table_row, L, g)
        s = A.scores(sub[:, h], kb, scale)
        s = np.where(np.arange(L)[None, :] <= (L - n + np.arange(len(rows)))[:, None], s, -np.inf)
        P, m, l = A.softmax_rows(s)
        O[:, h], LSE[:, h] = P @ vb, m + np.log(l)
    return O, LSE


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
    "append_ignores_prefix": ("kv_append", _append_ignores_prefix),
    "append_prefix_from_offsets": ("kv_append", _append_prefix_from_offsets),
    "append_k_only": ("kv_append", _append_k_only),
    "ragged_top_left_mask": ("paged_prefill_request", _ragged_top_left),
    "ragged_non_causal": ("paged_prefill_request", _ragged_non_causal),
    "ragged_prefix_keys_only": ("paged_prefill", _ragged_prefix_keys_only),
    "bwd_no_rowsum": ("attention_head_backward", _bwd_variant("no_rowsum")),
    "bwd_no_scale": ("attention_head_backward", _bwd_variant("no_scale")),
    "bwd_dk_from_p": ("attention_head_backward", _bwd_variant("dk_from_p")),
    "bwd_gqa_first_head": ("prefill_backward", _bwd_gqa_first_head),
    "head_rows_reindexed": ("attention_head", _head_rows_reindexed),
    "prefill_block_positions": ("prefill", _prefill_block_positions),
    "prefill_heads_sorted": ("prefill", _prefill_heads_sorted),
    "prefill_last_block_dropped": ("prefill", _prefill_last_block_dropped),
    "decode_len_by_slot": ("paged_decode", _decode_len_by_slot),
    "ragged_rows_before_mask": ("paged_prefill_request", _ragged_rows_before_mask),
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
