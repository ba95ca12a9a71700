"""Exact attention in numpy float64 (test infrastructure; see package docstring).

The method's result is standard attention, softmax(Q K^T / sqrt(d)) V, and the
pages state that the tiled method reaches it exactly (no approximation), so
this oracle is that definition written out: it materialises each head's score
matrix, applies the ordinary row softmax and multiplies by V. It contains no
tiling, no online softmax and no split of the key axis.

Sources (titles of the pages, with the part used):
  [FIA] "FIA / FlashAttention" help-centre Q&A, section 1 (FlashAttention core
        principle: the attention formula, exactness) and section 4 (the
        causal flag of the packed-QKV call).
  [FPA] "Flash Attention & Paged Attention" blog, "FA and the decode phase"
        (Flash-Decoding: split the KV sequence, per-split partial result plus
        LogSumExp, light reduction) and "2. PagedAttention" (fixed-size pages,
        logical page table over non-contiguous physical memory).
  [CRS] "FlashAttention attention inference optimisation" course, chapter 1,
        section 1.2 (decode-time standard attention: Q [1,H,1,d], K/V
        [1,H,seq,d], scores / sqrt(head_dim), softmax, weights @ V).
  [ARC] "FlashAttention breakthrough architecture" article, "paged storage
        system" (64-token blocks behind a page table).
  [FBW] the backward pass: "Flash Attention & Paged Attention" blog,
        "1. FlashAttention" (recomputation: the backward does not keep the
        N x N matrix but recomputes the attention gradients from the small
        statistics the forward saved); "FasterTransformer vs FlashAttention",
        section 3 (recomputation trades compute for memory); "FIA /
        FlashAttention" Q&A, section 3's table (FlashAttention's backward is
        complete and needed for training).
  [FPF] "Flash Attention & Paged Attention" blog, "FA and the prefill phase"
        (prefill attends over the whole prompt and stores the computed K and V
        in device memory as the initial KV cache).

Readings where the pages leave a step open (each is stated where used):
  * LSE is the natural log of the sum of exp over the scaled, unmasked scores
    of one query row.
  * Causal masking is aligned bottom-right: key j is visible to query i iff
    j <= i + (Sk - Sq). A row with no visible key has O = 0, LSE = -inf.
  * GQA: query head h reads KV head h // (Hq / Hkv) unless a map is given.
  * fp8 KV values are OCP e4m3fn codes times a per-(page, KV head) scale.
  * A ragged prefill chunk of n new tokens for a request whose cache ends up
    L tokens long occupies logical positions L - n .. L - 1 (the new tokens
    follow the cached prefix); causal masking over its L keys is then the
    bottom-right rule above with Sq = n, Sk = L.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf
PAGE = 64


# --------------------------------------------------------------------------
# Steps of the definition, one head at a time.
# --------------------------------------------------------------------------

def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = scale * <q_i, k_j>  ([FIA] section 1 formula; [CRS] 1.2).

    ``q`` [R, D], ``k`` [Sk, D], float64. ``scale`` is the fp32 value the GPU
    receives, widened exactly.
    """
    return float(scale) * (q @ k.T)


def causal_allowed(rows: np.ndarray, Sq: int, Sk: int) -> np.ndarray:
    """Boolean [R, Sk]: key j visible to query row i iff j <= i + (Sk - Sq).

    [FIA] section 4 passes causal=True; bottom-right alignment is the reading
    for Sq != Sk (it reduces to j <= i when Sq == Sk and to "all keys" for a
    single decode query at the end of the context).
    """
    return np.arange(Sk)[None, :] <= (np.asarray(rows)[:, None] + (Sk - Sq))


def softmax_rows(s: np.ndarray):
    """Row softmax of a score block with -inf entries meaning "masked".

    Returns (P, m, l): m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i),
    P_ij = exp(s_ij - m_i) / l_i. Rows that are entirely masked get P = 0,
    m = -inf, l = 0. ([CRS] 1.2: weights = softmax(scores).)
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    empty = ~np.isfinite(m)
    shift = np.where(empty, 0.0, m)
    e = np.exp(s - shift[:, None])
    l = e.sum(axis=1)
    P = e / np.where(empty, 1.0, l)[:, None]
    return P, m, l


def attention_head(q, k, v, scale, causal=False, rows=None):
    """One head of exact attention, optionally only for some query rows.

    ``q`` [Sq, D], ``k`` [Sk, D], ``v`` [Sk, Dv] float64. Returns
    (O [R, Dv], LSE [R]) for ``rows`` (default: all Sq rows).
    O = P V ([CRS] 1.2: output = weights @ V); LSE = m + ln l.
    """
    Sq, Sk = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    s = scores(q[rows], k, scale)
    if causal:
        s = np.where(causal_allowed(rows, Sq, Sk), s, NEG_INF)
    P, m, l = softmax_rows(s)
    o = P @ v if Sk else np.zeros((len(rows), v.shape[1]))
    lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


def kv_head_of(h: int, Hq: int, Hkv: int, kv_head_map=None) -> int:
    """KV head read by query head h ([FIA] section 3: grouped-query attention).

    Default grouping is contiguous: h // (Hq / Hkv).
    """
    if kv_head_map is not None:
        return int(kv_head_map[h])
    return h // (Hq // Hkv)


# --------------------------------------------------------------------------
# Prefill: B x Hq heads of the definition.
# --------------------------------------------------------------------------

def prefill(q, k, v, scale, causal, kv_head_map=None, row_block=512, heads=None,
            rows=None):
    """Exact attention over BHSD tensors.

    q [B, Hq, Sq, D], k/v [B, Hkv, Sk, D] float64 (or anything numpy widens
    exactly). Returns O [B, Hq, R, D] and LSE [B, Hq, R] where R = Sq, or the
    given ``rows``. ``heads`` restricts to a list of (b, h) pairs, returned in
    that order as O [n, R, D], LSE [n, R]. Scores are materialised
    ``row_block`` rows at a time (memory only; every row is independent).
    """
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    O = np.zeros((len(pairs), len(rows), v.shape[3]))
    LSE = np.zeros((len(pairs), len(rows)))
    for n, (b, h) in enumerate(pairs):
        g = kv_head_of(h, Hq, Hkv, kv_head_map)
        qh = np.asarray(q[b, h], dtype=np.float64)
        kh = np.asarray(k[b, g], dtype=np.float64)
        vh = np.asarray(v[b, g], dtype=np.float64)
        for r0 in range(0, len(rows), row_block):
            rr = rows[r0:r0 + row_block]
            O[n, r0:r0 + len(rr)], LSE[n, r0:r0 + len(rr)] = attention_head(
                qh, kh, vh, scale, causal, rr)
    if heads is None:
        O = O.reshape(B, Hq, len(rows), -1)
        LSE = LSE.reshape(B, Hq, len(rows))
    return O, LSE


# --------------------------------------------------------------------------
# Decode over a paged KV cache.
# --------------------------------------------------------------------------

def e4m3fn_to_float(codes) -> np.ndarray:
    """Decode OCP 8-bit e4m3fn codes to float64 from the format's definition.

    Bit layout s eeee mmm, exponent bias 7. e = 0: subnormal m/8 * 2^-6;
    otherwise (1 + m/8) * 2^(e-7); the two codes s1111111 are NaN; there is
    no infinity (max finite 448). The pages name FP8 KV kernels ([FIA]
    section 3) without the format; e4m3fn is the reading because a scale of
    max|x|/448 maps the largest value onto this format's largest finite value.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def gather_pages(pool, table_row, L: int, g: int, scale=None):
    """Logical token sequence of one request and KV head from a paged pool.

    ``pool`` [P, Hkv, 64, D] (float values, or uint8 e4m3fn codes when
    ``scale`` [P, Hkv] is given). Logical page j of the request is physical
    page ``table_row[j]`` ([FPA] "2. PagedAttention": fixed-size pages and a
    logical-to-physical table; [ARC]: 64-token blocks). Returns [L, D] float64,
    the pages concatenated in logical order and cut to L tokens.
    """
    n = (L + PAGE - 1) // PAGE
    if n == 0:
        return np.zeros((0, pool.shape[3]))
    ids = np.asarray(table_row[:n], dtype=np.int64)
    blocks = np.asarray(pool[ids, g])  # [n, 64, D]
    if scale is not None:
        vals = e4m3fn_to_float(blocks) * np.asarray(scale, dtype=np.float64)[ids, g][:, None, None]
    else:
        vals = blocks.astype(np.float64)
    return vals.reshape(n * PAGE, -1)[:L]


def paged_decode(q, k_pages, v_pages, page_table, seqlens, scale,
                 k_scale=None, v_scale=None, requests=None):
    """Single-token decode attention against each request's whole cache.

    q [B, Hq, D]; pools [P, Hkv, 64, D]; page_table [B, max_pages]; seqlens [B].
    For each request b and query head h: gather the L_b cached tokens of KV
    head g(h), then one query row of exact attention over all of them, no mask
    ([CRS] 1.2: the current query sees the whole cache). Returns O [B, Hq, D],
    LSE [B, Hq] (or [n, Hq, D] / [n, Hq] for ``requests``).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    reqs = range(B) if requests is None else list(requests)
    O = np.zeros((len(reqs), Hq, v_pages.shape[3]))
    LSE = np.zeros((len(reqs), Hq))
    for n, b in enumerate(reqs):
        L = int(seqlens[b])
        for g in range(Hkv):
            kb = gather_pages(k_pages, page_table[b], L, g, k_scale)
            vb = gather_pages(v_pages, page_table[b], L, g, v_scale)
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) != g:
                    continue
                o, lse = attention_head(q[b, h][None, :], kb, vb, scale, False)
                O[n, h], LSE[n, h] = o[0], lse[0]
    return O, LSE


def lse_merge(partial_o, partial_lse):
    """Merge per-split attention results by their LogSumExp ([FPA] Flash-Decoding).

    Split s holds O_s (normalised over its own keys) and lse_s. The exact
    result over the union of the splits is lse = ln sum_s exp(lse_s) and
    O = sum_s exp(lse_s - lse) O_s. Splits with lse_s = -inf (no keys) weigh 0;
    if every split is empty the result is O = 0, lse = -inf.
    ``partial_o`` [n, D], ``partial_lse`` [n].
    """
    lse_s = np.asarray(partial_lse, dtype=np.float64)
    o_s = np.asarray(partial_o, dtype=np.float64)
    finite = np.isfinite(lse_s)
    if not finite.any():
        return np.zeros(o_s.shape[1]), NEG_INF
    mx = lse_s[finite].max()
    w = np.where(finite, np.exp(np.where(finite, lse_s, 0.0) - mx), 0.0)
    tot = w.sum()
    lse = mx + np.log(tot)
    o = (w / tot) @ o_s
    return o, lse


# --------------------------------------------------------------------------
# Ragged prefill over paged KV caches, and the KV append that precedes it.
# --------------------------------------------------------------------------

def kv_append(k_pages, v_pages, page_table, seqlens, cu_seqlens_q, k_new, v_new):
    """Store each request's new tokens' K/V in its pages ([FPF]; [FPA] "2. PagedAttention").

    Request b owns the packed new tokens cu[b] .. cu[b+1]-1; with n_b of them
    and a final length L_b, new token i sits at logical position
    t = L_b - n_b + i, i.e. slot t mod 64 of physical page table[b, t // 64].
    ``k_new`` / ``v_new`` [T, Hkv, D]. Returns copies of the pools with those
    slots overwritten and every other element unchanged. Pure data movement:
    any element type works (pass raw bit patterns for a bitwise check).
    """
    kp, vp = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    cu = np.asarray(cu_seqlens_q)
    for b in range(len(seqlens)):
        L, n = int(seqlens[b]), int(cu[b + 1] - cu[b])
        for i in range(n):
            t = L - n + i
            pid = int(page_table[b][t // PAGE])
            kp[pid, :, t % PAGE, :] = k_new[cu[b] + i]
            vp[pid, :, t % PAGE, :] = v_new[cu[b] + i]
    return kp, vp


def paged_prefill_request(q_b, k_pages, v_pages, table_row, L: int, scale, rows=None):
    """Causal attention of one request's new tokens over its whole paged cache.

    ``q_b`` [n, Hq, D]: the request's new tokens, the last n of its L
    positions. Each KV head's L tokens are gathered in logical order, then
    every query head runs the definition with the bottom-right causal mask
    (Sq = n, Sk = L), so new token i sees keys 0 .. L - n + i. Returns
    O [R, Hq, D] and LSE [R, Hq] for ``rows`` (default all n).
    """
    q_b = np.asarray(q_b, dtype=np.float64)
    n, Hq, _ = q_b.shape
    Hkv = k_pages.shape[1]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    O = np.zeros((len(rows), Hq, v_pages.shape[3]))
    LSE = np.zeros((len(rows), Hq))
    if len(rows) == 0:
        return O, LSE
    for g in range(Hkv):
        kb = gather_pages(k_pages, table_row, L, g)
        vb = gather_pages(v_pages, table_row, L, g)
        for h in range(Hq):
            if kv_head_of(h, Hq, Hkv) != g:
                continue
            O[:, h], LSE[:, h] = attention_head(q_b[:, h], kb, vb, scale, True, rows)
    return O, LSE


def paged_prefill(q, k_pages, v_pages, page_table, seqlens, cu_seqlens_q, scale):
    """Ragged causal prefill of a packed batch against paged caches.

    q [T, Hq, D] packed by request (cu_seqlens_q [B+1]); pools [P, Hkv, 64, D]
    already holding every request's L_b tokens, new ones included. Returns
    O [T, Hq, D], LSE [T, Hq] ([FPF]: prefill over the whole sequence; [FIA]
    section 2: variable-length batches over paged KV).
    """
    q = np.asarray(q)
    cu = np.asarray(cu_seqlens_q)
    O = np.zeros((q.shape[0], q.shape[1], v_pages.shape[3]))
    LSE = np.zeros((q.shape[0], q.shape[1]))
    for b in range(len(seqlens)):
        s, e = int(cu[b]), int(cu[b + 1])
        O[s:e], LSE[s:e] = paged_prefill_request(q[s:e], k_pages, v_pages, page_table[b],
                                                 int(seqlens[b]), scale)
    return O, LSE


# --------------------------------------------------------------------------
# Backward: gradients of O = softmax(scale Q K^T) V with respect to Q, K, V.
# --------------------------------------------------------------------------

def attention_head_backward(q, k, v, do, scale, causal=False):
    """Gradients of one head ([FBW]) by the chain rule on the definition.

    With P the row softmax of the (masked) scores and O = P V, for an upstream
    gradient dO:  dV = P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(dO * O))
    (the softmax Jacobian applied row by row);  dQ = scale dS K;
    dK = scale dS^T Q. Masked entries have P = 0 and so no gradient. Rows with
    no visible key contribute nothing. All float64. Returns (dQ, dK, dV).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    Sq, Sk = q.shape[0], k.shape[0]
    s = scores(q, k, scale)
    if causal:
        s = np.where(causal_allowed(np.arange(Sq), Sq, Sk), s, NEG_INF)
    P, _, _ = softmax_rows(s)
    o = P @ v
    dv = P.T @ do
    dp = do @ v.T
    Di = np.sum(do * o, axis=1)
    ds = P * (dp - Di[:, None])
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def prefill_backward(q, k, v, do, scale, causal):
    """Gradients over BHSD tensors: dQ [B, Hq, Sq, D], dK/dV [B, Hkv, Sk, D].

    Query head h reads KV head h // (Hq / Hkv); a KV head's gradient is the sum
    over the query heads that read it.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dq = np.zeros((B, Hq, Sq, D))
    dk = np.zeros((B, Hkv, Sk, D))
    dv = np.zeros((B, Hkv, Sk, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            a, bb, c = attention_head_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[b, h] = a
            dk[b, g] += bb
            dv[b, g] += c
    return dq, dk, dv
