"""Pins that tie the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, an invariant of exact attention, a hand-derived worked example
(``tests/golden/hand_examples.json``), brute force on tiny inputs or a library
routine that computes the same quantity. The functions look up the oracle's
steps through the module object at call time, so ``test_oracle_mutations``
can plant a mistake in one step and check that some pin fails.

Tolerances: closed forms and identities hold to ~1e-12 in fp64; "bitwise"
pins compare exact equality.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "inf": math.inf,
                                                   "nan": math.nan}))


def _arr(rows):
    return np.array([[_ev(x) for x in r] for r in rows], dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    assert err.max(initial=0.0) <= tol, f"{what}: max err {err.max():.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_golden_attention():
    """Hand-derived worked examples (closed forms) for attention rows."""
    for ex in json.load(open(GOLDEN))["attention"]:
        q, k, v = _arr(ex["q"]), _arr(ex["k"]), _arr(ex["v"])
        o, lse = A.attention_head(q, k, v, _ev(ex["scale"]), ex["causal"])
        _close(o, _arr(ex["o"]), 1e-12, ex["name"] + " O")
        _close(lse, [_ev(x) for x in ex["lse"]], 1e-12, ex["name"] + " LSE")
        # the same example through the batched prefill entry
        O, L = A.prefill(q[None, None], k[None, None], v[None, None], _ev(ex["scale"]), ex["causal"])
        _close(O[0, 0], _arr(ex["o"]), 1e-12, ex["name"] + " prefill O")
        _close(L[0, 0], [_ev(x) for x in ex["lse"]], 1e-12, ex["name"] + " prefill LSE")


def pin_golden_merge():
    for ex in json.load(open(GOLDEN))["lse_merge"]:
        o, lse = A.lse_merge(_arr(ex["partial_o"]), [_ev(x) for x in ex["partial_lse"]])
        _close(o, [_ev(x) for x in ex["o"]], 1e-12, ex["name"] + " O")
        _close(lse, _ev(ex["lse"]), 1e-12, ex["name"] + " LSE")


def pin_golden_e4m3fn():
    codes = json.load(open(GOLDEN))["e4m3fn"]["codes"]
    for c, expr in codes.items():
        got = float(A.e4m3fn_to_float(np.array([int(c)], dtype=np.uint8))[0])
        want = _ev(expr)
        if math.isnan(want):
            assert math.isnan(got), f"code {c}: {got} is not NaN"
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), \
                f"code {c}: {got} != {want}"


def pin_golden_gather():
    ex = json.load(open(GOLDEN))["paged_gather"]
    P = ex["num_pages"]
    pool = (100.0 * np.arange(P)[:, None] + np.arange(64)[None, :])[:, None, :, None]  # [P,1,64,1]
    got = A.gather_pages(pool, np.array(ex["table"]), ex["L"], 0)[:, 0]
    assert got.shape == (ex["L"],)
    assert list(got[:3]) == ex["expected_first"]
    assert got[63] == ex["expected_at_63"]
    assert list(got[64:]) == ex["expected_tail"]


def pin_identical_keys():
    """All keys equal -> uniform weights -> O = mean(V) (causal: prefix mean)."""
    g = _rng(1)
    Sq = Sk = 9
    q = g.standard_normal((Sq, 5))
    k = np.repeat(g.standard_normal((1, 5)), Sk, axis=0)
    v = g.standard_normal((Sk, 3))
    o, lse = A.attention_head(q, k, v, 0.7, False)
    _close(o, np.repeat(v.mean(axis=0, keepdims=True), Sq, axis=0), 1e-12, "identical keys")
    s0 = 0.7 * q @ k[0]
    _close(lse, s0 + math.log(Sk), 1e-12, "identical keys LSE")
    o, lse = A.attention_head(q, k, v, 0.7, True)
    pref = np.cumsum(v, axis=0) / np.arange(1, Sk + 1)[:, None]
    _close(o, pref, 1e-12, "identical keys causal")
    _close(lse, s0 + np.log(np.arange(1, Sk + 1)), 1e-12, "identical keys causal LSE")


def pin_dominant_score():
    """One key far ahead of the rest (gap >= 60 in the exponent) -> O = that V row."""
    g = _rng(2)
    D, Sk = 8, 20
    q = g.standard_normal((1, D))
    k = g.standard_normal((Sk, D)) * 0.1
    j = 13
    k[j] = 200.0 * q[0] / np.linalg.norm(q[0])
    v = g.standard_normal((Sk, 4))
    o, lse = A.attention_head(q, k, v, 1.0, False)
    gap = float(q[0] @ k[j]) - max(float(q[0] @ k[i]) for i in range(Sk) if i != j)
    assert gap > 60
    _close(o[0], v[j], 1e-12, "dominant score")
    _close(lse[0], float(q[0] @ k[j]), 1e-12, "dominant LSE")


def pin_single_key():
    g = _rng(3)
    q, k, v = g.standard_normal((4, 6)), g.standard_normal((1, 6)), g.standard_normal((1, 6))
    o, lse = A.attention_head(q, k, v, 0.3, False)
    _close(o, np.repeat(v, 4, axis=0), 0.0, "single key O")
    _close(lse, 0.3 * (q @ k[0]), 1e-12, "single key LSE")


def pin_causal_row0():
    g = _rng(4)
    q, k, v = g.standard_normal((7, 6)), g.standard_normal((7, 6)), g.standard_normal((7, 6))
    o, lse = A.attention_head(q, k, v, 0.5, True)
    _close(o[0], v[0], 0.0, "causal row 0")
    _close(lse[0], 0.5 * float(q[0] @ k[0]), 1e-12, "causal row 0 LSE")


def pin_empty_rows():
    """Causal with Sq > Sk: rows with no visible key are O = 0, LSE = -inf (reading)."""
    g = _rng(5)
    q, k, v = g.standard_normal((5, 4)), g.standard_normal((3, 4)), g.standard_normal((3, 4))
    o, lse = A.attention_head(q, k, v, 1.0, True)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    _close(o[2], v[0], 0.0, "first visible row")
    o, lse = A.attention_head(q, k[:0], v[:0], 1.0, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# Brute force
# --------------------------------------------------------------------------

def _brute(q, k, v, scale, causal):
    """Pure-Python triple loops, math.fsum / math.exp: the textbook formula."""
    Sq, Sk, D = len(q), len(k), len(q[0])
    O, L = [], []
    for i in range(Sq):
        s = []
        for j in range(Sk):
            if causal and j > i + (Sk - Sq):
                continue
            s.append((j, scale * math.fsum(q[i][d] * k[j][d] for d in range(D))))
        if not s:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        mx = max(x for _, x in s)
        w = [(j, math.exp(x - mx)) for j, x in s]
        tot = math.fsum(x for _, x in w)
        O.append([math.fsum(x * v[j][d] for j, x in w) / tot for d in range(len(v[0]))])
        L.append(mx + math.log(tot))
    return np.array(O), np.array(L)


def pin_brute_force():
    g = _rng(6)
    for Sq, Sk, D, causal in [(1, 1, 1, False), (3, 5, 2, False), (5, 5, 4, True),
                              (4, 7, 3, True), (8, 8, 4, False), (6, 3, 4, True)]:
        q, k, v = g.standard_normal((Sq, D)), g.standard_normal((Sk, D)), g.standard_normal((Sk, D))
        o, lse = A.attention_head(q, k, v, 0.8, causal)
        bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.8, causal)
        _close(o, bo, 1e-13, f"brute O {Sq}x{Sk}")
        _close(lse, bl, 1e-13, f"brute LSE {Sq}x{Sk}")


# --------------------------------------------------------------------------
# Subsets of rows, heads and requests, and the row-block loop. The full-size
# parity checks and the CPU baseline compute only some rows, heads or
# requests, so these paths are pinned on their own: against brute force read
# slot by slot, against the full call, and against a library routine.
# --------------------------------------------------------------------------

def pin_subset_rows_brute_force():
    """attention_head(rows=R) on a head with Sq != Sk equals brute force on
    those rows (R unsorted, both ends, one row twice) and rows R of the full call."""
    g = _rng(40)
    Sq, Sk, D = 13, 21, 3
    q, k, v = g.standard_normal((Sq, D)), g.standard_normal((Sk, D)), g.standard_normal((Sk, D))
    R = np.array([12, 0, 7, 3, 7, 1])
    for causal in (False, True):
        bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
        so, sl = A.attention_head(q, k, v, 0.6, causal, rows=R)
        _close(so, bo[R], 1e-13, f"rows subset vs brute O causal={causal}")
        _close(sl, bl[R], 1e-13, f"rows subset vs brute LSE causal={causal}")
        fo, fl = A.attention_head(q, k, v, 0.6, causal)
        _close(so, fo[R], 1e-13, f"rows subset vs full O causal={causal}")
        _close(sl, fl[R], 1e-13, f"rows subset vs full LSE causal={causal}")


def pin_subset_heads_rows_prefill():
    """prefill(heads=H, rows=R) equals the full prefill at those (b, h) and
    rows, for an unsorted head list across batches and GQA groups, unsorted
    rows, and a row block much smaller than the rows asked for (the block
    loop runs several times and its last block is ragged); the whole tensor
    computed in small row blocks equals the one-block result."""
    g = _rng(41)
    B, Hq, Hkv, Sq, Sk, D = 2, 6, 2, 45, 60, 4
    q = g.standard_normal((B, Hq, Sq, D))
    k = g.standard_normal((B, Hkv, Sk, D))
    v = g.standard_normal((B, Hkv, Sk, D))
    H = [(1, 5), (0, 0), (1, 2), (0, 3)]
    R = g.permutation(Sq)[:31]
    for causal in (False, True):
        fo, fl = A.prefill(q, k, v, 0.5, causal)
        so, sl = A.prefill(q, k, v, 0.5, causal, row_block=7, heads=H, rows=R)
        assert so.shape == (len(H), len(R), D) and sl.shape == (len(H), len(R))
        for n, (b, h) in enumerate(H):
            _close(so[n], fo[b, h][R], 1e-13, f"head subset O {b},{h} causal={causal}")
            _close(sl[n], fl[b, h][R], 1e-13, f"head subset LSE {b},{h} causal={causal}")
        bo, bl = A.prefill(q, k, v, 0.5, causal, row_block=4)
        _close(bo, fo, 1e-13, f"row blocks of 4 O causal={causal}")
        _close(bl, fl, 1e-13, f"row blocks of 4 LSE causal={causal}")
    # one subset head against brute force, so the comparison is not only oracle vs oracle
    b, h = H[0]
    bo, bl = _brute(q[b, h].tolist(), k[b, h // 3].tolist(), v[b, h // 3].tolist(), 0.5, True)
    so, sl = A.prefill(q, k, v, 0.5, True, row_block=7, heads=[(b, h)], rows=R)
    _close(so[0], bo[R], 1e-13, "head subset vs brute O")
    _close(sl[0], bl[R], 1e-13, "head subset vs brute LSE")


def pin_row_blocks_torch_sdpa():
    """S = 1100 rows, more than the default row block (512) and many times a
    small one (64): O equals torch's scaled_dot_product_attention and LSE
    equals torch.logsumexp, in float64, causal and not."""
    g = _rng(42)
    B, Hq, Hkv, S, D = 1, 2, 1, 1100, 8
    q = g.standard_normal((B, Hq, S, D))
    k = g.standard_normal((B, Hkv, S, D))
    v = g.standard_normal((B, Hkv, S, D))
    tq = torch.from_numpy(q)
    ke = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    ve = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, is_causal=causal, scale=0.3).numpy()
        s = 0.3 * tq @ ke.transpose(2, 3)
        if causal:
            s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
        ref_lse = torch.logsumexp(s, dim=3).numpy()
        for row_block in (512, 64):
            O, LSE = A.prefill(q, k, v, 0.3, causal, row_block=row_block)
            _close(O, ref, 1e-12, f"sdpa S=1100 block {row_block} causal={causal}")
            _close(LSE, ref_lse, 1e-12, f"logsumexp S=1100 block {row_block} causal={causal}")


def pin_subset_requests_decode():
    """paged_decode(requests=S) for an unsorted subset equals brute force over
    each request's tokens read slot by slot through the table, and those
    requests of the full call."""
    g = _rng(43)
    B, Hq, Hkv, D = 4, 4, 2, 3
    L = np.array([70, 1, 129, 64])
    n = (L + 63) // 64
    P = int(n.sum()) + 1
    perm = g.permutation(P)
    table = np.full((B, 3), -1)
    off = 0
    for b in range(B):
        table[b, :n[b]] = perm[off:off + n[b]]
        off += n[b]
    kp, vp = g.standard_normal((P, Hkv, 64, D)), g.standard_normal((P, Hkv, 64, D))
    q = g.standard_normal((B, Hq, D))
    S = [2, 0, 3]
    so, sl = A.paged_decode(q, kp, vp, table, L, 0.55, requests=S)
    fo, fl = A.paged_decode(q, kp, vp, table, L, 0.55)
    assert so.shape == (len(S), Hq, D)
    for i, b in enumerate(S):
        _close(so[i], fo[b], 1e-13, f"request subset O b={b}")
        _close(sl[i], fl[b], 1e-13, f"request subset LSE b={b}")
        for h in range(Hq):
            gg = h * Hkv // Hq
            ks = [kp[table[b][t // 64], gg, t % 64].tolist() for t in range(L[b])]
            vs = [vp[table[b][t // 64], gg, t % 64].tolist() for t in range(L[b])]
            bo, bl = _brute([q[b, h].tolist()], ks, vs, 0.55, False)
            _close(so[i, h], bo[0], 1e-13, f"request subset vs brute O b={b} h={h}")
            _close(sl[i, h], bl[0], 1e-13, f"request subset vs brute LSE b={b} h={h}")


def pin_subset_rows_paged_prefill():
    """paged_prefill_request(rows=R) equals rows R of the hand-indexed brute
    force and of the full call (R unsorted, first and last new token)."""
    Hq, Hkv, D = 4, 2, 3
    nq, pre = [9, 70], [66, 3]
    q, kn, vn, kp, vp, table, L, cu = _ragged_case(44, Hq, Hkv, D, nq, pre)
    kp, vp = A.kv_append(kp, vp, table, L, cu, kn, vn)
    bo, bl = _brute_ragged(q, kp, vp, table, L, cu, 0.65, Hkv)
    for b, R in ((0, np.array([8, 0, 4])), (1, np.array([69, 2, 0, 63, 64]))):
        s, e = int(cu[b]), int(cu[b + 1])
        so, sl = A.paged_prefill_request(q[s:e], kp, vp, table[b], int(L[b]), 0.65, rows=R)
        fo, fl = A.paged_prefill_request(q[s:e], kp, vp, table[b], int(L[b]), 0.65)
        _close(so, bo[s:e][R], 1e-13, f"paged rows subset vs brute O b={b}")
        _close(sl, bl[s:e][R], 1e-13, f"paged rows subset vs brute LSE b={b}")
        _close(so, fo[R], 1e-13, f"paged rows subset vs full O b={b}")
        _close(sl, fl[R], 1e-13, f"paged rows subset vs full LSE b={b}")


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_causal_dependency():
    """Perturbing K/V at positions j > i leaves causal row i bit-identical."""
    g = _rng(7)
    S, D = 16, 8
    q, k, v = g.standard_normal((S, D)), g.standard_normal((S, D)), g.standard_normal((S, D))
    o, lse = A.attention_head(q, k, v, 0.4, True)
    for i in (0, 5, 11):
        k2, v2 = k.copy(), v.copy()
        k2[i + 1:] += g.standard_normal((S - i - 1, D)) * 3
        v2[i + 1:] += g.standard_normal((S - i - 1, D)) * 3
        o2, lse2 = A.attention_head(q, k2, v2, 0.4, True)
        assert np.array_equal(o2[i], o[i]) and lse2[i] == lse[i], f"row {i} changed"
        assert not np.array_equal(o2[i + 1:], o[i + 1:]), "later rows must change"


def pin_shift_invariance():
    """k_j -> k_j + u for all j: O unchanged, LSE shifts by scale * q.u."""
    g = _rng(8)
    q, k, v = g.standard_normal((6, 5)), g.standard_normal((9, 5)), g.standard_normal((9, 5))
    u = g.standard_normal(5)
    o, lse = A.attention_head(q, k, v, 0.6, False)
    o2, lse2 = A.attention_head(q, k + u, v, 0.6, False)
    _close(o2, o, 1e-12, "shift O")
    _close(lse2, lse + 0.6 * (q @ u), 1e-12, "shift LSE")


def pin_key_permutation():
    g = _rng(9)
    q, k, v = g.standard_normal((6, 5)), g.standard_normal((9, 5)), g.standard_normal((9, 3))
    p = g.permutation(9)
    o, lse = A.attention_head(q, k, v, 0.6, False)
    o2, lse2 = A.attention_head(q, k[p], v[p], 0.6, False)
    _close(o2, o, 1e-12, "perm O")
    _close(lse2, lse, 1e-12, "perm LSE")


def pin_convex_hull():
    g = _rng(10)
    q, k, v = g.standard_normal((12, 4)) * 3, g.standard_normal((12, 4)), g.standard_normal((12, 6))
    o, _ = A.attention_head(q, k, v, 1.0, True)
    for i in range(12):
        lo, hi = v[:i + 1].min(axis=0), v[:i + 1].max(axis=0)
        assert np.all(o[i] >= lo - 1e-12) and np.all(o[i] <= hi + 1e-12), f"row {i} outside hull"


def pin_gqa_expansion():
    """GQA equals MHA on K/V repeated per group; an explicit map is honoured."""
    g = _rng(11)
    B, Hq, Hkv, S, D = 2, 6, 2, 10, 4
    q = g.standard_normal((B, Hq, S, D))
    k = g.standard_normal((B, Hkv, S, D))
    v = g.standard_normal((B, Hkv, S, D))
    O, L = A.prefill(q, k, v, 0.5, True)
    ke, ve = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    O2, L2 = A.prefill(q, ke, ve, 0.5, True)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    hmap = [1, 0, 1, 1, 0, 0]
    O3, _ = A.prefill(q, k, v, 0.5, True, kv_head_map=hmap)
    O4, _ = A.prefill(q, k[:, hmap], v[:, hmap], 0.5, True, kv_head_map=list(range(Hq)))
    assert np.array_equal(O3, O4)


def pin_lse_merge_identity():
    """Splitting the keys into chunks and merging by LSE equals the unsplit result."""
    g = _rng(12)
    q, k, v = g.standard_normal((3, 8)), g.standard_normal((50, 8)), g.standard_normal((50, 8))
    o, lse = A.attention_head(q, k, v, 0.35, False)
    for cuts in ([10, 11, 30], [0, 25], [49], [7, 7, 7, 40]):
        edges = [0] + list(cuts) + [50]
        for i in range(3):
            parts = [A.attention_head(q[i:i + 1], k[a:b], v[a:b], 0.35, False)
                     for a, b in zip(edges[:-1], edges[1:])]
            mo, ml = A.lse_merge(np.array([p[0][0] for p in parts]), np.array([p[1][0] for p in parts]))
            _close(mo, o[i], 1e-12, f"merge O {cuts}")
            _close(ml, lse[i], 1e-12, f"merge LSE {cuts}")


def pin_paged_equals_contiguous():
    """A randomly permuted paged pool gives results bit-identical to the contiguous layout."""
    g = _rng(13)
    B, Hq, Hkv, D = 3, 4, 2, 8
    L = np.array([1, 130, 64])
    n = (L + 63) // 64
    P = int(n.sum())
    perm = g.permutation(P)
    table = np.full((B, 4), -1)
    contig_k = [g.standard_normal((Hkv, n[b] * 64, D)) for b in range(B)]
    contig_v = [g.standard_normal((Hkv, n[b] * 64, D)) for b in range(B)]
    kp = np.full((P, Hkv, 64, D), np.nan)
    vp = np.full((P, Hkv, 64, D), np.nan)
    off = 0
    for b in range(B):
        for j in range(n[b]):
            pid = perm[off + j]
            table[b, j] = pid
            kp[pid] = contig_k[b][:, 64 * j:64 * j + 64]
            vp[pid] = contig_v[b][:, 64 * j:64 * j + 64]
            if 64 * (j + 1) > L[b]:  # tail beyond the request stays NaN in the pool
                t = L[b] - 64 * j
                kp[pid][:, t:] = np.nan
                vp[pid][:, t:] = np.nan
        off += n[b]
    q = g.standard_normal((B, Hq, D))
    O, LSE = A.paged_decode(q, kp, vp, table, L, 0.3)
    for b in range(B):
        for h in range(Hq):
            gg = h // (Hq // Hkv)
            o, lse = A.attention_head(q[b, h][None], contig_k[b][gg, :L[b]], contig_v[b][gg, :L[b]], 0.3)
            assert np.array_equal(O[b, h], o[0]) and LSE[b, h] == lse[0], f"paged != contiguous ({b},{h})"


# --------------------------------------------------------------------------
# Library routines computing the same quantity
# --------------------------------------------------------------------------

def pin_torch_sdpa():
    """O equals torch's CPU scaled_dot_product_attention in float64 (square shapes)."""
    g = _rng(14)
    B, Hq, Hkv, S, D = 2, 4, 2, 33, 16
    q = g.standard_normal((B, Hq, S, D))
    k = g.standard_normal((B, Hkv, S, D))
    v = g.standard_normal((B, Hkv, S, D))
    for causal in (False, True):
        O, _ = A.prefill(q, k, v, 0.21, causal)
        ke = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
        ve = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), ke, ve, is_causal=causal, scale=0.21).numpy()
        _close(O, ref, 1e-12, f"sdpa causal={causal}")


def pin_torch_logsumexp():
    """LSE equals torch.logsumexp of torch-computed scaled scores (masked entries dropped)."""
    g = _rng(15)
    Sq, Sk, D = 6, 11, 8
    q, k, v = g.standard_normal((Sq, D)), g.standard_normal((Sk, D)), g.standard_normal((Sk, D))
    for causal in (False, True):
        _, lse = A.attention_head(q, k, v, 0.9, causal)
        s = 0.9 * torch.from_numpy(q) @ torch.from_numpy(k).T
        if causal:
            keep = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + (Sk - Sq)
            s = s.masked_fill(~keep, float("-inf"))
        _close(lse, torch.logsumexp(s, dim=1).numpy(), 1e-12, f"logsumexp causal={causal}")


def pin_e4m3fn_vs_torch():
    """All 256 e4m3fn codes decode like torch's float8_e4m3fn -> float32 cast."""
    codes = np.arange(256, dtype=np.uint8)
    mine = A.e4m3fn_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def pin_fp8_paged_dequant():
    """The fp8 paged gather equals torch's dequantisation codes.float() * scale."""
    g = _rng(16)
    P, Hkv, D = 5, 2, 8
    codes = g.integers(0, 256, size=(P, Hkv, 64, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes in this check
    scale = g.uniform(0.01, 2.0, size=(P, Hkv)).astype(np.float32)
    table = np.array([3, 0, 4])
    L = 150
    for gg in range(Hkv):
        got = A.gather_pages(codes, table, L, gg, scale)
        t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
        ref = (t[table, gg] * torch.from_numpy(scale).double()[table, gg][:, None, None]).reshape(-1, D)[:L]
        _close(got, ref.numpy(), 0.0, f"fp8 gather head {gg}")


# --------------------------------------------------------------------------
# Ragged prefill over pages, and the KV append
# --------------------------------------------------------------------------

def _ragged_case(seed, Hq, Hkv, D, nq, pre, stride=None, fill=np.nan):
    """Tiny ragged batch: pools hold random prefixes, new-token slots ``fill``."""
    g = _rng(seed)
    nq, pre = np.asarray(nq), np.asarray(pre)
    L = pre + nq
    n_pages = (L + 63) // 64
    P = int(n_pages.sum()) + 2  # two pages nobody references
    perm = g.permutation(P)
    table = np.full((len(L), stride or max(int(n_pages.max()), 1)), -1)
    kp = g.standard_normal((P, Hkv, 64, D))
    vp = g.standard_normal((P, Hkv, 64, D))
    off = 0
    for b in range(len(L)):
        table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
        for t in range(pre[b], n_pages[b] * 64):  # new slots and the tail
            kp[table[b, t // 64], :, t % 64] = fill
            vp[table[b, t // 64], :, t % 64] = fill
    cu = np.concatenate([[0], np.cumsum(nq)])
    T = int(cu[-1])
    q = g.standard_normal((T, Hq, D))
    kn = g.standard_normal((T, Hkv, D))
    vn = g.standard_normal((T, Hkv, D))
    return q, kn, vn, kp, vp, table, L, cu


def pin_kv_append_layout():
    """Append writes new token i of request b at position prefix_b + i, bit for bit.

    The expected pool is built the other way round: each request's full
    logical sequence (prefix read from the pool by hand, then its new rows)
    is laid out page by page through the table; slots no request covers,
    and the tails of last pages, must keep their old bits.
    """
    Hkv, D = 2, 3
    nq, pre = [5, 0, 70, 64, 1], [0, 9, 60, 128, 63]
    q, kn, vn, kp, vp, table, L, cu = _ragged_case(20, 2, Hkv, D, nq, pre, fill=-7.0)
    # integer-valued, distinct contents so any misplaced copy shows
    kn = np.arange(kn.size, dtype=np.float64).reshape(kn.shape) + 1000.0
    vn = -kn
    got_k, got_v = A.kv_append(kp, vp, table, L, cu, kn, vn)
    exp_k, exp_v = kp.copy(), vp.copy()
    for b in range(len(L)):
        seq_k = [kp[table[b, t // 64], :, t % 64] for t in range(pre[b])] + list(kn[cu[b]:cu[b + 1]])
        seq_v = [vp[table[b, t // 64], :, t % 64] for t in range(pre[b])] + list(vn[cu[b]:cu[b + 1]])
        assert len(seq_k) == L[b]
        for t in range(L[b]):
            exp_k[table[b, t // 64], :, t % 64] = seq_k[t]
            exp_v[table[b, t // 64], :, t % 64] = seq_v[t]
    assert np.array_equal(got_k, exp_k) and np.array_equal(got_v, exp_v), "kv_append layout"
    assert not np.shares_memory(got_k, kp), "kv_append must not modify its input"


def _brute_ragged(q, kp, vp, table, L, cu, scale, Hkv):
    """Pure-Python loops: each new token against its request's keys 0 .. its own position."""
    T, Hq, D = q.shape
    O, LSE = np.zeros((T, Hq, vp.shape[3])), np.zeros((T, Hq))
    for b in range(len(L)):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            pos = int(L[b]) - n + i
            for h in range(Hq):
                g = h * Hkv // Hq
                ks = [kp[table[b][j // 64], g, j % 64].tolist() for j in range(pos + 1)]
                vs = [vp[table[b][j // 64], g, j % 64].tolist() for j in range(pos + 1)]
                qi = q[cu[b] + i, h].tolist()
                s = [scale * math.fsum(a * c for a, c in zip(qi, kj)) for kj in ks]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                O[cu[b] + i, h] = [math.fsum(w[j] * vs[j][d] for j in range(len(w))) / tot
                                   for d in range(len(vs[0]))]
                LSE[cu[b] + i, h] = mx + math.log(tot)
    return O, LSE


def pin_paged_prefill_brute_force():
    """Ragged paged prefill equals hand-indexed brute force on a tiny batch."""
    Hq, Hkv, D = 4, 2, 3
    nq, pre = [3, 0, 2, 66, 1], [0, 5, 62, 1, 64]
    q, kn, vn, kp, vp, table, L, cu = _ragged_case(21, Hq, Hkv, D, nq, pre, stride=3)
    kp, vp = A.kv_append(kp, vp, table, L, cu, kn, vn)
    O, LSE = A.paged_prefill(q, kp, vp, table, L, cu, 0.7)
    bo, bl = _brute_ragged(q, kp, vp, table, L, cu, 0.7, Hkv)
    _close(O, bo, 1e-13, "ragged brute O")
    _close(LSE, bl, 1e-13, "ragged brute LSE")


def pin_paged_prefill_torch_sdpa():
    """Each request equals torch SDPA (fp64) on its gathered cache with an explicit position mask."""
    Hq, Hkv, D = 4, 1, 8
    nq, pre = [40, 100, 1], [90, 0, 200]
    q, kn, vn, kp, vp, table, L, cu = _ragged_case(22, Hq, Hkv, D, nq, pre)
    kp, vp = A.kv_append(kp, vp, table, L, cu, kn, vn)
    O, LSE = A.paged_prefill(q, kp, vp, table, L, cu, 0.25)
    tk, tv = torch.from_numpy(kp), torch.from_numpy(vp)
    for b in range(len(L)):
        n, Lb = int(nq[b]), int(L[b])
        ids = torch.from_numpy(table[b, :(Lb + 63) // 64].astype(np.int64))
        kb = tk[ids].permute(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :Lb]  # [Hkv, L, D]
        vb = tv[ids].permute(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :Lb]
        qb = torch.from_numpy(q[cu[b]:cu[b + 1]]).permute(1, 0, 2)     # [Hq, n, D]
        keep = torch.arange(Lb)[None, :] <= (Lb - n + torch.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb, kb.expand(Hq, -1, -1), vb.expand(Hq, -1, -1), attn_mask=keep, scale=0.25)
        _close(O[cu[b]:cu[b + 1]], ref.permute(1, 0, 2).numpy(), 1e-12, f"ragged sdpa O b={b}")
        s = 0.25 * qb @ kb.expand(Hq, -1, -1).transpose(1, 2)
        lse = torch.logsumexp(s.masked_fill(~keep, float("-inf")), dim=2).T
        _close(LSE[cu[b]:cu[b + 1]], lse.numpy(), 1e-12, f"ragged logsumexp b={b}")


def pin_paged_prefill_reductions():
    """Special cases: no prefix == causal prefill; the last new token == paged decode."""
    Hq, Hkv, D = 4, 2, 8
    nq, pre = [70, 5], [0, 130]
    q, kn, vn, kp, vp, table, L, cu = _ragged_case(23, Hq, Hkv, D, nq, pre)
    kp, vp = A.kv_append(kp, vp, table, L, cu, kn, vn)
    O, LSE = A.paged_prefill(q, kp, vp, table, L, cu, 0.4)
    # request 0 has no prefix: ordinary square causal prefill on its own tokens
    po, pl = A.prefill(q[None, :70].transpose(0, 2, 1, 3), kn[None, :70].transpose(0, 2, 1, 3),
                       vn[None, :70].transpose(0, 2, 1, 3), 0.4, True)
    _close(O[:70], po[0].transpose(1, 0, 2), 1e-12, "no-prefix == prefill O")
    _close(LSE[:70], pl[0].T, 1e-12, "no-prefix == prefill LSE")
    # each request's last new token sees the whole cache: a decode query
    last = cu[1:] - 1
    do, dl = A.paged_decode(q[last], kp, vp, table, L, 0.4)
    _close(O[last], do, 1e-12, "last token == decode O")
    _close(LSE[last], dl, 1e-12, "last token == decode LSE")


def pin_shared_prefix_cascade():
    """Cascade decomposition: for requests sharing prefix pages, attention over
    the prefix (gathered once per group) and over each request's own suffix,
    merged by LSE, equals decode over the whole cache; an empty suffix merges
    as a split with LSE = -inf."""
    g = _rng(24)
    Hq, Hkv, D = 4, 2, 8
    pp = [2, 1]
    groups = [0, 0, -1, 1, 0]
    suffix = [0, 70, 5, 64, 130]
    P = sum(pp) + sum((x + 63) // 64 for x in suffix) + 1
    kp = g.standard_normal((P, Hkv, 64, D))
    vp = g.standard_normal((P, Hkv, 64, D))
    perm = g.permutation(P)
    pre_ids = [list(perm[:2]), list(perm[2:3])]
    nxt = 3
    table = np.full((5, 6), -1)
    L = np.zeros(5, dtype=np.int64)
    for b in range(5):
        row = list(pre_ids[groups[b]]) if groups[b] >= 0 else []
        n_own = (suffix[b] + 63) // 64
        row += list(perm[nxt:nxt + n_own])
        nxt += n_own
        table[b, :len(row)] = row
        L[b] = (64 * pp[groups[b]] if groups[b] >= 0 else 0) + suffix[b]
    q = g.standard_normal((5, Hq, D))
    O, LSE = A.paged_decode(q, kp, vp, table, L, 0.35)
    for b in range(5):
        P_tok = 64 * pp[groups[b]] if groups[b] >= 0 else 0
        for h in range(Hq):
            gg = h // (Hq // Hkv)
            kb = A.gather_pages(kp, table[b], int(L[b]), gg)
            vb = A.gather_pages(vp, table[b], int(L[b]), gg)
            parts_o, parts_l = [], []
            for lo, hi in ((0, P_tok), (P_tok, int(L[b]))):
                o, l = A.attention_head(q[b, h][None], kb[lo:hi], vb[lo:hi], 0.35)
                parts_o.append(o[0])
                parts_l.append(l[0])
            mo, ml = A.lse_merge(np.array(parts_o), np.array(parts_l))
            _close(mo, O[b, h], 1e-12, f"cascade O b={b} h={h}")
            _close(ml, LSE[b, h], 1e-12, f"cascade LSE b={b} h={h}")


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def pin_backward_torch_autograd():
    """dQ, dK, dV equal torch autograd through CPU SDPA in float64 (causal and not, GQA expanded)."""
    g = _rng(30)
    B, Hq, Hkv, S, D = 1, 4, 2, 19, 8
    q, k, v, do = (g.standard_normal(s) for s in ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D), (B, Hq, S, D)))
    for causal in (False, True):
        dq, dk, dv = A.prefill_backward(q, k, v, do, 0.37, causal)
        tq = torch.from_numpy(q).requires_grad_()
        tk = torch.from_numpy(k).requires_grad_()
        tv = torch.from_numpy(v).requires_grad_()
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(Hq // Hkv, dim=1), tv.repeat_interleave(Hq // Hkv, dim=1),
            is_causal=causal, scale=0.37)
        o.backward(torch.from_numpy(do))
        _close(dq, tq.grad.numpy(), 1e-12, f"autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-12, f"autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-12, f"autograd dV causal={causal}")


def pin_backward_finite_differences():
    """Central differences of L = sum(dO * O) along random directions match the
    gradients' inner products (brute force on a tiny head, Sq != Sk, causal)."""
    g = _rng(31)
    Sq, Sk, D = 3, 5, 4
    q, k, v, do = g.standard_normal((Sq, D)), g.standard_normal((Sk, D)), g.standard_normal((Sk, D)), g.standard_normal((Sq, D))
    dq, dk, dv = A.attention_head_backward(q, k, v, do, 0.8, True)
    f = lambda q_, k_, v_: float(np.sum(do * A.attention_head(q_, k_, v_, 0.8, True)[0]))  # noqa: E731
    eps = 1e-6
    for name, grad, idx in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        u = g.standard_normal(grad.shape)
        args_p = [q.copy(), k.copy(), v.copy()]
        args_m = [q.copy(), k.copy(), v.copy()]
        args_p[idx] += eps * u
        args_m[idx] -= eps * u
        fd = (f(*args_p) - f(*args_m)) / (2 * eps)
        _close(fd, np.sum(grad * u), 1e-7, f"finite differences {name}")


def pin_backward_gqa_sum():
    """A shared KV head's gradient is the sum of the MHA gradients of the query heads that read it."""
    g = _rng(32)
    B, Hq, Hkv, S, D = 1, 4, 2, 7, 4
    q, k, v, do = (g.standard_normal(s) for s in ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D), (B, Hq, S, D)))
    _, dk, dv = A.prefill_backward(q, k, v, do, 0.5, True)
    ke, ve = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    _, dke, dve = A.prefill_backward(q, ke, ve, do, 0.5, True)
    _close(dk, dke.reshape(B, Hkv, 2, S, D).sum(axis=2), 1e-12, "GQA dK sum")
    _close(dv, dve.reshape(B, Hkv, 2, S, D).sum(axis=2), 1e-12, "GQA dV sum")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
