"""Bit-exact page-table and head indexing of the production kernels, seen through their outputs.

Structured inputs make the exact answer of every output row one stored V row.
Query head h is one-hot on dimension h (or on a dimension chosen per row, for
prefill), and the key it must find holds the same one-hot; every other key of
that KV head is zero along that dimension. The score gap is about 360 (natural
log units), so exp of every other score is exactly 0 in fp32: the softmax
weight of the chosen key is 1 and all others are 0, whatever the tiling, the
lazy running max or the split of the keys. The output must then equal that
key's V row bit for bit (bf16 values, or e4m3fn codes times a power-of-two
scale, which bf16 holds exactly). The chosen positions sweep the first and
last token, both sides of page boundaries, partly filled last pages and, in
long requests, the split boundaries of the plan; a lookup that is off by one
page or one slot, or that reads another request's or head's row, changes bits.
The fp64 oracle is run on the same inputs as a check that the expected rows
are what the definition gives, and it gates the LSE.

Kernels covered: decode_mfma_kernel (4, 8 and 16 query heads per KV head; bf16
and fp8 KV), decode_split_kernel (1 and 2), automatic and forced splits
{1, 3}, the ragged paged prefill (the MFMA prefill kernel reading its key
tiles from pages) and the contiguous prefill (GQA head enumeration, explicit
head map, ragged last query tile).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import f64, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))
BETA, C_BF16 = 64.0, 64.0          # q = BETA e_d, chosen key = C e_d: score 4096 * scale ~ 362
FP8_448, FP8_KSCALE = 0x7E, 0.25   # e4m3fn code of 448; 448 * 0.25 * 64 * scale ~ 633


def _positions(L, rng, n):
    """Interesting logical positions of a request of length L, then random ones."""
    base = [0, L - 1, 63, 64, 65, 127, 128, 129, L - 64, L - 65, L // 2, 4095, 4096, 4097]
    pos = [p for p in base if 0 <= p < L]
    pos += [int(x) for x in rng.integers(0, L, size=max(0, n - len(pos)))] if L > 0 else []
    return pos


def _page_slot(table, b, t):
    return int(table[b, t // 64]), t % 64


def decode_case(L, Hq, Hkv, kv_dtype, seed):
    """Paged decode batch whose query head h of request b picks one chosen key."""
    rng = np.random.default_rng(seed)
    kv = workloads.paged_inputs(len(L), Hq, Hkv, 128, kv_dtype, L, 70 + seed, nan_tails=True,
                                extra_pages=2)
    table = kv.page_table.numpy()
    kp = kv.k_pages.clone()
    q = torch.zeros_like(kv.q)
    G = Hq // Hkv
    chosen = {}
    valid = torch.zeros(kp.shape[0], kp.shape[2], dtype=torch.bool)  # slots that hold tokens
    for b, Lb in enumerate(L):
        for t in range((Lb + 63) // 64):
            pid = int(table[b, t])
            valid[pid, :min(64, Lb - 64 * t)] = True
    if kv_dtype == "bf16":
        kp[valid.nonzero(as_tuple=True)[0], :, valid.nonzero(as_tuple=True)[1], :] = 0
    else:
        kp[valid.nonzero(as_tuple=True)[0], :, valid.nonzero(as_tuple=True)[1], :] = 0  # code 0 is +0.0
    for b, Lb in enumerate(L):
        pos = _positions(Lb, rng, Hq)
        for h in range(Hq):
            if Lb == 0:
                continue
            t = pos[(h + 3 * b) % len(pos)]
            pid, slot = _page_slot(table, b, t)
            g = h // G
            kp[pid, g, slot, h] = C_BF16 if kv_dtype == "bf16" else FP8_448
            q[b, h, h] = BETA
            chosen[(b, h)] = (pid, g, slot)
    ks = vs = None
    if kv_dtype == "fp8":
        P = kp.shape[0]
        ks = torch.full((P, Hkv), FP8_KSCALE, dtype=torch.float32)
        e = (np.arange(P)[:, None] + np.arange(Hkv)[None, :]) % 5
        vs = torch.from_numpy((2.0 ** -(4 + e)).astype(np.float32))
    kv2 = workloads.PagedKV(q, kp, kv.v_pages, ks, vs, kv.page_table, kv.seqlens, kv_dtype, kv.num_pages)
    return kv2, chosen


def expected_decode(kv, chosen):
    B, Hq, D = kv.q.shape
    exp = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    for (b, h), (pid, g, slot) in chosen.items():
        if kv.kv_dtype == "bf16":
            exp[b, h] = kv.v_pages[pid, g, slot]
        else:
            val = oracle.e4m3fn_to_float(kv.v_pages[pid, g, slot].numpy()) * float(kv.v_scale[pid, g])
            exp[b, h] = torch.from_numpy(val).to(torch.bfloat16)
            assert torch.equal(exp[b, h].double(), torch.from_numpy(val)), "expected row not exact in bf16"
    return exp


def oracle_decode(kv):
    if kv.kv_dtype == "fp8":
        kp, vp, ks, vs = kv.k_pages.numpy(), kv.v_pages.numpy(), kv.k_scale.numpy(), kv.v_scale.numpy()
    else:
        kp, vp, ks, vs = kv.k_pages.float().numpy(), kv.v_pages.float().numpy(), None, None
    return oracle.paged_decode(f64(kv.q), kp, vp, kv.page_table.numpy(), kv.seqlens.numpy(), SCALE, ks, vs)


DECODE_CASES = [
    # (lengths, Hq, Hkv): group sizes 1 and 2 take the VALU split kernel, 4-16 the MFMA one
    ([1, 63, 64, 65, 200, 5000], 2, 2),
    ([1, 63, 64, 65, 200, 5000], 4, 2),
    ([129, 64, 3, 4097, 0, 700], 8, 2),
    ([129, 64, 3, 4097, 0, 700], 16, 2),
    ([6000, 1, 65, 127, 128], 32, 2),
]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"G{c[1] // c[2]}")
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_decode_indexing_bit_exact(case, kv_dtype, num_splits):
    fa = need_gpu()
    L, Hq, Hkv = case
    say(f"[case] decode indexing L={L} Hq={Hq} Hkv={Hkv} {kv_dtype} num_splits={num_splits}")
    kv, chosen = decode_case(L, Hq, Hkv, kv_dtype, seed=len(L) + Hq)
    exp = expected_decode(kv, chosen)
    O, LSE = oracle_decode(kv)
    assert np.abs(O - exp.double().numpy()).max() <= 1e-12, "oracle disagrees with the expected rows"
    dt = fa.BF16 if kv_dtype == "bf16" else fa.FP8_E4M3FN
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, 128, dt, num_splits)
    d = dict(q=kv.q.cuda(), k=kv.k_pages.cuda(), v=kv.v_pages.cuda(), pt=kv.page_table.cuda(),
             sl=kv.seqlens.cuda())
    ks = kv.k_scale.cuda() if kv.k_scale is not None else None
    vs = kv.v_scale.cuda() if kv.v_scale is not None else None
    out, lse = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], ks, vs, SCALE)
    torch.cuda.synchronize()
    got = out.cpu()
    bad = [(b, h) for b in range(len(L)) for h in range(Hq) if not torch.equal(got[b, h], exp[b, h])]
    assert not bad, f"{len(bad)} rows differ from their chosen V row, first {bad[:4]}"
    lg, LSEn = f64(lse), LSE
    fin = np.isfinite(LSEn)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.abs(lg[fin] - LSEn[fin]).max() <= 1e-3


def ragged_case(nq, pre, Hq, Hkv, seed):
    """Ragged paged prefill whose (row, head) picks one chosen key among those it sees."""
    rng = np.random.default_rng(seed)
    r = workloads.ragged_inputs(Hq, Hkv, 128, nq, pre, wid=80 + seed, extra_pages=2, poison=True)
    table, L, cu = r.page_table.numpy(), r.seqlens.numpy(), r.cu_seqlens_q.numpy()
    kp = r.k_pages.clone()
    vp = r.v_pages.clone()
    q = torch.zeros_like(r.q)
    vfill = workloads.normal(90 + seed, 0, (int(L.sum()), Hkv, 128), "bf16")
    o = 0
    for b in range(len(L)):
        for t in range(int(L[b])):  # every token of the final cache: K zero, V random
            pid, slot = _page_slot(table, b, t)
            kp[pid, :, slot] = 0
            vp[pid, :, slot] = vfill[o]
            o += 1
    exp = torch.zeros(r.q.shape, dtype=torch.bfloat16)
    G = Hq // Hkv
    for b in range(len(L)):
        n, Lb = int(nq[b]), int(L[b])
        if n == 0:
            continue
        for g in range(Hkv):
            # dimension d of KV head g is carried by the key at logical position pos[d]
            pos = _positions(Lb, rng, 128)[:128]
            pos[0] = 0  # every row sees at least the key of dimension 0
            for dim, t in enumerate(pos):
                pid, slot = _page_slot(table, b, t)
                kp[pid, g, slot, dim] = C_BF16
            for i in range(n):
                lim = Lb - n + i  # new token i sees keys 0 .. lim
                vis = [dim for dim, t in enumerate(pos) if t <= lim]
                for j in range(G):
                    h = g * G + j
                    dim = vis[(3 * i + 5 * h) % len(vis)]
                    q[cu[b] + i, h, dim] = BETA
                    pid, slot = _page_slot(table, b, pos[dim])
                    exp[cu[b] + i, h] = vp[pid, g, slot]
    return workloads.RaggedPaged(q, r.k_new, r.v_new, kp, vp, r.page_table, r.seqlens, r.cu_seqlens_q,
                                 r.num_pages), exp


@pytest.mark.parametrize("case", [
    ([1, 63, 64, 65, 300, 700], [0, 1, 100, 4000, 63, 64], 8, 2),
    ([256, 257, 1, 0, 513], [0, 0, 4095, 17, 1000], 4, 4),
    ([129, 1000], [2000, 3], 32, 8),
], ids=lambda c: f"G{c[2] // c[3]}-B{len(c[0])}")
def test_paged_prefill_indexing_bit_exact(case):
    fa = need_gpu()
    nq, pre, Hq, Hkv = case
    say(f"[case] paged prefill indexing nq={nq} prefix={pre} Hq={Hq} Hkv={Hkv}")
    r, exp = ragged_case(nq, pre, Hq, Hkv, seed=len(nq) + Hq)
    O, LSE = oracle.paged_prefill(f64(r.q), r.k_pages.float().numpy(), r.v_pages.float().numpy(),
                                  r.page_table.numpy(), r.seqlens.numpy(), r.cu_seqlens_q.numpy(), SCALE)
    assert np.abs(O - exp.double().numpy()).max() <= 1e-12, "oracle disagrees with the expected rows"
    plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, Hq, Hkv)
    out, lse = fa.prefill_paged(plan, r.q.cuda(), r.k_pages.cuda(), r.v_pages.cuda(), r.page_table.cuda(),
                                r.seqlens.cuda(), r.cu_seqlens_q.cuda(), SCALE)
    torch.cuda.synchronize()
    got = out.cpu()
    bad = (got.view(torch.int16) != exp.view(torch.int16)).any(dim=2).nonzero().tolist()
    assert not bad, f"{len(bad)} (token, head) rows differ from their chosen V row, first {bad[:4]}"
    assert np.abs(f64(lse) - LSE).max() <= 1e-3


@pytest.mark.parametrize("B,Hq,Hkv,S,use_map", [(2, 8, 2, 700, False), (1, 8, 4, 513, True),
                                                 (4, 32, 8, 300, False)])
def test_prefill_head_and_row_indexing_bit_exact(B, Hq, Hkv, S, use_map):
    """Contiguous prefill: every (batch, head, row) finds its own chosen key, through the
    XCD-ordered head enumeration (or an explicit, non-contiguous head map) and the ragged last tile."""
    fa = need_gpu()
    say(f"[case] prefill indexing B={B} Hq={Hq} Hkv={Hkv} S={S} map={use_map}")
    rng = np.random.default_rng(S)
    k = torch.zeros(B, Hkv, S, 128, dtype=torch.bfloat16)
    v = workloads.normal(95, 0, (B, Hkv, S, 128), "bf16")
    q = torch.zeros(B, Hq, S, 128, dtype=torch.bfloat16)
    kv_map = [int(x) for x in rng.permutation(np.repeat(np.arange(Hkv), Hq // Hkv))] if use_map else None
    exp = torch.zeros(B, Hq, S, 128, dtype=torch.bfloat16)
    for b in range(B):
        for g in range(Hkv):
            pos = sorted(set([0, S - 1, 255, 256, 63, 64] + [int(x) for x in rng.integers(0, S, 200)]))[:128]
            for dim, t in enumerate(pos):
                k[b, g, t, dim] = C_BF16
            heads = [h for h in range(Hq) if (kv_map[h] if use_map else h // (Hq // Hkv)) == g]
            for h in heads:
                for i in range(S):
                    vis = [dim for dim, t in enumerate(pos) if t <= i]
                    dim = vis[(7 * i + 11 * h + b) % len(vis)]
                    q[b, h, i, dim] = BETA
                    exp[b, h, i] = v[b, g, pos[dim]]
    O, LSE = oracle.prefill(f64(q), f64(k), f64(v), SCALE, True, kv_head_map=kv_map)
    assert np.abs(O - exp.double().numpy()).max() <= 1e-12, "oracle disagrees with the expected rows"
    out, lse = fa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=SCALE, kv_head_map=kv_map)
    torch.cuda.synchronize()
    bad = (out.cpu().view(torch.int16) != exp.view(torch.int16)).any(dim=3).nonzero().tolist()
    assert not bad, f"{len(bad)} (b, h, row) rows differ from their chosen V row, first {bad[:4]}"
    assert np.abs(f64(lse) - LSE).max() <= 1e-3
