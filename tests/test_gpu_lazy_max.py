"""Parity where the running max must move again and again.

The kernels keep a lazy running max: it moves only when a tile's scores rise
more than 2^8 (in exp2 units) above it, and O and the normalisers are then
rescaled. Random inputs settle the max after the first tile or two. Here the
scores of every row ramp with the key's logical position, about 0.25 natural
units per key (about 23 exp2 units per 64-key tile or page), so the max moves
on nearly every tile; a sawtooth variant lets it rise, fall back and rise
above its old level. The oracle gets the same bf16 inputs, so an error in the
rescale path shows up against it. The fp8 prefill gets the same offsets
spread over all 128 dims, quantised per head to e4m3, against the oracle on
the dequantised values (gfx950's fp8 matrix product drops the low bits of
products far below the largest of their 64-product block, so the ramp is not
carried by one dim there: every product of a score is then of similar size)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check, check_fp8_prefill, f64, fp8_weight_bound, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))
RISE = 0.25    # natural-log units of score per key


def offset(pos, shape):
    """Score offset of the key at logical position pos (natural-log units)."""
    pos = np.asarray(pos, np.float64)
    if shape == "ramp":
        return RISE * pos
    # sawtooth: three pages up, then back down; each peak above the last
    return RISE * (pos % 192) + 0.05 * pos


def shape_query(q):
    """Query dim 0 := 4 and the other dims scaled down, so dim 0 carries the score."""
    q[..., 0] = 4.0
    q[..., 1:] *= 0.1


def key_dim0(pos, shape):
    """Key dim 0 that gives the offset through a query dim 0 of 4."""
    return torch.from_numpy((offset(pos, shape) / (4.0 * SCALE)).astype(np.float32))


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_moving_max(shape, causal):
    fa = need_gpu()
    B, Hq, Hkv, S, D = 1, 4, 2, 777, 128
    say(f"[case] prefill moving max {shape} causal={causal}")
    q, k, v = workloads.prefill_inputs(B, Hq, Hkv, S, S, D, "bf16", 61)
    q, k = q.float(), k.float()
    shape_query(q)
    k[..., 0] = key_dim0(np.arange(S), shape)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    out, lse = fa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    O, L = oracle.prefill(f64(q), f64(k), f64(v), SCALE, causal)
    check(f"prefill moving max {shape} causal={causal}", f64(out), O, f64(lse), L, "bf16")


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_decode_moving_max(shape, num_splits):
    fa = need_gpu()
    lengths = [1, 65, 700, 2049]
    Hq, Hkv, D = 8, 2, 128
    say(f"[case] decode moving max {shape} splits={num_splits}")
    kv = workloads.paged_inputs(len(lengths), Hq, Hkv, D, "bf16", lengths, 62, nan_tails=False)
    q, kp = kv.q.float(), kv.k_pages.float()
    shape_query(q)
    table = kv.page_table.numpy()
    for b, n in enumerate(lengths):
        t = np.arange(n)
        # every KV head of the token's physical page slot
        kp[table[b, t // 64], :, t % 64, 0] = key_dim0(t, shape)[:, None].expand(n, Hkv)
    q, kp = q.to(torch.bfloat16), kp.to(torch.bfloat16)
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, D, fa.BF16, num_splits)
    out, lse = fa.decode(plan, q.cuda(), kp.cuda(), kv.v_pages.cuda(), kv.page_table.cuda(),
                         kv.seqlens.cuda(), None, None, SCALE)
    torch.cuda.synchronize()
    O, L = oracle.paged_decode(f64(q), kp.float().numpy(), kv.v_pages.float().numpy(), kv.page_table.numpy(),
                               kv.seqlens.numpy(), SCALE)
    check(f"decode moving max {shape} splits={num_splits}", f64(out), O, f64(lse), L, "bf16")


def fp8_moving_max_inputs(B, Hq, Hkv, S, shape, wid=63):
    """Float32 Q/K/V quantised per head: (q8, k8, v8, q_scale, k_scale,
    v_scale), host tensors. Query dim d is sign_d (1 + 0.1 n) and key dim d of
    position j is sign_d offset(j) / (D scale) + 0.1 n, with one random sign
    per dim, so every score carries the offset of its key spread evenly over
    the dims."""
    D = 128
    q = workloads.rng(wid, workloads.STREAM_Q).standard_normal(size=(B, Hq, S, D), dtype=np.float32)
    k = workloads.rng(wid, workloads.STREAM_K).standard_normal(size=(B, Hkv, S, D), dtype=np.float32)
    v = workloads.rng(wid, workloads.STREAM_V).standard_normal(size=(B, Hkv, S, D), dtype=np.float32)
    sign = np.where(workloads.rng(wid, workloads.STREAM_PERM).random(D) < 0.5, -1.0, 1.0).astype(np.float32)
    q = sign * (1.0 + 0.1 * q)
    r = (offset(np.arange(S), shape) / (D * SCALE)).astype(np.float32)
    k = sign * r[:, None] + 0.1 * k
    q8, qs = workloads.quantise_heads_e4m3fn(q)
    k8, ks = workloads.quantise_heads_e4m3fn(k)
    v8, vs = workloads.quantise_heads_e4m3fn(v)
    return q8, k8, v8, qs, ks, vs


def dequantise(codes, scale):
    return oracle.e4m3fn_to_float(codes.numpy()) * scale.numpy().astype(np.float64)[:, :, None, None]


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_moving_max(shape, causal):
    fa = need_gpu()
    B, Hq, Hkv, S = 1, 4, 2, 777
    say(f"[case] fp8 prefill moving max {shape} causal={causal}")
    q8, k8, v8, qs, ks, vs = fp8_moving_max_inputs(B, Hq, Hkv, S, shape)
    out, lse = fa.prefill_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs.cuda(), ks.cuda(), vs.cuda(), causal, SCALE)
    torch.cuda.synchronize()
    qd, kd, vd = dequantise(q8, qs), dequantise(k8, ks), dequantise(v8, vs)
    O, L = oracle.prefill(qd, kd, vd, SCALE, causal)
    bound = np.zeros_like(O)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        bound[0, h] = fp8_weight_bound(qd[0, h], kd[0, g], vd[0, g], SCALE, causal)
    check_fp8_prefill(f"fp8 prefill moving max {shape} causal={causal}", f64(out), O, bound, f64(lse), L)


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
def test_cascade_moving_max(shape):
    """Shared-prefix decode: the prefix pass (prefill kernel over the group's
    pages, rows = members x heads) and the suffix split kernel both see the
    max move, and the merge combines their partials."""
    fa = need_gpu()
    groups, suffix, pp, Hq, Hkv = [0, 0, 0, -1, 1, 1], [5, 300, 900, 1200, 64, 0], [24, 9], 8, 2
    say(f"[case] cascade moving max {shape}")
    r = workloads.shared_prefix_inputs(Hq, Hkv, 128, groups, suffix, pp, wid=64, nan_tails=False)
    q, kp = r.q.float(), r.k_pages.float()
    shape_query(q)
    table = r.page_table.numpy()
    for b, n in enumerate(r.seqlens.tolist()):
        t = np.arange(n)
        kp[table[b, t // 64], :, t % 64, 0] = key_dim0(t, shape)[:, None].expand(n, Hkv)
    q, kp = q.to(torch.bfloat16), kp.to(torch.bfloat16)
    plan = fa.fa_decode_plan_cascade(r.seqlens, r.page_table, r.num_pages, Hq, Hkv, r.prefix_group,
                                     r.prefix_pages.tolist())
    out, lse = fa.decode(plan, q.cuda(), kp.cuda(), r.v_pages.cuda(), r.page_table.cuda(), r.seqlens.cuda(),
                         scale=SCALE)
    torch.cuda.synchronize()
    O, L = oracle.paged_decode(f64(q), kp.float().numpy(), r.v_pages.float().numpy(), table, r.seqlens.numpy(),
                               SCALE)
    check(f"cascade moving max {shape}", f64(out), O, f64(lse), L, "bf16")


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
def test_ragged_prefill_moving_max(shape):
    """Ragged paged prefill after the KV append: cached prefix keys and the
    appended new keys carry the ramp of their logical positions."""
    fa = need_gpu()
    nq, pre, Hq, Hkv = [1, 300, 129, 700], [0, 100, 1500, 64], 8, 2
    say(f"[case] ragged prefill moving max {shape}")
    r = workloads.ragged_inputs(Hq, Hkv, 128, nq, pre, wid=65, poison=False)
    q, kp, kn = r.q.float(), r.k_pages.float(), r.k_new.float()
    shape_query(q)
    table, cu = r.page_table.numpy(), r.cu_seqlens_q.numpy()
    for b in range(len(nq)):
        t = np.arange(pre[b])
        kp[table[b, t // 64], :, t % 64, 0] = key_dim0(t, shape)[:, None].expand(len(t), Hkv)
        kn[cu[b]:cu[b + 1], :, 0] = key_dim0(pre[b] + np.arange(nq[b]), shape)[:, None].expand(nq[b], Hkv)
    r.q, r.k_pages, r.k_new = q.to(torch.bfloat16), kp.to(torch.bfloat16), kn.to(torch.bfloat16)
    d = dict(q=r.q.cuda(), kn=r.k_new.cuda(), vn=r.v_new.cuda(), k=r.k_pages.cuda(), v=r.v_pages.cuda(),
             pt=r.page_table.cuda(), sl=r.seqlens.cuda(), cu=r.cu_seqlens_q.cuda())
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, Hq, Hkv)
    out, lse = fa.prefill_paged(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], SCALE)
    torch.cuda.synchronize()
    kpo, vpo = oracle.kv_append(r.k_pages.float().numpy(), r.v_pages.float().numpy(), table, r.seqlens.numpy(),
                                cu, r.k_new.float().numpy(), r.v_new.float().numpy())
    O, L = oracle.paged_prefill(f64(r.q), kpo, vpo, table, r.seqlens.numpy(), cu, SCALE)
    check(f"ragged prefill moving max {shape}", f64(out), O, f64(lse), L, "bf16")


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_fp8_decode_moving_max(shape, num_splits):
    """Paged decode over an fp8 cache (codes with one scale per page and KV
    head), the same construction quantised after the ramp is set."""
    fa = need_gpu()
    lengths = [1, 65, 700, 2049]
    Hq, Hkv, D = 8, 2, 128
    say(f"[case] fp8 decode moving max {shape} splits={num_splits}")
    kv = workloads.paged_inputs(len(lengths), Hq, Hkv, D, "bf16", lengths, 66, nan_tails=False)
    q, kp = kv.q.float(), kv.k_pages.float()
    shape_query(q)
    table = kv.page_table.numpy()
    for b, n in enumerate(lengths):
        t = np.arange(n)
        kp[table[b, t // 64], :, t % 64, 0] = key_dim0(t, shape)[:, None].expand(n, Hkv)
    q = q.to(torch.bfloat16)
    k8, ks = workloads._quantise_e4m3fn(kp.numpy().copy(), [], False)
    v8, vs = workloads._quantise_e4m3fn(kv.v_pages.float().numpy().copy(), [], False)
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, D, fa.FP8_E4M3FN, num_splits)
    out, lse = fa.decode(plan, q.cuda(), k8.cuda(), v8.cuda(), kv.page_table.cuda(), kv.seqlens.cuda(),
                         ks.cuda(), vs.cuda(), SCALE)
    torch.cuda.synchronize()
    O, L = oracle.paged_decode(f64(q), k8.numpy(), v8.numpy(), table, kv.seqlens.numpy(), SCALE,
                               ks.numpy(), vs.numpy())
    check(f"fp8 decode moving max {shape} splits={num_splits}", f64(out), O, f64(lse), L, "fp8")
