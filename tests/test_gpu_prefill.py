"""Prefill parity: the HIP path (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check, f64, need_gpu, say

pytestmark = pytest.mark.gpu


def run_case(fa, B, Hq, Hkv, Sq, Sk, D, dtype, causal, wid, kv_head_map=None, scale=None):
    say(f"[case] prefill B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} {dtype} causal={causal} wid={wid} map={kv_head_map}")
    q, k, v = workloads.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, wid)
    sc = float(np.float32(scale if scale else 1.0 / np.sqrt(D)))
    out, lse = fa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=sc, kv_head_map=kv_head_map)
    torch.cuda.synchronize()
    O, L = oracle.prefill(f64(q), f64(k), f64(v), sc, causal, kv_head_map=kv_head_map)
    return out, lse, O, L


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_fp32_workload(causal):
    fa = need_gpu()
    w = workloads.WORKLOADS[1]
    out, lse, O, L = run_case(fa, w.B, w.Hq, w.Hkv, w.S, w.S, w.D, "f32", causal, w.wid)
    assert out.shape == (1, 2, 128, 64) and lse.shape == (1, 2, 128)
    check(f"wl1 causal={causal}", f64(out), O, f64(lse), L, "f32")


@pytest.mark.parametrize("shape", [
    (1, 2, 2, 65, 65, 64, True), (2, 3, 1, 200, 200, 128, True), (1, 2, 2, 1, 1, 128, False),
    (1, 2, 2, 100, 300, 128, True), (1, 2, 2, 130, 33, 128, True), (1, 1, 1, 7, 0, 64, False),
])
def test_fp32_shapes(shape):
    fa = need_gpu()
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    out, lse, O, L = run_case(fa, B, Hq, Hkv, Sq, Sk, D, "f32", causal, 11)
    check(f"f32 {shape}", f64(out), O, f64(lse), L, "f32")


@pytest.mark.parametrize("shape", [
    # (B, Hq, Hkv, Sq, Sk, causal): several 128-row / 64-key tiles plus ragged tails
    (1, 2, 2, 300, 300, True), (1, 2, 2, 300, 300, False), (2, 4, 2, 257, 257, True),
    (1, 8, 2, 384, 384, True), (1, 2, 2, 1, 1, True), (1, 2, 2, 63, 63, True), (1, 2, 2, 65, 65, True),
    (1, 2, 2, 127, 127, False), (1, 2, 2, 129, 129, True), (1, 2, 1, 100, 333, True),
    (1, 2, 1, 333, 100, True), (1, 2, 2, 64, 1000, False), (3, 1, 1, 517, 517, True),
])
def test_bf16_shapes(shape):
    fa = need_gpu()
    B, Hq, Hkv, Sq, Sk, causal = shape
    out, lse, O, L = run_case(fa, B, Hq, Hkv, Sq, Sk, 128, "bf16", causal, 21)
    check(f"bf16 {shape}", f64(out), O, f64(lse), L, "bf16")


def test_bf16_empty_rows_and_zero_keys():
    fa = need_gpu()
    # Sq > Sk causal: the first Sq-Sk rows see no key -> O = 0, LSE = -inf
    out, lse, O, L = run_case(fa, 1, 2, 2, 200, 70, 128, "bf16", True, 22)
    assert torch.all(out[:, :, :130] == 0) and torch.all(torch.isneginf(lse[:, :, :130]))
    check("bf16 empty rows", f64(out), O, f64(lse), L, "bf16")
    out, lse, O, L = run_case(fa, 1, 2, 2, 10, 0, 128, "bf16", False, 22)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_bf16_explicit_head_map():
    fa = need_gpu()
    hmap = [2, 0, 1, 1, 0, 2]
    out, lse, O, L = run_case(fa, 2, 6, 3, 150, 150, 128, "bf16", True, 23, kv_head_map=hmap)
    check("bf16 head map", f64(out), O, f64(lse), L, "bf16")


def test_bf16_custom_scale():
    fa = need_gpu()
    out, lse, O, L = run_case(fa, 1, 2, 2, 200, 200, 128, "bf16", True, 24, scale=0.3)
    check("bf16 scale 0.3", f64(out), O, f64(lse), L, "bf16")


def test_causal_future_independence():
    """Changing K/V at positions > i leaves GPU row i bitwise unchanged."""
    fa = need_gpu()
    q, k, v = workloads.prefill_inputs(1, 2, 2, 256, 256, 128, "bf16", 25)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    out1, lse1 = fa.prefill(q, k, v, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 150:] = torch.randn_like(k2[:, :, 150:].float()).bfloat16()
    v2[:, :, 150:] = torch.randn_like(v2[:, :, 150:].float()).bfloat16()
    out2, lse2 = fa.prefill(q, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, :, :150], out2[:, :, :150])
    assert torch.equal(lse1[:, :, :150], lse2[:, :, :150])
    assert not torch.equal(out1[:, :, 150:], out2[:, :, 150:])


def test_repeatable_bitwise():
    fa = need_gpu()
    q, k, v = workloads.prefill_inputs(2, 4, 4, 1000, 1000, 128, "bf16", 26)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    a = fa.prefill(q, k, v, causal=True)
    b = fa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _sample_rows(S, rng):
    rows = set(range(0, 130)) | set(range(S - 64, S))
    for t in range(128, S, 128):
        rows |= {t - 1, t}
    rows |= set(rng.choice(S, size=min(256, S), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < S))


@pytest.mark.parametrize("wid", [2, 3])
def test_full_workload_sampled(wid):
    """Full-size workloads in the benchmark's launch configuration; sampled heads and rows."""
    fa = need_gpu()
    w = workloads.WORKLOADS[wid]
    say(f"[case] full workload {wid} {w.name}")
    q, k, v = workloads.workload_prefill_inputs(w)
    out, lse = fa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    rng = np.random.default_rng(wid)
    heads = [(0, 0), (w.B - 1, w.Hq - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(2)]
    rows = _sample_rows(w.S, rng)
    qn, kn, vn = f64(q), f64(k), f64(v)
    O, L = oracle.prefill(qn, kn, vn, w.scale, True, heads=heads, rows=rows)
    og = np.stack([f64(out[b, h, rows]) for b, h in heads])
    lg = np.stack([f64(lse[b, h, rows]) for b, h in heads])
    check(f"workload {wid} sampled {len(heads)} heads x {len(rows)} rows", og, O, lg, L, "bf16")
    # every (b, h): first and last row, and both sides of the 256-row tile boundaries at the
    # start, middle and end (the XCD-ordered head enumeration covers all B * Hq heads)
    few = np.array(sorted({0, 255, 256, w.S // 2 - 1, w.S // 2, w.S - 257, w.S - 256, w.S - 1}))
    every = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    O2, L2 = oracle.prefill(qn, kn, vn, w.scale, True, heads=every, rows=few)
    og2 = f64(out[:, :, few]).reshape(len(every), len(few), -1)
    lg2 = f64(lse[:, :, few]).reshape(len(every), len(few))
    check(f"workload {wid} all {len(every)} heads x {len(few)} rows", og2, O2, lg2, L2, "bf16")
