"""fp8 (e4m3fn) prefill through the C ABI against the oracle on the dequantised inputs.

The oracle runs the definition in fp64 on code * scale, so input quantisation
is not charged to the kernel; the rounding of the softmax weights to e4m3
inside the kernel is, through the per-element bound in parity.fp8_weight_bound.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_fp8_prefill, f64, fp8_weight_bound, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))


def deq(codes, scale):
    return oracle.e4m3fn_to_float(codes.numpy()) * scale.numpy().astype(np.float64)[:, :, None, None]


def run(fa, B, Hq, Hkv, Sq, Sk, causal, wid):
    q8, k8, v8, qs, ks, vs = workloads.fp8_prefill_inputs(B, Hq, Hkv, Sq, Sk, 128, wid)
    out, lse = fa.prefill_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs.cuda(), ks.cuda(), vs.cuda(), causal, SCALE)
    torch.cuda.synchronize()
    return (q8, k8, v8, qs, ks, vs), out, lse


SHAPES = [
    # (B, Hq, Hkv, Sq, Sk, causal)
    (1, 2, 2, 1, 1, True), (1, 2, 2, 64, 64, True), (2, 4, 2, 300, 300, True), (1, 8, 2, 257, 700, True),
    (1, 4, 4, 700, 257, False), (1, 2, 1, 1000, 1000, False), (1, 4, 1, 513, 513, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_prefill_shapes(shape):
    fa = need_gpu()
    B, Hq, Hkv, Sq, Sk, causal = shape
    say(f"[case] fp8 prefill {shape}")
    (q8, k8, v8, qs, ks, vs), out, lse = run(fa, B, Hq, Hkv, Sq, Sk, causal, 70)
    qd, kd, vd = deq(q8, qs), deq(k8, ks), deq(v8, vs)
    O, LSE = oracle.prefill(qd, kd, vd, SCALE, causal)
    bound = np.zeros_like(O)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            bound[b, h] = fp8_weight_bound(qd[b, h], kd[b, g], vd[b, g], SCALE, causal)
    check_fp8_prefill(f"fp8 prefill {shape}", f64(out), O, bound, f64(lse), LSE)


def test_fp8_full_workload_sampled():
    """Workload 8 (fp8, 4 x 32 heads x 4096, causal) in the bench launch configuration, sampled rows."""
    fa = need_gpu()
    w = workloads.WORKLOADS[8]
    say(f"[case] fp8 prefill workload {w.name}")
    (q8, k8, v8, qs, ks, vs), out, lse = run(fa, w.B, w.Hq, w.Hkv, w.S, w.S, True, w.wid)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.S - 32, w.S), rng.integers(0, w.S, 96)]))
    for b, h in [(0, 0), (1, 7), (3, 31)]:
        qd = oracle.e4m3fn_to_float(q8[b, h].numpy()) * float(qs[b, h])
        kd = oracle.e4m3fn_to_float(k8[b, h].numpy()) * float(ks[b, h])
        vd = oracle.e4m3fn_to_float(v8[b, h].numpy()) * float(vs[b, h])
        o, l = oracle.attention_head(qd, kd, vd, SCALE, True, rows)
        bound = fp8_weight_bound(qd, kd, vd, SCALE, True, rows)
        check_fp8_prefill(f"fp8 workload (b={b}, h={h}, {len(rows)} rows)", f64(out[b, h][torch.from_numpy(rows).cuda()]),
                          o, bound, f64(lse[b, h][torch.from_numpy(rows).cuda()]), l)
