"""Attention backward (dQ, dK, dV) through the C ABI against the fp64 oracle.

The GPU backward consumes the GPU forward's O (bf16) and LSE, as a training
step does; the oracle differentiates the definition exactly. Gate, per
gradient tensor: RMS error <= 1e-2 * max(RMS of the reference, 1e-3) and max
|error| <= 2e-2 * max(max |reference|, 1e-2). Three independent bf16
roundings reach each gradient element (P or dS entering the matrix cores, O
inside D = rowsum(dO * O), and the output), each 2^-9 relative, which
combine to about 3 * 2^-9 = 6e-3 relative RMS; the floors cover gradients
that vanish exactly (a row with one visible key has dS = 0) where only fp32
residue remains.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import f64, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))


def check_grad(name, got, ref, rel_rms=1e-2, rel_max=2e-2):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt((err ** 2).mean()) / max(np.sqrt((ref ** 2).mean()), 1e-3))
    mx = float(err.max(initial=0.0)) / max(float(np.abs(ref).max(initial=0.0)), 1e-2)
    say(f"[parity] {name}: rel_rms={rms:.3e} max_err/max_ref={mx:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    assert rms <= rel_rms, f"{name}: rel_rms {rms:.3e} > {rel_rms}"
    assert mx <= rel_max, f"{name}: max error {mx:.3e} of max |ref| > {rel_max}"


def run(fa, B, Hq, Hkv, Sq, Sk, causal, wid):
    q, k, v, do = workloads.backward_inputs(B, Hq, Hkv, Sq, Sk, 128, wid)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.prefill(qd, kd, vd, causal=causal, scale=SCALE)
    dq, dk, dv = fa.prefill_bwd(qd, kd, vd, o, lse, dod, causal, SCALE)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


SHAPES = [
    # (B, Hq, Hkv, Sq, Sk, causal)
    (1, 2, 2, 64, 64, True), (1, 2, 2, 300, 300, True), (2, 4, 2, 257, 257, True), (1, 8, 2, 200, 600, True),
    (1, 4, 4, 600, 200, False), (1, 2, 1, 1, 1, True), (1, 4, 1, 513, 513, False), (1, 2, 2, 700, 300, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_shapes(shape):
    fa = need_gpu()
    B, Hq, Hkv, Sq, Sk, causal = shape
    say(f"[case] backward {shape}")
    (q, k, v, do), (dq, dk, dv) = run(fa, B, Hq, Hkv, Sq, Sk, causal, 80)
    rq, rk, rv = oracle.prefill_backward(f64(q), f64(k), f64(v), f64(do), SCALE, causal)
    check_grad(f"dQ {shape}", f64(dq), rq)
    check_grad(f"dK {shape}", f64(dk), rk)
    check_grad(f"dV {shape}", f64(dv), rv)


def test_backward_full_workload_sampled():
    """Workload 2's shape (4 x 32 heads x 4096, causal) in the bench launch configuration: three heads."""
    fa = need_gpu()
    w = workloads.WORKLOADS[2]
    say(f"[case] backward workload {w.name}")
    (q, k, v, do), (dq, dk, dv) = run(fa, w.B, w.Hq, w.Hkv, w.S, w.S, True, w.wid)
    for b, h in [(0, 0), (2, 17), (3, 31)]:
        rq, rk, rv = oracle.attention_head_backward(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h]),
                                                    w.scale, True)
        check_grad(f"dQ workload (b={b}, h={h})", f64(dq[b, h]), rq)
        check_grad(f"dK workload (b={b}, h={h})", f64(dk[b, h]), rk)
        check_grad(f"dV workload (b={b}, h={h})", f64(dv[b, h]), rv)
