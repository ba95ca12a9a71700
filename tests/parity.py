"""Helpers for GPU-vs-oracle parity: metrics, gates and tensor conversions."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Gates for the HIP path against the fp64 oracle.
#  bf16 outputs: max |dO| <= 1e-2, relative RMS <= 5e-3, max |dLSE| <= 1e-3.
#  fp8-KV decode: max |dO| <= 5e-2, max |dLSE| <= 1e-3 (against the oracle on
#  the dequantised fp8 values, so quantisation error is not counted).
#  fp32 prefill: fp32 accumulation of exact inputs; rounding-order error only.
GATES = {
    "bf16": dict(max_abs=1e-2, rel_rms=5e-3, lse_abs=1e-3),
    "fp8": dict(max_abs=5e-2, rel_rms=None, lse_abs=1e-3),
    "f32": dict(max_abs=1e-4, rel_rms=1e-5, lse_abs=1e-4),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_20_amd as fa
    fa.load()  # raises if the HIP library is missing: never a silent fallback
    return fa


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def metrics(o_gpu, o_ref, lse_gpu, lse_ref):
    o_gpu, o_ref = np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64)
    lse_gpu, lse_ref = np.asarray(lse_gpu, np.float64), np.asarray(lse_ref, np.float64)
    d = np.abs(o_gpu - o_ref)
    rms = float(np.sqrt(np.sum((o_gpu - o_ref) ** 2)) / max(np.sqrt(np.sum(o_ref ** 2)), 1e-300))
    both_ninf = np.isneginf(lse_gpu) & np.isneginf(lse_ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf on rows with no key; masked just below
        dl = np.where(both_ninf, 0.0, np.abs(lse_gpu - lse_ref))
    return dict(max_abs=float(d.max(initial=0.0)) if np.all(np.isfinite(d)) else float("inf"),
                rel_rms=rms if np.isfinite(rms) else float("inf"),
                lse_abs=float(dl.max(initial=0.0)) if np.all(np.isfinite(dl)) else float("inf"))


def check(name, o_gpu, o_ref, lse_gpu, lse_ref, gate):
    m = metrics(o_gpu, o_ref, lse_gpu, lse_ref)
    g = GATES[gate]
    say(f"[parity] {name}: max_abs={m['max_abs']:.3e} rel_rms={m['rel_rms']:.3e} lse_abs={m['lse_abs']:.3e} gate={gate}")
    assert m["max_abs"] <= g["max_abs"], f"{name}: max_abs {m['max_abs']:.3e} > {g['max_abs']}"
    if g["rel_rms"] is not None:
        assert m["rel_rms"] <= g["rel_rms"], f"{name}: rel_rms {m['rel_rms']:.3e} > {g['rel_rms']}"
    assert m["lse_abs"] <= g["lse_abs"], f"{name}: lse_abs {m['lse_abs']:.3e} > {g['lse_abs']}"
    return m


def fp8_weight_bound(q, k, v, scale, causal, rows=None):
    """Per-element bound on |O_gpu - O| when the softmax weights enter P V as
    e4m3 (round to nearest even) and O is divided by the sum of the unrounded
    weights. In the frame of the row's true max, p_j = exp(s_j - max) <= 1;
    the kernel's (lazy) frame only scales p up, which never increases the
    relative error. An e4m3 value carries relative error <= 2^-4 when normal
    (p >= 2^-6) and absolute error <= 2^-10 when subnormal, so
        |O_gpu - O| <= sum_j max(2^-4 p_j, 2^-10) |v_j| / sum_j p_j.
    ``q`` [Sq, D], ``k``/``v`` [Sk, D] float64 (one head). Returns [R, D]."""
    import oracle
    Sq, Sk = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    s = oracle.scores(q[rows], k, scale)
    ok = oracle.causal_allowed(rows, Sq, Sk) if causal else np.ones_like(s, dtype=bool)
    s = np.where(ok, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.where(ok, np.exp(s - np.where(np.isfinite(mx), mx, 0.0)), 0.0)
    w = np.where(ok, np.maximum(p * 2.0 ** -4, 2.0 ** -10), 0.0)
    den = p.sum(axis=1, keepdims=True)
    return (w @ np.abs(v)) / np.where(den > 0, den, 1.0)


def check_fp8_prefill(name, o_gpu, o_ref, bound, lse_gpu, lse_ref):
    """fp8 prefill gate: every element within its weight-rounding bound plus
    bf16 output rounding (2^-8 |O|) and fp32 slack (1e-5); LSE within 1e-3."""
    o_gpu, o_ref = np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64)
    m = metrics(o_gpu, o_ref, lse_gpu, lse_ref)
    err = np.abs(o_gpu - o_ref)
    lim = np.asarray(bound) + 2.0 ** -8 * np.abs(o_ref) + 1e-5
    ratio = float((err / lim).max(initial=0.0))
    say(f"[parity] {name}: max_abs={m['max_abs']:.3e} rel_rms={m['rel_rms']:.3e} lse_abs={m['lse_abs']:.3e} "
        f"max(err/bound)={ratio:.3f} gate=fp8-prefill")
    assert np.all(np.isfinite(o_gpu)), f"{name}: non-finite output"
    assert ratio <= 1.0, f"{name}: error exceeds the fp8 weight-rounding bound (ratio {ratio:.3f})"
    assert m["lse_abs"] <= 1e-3, f"{name}: lse_abs {m['lse_abs']:.3e} > 1e-3"
    return m, ratio
