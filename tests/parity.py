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
