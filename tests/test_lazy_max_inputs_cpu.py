"""The moving-max parity inputs (test_gpu_lazy_max) are only useful if a
kernel that mishandles the lazy running max fails on them. A plain model of
the tiled loop (64-key tiles, the max moved only when a tile's scores exceed
it by more than 2^8 in exp2 units, O and the normaliser rescaled when it
moves) matches the oracle on them; the same loop with the rescale of O left
out misses the bf16 gate by far, and on the fp8 inputs of the same shape the
per-element fp8 bound as well."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import fp8_weight_bound
from test_gpu_lazy_max import SCALE, dequantise, fp8_moving_max_inputs, key_dim0, shape_query

TAU = 8.0
LOG2E = 1.4426950408889634


def tiled_lazy(q, k, v, rescale_o=True):
    """One head, causal: q, k, v [S, D] float64; returns O [S, D]."""
    S = q.shape[0]
    out = np.zeros_like(q)
    for i in range(S):
        m, l, o = -np.inf, 0.0, np.zeros(q.shape[1])
        for t0 in range(0, i + 1, 64):
            keys = np.arange(t0, min(t0 + 64, i + 1))
            s = (k[keys] @ q[i]) * SCALE * LOG2E
            mx = s.max()
            if mx > m + TAU:
                alpha = 2.0 ** (m - mx) if m > -np.inf else 0.0
                l *= alpha
                if rescale_o:
                    o *= alpha
                m = mx
            p = 2.0 ** (s - m)
            l += p.sum()
            o += p @ v[keys]
        out[i] = o / l
    return out


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
def test_missed_rescale_is_visible(shape):
    S, D = 300, 128
    q, k, v = workloads.prefill_inputs(1, 1, 1, S, S, D, "bf16", 61)
    q, k = q.float(), k.float()
    shape_query(q)
    k[..., 0] = key_dim0(np.arange(S), shape)
    q, k, v = (x.to(torch.bfloat16).double().numpy()[0, 0] for x in (q, k, v))
    O, _ = oracle.prefill(q[None, None], k[None, None], v[None, None], SCALE, True)
    good = tiled_lazy(q, k, v)
    bad = tiled_lazy(q, k, v, rescale_o=False)
    assert np.abs(good - O[0, 0]).max() < 1e-9
    assert np.abs(bad - O[0, 0]).max() > 1.0   # the bf16 gate is 1e-2


@pytest.mark.parametrize("shape", ["ramp", "sawtooth"])
def test_missed_rescale_is_visible_fp8(shape):
    S = 300
    q8, k8, v8, qs, ks, vs = fp8_moving_max_inputs(1, 1, 1, S, shape)
    q, k, v = (dequantise(c, sc)[0, 0] for c, sc in ((q8, qs), (k8, ks), (v8, vs)))
    O, _ = oracle.prefill(q[None, None], k[None, None], v[None, None], SCALE, True)
    bound = fp8_weight_bound(q, k, v, SCALE, True) + 2.0 ** -8 * np.abs(O[0, 0]) + 1e-5
    good = tiled_lazy(q, k, v)
    bad = tiled_lazy(q, k, v, rescale_o=False)
    assert (np.abs(good - O[0, 0]) / bound).max() < 1e-6
    assert (np.abs(bad - O[0, 0]) / bound).max() > 10.0   # the fp8 gate is a ratio of 1
