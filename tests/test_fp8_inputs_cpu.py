"""The fp8 input quantisers against the e4m3fn format's rounding bound.

Both quantisers (per (page, KV head) for the paged cache, per (batch, head)
for fp8 prefill) take scale = max|x| / 448 and round x / scale to the nearest
e4m3fn value. e4m3fn keeps 3 mantissa bits, so a normal code (|x/scale| >= 2^-6)
is within half an ulp, 2^-4 of its magnitude, and a subnormal code within
half the subnormal step, 2^-10, times the scale. The largest magnitude maps
onto 448 exactly, nothing overflows to NaN, and unused page tails hold NaN
codes when asked. Codes are decoded with the oracle's e4m3fn decoder, which
its own pins tie to the format definition and to torch's cast.
"""
import numpy as np
import torch

import oracle
import workloads


def _check_bound(x, codes, scale):
    deq = oracle.e4m3fn_to_float(codes) * scale
    y = np.abs(x) / scale
    err = np.abs(x - deq)
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)), "normal-range error above half an ulp"
    sub = ~normal
    assert np.all(err[sub] <= 2.0 ** -10 * np.broadcast_to(scale, x.shape)[sub] * (1 + 1e-6)), \
        "subnormal-range error above half a step"


def test_prefill_quantiser_half_ulp():
    g = np.random.default_rng(5)
    x = g.standard_normal((2, 3, 40, 16)).astype(np.float32)
    x[0, 1, :4] *= 1e-4        # rows far below the head's max: subnormal codes
    x[1, 2, 5, 7] = 30.0        # one outlier sets that head's scale
    codes, scale = workloads.quantise_heads_e4m3fn(x)
    c, s = codes.numpy(), scale.numpy().astype(np.float64)[:, :, None, None]
    assert not np.isnan(oracle.e4m3fn_to_float(c)).any()
    _check_bound(x.astype(np.float64), c, s)
    dq = oracle.e4m3fn_to_float(c)
    assert np.all(np.abs(dq).reshape(2, 3, -1).max(axis=2) == 448.0), "max |x| must map onto 448"
    assert (np.abs(x[0, 1]) / s[0, 1] < 2.0 ** -6).any(), "the small head should reach the subnormal codes"


def test_paged_quantiser_half_ulp_and_tails():
    L = [70, 64, 1]
    kv = workloads.paged_inputs(len(L), 4, 2, 16, "fp8", L, 91, nan_tails=True)
    # the float32 draws the quantiser started from (same seeded stream)
    k32 = workloads.rng(91, workloads.STREAM_K).standard_normal(size=tuple(kv.k_pages.shape), dtype=np.float32)
    table, ks = kv.page_table.numpy(), kv.k_scale.numpy().astype(np.float64)
    kc = kv.k_pages.numpy()
    for b, n in enumerate(L):
        for j in range((n + 63) // 64):
            pid = int(table[b, j])
            valid = min(64, n - 64 * j)
            for g in range(2):
                x = k32[pid, g, :valid].astype(np.float64)
                _check_bound(x, kc[pid, g, :valid], ks[pid, g])
                assert np.abs(oracle.e4m3fn_to_float(kc[pid, g, :valid])).max() == 448.0
                if valid < 64:
                    assert np.isnan(oracle.e4m3fn_to_float(kc[pid, g, valid:])).all(), "tail not NaN"
