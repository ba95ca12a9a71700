"""The backward entry point that allocates nothing, against the one that takes a workspace.

fa_prefill_bwd_noalloc runs the backward's kernels with the library's static
device scratch in place of the caller's workspace. Through the C ABI, two calls
in a row (the second on a smaller problem, so stale rows of the first are left
in the shared scratch) must give dQ, dK, dV identical to fa_prefill_bwd on the
same inputs with a workspace of its own, and both must meet the backward's
parity gate against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import f64, need_gpu, say

pytestmark = pytest.mark.gpu


def _grads(fa, fn, q, k, v, o, lse, do, scale, **kw):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fn(q, k, v, o, lse, do, dq, dk, dv, True, scale, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def _gate(name, got, ref):
    g, r = f64(got), ref
    mx = np.abs(g - r).max()
    rms = np.sqrt(np.mean((g - r) ** 2))
    say(f"[parity] {name}: max_abs={mx:.3e} rms={rms:.3e}")
    assert mx <= 2e-2 * max(np.abs(r).max(), 1e-2)
    assert rms <= 1e-2 * max(np.sqrt(np.mean(r ** 2)), 1e-3)


@pytest.mark.parametrize("shapes", [[(2, 8, 2, 700, 700), (1, 4, 4, 300, 300)],
                                    [(1, 8, 8, 1030, 1030), (1, 2, 1, 65, 65)]])
def test_noalloc_backward_matches_workspace_backward(shapes):
    fa = need_gpu()
    for i, (B, Hq, Hkv, Sq, Sk) in enumerate(shapes):
        say(f"[case] backward noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} S={Sq}")
        q, k, v, do = workloads.backward_inputs(B, Hq, Hkv, Sq, Sk, 128, 60 + i)
        scale = float(np.float32(1 / np.sqrt(128)))
        q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        o, lse = fa.prefill(q, k, v, causal=True, scale=scale)
        ref = _grads(fa, fa.fa_prefill_bwd, q, k, v, o, lse, do, scale)
        got = _grads(fa, fa.fa_prefill_bwd_noalloc, q, k, v, o, lse, do, scale)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from fa_prefill_bwd"
        dq, dk, dv = oracle.prefill_backward(f64(q), f64(k), f64(v), f64(do), scale, True)
        for name, a, r in zip(("dq", "dk", "dv"), got, (dq, dk, dv)):
            _gate(f"noalloc call {i} {name}", a, r)
