"""Shared-prefix (cascade) decode (through the C ABI) against the oracle's decode definition."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check, f64, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))


def to_dev(r):
    return dict(q=r.q.cuda(), k=r.k_pages.cuda(), v=r.v_pages.cuda(), pt=r.page_table.cuda(), sl=r.seqlens.cuda())


def run_cascade(fa, r, d, scale=SCALE):
    Hq, Hkv = r.q.shape[1], r.k_pages.shape[1]
    plan = fa.fa_decode_plan_cascade(r.seqlens, r.page_table, r.num_pages, Hq, Hkv, r.prefix_group,
                                     r.prefix_pages.tolist())
    out, lse = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], scale=scale)
    torch.cuda.synchronize()
    return out, lse, plan


def oracle_decode(r, scale=SCALE, requests=None):
    return oracle.paged_decode(f64(r.q), r.k_pages.float().numpy(), r.v_pages.float().numpy(),
                               r.page_table.numpy(), r.seqlens.numpy(), scale, requests=requests)


CASES = [
    # (groups, suffix lengths, prefix pages per group, Hq, Hkv)
    ([0, 0, -1, 1, 0], [0, 70, 5, 64, 130], [2, 1], 8, 2),
    ([0] * 70 + [-1, 1, 1], [17] * 35 + [1000] * 35 + [3000, 1, 0], [20, 3], 32, 8),
    ([0, 0, 0], [0, 0, 0], [1], 4, 4),
    ([0, 1, 2, 2], [63, 64, 65, 0], [5, 0, 40], 16, 1),
    ([0, 0], [1, 1], [130], 32, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{len(c[0])}-G{c[3] // c[4]}-P{sum(c[2])}")
def test_cascade_matches_decode_definition(case):
    fa = need_gpu()
    groups, suffix, pp, Hq, Hkv = case
    say(f"[case] cascade groups={len(pp)} B={len(groups)} prefix_pages={pp} Hq={Hq} Hkv={Hkv}")
    r = workloads.shared_prefix_inputs(Hq, Hkv, 128, groups, suffix, pp, wid=61, nan_tails=True)
    out, lse, plan = run_cascade(fa, r, to_dev(r))
    O, LSE = oracle_decode(r)
    check(f"cascade {len(groups)} requests", f64(out), O, f64(lse), LSE, "bf16")


def test_cascade_agrees_with_plain_decode():
    """The same batch planned as an ordinary decode gives the same result up to rounding order."""
    fa = need_gpu()
    r = workloads.shared_prefix_inputs(32, 8, 128, [0] * 40 + [1] * 24, [500] * 64, [64, 16], wid=62)
    d = to_dev(r)
    out_c, lse_c, _ = run_cascade(fa, r, d)
    plan = fa.fa_decode_plan(r.seqlens, r.page_table, r.num_pages, 32, 8, 128, fa.BF16, 0)
    out_p, lse_p = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], scale=SCALE)
    torch.cuda.synchronize()
    assert (out_c.float() - out_p.float()).abs().max().item() <= 4e-3
    assert (lse_c - lse_p).abs().max().item() <= 1e-4


def test_full_workload():
    """The shared-prefix workload at full size, in the benchmark's launch configuration."""
    fa = need_gpu()
    w = workloads.WORKLOADS[7]
    say(f"[case] full shared-prefix workload {w.name}")
    r = workloads.workload_shared_prefix_inputs(w)
    out, lse, plan = run_cascade(fa, r, to_dev(r), w.scale)
    say(f"[plan] num_splits={plan.num_splits} pages={r.num_pages}")
    L = r.seqlens.numpy()
    rng = np.random.default_rng(7)
    reqs = sorted({int(np.argmax(L)), int(np.argmin(L))} | set(rng.choice(w.B, 10, replace=False).tolist()))
    O, LSE = oracle_decode(r, w.scale, requests=reqs)
    check(f"shared-prefix workload ({len(reqs)} requests)", f64(out[reqs]), O, f64(lse[reqs]), LSE, "bf16")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
