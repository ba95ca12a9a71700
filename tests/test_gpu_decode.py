"""Paged decode parity: plan + split-KV + LSE merge (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check, f64, need_gpu, say

SCALE = float(np.float32(1 / np.sqrt(128)))

pytestmark = pytest.mark.gpu


def to_dev(kv):
    d = dict(q=kv.q.cuda(), k=kv.k_pages.cuda(), v=kv.v_pages.cuda(), pt=kv.page_table.cuda(),
             sl=kv.seqlens.cuda())
    d["ks"] = kv.k_scale.cuda() if kv.k_scale is not None else None
    d["vs"] = kv.v_scale.cuda() if kv.v_scale is not None else None
    return d


def oracle_decode(kv, scale, requests=None):
    if kv.kv_dtype == "fp8":
        kp, vp = kv.k_pages.numpy(), kv.v_pages.numpy()
        ks, vs = kv.k_scale.numpy(), kv.v_scale.numpy()
    else:
        kp, vp = kv.k_pages.float().numpy(), kv.v_pages.float().numpy()
        ks = vs = None
    return oracle.paged_decode(f64(kv.q), kp, vp, kv.page_table.numpy(), kv.seqlens.numpy(), scale,
                               ks, vs, requests=requests)


def run(fa, kv, d, num_splits=0, scale=None):
    dt = fa.BF16 if kv.kv_dtype == "bf16" else fa.FP8_E4M3FN
    B, Hq, D = kv.q.shape
    Hkv = kv.k_pages.shape[1]
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, D, dt, num_splits)
    out, lse = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["ks"], d["vs"], scale)
    torch.cuda.synchronize()
    return out, lse, plan


CASES = [
    # (lengths, Hq, Hkv, kv_dtype)
    ([1, 63, 64, 65, 1000], 8, 2, "bf16"),
    ([1, 63, 64, 65, 1000], 8, 2, "fp8"),
    ([700, 0, 129, 4097], 8, 8, "bf16"),
    ([300, 2000], 4, 2, "bf16"),
    ([5000, 17, 640], 16, 2, "bf16"),
    ([5000, 17, 640], 16, 2, "fp8"),
    ([1, 700, 2049], 32, 2, "bf16"),
    ([1, 700, 2049], 32, 2, "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}-G{c[1] // c[2]}-L{len(c[0])}")
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_small_batches(case, num_splits):
    fa = need_gpu()
    L, Hq, Hkv, dt = case
    say(f"[case] decode L={L} Hq={Hq} Hkv={Hkv} {dt} num_splits={num_splits}")
    kv = workloads.paged_inputs(len(L), Hq, Hkv, 128, dt, L, 31, nan_tails=True, max_pages=80, extra_pages=3)
    d = to_dev(kv)
    scale = float(np.float32(1 / np.sqrt(128)))
    out, lse, _ = run(fa, kv, d, num_splits, scale)
    O, LSE = oracle_decode(kv, scale)
    empty = kv.seqlens.numpy() == 0
    if empty.any():
        assert torch.all(out[torch.from_numpy(empty)] == 0)
        assert torch.all(torch.isneginf(lse[torch.from_numpy(empty)]))
    check(f"decode {case} splits={num_splits}", f64(out), O, f64(lse), LSE, "fp8" if dt == "fp8" else "bf16")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_gather_bit_exact(dt):
    """The kernel's page-table indexing, exported as a gather, reproduces the logical sequence exactly."""
    fa = need_gpu()
    L = [1, 64, 65, 3000]
    kv = workloads.paged_inputs(4, 8, 2, 128, dt, L, 32, nan_tails=True)
    d = to_dev(kv)
    kdt = fa.BF16 if dt == "bf16" else fa.FP8_E4M3FN
    for b, Lb in enumerate(L):
        for g in range(2):
            got = fa.fa_debug_gather_kv(d["k"], kdt, d["pt"], kv.num_pages, b, Lb, g)
            torch.cuda.synchronize()
            raw = kv.k_pages.float().numpy() if dt == "bf16" else kv.k_pages.numpy()
            ref = oracle.gather_pages(raw, kv.page_table[b].numpy(), Lb, g)
            gotn = got.cpu().float().numpy() if dt == "bf16" else got.cpu().numpy().astype(np.float64)
            assert np.array_equal(gotn, ref), f"gather mismatch b={b} g={g}"


def test_page_permutation_bitwise():
    """The same logical cache under a different physical page permutation gives identical bits."""
    fa = need_gpu()
    L = [900, 130, 2500]
    kv = workloads.paged_inputs(3, 8, 2, 128, "bf16", L, 33, nan_tails=True)
    d = to_dev(kv)
    out1, lse1, _ = run(fa, kv, d, 0)
    P = kv.num_pages
    perm = torch.from_numpy(np.random.default_rng(5).permutation(P).astype(np.int64))
    k2 = torch.empty_like(kv.k_pages)
    v2 = torch.empty_like(kv.v_pages)
    k2[perm] = kv.k_pages
    v2[perm] = kv.v_pages
    pt2 = kv.page_table.clone()
    used = pt2 >= 0
    pt2[used] = perm[pt2[used].long()].int()
    kv2 = workloads.PagedKV(kv.q, k2, v2, None, None, pt2, kv.seqlens, "bf16", P)
    out2, lse2, _ = run(fa, kv2, to_dev(kv2), 0)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_num_splits_invariance():
    fa = need_gpu()
    L = [4000, 10000, 64]
    kv = workloads.paged_inputs(3, 16, 4, 128, "bf16", L, 34, nan_tails=True)
    d = to_dev(kv)
    res = [run(fa, kv, d, ns)[:2] for ns in (1, 2, 7, 0)]
    for o, l in res[1:]:
        assert (o.float() - res[0][0].float()).abs().max().item() <= 4e-3
        assert (l - res[0][1]).abs().max().item() <= 1e-4


@pytest.mark.parametrize("num_splits", [0, 3])
def test_repeated_runs_and_graph_replays(num_splits):
    """A run allocates nothing and leaves no state behind in the plan's workspace, so it can be
    captured in a graph: later runs of the same plan, eager or replays of the captured graph with
    eager runs between them, give the same bits as the first (which matches the oracle)."""
    fa = need_gpu()
    for L, Hq, Hkv in (([700, 0, 129, 4097], 8, 2), ([5000, 17, 640], 4, 2)):
        say(f"[case] repeated decode runs L={L} Hq={Hq} Hkv={Hkv} num_splits={num_splits}")
        kv = workloads.paged_inputs(len(L), Hq, Hkv, 128, "bf16", L, 36, nan_tails=True)
        d = to_dev(kv)
        plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, 128, fa.BF16, num_splits)
        args = (plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], None, None, SCALE)
        o0, l0 = fa.decode(*args)
        torch.cuda.synchronize()
        O, LSE = oracle_decode(kv, SCALE)
        check(f"decode first run {L}", f64(o0), O, f64(l0), LSE, "bf16")
        for _ in range(2):
            o, l = fa.decode(*args)
            torch.cuda.synchronize()
            assert torch.equal(o, o0) and torch.equal(l, l0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side), torch.cuda.graph(g):
            og, lg = fa.decode(*args)
        torch.cuda.synchronize()
        for _ in range(3):
            og.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(og, o0) and torch.equal(lg, l0)
            o, l = fa.decode(*args)
            torch.cuda.synchronize()
            assert torch.equal(o, o0) and torch.equal(l, l0)


WINDOW_CASES = [
    # (lengths, Hq, Hkv, kv_dtype, num_cus): planned for a small CU count so
    # that the auto plan cuts cost-balanced windows (several items per
    # workgroup, windows crossing request boundaries, padding items)
    ([3362, 320, 997, 1431, 3493, 237, 1691], 8, 2, "bf16", 16),
    ([785, 1231, 211, 2060, 2061, 167, 676, 1710, 246], 8, 2, "fp8", 16),
    ([932, 2912, 576, 2164, 699, 207, 1597], 2, 2, "bf16", 16),
    ([1784, 1727, 425, 379, 628, 947], 4, 4, "fp8", 16),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: f"{c[3]}-G{c[1] // c[2]}-B{len(c[0])}")
def test_window_plans(case):
    fa = need_gpu()
    L, Hq, Hkv, dt, cus = case
    say(f"[case] window plan L={L} Hq={Hq} Hkv={Hkv} {dt} cus={cus}")
    kv = workloads.paged_inputs(len(L), Hq, Hkv, 128, dt, L, 36, nan_tails=True)
    items, _, _, _, grid = fa.fa_decode_plan_host(kv.seqlens, kv.page_table.shape[1], Hq, Hkv, 0, cus)
    assert grid < len(items), "the case must exercise a window plan"
    d = to_dev(kv)
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, Hq, Hkv, 128,
                             fa.BF16 if dt == "bf16" else fa.FP8_E4M3FN, 0, cus)
    out, lse = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["ks"], d["vs"], SCALE)
    torch.cuda.synchronize()
    O, LSE = oracle_decode(kv, SCALE)
    check(f"window plan {case}", f64(out), O, f64(lse), LSE, dt)


def test_run_rejects_a_foreign_workspace():
    """A run handed any buffer but the plan's own is refused before a launch
    (the work list lives in the plan's workspace); the plan still runs after."""
    fa = need_gpu()
    kv = workloads.paged_inputs(2, 8, 2, 128, "bf16", [300, 1000], 35, nan_tails=True)
    d = to_dev(kv)
    out, lse, plan = run(fa, kv, d, 0)
    own = plan.workspace
    plan.workspace = torch.zeros_like(own)
    with pytest.raises(fa.FAError) as e:
        fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["ks"], d["vs"])
    assert e.value.status == 1 and "workspace" in str(e.value)
    plan.workspace = own
    out2, lse2 = fa.decode(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["ks"], d["vs"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("wid", [4, 5])
def test_full_workload(wid):
    """Full-size decode workloads in the benchmark's launch configuration (plan-chosen splits)."""
    fa = need_gpu()
    w = workloads.WORKLOADS[wid]
    say(f"[case] full decode workload {wid} {w.name}")
    kv = workloads.workload_paged_inputs(w, nan_tails=True)
    d = to_dev(kv)
    out, lse, plan = run(fa, kv, d, 0, w.scale)
    say(f"[plan] items={len(plan.items()[0])} num_splits={plan.num_splits} pages={kv.num_pages}")
    rng = np.random.default_rng(wid)
    L = kv.seqlens.numpy()
    reqs = sorted({int(np.argmax(L)), int(np.argmin(L))} |
                  set(rng.choice(w.B, size=min(w.B, 12), replace=False).tolist()))
    O, LSE = oracle_decode(kv, w.scale, requests=reqs)
    check(f"decode workload {wid} ({len(reqs)} requests)", f64(out[reqs]), O, f64(lse[reqs]), LSE,
          "fp8" if w.kv_dtype == "fp8" else "bf16")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
