"""Ragged paged prefill and KV append (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check, f64, need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))


def to_dev(r):
    return dict(q=r.q.cuda(), kn=r.k_new.cuda(), vn=r.v_new.cuda(), k=r.k_pages.cuda(),
                v=r.v_pages.cuda(), pt=r.page_table.cuda(), sl=r.seqlens.cuda(),
                cu=r.cu_seqlens_q.cuda())


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def append_and_run(fa, r, d, scale=SCALE):
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    Hq, Hkv = r.q.shape[1], r.k_pages.shape[1]
    plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, Hq, Hkv)
    out, lse = fa.prefill_paged(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], scale)
    torch.cuda.synchronize()
    return out, lse, plan


def oracle_pools(r):
    """Pools after the oracle's append, as float64 (bf16 values widen exactly)."""
    kp, vp = oracle.kv_append(r.k_pages.float().numpy(), r.v_pages.float().numpy(),
                              r.page_table.numpy(), r.seqlens.numpy(), r.cu_seqlens_q.numpy(),
                              r.k_new.float().numpy(), r.v_new.float().numpy())
    return kp, vp


CASES = [
    # (new tokens per request, cached prefix per request, Hq, Hkv)
    ([1, 63, 64, 65, 300, 700], [0, 1, 100, 4000, 63, 64], 8, 2),
    ([256, 257, 1, 0, 513], [0, 0, 4095, 17, 1000], 4, 4),
    ([700, 5], [0, 0], 16, 2),
    ([129, 1000], [2000, 3], 32, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"G{c[2] // c[3]}-B{len(c[0])}")
def test_append_bit_exact(case):
    fa = need_gpu()
    nq, pre, Hq, Hkv = case
    say(f"[case] kv_append nq={nq} prefix={pre} Hkv={Hkv}")
    r = workloads.ragged_inputs(Hq, Hkv, 128, nq, pre, wid=50, max_pages=90, extra_pages=4)
    d = to_dev(r)
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(bits(r.k_pages), bits(r.v_pages), r.page_table.numpy(), r.seqlens.numpy(),
                              r.cu_seqlens_q.numpy(), bits(r.k_new), bits(r.v_new))
    assert np.array_equal(bits(d["k"]), kp), "K pool differs from the oracle's append"
    assert np.array_equal(bits(d["v"]), vp), "V pool differs from the oracle's append"


@pytest.mark.parametrize("Hkv", [12, 40])
def test_append_many_kv_heads(Hkv):
    """A token's Hkv rows go over the wavefront's 64 lanes in 16-byte units, up to 4 per lane
    at a time: 12 KV heads fill 3 of the 4 (a ragged last unit), 40 heads take three rounds,
    the last one partial."""
    fa = need_gpu()
    nq, pre = [1, 65, 130], [0, 63, 200]
    say(f"[case] kv_append Hkv={Hkv} nq={nq} prefix={pre}")
    r = workloads.ragged_inputs(Hkv, Hkv, 128, nq, pre, wid=53, extra_pages=2)
    d = to_dev(r)
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(bits(r.k_pages), bits(r.v_pages), r.page_table.numpy(), r.seqlens.numpy(),
                              r.cu_seqlens_q.numpy(), bits(r.k_new), bits(r.v_new))
    assert np.array_equal(bits(d["k"]), kp), "K pool differs from the oracle's append"
    assert np.array_equal(bits(d["v"]), vp), "V pool differs from the oracle's append"


@pytest.mark.parametrize("B", [1024, 1100])
def test_append_large_batches(B):
    """Batches of over a thousand requests (the request of each token is a binary search over
    cu_seqlens_q) give the oracle's pools bit for bit, empty requests and requests whose new
    tokens start mid-page included."""
    fa = need_gpu()
    rng = np.random.default_rng(B)
    nq = rng.integers(0, 4, B)
    pre = rng.integers(0, 130, B)
    say(f"[case] kv_append B={B} T={int(nq.sum())}")
    r = workloads.ragged_inputs(8, 2, 128, nq, pre, wid=52, extra_pages=3)
    d = to_dev(r)
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(bits(r.k_pages), bits(r.v_pages), r.page_table.numpy(), r.seqlens.numpy(),
                              r.cu_seqlens_q.numpy(), bits(r.k_new), bits(r.v_new))
    assert np.array_equal(bits(d["k"]), kp), "K pool differs from the oracle's append"
    assert np.array_equal(bits(d["v"]), vp), "V pool differs from the oracle's append"


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"G{c[2] // c[3]}-B{len(c[0])}")
def test_ragged_prefill(case):
    fa = need_gpu()
    nq, pre, Hq, Hkv = case
    say(f"[case] ragged prefill nq={nq} prefix={pre} Hq={Hq} Hkv={Hkv}")
    r = workloads.ragged_inputs(Hq, Hkv, 128, nq, pre, wid=51, max_pages=90, extra_pages=4)
    d = to_dev(r)
    out, lse, plan = append_and_run(fa, r, d)
    kp, vp = oracle_pools(r)
    O, LSE = oracle.paged_prefill(f64(r.q), kp, vp, r.page_table.numpy(), r.seqlens.numpy(),
                                  r.cu_seqlens_q.numpy(), SCALE)
    check(f"ragged prefill {case}", f64(out), O, f64(lse), LSE, "bf16")


@pytest.mark.parametrize("n,prefix", [(300, 0), (700, 1000), (64, 63)])
def test_matches_contiguous_kernel_bitwise(n, prefix):
    """One request through pages gives the same bits as the contiguous prefill
    kernel on the gathered cache (Sq = n, Sk = prefix + n, causal)."""
    fa = need_gpu()
    Hq, Hkv = 8, 2
    say(f"[case] paged vs contiguous n={n} prefix={prefix}")
    r = workloads.ragged_inputs(Hq, Hkv, 128, [n], [prefix], wid=52)
    d = to_dev(r)
    out, lse, _ = append_and_run(fa, r, d)
    L = prefix + n
    ids = r.page_table[0, :(L + 63) // 64].long().cuda()
    kc = d["k"][ids].permute(1, 0, 2, 3).reshape(Hkv, -1, 128)[:, :L].contiguous()[None]
    vc = d["v"][ids].permute(1, 0, 2, 3).reshape(Hkv, -1, 128)[:, :L].contiguous()[None]
    qc = d["q"].permute(1, 0, 2).contiguous()[None]
    oc, lc = fa.prefill(qc, kc, vc, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, oc[0].permute(1, 0, 2)), "paged output differs from the contiguous kernel"
    assert torch.equal(lse, lc[0].T), "paged LSE differs from the contiguous kernel"


def test_run_rejects_a_foreign_workspace():
    """fa_prefill_paged_run refuses a workspace other than the plan's."""
    fa = need_gpu()
    r = workloads.ragged_inputs(8, 2, 128, [300, 5], [64, 0], wid=54)
    d = to_dev(r)
    out, lse, plan = append_and_run(fa, r, d)
    own = plan.workspace
    plan.workspace = torch.zeros_like(own)
    with pytest.raises(fa.FAError) as e:
        fa.prefill_paged(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], SCALE)
    assert e.value.status == 1 and "workspace" in str(e.value)
    plan.workspace = own
    out2, lse2 = fa.prefill_paged(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_page_permutation_bitwise():
    """The same logical caches under another physical page permutation give identical bits."""
    fa = need_gpu()
    r = workloads.ragged_inputs(8, 2, 128, [300, 64, 900], [130, 2000, 0], wid=53)
    out1, lse1, _ = append_and_run(fa, r, to_dev(r))
    P = r.num_pages
    perm = torch.from_numpy(np.random.default_rng(6).permutation(P).astype(np.int64))
    k2, v2 = torch.empty_like(r.k_pages), torch.empty_like(r.v_pages)
    k2[perm], v2[perm] = r.k_pages, r.v_pages
    pt2 = r.page_table.clone()
    used = pt2 >= 0
    pt2[used] = perm[pt2[used].long()].int()
    r2 = workloads.RaggedPaged(r.q, r.k_new, r.v_new, k2, v2, pt2, r.seqlens, r.cu_seqlens_q, P)
    out2, lse2, _ = append_and_run(fa, r2, to_dev(r2))
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_full_workload():
    """The ragged prefill workload at full size, in the benchmark's launch configuration:
    append bit-exact everywhere, attention on sampled rows of sampled requests."""
    fa = need_gpu()
    w = workloads.WORKLOADS[6]
    say(f"[case] full ragged prefill workload {w.name}")
    r = workloads.workload_ragged_inputs(w)
    d = to_dev(r)
    out, lse, plan = append_and_run(fa, r, d, w.scale)
    say(f"[plan] items={plan.n_items} tokens={r.q.shape[0]} pages={r.num_pages}")
    kp, vp = oracle.kv_append(bits(r.k_pages), bits(r.v_pages), r.page_table.numpy(), r.seqlens.numpy(),
                              r.cu_seqlens_q.numpy(), bits(r.k_new), bits(r.v_new))
    assert np.array_equal(bits(d["k"]), kp) and np.array_equal(bits(d["v"]), vp), "append differs"
    kp = torch.from_numpy(kp).view(torch.bfloat16).float().numpy()
    vp = torch.from_numpy(vp).view(torch.bfloat16).float().numpy()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    L, cu = r.seqlens.numpy(), r.cu_seqlens_q.numpy()
    rng = np.random.default_rng(6)
    nq = cu[1:] - cu[:-1]
    reqs = sorted({int(np.argmax(L)), int(np.argmin(nq))} | set(rng.choice(w.B, 4, replace=False).tolist()))
    for b in reqs:
        n = int(nq[b])
        rows = np.unique(np.concatenate([[0, 255, 256, n - 1], rng.integers(0, n, 6)]))
        rows = rows[rows < n]
        O, LSE = oracle.paged_prefill_request(f64(r.q[cu[b]:cu[b + 1]]), kp, vp, r.page_table[b].numpy(),
                                              int(L[b]), w.scale, rows)
        got = out[int(cu[b]) + torch.from_numpy(rows).cuda()]
        gl = lse[int(cu[b]) + torch.from_numpy(rows).cuda()]
        check(f"ragged workload request {b} rows {len(rows)}", f64(got), O, f64(gl), LSE, "bf16")
