"""The device status word: kernels that meet bad device page-table metadata
(a page id outside the pool, an appended token past its table row or with a
negative position) skip it and set a bit that fa_device_status reads back.
The plans are built from valid host copies; only the device copies are
corrupted afterwards, which no host check can see."""
import numpy as np
import pytest
import torch

import workloads
from parity import need_gpu, say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / np.sqrt(128)))
BAD = 1 << 20   # a page id far outside every pool here


def ragged_dev(fa, wid):
    r = workloads.ragged_inputs(8, 2, 128, [70, 5, 130], [0, 100, 60], wid=wid, extra_pages=2, poison=False)
    d = dict(q=r.q.cuda(), kn=r.k_new.cuda(), vn=r.v_new.cuda(), k=r.k_pages.cuda(), v=r.v_pages.cuda(),
             pt=r.page_table.cuda(), sl=r.seqlens.cuda(), cu=r.cu_seqlens_q.cuda())
    return r, d


def test_clean_calls_leave_it_clear():
    fa = need_gpu()
    fa.device_status(clear=True)
    r, d = ragged_dev(fa, 60)
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, 8, 2)
    fa.prefill_paged(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], SCALE)
    kv = workloads.paged_inputs(3, 8, 2, 128, "bf16", [1, 64, 300], 61, nan_tails=False)
    dplan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, 8, 2, 128, fa.BF16, 0)
    fa.decode(dplan, kv.q.cuda(), kv.k_pages.cuda(), kv.v_pages.cuda(), kv.page_table.cuda(),
              kv.seqlens.cuda(), None, None, SCALE)
    assert fa.device_status() == 0


def test_append_reports_bad_page_and_position():
    fa = need_gpu()
    fa.device_status(clear=True)
    r, d = ragged_dev(fa, 62)
    pt = d["pt"].clone()
    pt[0, 0] = BAD                      # request 0's first page: outside the pool
    say("[case] kv_append with a bad page id")
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], pt, d["sl"], d["cu"])
    assert fa.device_status() == fa.STATUS_BAD_PAGE
    assert fa.device_status() == 0      # cleared by the read before
    sl = d["sl"].clone()
    sl[1] = 2                           # 5 new tokens but a length of 2: negative positions
    say("[case] kv_append with negative positions")
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], sl, d["cu"])
    assert fa.device_status() == fa.STATUS_BAD_POSITION


def test_decode_reports_bad_page():
    fa = need_gpu()
    fa.device_status(clear=True)
    kv = workloads.paged_inputs(3, 8, 2, 128, "bf16", [1, 64, 300], 63, nan_tails=False)
    plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, 8, 2, 128, fa.BF16, 0)
    pt = kv.page_table.cuda()
    pt[2, 1] = BAD                      # request 2's second page
    say("[case] decode with a bad page id")
    out, lse = fa.decode(plan, kv.q.cuda(), kv.k_pages.cuda(), kv.v_pages.cuda(), pt, kv.seqlens.cuda(),
                         None, None, SCALE)
    assert fa.device_status() == fa.STATUS_BAD_PAGE
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()   # the page reads as zeros


def test_paged_prefill_reports_bad_page():
    fa = need_gpu()
    fa.device_status(clear=True)
    r, d = ragged_dev(fa, 64)
    fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"])
    plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, 8, 2)
    assert fa.device_status() == 0
    pt = d["pt"].clone()
    pt[2, 0] = BAD                      # request 2's first page
    say("[case] paged prefill with a bad page id")
    out, lse = fa.prefill_paged(plan, d["q"], d["k"], d["v"], pt, d["sl"], d["cu"], SCALE)
    assert fa.device_status() == fa.STATUS_BAD_PAGE
    assert torch.isfinite(out.float()).all()
