"""Shared-prefix (cascade) decode on the CPU: the host plan and argument checks.

No test here launches a kernel.
"""
import ctypes as C
import os

import numpy as np
import pytest

import exact_attention_20_amd as fa
import workloads

from test_abi_cpu import declared_functions


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.skip("libfa.so not built")
    return fa.load()


def test_header_declares_cascade_calls():
    names = declared_functions()
    for n in ("fa_decode_plan_cascade", "fa_decode_cascade_workspace_size", "fa_decode_plan_cascade_host"):
        assert n in names


CASES = [
    # (groups, suffix lengths, prefix pages per group, Hq, Hkv)
    ([0, 0, -1, 1, 0], [0, 70, 5, 64, 130], [2, 1], 4, 2),
    ([0] * 80 + [-1, 1], [100] * 80 + [3000, 1], [40, 0], 32, 8),
    ([0, 1, 2], [0, 0, 0], [1, 3, 64], 8, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{len(c[0])}-G{c[3] // c[4]}")
def test_plan_covers_prefix_and_suffix_once(lib, case):
    """Every (request, head) gets each prefix page from exactly one prefix item and each
    suffix page from exactly one suffix item; slots are distinct and within the count."""
    groups, suffix, pp, Hq, Hkv = case
    r = workloads.shared_prefix_inputs(Hq, Hkv, 128, groups, suffix, pp, wid=60)
    stride = r.page_table.shape[1]
    items, pitems, splits, ns = fa.fa_decode_plan_cascade_host(r.seqlens, stride, Hq, Hkv, r.prefix_group,
                                                                r.prefix_pages, num_cus=16)
    G = Hq // Hkv
    L = r.seqlens.numpy()
    B = len(groups)
    members = {j: [b for b in range(B) if groups[b] == j] for j in range(len(pp))}
    seen = {}  # (b, h, page) -> slot
    for off, g, row0, nrows, p0, p1, slot, first in pitems.tolist():
        assert nrows <= 256 and 0 <= g < Hkv
        for f in range(row0, row0 + nrows):
            j = groups[first]
            b = members[j][f // G]
            assert r.page_table[b, :pp[j]].tolist() == r.page_table[first, :pp[j]].tolist()
            h = g * G + f % G
            for p in range(p0, p1):
                assert (b, h, p) not in seen
                seen[(b, h, p)] = slot
    for b, gs, p0, p1 in items.tolist():
        g, s = gs & 255, gs >> 8
        for h in range(g * G, g * G + G):
            for p in range(p0, p1):
                assert (b, h, p) not in seen
                seen[(b, h, p)] = s
    for b in range(B):
        pages = (int(L[b]) + 63) // 64
        for h in range(Hq):
            got = sorted(p for (bb, hh, p) in seen if bb == b and hh == h)
            assert got == list(range(pages)), f"request {b} head {h} pages {got}"
            slots = {seen[(b, h, p)] for p in got}
            assert slots == set(range(int(splits[b]))) or (pages == 0 and splits[b] == 0)
    assert ns == int(splits.max())


def _plan(lib, **kw):
    a = dict(L=[128, 200], table=[0, 1, -1, -1, 0, 1, 2, 3], B=2, stride=4, P=4, Hq=4, Hkv=2, D=128,
             group=[0, 0], pp=[2], ng=1, ws=C.c_void_p(256), ws_bytes=1 << 24)
    a.update(kw)
    arr = lambda x: (C.c_int32 * len(x))(*x)  # noqa: E731
    Lb, tb, gb, pb = arr(a["L"]), arr(a["table"]), arr(a["group"]), arr(a["pp"] or [0])
    i32 = C.POINTER(C.c_int32)
    h, ns = C.c_void_p(), C.c_int(0)
    st = lib.fa_decode_plan_cascade(C.cast(Lb, i32), C.cast(tb, i32), a["B"], a["stride"], a["P"], a["Hq"], a["Hkv"],
                                    a["D"], C.cast(gb, i32), C.cast(pb, i32), a["ng"], 4, a["ws"], a["ws_bytes"], None,
                                    C.byref(h), C.byref(ns))
    assert not h.value
    return st


@pytest.mark.parametrize("kw,code", [
    (dict(group=[0, 2]), 1),                                  # group id out of range
    (dict(pp=[3]), 1),                                        # request 0 shorter than the prefix
    (dict(table=[0, 1, -1, -1, 0, 2, 1, 3]), 1),              # request 1 does not share page 1
    (dict(table=[0, 1, -1, -1, 0, 1, 2, 9]), 1),              # page id outside the pool
    (dict(Hq=3), 1), (dict(D=64), 2), (dict(ng=-1), 1),
    (dict(ws=None), 3), (dict(ws_bytes=16), 3),
])
def test_cascade_plan_rejects_before_device_work(lib, kw, code):
    assert _plan(lib, **kw) == code
    assert lib.fa_last_error().decode()
