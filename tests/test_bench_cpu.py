"""CPU checks of bench.py's measurement arithmetic: the algorithmic FLOP and
byte counts behind every roofline, against brute-force counts over small
shapes; the rule that a counter summary only yields traffic while its kernel
source is unchanged; and the per-dispatch reading of a counter CSV."""
import itertools
import os
import types

import numpy as np
import pytest

import bench


def _w(**kw):
    return types.SimpleNamespace(**kw)


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 1, 1, 1, 8), (2, 3, 1, 7, 8), (1, 4, 2, 13, 16)])
def test_prefill_flops_counts_causal_pairs(B, Hq, Hkv, S, D):
    # Two products per visible (query, key) pair, 2 FLOPs per multiply-add.
    visible = sum(1 for i, j in itertools.product(range(S), range(S)) if j <= i)
    assert bench.prefill_flops(_w(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D)) == 4.0 * B * Hq * D * visible


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 2, 2, 5, 8), (3, 8, 2, 9, 128)])
def test_prefill_bytes_is_tensor_sizes(B, Hq, Hkv, S, D):
    q = o = B * Hq * S * D * 2
    k = v = B * Hkv * S * D * 2
    lse = B * Hq * S * 4
    assert bench.prefill_bytes(_w(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D)) == q + k + v + o + lse


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_decode_bytes_brute_force(kv_dtype):
    L = [1, 63, 64, 65, 500, 0]
    w = _w(B=len(L), Hq=8, Hkv=2, D=16, kv_dtype=kv_dtype)
    eb = 1 if kv_dtype == "fp8" else 2
    expect = 0
    for n in L:
        pages = -(-n // 64)
        expect += n * w.Hkv * w.D * eb * 2              # each valid K and V row once
        if kv_dtype == "fp8":
            expect += pages * w.Hkv * 4 * 2             # K and V scale per (page, head)
        expect += pages * 4 + 4                         # its page-table entries and its length
        expect += w.Hq * w.D * 2 * 2 + w.Hq * 4         # q in, out and lse out
    assert bench.decode_bytes(L, w) == expect


def test_ragged_flops_brute_force():
    nq, pre = [3, 1, 5], [0, 7, 64]
    w = _w(Hq=4, D=8)
    pairs = 0
    for n, p in zip(nq, pre):
        for i in range(n):          # new token i sees the prefix and new tokens 0..i
            pairs += sum(1 for key in range(p + n) if key <= p + i)
    assert bench.ragged_flops(nq, pre, w) == 4.0 * w.Hq * w.D * pairs


def test_cascade_bytes_reads_each_prefix_once():
    w = _w(B=4, Hq=8, Hkv=2, D=16, kv_dtype="bf16")
    L = np.array([700, 900, 200, 64 * 3 + 5])
    # Without groups the cascade reads what plain decode reads.
    assert bench.cascade_bytes(L, [-1] * 4, [], w) == bench.decode_bytes(L, w)
    # Requests 0, 1 and 3 share a 3-page prefix: it is read once instead of three times.
    row = w.Hkv * w.D * 2 * 2
    saved = 2 * 3 * 64 * row
    assert bench.cascade_bytes(L, [0, 0, -1, 0], [3], w) == bench.decode_bytes(L, w) - saved


def test_read_traffic_needs_the_profiled_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "kernel.hip"
    src.write_text("// version 1\n")
    (tmp_path / "profiles" / "leg_traffic.txt").write_text(
        "# header: with a colon\n"
        f"source_sha256_16: {bench.source_sha('kernel.hip')}\n"
        "fetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 234\n")
    assert bench.read_traffic("leg_traffic.txt", "kernel.hip") == 1234
    src.write_text("// version 2\n")
    assert bench.read_traffic("leg_traffic.txt", "kernel.hip") is None
    assert bench.read_traffic("missing.txt", "kernel.hip") is None


def test_pmc_dispatches_keeps_each_dispatch_apart(tmp_path):
    head = ('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
    rows = [
        (1, "void fa::k<1>(int)", "SQ_BUSY_CYCLES", 100.0, 1000, 3000),
        (1, "void fa::k<1>(int)", "SQ_BUSY_CYCLES", 60.0, 1000, 3000),   # second row of the same dispatch
        (2, "void other(int)", "SQ_BUSY_CYCLES", 7.0, 4000, 5000),
        (3, "void fa::k<1>(int)", "SQ_BUSY_CYCLES", 320.0, 6000, 7000),
    ]
    body = "".join(f'{d},"{k}","{c}",{v},{s},{e}\n' for d, k, c, v, s, e in rows)
    (tmp_path / "pmc_counter_collection.csv").write_text(head + body)
    disp = bench._pmc_dispatches(str(tmp_path), "fa::k<1>")
    assert [c["SQ_BUSY_CYCLES"] for c, _ in disp] == [160.0, 320.0]
    assert [t for _, t in disp] == [2.0, 1.0]  # microseconds, from each dispatch's own timestamps


def test_time_calls_divides_each_run_by_its_calls(monkeypatch):
    # Fake events on a fake clock: each call advances it by the next duration.
    import sys
    durs = iter([1.0, 2.0] + [float(x) for x in range(3, 28)])
    clock = [0.0]

    class Ev:
        def __init__(self, enable_timing=True):
            self.t = None

        def record(self, stream=None):
            self.t = clock[0]

        def elapsed_time(self, other):
            return other.t - self.t

    def fn():
        clock[0] += next(durs)

    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=Ev, synchronize=lambda: None))
    monkeypatch.setitem(sys.modules, "torch", fake)
    out = bench.time_calls(fn, steps=25, warmup=2, stream=None, prewarm_s=0.0, runs=5)
    # warmup takes 1 and 2; 25 calls make two runs (at least 10 calls each) of
    # 13 and 12 calls: 3..15 and 16..27
    assert out == [9.0] * 13 + [21.5] * 12
    assert sum(out) == sum(range(3, 28))     # the mean is total time over calls
