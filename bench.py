"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-s S] [--no-cpu-baseline]
                    [--only prefill|decode|ragged|cascade|fp8|bwd|copy] [--prefill-workload 2|3]
                    [--decode-workload 4|5]

One step = one pass of the whole path over one synthetic batch:
  * prefill: fa_prefill_fwd on the long-context causal GQA bf16 workload
    (B=1, 32 query heads over 8 KV heads, 32768 tokens, head dim 128): the
    headline ``value``, ``roofline`` and ``cpu_baseline``; and
  * decode: fa_decode_run (split-KV kernel + LSE merge) on the paged bf16
    workload (64 requests, 32/8 heads, lengths U[512, 16384]), planned once
    beforehand (the host plan is timed separately and reported).
Two more legs of the same two steps are timed on their own, each with its
own roofline and CPU baseline, and are not part of ``ms_per_step``: the
causal bf16 prefill of B=4 x 32 heads x 4096 tokens, and the long ragged
decode with fp8 (e4m3fn) KV (8 requests, log-uniform lengths in
[4096, 131072]; four copies of its pools rotate so that the 256 MB
last-level cache cannot serve it). ``prefill`` and ``decode`` hold one object
per workload, keyed by workload name.
A further leg, reported as its own ``ragged_prefill`` object, measures the
ragged paged prefill: fa_kv_append of 16 requests' new tokens (256..2048
each) into their paged caches, then fa_prefill_paged_run of those tokens over
prefix + new keys (prefixes 0..16384), each timed on its own. The
``shared_prefix_decode`` object times the cascade decode of 64 requests
sharing an 8192-token prefix (suffixes 256..4096) against plain split-KV
decode of the same batch; ``fp8_prefill`` times the fp8 (e4m3) causal prefill
of the 4 x 32-head x 4096 shape, and ``backward`` the gradients (dQ, dK, dV)
of that bf16 shape.
Inputs are resident in HBM before timing. Each leg first runs untimed for
--prewarm-s seconds (default 1 s: GPU clocks and power reach steady state)
and --warmup more times; the timed calls then run back to back in up to five
runs of at least 10 calls, each bracketed by HIP events on the stream it runs
on (time per call = a run's duration over its calls).

Prints ONE JSON line. ``value`` is the headline prefill throughput in
TFLOP/s (algorithmic FLOPs 4*B*H*D*S(S+1)/2 over the measured time); decode
legs carry HBM throughput (algorithmic bytes over the measured time).
``roofline`` is for the dominant kernel (the MFMA prefill), and
``cpu_baseline`` times the fp64 oracle on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal bf16 prefill TFLOP/s (% MFMA peak); paged decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published


def prefill_bytes(w):
    """Algorithmic HBM bytes of one prefill launch: Q, K, V read and O written
    once (bf16), the fp32 LSE written once."""
    return 2 * w.B * w.S * w.D * (2 * w.Hq + 2 * w.Hkv) + 4 * w.B * w.Hq * w.S


def prefill_flops(w):
    pairs = w.S * (w.S + 1) // 2
    return 4.0 * w.B * w.Hq * w.D * pairs


def decode_bytes(L, w):
    """Algorithmic HBM bytes of one decode step for context lengths L."""
    import numpy as np
    L = np.asarray(L).astype(np.int64)
    pages = (L + 63) // 64
    eb = 1 if w.kv_dtype == "fp8" else 2
    b = int(L.sum()) * w.Hkv * w.D * 2 * eb          # K and V of the valid tokens
    if w.kv_dtype == "fp8":
        b += int(pages.sum()) * w.Hkv * 8             # one fp32 scale per (page, head), K and V
    b += 2 * w.B * w.Hq * w.D * 2                     # q in, out
    b += w.B * w.Hq * 4                               # lse
    b += int(pages.sum()) * 4 + w.B * 4               # page-table entries read, seqlens
    return b


def ragged_flops(nq, pre, w):
    """Causal score/value FLOPs of a ragged batch: new token i of a request
    with prefix p sees p + i + 1 keys; 4 D FLOPs per (query, key, head)."""
    tot = 0
    for n, p in zip(nq, pre):
        n, p = int(n), int(p)
        tot += n * p + n * (n + 1) // 2
    return 4.0 * w.Hq * w.D * tot


def ragged_bytes(nq, pre, w):
    """Algorithmic HBM bytes of one paged prefill launch: Q read and O written
    once (bf16), LSE written (fp32), every cached K/V row of each request read
    once (bf16), page-table entries and lengths read."""
    import numpy as np
    nq, pre = np.asarray(nq, np.int64), np.asarray(pre, np.int64)
    T, L = int(nq.sum()), nq + pre
    return (2 * T * w.Hq * w.D * 2 + 4 * T * w.Hq + int(L.sum()) * w.Hkv * w.D * 2 * 2
            + int(((L + 63) // 64).sum()) * 4 + 8 * len(L))


def append_bytes(nq, w):
    """HBM bytes of one KV append: new K and V rows read once and written once."""
    return 4 * int(sum(int(n) for n in nq)) * w.Hkv * w.D * 2


def cascade_bytes(L, groups, prefix_pages, w):
    """Algorithmic HBM bytes of a cascade decode step: every group's prefix
    K/V read once, every request's suffix K/V once, q in, out and lse out,
    page-table entries and lengths read."""
    import numpy as np
    L = np.asarray(L, np.int64)
    pre = np.array([64 * int(prefix_pages[j]) if j >= 0 else 0 for j in groups], np.int64)
    row = w.Hkv * w.D * 2 * 2                                # K and V bytes of one token
    b = int(sum(int(p) for p in prefix_pages)) * 64 * row      # each prefix once
    b += int((L - pre).sum()) * row                          # suffixes
    b += 2 * len(L) * w.Hq * w.D * 2 + len(L) * w.Hq * 4      # q, out, lse
    b += int(((L + 63) // 64).sum()) * 4 + len(L) * 4
    return b


def source_sha(rel):
    """sha256[:16] of a source file, or of several joined by '+'."""
    h = hashlib.sha256()
    for part in rel.split("+"):
        with open(os.path.join(ROOT, part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name, src_rel):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if the
    kernel source is unchanged since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_sha(src_rel):
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def time_calls(fn, steps, warmup, stream, prewarm_s=0.0, runs=5):
    """HIP-event time (ms) per call of `steps` calls of fn on `stream`, after
    running fn for at least `prewarm_s` seconds (GPU clocks and power reach
    their steady state; an idle GPU runs the first ~0.1 s of work up to 15%
    slower) and then `warmup` more untimed calls.

    The timed calls run back to back in up to `runs` runs of at least 10
    calls, each run bracketed by one pair of events on `stream`; a call's time is its
    run's duration over the run's number of calls. So the mean is the average
    launch duration over the timed region, and the median is taken over runs.
    (An event pair around every call adds about 2.5 us of event overhead to
    each: 8% of the 28 us KV append, against its kernel trace.)"""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    runs = max(1, min(runs, steps // 10))   # at least 10 calls a run
    sizes = [steps // runs + (1 if i < steps % runs else 0) for i in range(runs)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for (a, b), n in zip(evs, sizes):
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
    torch.cuda.synchronize()
    out = []
    for (a, b), n in zip(evs, sizes):
        out += [a.elapsed_time(b) / n] * n
    return out


def cpu_baseline_prefill(w, q, k, v, budget_s=15.0):
    """fp64 oracle on the prefill workload, threads over jobs. Whole heads
    when S <= 8192; for longer sequences, seeded 64-row blocks of random heads
    (the first and last block of a head, the blocks on either side of a
    256-row tile boundary, and random blocks), each with all its causal keys."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    G = w.Hq // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    whole = w.S <= 8192
    if whole:
        jobs = [(b, h, None) for b, h in heads]
    else:
        g = np.random.default_rng(0)
        nblk = w.S // 64
        jobs = []
        for i in g.permutation(len(heads)):
            b, h = heads[i]
            bd = 4 * int(g.integers(1, nblk // 4))
            jobs += [(b, h, 0), (b, h, nblk - 1), (b, h, bd - 1), (b, h, bd)]
        jobs += [(b, h, int(g.integers(0, nblk))) for b, h in (heads[i] for i in g.integers(0, len(heads), 4096))]

    def one(job):
        b, h, blk = job
        gg = h // G
        qh = q[b:b + 1, h:h + 1].float().numpy()
        kh = k[b:b + 1, gg:gg + 1].float().numpy()
        vh = v[b:b + 1, gg:gg + 1].float().numpy()
        rows = None if blk is None else np.arange(64 * blk, 64 * blk + 64)
        oracle.prefill(qh, kh, vh, w.scale, True, rows=rows)
        r = np.arange(w.S) if rows is None else rows
        return 4.0 * w.D * float(np.sum(r + 1))

    done, flops = 0, 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < len(jobs) and time.perf_counter() - t0 < budget_s:
            batch = jobs[done:done + cores]
            flops += sum(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    if whole:
        sample = f"{done} of {len(jobs)} whole heads (all {w.S} causal rows)"
    else:
        sample = (f"{done} 64-row blocks (of {w.S // 64} per head; first, last, either side of a 256-row "
                  f"tile boundary and random, seeded) across {len(set((b, h) for b, h, _ in jobs[:done]))} "
                  f"of {len(heads)} heads, each row with all its causal keys")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample} of the prefill workload {w.name}, {dt:.1f} s wall, fp64 numpy, "
                      f"BLAS 1 thread per worker"}


def cpu_baseline_decode(w, kv, budget_s=10.0):
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    q = kv.q.double().numpy()
    if w.kv_dtype == "fp8":
        kp, vp, ks, vs = kv.k_pages.numpy(), kv.v_pages.numpy(), kv.k_scale.numpy(), kv.v_scale.numpy()
    else:
        kp, vp, ks, vs = kv.k_pages.float().numpy(), kv.v_pages.float().numpy(), None, None
    pt, sl = kv.page_table.numpy(), kv.seqlens.numpy()
    eb = 1 if w.kv_dtype == "fp8" else 2

    def one(b):
        oracle.paged_decode(q, kp, vp, pt, sl, w.scale, ks, vs, requests=[b])
        return int(sl[b]) * w.Hkv * w.D * 2 * eb

    done, nbytes = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < w.B and time.perf_counter() - t0 < budget_s:
            batch = list(range(done, min(w.B, done + cores)))
            nbytes += sum(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.B} requests of the decode workload (all heads), {dt:.1f} s wall, "
                      f"fp64 numpy, BLAS 1 thread per worker"}


def cpu_baseline_ragged(w, r, budget_s=10.0):
    """fp64 oracle on 64-row blocks of the ragged batch's requests (all heads), threads over blocks."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    kp, vp = oracle.kv_append(r.k_pages.float().numpy(), r.v_pages.float().numpy(), r.page_table.numpy(),
                              r.seqlens.numpy(), r.cu_seqlens_q.numpy(), r.k_new.float().numpy(),
                              r.v_new.float().numpy())
    q = r.q.double().numpy()
    L, cu, pt = r.seqlens.numpy(), r.cu_seqlens_q.numpy(), r.page_table.numpy()
    jobs = [(b, s) for b in range(w.B) for s in range(0, int(cu[b + 1] - cu[b]), 64)]
    jobs = [jobs[i] for i in np.random.default_rng(0).permutation(len(jobs))]

    def one(job):
        b, s = job
        n = int(cu[b + 1] - cu[b])
        rows = np.arange(s, min(n, s + 64))
        oracle.paged_prefill_request(q[cu[b]:cu[b + 1]], kp, vp, pt[b], int(L[b]), w.scale, rows)
        return 4.0 * w.Hq * w.D * float(np.sum(int(L[b]) - n + rows + 1))

    done, flops = 0, 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < len(jobs) and time.perf_counter() - t0 < budget_s:
            batch = jobs[done:done + cores]
            flops += sum(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(jobs)} random 64-row blocks (all heads, all visible keys) of the "
                      f"ragged prefill workload, {dt:.1f} s wall, fp64 numpy, BLAS 1 thread per worker"}


def cpu_baseline_cascade(w, r, budget_s=10.0):
    """fp64 oracle decode (the cascade's definition) on whole requests, threads over requests."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    q = r.q.double().numpy()
    kp, vp = r.k_pages.float().numpy(), r.v_pages.float().numpy()
    pt, sl = r.page_table.numpy(), r.seqlens.numpy()

    def one(b):
        oracle.paged_decode(q, kp, vp, pt, sl, w.scale, requests=[b])
        return int(sl[b])

    done, toks = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < w.B and time.perf_counter() - t0 < budget_s:
            batch = list(range(done, min(w.B, done + cores)))
            toks += sum(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    return {"value": toks * w.Hkv * w.D * 4 / dt / 1e9, "unit": "GB/s (plain-decode bytes)", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {w.B} requests of the shared-prefix workload (all heads, plain decode "
                      f"definition), {dt:.1f} s wall, fp64 numpy, BLAS 1 thread per worker"}


def cpu_baseline_fp8(w, q8, k8, v8, qs, ks, vs, budget_s=10.0):
    """fp64 oracle on whole heads of the fp8 workload (dequantised inputs), threads over heads."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]

    def one(bh):
        b, h = bh
        g = h // (w.Hq // w.Hkv)
        qd = oracle.e4m3fn_to_float(q8[b, h].numpy()) * float(qs[b, h])
        kd = oracle.e4m3fn_to_float(k8[b, g].numpy()) * float(ks[b, g])
        vd = oracle.e4m3fn_to_float(v8[b, g].numpy()) * float(vs[b, g])
        oracle.attention_head(qd, kd, vd, w.scale, True)

    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < len(heads) and time.perf_counter() - t0 < budget_s:
            batch = heads[done:done + cores]
            list(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * (w.S * (w.S + 1) // 2) * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(heads)} whole heads of the fp8 prefill workload (dequantised inputs), "
                      f"{dt:.1f} s wall, fp64 numpy, BLAS 1 thread per worker"}


def cpu_baseline_bwd(w, q, k, v, do, budget_s=10.0):
    """fp64 oracle backward on whole heads of the workload, threads over heads."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    qn, kn, vn, dn = (x.double().numpy() for x in (q, k, v, do))
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]

    def one(bh):
        b, h = bh
        g = h // (w.Hq // w.Hkv)
        oracle.attention_head_backward(qn[b, h], kn[b, g], vn[b, g], dn[b, h], w.scale, True)

    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(cores) as ex:
        while done < len(heads) and time.perf_counter() - t0 < budget_s:
            batch = heads[done:done + cores]
            list(ex.map(one, batch))
            done += len(batch)
    dt = time.perf_counter() - t0
    flops = 2.5 * 4.0 * w.D * (w.S * (w.S + 1) // 2) * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(heads)} whole heads of the backward workload, {dt:.1f} s wall, "
                      f"fp64 numpy, BLAS 1 thread per worker"}


COPY_BYTES = 1 << 30   # calibration copy: bytes read, and bytes written, per launch


def copy_calibration(steps, warmup):
    """A plain device copy of COPY_BYTES (every byte read once and written
    once, y = -x on bf16): the known-size kernel that calibrates the HBM byte
    counters of the attention kernels."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    t = time_calls(lambda: torch.neg(src, out=dst), steps, warmup, stream, 0.5)
    ms = statistics.mean(t)
    print(json.dumps({"metric": "plain copy HBM GB/s (counter calibration)", "unit": "GB/s",
                      "value": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1), "ms_mean": round(ms, 5),
                      "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "steps": steps}), flush=True)


# ---- Turning rocprofv3 output into the text summaries kept under profiles/.
# Expected layout under DIR (each a rocprofv3 ``-d`` directory, ``-o pmc`` or
# ``-o kt``), made by the commands that PROFILE_COMMANDS lists:
#   DIR/kt                      --kernel-trace --stats of the default bench run
#   DIR/pmc_<leg>_<COUNTER>     --pmc COUNTER of one leg, COUNTER in FETCH_SIZE, WRITE_SIZE
DECODE_SRC = ("exact_attention_20_amd/csrc/decode.hip+exact_attention_20_amd/csrc/decode_mfma.hip"
              "+exact_attention_20_amd/csrc/decode_common.h")
PMC_LEGS = {
    "prefill_bf16_wl2": ("--only prefill --prefill-workload 2", ["prefill_bf16_kernel"],
                         "exact_attention_20_amd/csrc/prefill_bf16.hip"),
    "prefill_bf16_wl3": ("--only prefill --prefill-workload 3", ["prefill_bf16_kernel"],
                         "exact_attention_20_amd/csrc/prefill_bf16.hip"),
    "decode_wl4": ("--only decode --decode-workload 4", ["decode_mfma_kernel", "lse_merge_kernel"], DECODE_SRC),
    "decode_wl5": ("--only decode --decode-workload 5", ["decode_mfma_kernel", "lse_merge_kernel"], DECODE_SRC),
    "ragged_prefill_wl6": ("--only ragged", ["prefill_bf16_kernel"],
                           "exact_attention_20_amd/csrc/prefill_bf16.hip"),
    "cascade_wl7": ("--only cascade --no-plain-compare", ["prefill_bf16_kernel", "decode_mfma_kernel", "lse_merge_kernel"],
                    "exact_attention_20_amd/csrc/prefill_bf16.hip+" + DECODE_SRC),
    "prefill_fp8_wl8": ("--only fp8", ["prefill_fp8_kernel"], "exact_attention_20_amd/csrc/prefill_fp8.hip"),
    "backward_wl2": ("--only bwd", ["bwd_dq_kernel", "bwd_dkdv_kernel"],
                     "exact_attention_20_amd/csrc/prefill_bwd.hip"),
    "copy": ("--only copy", ["neg"], None),
}
PMC_RUN = "--steps 3 --warmup 1 --prewarm-s 0 --no-cpu-baseline"
# Shader-sequencer counters of the 32K-token prefill (one pass): matrix-core
# busy cycles, co-issue, shader-engine busy cycles (with the kernel time they
# give the clock the chip held), wave time and waits.
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
               "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA")
SQ_LEG = ("prefill_bf16_wl3_sq", "--only prefill --prefill-workload 3", "prefill_bf16_kernel")
N_SE, N_SIMD = 32, 1024   # MI355X: 8 XCDs x 4 shader engines; 256 CUs x 4 SIMDs


def profile_commands(d):
    cmds = [f"rocprofv3 --kernel-trace --stats -f csv -d {d}/kt -o kt -- python3 bench.py > {d}/kt_bench.json"]
    for leg, (flags, _, _) in PMC_LEGS.items():
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            cmds.append(f"rocprofv3 --pmc {c} -f csv -d {d}/pmc_{leg}_{c} -o pmc -- python3 bench.py {flags} {PMC_RUN}")
    cmds.append(f"rocprofv3 --pmc {SQ_COUNTERS} -f csv -d {d}/pmc_{SQ_LEG[0]} -o pmc -- python3 bench.py "
                f"{SQ_LEG[1]} {PMC_RUN}")
    return cmds


def _pmc_means(path, names):
    """Mean per dispatch of the counter in one rocprofv3 --pmc csv, summed over
    the kernels whose name contains one of ``names``; (mean KiB, dispatches)."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "*counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    per_disp = {}
    kname = {}
    for r in csv.DictReader(open(files[0])):
        key = r["Dispatch_Id"]
        per_disp[key] = per_disp.get(key, 0.0) + float(r["Counter_Value"])
        kname[key] = r["Kernel_Name"]
    total, counts = 0.0, []
    for n in names:
        vals = [v for k, v in per_disp.items() if n in kname[k]]
        if not vals:
            raise ValueError(f"no dispatch of a kernel named *{n}* in {files[0]}: "
                             f"{sorted(set(kname.values()))}")
        total += statistics.mean(vals)
        counts.append(len(vals))
    return total, min(counts)


def _pmc_means_one(path, kernel, counter):
    """Mean per dispatch of one counter over the kernel's dispatches in a --pmc csv."""
    import csv
    import glob
    f = glob.glob(os.path.join(path, "*counter_collection.csv"))[0]
    per = {}
    for r in csv.DictReader(open(f)):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return statistics.mean(per.values()) if per else float("nan")


def _pmc_dispatches(path, kernel):
    """Per dispatch of the kernel in a --pmc csv, in dispatch order: its counters
    (summed over the csv's rows) and its duration in us from the same rows'
    timestamps."""
    import csv
    import glob
    f = glob.glob(os.path.join(path, "*counter_collection.csv"))[0]
    per = {}
    for r in csv.DictReader(open(f)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), [{}, 0.0])
        d[0][r["Counter_Name"]] = d[0].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d[1] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return [per[k] for k in sorted(per)]


def _trace_mean_us(path, prefix, min_us=0.0):
    """Mean duration (us) of the dispatches of kernels whose short name starts with
    ``prefix`` and that run at least ``min_us``, from a --kernel-trace csv."""
    import csv
    import glob
    f = glob.glob(os.path.join(path, "*kernel_trace.csv"))
    if not f:
        return None
    ds = []
    for r in csv.DictReader(open(f[0])):
        m = re.search(r"::(\w+(?:<[^>]*>)?)\(", r["Kernel_Name"])
        k = m.group(1) if m else r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if k.startswith(prefix) and dur >= min_us:
            ds.append(dur)
    return statistics.mean(ds) if ds else None


def summarize_profiles(d):
    """Write profiles/<leg>_traffic.txt for every counter leg found under d,
    and profiles/kernel_trace_bench.txt from the kernel trace."""
    import csv
    import glob
    import workloads
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    cmds = profile_commands(d)
    header = ["# Commands, run from the repository root on one MI355X (TMPDIR=/tmp):"]
    header += [f"#   {c}" for c in cmds]
    header += [f"#   python3 bench.py --summarize-profiles {d}"]
    written = []
    copy_f, _ = _pmc_means(f"{d}/pmc_copy_FETCH_SIZE", PMC_LEGS["copy"][1])
    copy_w, _ = _pmc_means(f"{d}/pmc_copy_WRITE_SIZE", PMC_LEGS["copy"][1])
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    for leg, (flags, names, src) in PMC_LEGS.items():
        if src is None or not os.path.isdir(f"{d}/pmc_{leg}_FETCH_SIZE"):
            continue
        fk, n = _pmc_means(f"{d}/pmc_{leg}_FETCH_SIZE", names)
        wk, _ = _pmc_means(f"{d}/pmc_{leg}_WRITE_SIZE", names)
        wid = int(leg.rsplit("wl", 1)[1])
        w = workloads.WORKLOADS[wid]
        if leg.startswith("backward"):
            # q, o, dO read and dq written (Hq heads), k, v read and dk, dv written (Hkv heads), once
            # each in bf16; lse read, D written and read (fp32)
            alg = 2 * w.B * w.S * w.D * (4 * w.Hq + 4 * w.Hkv) + 12 * w.B * w.Hq * w.S
        elif leg.startswith("prefill_fp8"):
            alg = w.B * w.S * w.D * (w.Hq + 2 * w.Hkv) + 2 * w.B * w.Hq * w.S * w.D + 4 * w.B * w.Hq * w.S
        elif leg.startswith("prefill"):
            alg = prefill_bytes(w)
        elif leg.startswith("cascade"):
            x = workloads.workload_shared_prefix_inputs(w)
            alg = cascade_bytes(x.seqlens.numpy(), x.prefix_group.numpy(), list(w.prefix_pages), w)
        elif leg.startswith("ragged"):
            alg = ragged_bytes(workloads.context_lengths(wid, w.B, w.new_lens),
                               workloads.context_lengths(wid, w.B, w.prefix_lens, workloads.STREAM_PREFIX), w)
        else:
            alg = decode_bytes(workloads.context_lengths(wid, w.B, w.lengths), w)
        fb, wb = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        lines = [f"# HBM traffic per launch of {' + '.join(names)} on workload {wid} ({w.name}),",
                 "# from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch, one pass each), scaled by",
                 f"# what the same counters read for a plain {COPY_BYTES} B copy (torch.neg on bf16).",
                 *header,
                 f"source: {src}",
                 f"source_sha256_16: {source_sha(src)}",
                 f"dispatches_per_kernel: {n}",
                 f"fetch_kib_raw: {fk:.1f}",
                 f"write_kib_raw: {wk:.1f}",
                 f"copy_fetch_kib_raw: {copy_f:.1f}",
                 f"copy_write_kib_raw: {copy_w:.1f}",
                 f"fetch_scale: {f_scale:.4f}",
                 f"write_scale: {w_scale:.4f}",
                 f"fetch_bytes_per_launch: {fb:.0f}",
                 f"write_bytes_per_launch: {wb:.0f}",
                 f"algorithmic_bytes_per_launch: {alg}",
                 f"traffic_over_algorithmic: {(fb + wb) / alg:.3f}"]
        path = os.path.join(out_dir, f"{leg}_traffic.txt")
        open(path, "w").write("\n".join(lines) + "\n")
        written.append(path)
    sq_dir = f"{d}/pmc_{SQ_LEG[0]}"
    if os.path.isdir(sq_dir):
        # The pass runs a few dispatches from a cold start; the chip's clock rises
        # over them. Every figure below is the last (warmest) dispatch's own:
        # its counters and its duration from the same rows' timestamps.
        names = SQ_COUNTERS.split()
        disp = _pmc_dispatches(sq_dir, SQ_LEG[2])
        vals, dur_us = disp[-1]
        lines = ["# Shader-sequencer counters of the 32K-token GQA prefill kernel (rocprofv3 --pmc, one",
                 "# pass), for the pass's last dispatch. SQ_BUSY_CYCLES is summed over the 32 shader",
                 "# engines, the MFMA counters over the 1,024 SIMDs; wave counters are in quad-cycles.",
                 *header, f"source_sha256_16: {source_sha('exact_attention_20_amd/csrc/prefill_bf16.hip')}"]
        lines += [f"{n}: {vals[n]:.6g}" for n in names]
        se_cycles = vals["SQ_BUSY_CYCLES"] / N_SE
        mfma = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD
        lines.append(f"cycles_per_shader_engine: {se_cycles:.6g}")
        lines.append(f"mfma_busy_fraction_of_cycles: {mfma / se_cycles:.4f}")
        lines.append(f"mfma_coexec_fraction_of_mfma_busy: {vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / vals['SQ_VALU_MFMA_BUSY_CYCLES']:.4f}")
        lines.append(f"dispatch_us: {dur_us:.1f}")
        lines.append(f"implied_clock_ghz: {se_cycles / (dur_us * 1e3):.3f}")
        lines.append(f"bf16_mfma_peak_at_that_clock_tflops: {2500.0 * se_cycles / (dur_us * 1e3) / 2.4:.0f}")
        lines.append("# every dispatch of the pass (us, implied GHz): " + ", ".join(
            f"{t:.0f} {c['SQ_BUSY_CYCLES'] / N_SE / (t * 1e3):.3f}" for c, t in disp))
        t_us = _trace_mean_us(f"{d}/kt", "prefill_bf16_kernel<8, 1, 0", min_us=2000.0)
        if t_us:
            lines.append(f"# kernel trace of the default bench run (another process), mean: {t_us:.1f} us")
        path = os.path.join(out_dir, f"{SQ_LEG[0]}_counters.txt")
        open(path, "w").write("\n".join(lines) + "\n")
        written.append(path)
    kt = glob.glob(f"{d}/kt/*kernel_stats.csv")
    if kt:
        rows = list(csv.DictReader(open(kt[0])))
        lines = ["# rocprofv3 --kernel-trace --stats of the default bench run (one process, all legs).",
                 *header[:2], f"#   python3 bench.py --summarize-profiles {d}",
                 "# kernel | calls | average us | min us | max us | total ms | % of GPU time"]
        for r in rows:
            name = r["Name"]
            m = re.search(r"::(\w+(?:<[^>]*>)?)\(", name)   # "void fa::(anon)::NAME<...>(args)"
            short = m.group(1) if m else name[:70]
            lines.append(f"{short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}")
        tr = glob.glob(f"{d}/kt/*kernel_trace.csv")
        if tr:
            # Per leg: the legs run one after another in a fixed order, so a
            # dispatch belongs to the leg whose first kernel came last before
            # it; in the shared-prefix leg a split kernel right after a prefix
            # pass (and the merge after it) belongs to the cascade, the others
            # to the plain-decode comparison.
            disp = sorted(csv.DictReader(open(tr[0])), key=lambda r: int(r["Start_Timestamp"]))
            leg, prev, per, dsub = "prefill", "", {}, "decode"
            for r in disp:
                m = re.search(r"::(\w+(?:<[^>]*>)?)\(", r["Kernel_Name"])
                k = m.group(1) if m else r["Kernel_Name"][:60]
                if leg == "prefill" and k.startswith(("decode_", "lse_merge")):
                    leg = "decode"
                if k.startswith("kv_append"):
                    leg = "ragged"
                if k.startswith("prefill_bf16_kernel<8, 1, 2"):
                    leg = "cascade"
                if k.startswith("prefill_fp8"):
                    leg = "fp8"
                if k.startswith("bwd_") or (k.startswith("prefill_bf16_kernel<8, 1, 0") and leg != "prefill"):
                    leg = "backward"  # the backward leg starts with one forward call for O and LSE
                sub = leg
                if leg in ("cascade", "cascade (plain-decode comparison)"):
                    if k.startswith("decode_"):
                        leg = sub = ("cascade" if prev.startswith("prefill_bf16_kernel<8, 1, 2")
                                     else "cascade (plain-decode comparison)")
                    elif k.startswith("lse_merge"):
                        sub = leg
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                if leg == "prefill" and k.startswith("prefill_bf16_kernel<8, 1, 0"):
                    # two prefill workloads share the kernel: the 32K-token GQA launch
                    # runs ~8 ms, the 4 x 4096-token one well under 2 ms
                    sub = "prefill (B1 Hq32/Hkv8 S32768)" if dur > 2000.0 else "prefill (B4 H32 S4096)"
                if leg == "decode" and k.startswith(("decode_", "lse_merge")):
                    if k.startswith("decode_"):
                        dsub = "decode (fp8 KV, 8 long requests)" if ", true," in k else "decode (bf16 KV, 64 requests)"
                    sub = dsub
                per.setdefault((sub, k), []).append(dur)
                prev = k
            lines.append("# per leg (dispatches attributed by order): leg | kernel | calls | average us")
            for (lg, k), v in per.items():
                lines.append(f"leg {lg} | {k} | {len(v)} | {statistics.mean(v):.2f}")
        bj = f"{d}/kt_bench.json"
        if os.path.exists(bj):
            txt = [x for x in open(bj).read().splitlines() if x.startswith("{")]
            if txt:
                b = json.loads(txt[-1])
                lines.append("# the same run's bench line, HIP-event means per launch:")
                for name, o in b.get("prefill", {}).items():
                    lines.append(f"bench prefill {name} launch ms_mean: {o.get('ms_mean')}")
                for name, o in b.get("decode", {}).items():
                    lines.append(f"bench decode {name} step ms_mean: {o.get('ms_mean')}")
                if "shared_prefix_decode" in b:
                    lines.append(f"bench shared-prefix decode step ms_mean: {b['shared_prefix_decode'].get('ms_mean')}")
                if "backward" in b:
                    lines.append(f"bench backward step ms_mean: {b['backward'].get('ms_mean')}")
                if "fp8_prefill" in b:
                    lines.append(f"bench fp8 prefill launch ms_mean: {b['fp8_prefill'].get('ms_mean')}")
                if "ragged_prefill" in b:
                    rg = b["ragged_prefill"]
                    lines.append(f"bench ragged paged prefill launch ms_mean: {rg.get('ms_mean')}")
                    lines.append(f"bench kv append launch ms_mean: {rg['append'].get('ms_mean')}")
                lines.append(f"bench value: {b['value']} {b['unit']}")
        path = os.path.join(out_dir, "kernel_trace_bench.txt")
        open(path, "w").write("\n".join(lines) + "\n")
        written.append(path)
    for p in written:
        print("wrote", os.path.relpath(p, ROOT))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (GPU clock ramp-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain-compare", action="store_true",
                    help="shared-prefix leg: skip timing plain decode of the same batch")
    ap.add_argument("--only", choices=["prefill", "decode", "ragged", "cascade", "fp8", "bwd", "copy"], default=None)
    ap.add_argument("--prefill-workload", type=int, default=None, choices=[2, 3],
                    help="time only this prefill workload (default: 3, the headline, then 2)")
    ap.add_argument("--decode-workload", type=int, default=None, choices=[4, 5],
                    help="time only this decode workload (default: 4, in the step, then 5)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/*.txt from rocprofv3 output under DIR (no GPU needed)")
    ap.add_argument("--print-profile-commands", metavar="DIR", default=None)
    args = ap.parse_args()
    if args.print_profile_commands:
        print("\n".join(profile_commands(args.print_profile_commands)))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(prefill and decode would shard by request and KV-head group with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_20_amd as fa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    fa.load()
    stream = torch.cuda.current_stream()
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    if args.only == "copy":
        copy_calibration(args.steps, args.warmup)
        return

    res = {"prefill": [], "decode": []}
    pws = [args.prefill_workload] if args.prefill_workload else [3, 2]
    dws = [args.decode_workload] if args.decode_workload else [4, 5]

    if args.only in (None, "prefill"):
        for wid in pws:
            wp = workloads.WORKLOADS[wid]
            log(f"[bench] generating prefill workload {wp.name}")
            q, k, v = workloads.workload_prefill_inputs(wp)
            qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
            out = torch.empty_like(qd)
            lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=qd.device)
            pf = lambda: fa.fa_prefill_fwd(qd, kd, vd, out, lse, True, wp.scale, None, stream)  # noqa: E731
            t = time_calls(pf, args.steps, args.warmup, stream, args.prewarm_s)
            log(f"[bench] prefill {wp.name} median {statistics.median(t):.4f} ms min {min(t):.4f} ms")
            del qd, kd, vd, out, lse
            cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(wp, q, k, v)
            res["prefill"].append(dict(w=wp, t=t, cpu=cpu))
            del q, k, v

    if args.only in (None, "decode"):
        for wid in dws:
            wd = workloads.WORKLOADS[wid]
            log(f"[bench] generating decode workload {wd.name}")
            kv = workloads.workload_paged_inputs(wd, nan_tails=True)
            dt = fa.BF16 if wd.kv_dtype == "bf16" else fa.FP8_E4M3FN
            d = dict(q=kv.q.cuda(), k=kv.k_pages.cuda(), v=kv.v_pages.cuda(), pt=kv.page_table.cuda(),
                     sl=kv.seqlens.cuda(), ks=None if kv.k_scale is None else kv.k_scale.cuda(),
                     vs=None if kv.v_scale is None else kv.v_scale.cuda())
            t0 = time.perf_counter()
            plan = fa.fa_decode_plan(kv.seqlens, kv.page_table, kv.num_pages, wd.Hq, wd.Hkv, wd.D, dt, 0)
            plan_ms = (time.perf_counter() - t0) * 1e3
            items, _, chunk = plan.items()
            out = torch.empty_like(d["q"])
            lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=d["q"].device)
            # Rotate copies of the KV pools when they would fit in the 256 MB
            # last-level cache, so every step reads from HBM.
            pool_bytes = d["k"].numel() * d["k"].element_size() * 2
            n_copies = 1 if pool_bytes > 1024 ** 3 else 4
            pools = [(d["k"], d["v"])] + [(d["k"].clone(), d["v"].clone()) for _ in range(n_copies - 1)]
            it = [0]

            def dec():
                kk, vv = pools[it[0] % n_copies]
                it[0] += 1
                fa.fa_decode_run(plan, d["q"], kk, vv, d["pt"], d["sl"], plan.num_splits, out, lse,
                                 d["ks"], d["vs"], wd.scale, stream)

            t = time_calls(dec, args.steps, args.warmup, stream, args.prewarm_s)
            log(f"[bench] decode {wd.name} median {statistics.median(t):.4f} ms min {min(t):.4f} ms "
                f"plan {plan_ms:.2f} ms")
            del d, pools, out, lse
            cpu = None if args.no_cpu_baseline else cpu_baseline_decode(wd, kv)
            res["decode"].append(dict(w=wd, t=t, bytes=decode_bytes(kv.seqlens.numpy(), wd), cpu=cpu,
                                      total_tokens=int(kv.seqlens.sum()),
                                      plan=dict(plan_ms=round(plan_ms, 3), items=int(len(items)),
                                                chunk_pages=chunk, num_splits=plan.num_splits,
                                                pages=int(kv.num_pages), pool_copies_rotated=n_copies)))
            del kv

    if args.only in (None, "ragged"):
        wr = workloads.WORKLOADS[6]
        log(f"[bench] generating ragged prefill workload {wr.name}")
        r = workloads.workload_ragged_inputs(wr)
        d = dict(q=r.q.cuda(), kn=r.k_new.cuda(), vn=r.v_new.cuda(), k=r.k_pages.cuda(), v=r.v_pages.cuda(),
                 pt=r.page_table.cuda(), sl=r.seqlens.cuda(), cu=r.cu_seqlens_q.cuda())
        t0 = time.perf_counter()
        plan = fa.fa_prefill_paged_plan(r.seqlens, r.cu_seqlens_q, r.page_table, r.num_pages, wr.Hq, wr.Hkv)
        plan_ms = (time.perf_counter() - t0) * 1e3
        out = torch.empty_like(d["q"])
        lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=d["q"].device)
        app = lambda: fa.fa_kv_append(d["kn"], d["vn"], d["k"], d["v"], d["pt"], d["sl"], d["cu"], stream)  # noqa: E731
        run = lambda: fa.fa_prefill_paged_run(plan, d["q"], d["k"], d["v"], d["pt"], d["sl"], d["cu"],  # noqa: E731
                                              out, lse, wr.scale, stream)
        t_app = time_calls(app, args.steps, args.warmup, stream, min(args.prewarm_s, 0.3))
        t_run = time_calls(run, args.steps, args.warmup, stream, args.prewarm_s)
        nq = (r.cu_seqlens_q[1:] - r.cu_seqlens_q[:-1]).numpy()
        pre = r.seqlens.numpy() - nq
        res["ragged"] = dict(app=t_app, run=t_run, flops=ragged_flops(nq, pre, wr),
                             bytes=ragged_bytes(nq, pre, wr), app_bytes=append_bytes(nq, wr),
                             plan=dict(plan_ms=round(plan_ms, 3), items=plan.n_items, pages=int(r.num_pages),
                                       tokens=int(nq.sum())), w=wr)
        log(f"[bench] ragged append median {statistics.median(t_app):.4f} ms, "
            f"prefill median {statistics.median(t_run):.4f} ms")
        res["ragged_cpu"] = None if args.no_cpu_baseline else cpu_baseline_ragged(wr, r)
        del d

    if args.only in (None, "cascade"):
        wc = workloads.WORKLOADS[7]
        log(f"[bench] generating shared-prefix workload {wc.name}")
        r = workloads.workload_shared_prefix_inputs(wc)
        d = dict(q=r.q.cuda(), k=r.k_pages.cuda(), v=r.v_pages.cuda(), pt=r.page_table.cuda(), sl=r.seqlens.cuda())
        t0 = time.perf_counter()
        plan_c = fa.fa_decode_plan_cascade(r.seqlens, r.page_table, r.num_pages, wc.Hq, wc.Hkv, r.prefix_group,
                                           list(wc.prefix_pages))
        plan_ms = (time.perf_counter() - t0) * 1e3
        plan_p = fa.fa_decode_plan(r.seqlens, r.page_table, r.num_pages, wc.Hq, wc.Hkv, wc.D, fa.BF16, 0)
        out = torch.empty_like(d["q"])
        lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=d["q"].device)
        casc = lambda: fa.fa_decode_run(plan_c, d["q"], d["k"], d["v"], d["pt"], d["sl"], plan_c.num_splits,  # noqa: E731
                                        out, lse, None, None, wc.scale, stream)
        plain = lambda: fa.fa_decode_run(plan_p, d["q"], d["k"], d["v"], d["pt"], d["sl"], plan_p.num_splits,  # noqa: E731
                                         out, lse, None, None, wc.scale, stream)
        t_c = time_calls(casc, args.steps, args.warmup, stream, args.prewarm_s)
        t_p = [float("nan")] if args.no_plain_compare else time_calls(plain, args.steps, args.warmup, stream,
                                                                      min(args.prewarm_s, 0.3))
        L = r.seqlens.numpy()
        res["cascade"] = dict(c=t_c, p=t_p, w=wc, bytes=cascade_bytes(L, r.prefix_group.numpy(), list(wc.prefix_pages), wc),
                              plain_bytes=decode_bytes(L, workloads.DecodeWorkload(7, "", wc.B, wc.Hq, wc.Hkv, wc.D, "bf16")),
                              plan=dict(plan_ms=round(plan_ms, 3), num_splits=plan_c.num_splits, pages=int(r.num_pages),
                                        total_tokens=int(L.sum())))
        log(f"[bench] cascade median {statistics.median(t_c):.4f} ms, plain decode median {statistics.median(t_p):.4f} ms")
        res["cascade_cpu"] = None if args.no_cpu_baseline else cpu_baseline_cascade(wc, r)
        del d

    if args.only in (None, "fp8"):
        w8 = workloads.WORKLOADS[8]
        log(f"[bench] generating fp8 prefill workload {w8.name}")
        q8, k8, v8, qs, ks, vs = workloads.fp8_prefill_inputs(w8.B, w8.Hq, w8.Hkv, w8.S, w8.S, w8.D, w8.wid)
        d = [x.cuda() for x in (q8, k8, v8, qs, ks, vs)]
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(q8.shape[:3], dtype=torch.float32, device="cuda")
        f8 = lambda: fa.fa_prefill_fp8_fwd(*d, out, lse, True, w8.scale, stream)  # noqa: E731
        t = time_calls(f8, args.steps, args.warmup, stream, args.prewarm_s)
        res["fp8"] = dict(t=t, w=w8)
        log(f"[bench] fp8 prefill median {statistics.median(t):.4f} ms")
        res["fp8_cpu"] = None if args.no_cpu_baseline else cpu_baseline_fp8(w8, q8, k8, v8, qs, ks, vs)
        del d

    if args.only in (None, "bwd"):
        wb = workloads.WORKLOADS[2]
        log(f"[bench] generating backward inputs for {wb.name}")
        q, k, v, do = workloads.backward_inputs(wb.B, wb.Hq, wb.Hkv, wb.S, wb.S, wb.D, wb.wid)
        qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        o, lse = fa.prefill(qd, kd, vd, causal=True, scale=wb.scale)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(fa.fa_prefill_bwd_workspace_size(wb.B, wb.Hq, wb.S), dtype=torch.uint8, device="cuda")
        bw = lambda: fa.fa_prefill_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, True, wb.scale, ws, stream)  # noqa: E731
        t = time_calls(bw, args.steps, args.warmup, stream, args.prewarm_s)
        res["bwd"] = dict(t=t, w=wb)
        log(f"[bench] backward median {statistics.median(t):.4f} ms")
        res["bwd_cpu"] = None if args.no_cpu_baseline else cpu_baseline_bwd(wb, q, k, v, do)
        del qd, kd, vd, dod, o, lse, dq, dk, dv, ws

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    ms_step = 0.0
    pre_objs, dec_objs = {}, {}
    for i, g in enumerate(res["prefill"]):
        wp = g["w"]
        t_pf = statistics.mean(g["t"])
        flops = prefill_flops(wp)
        tflops = flops / (t_pf * 1e-3) / 1e12
        pre_objs[wp.name] = {
            "metric": "causal bf16 prefill TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
            "ms_mean": round(t_pf, 5), "ms_median": round(statistics.median(g["t"]), 5),
            "in_step": i == 0,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": read_traffic(f"prefill_bf16_wl{wp.wid}_traffic.txt",
                                                 "exact_attention_20_amd/csrc/prefill_bf16.hip"),
                         "kernel": "prefill_bf16_kernel", "launch_ms_mean": round(t_pf, 5),
                         "launch_ms_median": round(statistics.median(g["t"]), 5), "flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": prefill_bytes(wp)},
            "cpu_baseline": g["cpu"],
            "config": {"workload": wp.name, "B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "S": wp.S, "D": wp.D,
                       "causal": True, "dtype": "bf16"}}
        if i == 0:
            ms_step += t_pf
            line.update(value=round(tflops, 2), unit="TFLOP/s")
            line["roofline"] = pre_objs[wp.name]["roofline"]
            line["cpu_baseline"] = g["cpu"]
    for i, g in enumerate(res["decode"]):
        wd = g["w"]
        t_dc = statistics.mean(g["t"])
        gbs = g["bytes"] / (t_dc * 1e-3) / 1e9
        dec_objs[wd.name] = {
            "metric": "paged decode HBM GB/s (split-KV + LSE merge)", "value": round(gbs, 1), "unit": "GB/s",
            "ms_mean": round(t_dc, 5), "ms_median": round(statistics.median(g["t"]), 5), "in_step": i == 0,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic(f"decode_wl{wd.wid}_traffic.txt", DECODE_SRC),
                         "kernel": "decode_mfma_kernel + lse_merge_kernel", "bytes_per_launch": g["bytes"]},
            "plan": g["plan"], "cpu_baseline": g["cpu"],
            "config": {"workload": wd.name, "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "D": wd.D,
                       "kv_dtype": wd.kv_dtype, "page": 64, "lengths": list(wd.lengths),
                       "total_tokens": g["total_tokens"]}}
        if i == 0:
            ms_step += t_dc
            if "value" not in line:
                line.update(value=round(gbs, 1), unit="GB/s")
                line["roofline"] = dec_objs[wd.name]["roofline"]
                line["cpu_baseline"] = g["cpu"]
    if pre_objs:
        line["prefill"] = pre_objs
    if dec_objs:
        line["decode"] = dec_objs
    if "ragged" in res:
        g = res["ragged"]
        wr = g["w"]
        t_run, t_app = statistics.mean(g["run"]), statistics.mean(g["app"])
        tf = g["flops"] / (t_run * 1e-3) / 1e12
        app_gbs = g["app_bytes"] / (t_app * 1e-3) / 1e9
        rag = {"metric": "ragged paged causal prefill TFLOP/s (KV append timed separately)",
               "value": round(tf, 2), "unit": "TFLOP/s",
               "ms_mean": round(t_run, 5), "ms_median": round(statistics.median(g["run"]), 5),
               "tflops_incl_append": round(g["flops"] / ((t_run + t_app) * 1e-3) / 1e12, 2),
               "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                            "traffic": read_traffic("ragged_prefill_wl6_traffic.txt",
                                                    "exact_attention_20_amd/csrc/prefill_bf16.hip"),
                            "kernel": "prefill_bf16_kernel (paged)", "flops_per_launch": g["flops"],
                            "algorithmic_bytes_per_launch": g["bytes"]},
               "append": {"ms_mean": round(t_app, 5), "value": round(app_gbs, 1), "unit": "GB/s",
                          "roofline": {"bound": "hbm", "achieved": round(app_gbs, 1), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(app_gbs / PEAK_HBM_GBS, 4),
                                       "kernel": "kv_append_kernel", "bytes_per_launch": g["app_bytes"]}},
               "plan": g["plan"], "cpu_baseline": res["ragged_cpu"],
               "config": {"workload": wr.name, "B": wr.B, "Hq": wr.Hq, "Hkv": wr.Hkv, "D": wr.D,
                          "new_tokens": list(wr.new_lens), "prefix": list(wr.prefix_lens), "page": 64}}
        line["ragged_prefill"] = rag
        if "value" not in line:
            line.update(value=rag["value"], unit="TFLOP/s")
            line["roofline"] = rag["roofline"]
            line["cpu_baseline"] = rag["cpu_baseline"]
            ms_step = t_run + t_app
    if "cascade" in res:
        g = res["cascade"]
        wc = g["w"]
        tc, tp = statistics.mean(g["c"]), statistics.mean(g["p"])
        gbs = g["bytes"] / (tc * 1e-3) / 1e9
        cas = {"metric": "shared-prefix (cascade) decode HBM GB/s of its algorithmic bytes",
               "value": round(gbs, 1), "unit": "GB/s", "ms_mean": round(tc, 5),
               "ms_median": round(statistics.median(g["c"]), 5),
               "plain_decode_ms_mean": round(tp, 5), "speedup_vs_plain_decode": round(tp / tc, 3),
               "plain_decode_bytes_per_step": g["plain_bytes"],
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": read_traffic("cascade_wl7_traffic.txt",
                                                    "exact_attention_20_amd/csrc/prefill_bf16.hip+" + DECODE_SRC),
                            "kernel": "prefill_bf16_kernel (prefix pass) + decode_mfma_kernel + lse_merge_kernel",
                            "bytes_per_launch": g["bytes"]},
               "plan": g["plan"], "cpu_baseline": res["cascade_cpu"],
               "config": {"workload": wc.name, "B": wc.B, "Hq": wc.Hq, "Hkv": wc.Hkv, "D": wc.D,
                          "group_sizes": list(wc.group_sizes), "prefix_pages": list(wc.prefix_pages),
                          "suffix": list(wc.suffix_lens), "page": 64}}
        line["shared_prefix_decode"] = cas
        if "value" not in line:
            line.update(value=cas["value"], unit="GB/s")
            line["roofline"] = cas["roofline"]
            line["cpu_baseline"] = cas["cpu_baseline"]
            ms_step = tc
    if "fp8" in res:
        g = res["fp8"]
        w8 = g["w"]
        t8 = statistics.mean(g["t"])
        flops = prefill_flops(w8)
        tf = flops / (t8 * 1e-3) / 1e12
        f8o = {"metric": "causal fp8 (e4m3) prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
               "ms_mean": round(t8, 5), "ms_median": round(statistics.median(g["t"]), 5),
               "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                            "traffic": read_traffic("prefill_fp8_wl8_traffic.txt",
                                                    "exact_attention_20_amd/csrc/prefill_fp8.hip"),
                            "kernel": "prefill_fp8_kernel", "flops_per_launch": flops},
               "cpu_baseline": res["fp8_cpu"],
               "config": {"workload": w8.name, "B": w8.B, "Hq": w8.Hq, "Hkv": w8.Hkv, "S": w8.S, "D": w8.D,
                          "causal": True, "dtype": "fp8 e4m3fn, per-(batch, head) scales"}}
        line["fp8_prefill"] = f8o
        if "value" not in line:
            line.update(value=f8o["value"], unit="TFLOP/s", dtype="fp8")
            line["roofline"] = f8o["roofline"]
            line["cpu_baseline"] = f8o["cpu_baseline"]
            ms_step = t8
    if "bwd" in res:
        g = res["bwd"]
        wb = g["w"]
        tb = statistics.mean(g["t"])
        flops = 2.5 * prefill_flops(wb)  # five products of the forward's size: S, dP, dV, dK, dQ
        tf = flops / (tb * 1e-3) / 1e12
        bwo = {"metric": "causal bf16 attention backward TFLOP/s (5 products counted; S and dP are recomputed)",
               "value": round(tf, 2), "unit": "TFLOP/s", "ms_mean": round(tb, 5),
               "ms_median": round(statistics.median(g["t"]), 5),
               "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                            "traffic": read_traffic("backward_wl2_traffic.txt", "exact_attention_20_amd/csrc/prefill_bwd.hip"),
                            "kernel": "bwd_dq_kernel + bwd_dkdv_kernel", "flops_per_launch": flops},
               "cpu_baseline": res["bwd_cpu"],
               "config": {"workload": wb.name + " (backward)", "B": wb.B, "Hq": wb.Hq, "Hkv": wb.Hkv, "S": wb.S,
                          "D": wb.D, "causal": True}}
        line["backward"] = bwo
        if "value" not in line:
            line.update(value=bwo["value"], unit="TFLOP/s")
            line["roofline"] = bwo["roofline"]
            line["cpu_baseline"] = bwo["cpu_baseline"]
            ms_step = tb
    line["ms_per_step"] = round(ms_step, 5)
    step_names = ([res["prefill"][0]["w"].name] if res["prefill"] else []) + \
                 ([res["decode"][0]["w"].name] if res["decode"] else [])
    if not step_names:
        for key in ("ragged", "cascade", "fp8", "bwd"):
            if key in res:
                step_names = [res[key]["w"].name + (" (backward)" if key == "bwd" else "")]
                break
    cfg = {"workload": " + ".join(step_names)}
    if res["prefill"]:
        wp = res["prefill"][0]["w"]
        cfg["prefill"] = dict(B=wp.B, Hq=wp.Hq, Hkv=wp.Hkv, S=wp.S, D=wp.D, causal=True, dtype="bf16")
    if res["decode"]:
        g = res["decode"][0]
        wd = g["w"]
        cfg["decode"] = dict(B=wd.B, Hq=wd.Hq, Hkv=wd.Hkv, D=wd.D, kv_dtype=wd.kv_dtype, page=64,
                             lengths=list(wd.lengths), total_tokens=g["total_tokens"])
    line["config"] = cfg
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
