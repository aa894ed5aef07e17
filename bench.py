#!/usr/bin/env python3
"""Benchmark of the sliding-window GQA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (`value`): useful (unmasked) TFLOP/s of swa_prefill on the largest
workload, one 16384-token document, Hq = 16, Hkv = 8 (GQA), D = 512,
W = 4096, causal, bf16 ([SDPA] Benchmark: the Gemma-4 full-attention row
"16K, 1 doc, 4K window").  A step is one swa_prefill over one batch; inputs
rotate over resident copies larger than the 256 MB Infinity Cache.  The
other prefill workloads, the backward and the two ring-decode workloads are
measured in the same run and reported under "workloads", each with its own
roofline block.  Times come from HIP events on the stream the kernels run
on, taken on settled GPU clocks: every timed region, the headline's
included, follows the given warm-up and at least 60 ms of untimed work (an
idle GPU runs the first launches at lower clocks).

`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the headline
workload on this host's cores.  A workload's `roofline.traffic` is read from
the counter summary under profiles/ only while its kernel sources still
hash to the value recorded there.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import swa_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # HBM3E
HEADLINE = "prefill_16k_gqa_d512"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the kernel each workload's roofline is about, and the sources it is built from
_PF = ["prefill_kernel.h", "prefill_launch.h"]
WORKLOAD_KERNELS = {
    "prefill_16k_gqa_d512": ("prefill_fwd_kernel", "prefill_fwd_kernel<512, bf16>",
                             _PF + ["prefill_d512.hip"]),
    "prefill_4x1024_mha_d128": ("prefill_fwd_kernel", "prefill_fwd_kernel<128, bf16>",
                                _PF + ["prefill_d128.hip"]),
    "prefill_16k_mha_d128_w4k": ("prefill_fwd_kernel", "prefill_fwd_kernel<128, bf16>",
                                 _PF + ["prefill_d128.hip"]),
    "prefill_vlm_4096_d256": ("prefill_fwd_kernel", "prefill_fwd_kernel<256, bf16>",
                              _PF + ["prefill_d256.hip"]),
    "prefill_4x1024_gqa_d320": ("prefill_fwd_kernel", "prefill_fwd_kernel<384 (320 in memory), bf16>",
                                _PF + ["prefill_d320.hip"]),
    "prefill_16k_gqa4_d128_w4k": ("prefill_fwd_kernel", "prefill_fwd_kernel<128, bf16>",
                                  _PF + ["prefill_d128.hip"]),
    "prefill_16k_gqa2_d128_w4k": ("prefill_fwd_kernel", "prefill_fwd_kernel<128, bf16>",
                                  _PF + ["prefill_d128.hip"]),
    "decode_b64_d256": ("decode_split_kernel", "decode_split_kernel<256, bf16> (decode alone)",
                        ["decode.hip"]),
    "decode_single_d256": ("decode_split_kernel", "decode_split_kernel<256, bf16> (decode alone)",
                           ["decode.hip"]),
}


# ------------------------------------------------------------ work counts
# untimed GPU work before each timed region of the non-headline workloads,
# so that it starts on settled clocks (see settle())
SETTLE_MS = 60.0


def causal_window_pairs(n: int, W: int) -> int:
    """Pairs (i, j), j <= i, i - j < W in one document of n tokens."""
    if W <= 0 or W >= n:
        return n * (n + 1) // 2
    return W * (W + 1) // 2 + (n - W) * W


def useful_pairs(c: si.PrefillCase) -> int:
    """Allowed (query, key) pairs per query head.  The blockwise extra is
    every later key of the same image run (the window is one-sided)."""
    cu = c.cu_seqlens
    total = sum(causal_window_pairs(int(b - a), c.window) for a, b in zip(cu[:-1], cu[1:]))
    if c.mode == si.BLOCKWISE:
        ids = c.ids
        for a, b in zip(cu[:-1], cu[1:]):
            t = int(a)
            while t < int(b):
                e = t
                while e + 1 < int(b) and ids[e + 1] == ids[t]:
                    e += 1
                if ids[t] >= 0:
                    n = e - t + 1
                    total += n * (n - 1) // 2
                t = e + 1
    return total


def useful_flops(c: si.PrefillCase) -> int:
    return 4 * c.d * c.hq * useful_pairs(c)  # 2D for QK^T + 2D for PV per pair


def decode_valid_rows(pos, lo, W):
    low = np.maximum(np.maximum(lo, pos - W + 1), 0)
    return pos - low + 1


def sources_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in WORKLOAD_KERNELS[workload][2]:
        with open(os.path.join(ROOT, "sliding_window_gqa_swa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(workload: str):
    """HBM bytes per launch of the workload's kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on different
    kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def roofline(workload: str, achieved: float, bound: str) -> dict:
    """Roofline block of one workload's dominant kernel: achieved
    algorithmic rate against the MI355X peak of its bound."""
    peak, unit = (PEAK_BF16_TFLOPS, "TFLOP/s") if bound == "mfma" else (PEAK_HBM_GBS, "GB/s")
    return {"bound": bound, "kernel": WORKLOAD_KERNELS[workload][1], "achieved": achieved,
            "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": read_traffic(workload)}


# ------------------------------------------------------------ GPU timing
def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def settle(fn, torch, ms):
    """Call fn(i) until at least `ms` of GPU time has passed: an idle MI355X
    runs the first launches at lower clocks (the headline prefill takes ~68
    us per call from idle, ~60 us after 15 ms of sustained work and 53-56 us
    after 30 ms, measured), so every timed region starts on settled clocks."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    done, n, i = 0.0, 4, 0
    while done < ms:
        e0.record()
        for _ in range(n):
            fn(i)
            i += 1
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)
        n = min(n * 2, 4096)


def time_loop(fn, steps, warmup, torch, settle_ms=0.0):
    """ms per call of fn(i) over `steps` calls, HIP events on the current
    stream, after `warmup` untimed calls (and, with settle_ms, untimed calls
    until the clocks have settled)."""
    for i in range(warmup):
        fn(i)
    if settle_ms > 0:
        settle(fn, torch, settle_ms)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill(name, steps, warmup, torch, api, nsets=None, settle_ms=0.0):
    c = si.PREFILL_WORKLOADS[name]()
    q, k, v = c.tensors("bf16")
    in_bytes = (q.nbytes + k.nbytes + v.nbytes) * 2  # + out
    if nsets is None:
        nsets = max(1, min(6, int(np.ceil(1.1e9 / in_bytes))))
    sets = []
    for s in range(nsets):
        if s == 0:
            qq, kk, vv = q, k, v
        else:
            qq, kk, vv = c.tensors("bf16", seed=c.seed * 1000 + s)
        sets.append((to_dev(qq, torch), to_dev(kk, torch), to_dev(vv, torch)))
    cu = to_dev(c.cu_seqlens, torch)
    ids = to_dev(c.ids, torch) if c.ids is not None else None
    outs = [torch.empty_like(s[0]) for s in sets]

    def step(i):
        s = i % nsets
        api.prefill(sets[s][0], sets[s][1], sets[s][2], cu, ids, c.window, c.mode, out=outs[s])

    ms = time_loop(step, steps, warmup, torch, settle_ms)
    # warm: one input set every call (K/V and Q stay in the Infinity Cache)
    warm_ms = time_loop(lambda i: step(0), steps, warmup, torch, settle_ms)
    fl = useful_flops(c)
    tflops = fl / (ms * 1e-3) / 1e12
    return {
        "workload": name, "T": c.T, "docs": int(c.cu_seqlens.size - 1), "hq": c.hq,
        "hkv": c.hkv, "d": c.d, "window": c.window,
        "mask": "blockwise" if c.mode == si.BLOCKWISE else "causal",
        "useful_flop": fl, "ms_per_call": ms, "tflops": tflops,
        "ms_per_call_warm": warm_ms, "tflops_warm": fl / (warm_ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "input_sets": nsets, "settle_ms": settle_ms,
        "roofline": roofline(name, tflops, "mfma"),
    }


def bench_prefill_chunked(name, nchunks, steps, warmup, torch, api):
    """The workload's single document prefilled in `nchunks` equal chunks
    (swa_prefill_chunk: chunk j's queries against keys 0 .. end of chunk j),
    one after another; useful work equals the whole-prompt prefill's."""
    c = si.PREFILL_WORKLOADS[name]()
    assert c.cu_seqlens.size == 2 and c.T % nchunks == 0 and c.ids is None
    q, k, v = c.tensors("bf16")
    qd, kd, vd = to_dev(q, torch), to_dev(k, torch), to_dev(v, torch)
    out = torch.empty_like(qd)
    L = c.T // nchunks
    cuq = to_dev(np.array([0, L], np.int32), torch)
    cuks = [to_dev(np.array([0, (j + 1) * L], np.int32), torch) for j in range(nchunks)]

    def step(i):
        for j in range(nchunks):
            e = (j + 1) * L
            api.prefill_chunk(qd[j * L:e], kd[:e], vd[:e], cuq, cuks[j], None, c.window, c.mode,
                              out=out[j * L:e])

    ms = time_loop(step, steps, warmup, torch, SETTLE_MS)
    fl = useful_flops(c)
    return {"workload": name + "_in_%d_chunks" % nchunks, "chunk_tokens": L, "useful_flop": fl,
            "ms_per_prompt": ms, "tflops": fl / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_prefill_backward(name, steps, warmup, torch, api, pages_fwd_bwd_ms=None):
    """swa_prefill_backward (dq, dk, dv: three launches) on the workload, as
    a training step runs it: the forward (swa_prefill_lse) stores each row's
    log-sum-exp and the backward takes it.  Also timed: the backward that
    recomputes the log-sum-exp itself, and forward + backward.  Useful work
    of the backward: 2.5x the forward's useful FLOPs, the five products of
    2 * D FLOPs per allowed pair and head that a backward which keeps no
    score matrix needs (S again, dP, dv, dk, dq)."""
    c = si.PREFILL_WORKLOADS[name]()
    q, k, v = c.tensors("bf16")
    qd, kd, vd = to_dev(q, torch), to_dev(k, torch), to_dev(v, torch)
    cu = to_dev(c.cu_seqlens, torch)
    ids = to_dev(c.ids, torch) if c.ids is not None else None
    do = to_dev(si.normal(si.rng_for(c.seed + 500), q.shape, "bf16"), torch)
    out, lse = api.prefill_lse(qd, kd, vd, cu, ids, c.window, c.mode)
    ws = torch.empty(api.prefill_backward_workspace_bytes(c.T, c.hq), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)

    def bwd(i):
        api.prefill_backward(qd, kd, vd, out, do, cu, ids, c.window, c.mode, dq, dk, dv, ws,
                             lse=lse)

    def bwd_recompute(i):
        api.prefill_backward(qd, kd, vd, out, do, cu, ids, c.window, c.mode, dq, dk, dv, ws)

    def fwd_bwd(i):
        api.prefill_lse(qd, kd, vd, cu, ids, c.window, c.mode, out=out, lse=lse)
        bwd(i)

    ms = time_loop(bwd, steps, warmup, torch, SETTLE_MS)
    ms_rc = time_loop(bwd_recompute, steps, warmup, torch, SETTLE_MS)
    ms_fb = time_loop(fwd_bwd, steps, warmup, torch, SETTLE_MS)
    fl = 5 * useful_flops(c) // 2
    r = {"workload": name + "_backward", "useful_flop": fl, "ms_per_call": ms,
         "tflops": fl / (ms * 1e-3) / 1e12,
         "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
         "ms_per_call_recomputing_lse": ms_rc, "ms_forward_plus_backward": ms_fb}
    if pages_fwd_bwd_ms is not None:
        # context only: another machine's forward + backward of this shape
        r["pages_h100_sdpa_mask_fwd_bwd_ms"] = pages_fwd_bwd_ms
    return r


def bench_decode(name, torch, api, layers=4, warmup=3, reps=20):
    """Append + decode per step over `layers` independent ring sets (one per
    simulated sliding layer).  The roll is issued before every A-th append
    after compaction (A = ring_rows - window = 64): for a batch compacted
    together that is exactly when the rings are full.  The kernel itself
    decides per sequence on the device, so this cadence is only a saving of
    launches, never a correctness assumption.  The same steps are then timed
    as one swa_decode_step launch per layer (metadata roll + append +
    decode), eagerly and as one captured HIP graph of the whole run."""
    c = si.DECODE_WORKLOADS[name]()
    ks, vs = c.prompt_tail("bf16")
    B, hq, hkv, d, R, W = c.batch, c.hq, c.hkv, c.d, c.ring_rows, c.window
    rings = []
    for _ in range(layers):
        kr = torch.zeros((B, hkv, R, d), dtype=torch.bfloat16, device="cuda")
        vr = torch.zeros_like(kr)
        meta = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
        api.cache_compact(to_dev(ks, torch), to_dev(vs, torch), to_dev(c.cu_tail, torch), kr, vr,
                          meta, W, to_dev(c.prompt_lens, torch), to_dev(c.left_pad, torch))
        rings.append((kr, vr, meta))
    # timed steps: the workload's own, or 32 consecutive ones when it has
    # fewer (the single-sequence step at position 3000 is then timed over
    # positions 3000..3031, which include the roll at 3008)
    nsteps = max(c.steps, 32)
    steps_in = []
    for s in range(-c.pre_appends, nsteps):
        q, kn, vn = c.step_inputs(s, "bf16")
        steps_in.append((to_dev(q, torch), to_dev(kn, torch), to_dev(vn, torch)))
    ws = api.decode_workspace(steps_in[0][0], rings[0][0])
    outs = [torch.empty_like(steps_in[0][0]) for _ in range(layers)]
    A = R - W
    # pre-appends (not timed): bring the single-sequence case to position 3000
    for s in range(c.pre_appends):
        q, kn, vn = steps_in[s]
        for kr, vr, meta in rings:
            if s > 0 and s % A == 0:
                api.cache_roll(kr, vr, meta, W)
            api.cache_append(kn, vn, kr, vr, meta)
    torch.cuda.synchronize()
    timed = steps_in[c.pre_appends:]
    # settled clocks first (decode alone only reads the rings)
    q_last = timed[-1][0]
    settle(lambda i: api.decode(q_last, rings[i % layers][0], rings[i % layers][1],
                                rings[i % layers][2], W, out=outs[i % layers], workspace=ws),
           torch, SETTLE_MS)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for t, (q, kn, vn) in enumerate(timed):
        n_app = c.pre_appends + t  # appends since compaction
        for li, (kr, vr, meta) in enumerate(rings):
            if n_app > 0 and n_app % A == 0:
                api.cache_roll(kr, vr, meta, W)
            api.cache_append(kn, vn, kr, vr, meta)
            api.decode(q, kr, vr, meta, W, out=outs[li], workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / (len(timed) * layers)
    # decode alone on the final state, rotating over the ring sets (cold)
    q = timed[-1][0]

    def dstep(i):
        kr, vr, meta = rings[i % layers]
        api.decode(q, kr, vr, meta, W, out=outs[i % layers], workspace=ws)

    dec_ms = time_loop(dstep, reps * layers, warmup * layers, torch, SETTLE_MS)
    # cold: copies of the final ring state, as many as exceed 512 MB (twice
    # the 256 MB Infinity Cache), so that every decode reads its rings from HBM
    set_bytes = rings[0][0].numel() * rings[0][0].element_size() * 2
    ncold = max(layers, int(np.ceil(512e6 / set_bytes)))
    cold = [(rings[0][0].clone(), rings[0][1].clone(), rings[0][2].clone())
            for _ in range(ncold)]

    def cstep(i):
        kr, vr, meta = cold[i % ncold]
        api.decode(q, kr, vr, meta, W, out=outs[0], workspace=ws)

    cold_ms = time_loop(cstep, max(reps * layers, ncold), ncold, torch, SETTLE_MS)
    del cold
    # warm: the same ring set every call
    warm_ms = time_loop(lambda i: api.decode(q, rings[0][0], rings[0][1], rings[0][2], W,
                                             out=outs[0], workspace=ws), reps, warmup, torch,
                        SETTLE_MS)

    # the same steps as one swa_decode_step launch per layer (roll by
    # metadata + append + decode), on freshly compacted ring sets
    def fresh_rings():
        for kr, vr, meta in rings:
            api.cache_compact(to_dev(ks, torch), to_dev(vs, torch), to_dev(c.cu_tail, torch), kr, vr,
                              meta, W, to_dev(c.prompt_lens, torch), to_dev(c.left_pad, torch))
        for s in range(c.pre_appends):
            q0, kn0, vn0 = steps_in[s]
            for li, (kr, vr, meta) in enumerate(rings):
                api.decode_step(q0, kn0, vn0, kr, vr, meta, W, out=outs[li], workspace=ws)
        torch.cuda.synchronize()

    settle(dstep, torch, SETTLE_MS)
    fresh_rings()
    e0.record()
    for t, (qq, kn, vn) in enumerate(timed):
        for li, (kr, vr, meta) in enumerate(rings):
            api.decode_step(qq, kn, vn, kr, vr, meta, W, out=outs[li], workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    fused_us = e0.elapsed_time(e1) * 1e3 / (len(timed) * layers)
    # and the whole run (every step of every layer) captured in one HIP graph
    # and replayed: no host launch cost per kernel
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t, (qq, kn, vn) in enumerate(timed):
            for li, (kr, vr, meta) in enumerate(rings):
                api.decode_step(qq, kn, vn, kr, vr, meta, W, out=outs[li], workspace=ws)
    fresh_rings()
    graph.replay()  # warm-up
    settle(dstep, torch, SETTLE_MS)
    fresh_rings()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (len(timed) * layers)
    alg_bytes = decode_alg_bytes(c, nsteps)
    scanned = B * hkv * R * d * 2 * 2
    gbs = alg_bytes / (cold_ms * 1e-3) / 1e9
    return {
        "workload": name, "batch": B, "hq": hq, "hkv": hkv, "d": d, "window": W,
        "ring_rows": R, "steps": len(timed), "layers_rotated": layers,
        "us_per_step_append_decode_roll": step_us, "rolls_in_run": sum(
            1 for t in range(len(timed)) if (c.pre_appends + t) > 0 and (c.pre_appends + t) % A == 0),
        "decode_us": cold_ms * 1e3, "decode_cold_ring_sets": ncold,
        "decode_us_4_layers": dec_ms * 1e3, "decode_warm_us": warm_ms * 1e3,
        "us_per_step_fused": fused_us, "us_per_step_fused_graph": graph_us,
        "algorithmic_bytes": alg_bytes, "full_ring_bytes": scanned,
        "decode_gbs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
        "roofline": roofline(name, gbs, "hbm"),
    }


def peak_clock_mhz(device=0):
    """The GPU's peak shader clock as the HIP runtime of libswa reports it
    (hipDeviceGetAttribute with hipDeviceAttributeClockRate, in kHz), or
    None.  The clock under load is lower; kernel traces show it."""
    import ctypes
    from sliding_window_gqa_swa_amd import _lib
    try:
        fn = _lib.lib().hipDeviceGetAttribute  # resolved through libswa's HIP runtime
    except AttributeError:
        return None
    fn.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    fn.restype = ctypes.c_int
    v = ctypes.c_int(0)
    kClockRate = 5  # position of hipDeviceAttributeClockRate in hipDeviceAttribute_t
    return v.value / 1000.0 if fn(ctypes.byref(v), kClockRate, device) == 0 else None


# ------------------------------------------------------------ CPU baseline
def cpu_model_name():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=15.0):
    """fp64 oracle on a bounded, seeded sample of the headline workload."""
    from oracle import oracle as orc
    c = si.PREFILL_WORKLOADS[HEADLINE]()
    q, k, v = c.tensors("bf16")
    rng = si.rng_for(99)
    order = rng.permutation(c.T).astype(np.int32)
    threads = orc.max_threads()
    cu = c.cu_seqlens
    doc = np.searchsorted(cu, np.arange(c.T), side="right") - 1
    start = cu[doc]
    keys = np.minimum(np.arange(c.T) - start + 1, c.window)
    done, flops, t0 = 0, 0, time.perf_counter()
    chunk = 256
    while time.perf_counter() - t0 < budget_s and done < 32 * c.T:
        rows = order[np.arange(done, done + chunk) % c.T]
        orc.prefill(q, k, v, cu, None, c.window, c.mode, rows=rows, nthreads=threads)
        flops += int(keys[rows].sum()) * 4 * c.d * c.hq
        done += rows.size
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model_name(),
        "sample": "%d query rows x %d heads of %s (%.2f passes over its %d rows, seeded "
                  "random order), fp64, %.1f s" % (done, c.hq, HEADLINE, done / c.T, c.T, dt),
    }


def decode_alg_bytes(c, nsteps):
    """Algorithmic bytes of one decode of the workload's batch at its state
    after `nsteps` timed steps: K and V of the valid rows, q, out, meta."""
    pos = c.prompt_lens.astype(np.int64) - 1 + c.pre_appends + nsteps
    valid = decode_valid_rows(pos, c.left_pad.astype(np.int64), c.window)
    es = 2
    return int(valid.sum()) * c.hkv * c.d * es * 2 + 2 * c.batch * c.hq * c.d * es + c.batch * 16


def _kernel_matches(workload, name):
    """Is the dispatched kernel `name` (mangled) the one whose traffic the
    workload's roofline reports (bf16, plain variant)?"""
    import re
    if workload.startswith("prefill"):
        m = re.search(r"prefill_fwd_kernelILi(\d+)EDF16b.*?ELb(\d)ELb(\d)ELi(\d+)E", name)
        return m is not None and m.group(3) == "0"
    m = re.search(r"decode_split_kernelILi(\d+)EDF16bLi(\d+)ELb(\d)E", name)
    return m is not None and m.group(3) == "0"


def record_traffic(workload, fetch_dir, write_dir):
    """Add the workload's record to profiles/traffic.json from two rocprofv3
    --pmc runs of `bench.py --only WORKLOAD --copy-calibration`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled
    by what it reads for the 512 MiB device copy of the same run (known
    bytes)."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals, calib = {}, {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                tgt = vals if _kernel_matches(workload, r["Kernel_Name"]) else (
                    calib if "copyBuffer" in r["Kernel_Name"] else None)
                if tgt is not None:
                    tgt[key] = tgt.get(key, 0.0) + float(r["Counter_Value"])
        return list(vals.values()), max(calib.values()) if calib else None

    fetch, fcal = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, wcal = per_dispatch(write_dir, "WRITE_SIZE")
    if not fetch or not write or not fcal or not wcal:
        raise SystemExit("counter files lack the kernel or the copy calibration")
    copy_kib = 512 * 1024.0
    fs, ws = copy_kib / fcal, copy_kib / wcal
    if workload in si.PREFILL_WORKLOADS:
        c = si.PREFILL_WORKLOADS[workload]()
        q, k, v = c.tensors("bf16")
        alg = q.nbytes + k.nbytes + v.nbytes + q.nbytes  # q, k, v read once; out written once
    else:
        c = si.DECODE_WORKLOADS[workload]()
        alg = decode_alg_bytes(c, max(c.steps, 32))
    fb = float(np.mean(fetch)) * 1024 * fs
    wb = float(np.mean(write)) * 1024 * ws
    rec = {
        "workload": workload, "kernel": WORKLOAD_KERNELS[workload][1],
        "fetch_kib_raw": float(np.mean(fetch)), "write_kib_raw": float(np.mean(write)),
        "fetch_kib_min_max": [float(np.min(fetch)), float(np.max(fetch))],
        "dispatches": [len(fetch), len(write)],
        "copy_fetch_kib": fcal, "copy_write_kib": wcal,
        "fetch_scale": fs, "write_scale": ws,
        "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
        "bytes_per_launch": int(fb + wb), "algorithmic_bytes_per_launch": int(alg),
        "traffic_over_algorithmic": (fb + wb) / alg,
        "sources_sha256": sources_hash(workload),
    }
    try:
        with open(TRAFFIC_FILE) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {}
    allrec = {k2: v2 for k2, v2 in allrec.items() if k2 in WORKLOAD_KERNELS}
    allrec[workload] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=2, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec, indent=2))


def summarize_trace(trace_dir):
    """Per-kernel table (markdown) from a `rocprofv3 --kernel-trace` database
    under trace_dir: calls, total / average / min / max duration, grouped by
    kernel and grid size."""
    import glob
    import re
    import sqlite3
    dbs = glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit("no rocprofv3 database under %s" % trace_dir)
    cur = sqlite3.connect(dbs[0]).cursor()
    # (grouped by the mangled symbol: the trace's display names drop template
    # arguments of some kernels)
    rows = cur.execute(
        "select coalesce(s.kernel_name, k.name), k.grid_x, k.workgroup_x, count(*), "
        "sum(k.duration), avg(k.duration), min(k.duration), max(k.duration) from kernels k "
        "left join kernel_symbols s on s.kernel_id = k.kernel_id "
        "group by coalesce(s.kernel_name, k.name), k.grid_x "
        "order by sum(k.duration) desc").fetchall()
    tot = sum(r[4] for r in rows) or 1

    def short(nm):
        m = re.search(r"prefill_fwd_kernelILi(\d+)E(DF16b|f)Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d+)E", nm)
        if m:
            return "prefill_fwd_kernel<D=%s,%s,MB=%s,BN=%s,NW=%s,GH=%s%s%s%s>" % (
                m.group(1), "bf16" if m.group(2) == "DF16b" else "f32", m.group(3), m.group(4),
                m.group(5), m.group(6), ",pipelined" if m.group(7) == "1" else "",
                ",lse" if m.group(8) == "1" else "",
                "" if m.group(9) == m.group(1) else ",head size %s in memory" % m.group(9))
        m = re.search(r"bwd_dq_kernelILi(\d+)E(DF16b|f)Li(\d+)E", nm)
        if m:
            return "bwd_dq_kernel<D=%s,%s,MB=%s>" % (
                m.group(1), "bf16" if m.group(2) == "DF16b" else "f32", m.group(3))
        m = re.search(r"bwd_dkdv_kernelILi(\d+)E(DF16b|f)Li(\d+)ELi(\d+)ELi(\d+)E", nm)
        if m:
            return "bwd_dkdv_kernel<D=%s,%s,DS=%s,KB=%s>" % (
                m.group(1), "bf16" if m.group(2) == "DF16b" else "f32", m.group(3), m.group(4))
        if "bwd_rows_kernel" in nm:
            return "bwd_rows_kernel"
        m = re.search(r"decode_split_kernelILi(\d+)E(DF16b|f)Li(\d+)ELb(\d)", nm)
        if m:
            return "decode_split_kernel<D=%s,%s,GB=%s%s>" % (
                m.group(1), "bf16" if m.group(2) == "DF16b" else "f32", m.group(3),
                ",step" if m.group(4) == "1" else "")
        m = re.search(r"(ring_\w+_kernel)", nm)
        if m:
            return m.group(1)
        return nm.split("(")[0].replace("void ", "")[:48]

    print("| kernel | grid (threads) | calls | total us | avg us | min us | max us | % |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        print("| %s | %d | %d | %.1f | %.2f | %.2f | %.2f | %.1f |" % (
            short(r[0]), r[1], r[3], r[4] / 1e3, r[5] / 1e3, r[6] / 1e3, r[7] / 1e3,
            100.0 * r[4] / tot))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # (after the warm-up, every timed region, the headline's included, also
    # waits for 60 ms of untimed work: settled clocks)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="run one workload (a prefill or decode workload, or a prefill "
                         "workload name + '_backward') and print its result (for counter "
                         "runs; not the benchmark line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy 4 times (known bytes, for "
                         "scaling HBM counters)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="add the workload's record to profiles/traffic.json from two "
                         "rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) of "
                         "`--only WORKLOAD --copy-calibration` and exit (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print a per-kernel table from a rocprofv3 --kernel-trace database "
                         "and exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested); prefill and decode would shard by kv head or by "
              "sequence, with no exchange between GPUs" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from sliding_window_gqa_swa_amd import api
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def log(r, name):
        if "decode_us" in r:
            print("%s: %.2f us/step (roll + append + decode), fused %.2f us/step (graph %.2f), "
                  "decode %.2f us cold, %.2f us warm, %.0f GB/s" % (
                      name, r["us_per_step_append_decode_roll"], r["us_per_step_fused"],
                      r["us_per_step_fused_graph"], r["decode_us"], r["decode_warm_us"],
                      r["decode_gbs"]), file=sys.stderr, flush=True)
        elif "ms_per_call_recomputing_lse" in r:
            print("%s: %.3f ms, %.1f TFLOP/s (recomputing lse %.3f ms; forward + backward "
                  "%.3f ms)" % (name, r["ms_per_call"], r["tflops"],
                                r["ms_per_call_recomputing_lse"], r["ms_forward_plus_backward"]),
                  file=sys.stderr, flush=True)
        elif "ms_per_prompt" in r:
            print("%s: %.3f ms, %.1f TFLOP/s" % (name, r["ms_per_prompt"], r["tflops"]),
                  file=sys.stderr, flush=True)
        else:
            print("%s: %.3f ms, %.1f TFLOP/s (%.3f of bf16 peak)" % (
                name, r["ms_per_call"], r["tflops"], r["frac_of_bf16_peak"]),
                file=sys.stderr, flush=True)

    # ([SDPA] Benchmark: forward + backward on H100 with the explicit-mask
    # SDPA path: 612 ms for the 16K, window-4K, 16/8-head, D = 512 shape and
    # 50 ms for the 16K, window-4K, 32-head, D = 128 shape; context only)
    pages_fb = {"prefill_16k_gqa_d512": 612.0, "prefill_16k_mha_d128_w4k": 50.0}
    bwd_steps = {"prefill_16k_gqa_d512": 3, "prefill_16k_mha_d128_w4k": 5}
    if args.only:
        name = args.only
        if name in si.DECODE_WORKLOADS:
            r = bench_decode(name, torch, api)
        elif name.endswith("_backward") and name[:-9] in si.PREFILL_WORKLOADS:
            base = name[:-9]
            r = bench_prefill_backward(base, bwd_steps.get(base, 20), 2, torch, api,
                                       pages_fb.get(base))
        elif name in si.PREFILL_WORKLOADS:
            r = bench_prefill(name, args.steps, args.warmup, torch, api, settle_ms=SETTLE_MS)
        else:
            raise SystemExit("unknown workload %s" % name)
        log(r, name)
        print(json.dumps({"workloads": {name: r}}), flush=True)
        return

    head = bench_prefill(HEADLINE, args.steps, args.warmup, torch, api, settle_ms=SETTLE_MS)
    log(head, "headline " + HEADLINE)
    workloads = {HEADLINE: head}
    for name in ("prefill_4x1024_mha_d128", "prefill_vlm_4096_d256", "prefill_4x1024_gqa_d320",
                 "prefill_16k_mha_d128_w4k"):
        steps = max(5, args.steps) if si.PREFILL_WORKLOADS[name]().T <= 4096 else max(5, args.steps // 4)
        workloads[name] = bench_prefill(name, steps, 3, torch, api, settle_ms=SETTLE_MS)
        log(workloads[name], name)
    ch = bench_prefill_chunked("prefill_16k_gqa_d512", 8, 5, 2, torch, api)
    workloads[ch["workload"]] = ch
    log(ch, ch["workload"])
    for name, st in (("prefill_4x1024_mha_d128", 20), ("prefill_vlm_4096_d256", 20),
                     ("prefill_16k_gqa_d512", 3), ("prefill_16k_mha_d128_w4k", 5)):
        b = bench_prefill_backward(name, st, 2, torch, api, pages_fb.get(name))
        workloads[b["workload"]] = b
        log(b, b["workload"])
    for name in ("decode_b64_d256", "decode_single_d256"):
        workloads[name] = bench_decode(name, torch, api)
        log(workloads[name], name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
        print("cpu baseline: %.4f TFLOP/s on %d threads" % (cpu["value"], cpu["cores"]),
              file=sys.stderr, flush=True)
    c = si.PREFILL_WORKLOADS[HEADLINE]()
    line = {
        "metric": "SWA prefill useful TFLOP/s (one 16384-token causal document, GQA 16/8 heads, "
                  "D=512, W=4096); decode us/step + HBM GB/s under workloads",
        "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_call"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) rounded to bf16",
        "config": {"workload": HEADLINE, "docs": 1, "total_tokens": c.T, "hq": c.hq,
                   "hkv": c.hkv, "head_dim": c.d, "window": c.window, "mask": "causal",
                   "useful_flop_per_step": head["useful_flop"], "input_sets": head["input_sets"],
                   "settle_ms_before_timed_steps": SETTLE_MS},
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": props.gcnArchName,
                   "cus": props.multi_processor_count, "peak_clock_mhz": peak_clock_mhz()},
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
