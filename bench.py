#!/usr/bin/env python3
"""Benchmark of the KDA core (libkda) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one kda_chunk_fwd over the long-context workload: B=1, H=12
(one GPU's share of 96 heads), T=2^20 tokens, d_k=d_v=128, chunk 64, bf16
q/k/v, fp32 gate and beta logits, fp32 initial state; inputs drawn on the
device (seed 0) and resident in HBM before the timed region.  Value = tokens/s
of the whole call (prep + intra + chain kernels), inputs already in HBM.

Also reported: per-kernel durations from HIP events recorded by libkda on the
stream its kernels run on (kda_chunk_fwd_timed), the roofline of the dominant
kernel, the decode workload (256 sequences x 12 heads, 16 single-token
steps), the layer entry points, the family modes and the general DPLR
update on the same shapes, and the fp64 CPU oracle timed on a bounded prefix
of the same workload.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (12 heads, d=128, 1M ctx) + MFMA%; decode tokens/s + HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
# algorithmic work per token and head of the prefill (d = 128, C = 64):
#   bytes: q, k, v bf16 (3 x 256) + z fp32 (512) + beta logit (4) + o bf16 (256)
#   flops: 6 d_k d_v + C (3 d_k + 2 d_v)
PREFILL_BYTES = 1540
PREFILL_FLOPS = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128)
# the same bytes split by kernel: the intra kernel must read q, k, v, z, b;
# the chain kernel must write o (the 64 KiB initial/final states per head are
# added per launch)
INTRA_BYTES = 1284
CHAIN_BYTES = 256
# decode: read + write one fp32 state (2 x 64 KiB) + 1540 B of per-token I/O
DECODE_BYTES = 2 * 128 * 128 * 4 + PREFILL_BYTES
# general DPLR update, per token and head: q, k, v, a, b bf16 (5 x 256) + z fp32
# (512) + o bf16 (256); its intra kernel must read all but o
DPLR_BYTES = 2048
DPLR_INTRA_BYTES = 1792
# chunk records the intra kernels write (bytes per chunk and head)
KDA_RECORD_BYTES = 72192
DPLR_RECORD_BYTES = 98816


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def _event(h):
    e = ctypes.c_void_p()
    if h.hipEventCreate(ctypes.byref(e)) != 0:
        raise RuntimeError("hipEventCreate failed")
    return e


def _elapsed(h, a, b) -> float:
    ms = ctypes.c_float()
    if h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return float(ms.value)


def code_sha1(path: str) -> str:
    """sha1 of a C++/HIP source with comments and whitespace removed, so that
    a change to comments alone keeps a counter record valid."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha1(" ".join(text.split()).encode()).hexdigest()


# sources whose code the counter records in profiles/ were taken from
PREFILL_SOURCES = ["gated_delta_rule_77_amd/csrc/kda_chunk_fast.hip",
                   "gated_delta_rule_77_amd/csrc/kda_fast_common.hpp",
                   "gated_delta_rule_77_amd/csrc/kda_internal.hpp",
                   "gated_delta_rule_77_amd/csrc/kda_device.hpp"]
DECODE_SOURCES = ["gated_delta_rule_77_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_77_amd/csrc/kda_step.hpp",
                  "gated_delta_rule_77_amd/csrc/kda_internal.hpp",
                  "gated_delta_rule_77_amd/csrc/kda_device.hpp"]


def sources_sha1(paths) -> dict:
    return {p: code_sha1(os.path.join(ROOT, p)) for p in paths}


def _counter_record(name: str):
    """A committed counter record (profiles/<name>.json), or None when any of
    the sources it was taken from has changed since."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        rec = json.load(open(path))
        src = rec["sources"]
        if sources_sha1(src.keys()) != src:
            return None
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    return rec


def _traffic_for(kernel: str, split: bool = False):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic_long_1m.json), or None when the kernel code changed
    since the counters were taken.  With split, the (read, write) bytes."""
    rec = _counter_record("traffic_long_1m")
    k = None if rec is None else rec.get("kernels", {}).get(kernel)
    if k is None:
        return None
    if not split:
        return int(k["hbm_bytes"])
    cal = rec["calibration"]
    return [int(round(k["FETCH_SIZE_KiB"] * cal["fetch_factor"] * 1024)),
            int(round(k["WRITE_SIZE_KiB"] * cal["write_factor"] * 1024))]


def _path_traffic():
    """HBM bytes of one whole prefill call (every launch of the KDA core in
    the counter record), or None when any kernel's code changed since."""
    rec = _counter_record("traffic_long_1m")
    if rec is None:
        return None
    return int(sum(k["hbm_bytes"] for k in rec.get("kernels", {}).values()))


def _mfma_counters(call_ms: float):
    """MFMA utilisation of the prefill kernels from the committed counter
    record (profiles/mfma_long_1m.json): per kernel the busy fraction of the
    matrix cores (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) and
    the MFMA FLOPs the hardware executed (bf16 and f32 MOPS x 512), which
    include the chain's re-runs; None when the kernel code changed."""
    rec = _counter_record("mfma_long_1m")
    if rec is None:
        return None
    ks = rec["kernels"]
    hw = sum(k["bf16_flop"] + k["f32_flop"] for k in ks.values())
    return {"busy_frac": {n: k["busy_frac"] for n, k in ks.items()},
            "hw_mfma_TFLOP_per_call": round(hw / 1e12, 4),
            "hw_mfma_TFLOPs": round(hw / (call_ms * 1e-3) / 1e12, 1),
            "hw_mfma_frac": round(hw / (call_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}


def bench_prefill(args, kda, torch, KI):
    case = KI.CONFIGS["long_1m"]
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = KI.make_prefill(case, device=dev, seed=0)
    torch.cuda.synchronize()
    print(f"[bench] long_1m inputs drawn on the device in {time.time() - t0:.1f} s", flush=True)
    B, T, H, dk, dv, N, C = d["B"], d["T"], d["H"], d["dk"], d["dv"], d["N"], d["chunk"]
    L = kda.lib()
    wsb = kda.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, C, torch.bfloat16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    h = _hip()
    nsteps = args.warmup + args.steps
    evs = [[_event(h) for _ in range(6)] for _ in range(nsteps)]
    ptrs = (d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["z"].data_ptr(),
            d["b"].data_ptr(), d["A"].data_ptr(), d["h0"].data_ptr(), None, B, T, H, dk, dv, N,
            C, 1, o.data_ptr(), hT.data_ptr(), ws.data_ptr(), wsb)

    def step(i):
        arr = (ctypes.c_void_p * 6)(*[e.value for e in evs[i]])
        rc = L.kda_chunk_fwd_timed(*ptrs, arr, 6, stream)
        if rc != 0:
            raise RuntimeError(L.kda_status_string(rc).decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {"prep": [], "intra": [], "transition": [], "compose": [], "output": [], "chain": [],
           "call": []}
    for i in range(args.warmup, nsteps):
        e = evs[i]
        per["prep"].append(_elapsed(h, e[0], e[1]))
        per["intra"].append(_elapsed(h, e[1], e[2]))
        per["transition"].append(_elapsed(h, e[2], e[4]))
        per["compose"].append(_elapsed(h, e[4], e[5]))
        per["output"].append(_elapsed(h, e[5], e[3]))
        per["chain"].append(_elapsed(h, e[2], e[3]))
        per["call"].append(_elapsed(h, e[0], e[3]))
    for row in evs:
        for e in row:
            h.hipEventDestroy(e)
    avg = {k: sum(v) / len(v) for k, v in per.items()}
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] prefill: {ms_per_step:.3f} ms/step wall; events (ms): "
          + ", ".join(f"{k} {v:.3f}" for k, v in avg.items()), flush=True)
    tokens = B * T
    units = tokens * H
    kernels = {
        "fast_intra_kernel": {"ms": avg["intra"], "alg_bytes": INTRA_BYTES * units},
        "seg_out_kernel": {"ms": avg["output"],
                                  "alg_bytes": CHAIN_BYTES * units + 2 * N * H * dk * dv * 4},
    }
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    achieved = kd["alg_bytes"] / (kd["ms"] * 1e-3) / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic_for(dom),
            # reads are the kernel's inputs once; writes are the chunk records
            # the chain launches read back (the three-launch design)
            "traffic_read_write": _traffic_for(dom, split=True)}
    call_gbs = PREFILL_BYTES * units / (avg["call"] * 1e-3) / 1e9
    call_tfs = PREFILL_FLOPS * units / (avg["call"] * 1e-3) / 1e12
    mc = _mfma_counters(avg["call"])
    # the whole kda_chunk_fwd call beside the dominant kernel: the algorithmic
    # FLOPs (the MFMA side of the metric) and bytes of the path over the
    # call's event time, and the HBM bytes all its launches moved
    roof["call"] = {"ms": round(avg["call"], 4),
                    "mfma_frac": round(call_tfs / MFMA_BF16_PEAK_TFS, 4),
                    "achieved_TFLOPs": round(call_tfs, 2), "mfma_peak_TFLOPs": MFMA_BF16_PEAK_TFS,
                    "hbm_frac": round(call_gbs / HBM_PEAK_GBS, 4),
                    "achieved_GBps": round(call_gbs, 1),
                    "alg_bytes": PREFILL_BYTES * units, "alg_flops": PREFILL_FLOPS * units,
                    "traffic": _path_traffic(),
                    "hw_mfma_frac": None if mc is None else mc["hw_mfma_frac"]}
    extra = {
        "call_ms_events": round(avg["call"], 4),
        "kernels_ms": {k: round(v, 4) for k, v in avg.items() if k not in ("call", "chain")},
        "path_alg_GBps": round(call_gbs, 1),
        "path_hbm_frac": round(call_gbs / HBM_PEAK_GBS, 4),
        "path_alg_TFLOPs": round(call_tfs, 2),
        "mfma_frac_algorithmic": round(call_tfs / MFMA_BF16_PEAK_TFS, 4),
        "mfma_counters": mc,
    }
    del ws, o, hT, d
    torch.cuda.empty_cache()
    return tokens / (ms_per_step * 1e-3), ms_per_step, roof, extra


# decode states stepped in turn, standing in for as many layers of a model:
# their 4 x 192 MiB exceed the 256 MB Infinity Cache, so each step reads and
# writes its state in HBM (one layer's state is never cache-resident between
# its own steps in serving: the other layers' states pass through in between)
DECODE_STATE_SETS = 4


def _decode_loop_times(kda, torch, run, states, reps):
    """Per-step event times of reps passes over the 16 steps; step i updates
    states[i % len(states)] in place."""
    A, steps = run["A"], run["steps"]
    times = []
    for _ in range(reps):
        for i, s in enumerate(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            kda.kda_recurrent_step(s["q"], s["k"], s["v"], s["z"], s["b"], A, states[i % len(states)])
            b.record()
            times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    return ms


def _decode_summary(run, ms):
    mean = sum(ms) / len(ms)
    gbs = DECODE_BYTES * run["N"] * run["H"] / (mean * 1e-3) / 1e9
    return {"steps_timed": len(ms), "ms_per_step_mean": round(mean, 4),
            "ms_per_step_median": round(ms[len(ms) // 2], 4),
            "tokens_per_s": round(run["N"] / (mean * 1e-3), 1), "alg_GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_decode(args, kda, torch, KI, cpu=None):
    """The decode workload (256 sequences x 12 heads, 16 single-token steps).
    Headline: DECODE_STATE_SETS states stepped in turn (a working set of
    768 MiB, beyond the Infinity Cache), eagerly and replayed from one
    captured HIP graph.  Beside it, the same steps on one state in place
    (cache-warm: its 192 MiB can stay in the Infinity Cache)."""
    case = KI.CONFIGS["decode_256"]
    dev = torch.device("cuda:0")
    run = KI.make_decode(case, device=dev, seed=0)
    A, st = run["A"], run["state"]
    steps = run["steps"]
    for s in steps[:2]:                       # warm-up on a scratch copy
        kda.kda_recurrent_step(s["q"], s["k"], s["v"], s["z"], s["b"], A, st.clone())
    torch.cuda.synchronize()
    sets = [st.clone() for _ in range(DECODE_STATE_SETS)]
    rot = _decode_summary(run, _decode_loop_times(kda, torch, run, sets, args.decode_reps))
    rot_graph = bench_decode_graph(args, kda, torch, run, DECODE_STATE_SETS)
    del sets
    warm_ms = _decode_loop_times(kda, torch, run, [st], args.decode_reps)
    warm = _decode_summary(run, warm_ms)
    warm["graph"] = bench_decode_graph(args, kda, torch, run, 1)
    warm["note"] = ("one 192 MiB state stepped in place: it can stay in the 256 MB Infinity "
                    "Cache, so alg_GBps may exceed what HBM delivers")
    fold = bench_fold(args, kda, torch, run, rot["ms_per_step_mean"])
    out = {"workload": "decode_256: N=256 sequences, H=12, d=128, fp32 state, bf16 q/k/v; "
                       f"{DECODE_STATE_SETS} state sets stepped in turn "
                       f"({DECODE_STATE_SETS * 192} MiB, beyond the Infinity Cache)"}
    out.update(rot)
    out.update({"graph": rot_graph, "cache_warm": warm,
                "traffic": _decode_traffic(warm["ms_per_step_mean"]),
                "cpu_baseline": cpu, "fold": fold})
    return out


def bench_decode_graph(args, kda, torch, run, n_sets):
    """The 16 decode steps captured once into a HIP graph (the launch-bound
    serving loop) and replayed back to back: per-step time without the
    per-launch host and event overhead of the eager loop.  Step i updates
    state set i % n_sets.  The first replay's states are compared bit for bit
    with 16 eager steps from the same states."""
    A, steps = run["A"], run["steps"]
    st0 = [run["state"].clone() for _ in range(n_sets)]
    st = [x.clone() for x in st0]

    def loop(states):
        for i, s in enumerate(steps):
            kda.kda_recurrent_step(s["q"], s["k"], s["v"], s["z"], s["b"], A, states[i % n_sets])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop([x.clone() for x in st0])         # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop(st)
    for a, b in zip(st, st0):
        a.copy_(b)
    torch.cuda.synchronize()
    g.replay()
    ref = [x.clone() for x in st0]
    loop(ref)
    torch.cuda.synchronize()
    same = all(bool(torch.equal(a, b)) for a, b in zip(st, ref))
    del ref
    reps = max(4, 2 * args.decode_reps)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * len(steps))
    gbs = DECODE_BYTES * run["N"] * run["H"] / (ms * 1e-3) / 1e9
    return {"steps_timed": reps * len(steps), "ms_per_step": round(ms, 4),
            "tokens_per_s": round(run["N"] / (ms * 1e-3), 1), "alg_GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "replay_equals_eager": same}


def _decode_traffic(step_ms: float):
    """Bytes the decode kernel moved between L2 and the memory fabric per step
    (FETCH_SIZE and WRITE_SIZE, scaled as in the prefill record) from
    profiles/traffic_decode_256.json, and their rate at the measured step
    time; None when the kernel code changed since the counters were taken.
    The counters cannot tell HBM from Infinity Cache hits."""
    rec = _counter_record("traffic_decode_256")
    if rec is None:
        return None
    b = rec["kernels"]["decode_kernel"]["bytes"]
    return {"bytes_per_step": b, "GBps": round(b / (step_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(b / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# Replay fold: a window of 7 draft tokens (the pages' num_speculative_tokens),
# all accepted; per (sequence, head) the fold moves the state once in and out
# plus each token's k, v (bf16), gate logits (fp32) and beta logit.
FOLD_WINDOW = 7
FOLD_TOKEN_BYTES = 2 * 128 + 2 * 128 + 4 * 128 + 4


def bench_fold(args, kda, torch, run, step_ms):
    W = FOLD_WINDOW
    steps = run["steps"][:W]
    win = {key: torch.stack([s[key] for s in steps], dim=1).contiguous() for key in ("k", "v", "z", "b")}
    N, H = run["N"], run["H"]
    n_acc = torch.full((N,), W, dtype=torch.int32, device=win["k"].device)
    # the state sets of the decode headline, one per call in turn
    sts = [run["state"].clone() for _ in range(DECODE_STATE_SETS)]
    A = run["A"]
    for i in range(2):
        kda.kda_recurrent_fold(win["k"], win["v"], win["z"], win["b"], A, n_acc, sts[i % len(sts)])
    torch.cuda.synchronize()
    times = []
    for i in range(max(4, args.decode_reps * 4)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        kda.kda_recurrent_fold(win["k"], win["v"], win["z"], win["b"], A, n_acc, sts[i % len(sts)])
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    mean = sum(ms) / len(ms)
    per_unit = 2 * 128 * 128 * 4 + W * FOLD_TOKEN_BYTES
    gbs = per_unit * N * H / (mean * 1e-3) / 1e9
    # the verify pass over the same window: outputs of every draft token from
    # the checkpoint (read once, not written)
    qw = torch.stack([s["q"] for s in steps], dim=1).contiguous()
    for i in range(2):
        kda.kda_recurrent_verify(qw, win["k"], win["v"], win["z"], win["b"], A, sts[i % len(sts)])
    torch.cuda.synchronize()
    vt = []
    for i in range(max(4, args.decode_reps * 4)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        kda.kda_recurrent_verify(qw, win["k"], win["v"], win["z"], win["b"], A, sts[i % len(sts)])
        b.record()
        vt.append((a, b))
    torch.cuda.synchronize()
    vms = sum(a.elapsed_time(b) for a, b in vt) / len(vt)
    v_unit = 128 * 128 * 4 + W * (FOLD_TOKEN_BYTES + 2 * 128 + 2 * 128)   # state read + window in (+q) + o out
    return {
        "workload": f"decode_256 states ({DECODE_STATE_SETS} sets, one per call in turn), window of "
                    f"{W} draft tokens per sequence, all accepted",
        "calls_timed": len(ms),
        "ms_per_call_mean": round(mean, 4),
        "tokens_per_s": round(N * W / (mean * 1e-3), 1),
        "alg_GBps": round(gbs, 1),
        "vs_token_steps": round(W * step_ms / mean, 2),
        "verify": {
            "ms_per_call_mean": round(vms, 4),
            "tokens_per_s": round(N * W / (vms * 1e-3), 1),
            "alg_GBps": round(v_unit * N * H / (vms * 1e-3) / 1e9, 1),
            "vs_token_steps": round(W * step_ms / vms, 2),
        },
    }


def bench_layer(args, kda, torch, KI, call_ms, step_ms):
    """The layer entry points (short convolution, Swish and L2Norm before the
    core, gated RMSNorm after) on the long_1m and decode_256 shapes, against
    the core-only calls measured above."""
    dev = torch.device("cuda:0")
    case = KI.CONFIGS["long_1m"]
    d = KI.make_layer(case, device=dev, seed=0)
    B, T, H, dk, N, C = d["B"], d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    ws = torch.empty(kda.kda_layer_fwd_workspace_bytes(B, T, H, dk, N, C, torch.bfloat16),
                     dtype=torch.uint8, device=dev)

    def run():
        return kda.kda_layer_fwd(d["q_in"], d["k_in"], d["v_in"], d["conv_w"], d["z"], d["b"],
                                 d["A"], d["gate"], d["norm_w"], initial_state=d["h0"],
                                 conv_state=d["conv_state0"], chunk_size=C, workspace=ws)
    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(2, args.steps // 2)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in times) / len(times)
    del d, ws
    torch.cuda.empty_cache()
    # fused decode launch on the decode workload's shapes
    dc = KI.CONFIGS["decode_256"]
    lc = KI.PrefillCase("decode_layer", H=dc.H, dk=dc.dk, dv=dc.dv, chunk=64, dtype=dc.dtype,
                        B=dc.N, zero_h0=False)
    x = KI.make_layer(lc, device=dev, seed=0, T=1)
    tok = {k: x[k][:, 0].contiguous() for k in ("q_in", "k_in", "v_in", "gate", "z", "b")}
    # the core decode's rotation: DECODE_STATE_SETS sets of states stepped in
    # turn, so that no step finds its state in the Infinity Cache
    sts = [x["h0"].clone() for _ in range(DECODE_STATE_SETS)]
    css = [x["conv_state0"].clone() for _ in range(DECODE_STATE_SETS)]

    def step(i):
        u = i % DECODE_STATE_SETS
        return kda.kda_layer_step(tok["q_in"], tok["k_in"], tok["v_in"], x["conv_w"], css[u], tok["z"],
                                  tok["b"], x["A"], sts[u], tok["gate"], x["norm_w"])
    for i in range(2 * DECODE_STATE_SETS):
        step(i)
    torch.cuda.synchronize()
    stimes = []
    for i in range(16 * args.decode_reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step(i)
        b.record()
        stimes.append((a, b))
    torch.cuda.synchronize()
    sms = sum(a.elapsed_time(b) for a, b in stimes) / len(stimes)
    return {
        "workload": "long_1m and decode_256 shapes with projections, convolution taps, "
                    "carried convolution states, output-gate logits and RMSNorm weight; "
                    f"decode steps {DECODE_STATE_SETS} sets of states in turn",
        "prefill_ms_per_call": round(ms, 4),
        "prefill_tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "prefill_vs_core_call": round(ms / call_ms, 3),
        "decode_ms_per_step": round(sms, 4),
        "decode_tokens_per_s": round(dc.N / (sms * 1e-3), 1),
        "decode_vs_core_step": round(sms / step_ms, 3),
    }


def _stage_ms(h, evs):
    keys = {"prep": (0, 1), "intra": (1, 2), "transition": (2, 4), "compose": (4, 5),
            "output": (5, 3), "call": (0, 3)}
    return {k: sum(_elapsed(h, e[a], e[b]) for e in evs) / len(evs) for k, (a, b) in keys.items()}


def bench_short_prefill(args, kda, torch, KI):
    """The 4,096-token prefill (B=1, H=16, d=128, chunk 64): a latency-shaped
    call of five launches, timed eagerly and as a replay of one captured HIP
    graph (the serving form for short prompts); the replay's outputs are
    compared bit for bit with the eager call's."""
    dev = torch.device("cuda:0")
    d = KI.make_prefill(KI.CONFIGS["prefill_4k"], device=dev, seed=0)
    B, T, H, dk, dv, N, C = d["B"], d["T"], d["H"], d["dk"], d["dv"], d["N"], d["chunk"]
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, C, torch.bfloat16),
                     dtype=torch.uint8, device=dev)

    def call():
        return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                                 initial_state=d["h0"], chunk_size=C, workspace=ws)

    def timed(fn, reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    o_ref, h_ref = call()
    torch.cuda.synchronize()
    reps = max(20, 4 * args.steps)
    eager = timed(call, reps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, h_g = call()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(o_g, o_ref) and torch.equal(h_g, h_ref))
    graph = timed(g.replay, reps)
    # the stages of the same call, from events the library records between
    # its launches (the events themselves add a little to the call)
    L = kda.lib()
    h = _hip()
    evs = [[_event(h) for _ in range(6)] for _ in range(reps)]
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    h0 = d["h0"].data_ptr() if d["h0"] is not None else None
    for row in evs:
        arr = (ctypes.c_void_p * 6)(*[e.value for e in row])
        rc = L.kda_chunk_fwd_timed(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                   d["z"].data_ptr(), d["b"].data_ptr(), d["A"].data_ptr(), h0, None,
                                   B, T, H, dk, dv, N, C, 1, o.data_ptr(), hT.data_ptr(),
                                   ws.data_ptr(), ws.numel(), arr, 6, stream)
        if rc != 0:
            raise RuntimeError(L.kda_status_string(rc).decode())
    torch.cuda.synchronize()
    stages = _stage_ms(h, evs)
    for row in evs:
        for e in row:
            h.hipEventDestroy(e)
    tok = B * T
    return {"workload": "prefill_4k: B=1, H=16, T=4096, d_k=d_v=128, chunk=64, bf16, seed 0",
            "ms_per_call_eager": round(eager, 4), "tokens_per_s_eager": round(tok / (eager * 1e-3), 1),
            "ms_per_call_graph": round(graph, 4), "tokens_per_s_graph": round(tok / (graph * 1e-3), 1),
            "replay_equals_eager": same,
            "stages_ms_with_events": {k: round(v, 4) for k, v in stages.items()}}


def bench_family(args, kda, torch, KI, kda_stages):
    """The other rows of the family table (GLA with the erase step off,
    DeltaNet with alpha = 1) and the general DPLR update with the low-rank pair
    untied from k, on the long_1m shapes.  The DPLR line is the measurement
    behind the 2-vs-4 chunk-matrix comparison: KDA forms A_kk and A_qk per
    chunk, the general form A_ba, A_bk, A_qa and A_qk."""
    dev = torch.device("cuda:0")
    case = KI.CONFIGS["long_1m"]
    reps = max(2, args.steps // 2)
    out = {"workload": "long_1m shapes (B=1, H=12, T=1048576, d=128, C=64, bf16, seed 0)"}
    d = KI.make_prefill(case, device=dev, seed=0)
    B, T, H, dk, dv, N, C = d["B"], d["T"], d["H"], d["dk"], d["dv"], d["N"], d["chunk"]
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, C, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    modes = {}
    for mode in ("gla", "deltanet"):
        g, A = (None, None) if mode == "deltanet" else (d["z"], d["A"])

        def run():
            return kda.kda_chunk_fwd_mode(d["q"], d["k"], d["v"], g, d["b"], A, mode,
                                          initial_state=d["h0"], chunk_size=C, workspace=ws)
        run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ts) / len(ts)
        modes[mode] = {"ms_per_call": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1)}
    out["modes"] = modes
    del d, ws
    torch.cuda.empty_cache()

    d = KI.make_dplr(case, device=dev, seed=0)
    L = kda.lib()
    wsb = kda.kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, C, torch.bfloat16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    h = _hip()
    evs = [[_event(h) for _ in range(6)] for _ in range(reps + 1)]
    ptrs = (d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["la"].data_ptr(),
            d["lb"].data_ptr(), d["z"].data_ptr(), d["A"].data_ptr(), d["h0"].data_ptr(), None,
            B, T, H, dk, dv, N, C, 1, o.data_ptr(), hT.data_ptr(), ws.data_ptr(), wsb)
    for i in range(reps + 1):
        arr = (ctypes.c_void_p * 6)(*[e.value for e in evs[i]])
        rc = L.kda_dplr_chunk_fwd_timed(*ptrs, arr, 6, stream)
        if rc != 0:
            raise RuntimeError(L.kda_status_string(rc).decode())
    torch.cuda.synchronize()
    st = _stage_ms(h, evs[1:])
    for row in evs:
        for e in row:
            h.hipEventDestroy(e)
    units = B * T * H
    intra_gbs = DPLR_INTRA_BYTES * units / (st["intra"] * 1e-3) / 1e9
    out["dplr"] = {
        "call_ms_events": round(st["call"], 4),
        "tokens_per_s": round(B * T / (st["call"] * 1e-3), 1),
        "kernels_ms": {k: round(v, 4) for k, v in st.items() if k != "call"},
        "intra_alg_GBps": round(intra_gbs, 1),
        "intra_hbm_frac": round(intra_gbs / HBM_PEAK_GBS, 4),
        "path_alg_GBps": round(DPLR_BYTES * units / (st["call"] * 1e-3) / 1e9, 1),
    }
    out["study_2_vs_4"] = {
        "chunk_matrices": {"kda": 2, "dplr": 4},
        "intra_ms": {"kda": round(kda_stages["intra"], 4), "dplr": round(st["intra"], 4)},
        "call_ms": {"kda": round(kda_stages["call"], 4), "dplr": round(st["call"], 4)},
        "intra_time_ratio": round(st["intra"] / kda_stages["intra"], 3),
        "call_time_ratio": round(st["call"] / kda_stages["call"], 3),
        "input_bytes_per_token_head": {"kda": INTRA_BYTES, "dplr": DPLR_INTRA_BYTES},
        "record_bytes_per_chunk_head": {"kda": KDA_RECORD_BYTES, "dplr": DPLR_RECORD_BYTES},
    }
    print(f"[bench] family: modes {modes}; dplr call {st['call']:.3f} ms, intra {st['intra']:.3f} ms "
          f"(KDA {kda_stages['intra']:.3f})", flush=True)
    del d, ws, o, hT
    torch.cuda.empty_cache()
    return out


def _cpu_unit(job):
    """One work unit of the CPU baseline, run in a worker process: the oracle
    on a slice of a workload.  `job` = (kind, arrays); prefill slices are one
    head of one sequence, decode slices a block of sequences over all steps."""
    import numpy as np   # noqa: F401  (the oracle's own dependency)
    import oracle
    from threadpoolctl import threadpool_limits
    kind, a = job
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if kind == "prefill":
            oracle.recurrence(a["q"], a["k"], a["v"], a["z"], a["b"], a["A"], a["h0"])
        else:
            S = a["state"]
            for st in a["steps"]:
                _, S = oracle.decode_step(st["q"], st["k"], st["v"], st["z"], st["b"], a["A"], S)
        return time.perf_counter() - t0


def _warm_unit(_):
    import oracle  # noqa: F401
    return os.getpid()


def _under_profiler() -> bool:
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def cpu_baselines(args):
    """The fp64 oracle timed on the host's cores, before anything touches the
    GPU: a process pool (spawned workers, one BLAS thread each) over the
    independent (sequence, head) recurrences of three samples drawn on the
    host with the workloads' recipe (seed 0): the 1M-token workload's first
    `cpu_tokens` tokens (all 12 heads), the 4,096-token workload in full (16
    heads) and the decode workload's 16 steps (256 x 12 states, in blocks of
    16 sequences).  Returns (prefill baseline, {"prefill_4k": ..., "decode": ...})."""
    import multiprocessing as mp
    import torch
    import kda_inputs as KI
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    host = len(os.sched_getaffinity(0))
    # at most 16 workers: the host share of one GPU on the boxes this runs on
    procs = max(1, min(host, 16))

    def f32(x):
        return x.float().numpy()

    def prefill_jobs(case, T):
        d = KI.make_prefill(case, T=T, seed=0)
        return [("prefill", {"q": f32(d["q"][0, :, [h]]), "k": f32(d["k"][0, :, [h]]),
                             "v": f32(d["v"][0, :, [h]]), "z": f32(d["z"][0, :, [h]]),
                             "b": f32(d["b"][0, :, [h]]), "A": f32(d["A"][[h]]),
                             "h0": None if d["h0"] is None else f32(d["h0"][0, [h]])})
                for h in range(d["H"])]

    long_jobs = prefill_jobs(KI.CONFIGS["long_1m"], args.cpu_tokens)
    short_jobs = prefill_jobs(KI.CONFIGS["prefill_4k"], None)
    run = KI.make_decode(KI.CONFIGS["decode_256"], seed=0)
    blk = 16
    dec_jobs = []
    for n0 in range(0, run["N"], blk):
        sl = slice(n0, n0 + blk)
        dec_jobs.append(("decode", {"A": f32(run["A"]), "state": f32(run["state"][sl]),
                                    "steps": [{k: f32(st[k][sl]) for k in ("q", "k", "v", "z", "b")}
                                              for st in run["steps"]]}))
    out = {}
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs) as pool:
        pool.map(_warm_unit, range(procs))
        for name, jobs in (("long", long_jobs), ("short", short_jobs), ("decode", dec_jobs)):
            t0 = time.perf_counter()
            busy = sum(pool.map(_cpu_unit, jobs, chunksize=1))
            out[name] = (time.perf_counter() - t0, busy, min(procs, len(jobs)))
    wall, busy, used = out["long"]
    T = args.cpu_tokens
    full = KI.CONFIGS["long_1m"].T
    prefill = {"value": round(T / wall, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": f"first {T} tokens of the 1M-token recipe (drawn on the host, seed 0), "
                         f"all 12 heads: fp64 numpy token recurrence, {used} worker processes "
                         f"(one head each, one BLAS thread each; {host} host CPUs visible), "
                         f"{wall:.1f} s wall, {busy:.1f} s of worker time; the recurrence is "
                         f"linear in T, so 2^20 tokens would take about {wall * full / T:.0f} s "
                         f"(extrapolated, not run)",
               "blas_threads": 1, "host_cpus": host}
    sw, sb, su = out["short"]
    dw, db, du = out["decode"]
    dc = KI.CONFIGS["decode_256"]
    extra = {
        "prefill_4k": {"value": round(4096 / sw, 1), "unit": "tokens/s", "cores": su,
                       "kind": "oracle", "wall_s": round(sw, 2),
                       "sample": "the 4,096-token workload in full (16 heads, drawn on the "
                                 "host), one head per worker"},
        "decode": {"value": round(dc.N * dc.steps / dw, 1), "unit": "tokens/s", "cores": du,
                   "kind": "oracle", "wall_s": round(dw, 2),
                   "sample": f"all {dc.steps} steps of the decode workload (256 x 12 states, "
                             f"drawn on the host), blocks of {blk} sequences per worker"},
    }
    print(f"[bench] CPU oracle on {used} workers: long_1m prefix {T} tokens in {wall:.1f} s; "
          f"prefill_4k {sw:.1f} s; decode {dw:.1f} s", flush=True)
    del torch
    return prefill, extra


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-reps", type=int, default=4, help="passes over the 16 decode steps")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the 1M-token recipe the CPU oracle baseline runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer entry points (convolution and gated RMSNorm around the core)")
    ap.add_argument("--no-family", action="store_true",
                    help="skip the family modes and the general DPLR update")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="copy a buffer of this many MiB once before timing (a known-size "
                         "kernel for calibrating the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads shard across GPUs with no communication, one call per GPU). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    # the CPU baselines spawn their worker processes before anything here
    # touches the GPU (and never under a profiler, whose preloaded library
    # may initialise it in every process)
    cpu, cpu_extra = None, {}
    if not args.no_cpu_baseline:
        if _under_profiler():
            print("[bench] under a profiler: CPU baseline skipped", flush=True)
        else:
            cpu, cpu_extra = cpu_baselines(args)

    import torch
    import gated_delta_rule_77_amd as kda
    import kda_inputs as KI
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kda.lib()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + written", flush=True)
        del src, dst

    value, ms, roof, extra = bench_prefill(args, kda, torch, KI)
    if cpu_extra:
        extra["cpu_baseline_prefill_4k"] = cpu_extra["prefill_4k"]
    dec = None if args.no_decode else bench_decode(args, kda, torch, KI, cpu_extra.get("decode"))
    if dec:
        w = dec["cache_warm"]
        print(f"[bench] decode, {DECODE_STATE_SETS} state sets in turn: "
              f"{dec['ms_per_step_mean']:.4f} ms/step eager, "
              f"{dec['graph']['ms_per_step']:.4f} ms/step graph-replayed "
              f"({dec['hbm_frac']:.3f} / {dec['graph']['hbm_frac']:.3f} of HBM peak; replay equals "
              f"eager: {dec['graph']['replay_equals_eager']}); one state, cache-warm: "
              f"{w['ms_per_step_mean']:.4f} eager, {w['graph']['ms_per_step']:.4f} replayed",
              flush=True)
    layer = None
    if not args.no_layer:
        layer = bench_layer(args, kda, torch, KI, extra["call_ms_events"],
                            dec["ms_per_step_mean"] if dec else float("nan"))
    family = None
    if not args.no_family:
        family = bench_family(args, kda, torch, KI, {"intra": extra["kernels_ms"]["intra"],
                                                     "call": extra["call_ms_events"]})
    short = bench_short_prefill(args, kda, torch, KI)
    print(f"[bench] prefill_4k: {short['ms_per_call_eager']:.4f} ms/call eager, "
          f"{short['ms_per_call_graph']:.4f} ms/call graph-replayed "
          f"(replay equals eager: {short['replay_equals_eager']}); stages with events (ms): "
          + ", ".join(f"{k} {v:.4f}" for k, v in short["stages_ms_with_events"].items()), flush=True)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long_1m: B=1, H=12, T=1048576, d_k=d_v=128, chunk=64, bf16 "
                               "q/k/v, fp32 logits and state, seed 0",
                   "B": 1, "T": 1 << 20, "H": 12, "dk": 128, "dv": 128, "chunk": 64},
        "roofline": roof, "cpu_baseline": cpu, "prefill": extra, "decode": dec, "layer": layer,
        "family": family, "prefill_4k": short,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
