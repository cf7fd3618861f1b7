#!/usr/bin/env python3
"""Benchmark: one fused AdamW-SR step over the Llama-3-8B-shaped parameter
list (291 tensors, 8,030,261,248 bf16 params, bf16 grads, f32 m/v) on one
MI355X, through the C ABI.

Prints one JSON line: params updated per second (whole step, inputs resident
in HBM), the dominant kernel's achieved HBM bandwidth against the 8 TB/s
peak (algorithmic bytes: 22 per element), and the CPU oracle timed on a
bounded sample of the same workload on the host's cores.

    python bench.py [--steps K] [--warmup W]
                    [--workload llama3_8b|llama3_8b_rank|shards|convert|gemm|rng|hbm_probe|
                                bf16_64k|f32_16m]
    python bench.py --copy-probe      # plain copy of known size (counter scaling)

The llama3_8b_rank workload is one data-parallel rank's share of the same
list: the flattened list split into --ranks equal contiguous ranges
(ZeRO-1), rank --rank's pieces (default 3 of 8: 42 pieces, cut at both
ends), each with its global base_index.

The hbm_probe workload measures what HBM gives the step's launch structure
without the step's arithmetic: read-only, write-only and copy streams, and
the Llama-3-8B list's own 4-read/3-write traffic timed against the step.

The bf16_64k and f32_16m workloads step one small tensor: 65,536 bf16
params (cache-resident, launch-bound) and 16,777,216 f32 params (the f32
size-class launch; timed with the Infinity Cache flushed between steps).

The gemm workload times the bf16 GEMM with the SR epilogue on the gate/up
projection of one Llama-3-8B MLP over 8,192 tokens (M=8192, N=14336,
K=4096; --gemm-shape M,N,K overrides), against the 2.5 PFLOP/s dense bf16
matrix-core peak, with the same GEMM under RN and torch.matmul (the vendor
library, RN) timed beside it for context.
"""

import argparse
import hashlib
import json
import multiprocessing
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params updated/sec and achieved HBM GB/s (% of peak), fused AdamW-SR, 1 GPU"
HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "adamw_optimizer_stochastic_amd", "csrc", f)
                  for f in ("adamw_sr.hip", "device.hpp")]
GEMM_SOURCES = [os.path.join(ROOT, "adamw_optimizer_stochastic_amd", "csrc", f)
                for f in ("gemm_sr.hip", "device.hpp")]
RNG_SOURCES = [os.path.join(ROOT, "adamw_optimizer_stochastic_amd", "csrc", f)
               for f in ("random.hip", "device.hpp")]


def source_hash_of(files):
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so editing a comment keeps counter data valid and any code change voids it."""
    h = hashlib.sha256()
    for f in files:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def source_hash():
    """Hash of the AdamW step's kernel sources (see source_hash_of)."""
    return source_hash_of(KERNEL_SOURCES)


def gemm_source_hash():
    """Hash of the GEMM's kernel sources (see source_hash_of)."""
    return source_hash_of(GEMM_SOURCES)


def rng_source_hash():
    """Hash of the random fills' and dropout's kernel sources (see source_hash_of)."""
    return source_hash_of(RNG_SOURCES)


# ----------------------------------------------------------- CPU baseline
def _oracle_shard(args):
    import numpy as np
    import oracle
    from adamw_optimizer_stochastic_amd import workloads as wl
    shard, n = args
    rng = wl.host_rng(wl.CFG_LLAMA, 1000 + shard, 0)
    p = wl.f32_to_bf16_bits(wl.normal_f32(rng, n, 0.02))
    g = wl.f32_to_bf16_bits(wl.normal_f32(rng, n, 1e-3))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    t0 = time.perf_counter()
    oracle.step_tensor(p, g, m, v, param_dtype=oracle.BF16, grad_dtype=oracle.BF16,
                       base_index=shard * n, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                       weight_decay=0.01, step=2, seed=0)
    return time.perf_counter() - t0


# Worker processes for the CPU baseline: the CPUs this process may run on,
# at most 16 -- the host share of one GPU on the MI355X machines this runs
# on, whatever larger count the host reports.
HOST_SHARE_CPUS = 16


def host_cpus():
    """(cpus this process may run on, cpus the host reports)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return usable, os.cpu_count() or usable


def cpu_baseline(per_core=1 << 22):
    """The oracle (numpy, unmodified) on `cores` shards of `per_core` bf16
    elements each, one process per core, before the GPU is touched (the pool
    forks a process that has not initialised the GPU). Each shard times its
    own step (input generation excluded); the shards run concurrently, so
    the whole-host rate is the sum of the per-core rates."""
    usable, reported = host_cpus()
    cores = max(1, min(HOST_SHARE_CPUS, usable))
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        times = pool.map(_oracle_shard, [(k, per_core) for k in range(cores)])
    wall = time.perf_counter() - t0
    rates = sorted(per_core / t for t in times)
    n = cores * per_core
    return {"value": sum(rates), "unit": "params/s", "cores": cores, "kind": "oracle",
            "host_cpu_count": reported, "usable_cpus": usable,
            "cores_note": f"one process per core on {cores} cores: the host share of one GPU "
                          f"(at most {HOST_SHARE_CPUS}); the host reports {reported} CPUs, "
                          f"{usable} usable by this process",
            "one_core_value": rates[len(rates) // 2],
            "sample": f"{n} bf16 params ({cores} concurrent shards of {per_core}) of the same "
                      f"workload, one AdamW-SR step each, numpy oracle; step times "
                      f"{min(times):.2f}-{max(times):.2f} s ({sum(times):.1f} CPU-s), "
                      f"wall with input generation {wall:.1f} s"}


# ------------------------------------------------------------- GPU legs
def traffic_from_profile(workload, n_elems):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILE_DIR, f"adamw_sr_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != source_hash() or d.get("n_elems") != n_elems:
        return None
    return d.get("hbm_bytes_per_launch")


def stream_traffic_from_profile(name, source_hash_now, n_elems):
    """HBM bytes per launch of a single-kernel streaming workload (the
    conversion, dropout) from its committed counter summary, if it was taken
    on the current kernel sources at this size (else None)."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != source_hash_now or d.get("n_elems") != n_elems:
        return None
    return d.get("hbm_bytes_per_launch")


def gemm_traffic_from_profile(m, n, k):
    """HBM-side bytes per SR GEMM launch from the committed counter summary
    for this shape, if it was taken on the current GEMM sources (else None)."""
    path = os.path.join(PROFILE_DIR, f"gemm_bf16_sr_{m}x{n}x{k}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != gemm_source_hash() or d.get("shape") != [m, n, k]:
        return None
    return d.get("hbm_bytes_per_launch")


# A list of at most this many tensors travels in the kernel arguments (the
# library's inline launches); a longer one is uploaded first.
INLINE_TENSORS = 48
KERNEL_UPLOADED = ("upload_words (the descriptors) + adamw_sr_class<BF16,BF16,SR> (one launch per "
                   "size class) + adamw_sr_slots<BF16,BF16,SR> (the other tensors)")
KERNEL_INLINE = ("adamw_sr_inline<BF16,BF16,SR> (descriptors in the kernel arguments; one launch "
                 "per size class and one for the other pieces)")


def run_adamw(args, torch, ops, wl):
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    extra = {}
    if args.workload == "llama3_8b":
        state = wl.llama3_8b_state(dev, seed=0, states=args.state_layout)
        cfg_name = "llama3_8b_param_list"
    elif args.workload == "llama3_8b_rank":
        state = wl.llama3_8b_rank_state(dev, args.rank, args.ranks, seed=0,
                                        states=args.state_layout)
        cfg_name = f"llama3_8b_rank{args.rank}_of_{args.ranks}"
        extra = {"rank": args.rank, "ranks": args.ranks,
                 "first_piece": [state[0]["name"], state[0]["offset"]],
                 "last_piece": [state[-1]["name"], state[-1]["offset"],
                                state[-1]["param"].numel()]}
    else:  # shards: one 268,435,456-element tensor
        n = 268435456
        gen = wl.device_generator(dev, wl.CFG_SHARDS, 0)
        state = [dict(name="w", param=wl.device_normal(n, 0.02, gen, dev, torch.bfloat16),
                      grad=wl.device_normal(n, 1e-3, gen, dev, torch.bfloat16),
                      exp_avg=torch.zeros(n, dtype=torch.float32, device=dev),
                      exp_avg_sq=torch.zeros(n, dtype=torch.float32, device=dev),
                      base_index=0)]
        cfg_name = "single_tensor_268M"
        if args.odd_split:
            # two pieces cut at an odd element: the second piece's buffers all
            # start 1 element past a 16-byte boundary (shifted runs)
            state = odd_split(state[0], SHARDS_ODD_CUT)
            cfg_name = "single_tensor_268M_odd_split"
            extra = {"pieces": [[0, SHARDS_ODD_CUT], [SHARDS_ODD_CUT, n]]}
    n_elems = sum(t["param"].numel() for t in state)
    lists = ([t["param"] for t in state], [t["grad"] for t in state],
             [t["exp_avg"] for t in state], [t["exp_avg_sq"] for t in state],
             [t["base_index"] for t in state])
    ws = ops.make_workspace([t["param"].numel() for t in state], dev)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, seed=0,
              rounding="sr", workspace=ws)
    torch.cuda.synchronize()
    step = 0
    for _ in range(args.warmup):
        step += 1
        ops.adamw_step(*lists, step=step, **hp)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step += 1
        events[k][0].record(stream)
        ops.adamw_step(*lists, step=step, **hp)
        events[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in events]
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = sum(launch_ms) / len(launch_ms)
    kernel_ms_median = sorted(launch_ms)[len(launch_ms) // 2]
    bytes_per_launch = 22 * n_elems
    achieved = bytes_per_launch / (kernel_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(args.workload, n_elems)
    # The same list's traffic without the arithmetic (after the timed steps:
    # it overwrites the parameters), timed like the step.
    probe_ms = adamw_stream_probe_ms(torch, state, ws, stream, args.steps)
    probe_gbps = bytes_per_launch / (probe_ms * 1e-3) / 1e9
    copy_gbps = stream_copy_gbps(torch, dev, stream)
    context = {}
    if args.workload == "shards":
        context = whole_vs_odd_split(torch, ops, state, ws, stream, args.steps)
    return {
        "context": context,
        "metric": METRIC, "value": n_elems / (ms_per_step * 1e-3), "unit": "params/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg_name, "n_tensors": len(state), "params": n_elems,
                   "param_dtype": "bf16", "grad_dtype": "bf16", "state_dtype": "f32",
                   "rounding": "sr", "algorithmic_bytes_per_param": 22,
                   "state_layout": STATE_LAYOUT_NOTE[args.state_layout]
                   if args.workload != "shards" else "one tensor",
                   "parallelism": "single GPU", **extra},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": KERNEL_UPLOADED if len(state) > INLINE_TENSORS else KERNEL_INLINE,
                     "kernel_ms_avg": kernel_ms, "kernel_ms_median": kernel_ms_median,
                     "timing": "HIP events on the launch stream around each step call: all "
                               "kernels of one step",
                     "copy_GBps": copy_gbps, "frac_of_copy": achieved / copy_gbps,
                     "copy_note": "asr_stream_copy, 2 x 8 GiB, a 1:1 copy built like the step "
                                  "(same slots, 128-bit accesses, XCD windows, residency cap)",
                     "probe_GBps": probe_gbps, "frac_of_probe": achieved / probe_gbps,
                     "probe_note": "asr_adamw_stream_probe on the same list: the step's launch "
                                   "plan and accesses (4 streams read, 3 written) without its "
                                   "arithmetic, same timing"},
    }


def run_convert(args, torch, ops, wl):
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n = 1 << 30
    gen = wl.device_generator(dev, wl.CFG_CONVERT, 0)
    x = wl.device_normal(n, 1.0, gen, dev, torch.float32)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        ops.cvt_f32_bf16_sr(x, 7, 0, 0, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        events[k][0].record(stream)
        ops.cvt_f32_bf16_sr(x, 7, 0, 0, out=out)
        events[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(a.elapsed_time(b) for a, b in events) / args.steps
    achieved = 6 * n / (kernel_ms * 1e-3) / 1e9
    return {"metric": "elements converted/sec, cvt_f32_bf16_sr", "value": n / (wall / args.steps),
            "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": "cvt_f32_bf16_sr_2^30"},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": stream_traffic_from_profile(
                             "cvt_f32_bf16_sr_2pow30_hbm_counters.json", source_hash(), n),
                         "algorithmic_bytes": 6 * n, "kernel_ms_avg": kernel_ms}}


MALL_FLUSH_BYTES = 1 << 30   # > the 256 MB Infinity Cache


def run_small(args, torch, ops, wl):
    """One tensor far below the headline's size, stepped back to back:
    bf16_64k = 65,536 bf16 params and grads (cache-resident, bound by the
    launch), f32_16m = 16,777,216 f32 params and grads (28 B per element,
    469.8 MB per step, the f32 size-class launch). The f32 tensor's 256 MiB
    of params, grads and states fit the 256 MB Infinity Cache, so it is also
    timed with a 1 GiB read on the stream between steps (outside the
    events), which leaves the step to DRAM; that is the roofline figure."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.workload == "bf16_64k":
        n, dt, cfg, std_g, bpe = 65536, torch.bfloat16, wl.CFG_SMALL, 1e-3, 22
    else:
        n, dt, cfg, std_g, bpe = 16777216, torch.float32, wl.CFG_F32, 1e-2, 28
    gen = wl.device_generator(dev, cfg, 0)
    p = wl.device_normal(n, 0.02, gen, dev, dt)
    g = wl.device_normal(n, std_g, gen, dev, dt)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = ops.make_workspace([n], dev)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, seed=0,
              rounding="sr", workspace=ws)
    step = [0]

    def fn():
        step[0] += 1
        ops.adamw_step([p], [g], [m], [v], [0], step=step[0], **hp)

    steps = max(args.steps, 100) if n <= 65536 else args.steps
    for _ in range(max(args.warmup, 5)):
        fn()
    wall_s, ev_ms = _time_launches(torch, stream, fn, steps)
    res_ctx = {"back_to_back_kernel_ms": ev_ms, "back_to_back_wall_ms": wall_s * 1e3}
    kernel_ms, note = ev_ms, ("back-to-back steps: the tensor's 1.4 MB stay in the caches, "
                              "so the time is launch and latency, not HBM")
    if n > 65536:
        # the flush reads (a write would leave dirty lines that the step
        # then writes back)
        scratch = torch.zeros(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
        for k in range(steps):
            scratch.sum()
            events[k][0].record(stream)
            fn()
            events[k][1].record(stream)
        torch.cuda.synchronize()
        kernel_ms = sum(a.elapsed_time(b) for a, b in events) / steps
        res_ctx["back_to_back_GBps"] = bpe * n / (ev_ms * 1e-3) / 1e9
        note = ("each step after a 1 GiB read on the stream (outside the events), so its "
                "inputs come from DRAM; back-to-back steps partly hit the Infinity Cache")
        del scratch
    achieved = bpe * n / (kernel_ms * 1e-3) / 1e9
    name = "bf16 params and grads" if dt == torch.bfloat16 else "f32 params and grads"
    return {"metric": METRIC, "value": n / (kernel_ms * 1e-3), "unit": "params/s", "n_gpus": 1,
            "steps": steps, "warmup": max(args.warmup, 5), "ms_per_step": wall_s * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"single_tensor_{n}", "params": n,
                       "param_dtype": "bf16" if dt == torch.bfloat16 else "f32",
                       "grad_dtype": "bf16" if dt == torch.bfloat16 else "f32",
                       "state_dtype": "f32", "rounding": "sr" if dt == torch.bfloat16 else "none",
                       "algorithmic_bytes_per_param": bpe},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "adamw_sr_inline (one launch, the descriptor in the "
                                   "kernel arguments; " + name + ")",
                         "kernel_ms_avg": kernel_ms, "timing_note": note},
            "context": res_ctx}


GEMM_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def stream_copy_gbps(torch, dev, stream, nbytes=8 << 30, reps=10):
    """Bandwidth of the library's copy kernel (read + write bytes / time)."""
    from adamw_optimizer_stochastic_amd import _abi
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        _abi.asr_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream.cuda_stream)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        _abi.asr_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream.cuda_stream)
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


STATE_LAYOUT_NOTE = {
    "flat": "flat: f32 m and v of all tensors in two buffers, allocated after params and "
            "grads (AdamWSR's layout)",
    "separate": "separate: one f32 m and one f32 v allocation per tensor, after params and "
                "grads (zeros_like per parameter)"}
SHARDS_ODD_CUT = 33554433


def odd_split(t, cut):
    """Two pieces [0, cut) and [cut, n) of one tensor's state, each with its
    global base_index."""
    n = t["param"].numel()
    return [dict(name=f"{t['name']}[{a}:{b}]", param=t["param"][a:b], grad=t["grad"][a:b],
                 exp_avg=t["exp_avg"][a:b], exp_avg_sq=t["exp_avg_sq"][a:b],
                 base_index=t["base_index"] + a) for a, b in ((0, cut), (cut, n))]


def whole_vs_odd_split(torch, ops, state, ws, stream, steps):
    """The 268M-element tensor stepped whole and as two pieces cut at an odd
    element, in three alternating blocks of `steps` calls each (HIP events
    per call): the cost of a misaligned cut."""
    pieces = state if len(state) == 2 else odd_split(state[0], SHARDS_ODD_CUT)
    base = pieces[0]
    # the two pieces are views of one storage: rebuild the whole views from it
    n = sum(p["param"].numel() for p in pieces)
    whole = [dict(name="w", base_index=base["base_index"],
                  **{k: base[k].as_strided((n,), (1,)) for k in
                     ("param", "grad", "exp_avg", "exp_avg_sq")})]
    # one workspace that serves both forms (the two pieces need the larger)
    ws = ops.make_workspace([p["param"].numel() for p in pieces], pieces[0]["param"].device)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, seed=0,
              rounding="sr", workspace=ws)
    forms = {}
    for name, st in (("whole", whole), ("odd_split", pieces)):
        lists = ([t["param"] for t in st], [t["grad"] for t in st], [t["exp_avg"] for t in st],
                 [t["exp_avg_sq"] for t in st], [t["base_index"] for t in st])
        forms[name] = lists
    ms = {"whole": [], "odd_split": []}
    step = [1000]
    for _ in range(3):
        for name, lists in forms.items():
            def fn(lists=lists):
                step[0] += 1
                ops.adamw_step(*lists, step=step[0], **hp)
            fn()
            ms[name].append(_time_launches(torch, stream, fn, steps)[1])
    w, o = sum(ms["whole"]) / 3, sum(ms["odd_split"]) / 3
    n_bytes = 22 * n
    return {"whole_ms": w, "odd_split_ms": o, "whole_GBps": n_bytes / (w * 1e-3) / 1e9,
            "odd_split_GBps": n_bytes / (o * 1e-3) / 1e9, "odd_split_over_whole_rate": w / o,
            "blocks_ms": ms, "cut": SHARDS_ODD_CUT}


def adamw_stream_probe_ms(torch, state, ws, stream, steps):
    """Mean time of asr_adamw_stream_probe over the list (HIP events around
    each call on the launch stream), after 2 untimed calls."""
    from adamw_optimizer_stochastic_amd import _abi
    descs = [_abi.AsrTensor(t["param"].data_ptr(), t["grad"].data_ptr(),
                            t["exp_avg"].data_ptr(), t["exp_avg_sq"].data_ptr(),
                            t["param"].numel(), t["base_index"],
                            _abi.ASR_BF16 if t["param"].dtype == torch.bfloat16 else _abi.ASR_F32,
                            _abi.ASR_BF16 if t["grad"].dtype == torch.bfloat16 else _abi.ASR_F32)
             for t in state]
    nbytes = ws.numel() * ws.element_size()

    def fn():
        _abi.asr_adamw_stream_probe(descs, ws.data_ptr(), nbytes, stream.cuda_stream)

    for _ in range(2):
        fn()
    return _time_launches(torch, stream, fn, steps)[1]


def _time_launches(torch, stream, fn, steps):
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        events[k][0].record(stream)
        fn()
        events[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps, sum(a.elapsed_time(b) for a, b in events) / steps


def gemm_cpu_baseline(m, n, k, rows=4096):
    """The oracle's GEMM (binary64 product, then SR of the f32 result) on
    `rows` rows of the same shape, timed on the host (the product runs on the
    BLAS threads, the rounding on one)."""
    import numpy as np
    import oracle
    from adamw_optimizer_stochastic_amd import workloads as wl
    rows = min(rows, m)
    a, b = wl.gemm_operands_host(rows, n, k, "randn", seed=0)
    t0, c0 = time.perf_counter(), time.process_time()
    c = oracle.gemm_exact(a, b).astype(np.float32)
    oracle.gemm_round(c, "sr", 7, 1, 0)
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": 2.0 * rows * n * k / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of the {m} rows (numpy binary64 matmul, then the SR "
                      f"rounding), {dt:.1f} s wall, {cpu:.1f} CPU-s"}


def run_gemm(args, torch, ops, wl):
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.gemm_shape:
        m, n, k = (int(x) for x in args.gemm_shape.split(","))
        name = f"gemm_{m}x{n}x{k}"
    else:
        m, n, k = (wl.GEMM_LLAMA3_8B_MLP_UP[x] for x in ("m", "n", "k"))
        name = "llama3_8b_mlp_up_proj_8192_tokens"
    a, b = wl.gemm_operands_device(m, n, k, dev, seed=0)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = 2.0 * m * n * k
    step = [0]

    def sr():
        step[0] += 1
        ops.gemm_bf16(a, b, rounding="sr", seed=7, step=step[0], out=c)

    def rn():
        ops.gemm_bf16(a, b, rounding="rn", out=c)

    def lib():
        torch.matmul(a, b.t(), out=c)

    # the unfused alternative: the vendor library's GEMM to f32, then the
    # library's SR conversion of it (the same keying: position m*N + n)
    c32 = torch.empty((m, n), dtype=torch.float32, device=dev)

    def lib_then_sr():
        step[0] += 1
        torch.mm(a, b.t(), out_dtype=torch.float32, out=c32)
        ops.cvt_f32_bf16_sr(c32, 7, step[0], 0, out=c)

    try:
        lib_then_sr()
    except (RuntimeError, TypeError):   # no f32-output GEMM in this torch build
        lib_then_sr = None

    # clocks settle after a fraction of a second of matrix work: warm up on
    # the GEMM itself before any timed loop
    for _ in range(max(100, args.warmup)):
        sr()
    for fn in (sr, rn, lib, lib_then_sr):
        for _ in range(args.warmup if fn else 0):
            fn()
    # SR and RN timed in alternating blocks, so that clock drift during the
    # run does not favour whichever is timed later
    walls, srs, rns, libs, unfused = [], [], [], [], []
    for _ in range(3):
        w, k_ms = _time_launches(torch, stream, sr, args.steps)
        walls.append(w)
        srs.append(k_ms)
        rns.append(_time_launches(torch, stream, rn, args.steps)[1])
        libs.append(_time_launches(torch, stream, lib, args.steps)[1])
        if lib_then_sr:
            unfused.append(_time_launches(torch, stream, lib_then_sr, args.steps)[1])
    wall = sum(walls) / len(walls)
    kernel_ms = sum(srs) / len(srs)
    rn_ms = sum(rns) / len(rns)
    lib_ms = sum(libs) / len(libs)
    unfused_ms = sum(unfused) / len(unfused) if unfused else None
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {
        "metric": "bf16 GEMM with stochastic-rounding epilogue, TFLOP/s, 1 GPU",
        "value": flops / wall / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "timing_note": "3 alternating blocks of `steps` launches each of SR, RN, torch.matmul "
                       "and the unfused SR; value and ms_per_step from the SR blocks",
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "m": m, "n": n, "k": k, "layout": "C = A B^T",
                   "rounding": "sr", "accumulate": "f32"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": GEMM_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / GEMM_PEAK_TFLOPS,
                     "traffic": gemm_traffic_from_profile(m, n, k),
                     "algorithmic_bytes": 2 * (m * k + n * k + m * n),
                     "kernel": "asr_gemm::gemm_bf16<256x256 tile, SR>",
                     "kernel_ms_avg": kernel_ms},
        "context": {"same_kernel_rn_ms": rn_ms,
                    "same_kernel_rn_tflops": flops / (rn_ms * 1e-3) / 1e12,
                    "torch_matmul_rn_ms": lib_ms,
                    "torch_matmul_rn_tflops": flops / (lib_ms * 1e-3) / 1e12,
                    "sr_over_rn": kernel_ms / rn_ms,
                    "unfused_sr_ms": unfused_ms,
                    "unfused_sr_tflops": flops / (unfused_ms * 1e-3) / 1e12 if unfused_ms else None,
                    "unfused_note": "torch.mm to f32 (the vendor library) then asr_cvt_f32_bf16_sr "
                                    "of the f32 product: the same SR keying, without fusion"},
    }


def run_rng(args, torch, ops, wl):
    """Dropout over 2**30 f32 elements with its keep mask (read 4 B, write
    4 + 1 B per element: HBM-bound), with normal and uniform fills of the
    same size timed beside it."""
    from adamw_optimizer_stochastic_amd import random as arng
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n = 1 << 30
    x = torch.empty(n, dtype=torch.float32, device=dev)
    arng.normal_(x, seed=1, step=0)
    y = torch.empty_like(x)
    mask = torch.empty(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    from adamw_optimizer_stochastic_amd import _abi

    def drop():
        _abi.asr_dropout(x.data_ptr(), y.data_ptr(), mask.data_ptr(), _abi.ASR_F32, n, 0.1, 2, 0,
                         0, stream.cuda_stream)

    def normal():
        arng.normal_(y, seed=3, step=1)

    def uniform():
        arng.uniform_(y, seed=3, step=1)

    for fn in (drop, normal, uniform):
        for _ in range(args.warmup):
            fn()
    wall, drop_ms = _time_launches(torch, stream, drop, args.steps)
    _, normal_ms = _time_launches(torch, stream, normal, args.steps)
    _, uniform_ms = _time_launches(torch, stream, uniform, args.steps)
    achieved = 9 * n / (drop_ms * 1e-3) / 1e9
    return {
        "metric": "elements/sec, Philox dropout with keep mask, 1 GPU", "value": n / wall,
        "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "dropout_2^30_f32_p0.1", "algorithmic_bytes_per_element": 9},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stream_traffic_from_profile(
                         "rng_dropout_2pow30_hbm_counters.json", rng_source_hash(), n),
                     "algorithmic_bytes": 9 * n,
                     "kernel": "asr_rng::rng_kernel<dropout, f32>", "kernel_ms_avg": drop_ms},
        "context": {"normal_fill_ms": normal_ms,
                    "normal_fill_GBps": 4 * n / (normal_ms * 1e-3) / 1e9,
                    "uniform_fill_ms": uniform_ms,
                    "uniform_fill_GBps": 4 * n / (uniform_ms * 1e-3) / 1e9},
    }


def run_hbm_probe(args, torch, ops, wl):
    """What HBM gives the step's launch structure, without its arithmetic:
    the Llama-3-8B list's 4-read/3-write traffic (asr_adamw_stream_probe)
    against the step itself, alternated in three blocks so that drift during
    the run favours neither, with the list allocated first, as in the
    default benchmark; then read-only, write-only and 1:1 copy streams
    (asr_hbm_probe, 16 GiB each way) in the memory left."""
    from adamw_optimizer_stochastic_amd import _abi
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    state = wl.llama3_8b_state(dev, seed=0, states=args.state_layout)
    n_elems = sum(t["param"].numel() for t in state)
    lists = ([t["param"] for t in state], [t["grad"] for t in state],
             [t["exp_avg"] for t in state], [t["exp_avg_sq"] for t in state],
             [t["base_index"] for t in state])
    ws = ops.make_workspace([t["param"].numel() for t in state], dev)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, seed=0,
              rounding="sr", workspace=ws)
    step = [0]

    def adamw():
        step[0] += 1
        ops.adamw_step(*lists, step=step[0], **hp)

    for _ in range(max(2, args.warmup)):
        adamw()
    bytes_per_launch = 22 * n_elems
    step_ms, probe_ms = [], []
    for _ in range(3):
        step_ms.append(_time_launches(torch, stream, adamw, args.steps)[1])
        probe_ms.append(adamw_stream_probe_ms(torch, state, ws, stream, args.steps))
    st, pr = sum(step_ms) / 3, sum(probe_ms) / 3
    step_gbps = bytes_per_launch / (st * 1e-3) / 1e9
    probe_gbps = bytes_per_launch / (pr * 1e-3) / 1e9

    nbytes = 16 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    simple = {}
    for name, kind, moved in (("read", _abi.ASR_PROBE_READ, nbytes),
                              ("write", _abi.ASR_PROBE_WRITE, nbytes),
                              ("copy", _abi.ASR_PROBE_COPY, 2 * nbytes)):
        def fn(kind=kind):
            _abi.asr_hbm_probe(kind, dst.data_ptr(), src.data_ptr(), nbytes, s)
        for _ in range(max(2, args.warmup)):
            fn()
        ms = _time_launches(torch, stream, fn, args.steps)[1]
        simple[name] = {"bytes_per_launch": moved, "ms": ms,
                        "GBps": moved / (ms * 1e-3) / 1e9}
        print(f"[bench] hbm probe {name}: {simple[name]['GBps']:.0f} GB/s", file=sys.stderr,
              flush=True)
    del src, dst
    return {
        "metric": "HBM GB/s of the AdamW-SR step's access pattern without its arithmetic "
                  "(4 streams read, 3 written), 1 GPU",
        "value": probe_gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pr, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "hbm_probe_llama3_8b_param_list", "params": n_elems,
                   "state_layout": STATE_LAYOUT_NOTE[args.state_layout],
                   "algorithmic_bytes_per_param": 22, "simple_stream_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": probe_gbps, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": probe_gbps / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "stream_probe_class / stream_probe_slots (the step's launch "
                               "plan, no arithmetic)", "kernel_ms_avg": pr},
        "context": {"step_ms_blocks": step_ms, "probe_ms_blocks": probe_ms,
                    "step_GBps": step_gbps, "step_over_probe": step_gbps / probe_gbps,
                    "read_only": simple["read"], "write_only": simple["write"],
                    "copy_1to1": simple["copy"],
                    "timing": "HIP events on the launch stream around each call; step and "
                              "probe alternated in 3 blocks of `steps` calls"},
    }


def run_copy_probe(args, torch):
    """A plain device copy of 8 GiB (torch's copy kernel), for scaling the
    FETCH_SIZE/WRITE_SIZE counters: it moves exactly 8 GiB each way."""
    dev = torch.device("cuda", 0)
    n = 8 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(1, args.steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    return {"probe": "copy", "bytes_each_way": n, "ms": ms, "GBps": 2 * n / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["llama3_8b", "llama3_8b_rank", "shards", "convert", "gemm", "rng",
                             "hbm_probe", "bf16_64k", "f32_16m"])
    ap.add_argument("--rank", type=int, default=3, help="rank whose share --workload "
                    "llama3_8b_rank times")
    ap.add_argument("--ranks", type=int, default=8)
    ap.add_argument("--gemm-shape", default=None, help="M,N,K for --workload gemm")
    ap.add_argument("--state-layout", default="flat", choices=["flat", "separate"],
                    help="how the Llama lists' f32 moment states are allocated")
    ap.add_argument("--odd-split", action="store_true", help="--workload shards: time the "
                    "tensor as two pieces cut at an odd element")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if not 0 <= args.rank < args.ranks:
        ap.error("--rank must be in [0, --ranks)")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the optimizer step has no cross-GPU exchange "
              "(each rank would run the same kernel on its own shard with its own "
              "base_index); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline and not args.copy_probe and args.workload == "llama3_8b":
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    if not args.no_cpu_baseline and not args.copy_probe and args.workload == "gemm":
        print("[bench] cpu baseline (oracle gemm) ...", file=sys.stderr, flush=True)
        cpu = gemm_cpu_baseline(8192, 14336, 4096) if not args.gemm_shape else \
            gemm_cpu_baseline(*(int(x) for x in args.gemm_shape.split(",")))

    import torch
    from adamw_optimizer_stochastic_amd import ops
    from adamw_optimizer_stochastic_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        print(json.dumps(run_copy_probe(args, torch)))
        return
    print(f"[bench] {args.workload}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    if args.workload == "convert":
        res = run_convert(args, torch, ops, wl)
    elif args.workload == "gemm":
        res = run_gemm(args, torch, ops, wl)
    elif args.workload == "rng":
        res = run_rng(args, torch, ops, wl)
    elif args.workload == "hbm_probe":
        res = run_hbm_probe(args, torch, ops, wl)
    elif args.workload in ("bf16_64k", "f32_16m"):
        res = run_small(args, torch, ops, wl)
    else:
        res = run_adamw(args, torch, ops, wl)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res))


if __name__ == "__main__":
    main()
