#!/usr/bin/env python3
"""Benchmark of the selective state update on one MI355X.

One step = one ssu_update call over the whole workload (the decode workload
by default: batch 256, heads 128, dim 64, dstate 128, groups 8, fp32 state,
bf16 inputs, a 512-slot pool, read = write slots). Inputs are seeded,
synthetic and resident in HBM before timing starts. W untimed warmup steps,
then K timed steps bracketed by device synchronisation; HIP events on the
launch stream give the kernel's average duration.

Prints ONE JSON line:
  value      whole-job algorithmic GB/s (minimal bytes the method must move,
             per step, times K, over the timed wall time)
  roofline   the kernel against the 8 TB/s HBM peak; traffic = HBM bytes from
             the committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled
             by a plain copy of known size) when they were taken on the
             current kernel source, else null
  cpu_baseline  the CPU oracle timed on this host on the same workload
Timing: every timed call is bracketed by its own pair of HIP events on the
launch stream; kernel_us is their median (kernel_us_mean their mean), and
roofline.achieved uses the median.
  line_granular  (dim-major shift) the same call against the minimal bytes at
             cache-line granularity: its rows are shorter than a line
  ceiling    the same bytes moved by the runtime's device-to-device copy and
             by an in-place read-modify-write stream (libssu_ceiling.so):
             what this part sustains for a plain stream of that size
Options: --config {decode, decode_pad, mtp, varlen, varlen_disable, varlen_nodst, replay,
replay_spec, replay_lp, replay_mx4, spec_snapshots, tiny, conv_shift_sd, conv_shift_ds, memcpy_left, ssd,
ceiling}, --no-cpu-baseline, --calib-copy (also runs a plain device copy of the
state's size, the calibration kernel for the counters). --config ceiling
measures the streaming ceilings alone (1 GiB buffers, every pattern).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSU decode achieved HBM GB/s (% of peak) and token-head updates/s"
HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "mamba_selective_state_amd", "csrc")
# The sources each workload's kernels are built from: a counter reading is
# used only while these are unchanged.
_COMMON = ("ssu_internal.h",)
KERNEL_SOURCES = {
    "decode": ("ssu_kernels.hip", "ssu_device.h") + _COMMON,
    "replay": ("ssu_replay.hip", "ssu_device.h") + _COMMON,
    "copy": ("ssu_copy.hip",) + _COMMON,
    "ssd": ("ssu_ssd.hip",) + _COMMON,
}


REPLAY_CONFIGS = ("replay", "replay_spec", "replay_lp", "replay_mx4")
# the read copy's format of a replay workload
COPY_FORMAT = {"replay_lp": "mx8", "replay_mx4": "mx4"}


def source_family(config):
    if config in REPLAY_CONFIGS:
        return "replay"
    if config in ("conv_shift_sd", "conv_shift_ds", "memcpy_left"):
        return "copy"
    if config == "ssd":
        return "ssd"
    return "decode"

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / f16 matrix peak of MI355X


def workload(name):
    import workloads as W
    if name == "decode":
        return W.decode(), ("decode: batch 256, heads 128, dim 64, dstate 128, groups 8, "
                            "fp32 state (4 MiB per sequence), bf16 x/B/C/z/dt, 512-slot pool, "
                            "read = write slots")
    if name == "decode_pad":
        return W.decode_pad(), ("decode_pad: batch 1024, heads 128, dim 64, dstate 128, groups 8, "
                                "bf16 state, 2048-slot pool, 51 pad rows (pad id 0), out given")
    if name == "mtp":
        return W.mtp(), ("mtp: 64 sequences x 7 tokens, heads 128, dim 64, dstate 128, groups 8, "
                         "fp32 state, 2-D tables, write = read + 448, accepted ~ U{1..7}")
    if name == "replay":
        return W.replay(), ("replay: ReplaySSM decode step on the decode workload's layer (batch "
                            "256, heads 128, dim 64, dstate 128, groups 8, fp32 checkpoint), "
                            "buffer length L = 16, bf16 x/dt/B buffers, per-sequence buffer "
                            "pointers ~ U{0..15} (about 1/16 of the sequences fold each step)")
    if name == "replay_lp":
        return W.replay(), ("replay_lp: the replay workload with an MXFP8 read copy of the fp32 "
                            "checkpoint (E4M3 codes, one E8M0 scale per 32 values): output-only "
                            "steps read the copy, folds store the checkpoint and rewrite the copy")
    if name == "replay_mx4":
        return W.replay(), ("replay_mx4: the replay workload with an MXFP4 read copy of the fp32 "
                            "checkpoint (E2M1 codes two a byte, one E8M0 scale per 32 values): "
                            "output-only steps read the copy, folds store the checkpoint and "
                            "rewrite the copy")
    if name == "replay_spec":
        return W.replay_spec(), ("replay_spec: ReplaySSM speculative step, batch 512 x T = 4 draft "
                                 "tokens, heads 128, dim 64, dstate 128, groups 8, fp32 "
                                 "checkpoint, L = 16, bf16 buffers, committed pointers ~ U{0..12} "
                                 "(a sequence folds at h + 2T > L)")
    if name == "spec_snapshots":
        return W.spec_snapshots(), ("spec_snapshots: the same drafts through the plain update "
                                    "with one fp32 state snapshot per draft (batch 512 x T = 4, "
                                    "heads 128, dim 64, dstate 128, groups 8), the design "
                                    "ReplaySSM replaces")
    if name in ("conv_shift_sd", "conv_shift_ds"):
        layout = "SD" if name.endswith("sd") else "DS"
        return W.conv_shift(layout=layout), (
            "%s: 6144 convolution-state shifts (256 sequences x 24 layers), width 4, inner 8192, "
            "fp16 (64 KiB blocks), %s layout, half of them inside one block, bias ~ U{1..3}"
            % (name, "token-major" if layout == "SD" else "dim-major"))
    if name == "ssd":
        c = W.ssd_bench()
        return c, ("ssd: packed variable-length SSD prefill, 8 sequences of U{512..4096} tokens "
                   "(%d tokens, %d chunks of up to 256), heads 128, dim 64, dstate 128, groups 8, "
                   "bf16 x/B/C/z, f32 dt and states, initial states"
                   % (np.shape(c["x"])[0], len(c["seq_idx"])))
    if name == "memcpy_left":
        return W.memmove_rows(rows=4096, row_bytes=32 * 1024, shift=16, direction="left"), (
            "memcpy_left: 4096 rows of 32 KiB each copied onto itself shifted left by 16 bytes "
            "(the vLLM PR #50729 regression case, 32x the rows)")
    if name.startswith("varlen"):
        dst = name != "varlen_nodst"
        dis = name == "varlen_disable"
        return W.varlen(dst=dst, disable=dis), (
            "%s: 512 sequences, lengths U{0..8}, heads 64, dim 64, dstate 128, groups 1, "
            "fp16 state, flat tables, per-head dt%s" % (
                name, ", disable_state_update" if dis else (", no dst table" if not dst else "")))
    raise SystemExit("unknown --config %s" % name)


def spans(case):
    x = np.asarray(case["x"])
    cu = case.get("cu_seqlens")
    if cu is not None:
        cu = np.asarray(cu, np.int64)
        return [(int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(cu.size - 1)]
    if x.ndim == 4:
        return [(b * x.shape[1], x.shape[1]) for b in range(x.shape[0])]
    return [(r, 1) for r in range(x.shape[0])]


def _entry(tab, b, first, t):
    tab = np.asarray(tab)
    return int(tab[first + t]) if tab.ndim == 1 else int(tab[b, t])


def algorithmic_bytes(case):
    """Minimal bytes one call must move: each distinct state tile read once
    (pad reads cost nothing), each tile stored once, every input row and
    per-head vector read once, y written once, table and metadata entries
    read once. Returns (bytes, token-head updates)."""
    slots, H, P, N = np.shape(case["state"])
    sb = DTYPE_BYTES[case["state_dtype"]]
    io = DTYPE_BYTES[case["io_dtype"]]
    dtb = DTYPE_BYTES[case.get("dt_dtype", case["io_dtype"])]
    x = np.asarray(case["x"])
    R = x.shape[0] * (x.shape[1] if x.ndim == 4 else 1)
    G = np.shape(case["B"])[-2]
    pad = int(case.get("pad_slot_id", -1))
    acc = case.get("num_accepted_tokens")
    rt, wt = case.get("state_batch_indices"), case.get("dst_state_batch_indices")
    wt = wt if wt is not None else rt
    tile = H * P * N * sb
    reads, writes, nseq = 0, 0, 0
    for b, (first, n) in enumerate(spans(case)):
        nseq += 1
        if n == 0:
            continue
        start = 0 if acc is None else max(int(acc[b]) - 1, 0)
        if (b if rt is None else _entry(rt, b, first, start)) != pad:
            reads += 1
        if not case.get("disable_state_update", False):
            for t in range(n):
                if (b if wt is None else _entry(wt, b, first, t)) != pad:
                    writes += 1
    per_head = np.ndim(case["dt"]) == x.ndim - 1
    row = H * P * io * 2 + (H * P * io if case.get("z") is not None else 0)  # x, out, z
    row += (H if per_head else H * P) * dtb + 2 * G * N * io                  # dt, B, C
    vec = 4 * H * (1 + (case.get("D") is not None) + (case.get("dt_bias") is not None))
    idx = 0
    for t in (case.get("state_batch_indices"), case.get("dst_state_batch_indices")):
        if t is not None:
            idx += np.asarray(t).itemsize * (nseq if t is rt else R)
    for t in (case.get("cu_seqlens"), acc):
        if t is not None:
            idx += np.asarray(t).nbytes
    total = (reads + writes) * tile + R * row + vec + idx
    return int(total), int(R * H)


def replay_algorithmic_bytes(case, lp=None):
    """Minimal bytes of one ReplaySSM step: each live sequence reads its
    checkpoint tile and its h committed entries; a folding sequence writes its
    checkpoint; the step's tokens are appended (one entry per token, or none
    for a one-token fold); plus the step's inputs and y, and per-head vectors
    and tables, as for the plain update. One-token steps fold at h + 1 = L,
    speculative steps (x [batch, T, ...]) at h + 2T > L. With a read copy
    (lp "mx8": 1 + 1/32 bytes a value; "mx4": 1/2 + 1/32) an output-only step
    reads the copy in place of the tile, and a fold also writes the copy.
    Returns (bytes, token-head updates)."""
    slots, H, P, N = np.shape(case["state"])
    sb = DTYPE_BYTES[case["state_dtype"]]
    io = DTYPE_BYTES[case["io_dtype"]]
    dtb = DTYPE_BYTES[case.get("dt_dtype", case["io_dtype"])]
    G = np.shape(case["B"])[-2]
    L = int(case["L"])
    x = np.asarray(case["x"])
    spec = x.ndim == 4
    T = x.shape[1] if spec else 1
    per_head = np.ndim(case["buf_dt"]) == 3
    entry = H * P * io + (H if per_head else H * P) * dtb + G * N * io
    tile = H * P * N * sb
    copy = H * P * N // (2 if lp == "mx4" else 1) + H * P * N // 32
    pad = int(case.get("pad_slot_id", -1))
    tab = case.get("state_batch_indices")
    total = 0
    batch = x.shape[0]
    for b in range(batch):
        s = b if tab is None else int(np.asarray(tab)[b])
        if s == pad:
            continue
        h = int(case["buf_len"][b])
        fold = h + 2 * T > L if spec else h + 1 == L
        total += (copy if lp and not fold else tile) + h * entry
        if not case.get("disable_state_update", False):
            if spec:
                total += (tile if fold else 0) + T * entry
            else:
                total += tile + (copy if lp else 0) if fold else entry
    R = batch * T
    row = H * P * io * 2 + (H * P * io if case.get("z") is not None else 0)
    row += (H if np.ndim(case["dt"]) == x.ndim - 1 else H * P) * dtb + 2 * G * N * io
    vec = 4 * H * (1 + (case.get("D") is not None) + (case.get("dt_bias") is not None))
    idx = (np.asarray(tab).itemsize * batch if tab is not None else 0) + \
        np.asarray(case["buf_len"]).nbytes
    return int(total + R * row + vec + idx), int(R * H)


# ---------------------------------------------------------------- timing

def time_calls(launch, stream, steps, warmup):
    """Warm up, then `steps` calls, each between its own pair of HIP events
    on `stream` (the stream the library launches on), the whole bracketed by
    device synchronisation. Returns (per-call ms list, wall s)."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize(stream.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize(stream.device)
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def kernel_times(ms):
    """(median, mean) of per-call durations, in ms."""
    return statistics.median(ms), statistics.fmean(ms)


_ceiling_lib = None


def ceiling_lib():
    global _ceiling_lib
    if _ceiling_lib is None:
        import ctypes
        from mamba_selective_state_amd import build as B
        if not os.path.exists(B.CEILING_LIB):
            raise SystemExit("libssu_ceiling.so is not built (run mamba_selective_state_amd/build.py)")
        lib = ctypes.CDLL(B.CEILING_LIB)
        lib.ssu_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
        lib.ssu_ceiling_run.restype = ctypes.c_int
        _ceiling_lib = lib
    return _ceiling_lib


CEILING_KINDS = {"rmw": 0, "copy": 1, "write": 2, "read": 3}
# launch shapes tried for each pattern: (lanes per workgroup, 16-byte words
# per lane per pass, grid: "pass" = one workgroup per pass-sized piece, or a
# fixed count walking the buffer grid-stride)
CEILING_SHAPES = ((64, 8, "pass"), (64, 4, "pass"), (256, 4, "pass"), (256, 8, "pass"),
                  (256, 4, 2048), (256, 8, 4096))


def stream_ceiling(dev, kind, nbytes, nt=True, reps=10, shapes=CEILING_SHAPES):
    """Best GB/s of one ceiling pattern over a buffer of `nbytes` (bytes
    moved per call: read + written) among the launch shapes, median of `reps`
    calls each; returns (GB/s, shape)."""
    import torch
    lib = ceiling_lib()
    nbytes = nbytes // 16 * 16
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = a if kind in ("rmw", "read") else torch.empty_like(a)
    stream = torch.cuda.current_stream(dev)
    moved = nbytes * (2 if kind in ("rmw", "copy") else 1)
    best = (0.0, None)
    for threads, words, grid in shapes:
        if grid == "pass":
            grid = (nbytes // 16 + threads * words - 1) // (threads * words)
        sink = torch.empty(grid, dtype=torch.float32, device=dev)

        def launch():
            e = lib.ssu_ceiling_run(CEILING_KINDS[kind], int(nt), a.data_ptr(), b.data_ptr(), nbytes,
                                    sink.data_ptr(), grid, threads, words, stream.cuda_stream)
            if e:
                raise RuntimeError("ceiling kernel launch failed: %d" % e)

        ms, _ = time_calls(launch, stream, reps, 3)
        gbs = moved / (statistics.median(ms) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, "%d lanes x %d words, grid %d" % (threads, words, grid))
    return best


def copy_ceiling(dev, nbytes, reps=10):
    """GB/s of the runtime's device-to-device copy (hipMemcpyAsync) moving
    `nbytes` (half read, half written), median of `reps` calls."""
    import torch
    half = nbytes // 2 // 16 * 16
    src = torch.empty(half // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    ms, _ = time_calls(lambda: dst.copy_(src), stream, reps, 3)
    return 2 * half / (statistics.median(ms) * 1e-3) / 1e9


def ceiling_fields(dev, nbytes):
    """The streaming ceilings for `nbytes` moved (reported beside a result)."""
    return {"bytes": int(nbytes),
            "d2d_copy_gbs": round(copy_ceiling(dev, nbytes), 1),
            "rmw_nt_gbs": round(stream_ceiling(dev, "rmw", nbytes // 2)[0], 1),
            "note": "the same bytes through hipMemcpyAsync device-to-device and through an "
                    "in-place 16-byte non-temporal read-modify-write stream (libssu_ceiling.so)"}


def ceiling_bench(args):
    """--config ceiling: every streaming pattern over 1 GiB buffers."""
    import torch
    dev = torch.device("cuda", 0)
    size = 1 << 30
    res, shapes = {}, {}
    for kind in ("rmw", "copy", "write", "read"):
        for nt in (True, False):
            key = "%s_%s" % (kind, "nt" if nt else "plain")
            gbs, shape = stream_ceiling(dev, kind, size, nt)
            res[key], shapes[key] = round(gbs, 1), shape
    res["d2d_copy_runtime"] = round(copy_ceiling(dev, 2 * size), 1)
    best = max(res.values())
    result = {"metric": "HBM streaming ceilings (GB/s moved, read + written)", "value": best,
              "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 3, "ms_per_step": None,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
              "data": "synthetic",
              "config": {"workload": "ceiling: 1 GiB buffers, 16-byte accesses, the best of %d "
                                     "launch shapes per pattern; rmw = in place p = 0.5 p + 1, "
                                     "copy, write-only, read-only; nt = non-temporal hint"
                                     % len(CEILING_SHAPES)},
              "patterns_gbs": res, "best_shapes": shapes,
              "pct_of_hbm_peak": {k: round(100 * v / HBM_PEAK_GBS, 1) for k, v in res.items()}}
    print(json.dumps(result), flush=True)


def oracle_threads():
    """Threads for the threaded oracle leg: the cores this process may run
    on, at most the 16 host cores of a one-GPU share."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def timed_oracle(run, case, reps, threads):
    """Median wall time of `reps` oracle calls on `threads` threads, and the
    last result."""
    from oracle import ssu_oracle
    orc = ssu_oracle.default()
    before = orc.threads()
    orc.set_threads(threads)
    try:
        times, res = [], None
        for _ in range(reps):
            t0 = time.perf_counter()
            res = run(case)
            times.append(time.perf_counter() - t0)
    finally:
        orc.set_threads(before)
    return statistics.median(times), res


def same_result(a, b):
    return all(np.array_equal(np.asarray(a[k]), np.asarray(b[k])) for k in a)


COPY_CONFIGS = ("conv_shift_sd", "conv_shift_ds", "memcpy_left")


def ssd_algorithmic(case):
    """Bytes the prefill must move (inputs read once, y and the returned
    states written once) and the chunked algorithm's matrix flops: per chunk
    of L tokens and head, the chunk state 2 L P N, the masked C.B^T's product
    with x L (L + 1) P and the entering state read out 2 L N P; per chunk and
    group (C.B^T does not depend on the head) C.B^T over the causal half
    L (L + 1) N. Returns (bytes, flops)."""
    T, H, P = np.shape(case["x"])
    G, N = np.shape(case["B"])[1:]
    io = DTYPE_BYTES[case["io_dtype"]]
    sb = DTYPE_BYTES[case["state_dtype"]]
    batch = len(case["last_chunk_indices"])
    nbytes = T * H * P * io * (2 + (case.get("z") is not None))          # x, out, z
    nbytes += T * H * DTYPE_BYTES[case["dt_dtype"]] + 2 * T * G * N * io  # dt, B, C
    nbytes += batch * H * P * N * sb * (1 + (case.get("initial_states") is not None))
    cu = np.asarray(case["cu_chunk_seqlens"])
    flops = 0
    for L in np.diff(cu):
        L = int(L)
        flops += H * (2 * L * P * N + L * (L + 1) * P + 2 * L * N * P) + G * L * (L + 1) * N
    return int(nbytes), int(flops)


def ssd_bench_run(args, case, desc):
    import torch
    import mamba_selective_state_amd as ssu
    from workloads.device import TORCH, dev as to_dev
    d = torch.device("cuda", 0)
    io, sd = case["io_dtype"], case["state_dtype"]
    x, B, C, z = (to_dev(case[k], io, d) for k in ("x", "B", "C", "z"))
    dt = to_dev(case["dt"], case["dt_dtype"], d)
    A, D, bias = (torch.from_numpy(case[k]).to(d) for k in ("A", "D", "dt_bias"))
    idx = {k: torch.from_numpy(np.asarray(case[k])).to(d)
           for k in ("cu_seqlens", "cu_chunk_seqlens", "last_chunk_indices", "seq_idx")}
    init = to_dev(case["initial_states"], sd, d)
    out = torch.empty_like(x)
    def step():
        return ssu.ssd_combined_fwd_varlen(
            x, dt, A, B, C, case["chunk_size"], idx["cu_seqlens"], idx["cu_chunk_seqlens"],
            idx["last_chunk_indices"], idx["seq_idx"], out=out, D=D, z=z, dt_bias=bias,
            dt_softplus=case["dt_softplus"], dt_limit=case["dt_limit"], initial_states=init,
            state_dtype=TORCH[sd])
    stream = torch.cuda.current_stream(d)
    per_call, wall = time_calls(step, stream, args.steps, args.warmup)
    event_ms, mean_ms = kernel_times(per_call)
    if args.calib_copy:
        src_c = torch.empty((1 << 30) // 4, dtype=torch.float32, device=d).fill_(1.0)
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize(d)
    nbytes, flops = ssd_algorithmic(case)
    tflops = flops / (event_ms * 1e-3) / 1e12
    gbs = nbytes / (event_ms * 1e-3) / 1e9
    # the binding roofline: the larger of the time the flops need at the bf16
    # MFMA peak and the time the bytes need at the HBM peak
    hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    result = {
        "metric": "SSD prefill matrix TFLOP/s (bf16 MFMA) and tokens/s", "value": round(flops * args.steps / wall / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "flops_per_step": flops, "bytes_per_step": nbytes,
                   "kernels": "ssd_prep_kernel, ssd_fused_kernel"},
        "tokens_per_s": round(np.shape(case["x"])[0] * args.steps / wall, 1),
        "hbm_gbs_algorithmic": round(nbytes / (event_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm" if hbm_bound else "mfma",
                     "achieved": round(gbs if hbm_bound else tflops, 3),
                     "peak": HBM_PEAK_GBS if hbm_bound else MFMA_BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": round(gbs / HBM_PEAK_GBS if hbm_bound else tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                     "traffic": traffic_from_counters("ssd"),
                     "kernel_us": round(event_ms * 1e3, 2),
                     "kernel_us_mean": round(mean_ms * 1e3, 2),
                     "intensity_flop_per_byte": round(flops / nbytes, 1),
                     "ridge_flop_per_byte": round(MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS, 1),
                     "mfma_tflops": round(tflops, 3), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                     "note": "the launches of one call timed together"},
        "ceiling": ceiling_fields(d, nbytes),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = ssd_cpu_baseline(case, flops)
    print(json.dumps(result), flush=True)


def ssd_cpu_baseline(case, flops):
    """The SSD oracle on sampled heads (heads are independent): one head pair
    on one thread, then one head pair per thread on `threads` threads at once
    (the oracle's C call runs without the interpreter lock), each scaled to
    all heads; the threads' first pair must equal the serial run byte for
    byte."""
    import threading
    from oracle import ssu_oracle
    import workloads as W
    H = np.shape(case["x"])[1]
    threads = oracle_threads()
    pairs = [[(2 * i) % H, (2 * i + 64) % H] for i in range(threads)]
    subs = [W.ssd_heads(case, hp) for hp in pairs]
    t1 = time.perf_counter()
    serial = ssu_oracle.run_ssd(subs[0])
    t_serial = (time.perf_counter() - t1) * H / 2
    results = [None] * threads

    def work(i):
        results[i] = ssu_oracle.run_ssd(subs[i])

    workers = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    t1 = time.perf_counter()
    for w in workers:
        w.start()
    for w in workers:
        w.join()
    t_threads = (time.perf_counter() - t1) * H / (2 * threads)
    identical = same_result(serial, results[0])
    assert identical, "the threaded SSD oracle differs from the serial one"
    return {"value": round(flops / t_threads / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "nproc": os.cpu_count(),
            "serial_value": round(flops / t_serial / 1e12, 6),
            "identical_to_serial": bool(identical),
            "sample": "head pairs (heads are independent): one pair on one thread (%.1f s per call "
                      "scaled to all %d heads), then %d pairs on %d threads at once (%.1f s per "
                      "call scaled); token-by-token C oracle" % (t_serial, H, threads, threads,
                                                                 t_threads)}


def copy_algorithmic_bytes(case):
    """Bytes a copy must read and write: every moved byte once each way, plus
    the request vectors. Returns (bytes, requests)."""
    if "pool" in case:
        pool = case["pool"]
        Wd = pool.shape[1] if case["layout"] == "SD" else pool.shape[2]
        inner = pool.shape[2] if case["layout"] == "SD" else pool.shape[1]
        moved = int(np.sum(Wd - np.asarray(case["bias"]))) * inner * pool.itemsize
        return 2 * moved + 3 * 8 * len(case["bias"]), len(case["bias"])
    sizes = np.asarray(case["sizes"])
    return int(2 * np.sum(np.maximum(sizes, 0)) + 3 * 8 * len(sizes)), len(sizes)


def copy_line_bytes(case):
    """Minimal HBM bytes at cache-line granularity (128 B): the dim-major
    shift moves (W - bias) elements of rows only W elements long (8 bytes at
    width 4, fp16), so every line of the source block is read and every line
    of the destination block written; the other copies move whole lines (the
    byte-exact count). Returns bytes per step."""
    if "pool" in case and case["layout"] == "DS":
        pool = case["pool"]
        block = pool.shape[1] * pool.shape[2] * pool.itemsize
        return 2 * block * len(case["bias"]) + 3 * 8 * len(case["bias"])
    return copy_algorithmic_bytes(case)[0]


def copy_bench(args, name, case, desc):
    """bench.py for the state copies: one step is one call over the workload."""
    import torch
    import mamba_selective_state_amd as ssu
    dev = torch.device("cuda", 0)
    alg_bytes, requests = copy_algorithmic_bytes(case)
    if "pool" in case:
        pool = case["pool"]
        t = torch.from_numpy(pool.view(np.uint8)).to(dev).view(torch.float16).reshape(pool.shape)
        idx = [torch.from_numpy(np.asarray(case[k])).to(dev) for k in ("src_blk", "dst_blk", "bias")]
        cargs = ssu.make_conv_shift_args(t, *idx, layout=case["layout"])
        launch = lambda h: ssu.ssu_conv_state_shift(cargs, h)  # noqa: E731
        kernel = "conv_shift_%s_kernel" % ("token_major" if case["layout"] == "SD" else "dim_major")
    else:
        buf = torch.from_numpy(case["buf"]).to(dev)
        base = buf.data_ptr()
        src = (torch.from_numpy(np.asarray(case["src_off"])) + base).to(dev)
        dst = (torch.from_numpy(np.asarray(case["dst_off"])) + base).to(dev)
        sizes = torch.from_numpy(np.asarray(case["sizes"])).to(dev)
        from mamba_selective_state_amd import ssu as binding
        descs = [binding.tensor_desc(v, dev) for v in (src, dst, sizes)]
        max_size = int(np.max(case["sizes"]))
        launch = lambda h: ssu.ssu_batch_memcpy(*descs, max_size, h)  # noqa: E731
        kernel = "batch_memcpy_kernel"
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    per_call, wall = time_calls(lambda: launch(handle), stream, args.steps, args.warmup)
    event_ms, mean_ms = kernel_times(per_call)
    if args.calib_copy:
        nbytes = 1 << 30
        src_c = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize(dev)
        print("[bench] calibration copy: %d bytes read, %d written" % (nbytes, nbytes),
              file=sys.stderr, flush=True)
    achieved = alg_bytes / (event_ms * 1e-3) / 1e9
    result = {
        "metric": "state copy achieved HBM GB/s (% of peak)", "value": round(alg_bytes * args.steps / wall / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": desc, "bytes_per_step": alg_bytes, "requests_per_step": requests,
                   "kernel": kernel},
        "pct_of_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_counters(name),
                     "kernel_us": round(event_ms * 1e3, 2), "kernel_us_mean": round(mean_ms * 1e3, 2)},
        "ceiling": ceiling_fields(dev, alg_bytes),
    }
    line = copy_line_bytes(case)
    if line != alg_bytes:
        result["line_granular"] = {"bytes_per_step": line,
                                   "achieved": round(line / (event_ms * 1e-3) / 1e9, 2),
                                   "frac": round(line / (event_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_cpu_baseline:
        from oracle import ssu_oracle
        times = []
        for _ in range(args.cpu_reps):
            t1 = time.perf_counter()
            if "pool" in case:
                ssu_oracle.run_conv_shift(case["pool"], case["layout"], case["src_blk"], case["dst_blk"],
                                          case["bias"])
            else:
                ssu_oracle.run_batch_memmove(case["buf"], case["src_off"], case["dst_off"], case["sizes"])
            times.append(time.perf_counter() - t1)
        tm = statistics.median(times)
        result["cpu_baseline"] = {"value": round(alg_bytes / tm / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "the whole workload, median of %d calls (%.3f s each), "
                                            "plain-C memmove oracle incl. its NumPy wrapper"
                                            % (args.cpu_reps, tm)}
    print(json.dumps(result), flush=True)


def tiny_bench(args):
    """The MATE page's minimal example (batch 2, heads 8, dim 8, dstate 128,
    fp16 state): one step is its two chained calls (no tables, then tables
    [0, 1]). Launch-bound: reported as latency per step on the stream (HIP
    events, eager launches), with the wall time and the replay of a HIP graph
    holding both calls alongside."""
    import torch
    import mamba_selective_state_amd as ssu
    from workloads import one_token_tiny
    from workloads.device import TORCH, device_case
    dev = torch.device("cuda", 0)
    cases = [one_token_tiny(tables=False), one_token_tiny(tables=True)]
    d0 = device_case(cases[0], dev)
    calls = []
    for c in cases:
        d = device_case(c, dev)
        d["state"] = d0["state"]  # the two calls share the pool, as on the page
        out = torch.empty(np.shape(c["x"]), dtype=TORCH[c["io_dtype"]], device=dev)
        calls.append(ssu.make_args(d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                   d["dt_bias"], False, d["state_batch_indices"], -1, out, False,
                                   d["dst_state_batch_indices"], None, None))
        calls[-1]._keep = (d, out)
    nbytes = sum(algorithmic_bytes(c)[0] for c in cases)
    updates = sum(algorithmic_bytes(c)[1] for c in cases)
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        handle = stream.cuda_stream

        def step():
            for a in calls:
                ssu.ssu_update(a, handle)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize(dev)
        steps = max(args.steps, 1000)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize(dev)
        eager = (time.perf_counter() - t0) / steps
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(steps):
            step()
        s1.record(stream)
        torch.cuda.synchronize(dev)
        eager_events = s0.elapsed_time(s1) / steps * 1e-3
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize(dev)
        s0.record(stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        s1.record(stream)
        torch.cuda.synchronize(dev)
        graph_wall = (time.perf_counter() - t0) / steps
        graph = s0.elapsed_time(s1) / steps * 1e-3
    achieved = nbytes / eager_events / 1e9
    result = {
        "metric": "SSU decode latency, MATE minimal example (two chained calls)",
        "value": round(eager_events * 1e6, 3), "unit": "us", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(eager_events * 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "tiny: the MATE page's minimal example, batch 2, heads 8, dim 8, "
                               "dstate 128, groups 2, fp16 state, two chained calls (no tables, then "
                               "tables [0, 1])", "bytes_per_step": nbytes,
                   "token_head_updates_per_step": updates},
        "eager_us_per_step_wall": round(eager * 1e6, 3),
        "eager_us_per_step_events": round(eager_events * 1e6, 3),
        "graph_us_per_step_events": round(graph * 1e6, 3),
        "graph_us_per_step_wall": round(graph_wall * 1e6, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 6), "traffic": None,
                     "note": "launch-bound: the two launches move %d bytes" % nbytes},
    }
    if not args.no_cpu_baseline:
        from oracle import ssu_oracle
        ssu_oracle.default()
        reps = 200
        t0 = time.perf_counter()
        for _ in range(reps):
            for c in cases:
                ssu_oracle.run(c)
        t = (time.perf_counter() - t0) / reps
        result["cpu_baseline"] = {"value": round(t * 1e6, 2), "unit": "us", "cores": 1, "kind": "oracle",
                                  "sample": "the two calls, mean of %d repetitions; single-threaded "
                                            "plain-C oracle incl. its NumPy wrapper" % reps}
    print(json.dumps(result), flush=True)


def kernel_source_hash(config):
    """sha256 over the sources the workload's kernels are built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[source_family(config)]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_from_counters(config):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing, for another workload, or taken on other kernel sources."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    entry = c.get("workloads", {}).get(config)
    if not entry or entry.get("kernel_source_sha256") != kernel_source_hash(config):
        return None
    return entry.get("hbm_bytes_per_dispatch")


def cpu_baseline(case, alg_bytes, updates, reps, lp=None):
    """The oracle on the whole workload: median of `reps` calls on one
    thread, then on oracle_threads() threads over sequences; the two results
    must be byte-identical."""
    from oracle import ssu_oracle
    ssu_oracle.default()
    if "buf_len" in case:
        run = ssu_oracle.run_replay_spec if np.ndim(case["x"]) == 4 else ssu_oracle.run_replay
        if lp:
            case = dict(case, lp_format=lp)
            quantize = ssu_oracle.mx4_quantize if lp == "mx4" else ssu_oracle.mx8_quantize
            case["lp"], case["lp_scale"] = quantize(np.asarray(case["state"], np.float32))
    else:
        run = ssu_oracle.run
    threads = oracle_threads()
    t1, r1 = timed_oracle(run, case, reps, 1)
    tn, rn = timed_oracle(run, case, reps, threads)
    identical = same_result(r1, rn)
    assert identical, "the threaded oracle differs from the serial one"
    return {"value": round(alg_bytes / tn / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "updates_per_s": round(updates / tn, 1), "nproc": os.cpu_count(),
            "serial_value": round(alg_bytes / t1 / 1e9, 4),
            "serial_updates_per_s": round(updates / t1, 1),
            "identical_to_serial": bool(identical),
            "sample": "the whole workload, one call per repetition, median of %d: %.2f s on %d "
                      "threads over sequences, %.2f s on one thread; plain-C fp32 oracle incl. "
                      "its NumPy wrapper" % (reps, tn, threads, t1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--calib-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selective state update has no cross-GPU step "
              "(sequences and heads shard with no exchange); run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.config == "ceiling":
        import torch
        if not torch.cuda.is_available():
            raise SystemExit("bench.py needs a GPU")
        ceiling_bench(args)
        return
    if args.config == "ssd":
        import torch
        if not torch.cuda.is_available():
            raise SystemExit("bench.py needs a GPU")
        case, desc = workload(args.config)
        ssd_bench_run(args, case, desc)
        return
    if args.config in COPY_CONFIGS:
        import torch
        if not torch.cuda.is_available():
            raise SystemExit("bench.py needs a GPU")
        case, desc = workload(args.config)
        copy_bench(args, args.config, case, desc)
        return
    if args.config == "tiny":
        import torch
        if not torch.cuda.is_available():
            raise SystemExit("bench.py needs a GPU")
        tiny_bench(args)
        return

    import torch
    import mamba_selective_state_amd as ssu
    from workloads.device import TORCH, device_case, device_replay

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda", 0)
    case, desc = workload(args.config)
    is_replay = args.config in REPLAY_CONFIGS
    lp = COPY_FORMAT.get(args.config)
    alg_bytes, updates = replay_algorithmic_bytes(case, lp) if is_replay else \
        algorithmic_bytes(case)
    print("[bench] %s: %.3f GB per step" % (args.config, alg_bytes / 1e9), file=sys.stderr,
          flush=True)
    d = device_replay(case, dev) if is_replay else device_case(case, dev)
    out = torch.empty(np.shape(case["x"]), dtype=TORCH[case["io_dtype"]], device=dev)
    if is_replay:
        args_c = ssu.make_replay_args(d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                      d["buf_x"], d["buf_dt"], d["buf_B"], d["buf_len"], d["z"],
                                      d["dt_bias"], case.get("dt_softplus", False),
                                      d["state_batch_indices"], case.get("pad_slot_id", -1), out,
                                      case.get("disable_state_update", False))
        launch = ssu.ssu_replay_spec_update if args.config == "replay_spec" else \
            ssu.ssu_replay_update
        if lp:
            # the read copy is resident state like the checkpoint: made once,
            # on the GPU, before the timed steps
            quantize = ssu.mx4_quantize if lp == "mx4" else ssu.mx8_quantize
            d["lp"], d["lp_scale"] = quantize(d["state"])
            args_c = ssu.make_replay_lp_args(
                d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["buf_x"],
                d["buf_dt"], d["buf_B"], d["buf_len"], d["lp"], d["lp_scale"], d["z"],
                d["dt_bias"], case.get("dt_softplus", False), d["state_batch_indices"],
                case.get("pad_slot_id", -1), out, case.get("disable_state_update", False))
            launch = ssu.ssu_replay_mx4_update if lp == "mx4" else ssu.ssu_replay_lp_update
    else:
        args_c = ssu.make_args(d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                               d["z"], d["dt_bias"], case.get("dt_softplus", False),
                               d["state_batch_indices"], case.get("pad_slot_id", -1), out,
                               case.get("disable_state_update", False),
                               d["dst_state_batch_indices"], d["cu_seqlens"],
                               d["num_accepted_tokens"])
        launch = ssu.ssu_update
    x = np.asarray(case["x"])
    plan = {"kernel": "ssu_replay_spec_kernel" if args.config == "replay_spec"
            else "ssu_replay_kernel"} if is_replay else ssu.prewarm_selective_state_update(
        state_dtype=TORCH[case["state_dtype"]], io_dtype=TORCH[case["io_dtype"]],
        batch=x.shape[0], heads=x.shape[-2], dim=x.shape[-1], dstate=np.shape(case["state"])[-1],
        groups=np.shape(case["B"])[-2],
        slot_dtype=torch.int64 if np.asarray(case["state_batch_indices"]).dtype == np.int64
        else torch.int32,
        packed=x.ndim == 4 or case.get("cu_seqlens") is not None
        or case.get("num_accepted_tokens") is not None,
        dt_dtype=TORCH[case.get("dt_dtype", case["io_dtype"])],
        disable_state_update=case.get("disable_state_update", False))
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    per_call, wall = time_calls(lambda: launch(args_c, handle), stream, args.steps, args.warmup)
    event_ms, mean_ms = kernel_times(per_call)
    print("[bench] %d steps: %.1f us per call (median of events; mean %.1f), %.1f us per step "
          "(wall)" % (args.steps, event_ms * 1e3, mean_ms * 1e3, wall / args.steps * 1e6),
          file=sys.stderr, flush=True)

    if args.calib_copy:
        nbytes = int(np.prod(np.shape(case["state"]))) * DTYPE_BYTES[case["state_dtype"]] // 2
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print("[bench] calibration copy: %d bytes read, %d written" % (nbytes, nbytes),
              file=sys.stderr, flush=True)

    achieved = alg_bytes / (event_ms * 1e-3) / 1e9
    traffic = traffic_from_counters(args.config)
    result = {
        "metric": METRIC,
        "value": round(alg_bytes * args.steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "bytes_per_step": alg_bytes,
                   "token_head_updates_per_step": updates, "kernel": plan["kernel"]},
        "pct_of_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "token_head_updates_per_s": round(updates * args.steps / wall, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(event_ms * 1e3, 2),
                     "kernel_us_mean": round(mean_ms * 1e3, 2)},
        "ceiling": ceiling_fields(dev, alg_bytes),
    }
    if args.config == "replay_spec":
        result["roofline"]["note"] = ("each call is the step and the append of the drafts' B "
                                      "rows and per-head dt, timed together")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, alg_bytes, updates, args.cpu_reps, lp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
