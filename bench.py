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
Options: --config {decode, decode_pad, mtp, varlen, varlen_disable, varlen_nodst, replay,
replay_spec, replay_lp, spec_snapshots, tiny, conv_shift_sd, conv_shift_ds, memcpy_left, ssd},
--no-cpu-baseline, --calib-copy (also runs a plain device copy of the state's
size, the calibration kernel for the counters).
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
KERNEL_SOURCES = [os.path.join(ROOT, "mamba_selective_state_amd", "csrc", f)
                  for f in ("ssu_kernels.hip", "ssu_copy.hip", "ssu_ssd.hip", "ssu_internal.h")]

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


def replay_algorithmic_bytes(case, lp=False):
    """Minimal bytes of one ReplaySSM step: each live sequence reads its
    checkpoint tile and its h committed entries; a folding sequence writes its
    checkpoint; the step's tokens are appended (one entry per token, or none
    for a one-token fold); plus the step's inputs and y, and per-head vectors
    and tables, as for the plain update. One-token steps fold at h + 1 = L,
    speculative steps (x [batch, T, ...]) at h + 2T > L. With the MXFP8 read
    copy (lp) an output-only step reads the copy (1 + 1/32 bytes a value) in
    place of the tile, and a fold also writes the copy. Returns (bytes,
    token-head updates)."""
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
    copy = H * P * N + H * P * N // 32
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


COPY_CONFIGS = ("conv_shift_sd", "conv_shift_ds", "memcpy_left")


def ssd_algorithmic(case):
    """Bytes the prefill must move (inputs read once, y and the returned
    states written once) and the chunked algorithm's matrix flops: per chunk
    of L tokens and head, the chunk state 2 L P N, C.B^T over the causal half
    L (L + 1) N, its product with x L (L + 1) P, and the entering state read
    out 2 L N P. Returns (bytes, flops)."""
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
        flops += H * (2 * L * P * N + L * (L + 1) * N + L * (L + 1) * P + 2 * L * N * P)
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
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(d)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize(d)
    wall = time.perf_counter() - t0
    event_ms = start.elapsed_time(end) / args.steps
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
                   "kernels": "ssd_chunk_state_kernel, ssd_state_pass_kernel, ssd_chunk_scan_kernel"},
        "tokens_per_s": round(np.shape(case["x"])[0] * args.steps / wall, 1),
        "hbm_gbs_algorithmic": round(nbytes / (event_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm" if hbm_bound else "mfma",
                     "achieved": round(gbs if hbm_bound else tflops, 3),
                     "peak": HBM_PEAK_GBS if hbm_bound else MFMA_BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": round(gbs / HBM_PEAK_GBS if hbm_bound else tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                     "traffic": traffic_from_counters("ssd"),
                     "kernel_us": round(event_ms * 1e3, 2),
                     "intensity_flop_per_byte": round(flops / nbytes, 1),
                     "ridge_flop_per_byte": round(MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS, 1),
                     "mfma_tflops": round(tflops, 3), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                     "note": "the three launches of one call timed together"},
    }
    if not args.no_cpu_baseline:
        from oracle import ssu_oracle
        import workloads as W
        heads = [0, 64]
        sub = W.ssd_heads(case, heads)
        t1 = time.perf_counter()
        ssu_oracle.run_ssd(sub)
        tm = (time.perf_counter() - t1) * np.shape(case["x"])[1] / len(heads)
        result["cpu_baseline"] = {"value": round(flops / tm / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "2 of the 128 heads (heads are independent), scaled to all "
                                            "heads: %.1f s per call; single-threaded token-by-token C oracle"
                                            % tm}
    print(json.dumps(result), flush=True)


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
    for _ in range(args.warmup):
        launch(handle)
    torch.cuda.synchronize(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        launch(handle)
    end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    event_ms = start.elapsed_time(end) / args.steps
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
                     "kernel_us": round(event_ms * 1e3, 2)},
    }
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


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def traffic_from_counters(config):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing, for another workload, or taken on another kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    entry = c.get("workloads", {}).get(config)
    if not entry or c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_dispatch")


def cpu_baseline(case, alg_bytes, updates, reps, lp=False):
    from oracle import ssu_oracle
    ssu_oracle.default()
    if "buf_len" in case:
        run = ssu_oracle.run_replay_spec if np.ndim(case["x"]) == 4 else ssu_oracle.run_replay
        if lp:
            case = dict(case)
            case["lp"], case["lp_scale"] = ssu_oracle.mx8_quantize(
                np.asarray(case["state"], np.float32))
    else:
        run = ssu_oracle.run
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run(case)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(alg_bytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "updates_per_s": round(updates / t, 1),
            "sample": "the whole workload, one call per repetition, median of %d (%.2f s each); "
                      "single-threaded plain-C fp32 oracle incl. its NumPy wrapper" % (reps, t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=4)
    ap.add_argument("--calib-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selective state update has no cross-GPU step "
              "(sequences and heads shard with no exchange); run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

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
    is_replay = args.config in ("replay", "replay_spec", "replay_lp")
    lp = args.config == "replay_lp"
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
            d["lp"], d["lp_scale"] = ssu.mx8_quantize(d["state"])
            args_c = ssu.make_replay_lp_args(
                d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["buf_x"],
                d["buf_dt"], d["buf_B"], d["buf_len"], d["lp"], d["lp_scale"], d["z"],
                d["dt_bias"], case.get("dt_softplus", False), d["state_batch_indices"],
                case.get("pad_slot_id", -1), out, case.get("disable_state_update", False))
            launch = ssu.ssu_replay_lp_update
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
        dt_dtype=TORCH[case.get("dt_dtype", case["io_dtype"])])
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    for _ in range(args.warmup):
        launch(args_c, handle)
    torch.cuda.synchronize(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        launch(args_c, handle)
    end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    event_ms = start.elapsed_time(end) / args.steps
    print("[bench] %d steps: %.1f us per launch (events), %.1f us per step (wall)"
          % (args.steps, event_ms * 1e3, wall / args.steps * 1e6), file=sys.stderr, flush=True)

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
                     "traffic": traffic, "kernel_us": round(event_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, alg_bytes, updates, args.cpu_reps, lp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
