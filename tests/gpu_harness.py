"""Runs a workload case (numpy, the format of oracle/ssu_oracle.py) through
the GPU library and compares it with the oracle.

Comparison (the snapshot method of the vLLM PR #50729 digest, section
"测试配套": expected values come from the untouched input, never from a second
implementation that could share a bug):
  - every slot the oracle does not write is byte-identical to the input pool;
  - written slots: fp32 state max abs error <= 1e-5; 16-bit state max abs
    error <= 2e-2 * max|ref|;
  - y: 16-bit max abs error <= 2e-2 * max|ref|; fp32 y <= 1e-5 * max(1, max|ref|)
    (a dstate-long fp32 dot product in another summation order);
  - every row of y is written (out starts as NaN).
"""
import os
import sys

import numpy as np
import torch

import workloads as W
from oracle import brute64, ssu_oracle
from workloads.device import TORCH, dev, dev_index, device_case, device_replay, host  # noqa: F401
import mamba_selective_state_amd as ssu

def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# The oracle runs whole workloads for the full-size tests: threads over
# sequences (byte-identical to one thread), at most the 16 host cores a
# one-GPU share has.
ssu_oracle.default().set_threads(max(1, min(16, os.cpu_count() or 1)))


def run_gpu(case, device="cuda:0", d=None, out=True, sync=True):
    """One call through the Python binding; returns (y, state) on the host
    (or the device tensors when sync is False)."""
    if d is None:
        d = device_case(case, device)
    o = None
    if out:
        o = torch.full(np.shape(case["x"]), float("nan"), dtype=TORCH[case["io_dtype"]],
                       device=device)
    y = ssu.selective_state_update(
        d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], z=d["z"],
        dt_bias=d["dt_bias"], dt_softplus=case.get("dt_softplus", False),
        state_batch_indices=d["state_batch_indices"], pad_slot_id=case.get("pad_slot_id", -1),
        out=o, disable_state_update=case.get("disable_state_update", False),
        dst_state_batch_indices=d["dst_state_batch_indices"], cu_seqlens=d["cu_seqlens"],
        num_accepted_tokens=d["num_accepted_tokens"])
    if out:
        assert y is o
    if not sync:
        return y, d
    torch.cuda.synchronize()
    return host(y, case["io_dtype"]), host(d["state"], case["state_dtype"])


def tol_state(sd, ref):
    if sd == "f32":
        return 1e-5
    return 2e-2 * max(float(np.abs(ref).max()), 1e-30)


def tol_y(io, ref):
    m = float(np.abs(ref).max()) if ref.size else 0.0
    if io == "f32":
        return 1e-5 * max(1.0, m)
    return 2e-2 * max(m, 1e-30)


def compare(case, y, state, ref, name=""):
    """Asserts the GPU result (y, state) matches the oracle's `ref`; returns
    the largest errors."""
    sd, io = case["state_dtype"], case["io_dtype"]
    written = ref["written"]
    assert np.array_equal(state[~written], case["state"][~written]), \
        "%s: a slot the oracle leaves alone changed" % name
    stats = {}
    if written.any():
        g = brute64.to_f64(state[written], sd)
        r = brute64.to_f64(ref["state"][written], sd)
        err = float(np.abs(g - r).max())
        stats["state_err"], stats["state_tol"] = err, tol_state(sd, r)
        assert err <= stats["state_tol"], "%s: state error %g > %g" % (name, err, stats["state_tol"])
    if np.size(y):
        gy = brute64.to_f64(y, io)
        ry = brute64.to_f64(ref["y"], io)
        assert not np.isnan(gy).any(), "%s: a row of y was not written" % name
        err = float(np.abs(gy - ry).max())
        stats["y_err"], stats["y_tol"] = err, tol_y(io, ry)
        assert err <= stats["y_tol"], "%s: y error %g > %g" % (name, err, stats["y_tol"])
    return stats


def compare_full(case, ref, y_dev, state_dev, snap_dev, name="", chunk=32):
    """compare() for full-size cases, every sequence: untouched slots
    byte-identical on the device, written slots and y against the oracle's
    whole result, copied back `chunk` slots at a time."""
    sd, io = case["state_dtype"], case["io_dtype"]
    device = state_dev.device
    written = ref["written"]
    idx_u = torch.from_numpy(np.flatnonzero(~written)).to(device)
    assert torch.equal(state_dev[idx_u], snap_dev[idx_u]), \
        "%s: a slot the oracle leaves alone changed" % name
    ws = np.flatnonzero(written)
    stats = {"slots_written": float(ws.size)}
    if ws.size:
        rmax, err = 0.0, 0.0
        for i in range(0, ws.size, chunk):
            r = brute64.to_f64(ref["state"][ws[i:i + chunk]], sd)
            rmax = max(rmax, float(np.abs(r).max()))
            g = host(state_dev[torch.from_numpy(ws[i:i + chunk]).to(device)], sd)
            err = max(err, float(np.abs(brute64.to_f64(g, sd) - r).max()))
        stats["state_err"] = err
        stats["state_tol"] = 1e-5 if sd == "f32" else 2e-2 * max(rmax, 1e-30)
        assert err <= stats["state_tol"], "%s: state error %g > %g" % (name, err, stats["state_tol"])
    y = host(y_dev, io)
    if y.size:
        gy = brute64.to_f64(y, io)
        ry = brute64.to_f64(ref["y"], io)
        assert not np.isnan(gy).any(), "%s: a row of y was not written" % name
        err = float(np.abs(gy - ry).max())
        stats["y_err"], stats["y_tol"] = err, tol_y(io, ry)
        assert err <= stats["y_tol"], "%s: y error %g > %g" % (name, err, stats["y_tol"])
    return stats


def check(case, name, device="cuda:0"):
    """Oracle first (it also refuses out-of-range or aliased slots, so no
    such input reaches the GPU), then the GPU, then the comparison."""
    ref = ssu_oracle.run(case)
    say("[gpu] %s: launching" % name)
    y, state = run_gpu(case, device)
    stats = compare(case, y, state, ref, name)
    say("[gpu] %s: ok %s" % (name, {k: "%.3g" % v for k, v in stats.items()}))
    return stats


# ---------------------------------------------------------------- sampling

def seq_spans(case):
    """[(first row, length)] per sequence."""
    x = np.asarray(case["x"])
    cu = case.get("cu_seqlens")
    if cu is not None:
        cu = np.asarray(cu, np.int64)
        return [(int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(cu.size - 1)]
    if x.ndim == 4:
        return [(b * x.shape[1], x.shape[1]) for b in range(x.shape[0])]
    return [(r, 1) for r in range(x.shape[0])]


def written_slots(case):
    """The oracle's written-slot mask for a case, computed on a copy shrunk to
    one head, one dim row and dstate 16 (slot rules do not depend on them)."""
    x = np.asarray(case["x"])
    slots = np.shape(case["state"])[0]
    lead = x.shape[:-2]
    per_head = np.ndim(case["dt"]) == x.ndim - 1
    shadow = dict(case)
    shadow.update(
        state=np.zeros((slots, 1, 1, 16), np.float32), state_dtype="f32", io_dtype="f32",
        dt_dtype="f32", x=np.zeros(lead + (1, 1), np.float32),
        dt=np.zeros(lead + ((1,) if per_head else (1, 1)), np.float32),
        A=np.zeros(1, np.float32), B=np.zeros(lead + (1, 16), np.float32),
        C=np.zeros(lead + (1, 16), np.float32), z=None, D=None, dt_bias=None)
    return ssu_oracle.run(shadow)["written"]


def subcase(case, seqs):
    """The case restricted to sequences `seqs`, with a compact pool. Returns
    (sub, rows, slots): the original rows and slots of the sub-case's rows and
    pool entries. The pad id becomes -1 in the sub-case."""
    x = np.asarray(case["x"])
    dense = x.ndim == 4
    spans = seq_spans(case)
    rows = np.concatenate([np.arange(spans[b][0], spans[b][0] + spans[b][1]) for b in seqs]
                          ).astype(np.int64) if len(seqs) else np.zeros(0, np.int64)
    lens = np.array([spans[b][1] for b in seqs], np.int64)
    pad = int(case.get("pad_slot_id", -1))

    def rowsel(a):
        a = np.asarray(a)
        if dense:
            return a[np.asarray(seqs)]
        return a[rows]

    sub = dict(case)
    for k in ("x", "dt", "B", "C", "z"):
        if case.get(k) is not None:
            sub[k] = rowsel(case[k])
    if case.get("cu_seqlens") is not None:
        sub["cu_seqlens"] = np.concatenate([[0], np.cumsum(lens)]).astype(
            np.asarray(case["cu_seqlens"]).dtype)
    if case.get("num_accepted_tokens") is not None:
        sub["num_accepted_tokens"] = np.asarray(case["num_accepted_tokens"])[np.asarray(seqs)]
    tabs = {}
    for k in ("state_batch_indices", "dst_state_batch_indices"):
        t = case.get(k)
        if t is None:
            tabs[k] = None
            continue
        t = np.asarray(t)
        if t.ndim == 1:
            tabs[k] = t[rows] if not dense else t.reshape(x.shape[0], -1)[seqs].ravel()
        else:
            tabs[k] = t[np.asarray(seqs)]
    if tabs["state_batch_indices"] is None:
        # without tables the slot is the sequence index: make it explicit
        base = np.asarray(seqs, np.int64)
        if dense or case.get("cu_seqlens") is not None:
            tabs["state_batch_indices"] = np.repeat(base[:, None], int(max(lens.max(), 1)),
                                                    axis=1) if len(seqs) else base[:, None]
        else:
            tabs["state_batch_indices"] = base
    used = np.concatenate([np.asarray(v).ravel() for v in tabs.values() if v is not None])
    used = np.unique(used[used != pad])
    remap = {int(s): i for i, s in enumerate(used)}
    for k, t in tabs.items():
        if t is None:
            sub[k] = None
            continue
        m = np.vectorize(lambda s: -1 if s == pad else remap[int(s)], otypes=[np.int64])(t)
        sub[k] = m.astype(np.asarray(t).dtype if np.asarray(t).dtype != np.uint64 else np.int64)
    sub["pad_slot_id"] = -1
    sub["state"] = np.asarray(case["state"])[used]
    return sub, rows, used


# ---------------------------------------------------------------- ReplaySSM

def run_gpu_replay(case, d=None, device="cuda:0"):
    """One ReplaySSM step (the speculative one for a 4-D x) through the
    binding; returns host copies of y, the checkpoint pool and the three
    buffers."""
    if d is None:
        d = device_replay(case, device)
    o = torch.full(np.shape(case["x"]), float("nan"), dtype=TORCH[case["io_dtype"]],
                   device=device)
    fn = ssu.replay_spec_selective_state_update if np.ndim(case["x"]) == 4 else \
        ssu.replay_selective_state_update
    y = fn(
        d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["buf_x"], d["buf_dt"],
        d["buf_B"], d["buf_len"], z=d["z"], dt_bias=d["dt_bias"],
        dt_softplus=case.get("dt_softplus", False), state_batch_indices=d["state_batch_indices"],
        pad_slot_id=case.get("pad_slot_id", -1), out=o,
        disable_state_update=case.get("disable_state_update", False))
    assert y is o
    torch.cuda.synchronize()
    io, dtd = case["io_dtype"], case.get("dt_dtype", case["io_dtype"])
    return {"y": host(y, io), "state": host(d["state"], case["state_dtype"]),
            "buf_x": host(d["buf_x"], io), "buf_dt": host(d["buf_dt"], dtd),
            "buf_B": host(d["buf_B"], io)}


def compare_replay(case, got, ref, name=""):
    """The checkpoint pool as compare() checks a pool; the buffers bit for
    bit (they hold raw copies of inputs)."""
    stats = compare(case, got["y"], got["state"], ref, name)
    for k in ("buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(got[k], ref[k]), "%s: %s differs from the oracle" % (name, k)
    return stats


def oracle_replay(case):
    """The oracle's one-token or speculative replay step, by x's rank."""
    if np.ndim(case["x"]) == 4:
        return ssu_oracle.run_replay_spec(case)
    return ssu_oracle.run_replay(case)


def check_replay(case, name, device="cuda:0"):
    ref = oracle_replay(case)
    say("[gpu] %s: launching" % name)
    got = run_gpu_replay(case, device=device)
    stats = compare_replay(case, got, ref, name)
    say("[gpu] %s: ok %s" % (name, {k: "%.3g" % v for k, v in stats.items()}))
    return stats


def replay_subcase(case, seqs):
    """The replay case restricted to sequences `seqs` with a compact pool and
    buffers; returns (sub, slots) with the original slots of the pool
    entries (pad rows keep the pad id, -1 in the sub-case)."""
    seqs = np.asarray(seqs)
    pad = int(case.get("pad_slot_id", -1))
    tab = np.asarray(case["state_batch_indices"])[seqs]
    used = np.unique(tab[tab != pad])
    remap = {int(s): i for i, s in enumerate(used)}
    sub = dict(case)
    for k in ("x", "dt", "B", "C", "z"):
        if case.get(k) is not None:
            sub[k] = np.asarray(case[k])[seqs]
    sub["state_batch_indices"] = np.array([-1 if s == pad else remap[int(s)] for s in tab],
                                          np.int64)
    sub["pad_slot_id"] = -1
    sub["buf_len"] = np.asarray(case["buf_len"])[seqs]
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        sub[k] = np.asarray(case[k])[used]
    return sub, used


# ---------------------------------------------------------------- MX read copies

def quantizers(case):
    """The oracle's (quantize, dequantize) pair for the case's copy format."""
    if case.get("lp_format", "mx8") == "mx4":
        return ssu_oracle.mx4_quantize, ssu_oracle.mx4_dequantize
    return ssu_oracle.mx8_quantize, ssu_oracle.mx8_dequantize


def with_copy(case, source=None, fmt="mx8"):
    """The case with an MXFP8 (fmt "mx8") or MXFP4 ("mx4") read copy of
    `source` (default: its own pool), made by the oracle's quantizer."""
    c = dict(case, lp_format=fmt)
    c["lp"], c["lp_scale"] = quantizers(c)[0](
        np.asarray(case["state"] if source is None else source, np.float32))
    return c


def device_replay_lp(case, device="cuda:0"):
    d = device_replay(case, device)
    d["lp"] = torch.from_numpy(np.ascontiguousarray(case["lp"])).to(device)
    d["lp_scale"] = torch.from_numpy(np.ascontiguousarray(case["lp_scale"])).to(device)
    return d


def run_gpu_replay_lp(case, d=None, device="cuda:0"):
    """One ReplaySSM step with the read copy through the binding; returns host
    copies of y, the pool, the buffers and the copy."""
    if d is None:
        d = device_replay_lp(case, device)
    o = torch.full(np.shape(case["x"]), float("nan"), dtype=TORCH[case["io_dtype"]],
                   device=device)
    step = (ssu.replay_mx4_selective_state_update if case.get("lp_format") == "mx4"
            else ssu.replay_lp_selective_state_update)
    y = step(
        d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["buf_x"], d["buf_dt"],
        d["buf_B"], d["buf_len"], d["lp"], d["lp_scale"], z=d["z"], dt_bias=d["dt_bias"],
        dt_softplus=case.get("dt_softplus", False), state_batch_indices=d["state_batch_indices"],
        pad_slot_id=case.get("pad_slot_id", -1), out=o,
        disable_state_update=case.get("disable_state_update", False))
    assert y is o
    torch.cuda.synchronize()
    io, dtd = case["io_dtype"], case.get("dt_dtype", case["io_dtype"])
    return {"y": host(y, io), "state": host(d["state"], "f32"), "buf_x": host(d["buf_x"], io),
            "buf_dt": host(d["buf_dt"], dtd), "buf_B": host(d["buf_B"], io),
            "lp": d["lp"].cpu().numpy(), "lp_scale": d["lp_scale"].cpu().numpy()}


def compare_copy(case, got, ref, name=""):
    """The read copy: slots the oracle does not write keep their bytes; a
    written slot's copy is, byte for byte, the quantization of the state the
    GPU stored (the codes are decided on the same fp32 values), and within one
    element step of the oracle's copy (its state differs by rounding order)."""
    written = ref["written"]
    for k in ("lp", "lp_scale"):
        assert np.array_equal(got[k][~written], np.asarray(case[k])[~written]), \
            "%s: %s of a slot the oracle leaves alone changed" % (name, k)
    if not written.any():
        return 0
    quantize, dequantize = quantizers(case)
    codes, scales = quantize(got["state"][written])
    assert np.array_equal(got["lp_scale"][written], scales), "%s: scale bytes" % name
    assert np.array_equal(got["lp"][written], codes), "%s: code bytes" % name
    g = dequantize(got["lp"][written], got["lp_scale"][written]).astype(np.float64)
    r = dequantize(ref["lp"][written], ref["lp_scale"][written]).astype(np.float64)
    # the block scale X = 2^(byte - 127) of every element
    sc = np.repeat(np.ldexp(1.0, ref["lp_scale"][written].astype(np.int64) - 127), 32, axis=-1)
    if case.get("lp_format") == "mx4":
        # one E2M1 step: at most |v| / 2 for a normal value, X / 2 below 1;
        # a block whose largest value crossed a power of two between the two
        # states takes the other scale: X more
        assert (np.abs(g - r) <= np.abs(r) / 2 + sc * 1.5001).all(), \
            "%s: copy more than one E2M1 step from the oracle's" % name
    else:
        # one E4M3 step: |v| / 8 for a normal value, 2^-9 X for a subnormal
        assert (np.abs(g - r) <= np.abs(r) / 8 + sc * 2.0 ** -9 * 1.0001).all(), \
            "%s: copy more than one E4M3 step from the oracle's" % name
    return int((got["lp"][written] != ref["lp"][written]).sum())


def check_replay_lp(case, name, device="cuda:0"):
    ref = ssu_oracle.run_replay(case)
    say("[gpu] %s: launching" % name)
    got = run_gpu_replay_lp(case, device=device)
    stats = compare_replay(case, got, ref, name)
    stats["copy_mismatch"] = compare_copy(case, got, ref, name)
    say("[gpu] %s: ok %s" % (name, {k: "%.3g" % v for k, v in stats.items()}))
    return stats
