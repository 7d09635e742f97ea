"""Seeded synthetic inputs for the selective state update.

Data only: this module draws random inputs and slot tables and holds none of
the method's arithmetic. Both the CPU oracle and the GPU path take their inputs
from here, as NumPy arrays in the format documented in oracle/ssu_oracle.py
(16-bit floats are carried as uint16 bit patterns; PyTorch's CPU casts round
float32 to them, nearest-even).

The shapes follow the pages' workloads:
  one_token_tiny  the MATE page's minimal example (batch 2, heads 8, dim 8,
                  dstate 128, groups 2, 8 slots, fp16 state of zeros)
  decode          one-token decode of a Mamba-2 layer (heads 128, dim 64,
                  dstate 128, groups 8): a 4 MiB fp32 state per sequence, the
                  size the ReplaySSM article quotes, at batch 256
  decode_pad      the same layer with bf16 state at batch 1024, 5% pad rows,
                  output into a caller-provided buffer
  mtp             MTP packed decode, 64 sequences x 7 steps, 2-D read table and
                  write table = read + rows, num_accepted_tokens ~ U{1..7}
  varlen          512 sequences of lengths U{0..8}, flat tables, heads 64,
                  groups 1, fp16 state, per-head dt, z gate and D
Every builder takes keyword overrides so tests can shrink a workload.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = ["to_storage", "one_token_tiny", "decode", "decode_pad", "mtp", "varlen",
           "Strided", "BUILDERS"]

_CHUNK = 1 << 24
_THREADS = min(16, os.cpu_count() or 1)


class Strided:
    """A strided view of a 1-D integer table: entry (i, j) is
    base[i * strides[0] + j * strides[1]]."""

    def __init__(self, base, shape, strides):
        self.base = np.asarray(base)
        self.shape = tuple(shape)
        self.strides = tuple(strides)


def to_storage(a, dtype):
    """float32 array -> storage of `dtype` ('f32' | 'f16' | 'bf16')."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    out = np.empty(a.shape, dtype=np.uint16)
    fa, fo = a.reshape(-1), out.reshape(-1)
    for i in range(0, fa.size, _CHUNK):
        t = torch.from_numpy(fa[i:i + _CHUNK]).to(tdt)
        fo[i:i + _CHUNK] = t.view(torch.int16).numpy().view(np.uint16)
    return out


def _normal(rng, shape, dtype):
    """N(0,1) stored in `dtype`. Chunk i is drawn from stream i spawned from
    one seed taken off `rng`, so the values do not depend on how many threads
    draw them."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    starts = list(range(0, n, _CHUNK))
    streams = np.random.SeedSequence(int(rng.integers(1 << 63))).spawn(len(starts))

    def fill(k):
        i = starts[k]
        m = min(_CHUNK, n - i)
        g = np.random.Generator(np.random.PCG64(streams[k]))
        out[i:i + m] = to_storage(g.standard_normal(m, dtype=np.float32), dtype)

    if len(starts) <= 1:
        for k in range(len(starts)):
            fill(k)
    else:
        with ThreadPoolExecutor(min(_THREADS, len(starts))) as ex:
            list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


def _pattern(shape, dtype):
    """Deterministic filler for slots no row reads: the values
    ((k % 251) - 125) / 64 for the flat element index k, so a stray store
    cannot go unnoticed. Built by tiling one period."""
    n = int(np.prod(shape))
    period = to_storage((np.arange(251, dtype=np.float32) - 125.0) / 64.0, dtype)
    return np.resize(period, n).reshape(shape)


def _pool(rng, slots, H, P, N, dtype, live_slots=None):
    """State pool: N(0,1) on `live_slots` (all slots if None), the filler
    pattern elsewhere."""
    if live_slots is None:
        return _normal(rng, (slots, H, P, N), dtype)
    pool = _pattern((slots, H, P, N), dtype)
    live = np.unique(np.asarray(live_slots))
    live = live[(live >= 0) & (live < slots)]
    if live.size:
        pool[live] = _normal(rng, (live.size, H, P, N), dtype)
    return pool


def _layer(rng, R, H, P, N, G, io="bf16", dt_dtype="bf16", dt_per_head=False, z=True, D=True,
           softplus=True, dt_dist="normal"):
    """Per-row inputs of one Mamba-2 layer: x, dt, B, C, z, and the per-head
    A, D, dt_bias (fp32). dt_bias = log(expm1(u)) with u log-uniform on
    [1e-3, 1e-1], so softplus(dt_bias) = u, p. dt itself ~ N(0,1), or U[0,0.1)
    for dt_dist='small' (the MATE example)."""
    c = {"io_dtype": io, "dt_dtype": dt_dtype}
    c["x"] = _normal(rng, (R, H, P), io)
    dshape = (R, H) if dt_per_head else (R, H, P)
    if dt_dist == "small":
        c["dt"] = to_storage(rng.random(dshape, dtype=np.float32) * np.float32(0.1), dt_dtype)
    else:
        c["dt"] = _normal(rng, dshape, dt_dtype)
    c["A"] = (-np.exp(rng.uniform(0.0, 4.0, H))).astype(np.float32)
    c["B"] = _normal(rng, (R, G, N), io)
    c["C"] = _normal(rng, (R, G, N), io)
    c["z"] = _normal(rng, (R, H, P), io) if z else None
    c["D"] = rng.standard_normal(H).astype(np.float32) if D else None
    if softplus:
        u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H))
        c["dt_bias"] = np.log(np.expm1(u)).astype(np.float32)
    else:
        c["dt_bias"] = None
    c["dt_softplus"] = bool(softplus)
    return c


def one_token_tiny(seed=0, tables=False):
    """The MATE page's minimal example: batch 2, heads 8, dim 8, dstate 128,
    groups 2, 8 slots; fp16 state of zeros; x, B, C bf16 N(0,1); dt fp32
    U[0, 0.1); A = -U[0, 1); no D, z or dt_bias. Without tables each sequence
    uses slot b; with tables, state_batch_indices = dst = [0, 1]."""
    rng = np.random.default_rng(seed)
    batch, H, P, N, G, slots = 2, 8, 8, 128, 2, 8
    c = {"state_dtype": "f16", "io_dtype": "bf16", "dt_dtype": "f32"}
    c["state"] = np.zeros((slots, H, P, N), dtype=np.uint16)
    c["x"] = _normal(rng, (batch, H, P), "bf16")
    c["dt"] = rng.random((batch, H, P), dtype=np.float32) * np.float32(0.1)
    c["A"] = (-rng.random(H, dtype=np.float32)).astype(np.float32)
    c["B"] = _normal(rng, (batch, G, N), "bf16")
    c["C"] = _normal(rng, (batch, G, N), "bf16")
    c.update(D=None, z=None, dt_bias=None, dt_softplus=False, pad_slot_id=-1,
             disable_state_update=False, cu_seqlens=None, num_accepted_tokens=None)
    if tables:
        idx = np.array([0, 1], dtype=np.int32)
        c["state_batch_indices"] = idx
        c["dst_state_batch_indices"] = idx.copy()
    else:
        c["state_batch_indices"] = c["dst_state_batch_indices"] = None
    return c


def decode(seed=1, batch=256, heads=128, dim=64, dstate=128, groups=8, slots=512,
           state_dtype="f32", io="bf16", index_dtype=np.int32, fill_unread=True):
    """One-token decode of a Mamba-2 layer. Read = write slots are the first
    `batch` entries of a random permutation of the pool (distinct slots).
    Slots no row reads hold the deterministic filler when fill_unread."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(slots)[:batch].astype(index_dtype)
    c = {"state_dtype": state_dtype}
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype,
                       perm if fill_unread else None)
    c.update(_layer(rng, batch, heads, dim, dstate, groups, io=io, dt_dtype=io))
    c.update(state_batch_indices=perm, dst_state_batch_indices=perm.copy(), pad_slot_id=-1,
             disable_state_update=False, cu_seqlens=None, num_accepted_tokens=None)
    return c


def decode_pad(seed=2, batch=1024, heads=128, dim=64, dstate=128, groups=8, slots=2048,
               state_dtype="bf16", io="bf16", pad_frac=0.05, pad_slot_id=0,
               index_dtype=np.int32):
    """Decode with pad rows: round(pad_frac * batch) rows read and write
    pad_slot_id; live rows use distinct slots other than the pad id. With
    pad_slot_id = 0, slot 0 holds non-zero data that must stay as it is."""
    rng = np.random.default_rng(seed)
    npad = int(round(pad_frac * batch))
    pad_rows = rng.choice(batch, size=npad, replace=False)
    cand = np.arange(slots)
    cand = cand[cand != pad_slot_id]
    live = rng.permutation(cand)[:batch - npad]
    idx = np.empty(batch, dtype=np.int64)
    mask = np.zeros(batch, dtype=bool)
    mask[pad_rows] = True
    idx[mask] = pad_slot_id
    idx[~mask] = live
    idx = idx.astype(index_dtype)
    c = {"state_dtype": state_dtype}
    live_and_pad = np.concatenate([live, [pad_slot_id]]) if pad_slot_id >= 0 else live
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype, live_and_pad)
    c.update(_layer(rng, batch, heads, dim, dstate, groups, io=io, dt_dtype=io))
    c.update(state_batch_indices=idx, dst_state_batch_indices=idx.copy(),
             pad_slot_id=pad_slot_id, disable_state_update=False, cu_seqlens=None,
             num_accepted_tokens=None, pad_rows=np.sort(pad_rows))
    return c


def mtp(seed=3, nseq=64, steps=7, heads=128, dim=64, dstate=128, groups=8,
        state_dtype="f32", io="bf16", pad_slot_id=0, index_dtype=np.int32,
        meta_dtype=np.int32):
    """MTP packed decode, as in the MATE page's MTP example: rows = nseq *
    steps; read table arange(rows).view(nseq, steps), write table = read +
    rows; cu_seqlens = arange(0, rows + 1, steps); num_accepted_tokens drawn
    from U{1..steps}. The pool has 2 * rows slots."""
    rng = np.random.default_rng(seed)
    rows = nseq * steps
    slots = 2 * rows
    read = np.arange(rows, dtype=index_dtype).reshape(nseq, steps)
    write = (read + rows).astype(index_dtype)
    acc = rng.integers(1, steps + 1, nseq).astype(meta_dtype)
    c = {"state_dtype": state_dtype}
    read_slots = read[np.arange(nseq), np.maximum(acc.astype(np.int64) - 1, 0)]
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype, read_slots)
    c.update(_layer(rng, rows, heads, dim, dstate, groups, io=io, dt_dtype=io))
    c.update(state_batch_indices=read, dst_state_batch_indices=write, pad_slot_id=pad_slot_id,
             disable_state_update=False,
             cu_seqlens=np.arange(0, rows + 1, steps).astype(meta_dtype),
             num_accepted_tokens=acc)
    return c


def varlen(seed=4, nseq=512, max_len=8, heads=64, dim=64, dstate=128, groups=1,
           state_dtype="f16", io="bf16", dst=True, disable=False, index_dtype=np.int32,
           meta_dtype=np.int32, lengths=None):
    """Variable-length packed decode: lengths ~ U{0..max_len} (empty sequences
    included), flat [rows] tables (row-indexed), per-head dt, z gate and D.
    The read table takes R distinct slots of a 2R-slot pool, the write table
    the other R. dst=False omits the write table (stores go to the read
    table's entries); disable=True sets disable_state_update."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(0, max_len + 1, nseq)
    lengths = np.asarray(lengths, dtype=np.int64)
    rows = int(lengths.sum())
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(meta_dtype)
    slots = max(2 * rows, 1)
    perm = rng.permutation(slots).astype(index_dtype)
    read, write = perm[:rows], perm[rows:2 * rows]
    starts = cu[:-1].astype(np.int64)[lengths > 0]
    c = {"state_dtype": state_dtype}
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype, read[starts])
    c.update(_layer(rng, rows, heads, dim, dstate, groups, io=io, dt_dtype=io, dt_per_head=True))
    c.update(state_batch_indices=read, dst_state_batch_indices=write if dst else None,
             pad_slot_id=-1, disable_state_update=bool(disable), cu_seqlens=cu,
             num_accepted_tokens=None)
    return c


BUILDERS = {"one_token_tiny": one_token_tiny, "decode": decode, "decode_pad": decode_pad,
            "mtp": mtp, "varlen": varlen}


def replay(seed=5, batch=256, heads=128, dim=64, dstate=128, groups=8, slots=512, L=16,
           state_dtype="f32", io="bf16", buf_len=None, dt_per_head=False, index_dtype=np.int32,
           fill_unread=True):
    """A ReplaySSM decode step on the decode workload's layer: a checkpoint
    pool, one slot per sequence (the first `batch` of a permutation), and per
    slot an input buffer of L entries (x, dt, B as earlier steps would have
    appended them, drawn like the current step's inputs). buf_len (entries
    already buffered per sequence) defaults to U{0..L-1}."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(slots)[:batch].astype(index_dtype)
    c = {"state_dtype": state_dtype}
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype,
                       perm if fill_unread else None)
    c.update(_layer(rng, batch, heads, dim, dstate, groups, io=io, dt_dtype=io,
                    dt_per_head=dt_per_head))
    c.update(state_batch_indices=perm, dst_state_batch_indices=None, pad_slot_id=-1,
             disable_state_update=False, cu_seqlens=None, num_accepted_tokens=None)
    c["L"] = int(L)
    c["buf_x"] = _normal(rng, (slots, L, heads, dim), io)
    c["buf_dt"] = _normal(rng, (slots, L, heads) if dt_per_head else (slots, L, heads, dim), io)
    c["buf_B"] = _normal(rng, (slots, L, groups, dstate), io)
    if buf_len is None:
        buf_len = rng.integers(0, L, batch)
    c["buf_len"] = np.broadcast_to(np.asarray(buf_len, dtype=np.int32), (batch,)).copy()
    return c


BUILDERS["replay"] = replay


def replay_spec(seed=6, batch=512, T=4, heads=128, dim=64, dstate=128, groups=8, slots=1024,
                L=16, state_dtype="f32", io="bf16", buf_len=None, dt_per_head=False,
                index_dtype=np.int32, fill_unread=True):
    """A ReplaySSM speculative step (T draft tokens per sequence) on the decode
    workload's layer: the replay() pool and buffers, with x, dt, z [batch, T,
    heads, dim] and B, C [batch, T, groups, dstate]. buf_len defaults to
    U{0..L-T} (the pointers a caller that folds at h + 2T > L can hold)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(slots)[:batch].astype(index_dtype)
    c = {"state_dtype": state_dtype}
    c["state"] = _pool(rng, slots, heads, dim, dstate, state_dtype,
                       perm if fill_unread else None)
    lay = _layer(rng, batch * T, heads, dim, dstate, groups, io=io, dt_dtype=io,
                 dt_per_head=dt_per_head)
    for k in ("x", "dt", "B", "C", "z"):
        if lay[k] is not None:
            lay[k] = lay[k].reshape((batch, T) + lay[k].shape[1:])
    c.update(lay)
    c.update(state_batch_indices=perm, dst_state_batch_indices=None, pad_slot_id=-1,
             disable_state_update=False, cu_seqlens=None, num_accepted_tokens=None)
    c["L"] = int(L)
    c["buf_x"] = _normal(rng, (slots, L, heads, dim), io)
    c["buf_dt"] = _normal(rng, (slots, L, heads) if dt_per_head else (slots, L, heads, dim), io)
    c["buf_B"] = _normal(rng, (slots, L, groups, dstate), io)
    if buf_len is None:
        buf_len = rng.integers(0, L - T + 1, batch)
    c["buf_len"] = np.broadcast_to(np.asarray(buf_len, dtype=np.int32), (batch,)).copy()
    return c


BUILDERS["replay_spec"] = replay_spec


def spec_snapshots(seed=7, batch=512, T=4, heads=128, dim=64, dstate=128, groups=8,
                   state_dtype="f32", io="bf16", index_dtype=np.int32):
    """The speculative step done the way ReplaySSM replaces (its article,
    section "三个瓶颈其实来自同一个动作": one full state snapshot per draft
    token): T draft tokens per sequence through the plain multi-token update
    ([batch, T, ...] dense form), read table [batch, T] naming the sequence's
    committed slot (read at position 0), write table [batch, T] naming T
    snapshot slots per sequence. Pool: batch committed slots (N(0,1)) plus
    batch*T snapshot slots (zeros)."""
    rng = np.random.default_rng(seed)
    slots = batch * (1 + T)
    c = {"state_dtype": state_dtype}
    pool = np.zeros((slots, heads, dim, dstate),
                    dtype=np.float32 if state_dtype == "f32" else np.uint16)
    pool[:batch] = _normal(rng, (batch, heads, dim, dstate), state_dtype)
    c["state"] = pool
    lay = _layer(rng, batch * T, heads, dim, dstate, groups, io=io, dt_dtype=io)
    for k in ("x", "dt", "B", "C", "z"):
        lay[k] = lay[k].reshape((batch, T) + lay[k].shape[1:])
    c.update(lay)
    read = np.repeat(np.arange(batch, dtype=index_dtype)[:, None], T, axis=1)
    write = (batch + np.arange(batch * T, dtype=index_dtype)).reshape(batch, T)
    c.update(state_batch_indices=read, dst_state_batch_indices=write, pad_slot_id=-1,
             disable_state_update=False, cu_seqlens=None, num_accepted_tokens=None)
    return c


BUILDERS["spec_snapshots"] = spec_snapshots


# ------------------------------------------------------------ state copies

def memmove_rows(rows=128, row_bytes=32 * 1024, shift=16, direction="left", seed=8):
    """Rows of a byte buffer, each copied onto itself shifted by `shift`
    bytes: 'left' moves row[shift:] to row[:-shift] (the vLLM PR #50729
    regression test: 128 rows x 32 KiB, shift 16, a mod-251 pattern), 'right'
    the mirror case, 'apart' copies row i to row rows + i. Returns dict(buf
    uint8, src_off, dst_off, sizes)."""
    n_rows = rows * (2 if direction == "apart" else 1)
    buf = ((np.arange(n_rows * row_bytes, dtype=np.int64) + seed) % 251).astype(np.uint8)
    base = np.arange(rows, dtype=np.int64) * row_bytes
    size = row_bytes - shift
    if direction == "left":
        src, dst = base + shift, base
    elif direction == "right":
        src, dst = base, base + shift
    else:
        src, dst = base, base + rows * row_bytes
        size = row_bytes
    return {"buf": buf, "src_off": src, "dst_off": dst, "sizes": np.full(rows, size, np.int64)}


def conv_shift(seed=9, requests=6144, width=4, inner=8192, dtype=np.float16, layout="SD",
               same_frac=0.5, max_bias=3):
    """Convolution-state shifts on a pool of 2 * requests blocks ([blocks, W,
    inner] for 'SD', [blocks, inner, W] for 'DS'), N(0,1) values stored in
    `dtype` (for floats) or random bits. Request r reads block 2r and writes
    block 2r (a shift inside one block) for a `same_frac` share of the
    requests, else block 2r + 1; bias ~ U{1..max_bias} (accepted-token biases
    1..3 in the vLLM tests)."""
    rng = np.random.default_rng(seed)
    blocks = 2 * requests
    shape = (blocks, width, inner) if layout == "SD" else (blocks, inner, width)
    dt = np.dtype(dtype)
    if dt.kind == "f":
        pool = rng.standard_normal(shape, dtype=np.float32).astype(dt)
    else:
        pool = rng.integers(0, 256, size=shape + (dt.itemsize,), dtype=np.uint8).view(dt)[..., 0]
    src = 2 * np.arange(requests, dtype=np.int64)
    same = rng.random(requests) < same_frac
    dst = np.where(same, src, src + 1)
    bias = rng.integers(1, max_bias + 1, requests).astype(np.int64)
    return {"pool": pool, "layout": layout, "src_blk": src, "dst_blk": dst, "bias": bias}


BUILDERS["memmove_rows"] = memmove_rows
BUILDERS["conv_shift"] = conv_shift


# ------------------------------------------------------------ SSD prefill

def ssd(seed=10, lengths=(700, 256, 1, 513, 1200), heads=8, dim=64, dstate=128, groups=2,
        chunk_size=256, io="bf16", state_dtype="f32", dt_dtype="f32", initial_states=True,
        dt_limit=(0.0, float("inf")), z=True, D=True, softplus=True):
    """A packed variable-length prefill: sequences of the given lengths,
    each split from its start into chunks of chunk_size tokens (the last one
    partial), x / z [T, H, P] and B / C [T, G, N] ~ N(0,1) in the io dtype,
    dt [T, H] ~ N(0,1) in dt_dtype with the decode layer's dt_bias (softplus
    on) and A, optional initial states ~ N(0,1) in the state dtype. cu_seqlens,
    cu_chunk_seqlens, seq_idx and last_chunk_indices follow from the lengths."""
    rng = np.random.default_rng(seed)
    lengths = [int(n) for n in lengths]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    chunks, seq, last = [0], [], []
    for b, n in enumerate(lengths):
        start = int(cu[b])
        for off in range(0, max(n, 1), chunk_size):
            if n == 0:
                break
            chunks.append(start + min(off + chunk_size, n))
            seq.append(b)
        last.append(len(seq) - 1)
    c = {"io_dtype": io, "dt_dtype": dt_dtype, "state_dtype": state_dtype,
         "chunk_size": int(chunk_size), "dt_softplus": bool(softplus), "dt_limit": tuple(dt_limit)}
    c["x"] = _normal(rng, (T, heads, dim), io)
    c["dt"] = _normal(rng, (T, heads), dt_dtype)
    c["A"] = (-np.exp(rng.uniform(0.0, 4.0, heads))).astype(np.float32)
    c["B"] = _normal(rng, (T, groups, dstate), io)
    c["C"] = _normal(rng, (T, groups, dstate), io)
    c["z"] = _normal(rng, (T, heads, dim), io) if z else None
    c["D"] = rng.standard_normal(heads).astype(np.float32) if D else None
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), heads))
    c["dt_bias"] = np.log(np.expm1(u)).astype(np.float32) if softplus else None
    c["initial_states"] = _normal(rng, (len(lengths), heads, dim, dstate), state_dtype) \
        if initial_states else None
    c["cu_seqlens"] = cu
    c["cu_chunk_seqlens"] = np.asarray(chunks, np.int64)
    c["seq_idx"] = np.asarray(seq, np.int64)
    c["last_chunk_indices"] = np.asarray(last, np.int64)
    return c


BUILDERS["ssd"] = ssd


def ssd_bench(seed=11, nseq=8, heads=128, dim=64, dstate=128, groups=8, chunk_size=256,
              io="bf16", state_dtype="f32"):
    """The prefill benchmark: nseq sequences of lengths ~ U{512..4096} (a
    variable-length prefill batch of the decode workload's layer), chunk
    size 256, initial states (prefix-cached continuations)."""
    rng = np.random.default_rng(seed)
    lengths = tuple(int(v) for v in rng.integers(512, 4097, nseq))
    return ssd(seed=seed + 1, lengths=lengths, heads=heads, dim=dim, dstate=dstate, groups=groups,
               chunk_size=chunk_size, io=io, state_dtype=state_dtype, initial_states=True)


def ssd_heads(case, heads):
    """The prefill case restricted to the given heads (heads are independent
    in the recurrence): each kept head gets its own group, the one it reads
    in the full case."""
    heads = np.asarray(heads)
    H = np.shape(case["x"])[1]
    G = np.shape(case["B"])[1]
    groups = heads // (H // G)
    sub = dict(case)
    sub["x"] = np.ascontiguousarray(np.asarray(case["x"])[:, heads])
    sub["dt"] = np.ascontiguousarray(np.asarray(case["dt"])[:, heads])
    if case.get("z") is not None:
        sub["z"] = np.ascontiguousarray(np.asarray(case["z"])[:, heads])
    for k in ("A", "D", "dt_bias"):
        if case.get(k) is not None:
            sub[k] = np.ascontiguousarray(np.asarray(case[k])[heads])
    for k in ("B", "C"):
        sub[k] = np.ascontiguousarray(np.asarray(case[k])[:, groups])
    if case.get("initial_states") is not None:
        sub["initial_states"] = np.ascontiguousarray(np.asarray(case["initial_states"])[:, heads])
    return sub


BUILDERS["ssd_bench"] = ssd_bench
