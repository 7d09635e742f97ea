"""ctypes front end of the CPU oracle (oracle/ssu_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package entry's smoke check and
the benchmark's CPU-baseline leg are the only callers. The GPU package never
imports this module.

Input format (numpy, shared with the seeded workload generators): a dict with
  state        [slots, H, P, N]; float32, or uint16 bit patterns for f16/bf16
  state_dtype  'f32' | 'f16' | 'bf16'
  io_dtype     dtype of x, B, C, z and of the output y
  x            [R, H, P] (packed or one token per sequence) or [Bt, T, H, P]
  dt           like x, or without the last axis (one value per head)
  dt_dtype     'f32' or the io dtype
  A            float32 [H];  D, dt_bias: float32 [H] or None
  B, C         [R, G, N] or [Bt, T, G, N], io dtype
  z            like x, or None
  dt_softplus, disable_state_update: bool;  pad_slot_id: int
  state_batch_indices, dst_state_batch_indices: None, an integer array
               (1-D or 2-D), or an object with .base (1-D integer array),
               .shape and .strides (element strides) describing a strided view
  cu_seqlens, num_accepted_tokens: None or integer arrays
Output: dict(y=..., state=new pool, written=bool[slots], read_slot=int64[nseq]).
"""
import ctypes
import os

import numpy as np

from . import build as _build

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ONE_TOKEN, DENSE, CU = 0, 1, 2


class _Table(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("len", ctypes.c_int64),
                ("ndim", ctypes.c_int32), ("s0", ctypes.c_int64), ("s1", ctypes.c_int64)]


class _Args(ctypes.Structure):
    _fields_ = [
        ("pool_in", ctypes.c_void_p), ("pool_out", ctypes.c_void_p),
        ("state_dtype", ctypes.c_int32),
        ("slots", ctypes.c_int64), ("H", ctypes.c_int64), ("P", ctypes.c_int64),
        ("N", ctypes.c_int64), ("G", ctypes.c_int64),
        ("R", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p),
        ("dt_dtype", ctypes.c_int32), ("dt_per_head", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("D", ctypes.c_void_p), ("z", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dt_softplus", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("steps", ctypes.c_int64),
        ("cu", ctypes.c_void_p), ("nseq", ctypes.c_int64), ("acc", ctypes.c_void_p),
        ("rtab", _Table), ("wtab", _Table),
        ("pad", ctypes.c_int64), ("disable", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("written", ctypes.c_void_p), ("read_slot", ctypes.c_void_p),
    ]


class OracleError(ValueError):
    pass


class Oracle:
    """One loaded copy of the oracle library (tests may load a modified copy)."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIB
            if (not os.path.exists(path)
                    or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
                _build.build()
        self.lib = ctypes.CDLL(path)
        self.lib.oracle_ssu.argtypes = [ctypes.POINTER(_Args), ctypes.c_char_p, ctypes.c_int]
        self.lib.oracle_ssu.restype = ctypes.c_int
        self.lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        self.lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        self.lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        self.lib.oracle_f16_to_f32.restype = ctypes.c_float
        self.lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        self.lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        self.lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        self.lib.oracle_bf16_to_f32.restype = ctypes.c_float
        self.lib.oracle_softplus.argtypes = [ctypes.c_float]
        self.lib.oracle_softplus.restype = ctypes.c_float
        self.lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib.oracle_set_threads.restype = None
        self.lib.oracle_get_threads.argtypes = []
        self.lib.oracle_get_threads.restype = ctypes.c_int

    def set_threads(self, n):
        """Threads over sequences for every later call (1: serial); the
        result is byte-identical for any count."""
        self.lib.oracle_set_threads(int(n))

    def threads(self):
        return self.lib.oracle_get_threads()

    # scalar helpers, exported for the pins
    def f32_to_f16(self, v):
        return self.lib.oracle_f32_to_f16(float(v))

    def f16_to_f32(self, b):
        return self.lib.oracle_f16_to_f32(int(b))

    def f32_to_bf16(self, v):
        return self.lib.oracle_f32_to_bf16(float(v))

    def bf16_to_f32(self, b):
        return self.lib.oracle_bf16_to_f32(int(b))

    def softplus(self, v):
        return self.lib.oracle_softplus(float(v))

    def run(self, case):
        return _run(self, case)


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def run(case, oracle=None):
    return (oracle or default()).run(case)


def _np_dtype(name):
    return np.float32 if name == "f32" else np.uint16


def _arr(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise OracleError("array of dtype %s where %s was expected" % (a.dtype, np.dtype(dtype)))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _table(t, keep):
    if t is None:
        return _Table(None, 0, 0, 0, 0)
    if hasattr(t, "base") and hasattr(t, "strides") and not isinstance(t, np.ndarray):
        base = np.ascontiguousarray(t.base, dtype=np.int64).ravel()
        keep.append(base)
        ndim = len(t.shape)
        s0 = int(t.strides[0])
        s1 = int(t.strides[1]) if ndim == 2 else 0
        return _Table(base.ctypes.data, base.size, ndim, s0, s1)
    t = np.asarray(t)
    if t.ndim not in (1, 2):
        raise OracleError("slot tables are 1-D or 2-D")
    flat = np.ascontiguousarray(t, dtype=np.int64).ravel()
    keep.append(flat)
    if t.ndim == 1:
        return _Table(flat.ctypes.data, flat.size, 1, 1, 0)
    return _Table(flat.ctypes.data, flat.size, 2, t.shape[1], 1)


def _run(oracle, case):
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    state = _arr(case["state"], _np_dtype(sd))
    slots, H, P, N = state.shape
    x = np.asarray(case["x"])
    dense = x.ndim == 4
    if dense:
        Bt, T = x.shape[:2]
        R = Bt * T
    else:
        R = x.shape[0]
    xr = _arr(x.reshape(R, H, P), _np_dtype(io))
    dt = np.asarray(case["dt"])
    dt_per_head = dt.ndim == x.ndim - 1
    dtr = _arr(dt.reshape((R, H) if dt_per_head else (R, H, P)), _np_dtype(dtd))
    Bm = np.asarray(case["B"])
    G = Bm.shape[-2]
    Br = _arr(Bm.reshape(R, G, N), _np_dtype(io))
    Cr = _arr(np.asarray(case["C"]).reshape(R, G, N), _np_dtype(io))
    z = case.get("z")
    zr = None if z is None else _arr(np.asarray(z).reshape(R, H, P), _np_dtype(io))
    A = _arr(case["A"], np.float32)
    D = case.get("D")
    D = None if D is None else _arr(D, np.float32)
    bias = case.get("dt_bias")
    bias = None if bias is None else _arr(bias, np.float32)

    cu = case.get("cu_seqlens")
    acc = case.get("num_accepted_tokens")
    keep = []
    if cu is not None:
        if dense:
            raise OracleError("cu_seqlens goes with the packed [rows, heads, dim] form")
        cu = np.ascontiguousarray(cu, dtype=np.int64)
        layout, steps, nseq = CU, 0, cu.size - 1
    elif dense:
        layout, steps, nseq = DENSE, T, Bt
    else:
        layout, steps, nseq = ONE_TOKEN, 0, R
    if acc is not None:
        acc = np.ascontiguousarray(acc, dtype=np.int64)
        if acc.size != nseq:
            raise OracleError("num_accepted_tokens must have one entry per sequence")

    pool_out = state.copy()
    out = np.zeros((R, H, P), dtype=_np_dtype(io))
    written = np.zeros(slots, dtype=np.uint8)
    read_slot = np.zeros(max(nseq, 1), dtype=np.int64)
    args = _Args()
    args.pool_in, args.pool_out = _ptr(state), _ptr(pool_out)
    args.state_dtype = DTYPES[sd]
    args.slots, args.H, args.P, args.N, args.G = slots, H, P, N, G
    args.R, args.io_dtype = R, DTYPES[io]
    args.x, args.dt = _ptr(xr), _ptr(dtr)
    args.dt_dtype, args.dt_per_head = DTYPES[dtd], int(dt_per_head)
    args.A, args.B, args.C = _ptr(A), _ptr(Br), _ptr(Cr)
    args.D, args.z, args.dt_bias = _ptr(D), _ptr(zr), _ptr(bias)
    args.dt_softplus = int(bool(case.get("dt_softplus", False)))
    args.layout, args.steps, args.nseq = layout, steps, nseq
    args.cu, args.acc = _ptr(cu), _ptr(acc)
    args.rtab = _table(case.get("state_batch_indices"), keep)
    args.wtab = _table(case.get("dst_state_batch_indices"), keep)
    args.pad = int(case.get("pad_slot_id", -1))
    args.disable = int(bool(case.get("disable_state_update", False)))
    args.out, args.written, args.read_slot = _ptr(out), _ptr(written), _ptr(read_slot)
    err = ctypes.create_string_buffer(256)
    rc = oracle.lib.oracle_ssu(ctypes.byref(args), err, 256)
    if rc:
        raise OracleError(err.value.decode())
    y = out.reshape(x.shape) if dense else out
    return {"y": y, "state": pool_out, "written": written.astype(bool),
            "read_slot": read_slot[:nseq]}


# ---------------------------------------------------------------- ReplaySSM

class _ReplayArgs(ctypes.Structure):
    _fields_ = [("base", _Args), ("L", ctypes.c_int64),
                ("bx_in", ctypes.c_void_p), ("bx_out", ctypes.c_void_p),
                ("bdt_in", ctypes.c_void_p), ("bdt_out", ctypes.c_void_p),
                ("bB_in", ctypes.c_void_p), ("bB_out", ctypes.c_void_p),
                ("buf_len", ctypes.c_void_p),
                ("lp_in", ctypes.c_void_p), ("lps_in", ctypes.c_void_p),
                ("lp_out", ctypes.c_void_p), ("lps_out", ctypes.c_void_p),
                ("lp_bits", ctypes.c_int32)]


def run_replay(case, oracle=None):
    """ReplaySSM decode step (oracle_replay in ssu_oracle.c). With "lp" and
    "lp_scale" the output-only steps read that copy of the checkpoint pool:
    MXFP8 codes [slots, H, P, N], or with lp_format "mx4" MXFP4 codes
    [slots, H, P, N / 2]; scales [slots, H, P, N / 32]. The case holds
    the one-token update's inputs (state = checkpoint pool, a 1-D slot table
    or none, no destination table) plus
      L         buffer length
      buf_x     [slots, L, H, P]        io dtype
      buf_dt    [slots, L, H, P] or [slots, L, H]  dt dtype
      buf_B     [slots, L, G, N]        io dtype
      buf_len   [batch] integer: entries in each sequence's buffer (< L)
    Returns dict(y, state, buf_x, buf_dt, buf_B, written)."""
    return _run_replay(case, oracle, spec=False)


def run_replay_spec(case, oracle=None):
    """ReplaySSM speculative step (oracle_replay_spec): as run_replay with
    x, dt, z [batch, T, H, P] (dt [batch, T, H] per head) and B, C
    [batch, T, G, N] holding T draft tokens per sequence; buf_len in [0, L].
    y has x's shape."""
    return _run_replay(case, oracle, spec=True)


def _run_replay(case, oracle, spec):
    orc = oracle or default()
    lib = orc.lib
    if not hasattr(lib, "_replay_ready"):
        for f in (lib.oracle_replay, lib.oracle_replay_spec):
            f.argtypes = [ctypes.POINTER(_ReplayArgs), ctypes.c_char_p, ctypes.c_int]
            f.restype = ctypes.c_int
        lib._replay_ready = True
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    state = _arr(case["state"], _np_dtype(sd))
    slots, H, P, N = state.shape
    x = np.asarray(case["x"])
    if x.ndim != (4 if spec else 3) or case.get("cu_seqlens") is not None or \
            case.get("num_accepted_tokens") is not None or \
            case.get("dst_state_batch_indices") is not None:
        raise OracleError("replay takes x [batch, %sheads, dim], one slot table and nothing else"
                          % ("T, " if spec else ""))
    T = x.shape[1] if spec else 1
    R = x.shape[0] * T
    xr = _arr(x.reshape(R, H, P), _np_dtype(io))
    dt = np.asarray(case["dt"])
    dt_per_head = dt.ndim == x.ndim - 1
    dtr = _arr(dt.reshape((R, H) if dt_per_head else (R, H, P)), _np_dtype(dtd))
    Bm = np.asarray(case["B"])
    G = Bm.shape[-2]
    Br = _arr(Bm.reshape(R, G, N), _np_dtype(io))
    Cr = _arr(np.asarray(case["C"]).reshape(R, G, N), _np_dtype(io))
    z = case.get("z")
    zr = None if z is None else _arr(np.asarray(z).reshape(R, H, P), _np_dtype(io))
    A = _arr(case["A"], np.float32)
    D = case.get("D")
    D = None if D is None else _arr(D, np.float32)
    bias = case.get("dt_bias")
    bias = None if bias is None else _arr(bias, np.float32)
    L = int(case["L"])
    bx = _arr(case["buf_x"], _np_dtype(io))
    bdt = _arr(case["buf_dt"], _np_dtype(dtd))
    bB = _arr(case["buf_B"], _np_dtype(io))
    if bx.shape != (slots, L, H, P) or bB.shape != (slots, L, G, N) or \
            bdt.shape != ((slots, L, H) if dt_per_head else (slots, L, H, P)):
        raise OracleError("buffer shapes do not match the pool and L")
    blen = np.ascontiguousarray(case["buf_len"], dtype=np.int64)
    keep = []
    args = _ReplayArgs()
    base = args.base
    pool_out = state.copy()
    out = np.zeros((R, H, P), dtype=_np_dtype(io))
    written = np.zeros(slots, dtype=np.uint8)
    bx_out, bdt_out, bB_out = bx.copy(), bdt.copy(), bB.copy()
    base.pool_in, base.pool_out = _ptr(state), _ptr(pool_out)
    base.state_dtype = DTYPES[sd]
    base.slots, base.H, base.P, base.N, base.G = slots, H, P, N, G
    base.R, base.io_dtype = R, DTYPES[io]
    base.x, base.dt = _ptr(xr), _ptr(dtr)
    base.dt_dtype, base.dt_per_head = DTYPES[dtd], int(dt_per_head)
    base.A, base.B, base.C = _ptr(A), _ptr(Br), _ptr(Cr)
    base.D, base.z, base.dt_bias = _ptr(D), _ptr(zr), _ptr(bias)
    base.dt_softplus = int(bool(case.get("dt_softplus", False)))
    if spec:
        base.layout, base.steps, base.nseq = DENSE, T, x.shape[0]
    else:
        base.layout, base.steps, base.nseq = ONE_TOKEN, 0, R
    base.rtab = _table(case.get("state_batch_indices"), keep)
    base.wtab = _table(None, keep)
    base.pad = int(case.get("pad_slot_id", -1))
    base.disable = int(bool(case.get("disable_state_update", False)))
    base.out, base.written = _ptr(out), _ptr(written)
    args.L = L
    args.bx_in, args.bx_out = _ptr(bx), _ptr(bx_out)
    args.bdt_in, args.bdt_out = _ptr(bdt), _ptr(bdt_out)
    args.bB_in, args.bB_out = _ptr(bB), _ptr(bB_out)
    args.buf_len = _ptr(blen)
    lp = case.get("lp")
    out_lp = {}
    if lp is not None:
        lp = np.ascontiguousarray(lp, dtype=np.uint8)
        lps = np.ascontiguousarray(case["lp_scale"], dtype=np.uint8)
        mx4 = case.get("lp_format", "mx8") == "mx4"
        args.lp_bits = 4 if mx4 else 8
        want = state.shape[:3] + (N // 2,) if mx4 else state.shape
        if lp.shape != want or lps.shape != state.shape[:3] + (N // 32,):
            raise OracleError("read copy shapes do not match the pool")
        out_lp = {"lp": lp.copy(), "lp_scale": lps.copy()}
        args.lp_in, args.lps_in = _ptr(lp), _ptr(lps)
        args.lp_out, args.lps_out = _ptr(out_lp["lp"]), _ptr(out_lp["lp_scale"])
    err = ctypes.create_string_buffer(256)
    fn = lib.oracle_replay_spec if spec else lib.oracle_replay
    if fn(ctypes.byref(args), err, 256):
        raise OracleError(err.value.decode())
    return dict({"y": out.reshape(x.shape), "state": pool_out, "buf_x": bx_out, "buf_dt": bdt_out,
                 "buf_B": bB_out, "written": written.astype(bool)}, **out_lp)


# ---------------------------------------------------------------- state copies

CONV_LAYOUTS = {"SD": 0, "DS": 1}


def _copy_fns(lib):
    if not hasattr(lib, "_copy_ready"):
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_batch_memmove.argtypes = [ctypes.c_void_p, ctypes.c_int64, i64p, i64p, i64p,
                                             ctypes.c_int64, ctypes.c_char_p, ctypes.c_int]
        lib.oracle_batch_memmove.restype = ctypes.c_int
        lib.oracle_conv_shift.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, i64p,
                                          i64p, i64p, ctypes.c_int64, ctypes.c_char_p,
                                          ctypes.c_int]
        lib.oracle_conv_shift.restype = ctypes.c_int
        lib._copy_ready = True


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def run_batch_memmove(buf, src_off, dst_off, sizes, oracle=None):
    """Batched copy with memmove semantics (oracle_batch_memmove): copy i
    moves sizes[i] bytes from byte offset src_off[i] to dst_off[i] of `buf`
    (a uint8 array). Returns the new buffer."""
    lib = (oracle or default()).lib
    _copy_fns(lib)
    out = np.array(buf, dtype=np.uint8, copy=True).ravel()
    s, d, z = _i64(src_off), _i64(dst_off), _i64(sizes)
    err = ctypes.create_string_buffer(256)
    p = ctypes.POINTER(ctypes.c_int64)
    if lib.oracle_batch_memmove(out.ctypes.data, out.size, s.ctypes.data_as(p),
                                d.ctypes.data_as(p), z.ctypes.data_as(p), len(z), err, 256):
        raise OracleError(err.value.decode())
    return out.reshape(np.shape(buf))


def run_conv_shift(pool, layout, src_blk, dst_blk, bias, oracle=None):
    """Convolution-state shift (oracle_conv_shift): pool [blocks, W, inner]
    ("SD") or [blocks, inner, W] ("DS") of any element type; request r writes
    state[dst][:W - bias] = state[src][bias:]. Returns the new pool."""
    lib = (oracle or default()).lib
    _copy_fns(lib)
    pool = np.ascontiguousarray(pool)
    out = pool.copy()
    blocks = pool.shape[0]
    W, inner = (pool.shape[1], pool.shape[2]) if layout == "SD" else (pool.shape[2], pool.shape[1])
    s, d, b = _i64(src_blk), _i64(dst_blk), _i64(bias)
    err = ctypes.create_string_buffer(256)
    p = ctypes.POINTER(ctypes.c_int64)
    if lib.oracle_conv_shift(out.ctypes.data, blocks, CONV_LAYOUTS[layout], W, inner,
                             pool.itemsize, s.ctypes.data_as(p), d.ctypes.data_as(p),
                             b.ctypes.data_as(p), len(s), err, 256):
        raise OracleError(err.value.decode())
    return out


# ---------------------------------------------------------------- SSD prefill

class _SsdArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("T", "H", "P", "N", "G", "nchunks", "batch",
                                              "chunk_size")] + [
        ("io_dtype", ctypes.c_int32), ("dt_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("z", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
        ("dt_lo", ctypes.c_float), ("dt_hi", ctypes.c_float),
        ("cu_chunk", ctypes.c_void_p), ("seq_idx", ctypes.c_void_p), ("init", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("chunk_states", ctypes.c_void_p)]


def run_ssd(case, oracle=None):
    """SSD packed prefill (oracle_ssd): the case holds x [T, H, P], dt [T, H],
    A, B / C [T, G, N], D, z, dt_bias (as for the decode step), dt_softplus,
    dt_limit (lo, hi), chunk_size, cu_chunk_seqlens, seq_idx,
    last_chunk_indices, initial_states ([batch, H, P, N] or None),
    state_dtype, io_dtype, dt_dtype. Returns dict(y, chunk_states [nchunks,
    H, P, N], states = chunk_states[last_chunk_indices])."""
    lib = (oracle or default()).lib
    if not hasattr(lib, "_ssd_ready"):
        lib.oracle_ssd.argtypes = [ctypes.POINTER(_SsdArgs), ctypes.c_char_p, ctypes.c_int]
        lib.oracle_ssd.restype = ctypes.c_int
        lib._ssd_ready = True
    io, sd = case["io_dtype"], case["state_dtype"]
    dtd = case.get("dt_dtype", io)
    x = _arr(case["x"], _np_dtype(io))
    T, H, P = x.shape
    dt = _arr(case["dt"], _np_dtype(dtd))
    Bm, Cm = _arr(case["B"], _np_dtype(io)), _arr(case["C"], _np_dtype(io))
    G, N = Bm.shape[1:]
    z = case.get("z")
    z = None if z is None else _arr(z, _np_dtype(io))
    A = _arr(case["A"], np.float32)
    D = case.get("D")
    D = None if D is None else _arr(D, np.float32)
    bias = case.get("dt_bias")
    bias = None if bias is None else _arr(bias, np.float32)
    cu = _i64(case["cu_chunk_seqlens"])
    seq = _i64(case["seq_idx"])
    last = _i64(case["last_chunk_indices"])
    nchunks = len(seq)
    batch = len(last)
    init = case.get("initial_states")
    init = None if init is None else _arr(init, _np_dtype(sd))
    out = np.zeros((T, H, P), dtype=_np_dtype(io))
    states = np.zeros((nchunks, H, P, N), dtype=_np_dtype(sd))
    a = _SsdArgs()
    a.T, a.H, a.P, a.N, a.G, a.nchunks, a.batch = T, H, P, N, G, nchunks, batch
    a.chunk_size = int(case["chunk_size"])
    a.io_dtype, a.dt_dtype, a.state_dtype = DTYPES[io], DTYPES[dtd], DTYPES[sd]
    a.x, a.dt, a.A, a.B, a.C = _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm)
    a.D, a.z, a.dt_bias = _ptr(D), _ptr(z), _ptr(bias)
    a.dt_softplus = int(bool(case.get("dt_softplus", False)))
    lo, hi = case.get("dt_limit", (0.0, float("inf")))
    a.dt_lo, a.dt_hi = lo, hi
    a.cu_chunk, a.seq_idx, a.init = _ptr(cu), _ptr(seq), _ptr(init)
    a.out, a.chunk_states = _ptr(out), _ptr(states)
    err = ctypes.create_string_buffer(256)
    if lib.oracle_ssd(ctypes.byref(a), err, 256):
        raise OracleError(err.value.decode())
    if np.any((last < 0) | (last >= max(nchunks, 1))):
        raise OracleError("last_chunk_indices outside the chunks")
    return {"y": out, "chunk_states": states,
            "states": states[last] if nchunks else np.zeros((batch, H, P, N), states.dtype)}


# ---------------------------------------------------------------- MXFP8 copies

def _mx8_fns(lib):
    if not hasattr(lib, "_mx8_ready"):
        lib.oracle_mx8_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.oracle_mx8_quantize.restype = None
        lib.oracle_mx8_dequantize.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p]
        lib.oracle_mx8_dequantize.restype = None
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_float
        lib._mx8_ready = True


def mx8_quantize(x, oracle=None):
    """MXFP8 (E4M3, blocks of 32 along the last axis) of a float32 array:
    returns (codes uint8 like x, scales uint8 [..., last / 32])."""
    lib = (oracle or default()).lib
    _mx8_fns(lib)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape[-1] % 32:
        raise OracleError("the last axis must be a multiple of 32")
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1] + (x.shape[-1] // 32,), np.uint8)
    lib.oracle_mx8_quantize(x.ctypes.data, x.size // 32, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def mx8_dequantize(codes, scales, oracle=None):
    lib = (oracle or default()).lib
    _mx8_fns(lib)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    x = np.zeros(codes.shape, np.float32)
    lib.oracle_mx8_dequantize(codes.ctypes.data, scales.ctypes.data, codes.size // 32, x.ctypes.data)
    return x


def e4m3_encode(v, oracle=None):
    lib = (oracle or default()).lib
    _mx8_fns(lib)
    return int(lib.oracle_e4m3_encode(float(v)))


def e4m3_decode(b, oracle=None):
    lib = (oracle or default()).lib
    _mx8_fns(lib)
    return float(lib.oracle_e4m3_decode(int(b)))


# ---------------------------------------------------------------- MXFP4 copies

def _mx4_fns(lib):
    if not hasattr(lib, "_mx4_ready"):
        lib.oracle_mx4_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.oracle_mx4_quantize.restype = None
        lib.oracle_mx4_dequantize.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p]
        lib.oracle_mx4_dequantize.restype = None
        lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        lib.oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_decode.restype = ctypes.c_float
        lib._mx4_ready = True


def mx4_quantize(x, oracle=None):
    """MXFP4 (E2M1, blocks of 32 along the last axis, two codes a byte, the
    even element in the low nibble) of a float32 array: returns (codes uint8
    [..., last / 2], scales uint8 [..., last / 32])."""
    lib = (oracle or default()).lib
    _mx4_fns(lib)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape[-1] % 32:
        raise OracleError("the last axis must be a multiple of 32")
    codes = np.zeros(x.shape[:-1] + (x.shape[-1] // 2,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (x.shape[-1] // 32,), np.uint8)
    lib.oracle_mx4_quantize(x.ctypes.data, x.size // 32, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def mx4_dequantize(codes, scales, oracle=None):
    lib = (oracle or default()).lib
    _mx4_fns(lib)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    x = np.zeros(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float32)
    lib.oracle_mx4_dequantize(codes.ctypes.data, scales.ctypes.data, codes.size // 16, x.ctypes.data)
    return x


def e2m1_encode(v, oracle=None):
    lib = (oracle or default()).lib
    _mx4_fns(lib)
    return int(lib.oracle_e2m1_encode(float(v)))


def e2m1_decode(nib, oracle=None):
    lib = (oracle or default()).lib
    _mx4_fns(lib)
    return float(lib.oracle_e2m1_decode(int(nib)))
