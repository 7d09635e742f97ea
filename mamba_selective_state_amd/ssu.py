"""Python binding of libssu (include/ssu.h): argument marshalling only.

Every step of the update runs in the library's gfx950 kernels; PyTorch only
provides device memory and the current stream. The library must be built
(mamba_selective_state_amd/build.py); importing this module without it raises.

Low level, same names as the C ABI:  ssu_update, ssu_plan, ssu_last_error,
ssu_abi_version (ssu_update takes an SsuArgs built by make_args).
High level, same argument order and defaults as MATE's mate.mamba API (MATE
docs, "Mamba / SSU", API reference): selective_state_update and
prewarm_selective_state_update.
"""
import ctypes
import os

import torch

from . import build as _build

F32, F16, BF16, I32, I64, F64, U8 = 0, 1, 2, 3, 4, 5, 6
OK, ERR_VALUE, ERR_NOT_IMPLEMENTED, ERR_HIP = 0, 1, 2, 3
OPT_STATE_SCALE, OPT_INTERMEDIATE_STATES, OPT_RAND_SEED = 1, 2, 4
OPT_CACHE_STEPS, OPT_ALGORITHM, OPT_BACKEND = 8, 16, 32

_TORCH_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
                 torch.int32: I32, torch.int64: I64, torch.float64: F64, torch.uint8: U8}
CONV_TOKEN_MAJOR, CONV_DIM_MAJOR = 0, 1


class SsuTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("size", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class SsuArgs(ctypes.Structure):
    _fields_ = [(n, SsuTensor) for n in
                ("state", "x", "dt", "A", "B", "C", "D", "z", "dt_bias",
                 "state_batch_indices", "dst_state_batch_indices", "cu_seqlens",
                 "num_accepted_tokens", "out")] + [
        ("dt_softplus", ctypes.c_int32), ("disable_state_update", ctypes.c_int32),
        ("pad_slot_id", ctypes.c_int64), ("unsupported", ctypes.c_uint32)]


class SsuReplayArgs(ctypes.Structure):
    _fields_ = [("base", SsuArgs), ("buf_x", SsuTensor), ("buf_dt", SsuTensor),
                ("buf_B", SsuTensor), ("buf_len", SsuTensor)]


class SsuReplayLpArgs(ctypes.Structure):
    _fields_ = [("base", SsuReplayArgs), ("lp", SsuTensor), ("lp_scale", SsuTensor)]


class SsuConvShiftArgs(ctypes.Structure):
    _fields_ = [("state", SsuTensor), ("layout", ctypes.c_int32), ("src_block", SsuTensor),
                ("dst_block", SsuTensor), ("bias", SsuTensor)]


class SsuSsdArgs(ctypes.Structure):
    _fields_ = [(n, SsuTensor) for n in
                ("x", "dt", "A", "B", "C", "D", "z", "dt_bias", "cu_seqlens", "cu_chunk_seqlens",
                 "last_chunk_indices", "seq_idx", "initial_states", "out", "states")] + [
        ("chunk_size", ctypes.c_int64), ("dt_softplus", ctypes.c_int32),
        ("return_intermediate_states", ctypes.c_int32), ("dt_limit_lo", ctypes.c_float),
        ("dt_limit_hi", ctypes.c_float), ("unsupported", ctypes.c_uint32)]


OPT_SSD_CHECKPOINT = 64


class SsuSsdPlanDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("heads", "groups", "dim", "dstate", "chunk_size", "io_dtype", "state_dtype",
                 "dt_dtype", "block_M")]


class SsuSsdPlanInfo(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("kernels", (ctypes.c_char * 64) * 3),
                ("vgprs", ctypes.c_int32 * 3), ("workspace_bytes_per_chunk", ctypes.c_int64)]


class SsuPlanDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("state_dtype", "io_dtype", "dt_dtype", "slot_dtype", "meta_dtype", "heads",
                 "dim", "dstate", "groups", "dt_dim", "packed")] + [("max_rows", ctypes.c_int64),
                                                                     ("disable_state_update", ctypes.c_int32)]


class SsuPlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 64), ("block_threads", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("blocks_per_seq_head", ctypes.c_int32),
                ("vgprs", ctypes.c_int32), ("sgprs", ctypes.c_int32)]


EXPORTS = ("ssu_plan", "ssu_update", "ssu_replay_update", "ssu_replay_spec_update",
           "ssu_replay_lp_update", "ssu_mx8_quantize", "ssu_replay_mx4_update", "ssu_mx4_quantize",
           "ssu_batch_memcpy", "ssu_conv_state_shift", "ssu_ssd_workspace_bytes", "ssu_ssd_prefill",
           "ssu_ssd_prefill_noalloc", "ssu_ssd_plan", "ssu_last_error", "ssu_abi_version")
SSD_SCRATCH_BYTES = 64 << 20  # SSU_SSD_SCRATCH_BYTES


def load_library(path=None):
    """Load libssu.so; raises if it has not been built."""
    path = path or _build.LIB
    if not os.path.exists(path):
        raise ImportError("libssu.so is not built (run mamba_selective_state_amd/build.py): %s"
                          % path)
    lib = ctypes.CDLL(path)
    lib.ssu_plan.argtypes = [ctypes.POINTER(SsuPlanDesc), ctypes.POINTER(SsuPlanInfo)]
    lib.ssu_plan.restype = ctypes.c_int
    lib.ssu_update.argtypes = [ctypes.POINTER(SsuArgs), ctypes.c_void_p]
    lib.ssu_update.restype = ctypes.c_int
    lib.ssu_replay_update.argtypes = [ctypes.POINTER(SsuReplayArgs), ctypes.c_void_p]
    lib.ssu_replay_update.restype = ctypes.c_int
    lib.ssu_replay_spec_update.argtypes = [ctypes.POINTER(SsuReplayArgs), ctypes.c_void_p]
    lib.ssu_replay_spec_update.restype = ctypes.c_int
    lib.ssu_replay_lp_update.argtypes = [ctypes.POINTER(SsuReplayLpArgs), ctypes.c_void_p]
    lib.ssu_replay_lp_update.restype = ctypes.c_int
    lib.ssu_mx8_quantize.argtypes = [ctypes.POINTER(SsuTensor)] * 3 + [ctypes.c_void_p]
    lib.ssu_mx8_quantize.restype = ctypes.c_int
    lib.ssu_replay_mx4_update.argtypes = [ctypes.POINTER(SsuReplayLpArgs), ctypes.c_void_p]
    lib.ssu_replay_mx4_update.restype = ctypes.c_int
    lib.ssu_mx4_quantize.argtypes = [ctypes.POINTER(SsuTensor)] * 3 + [ctypes.c_void_p]
    lib.ssu_mx4_quantize.restype = ctypes.c_int
    lib.ssu_batch_memcpy.argtypes = [ctypes.POINTER(SsuTensor)] * 3 + [ctypes.c_int64,
                                                                       ctypes.c_void_p]
    lib.ssu_batch_memcpy.restype = ctypes.c_int
    lib.ssu_conv_state_shift.argtypes = [ctypes.POINTER(SsuConvShiftArgs), ctypes.c_void_p]
    lib.ssu_conv_state_shift.restype = ctypes.c_int
    lib.ssu_ssd_workspace_bytes.argtypes = [ctypes.c_int64] * 4
    lib.ssu_ssd_workspace_bytes.restype = ctypes.c_int64
    lib.ssu_ssd_prefill.argtypes = [ctypes.POINTER(SsuSsdArgs), ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    lib.ssu_ssd_prefill.restype = ctypes.c_int
    lib.ssu_ssd_plan.argtypes = [ctypes.POINTER(SsuSsdPlanDesc), ctypes.POINTER(SsuSsdPlanInfo)]
    lib.ssu_ssd_plan.restype = ctypes.c_int
    lib.ssu_ssd_prefill_noalloc.argtypes = [ctypes.POINTER(SsuSsdArgs), ctypes.c_void_p]
    lib.ssu_ssd_prefill_noalloc.restype = ctypes.c_int
    lib.ssu_last_error.argtypes = []
    lib.ssu_last_error.restype = ctypes.c_char_p
    lib.ssu_abi_version.argtypes = []
    lib.ssu_abi_version.restype = ctypes.c_int
    return lib


_lib = load_library()
LIBRARY_PATH = _build.LIB


class SsuError(RuntimeError):
    pass


def _raise(status, what):
    msg = "%s: %s" % (what, ssu_last_error())
    if status == ERR_VALUE:
        raise ValueError(msg)
    if status == ERR_NOT_IMPLEMENTED:
        raise NotImplementedError(msg)
    raise SsuError(msg)


def ssu_abi_version():
    return _lib.ssu_abi_version()


def ssu_last_error():
    return _lib.ssu_last_error().decode()


def ssu_update(args, stream=None):
    """Enqueue one update (include/ssu.h ssu_update) on `stream` (a HIP stream
    handle as int, or None for torch's current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_update(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_update")


def ssu_replay_update(args, stream=None):
    """Enqueue one ReplaySSM decode step (include/ssu.h ssu_replay_update)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_replay_update(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_replay_update")


def ssu_replay_spec_update(args, stream=None):
    """Enqueue one ReplaySSM speculative step (include/ssu.h ssu_replay_spec_update)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_replay_spec_update(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_replay_spec_update")


def ssu_replay_lp_update(args, stream=None):
    """Enqueue one ReplaySSM decode step with the MXFP8 read copy (include/ssu.h
    ssu_replay_lp_update)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_replay_lp_update(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_replay_lp_update")


def ssu_mx8_quantize(src, codes, scales, stream=None):
    """Enqueue an MXFP8 quantization (include/ssu.h ssu_mx8_quantize); the
    arguments are SsuTensor descriptors."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_mx8_quantize(ctypes.byref(src), ctypes.byref(codes), ctypes.byref(scales),
                               ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_mx8_quantize")


def ssu_replay_mx4_update(args, stream=None):
    """Enqueue one ReplaySSM decode step with the MXFP4 read copy (include/ssu.h
    ssu_replay_mx4_update)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_replay_mx4_update(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_replay_mx4_update")


def ssu_mx4_quantize(src, codes, scales, stream=None):
    """Enqueue an MXFP4 quantization (include/ssu.h ssu_mx4_quantize); the
    arguments are SsuTensor descriptors."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_mx4_quantize(ctypes.byref(src), ctypes.byref(codes), ctypes.byref(scales),
                               ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_mx4_quantize")


def ssu_plan(desc):
    """Validate and load one configuration (include/ssu.h ssu_plan); returns
    the selection as a dict."""
    info = SsuPlanInfo()
    st = _lib.ssu_plan(ctypes.byref(desc), ctypes.byref(info))
    if st != OK:
        _raise(st, "ssu_plan")
    return {"kernel": info.kernel.decode(), "block_threads": info.block_threads,
            "rows_per_block": info.rows_per_block,
            "blocks_per_seq_head": info.blocks_per_seq_head, "vgprs": info.vgprs}


def tensor_desc(t, device=None):
    """SsuTensor describing a torch tensor (None -> absent)."""
    d = SsuTensor()
    if t is None:
        return d
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, got %r" % type(t))
    if t.dtype not in _TORCH_DTYPES:
        raise ValueError("unsupported dtype %s" % t.dtype)
    if t.dim() > 4:
        raise ValueError("tensors have at most 4 dimensions")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError("every tensor must live on the state's GPU (%s), got %s"
                         % (device, t.device))
    d.data = t.data_ptr() if t.numel() > 0 else (t.data_ptr() or 16)
    d.dtype = _TORCH_DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.size[i] = s
        d.stride[i] = st
    return d


def make_args(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False,
              state_batch_indices=None, pad_slot_id=-1, out=None, disable_state_update=False,
              dst_state_batch_indices=None, cu_seqlens=None, num_accepted_tokens=None,
              unsupported=0):
    """SsuArgs for ssu_update; `out` must be given."""
    dev = state.device
    a = SsuArgs()
    for name, t in (("state", state), ("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C),
                    ("D", D), ("z", z), ("dt_bias", dt_bias),
                    ("state_batch_indices", state_batch_indices),
                    ("dst_state_batch_indices", dst_state_batch_indices),
                    ("cu_seqlens", cu_seqlens), ("num_accepted_tokens", num_accepted_tokens),
                    ("out", out)):
        setattr(a, name, tensor_desc(t, dev))
    a.dt_softplus = int(bool(dt_softplus))
    a.disable_state_update = int(bool(disable_state_update))
    a.pad_slot_id = int(pad_slot_id)
    a.unsupported = int(unsupported)
    return a


def selective_state_update(state, x, dt, A, B, C, D, z=None, dt_bias=None, dt_softplus=False,
                           state_batch_indices=None, pad_slot_id=-1, state_scale=None, out=None,
                           disable_state_update=False, intermediate_states_buffer=None,
                           intermediate_state_indices=None, intermediate_state_scales=None,
                           rand_seed=None, philox_rounds=10, cache_steps=0, algorithm="auto",
                           dst_state_batch_indices=None, cu_seqlens=None,
                           num_accepted_tokens=None, backend="auto"):
    """Apply one decode step of the selective state update and return y.

    Same arguments, order and defaults as MATE's selective_state_update (MATE
    docs, "Mamba / SSU", API reference); the call shape decides the kernel.
    Options the library does not implement raise NotImplementedError.
    """
    unsupported = 0
    if state_scale is not None:
        unsupported |= OPT_STATE_SCALE
    if (intermediate_states_buffer is not None or intermediate_state_indices is not None
            or intermediate_state_scales is not None):
        unsupported |= OPT_INTERMEDIATE_STATES
    if rand_seed is not None:
        unsupported |= OPT_RAND_SEED
    if cache_steps:
        unsupported |= OPT_CACHE_STEPS
    if algorithm != "auto":
        unsupported |= OPT_ALGORITHM
    if backend != "auto":
        unsupported |= OPT_BACKEND
    if out is None and not unsupported:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    args = make_args(state, x, dt, A, B, C, D, z, dt_bias, dt_softplus, state_batch_indices,
                     pad_slot_id, out, disable_state_update, dst_state_batch_indices, cu_seqlens,
                     num_accepted_tokens, unsupported)
    ssu_update(args, torch.cuda.current_stream(state.device).cuda_stream)
    return out


def prewarm_selective_state_update(*, state_dtype, io_dtype, batch, heads, dim, dstate, groups,
                                   slot_dtype, rows_per_cta=4, lanes_per_row=32, packed=False,
                                   meta_dtype=torch.int32, dt_dim=None, dt_dtype=None,
                                   disable_state_update=False):
    """Validate and load the kernel one configuration uses, before any graph
    capture (MATE prewarm_selective_state_update; rows_per_cta and
    lanes_per_row are accepted and ignored: the gfx950 kernels fix their own
    tiling). With packed and disable_state_update it selects the output-only
    variant such calls take. Returns the selection."""
    desc = SsuPlanDesc()
    desc.state_dtype = _TORCH_DTYPES[state_dtype]
    desc.io_dtype = _TORCH_DTYPES[io_dtype]
    desc.dt_dtype = _TORCH_DTYPES[dt_dtype] if dt_dtype is not None else desc.io_dtype
    desc.slot_dtype = _TORCH_DTYPES[slot_dtype]
    desc.meta_dtype = _TORCH_DTYPES[meta_dtype]
    desc.heads, desc.dim, desc.dstate, desc.groups = heads, dim, dstate, groups
    desc.dt_dim = dim if dt_dim is None else dt_dim
    desc.packed = int(bool(packed))
    desc.max_rows = batch
    desc.disable_state_update = int(bool(disable_state_update))
    return ssu_plan(desc)


def make_replay_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, z=None,
                     dt_bias=None, dt_softplus=False, state_batch_indices=None, pad_slot_id=-1,
                     out=None, disable_state_update=False):
    """SsuReplayArgs for ssu_replay_update; `out` must be given."""
    r = SsuReplayArgs()
    r.base = make_args(state, x, dt, A, B, C, D, z, dt_bias, dt_softplus, state_batch_indices,
                       pad_slot_id, out, disable_state_update)
    dev = state.device
    r.buf_x = tensor_desc(buf_x, dev)
    r.buf_dt = tensor_desc(buf_dt, dev)
    r.buf_B = tensor_desc(buf_B, dev)
    r.buf_len = tensor_desc(buf_len, dev)
    return r


def replay_selective_state_update(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, z=None,
                                  dt_bias=None, dt_softplus=False, state_batch_indices=None,
                                  pad_slot_id=-1, out=None, disable_state_update=False):
    """One ReplaySSM decode step (ReplaySSM article, section "核心做法"): the
    state is the checkpoint in `state` plus per-slot input buffers; buf_len[b]
    is the number of steps sequence b has buffered (< L = buf_x.shape[1]).
    A step that fills the buffer folds it into the checkpoint; any other step
    computes y from checkpoint and buffer and appends its inputs. The caller
    advances buf_len (to 0 after a fold). Returns y."""
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    args = make_replay_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, z, dt_bias,
                            dt_softplus, state_batch_indices, pad_slot_id, out,
                            disable_state_update)
    ssu_replay_update(args, torch.cuda.current_stream(state.device).cuda_stream)
    return out


def replay_spec_selective_state_update(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len,
                                       z=None, dt_bias=None, dt_softplus=False,
                                       state_batch_indices=None, pad_slot_id=-1, out=None,
                                       disable_state_update=False):
    """One ReplaySSM speculative step (ReplaySSM article, section
    "投机解码回滚变成挪指针"): x [batch, T, heads, dim] holds T draft tokens per
    sequence, buf_len[b] the committed entries of sequence b (0..L). When
    buf_len + 2T > L the committed entries are first folded into the
    checkpoint and the drafts go to entries 0..T-1, else to buf_len..; the
    caller then advances the pointer by the accepted count (from 0 after a
    fold). Returns y [batch, T, heads, dim]."""
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    args = make_replay_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, z, dt_bias,
                            dt_softplus, state_batch_indices, pad_slot_id, out,
                            disable_state_update)
    ssu_replay_spec_update(args, torch.cuda.current_stream(state.device).cuda_stream)
    return out


def make_replay_lp_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, lp, lp_scale,
                        z=None, dt_bias=None, dt_softplus=False, state_batch_indices=None,
                        pad_slot_id=-1, out=None, disable_state_update=False):
    """SsuReplayLpArgs for ssu_replay_lp_update or ssu_replay_mx4_update;
    `out` must be given."""
    r = SsuReplayLpArgs()
    r.base = make_replay_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, z, dt_bias,
                              dt_softplus, state_batch_indices, pad_slot_id, out,
                              disable_state_update)
    r.lp = tensor_desc(lp, state.device)
    r.lp_scale = tensor_desc(lp_scale, state.device)
    return r


def replay_lp_selective_state_update(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, lp,
                                     lp_scale, z=None, dt_bias=None, dt_softplus=False,
                                     state_batch_indices=None, pad_slot_id=-1, out=None,
                                     disable_state_update=False):
    """replay_selective_state_update with an MXFP8 copy of the f32 checkpoint
    (ReplaySSM article, section "数据与边界"; OCP MX v1.0 MXFP8 E4M3):
    output-only steps read lp (uint8 E4M3 codes, [slots, heads, dim, dstate])
    times lp_scale (uint8 E8M0, [slots, heads, dim, dstate / 32]) instead of
    the checkpoint; a fold stores the checkpoint and rewrites both. Returns y."""
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    args = make_replay_lp_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, lp,
                               lp_scale, z, dt_bias, dt_softplus, state_batch_indices,
                               pad_slot_id, out, disable_state_update)
    ssu_replay_lp_update(args, torch.cuda.current_stream(state.device).cuda_stream)
    return out


def replay_mx4_selective_state_update(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, lp,
                                      lp_scale, z=None, dt_bias=None, dt_softplus=False,
                                      state_batch_indices=None, pad_slot_id=-1, out=None,
                                      disable_state_update=False):
    """replay_lp_selective_state_update with an MXFP4 copy (OCP MX v1.0
    MXFP4, E2M1 elements): lp holds two codes a byte, the even-indexed value
    in the low nibble ([slots, heads, dim, dstate / 2]); lp_scale as for
    MXFP8. Returns y."""
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    args = make_replay_lp_args(state, x, dt, A, B, C, D, buf_x, buf_dt, buf_B, buf_len, lp,
                               lp_scale, z, dt_bias, dt_softplus, state_batch_indices,
                               pad_slot_id, out, disable_state_update)
    ssu_replay_mx4_update(args, torch.cuda.current_stream(state.device).cuda_stream)
    return out


def mx8_quantize(src, codes=None, scales=None):
    """MXFP8 (E4M3 elements, an E8M0 scale per 32 consecutive values) of a
    contiguous float32 CUDA tensor whose size is a multiple of 32; the codes
    take src's shape, the scales its shape with the last dimension / 32.
    Returns (codes, scales)."""
    if codes is None:
        codes = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    if scales is None:
        shape = tuple(src.shape[:-1]) + (src.shape[-1] // 32,) if src.dim() else (0,)
        scales = torch.empty(shape, dtype=torch.uint8, device=src.device)
    dev = src.device
    ssu_mx8_quantize(tensor_desc(src, dev), tensor_desc(codes, dev), tensor_desc(scales, dev),
                     torch.cuda.current_stream(dev).cuda_stream)
    return codes, scales


def mx4_quantize(src, codes=None, scales=None):
    """MXFP4 (E2M1 elements two a byte, an E8M0 scale per 32 consecutive
    values) of a contiguous float32 CUDA tensor whose size is a multiple of
    32; the codes take src's shape with the last dimension / 2, the scales
    with it / 32. Returns (codes, scales)."""
    last = src.shape[-1] if src.dim() else 0
    if codes is None:
        shape = tuple(src.shape[:-1]) + (last // 2,) if src.dim() else (0,)
        codes = torch.empty(shape, dtype=torch.uint8, device=src.device)
    if scales is None:
        shape = tuple(src.shape[:-1]) + (last // 32,) if src.dim() else (0,)
        scales = torch.empty(shape, dtype=torch.uint8, device=src.device)
    dev = src.device
    ssu_mx4_quantize(tensor_desc(src, dev), tensor_desc(codes, dev), tensor_desc(scales, dev),
                     torch.cuda.current_stream(dev).cuda_stream)
    return codes, scales


# ---------------------------------------------------------------- state copies

def ssu_batch_memcpy(src_ptrs, dst_ptrs, sizes, max_size, stream=None):
    """Enqueue a batched memmove-safe copy (include/ssu.h ssu_batch_memcpy);
    the first three arguments are SsuTensor descriptors."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_batch_memcpy(ctypes.byref(src_ptrs), ctypes.byref(dst_ptrs), ctypes.byref(sizes),
                               int(max_size), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_batch_memcpy")


def batch_memcpy(src_ptrs, dst_ptrs, sizes, max_size=None):
    """Copy sizes[i] bytes from device address src_ptrs[i] to dst_ptrs[i] for
    every i, with memmove semantics where a copy overlaps its own source (vLLM
    PR #50729 digest, "实现拆解"). src_ptrs, dst_ptrs: int64 CUDA tensors of
    addresses; sizes: int32/int64 CUDA tensor; max_size: a bound on the sizes
    (it only sets the parallelism; default 64 KiB)."""
    dev = src_ptrs.device
    ssu_batch_memcpy(tensor_desc(src_ptrs, dev), tensor_desc(dst_ptrs, dev),
                     tensor_desc(sizes, dev), 65536 if max_size is None else max_size,
                     torch.cuda.current_stream(dev).cuda_stream)


def ssu_conv_state_shift(args, stream=None):
    """Enqueue a convolution-state shift (include/ssu.h ssu_conv_state_shift)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_conv_state_shift(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_conv_state_shift")


def make_conv_shift_args(state, src_block, dst_block, bias, layout="SD"):
    a = SsuConvShiftArgs()
    dev = state.device
    a.state = tensor_desc(state, dev)
    a.layout = CONV_TOKEN_MAJOR if layout == "SD" else CONV_DIM_MAJOR
    a.src_block = tensor_desc(src_block, dev)
    a.dst_block = tensor_desc(dst_block, dev)
    a.bias = tensor_desc(bias, dev)
    return a


def conv_state_shift(state, src_block, dst_block, bias, layout="SD"):
    """state[dst_block[r]][:W - bias[r]] = state[src_block[r]][bias[r]:] for
    every request r (vLLM PR #50729 digest, "实现拆解"), in place and safe
    when a request shifts a block inside itself. state: [blocks, W, inner]
    for layout "SD" (token-major) or [blocks, inner, W] for "DS"."""
    ssu_conv_state_shift(make_conv_shift_args(state, src_block, dst_block, bias, layout),
                         torch.cuda.current_stream(state.device).cuda_stream)


# ---------------------------------------------------------------- SSD prefill

_ssd_workspaces = {}


def ssu_ssd_workspace_bytes(heads, dim, dstate, nchunks):
    return _lib.ssu_ssd_workspace_bytes(heads, dim, dstate, nchunks)


def ssu_ssd_prefill(args, workspace, workspace_bytes, stream=None):
    """Enqueue an SSD prefill (include/ssu.h ssu_ssd_prefill)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_ssd_prefill(ctypes.byref(args), ctypes.c_void_p(workspace), int(workspace_bytes),
                              ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_ssd_prefill")


def ssu_ssd_plan(desc):
    """Validate an SSD prefill configuration and load its kernels
    (include/ssu.h ssu_ssd_plan); returns what was loaded."""
    info = SsuSsdPlanInfo()
    st = _lib.ssu_ssd_plan(ctypes.byref(desc), ctypes.byref(info))
    if st != OK:
        _raise(st, "ssu_ssd_plan")
    return {"launches": info.launches,
            "kernels": [info.kernels[i].value.decode() for i in range(info.launches)],
            "vgprs": [info.vgprs[i] for i in range(info.launches)],
            "workspace_bytes_per_chunk": info.workspace_bytes_per_chunk}


def prewarm_ssd_combined_fwd_varlen(heads, groups, dim, dstate, chunk_size, io_dtype=torch.bfloat16,
                                    state_dtype=torch.bfloat16, dt_dtype=torch.float32, block_M=32):
    """Validate one SSD prefill configuration and load its kernels on the
    current device, before any graph capture (MATE
    prewarm_ssd_combined_fwd_varlen; block_M is accepted and ignored: the
    gfx950 kernels fix their own tiling). Token and chunk counts are runtime
    sizes. Returns what was loaded."""
    d = SsuSsdPlanDesc()
    d.heads, d.groups, d.dim, d.dstate, d.chunk_size = heads, groups, dim, dstate, chunk_size
    d.io_dtype = _TORCH_DTYPES[io_dtype]
    d.state_dtype = _TORCH_DTYPES[state_dtype]
    d.dt_dtype = _TORCH_DTYPES[dt_dtype]
    d.block_M = block_M
    return ssu_ssd_plan(d)


def ssu_ssd_prefill_noalloc(args, stream=None):
    """Enqueue an SSD prefill whose workspace is the library's own device
    array (include/ssu.h ssu_ssd_prefill_noalloc): nothing is allocated;
    calls whose workspace exceeds SSD_SCRATCH_BYTES raise ValueError."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = _lib.ssu_ssd_prefill_noalloc(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        _raise(st, "ssu_ssd_prefill_noalloc")


def ssd_workspace(device, stream, nbytes):
    """The cached workspace of (`device`, `stream`), grown to at least
    `nbytes` (a call of an already seen size allocates nothing). One per
    stream: calls on one stream are ordered, so they can share it; a grown
    workspace is allocated on that stream, so the caching allocator hands
    the old one's memory out again only behind the kernels that used it."""
    key = (device, stream)
    ws = _ssd_workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ssd_workspaces[key] = ws
    return ws


def make_ssd_args(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens, last_chunk_indices,
                  seq_idx, out, states, D=None, z=None, dt_bias=None, dt_softplus=False,
                  dt_limit=(0.0, float("inf")), initial_states=None,
                  return_intermediate_states=False, checkpoint=False):
    """An SsuSsdArgs for ssu_ssd_prefill / ssu_ssd_prefill_noalloc (out and
    states given)."""
    dev = x.device
    a = SsuSsdArgs()
    for k, v in (("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C), ("D", D), ("z", z),
                 ("dt_bias", dt_bias), ("cu_seqlens", cu_seqlens),
                 ("cu_chunk_seqlens", cu_chunk_seqlens), ("last_chunk_indices", last_chunk_indices),
                 ("seq_idx", seq_idx), ("initial_states", initial_states), ("out", out),
                 ("states", states)):
        setattr(a, k, tensor_desc(v, dev))
    a.chunk_size = int(chunk_size)
    a.dt_softplus = int(bool(dt_softplus))
    a.return_intermediate_states = int(bool(return_intermediate_states))
    a.dt_limit_lo, a.dt_limit_hi = float(dt_limit[0]), float(dt_limit[1])
    if checkpoint:
        a.unsupported |= OPT_SSD_CHECKPOINT
    return a


def ssd_combined_fwd_varlen(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens,
                            last_chunk_indices, seq_idx, out=None, D=None, z=None, dt_bias=None,
                            dt_softplus=False, dt_limit=(0.0, float("inf")), initial_states=None,
                            return_intermediate_states=False, state_dtype=None,
                            checkpoint_token_indices=None, checkpoint_state_slots=None,
                            checkpoint_states=None):
    """Packed variable-length SSD prefill (MATE docs, "SSD packed prefill"):
    x [tokens, heads, dim], dt [tokens, heads]; writes y into `out` (allocated
    when None) and returns the states after each sequence's last chunk
    [batch, heads, dim, dstate] (or after every chunk with
    return_intermediate_states), in state_dtype (default: initial_states'
    dtype, else C's)."""
    dev = x.device
    if state_dtype is None:
        state_dtype = initial_states.dtype if initial_states is not None else C.dtype
    nchunks = int(cu_chunk_seqlens.shape[0]) - 1
    rows = nchunks if return_intermediate_states else int(last_chunk_indices.shape[0])
    states = torch.empty((rows, x.shape[1], x.shape[2], B.shape[2]), dtype=state_dtype, device=dev)
    if out is None:
        out = torch.empty_like(x)
    a = make_ssd_args(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens, last_chunk_indices,
                      seq_idx, out, states, D=D, z=z, dt_bias=dt_bias, dt_softplus=dt_softplus,
                      dt_limit=dt_limit, initial_states=initial_states,
                      return_intermediate_states=return_intermediate_states,
                      checkpoint=any(v is not None for v in (checkpoint_token_indices,
                                                             checkpoint_state_slots,
                                                             checkpoint_states)))
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = ssu_ssd_workspace_bytes(x.shape[1], x.shape[2], B.shape[2], max(nchunks, 0))
    ws = ssd_workspace(dev, stream, nbytes)
    ssu_ssd_prefill(a, ws.data_ptr(), ws.numel(), stream)
    return states
