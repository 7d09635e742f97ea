"""C-ABI host logic on the CPU: the library loads, exports what include/ssu.h
declares, and rejects every malformed call before any device work. The
pointers below are fake (never dereferenced: validation only looks at shapes,
strides, dtypes and alignment), and no valid call is made without a GPU."""
import ctypes
import os
import re

import pytest

from mamba_selective_state_amd import ssu as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssu.h")
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SSU_API\s+[\w\s\*]*?\b(ssu_\w+)\s*\(", text)))


def test_exports_match_header():
    names = declared_functions()
    assert names == sorted(S.EXPORTS)
    lib = ctypes.CDLL(S.LIBRARY_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    text = open(HEADER).read()
    v = int(re.search(r"#define SSU_ABI_VERSION (\d+)", text).group(1))
    assert S.ssu_abi_version() == v


def test_struct_layout_matches_header(tmp_path):
    """Field offsets and sizes of the ctypes mirrors equal what a C compiler
    makes of include/ssu.h."""
    structs = {"ssu_tensor_t": S.SsuTensor, "ssu_args_t": S.SsuArgs,
               "ssu_plan_desc_t": S.SsuPlanDesc, "ssu_plan_info_t": S.SsuPlanInfo,
               "ssu_replay_args_t": S.SsuReplayArgs, "ssu_replay_lp_args_t": S.SsuReplayLpArgs,
               "ssu_conv_shift_args_t": S.SsuConvShiftArgs,
               "ssu_ssd_args_t": S.SsuSsdArgs, "ssu_ssd_plan_desc_t": S.SsuSsdPlanDesc,
               "ssu_ssd_plan_info_t": S.SsuSsdPlanInfo}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssu.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append('printf("%s SIZEOF %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in cls._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            k1, k2, v = line.split()
            got[(k1, k2)] = int(v)
    for cname, cls in structs.items():
        assert got[(cname, "SIZEOF")] == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def tdesc(shape, dtype, strides=None, ptr=FAKE):
    t = S.SsuTensor()
    t.data = ptr
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        t.size[i] = s
        t.stride[i] = st
    return t


def base_args(rows=4, H=8, P=16, N=128, G=2, slots=8, sd=S.F32, io=S.BF16):
    a = S.SsuArgs()
    a.state = tdesc((slots, H, P, N), sd)
    a.x = tdesc((rows, H, P), io)
    a.dt = tdesc((rows, H, P), io)
    a.A = tdesc((H,), S.F32)
    a.B = tdesc((rows, G, N), io)
    a.C = tdesc((rows, G, N), io)
    a.out = tdesc((rows, H, P), io)
    a.pad_slot_id = -1
    return a


def update(a):
    st = S._lib.ssu_update(ctypes.byref(a), None)
    return st, S.ssu_last_error()




def expect(a, status, words):
    st, msg = update(a)
    assert st == status, (st, msg)
    for w in words:
        assert w in msg, (w, msg)


def test_empty_batch_is_ok_without_launch():
    a = base_args(rows=0)
    assert update(a) == (S.OK, "")


def test_no_sequences_is_ok_without_launch():
    a = base_args(rows=0)
    a.cu_seqlens = tdesc((1,), S.I32)
    assert update(a)[0] == S.OK


def test_null_args():
    assert S._lib.ssu_update(None, None) == S.ERR_VALUE
    assert "NULL" in S.ssu_last_error()


@pytest.mark.parametrize("bit,word", [(S.OPT_STATE_SCALE, "state_scale"),
                                      (S.OPT_INTERMEDIATE_STATES, "intermediate"),
                                      (S.OPT_RAND_SEED, "rand_seed"),
                                      (S.OPT_CACHE_STEPS, "cache_steps"),
                                      (S.OPT_ALGORITHM, "algorithm"),
                                      (S.OPT_BACKEND, "backend")])
def test_unsupported_options(bit, word):
    a = base_args(rows=0)
    a.unsupported = bit
    expect(a, S.ERR_NOT_IMPLEMENTED, [word])


def test_state_errors():
    a = base_args(rows=0)
    a.state = S.SsuTensor()
    expect(a, S.ERR_VALUE, ["state is required"])
    a = base_args(rows=0)
    a.state = tdesc((8, 8, 16, 128), S.I32)
    expect(a, S.ERR_VALUE, ["state must be f32"])
    a = base_args(rows=0)
    a.state = tdesc((8, 8, 16, 128), S.F32, strides=(8 * 16 * 128, 16 * 128, 1, 16))
    expect(a, S.ERR_VALUE, ["contiguous"])
    a = base_args(rows=0)
    a.state = tdesc((8, 8, 16, 128), S.F32, ptr=FAKE + 4)
    expect(a, S.ERR_VALUE, ["16-byte"])
    a = base_args(rows=0, N=96)
    expect(a, S.ERR_NOT_IMPLEMENTED, ["dstate 96"])
    a = base_args(rows=0)
    a.state = tdesc((8, 8, 16), S.F32)
    expect(a, S.ERR_VALUE, ["[slots, heads, dim, dstate]"])


def test_x_errors():
    a = base_args(rows=0)
    a.x = tdesc((0, 8, 16, 1), S.BF16)
    a.x.ndim = 5
    expect(a, S.ERR_VALUE, ["x must be"])
    a = base_args(rows=0)
    a.x = tdesc((0, 128), S.BF16)
    expect(a, S.ERR_VALUE, ["x must be"])
    a = base_args(rows=0)
    a.x = tdesc((0, 4, 16), S.BF16)
    expect(a, S.ERR_VALUE, ["x axis 1"])
    a = base_args(rows=0)
    a.x = tdesc((0, 8, 16), S.BF16, strides=(256, 16, 2))
    expect(a, S.ERR_VALUE, ["unit stride"])
    a = base_args(rows=0)
    a.x = tdesc((0, 8, 16), S.I64)
    expect(a, S.ERR_VALUE, ["x must be f32"])


def test_dense_form_must_collapse_to_rows():
    a = base_args(rows=0)
    a.x = tdesc((2, 3, 8, 16), S.BF16, strides=(1000, 128, 16, 1))
    expect(a, S.ERR_NOT_IMPLEMENTED, ["batch stride"])


def test_dt_errors():
    a = base_args(rows=0)
    a.dt = tdesc((0, 8, 16), S.F16)
    expect(a, S.ERR_VALUE, ["dt must be f32 or the x dtype"])
    a = base_args(rows=0)
    a.dt = tdesc((0,), S.F32)
    expect(a, S.ERR_VALUE, ["dt must be shaped like x"])
    a = base_args(rows=0)
    a.dt = S.SsuTensor()
    expect(a, S.ERR_VALUE, ["dt is required"])


def test_head_vector_errors():
    a = base_args(rows=0)
    a.A = tdesc((4,), S.F32)
    expect(a, S.ERR_VALUE, ["A must be [heads]"])
    a = base_args(rows=0)
    a.A = tdesc((8,), S.BF16)
    expect(a, S.ERR_VALUE, ["A must be f32"])
    a = base_args(rows=0)
    a.D = tdesc((8, 16), S.F32)
    expect(a, S.ERR_VALUE, ["D must be per head"])
    a = base_args(rows=0)
    a.dt_bias = tdesc((7,), S.F32)
    expect(a, S.ERR_VALUE, ["dt_bias must be [heads]"])
    a = base_args(rows=0)
    a.A = tdesc((8, 16, 128), S.F32, strides=(1, 0, 0))  # broadcast view is fine
    assert update(a)[0] == S.OK


def test_groups_errors():
    a = base_args(rows=0, G=3)
    expect(a, S.ERR_VALUE, ["divisible by groups"])
    a = base_args(rows=0)
    a.B = tdesc((0, 2, 128), S.F16)
    expect(a, S.ERR_VALUE, ["x dtype"])
    a = base_args(rows=0)
    a.C = tdesc((0, 2, 64), S.BF16)
    expect(a, S.ERR_VALUE, ["C last axis"])
    a = base_args(rows=0)
    a.B = tdesc((0, 2, 128), S.BF16, ptr=FAKE + 2)
    expect(a, S.ERR_VALUE, ["byte boundaries"])
    a = base_args(rows=0)
    a.B = tdesc((0, 2, 128), S.BF16, strides=(258, 129, 1))
    expect(a, S.ERR_VALUE, ["byte boundaries"])


def test_out_and_z_errors():
    a = base_args(rows=0)
    a.out = S.SsuTensor()
    expect(a, S.ERR_VALUE, ["out is required"])
    a = base_args(rows=0)
    a.out = tdesc((0, 8, 16), S.F32)
    expect(a, S.ERR_VALUE, ["out must have the x dtype"])
    a = base_args(rows=0)
    a.z = tdesc((0, 8, 8), S.BF16)
    expect(a, S.ERR_VALUE, ["z last axis"])


def test_table_errors():
    a = base_args(rows=0)
    a.state_batch_indices = tdesc((3,), S.I32)
    expect(a, S.ERR_VALUE, ["one entry per row"])
    a = base_args(rows=0)
    a.state_batch_indices = tdesc((0,), S.F32)
    expect(a, S.ERR_VALUE, ["i32 or i64"])
    a = base_args(rows=0)
    a.dst_state_batch_indices = tdesc((0, 1, 1), S.I64)
    expect(a, S.ERR_VALUE, ["1-D [rows] or 2-D"])
    a = base_args(rows=0)
    a.x = tdesc((2, 3, 8, 16), S.BF16)
    a.dt = tdesc((2, 3, 8, 16), S.BF16)
    a.B = tdesc((2, 3, 2, 128), S.BF16)
    a.C = tdesc((2, 3, 2, 128), S.BF16)
    a.out = tdesc((2, 3, 8, 16), S.BF16)
    a.state_batch_indices = tdesc((2, 2), S.I32)
    expect(a, S.ERR_VALUE, ["columns"])


def test_meta_errors():
    a = base_args(rows=0)
    a.cu_seqlens = tdesc((2, 2), S.I32)
    expect(a, S.ERR_VALUE, ["cu_seqlens must be 1-D"])
    a = base_args(rows=0)
    a.cu_seqlens = tdesc((3,), S.I32)
    a.num_accepted_tokens = tdesc((3,), S.I32)
    expect(a, S.ERR_VALUE, ["num_accepted_tokens"])
    a = base_args(rows=0)
    a.x = tdesc((1, 1, 8, 16), S.BF16)
    a.cu_seqlens = tdesc((2,), S.I32)
    expect(a, S.ERR_VALUE, ["cu_seqlens goes with"])


def test_plan_validation():
    def plan(**kw):
        d = S.SsuPlanDesc()
        base = dict(state_dtype=S.F32, io_dtype=S.BF16, dt_dtype=S.BF16, slot_dtype=S.I32,
                    meta_dtype=S.I32, heads=8, dim=64, dstate=128, groups=2, dt_dim=64, packed=0)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        info = S.SsuPlanInfo()
        return S._lib.ssu_plan(ctypes.byref(d), ctypes.byref(info)), S.ssu_last_error()

    assert plan(groups=3)[0] == S.ERR_VALUE
    assert plan(dstate=48)[0] == S.ERR_NOT_IMPLEMENTED
    assert plan(dt_dtype=S.F16)[0] == S.ERR_VALUE
    assert plan(dt_dim=7)[0] == S.ERR_VALUE
    assert plan(slot_dtype=S.F32)[0] == S.ERR_VALUE
    assert plan(state_dtype=S.I32)[0] == S.ERR_VALUE
    assert S._lib.ssu_plan(None, None) == S.ERR_VALUE


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    t = torch.zeros(2, 2, 2, 16)
    with pytest.raises(ValueError, match="GPU"):
        S.tensor_desc(t, torch.device("cuda", 0))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError, match="not built"):
        S.load_library(str(tmp_path / "libssu.so"))


def test_package_never_touches_the_oracle():
    """The product path has no CPU fallback: no package source names the
    oracle or the workload generators."""
    pkg = os.path.join(ROOT, "mamba_selective_state_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, f
                assert "workloads" not in text, f


# ---------------------------------------------------------------- replay


def replay_args(rows=0, L=4, H=8, P=16, N=128, G=2, slots=8, dt_full=True):
    r = S.SsuReplayArgs()
    r.base = base_args(rows=rows, H=H, P=P, N=N, G=G, slots=slots)
    r.buf_x = tdesc((slots, L, H, P), S.BF16)
    r.buf_dt = tdesc((slots, L, H, P) if dt_full else (slots, L, H), S.BF16)
    r.buf_B = tdesc((slots, L, G, N), S.BF16)
    r.buf_len = tdesc((rows,), S.I32)
    return r


def replay(r):
    st = S._lib.ssu_replay_update(ctypes.byref(r), None)
    return st, S.ssu_last_error()


def test_replay_empty_is_ok_without_launch():
    assert replay(replay_args())[0] == S.OK


def test_replay_errors():
    assert S._lib.ssu_replay_update(None, None) == S.ERR_VALUE
    r = replay_args()
    r.base.dst_state_batch_indices = tdesc((0,), S.I32)
    assert replay(r)[0] == S.ERR_NOT_IMPLEMENTED
    r = replay_args()
    r.base.cu_seqlens = tdesc((1,), S.I32)
    assert replay(r)[0] == S.ERR_NOT_IMPLEMENTED
    r = replay_args()
    r.buf_x = tdesc((8, 4, 8, 8), S.BF16)
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "buf_x" in msg
    r = replay_args()
    r.buf_B = tdesc((8, 3, 2, 128), S.BF16)
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "buf_B" in msg
    r = replay_args()
    r.buf_dt = tdesc((8, 4, 8, 16), S.F32)
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "dt dtype" in msg
    r = replay_args(dt_full=False)  # per-head buffer but dt [rows, heads, dim]
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "per-head" in msg
    r = replay_args()
    r.buf_x = tdesc((8, 4, 8, 16), S.BF16, strides=(4 * 8 * 16, 8 * 16, 1, 8))
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "contiguous" in msg
    r = replay_args()
    r.buf_len = S.SsuTensor()
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "buf_len" in msg
    r = replay_args()
    r.buf_len = tdesc((3,), S.I32)
    st, msg = replay(r)
    assert st == S.ERR_VALUE and "buf_len" in msg


# ------------------------------------------------------ replay, speculative


def spec_args(batch=0, T=2, L=4, H=8, P=16, N=128, G=2, slots=8):
    r = replay_args(rows=batch, L=L, H=H, P=P, N=N, G=G, slots=slots)
    for k, tail in (("x", (H, P)), ("dt", (H, P)), ("B", (G, N)), ("C", (G, N)), ("out", (H, P))):
        setattr(r.base, k, tdesc((batch, T) + tail, S.BF16))
    return r


def spec(r):
    st = S._lib.ssu_replay_spec_update(ctypes.byref(r), None)
    return st, S.ssu_last_error()


def test_replay_spec_empty_is_ok_without_launch():
    assert spec(spec_args())[0] == S.OK


def test_replay_spec_errors():
    assert S._lib.ssu_replay_spec_update(None, None) == S.ERR_VALUE
    st, msg = spec(replay_args())  # a 3-D x
    assert st == S.ERR_NOT_IMPLEMENTED and "[batch, T, heads, dim]" in msg
    st, msg = replay(spec_args())  # the one-token entry point with a 4-D x
    assert st == S.ERR_NOT_IMPLEMENTED and "[batch, heads, dim]" in msg
    r = spec_args(batch=3)
    r.base.state_batch_indices = tdesc((6,), S.I32)  # one entry per row, not per sequence
    st, msg = spec(r)
    assert st == S.ERR_VALUE and "1-D [batch]" in msg
    r = spec_args(batch=3)
    r.base.state_batch_indices = tdesc((3, 2), S.I32)
    st, msg = spec(r)
    assert st == S.ERR_VALUE and "1-D [batch]" in msg
    r = spec_args(T=5, L=4)
    st, msg = spec(r)
    assert st == S.ERR_VALUE and "do not fit" in msg
    r = spec_args()
    r.base.num_accepted_tokens = tdesc((0,), S.I32)
    assert spec(r)[0] == S.ERR_NOT_IMPLEMENTED


# ---------------------------------------------------------------- state copies


def memcpy(src, dst, sizes, max_size=0):
    st = S._lib.ssu_batch_memcpy(ctypes.byref(src), ctypes.byref(dst), ctypes.byref(sizes),
                                 max_size, None)
    return st, S.ssu_last_error()


def test_batch_memcpy_empty_and_errors():
    assert memcpy(tdesc((0,), S.I64), tdesc((0,), S.I64), tdesc((0,), S.I64))[0] == S.OK
    assert S._lib.ssu_batch_memcpy(None, None, None, 0, None) == S.ERR_VALUE
    st, msg = memcpy(tdesc((3,), S.I32), tdesc((3,), S.I64), tdesc((3,), S.I64))
    assert st == S.ERR_VALUE and "src_ptrs" in msg
    st, msg = memcpy(tdesc((3,), S.I64), tdesc((2,), S.I64), tdesc((3,), S.I64))
    assert st == S.ERR_VALUE and "length" in msg
    st, msg = memcpy(tdesc((3,), S.I64), tdesc((3,), S.I64), tdesc((2,), S.I64))
    assert st == S.ERR_VALUE and "sizes" in msg
    st, msg = memcpy(tdesc((3,), S.I64), tdesc((3,), S.I64), tdesc((3,), S.F32))
    assert st == S.ERR_VALUE and "sizes" in msg
    st, msg = memcpy(tdesc((3,), S.I64), tdesc((3,), S.I64), S.SsuTensor())
    assert st == S.ERR_VALUE and "sizes" in msg


def shift(state, src, dst, bias, layout=S.CONV_TOKEN_MAJOR):
    a = S.SsuConvShiftArgs()
    a.state, a.layout, a.src_block, a.dst_block, a.bias = state, layout, src, dst, bias
    st = S._lib.ssu_conv_state_shift(ctypes.byref(a), None)
    return st, S.ssu_last_error()


# ---------------------------------------------------------------- MXFP8 read copy


def replay_lp_args(rows=0, N=128, sd=S.F32, slots=8, H=8, P=16):
    r = S.SsuReplayLpArgs()
    r.base = replay_args(rows=rows, N=N, slots=slots, H=H, P=P)
    r.base.base.state = tdesc((slots, H, P, N), sd)
    r.lp = tdesc((slots, H, P, N), S.U8)
    r.lp_scale = tdesc((slots, H, P, N // 32), S.U8)
    return r


def replay_lp(r):
    st = S._lib.ssu_replay_lp_update(ctypes.byref(r), None)
    return st, S.ssu_last_error()


def test_replay_lp_empty_is_ok_without_launch():
    assert replay_lp(replay_lp_args()) == (S.OK, "")


def test_replay_lp_errors():
    assert S._lib.ssu_replay_lp_update(None, None) == S.ERR_VALUE
    st, msg = replay_lp(replay_lp_args(sd=S.BF16))
    assert st == S.ERR_NOT_IMPLEMENTED and "f32" in msg
    r = replay_lp_args()
    r.lp = S.SsuTensor()
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "required" in msg
    r = replay_lp_args()
    r.lp = tdesc((8, 8, 16, 128), S.I32)
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "u8" in msg
    r = replay_lp_args()
    r.lp = tdesc((8, 8, 16, 64), S.U8)
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "lp must be" in msg
    r = replay_lp_args()
    r.lp_scale = tdesc((8, 8, 16, 8), S.U8)
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "lp_scale must be" in msg
    r = replay_lp_args()
    r.lp = tdesc((8, 8, 16, 128), S.U8, strides=(8 * 16 * 128, 16 * 128, 1, 16))
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "contiguous" in msg
    for off in (2, 8):  # the copy is read 16 bytes at a time
        r = replay_lp_args()
        r.lp = tdesc((8, 8, 16, 128), S.U8, ptr=FAKE + off)
        st, msg = replay_lp(r)
        assert st == S.ERR_VALUE and "16-byte" in msg
    # the replay checks still apply
    r = replay_lp_args()
    r.base.buf_len = S.SsuTensor()
    st, msg = replay_lp(r)
    assert st == S.ERR_VALUE and "buf_len" in msg


def quantize(src, codes, scales):
    st = S._lib.ssu_mx8_quantize(ctypes.byref(src), ctypes.byref(codes), ctypes.byref(scales), None)
    return st, S.ssu_last_error()


def test_mx8_quantize_empty_and_errors():
    assert quantize(tdesc((0,), S.F32), tdesc((0,), S.U8), tdesc((0,), S.U8)) == (S.OK, "")
    assert quantize(tdesc((4, 0, 32), S.F32), tdesc((0,), S.U8), tdesc((0,), S.U8))[0] == S.OK
    assert S._lib.ssu_mx8_quantize(None, None, None, None) == S.ERR_VALUE
    st, msg = quantize(tdesc((48,), S.F32), tdesc((48,), S.U8), tdesc((1,), S.U8))
    assert st == S.ERR_VALUE and "multiple of 32" in msg
    st, msg = quantize(tdesc((64,), S.BF16), tdesc((64,), S.U8), tdesc((2,), S.U8))
    assert st == S.ERR_VALUE and "f32" in msg
    st, msg = quantize(tdesc((64,), S.F32), tdesc((32,), S.U8), tdesc((2,), S.U8))
    assert st == S.ERR_VALUE and "codes" in msg
    st, msg = quantize(tdesc((64,), S.F32), tdesc((64,), S.U8), tdesc((3,), S.U8))
    assert st == S.ERR_VALUE and "scales" in msg
    st, msg = quantize(tdesc((2, 64), S.F32, strides=(128, 1)), tdesc((128,), S.U8),
                       tdesc((4,), S.U8))
    assert st == S.ERR_VALUE and "contiguous" in msg
    st, msg = quantize(tdesc((64,), S.F32, ptr=FAKE + 4), tdesc((64,), S.U8), tdesc((2,), S.U8))
    assert st == S.ERR_VALUE and "aligned" in msg


# ---------------------------------------------------------------- MXFP4 read copy


def replay_mx4(r):
    st = S._lib.ssu_replay_mx4_update(ctypes.byref(r), None)
    return st, S.ssu_last_error()


def replay_mx4_args(**kw):
    r = replay_lp_args(**kw)
    slots, H, P, N = (r.lp.size[i] for i in range(4))
    r.lp = tdesc((slots, H, P, N // 2), S.U8)
    return r


def test_replay_mx4_empty_is_ok_without_launch():
    assert replay_mx4(replay_mx4_args()) == (S.OK, "")
    # the MXFP8 entry point takes the full-width copy only
    st, msg = replay_lp(replay_mx4_args())
    assert st == S.ERR_VALUE and "lp must be [slots, heads, dim, dstate]" in msg


def test_replay_mx4_errors():
    assert S._lib.ssu_replay_mx4_update(None, None) == S.ERR_VALUE
    st, msg = replay_mx4(replay_mx4_args(sd=S.BF16))
    assert st == S.ERR_NOT_IMPLEMENTED and "MXFP4" in msg and "f32" in msg
    st, msg = replay_mx4(replay_mx4_args(N=16))
    assert st == S.ERR_VALUE and "multiple of 32" in msg
    r = replay_mx4_args()
    r.lp = tdesc((8, 8, 16, 128), S.U8)  # the MXFP8 width
    st, msg = replay_mx4(r)
    assert st == S.ERR_VALUE and "dstate / 2" in msg
    r = replay_mx4_args()
    r.lp_scale = tdesc((8, 8, 16, 8), S.U8)
    st, msg = replay_mx4(r)
    assert st == S.ERR_VALUE and "lp_scale must be" in msg
    r = replay_mx4_args()
    r.lp = tdesc((8, 8, 16, 64), S.U8, strides=(8 * 16 * 64, 16 * 64, 1, 16))
    st, msg = replay_mx4(r)
    assert st == S.ERR_VALUE and "contiguous" in msg
    r = replay_mx4_args()
    r.lp = tdesc((8, 8, 16, 64), S.U8, ptr=FAKE + 2)
    st, msg = replay_mx4(r)
    assert st == S.ERR_VALUE and "aligned" in msg


def quantize4(src, codes, scales):
    st = S._lib.ssu_mx4_quantize(ctypes.byref(src), ctypes.byref(codes), ctypes.byref(scales), None)
    return st, S.ssu_last_error()


def test_mx4_quantize_empty_and_errors():
    assert quantize4(tdesc((0,), S.F32), tdesc((0,), S.U8), tdesc((0,), S.U8)) == (S.OK, "")
    assert S._lib.ssu_mx4_quantize(None, None, None, None) == S.ERR_VALUE
    st, msg = quantize4(tdesc((48,), S.F32), tdesc((24,), S.U8), tdesc((1,), S.U8))
    assert st == S.ERR_VALUE and "multiple of 32" in msg
    st, msg = quantize4(tdesc((64,), S.F32), tdesc((64,), S.U8), tdesc((2,), S.U8))
    assert st == S.ERR_VALUE and "codes" in msg and "32 bytes" in msg
    st, msg = quantize4(tdesc((64,), S.F32), tdesc((32,), S.U8), tdesc((3,), S.U8))
    assert st == S.ERR_VALUE and "scales" in msg
    st, msg = quantize4(tdesc((64,), S.F32), tdesc((32,), S.U8, ptr=FAKE + 2), tdesc((2,), S.U8))
    assert st == S.ERR_VALUE and "4-byte" in msg


def test_conv_state_shift_empty_and_errors():
    pool = tdesc((6, 4, 32), S.F16)
    v0 = tdesc((0,), S.I32)
    assert shift(pool, v0, v0, v0)[0] == S.OK
    assert shift(tdesc((6, 32, 4), S.F64), v0, v0, v0, S.CONV_DIM_MAJOR)[0] == S.OK
    assert S._lib.ssu_conv_state_shift(None, None) == S.ERR_VALUE
    v3 = tdesc((3,), S.I64)
    st, msg = shift(tdesc((6, 128), S.F16), v3, v3, v3)
    assert st == S.ERR_VALUE and "3-D" in msg
    st, msg = shift(pool, v3, v3, v3, layout=7)
    assert st == S.ERR_VALUE and "layout" in msg
    st, msg = shift(tdesc((6, 4, 32), S.F16, strides=(256, 64, 2)), v3, v3, v3)
    assert st == S.ERR_VALUE and "contiguous" in msg
    st, msg = shift(pool, v3, tdesc((2,), S.I64), v3)
    assert st == S.ERR_VALUE and "dst_block" in msg
    st, msg = shift(pool, v3, v3, S.SsuTensor())
    assert st == S.ERR_VALUE and "required" in msg
    st, msg = shift(pool, v3, v3, tdesc((3,), S.F32))
    assert st == S.ERR_VALUE and "bias" in msg


# ---------------------------------------------------------------- SSD prefill


def ssd_args(T=0, H=8, P=64, N=128, G=2, nchunks=0, batch=0, chunk=256, io=S.BF16, sd=S.F32):
    a = S.SsuSsdArgs()
    a.x = tdesc((T, H, P), io)
    a.dt = tdesc((T, H), S.F32)
    a.A = tdesc((H,), S.F32)
    a.B = tdesc((T, G, N), io)
    a.C = tdesc((T, G, N), io)
    a.z = tdesc((T, H, P), io)
    a.out = tdesc((T, H, P), io)
    a.cu_chunk_seqlens = tdesc((nchunks + 1,), S.I32)
    a.seq_idx = tdesc((nchunks,), S.I32)
    a.last_chunk_indices = tdesc((batch,), S.I32)
    a.states = tdesc((batch, H, P, N), sd)
    a.chunk_size = chunk
    a.dt_limit_lo, a.dt_limit_hi = 0.0, float("inf")
    return a


def ssd(a, ws=0, ws_bytes=0):
    st = S._lib.ssu_ssd_prefill(ctypes.byref(a), ctypes.c_void_p(ws), ws_bytes, None)
    return st, S.ssu_last_error()


def test_ssd_empty_is_ok_without_workspace():
    assert ssd(ssd_args()) == (S.OK, "")
    assert ssd(ssd_args(batch=3)) == (S.OK, "")


def test_ssd_workspace_bytes():
    assert S.ssu_ssd_workspace_bytes(8, 64, 128, 0) >= 0
    assert S.ssu_ssd_workspace_bytes(8, 64, 128, 10) > S.ssu_ssd_workspace_bytes(8, 64, 128, 1)
    assert S.ssu_ssd_workspace_bytes(-1, 64, 128, 1) == -1


def test_ssd_errors():
    assert S._lib.ssu_ssd_prefill(None, None, 0, None) == S.ERR_VALUE
    a = ssd_args()
    a.unsupported = S.OPT_SSD_CHECKPOINT
    st, msg = ssd(a)
    assert st == S.ERR_NOT_IMPLEMENTED and "checkpoint" in msg
    st, msg = ssd(ssd_args(io=S.F32))
    assert st == S.ERR_NOT_IMPLEMENTED and "bf16 or f16" in msg
    st, msg = ssd(ssd_args(P=32))
    assert st == S.ERR_NOT_IMPLEMENTED and "head dim" in msg
    st, msg = ssd(ssd_args(N=96))
    assert st == S.ERR_NOT_IMPLEMENTED and "dstate" in msg
    st, msg = ssd(ssd_args(H=6, G=4))
    assert st == S.ERR_VALUE and "divisible" in msg
    for chunk in (0, 257):
        st, msg = ssd(ssd_args(chunk=chunk))
        assert st == S.ERR_NOT_IMPLEMENTED and "chunk_size" in msg
    a = ssd_args()
    a.dt_limit_lo, a.dt_limit_hi = 1.0, 0.5
    st, msg = ssd(a)
    assert st == S.ERR_VALUE and "dt_limit" in msg
    # rows of x, B, C, z and out start on 16-byte boundaries
    for name in ("x", "z", "out"):
        a = ssd_args(T=4)
        setattr(a, name, tdesc((4, 8, 64), S.BF16, strides=(8 * 68, 68, 1)))
        st, msg = ssd(a)
        assert st == S.ERR_VALUE and "16-byte" in msg, (name, msg)
    a = ssd_args(T=4)
    a.B = tdesc((4, 2, 128), S.BF16, strides=(2 * 132, 132, 1))
    st, msg = ssd(a)
    assert st == S.ERR_VALUE and "16-byte" in msg
    a = ssd_args(T=4, nchunks=1, batch=1)
    a.states = tdesc((2, 8, 64, 128), S.F32)
    st, msg = ssd(a)
    assert st == S.ERR_VALUE and "states" in msg
    a = ssd_args(T=4, nchunks=1, batch=1)
    st, msg = ssd(a, ws=FAKE, ws_bytes=16)
    assert st == S.ERR_VALUE and "workspace" in msg
    a = ssd_args(T=4, nchunks=1, batch=1)
    a.cu_chunk_seqlens = S.SsuTensor()
    st, msg = ssd(a)
    assert st == S.ERR_VALUE and "cu_chunk_seqlens" in msg


def test_ssd_noalloc_rejects_oversized_and_null():
    """The allocation-free prefill refuses, before any device call, a call
    whose workspace exceeds the library's array, naming both sizes."""
    assert S._lib.ssu_ssd_prefill_noalloc(None, None) == S.ERR_VALUE
    assert "NULL" in S.ssu_last_error()
    a = ssd_args(T=16, H=128, nchunks=200, batch=1)
    need = S.ssu_ssd_workspace_bytes(128, 64, 128, 200)
    assert need > S.SSD_SCRATCH_BYTES
    st = S._lib.ssu_ssd_prefill_noalloc(ctypes.byref(a), None)
    msg = S.ssu_last_error()
    assert st == S.ERR_VALUE and str(need) in msg and str(S.SSD_SCRATCH_BYTES) in msg, msg


def test_ssd_plan_validation():
    """The SSD prewarm refuses, before loading anything, configurations the
    prefill does not take, naming the rule or the capability."""
    def plan(**kw):
        d = S.SsuSsdPlanDesc()
        base = dict(heads=8, groups=2, dim=64, dstate=128, chunk_size=256, io_dtype=S.BF16,
                    state_dtype=S.F32, dt_dtype=S.F32, block_M=32)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        info = S.SsuSsdPlanInfo()
        return S._lib.ssu_ssd_plan(ctypes.byref(d), ctypes.byref(info)), S.ssu_last_error()

    assert S._lib.ssu_ssd_plan(None, None) == S.ERR_VALUE
    for kw, status, word in ((dict(heads=6, groups=4), S.ERR_VALUE, "divisible"),
                             (dict(heads=0), S.ERR_VALUE, "positive"),
                             (dict(io_dtype=S.F32), S.ERR_NOT_IMPLEMENTED, "bf16 or f16"),
                             (dict(state_dtype=S.I32), S.ERR_VALUE, "state_dtype"),
                             (dict(dt_dtype=S.F16), S.ERR_VALUE, "dt_dtype"),
                             (dict(dim=96), S.ERR_NOT_IMPLEMENTED, "head dim"),
                             (dict(dstate=256), S.ERR_NOT_IMPLEMENTED, "dstate"),
                             (dict(chunk_size=512), S.ERR_NOT_IMPLEMENTED, "chunk_size")):
        st, msg = plan(**kw)
        assert st == status and word in msg, (kw, st, msg)
