"""GPU path against the CPU oracle, element by element, through the C ABI
(the Python binding only marshals arguments).

Small cases (the oracle runs whole) span several workgroup tiles and ragged
dim tails; the workloads' full sizes run in the benchmark's launch
configuration and are checked whole: every sequence against the oracle and
the whole pool's untouched slots."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import workloads as W
from oracle import ssu_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


# ---------------------------------------------------------------- small cases

def test_one_token_tiny_chained():
    """The MATE minimal example: a call without tables, then a call with
    tables [0, 1], on the pool the first call left."""
    c0 = W.one_token_tiny(tables=False)
    c1 = W.one_token_tiny(tables=True)
    ref0 = ssu_oracle.run(c0)
    ref1 = ssu_oracle.run(dict(c1, state=ref0["state"]))
    G.say("[gpu] one_token_tiny: launching two calls")
    d = G.device_case(c0)
    y0, _ = G.run_gpu(c0, d=d, sync=True)
    d1 = dict(d)
    d1["state_batch_indices"] = G.dev_index(c1["state_batch_indices"], "cuda:0")
    d1["dst_state_batch_indices"] = G.dev_index(c1["dst_state_batch_indices"], "cuda:0")
    y1, s1 = G.run_gpu(c1, d=d1)
    G.compare(c0, y0, ref0["state"], ref0, "call 0 y")
    G.compare(dict(c1, state=ref0["state"]), y1, s1, ref1, "call 1")


DECODE = [
    # (state, io, dstate, dim, index dtype, dt dtype)
    ("f32", "bf16", 128, 64, np.int32, "io"),
    ("f32", "bf16", 128, 40, np.int64, "io"),
    ("f32", "f16", 128, 64, np.int32, "f32"),
    ("f32", "f32", 128, 20, np.int32, "f32"),
    ("bf16", "bf16", 128, 64, np.int32, "io"),
    ("f16", "bf16", 128, 36, np.int64, "io"),
    ("f32", "bf16", 16, 64, np.int32, "io"),
    ("bf16", "bf16", 16, 24, np.int32, "io"),
    ("f32", "bf16", 32, 64, np.int32, "io"),
    ("f16", "f16", 32, 64, np.int32, "io"),
    ("f32", "bf16", 64, 64, np.int32, "io"),
    ("bf16", "f16", 64, 72, np.int32, "io"),
    ("f32", "bf16", 256, 64, np.int32, "io"),
    ("bf16", "bf16", 256, 40, np.int64, "f32"),
]


@pytest.mark.parametrize("sd,io,N,P,idx,dtd", DECODE,
                         ids=["%s-%s-n%d-p%d-%s-dt%s" % (a, b, c, d, np.dtype(e).name, f)
                              for a, b, c, d, e, f in DECODE])
def test_decode(sd, io, N, P, idx, dtd):
    c = W.decode(seed=100 + N + P, batch=24, heads=16, dim=P, dstate=N, groups=4, slots=48,
                 state_dtype=sd, io=io, index_dtype=idx)
    if dtd == "f32":
        c["dt"] = W.to_storage(np.random.default_rng(5).standard_normal(c["x"].shape,
                                                                         dtype=np.float32), "f32")
        c["dt_dtype"] = "f32"
    G.check(c, "decode %s %s n%d p%d" % (sd, io, N, P))


@pytest.mark.parametrize("pad", [0, -1])
@pytest.mark.parametrize("sd", ["bf16", "f32"])
def test_decode_pad(sd, pad):
    c = W.decode_pad(batch=40, heads=16, dim=64, dstate=128, groups=4, slots=96, state_dtype=sd,
                     pad_frac=0.1, pad_slot_id=pad)
    G.check(c, "decode_pad %s pad=%d" % (sd, pad))


@pytest.mark.parametrize("pad", [0, -1])
@pytest.mark.parametrize("sd", ["f32", "f16", "bf16"])
def test_mtp(sd, pad):
    c = W.mtp(nseq=6, steps=7, heads=16, dim=64, dstate=128, groups=4, state_dtype=sd,
              pad_slot_id=pad, index_dtype=np.int64 if sd == "f16" else np.int32,
              meta_dtype=np.int64 if sd == "bf16" else np.int32)
    G.check(c, "mtp %s pad=%d" % (sd, pad))


@pytest.mark.parametrize("mode", ["dst", "disable", "omitted"])
def test_varlen(mode):
    c = W.varlen(nseq=40, heads=8, dim=64, dstate=128, state_dtype="f16", dst=mode != "omitted",
                 disable=mode == "disable")
    assert (np.diff(c["cu_seqlens"]) == 0).any()
    G.check(c, "varlen %s" % mode)


YONLY_CASES = [
    # (state, io, dstate, dim): the output-only variant (disable_state_update) on
    # the matrix cores (f16 state with f16 or bf16 io, bf16 with bf16) and on
    # the VALU (the rest)
    ("f16", "bf16", 128, 64), ("f16", "bf16", 32, 40), ("f16", "bf16", 256, 64),
    ("f16", "f16", 64, 64), ("bf16", "bf16", 128, 28), ("bf16", "bf16", 256, 64),
    ("bf16", "f16", 128, 64), ("f32", "bf16", 128, 64), ("f32", "f32", 64, 36),
    # two 64-row tiles per head on the matrix cores, the second partial or whole
    ("f16", "bf16", 128, 96), ("bf16", "bf16", 64, 128),
]


@pytest.mark.parametrize("sd,io,N,P", YONLY_CASES, ids=["%s-%s-n%d-p%d" % c for c in YONLY_CASES])
def test_varlen_disable_variants(sd, io, N, P):
    """Lengths 0..12: sequences of at most 8 tokens take the output-only
    path, longer ones the update path without stores."""
    rng = np.random.default_rng(N + P)
    lengths = rng.integers(0, 13, 24)
    lengths[:3] = [8, 9, 1]
    c = W.varlen(seed=11, nseq=24, heads=4, dim=P, dstate=N, groups=2, state_dtype=sd, io=io,
                 disable=True, lengths=lengths)
    G.check(c, "varlen disable %s %s n%d p%d" % (sd, io, N, P))


@pytest.mark.parametrize("groups,P", [(1, 64), (2, 40), (8, 64)])
def test_varlen_disable_groups(groups, P):
    """The matrix-core output-only variant with 8 heads in one group, in two
    groups, and one head per group; lengths 0..12 (the longer sequences take
    the update path without stores)."""
    rng = np.random.default_rng(5 + groups)
    lengths = rng.integers(0, 13, 20)
    lengths[:3] = [12, 8, 0]
    c = W.varlen(seed=13 + groups, nseq=20, heads=8, dim=P, dstate=128, groups=groups,
                 state_dtype="f16", io="bf16", disable=True, lengths=lengths)
    G.check(c, "varlen disable heads g%d p%d" % (groups, P))


@pytest.mark.parametrize("pad", [0, -1])
@pytest.mark.parametrize("sd", ["f32", "f16", "bf16"])
def test_mtp_disable(sd, pad):
    """MTP with disable_state_update: reads at the accepted count, the pad
    id read as zeros, nothing stored."""
    c = W.mtp(nseq=6, steps=7, heads=16, dim=64, dstate=128, groups=4, state_dtype=sd,
              pad_slot_id=pad)
    c["disable_state_update"] = True
    G.check(c, "mtp disable %s pad=%d" % (sd, pad))


def test_varlen_f32_ragged():
    c = W.varlen(seed=9, nseq=30, heads=4, dim=28, dstate=64, groups=2, state_dtype="f32",
                 io="f32")
    G.check(c, "varlen f32 ragged")


def test_dense_4d():
    c = W.mtp(nseq=5, steps=3, heads=8, dim=64, dstate=128, groups=2, pad_slot_id=-1)
    R = 15
    for k in ("x", "dt", "B", "C", "z"):
        c[k] = c[k].reshape((5, 3) + c[k].shape[1:])
    c["cu_seqlens"] = None
    assert c["x"].shape[0] * c["x"].shape[1] == R
    G.check(c, "dense 4-D")
    flat = dict(c, state_batch_indices=c["state_batch_indices"].ravel(),
                dst_state_batch_indices=c["dst_state_batch_indices"].ravel())
    G.check(flat, "dense 4-D, flat tables")


def test_one_token_with_accepted():
    """x [batch, heads, dim] with num_accepted_tokens and a 2-D read table:
    the multi-token kernel with one token per sequence."""
    c = W.mtp(nseq=12, steps=1, heads=8, dim=64, dstate=128, groups=2, pad_slot_id=-1)
    rt = np.arange(12 * 3, dtype=np.int32).reshape(12, 3)
    c["state"] = np.concatenate([c["state"], c["state"][:12 * 3 - 24]])  # 36 slots
    c.update(state_batch_indices=rt, dst_state_batch_indices=None, cu_seqlens=None,
             num_accepted_tokens=np.random.default_rng(3).integers(0, 4, 12).astype(np.int32))
    G.check(c, "one token with accepted counts")


def test_strided_literal_view():
    """A [rows, 1] table view with strides (1, 1): sequence b, position t is
    entry b + t (one sequence)."""
    c = W.mtp(nseq=1, steps=6, heads=8, dim=64, dstate=128, groups=2, pad_slot_id=-1)
    c["num_accepted_tokens"] = np.array([4], np.int32)
    c["state_batch_indices"] = W.Strided(c["state_batch_indices"].ravel(), (6, 1), (1, 1))
    c["dst_state_batch_indices"] = W.Strided(c["dst_state_batch_indices"].ravel(), (6, 1), (1, 1))
    G.check(c, "strided literal view")


def test_packed_without_tables():
    """cu_seqlens without tables: sequence b reads and writes slot b."""
    c = W.varlen(nseq=12, heads=8, dim=64, dstate=128, state_dtype="bf16")
    c["state_batch_indices"] = c["dst_state_batch_indices"] = None
    c["state"] = c["state"][:12]
    G.check(c, "packed without tables")


def test_per_head_dt_as_stride0_view():
    c = W.varlen(nseq=10, heads=8, dim=64, dstate=128, state_dtype="f32")
    ref = ssu_oracle.run(c)
    d = G.device_case(c)
    d["dt"] = d["dt"][:, :, None].expand(-1, -1, 64)  # stride 0 over dim
    assert d["dt"].stride(2) == 0
    G.say("[gpu] per-head dt stride-0 view: launching")
    y, s = G.run_gpu(c, d=d)
    G.compare(c, y, s, ref, "per-head dt view")


def test_empty_inputs():
    c = W.varlen(nseq=6, heads=4, dim=64, dstate=128, lengths=[0, 0, 0, 0, 0, 0])
    assert c["x"].shape[0] == 0
    G.say("[gpu] all-empty varlen: launching")
    y, s = G.run_gpu(c)
    assert y.shape[0] == 0 and np.array_equal(s, c["state"])
    c = W.varlen(nseq=6, heads=4, dim=64, dstate=128, lengths=[0, 3, 0, 0, 1, 0])
    G.check(c, "mostly empty varlen")
    c = W.decode(batch=0, heads=4, dim=64, dstate=128, groups=2, slots=4)
    y, s = G.run_gpu(c)
    assert y.shape[0] == 0 and np.array_equal(s, c["state"])


@pytest.mark.parametrize("kind", ["in_place_decode", "varlen_dst_omitted"])
def test_alias_repeat10(kind):
    """Read slot == write slot (in-place decode; a sequence writing the entry
    it read): 10 repeats from the same snapshot give the oracle's result
    every time (the repeat-10 snapshot method of the PR #50729 digest)."""
    if kind == "in_place_decode":
        c = W.decode(batch=64, heads=16, dim=64, dstate=128, groups=4, slots=96)
    else:
        c = W.varlen(nseq=48, heads=8, dim=64, dstate=128, dst=False)
    ref = ssu_oracle.run(c)
    d = G.device_case(c)
    snap = d["state"].clone()
    first = None
    for i in range(10):
        d["state"].copy_(snap)
        y, s = G.run_gpu(c, d=d)
        G.compare(c, y, s, ref, "%s repeat %d" % (kind, i))
        if first is None:
            first = (y.copy(), s.copy())
        else:
            assert np.array_equal(first[0], y) and np.array_equal(first[1], s)
    G.say("[gpu] %s: 10 repeats identical" % kind)


def test_prewarm_output_only():
    """With packed and disable_state_update, prewarm selects the variant such
    calls take and reports its tiling: the matrix-core form's 64-row tiles
    (fp16 state, bf16 io, dstate 128), the VALU form's 16-row tiles (fp32
    state); a 16-bit state with fp32 outputs has no output-only variant and
    keeps the update kernel."""
    def pre(sd, io, disable):
        return G.ssu.prewarm_selective_state_update(
            state_dtype=sd, io_dtype=io, batch=512, heads=64, dim=64, dstate=128, groups=1,
            slot_dtype=torch.int32, packed=True, disable_state_update=disable)
    info = pre(torch.float16, torch.bfloat16, True)
    assert info["kernel"] == "ssu_packed_output_only_f16_bf16_n128"
    assert (info["block_threads"], info["rows_per_block"], info["blocks_per_seq_head"]) == (64, 64, 1)
    info = pre(torch.float32, torch.bfloat16, True)
    assert info["kernel"] == "ssu_packed_output_only_f32_bf16_n128"
    assert (info["rows_per_block"], info["blocks_per_seq_head"]) == (16, 4)
    info = pre(torch.float16, torch.float32, True)
    assert info["kernel"] == "ssu_packed_f16_f32_n128"
    assert pre(torch.float16, torch.bfloat16, False)["kernel"] == "ssu_packed_f16_bf16_n128"


def test_prewarm_and_graph_replay():
    """prewarm selects and loads the kernel; the update captured in a HIP
    graph replays to the eager result (read and write slots differ, so each
    replay computes the same thing)."""
    info = G.ssu.prewarm_selective_state_update(
        state_dtype=torch.float32, io_dtype=torch.bfloat16, batch=16, heads=8, dim=64,
        dstate=128, groups=2, slot_dtype=torch.int32, packed=True)
    assert info["kernel"] == "ssu_packed_f32_bf16_n128"
    assert info["block_threads"] in (64, 128, 192, 256)
    assert info["rows_per_block"] * info["blocks_per_seq_head"] >= 64
    assert info["rows_per_block"] * (info["blocks_per_seq_head"] - 1) < 64
    c = W.mtp(nseq=8, steps=4, heads=8, dim=64, dstate=128, groups=2, pad_slot_id=-1)
    ref = ssu_oracle.run(c)
    d = G.device_case(c)
    snap = d["state"].clone()
    out = torch.empty(c["x"].shape, dtype=torch.bfloat16, device="cuda:0")
    stream = torch.cuda.Stream()
    args = G.ssu.make_args(d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                           d["z"], d["dt_bias"], True, d["state_batch_indices"], -1, out, False,
                           d["dst_state_batch_indices"], d["cu_seqlens"],
                           d["num_accepted_tokens"])
    G.say("[gpu] graph capture: capturing")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        G.ssu.ssu_update(args, torch.cuda.current_stream().cuda_stream)
    for i in range(3):
        out.fill_(float("nan"))
        d["state"].copy_(snap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        G.compare(c, G.host(out, "bf16"), G.host(d["state"], "f32"), ref, "replay %d" % i)
    G.say("[gpu] graph replay: ok")


# ---------------------------------------------------------------- full sizes

def _full(case, name):
    """Full-size case in the benchmark's launch configuration, every sequence
    against the oracle's whole result: untouched slots byte-identical,
    written slots and every row of y within the tolerances."""
    G.say("[gpu] %s: oracle" % name)
    ref = ssu_oracle.run(case)
    d = G.device_case(case)
    snap = d["state"].clone()
    G.say("[gpu] %s: launching" % name)
    y, d = G.run_gpu(case, d=d, sync=False)
    torch.cuda.synchronize()
    stats = G.compare_full(case, ref, y, d["state"], snap, name)
    G.say("[gpu] %s: ok %s" % (name, {k: "%.3g" % v for k, v in stats.items()}))


def test_full_decode():
    _full(W.decode(), "decode batch 256 fp32 state")


@pytest.mark.parametrize("pad", [0, -1])
def test_full_decode_pad(pad):
    _full(W.decode_pad(pad_slot_id=pad), "decode_pad batch 1024 bf16 state, pad id %d" % pad)


@pytest.mark.parametrize("pad", [0, -1])
def test_full_mtp(pad):
    _full(W.mtp(pad_slot_id=pad), "mtp 64x7 fp32 state, pad id %d" % pad)


@pytest.mark.parametrize("mode", ["dst", "disable", "omitted"])
def test_full_varlen(mode):
    c = W.varlen(dst=mode != "omitted", disable=mode == "disable")
    _full(c, "varlen 512 seqs fp16 state (%s)" % mode)
