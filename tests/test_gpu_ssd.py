"""SSD packed variable-length prefill on the GPU (ssu_ssd_prefill) against the
CPU oracle (MATE docs, "Mamba / SSU", section "SSD packed prefill").

Tolerance: the products run on bf16 / f16 matrix cores, so every operand
that is scaled before a product (w_t x_t in the chunk states, the masked
and scaled C.B^T in the scan, the entering state read out by C) is rounded to the x
dtype: 2^-9 relative per operand, summed over at most chunk_size + dstate
terms of random sign. y and the returned states are compared at
2e-2 x max|ref| (the 16-bit tolerance of the decode path), on every
element; the largest error over max|ref| observed on MI355X is 0.0057 for y
and 0.0032 for the states (each case prints its own).
"""
import numpy as np
import pytest
import torch

import gpu_harness as G
import workloads as W
from oracle import ssu_oracle

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


def run_gpu_ssd(c, intermediate=False):
    dev = "cuda:0"
    io, sd = c["io_dtype"], c["state_dtype"]
    d = {k: G.dev(c[k], io, dev) for k in ("x", "B", "C")}
    d["z"] = None if c.get("z") is None else G.dev(c["z"], io, dev)
    d["dt"] = G.dev(c["dt"], c["dt_dtype"], dev)
    idx = {k: torch.from_numpy(np.asarray(c[k])).to(dev)
           for k in ("cu_seqlens", "cu_chunk_seqlens", "last_chunk_indices", "seq_idx")}
    init = None if c.get("initial_states") is None else G.dev(c["initial_states"], sd, dev)
    out = torch.full(np.shape(c["x"]), float("nan"), dtype=G.TORCH[io], device=dev)
    states = G.ssu.ssd_combined_fwd_varlen(
        d["x"], d["dt"], torch.from_numpy(c["A"]).to(dev), d["B"], d["C"], c["chunk_size"],
        idx["cu_seqlens"], idx["cu_chunk_seqlens"], idx["last_chunk_indices"], idx["seq_idx"],
        out=out, D=None if c.get("D") is None else torch.from_numpy(c["D"]).to(dev), z=d["z"],
        dt_bias=None if c.get("dt_bias") is None else torch.from_numpy(c["dt_bias"]).to(dev),
        dt_softplus=c["dt_softplus"], dt_limit=c["dt_limit"], initial_states=init,
        return_intermediate_states=intermediate, state_dtype=G.TORCH[sd])
    torch.cuda.synchronize()
    return G.host(out, io), G.host(states, sd)


def check_ssd(c, name, intermediate=False, heads=None):
    """GPU against the oracle; with `heads`, the oracle runs on those heads
    only (they are independent) and the GPU's full result is sliced."""
    ref = ssu_oracle.run_ssd(c if heads is None else W.ssd_heads(c, heads))
    G.say("[gpu] %s: launching" % name)
    y, st = run_gpu_ssd(c, intermediate)
    if heads is not None:
        y, st = y[:, heads], st[:, heads]
    io, sd = c["io_dtype"], c["state_dtype"]
    gy, ry = G.brute64.to_f64(y, io), G.brute64.to_f64(ref["y"], io)
    assert not np.isnan(gy).any(), "%s: a row of y was not written" % name
    ey = float(np.abs(gy - ry).max())
    assert ey <= TOL * np.abs(ry).max(), "%s: y error %g (max |ref| %g)" % (name, ey, np.abs(ry).max())
    want = ref["chunk_states"] if intermediate else ref["states"]
    gs, rs = G.brute64.to_f64(st, sd), G.brute64.to_f64(want, sd)
    es = float(np.abs(gs - rs).max())
    assert es <= TOL * np.abs(rs).max(), "%s: state error %g (max |ref| %g)" % (name, es, np.abs(rs).max())
    G.say("[gpu] %s: ok y %.3g state %.3g" % (name, ey / np.abs(ry).max(), es / np.abs(rs).max()))


CASES = [
    # (io, state, dstate, chunk_size, lengths, initial states)
    ("bf16", "f32", 128, 256, (700, 256, 1, 513, 1200), True),
    ("bf16", "bf16", 128, 64, (70, 16, 1, 33, 300), True),
    ("f16", "f32", 64, 128, (129, 128, 127, 5), False),
    ("bf16", "f16", 64, 256, (1000,), True),
    ("f16", "f16", 128, 32, (31, 64, 1, 2), True),
]


@pytest.mark.parametrize("io,sd,N,L,lengths,init", CASES,
                         ids=["%s-%s-n%d-L%d-%dseq" % (a, b, c, d, len(e)) for a, b, c, d, e, f in CASES])
def test_ssd_prefill(io, sd, N, L, lengths, init):
    c = W.ssd(seed=N + L, lengths=lengths, heads=8, dim=64, dstate=N, groups=2, chunk_size=L, io=io,
              state_dtype=sd, initial_states=init)
    check_ssd(c, "ssd %s %s n%d L%d" % (io, sd, N, L))


def test_ssd_intermediate_states_and_options():
    c = W.ssd(seed=3, lengths=(300, 40, 260), heads=8, dim=64, dstate=128, groups=1, chunk_size=128,
              io="bf16", state_dtype="f32", z=False, D=False, dt_dtype="bf16")
    check_ssd(c, "ssd intermediate states", intermediate=True)
    c = W.ssd(seed=4, lengths=(90, 200), heads=4, dim=64, dstate=64, groups=4, chunk_size=64,
              io="bf16", state_dtype="f32", softplus=False, dt_limit=(0.0, 0.05))
    check_ssd(c, "ssd no softplus, dt_limit (0, 0.05)")


def test_ssd_seq_idx_authority():
    """seq_idx decides openings: relabelling the second sequence's chunks
    as the first's continues its state on the GPU exactly as in the oracle."""
    c = W.ssd(seed=5, lengths=(100, 80), heads=8, dim=64, dstate=128, groups=2, chunk_size=64,
              io="bf16", state_dtype="f32", initial_states=False)
    c["seq_idx"] = np.zeros_like(c["seq_idx"])
    check_ssd(c, "ssd seq_idx relabelled")


def test_ssd_empty_chunks():
    """Zero-token chunks (cu_chunk_seqlens repeating an entry; MATE docs,
    "SSD packed prefill": that array alone maps chunks to tokens) inside a
    sequence, opening a sequence and ending one: the state passes through
    them unchanged, and a sequence whose last chunk is empty returns the
    state its chunk before left."""
    c = W.ssd(seed=21, lengths=(300, 130, 70), heads=8, dim=64, dstate=64, groups=2, chunk_size=128,
              io="bf16", state_dtype="f32")
    cu, seq = np.asarray(c["cu_chunk_seqlens"]), np.asarray(c["seq_idx"])
    chunks = [(int(cu[k]), int(cu[k + 1]), int(seq[k])) for k in range(len(seq))]
    # seq 0: chunks 0..2, seq 1: 3..4, seq 2: 5
    out = []
    for k, (a0, a1, q) in enumerate(chunks):
        if k == 3:
            out.append((a0, a0, q))      # an empty chunk opening sequence 1
        out.append((a0, a1, q))
        if k == 0:
            out.append((a1, a1, q))      # an empty chunk inside sequence 0
        if k == 5:
            out.append((a1, a1, q))      # an empty last chunk of sequence 2
    c["cu_chunk_seqlens"] = np.asarray([out[0][0]] + [e[1] for e in out], np.int64)
    c["seq_idx"] = np.asarray([e[2] for e in out], np.int64)
    c["last_chunk_indices"] = np.asarray([max(k for k, e in enumerate(out) if e[2] == b)
                                          for b in range(3)], np.int64)
    assert [e[1] - e[0] for e in out].count(0) == 3
    check_ssd(c, "ssd empty chunks")
    check_ssd(c, "ssd empty chunks, intermediate", intermediate=True)


def test_ssd_full_workload():
    """The benchmark's prefill workload at full size, every token and
    sequence, sampled over heads (the oracle runs on 3 of the 128)."""
    c = W.ssd_bench()
    check_ssd(c, "ssd bench workload", heads=[0, 77, 127])


@pytest.mark.parametrize("heads,groups", [(6, 1), (12, 4), (20, 2), (18, 1)],
                         ids=["6-per-group", "3-per-group", "10-per-group", "18-per-group"])
def test_ssd_head_blocks(heads, groups):
    """Heads per group that the fused kernel's 8-head blocks do not divide
    (6 and 3: one partial block; 10: 8 + 2; 18: 8 + 8 + 2), so the (group,
    head block) streams come in counts that do not fill the 8 virtual XCDs
    evenly, with intermediate states so every chunk's state is checked."""
    c = W.ssd(seed=7 + heads, lengths=(300, 17, 129), heads=heads, dim=64, dstate=128, groups=groups,
              chunk_size=128, io="bf16", state_dtype="f32")
    check_ssd(c, "ssd %d heads / %d groups" % (heads, groups))
    check_ssd(c, "ssd %d heads / %d groups, intermediate" % (heads, groups), intermediate=True)


@pytest.mark.parametrize("dim,heads,groups,N", [(128, 4, 2, 128), (192, 3, 1, 64), (256, 2, 2, 128)],
                         ids=["dim128", "dim192-3heads", "dim256"])
def test_ssd_wide_heads(dim, heads, groups, N):
    """Head dims that are multiples of 64 (each head runs as dim / 64 parts
    sharing its dt, A, D and group), with initial and intermediate states."""
    c = W.ssd(seed=dim + heads, lengths=(300, 17, 129), heads=heads, dim=dim, dstate=N, groups=groups,
              chunk_size=128, io="bf16", state_dtype="f32", initial_states=True)
    check_ssd(c, "ssd dim %d, %d heads / %d groups" % (dim, heads, groups))
    check_ssd(c, "ssd dim %d, intermediate" % dim, intermediate=True)


def test_ssd_tiny_chunks():
    """Seventeen sequences of 1..17 tokens at chunk size 16: every chunk is
    shorter than a 32-token block and most are ragged 16-row tiles."""
    c = W.ssd(seed=9, lengths=tuple(range(1, 18)), heads=8, dim=64, dstate=64, groups=2, chunk_size=16,
              io="f16", state_dtype="f32")
    check_ssd(c, "ssd tiny chunks")
    check_ssd(c, "ssd tiny chunks, intermediate", intermediate=True)


def test_ssd_many_chunks():
    """A long chain: 1252 chunks of 16 tokens, the first sequence's state
    handed through 1000 of them, final and intermediate states."""
    c = W.ssd(seed=13, lengths=(16000, 3000, 1000, 7), heads=4, dim=64, dstate=64, groups=1, chunk_size=16,
              io="bf16", state_dtype="f32")
    assert len(c["seq_idx"]) > 1024 and c["seq_idx"][1023] == c["seq_idx"][1024] == 1
    check_ssd(c, "ssd 1252 chunks")
    check_ssd(c, "ssd 1252 chunks, intermediate", intermediate=True)


def test_ssd_prewarm_then_graph_replay():
    """The prewarm loads the two kernels for a configuration; a prefill
    captured in a HIP graph afterwards replays to the eager result, every
    replay (eager work and synchronisation in between), and matches the
    oracle."""
    info = G.ssu.prewarm_ssd_combined_fwd_varlen(8, 2, 64, 128, 128, io_dtype=torch.bfloat16,
                                                 state_dtype=torch.float32, dt_dtype=torch.float32)
    assert info["launches"] == 2 and all(v > 0 for v in info["vgprs"])
    assert info["kernels"] == ["ssd_prep_kernel", "ssd_fused_kernel"]
    c = W.ssd(seed=31, lengths=(300, 17, 129), heads=8, dim=64, dstate=128, groups=2, chunk_size=128,
              io="bf16", state_dtype="f32", initial_states=True)
    ref = ssu_oracle.run_ssd(c)
    dev = "cuda:0"
    d = {k: G.dev(c[k], "bf16", dev) for k in ("x", "B", "C", "z")}
    dt = G.dev(c["dt"], c["dt_dtype"], dev)
    idx = {k: torch.from_numpy(np.asarray(c[k])).to(dev)
           for k in ("cu_seqlens", "cu_chunk_seqlens", "last_chunk_indices", "seq_idx")}
    init = G.dev(c["initial_states"], "f32", dev)
    A, D, bias = (torch.from_numpy(c[k]).to(dev) for k in ("A", "D", "dt_bias"))
    nchunks = len(c["seq_idx"])
    out = torch.empty_like(d["x"])
    states = torch.empty((len(c["last_chunk_indices"]), 8, 64, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(G.ssu.ssu_ssd_workspace_bytes(8, 64, 128, nchunks), dtype=torch.uint8, device=dev)
    a = G.ssu.make_ssd_args(d["x"], dt, A, d["B"], d["C"], c["chunk_size"], idx["cu_seqlens"],
                            idx["cu_chunk_seqlens"], idx["last_chunk_indices"], idx["seq_idx"], out,
                            states, D=D, z=d["z"], dt_bias=bias, dt_softplus=c["dt_softplus"],
                            dt_limit=c["dt_limit"], initial_states=init)
    G.say("[gpu] ssd graph: eager")
    G.ssu.ssu_ssd_prefill(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    y_eager, s_eager = G.host(out, "bf16"), G.host(states, "f32")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    G.say("[gpu] ssd graph: capturing")
    with torch.cuda.graph(g, stream=stream):
        G.ssu.ssu_ssd_prefill(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    for i in range(3):
        out.fill_(float("nan"))
        states.fill_(float("nan"))
        ws.fill_(255)  # the workspace holds nothing a call reads before writing it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(G.host(out, "bf16"), y_eager), i
        assert np.array_equal(G.host(states, "f32"), s_eager), i
    ry = G.brute64.to_f64(ref["y"], "bf16")
    assert np.abs(G.brute64.to_f64(y_eager, "bf16") - ry).max() <= TOL * np.abs(ry).max()
    rs = ref["states"].astype(np.float64)
    assert np.abs(s_eager.astype(np.float64) - rs).max() <= TOL * np.abs(rs).max()
    G.say("[gpu] ssd graph: 3 replays identical to the eager call")
