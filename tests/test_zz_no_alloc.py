"""The allocation-free SSD prefill (ssu_ssd_prefill_noalloc: its workspace
is the library's own device array) through the C ABI, against the prefill
that takes a caller's workspace (ssu_ssd_prefill) on the same inputs, and
against the oracle: two calls in a row on one device, the second smaller,
so the second runs on an array that still holds the first call's data."""
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


def _device(c, dev="cuda:0"):
    io, sd = c["io_dtype"], c["state_dtype"]
    d = {k: G.dev(c[k], io, dev) for k in ("x", "B", "C")}
    d["z"] = None if c.get("z") is None else G.dev(c["z"], io, dev)
    d["dt"] = G.dev(c["dt"], c["dt_dtype"], dev)
    for k in ("cu_seqlens", "cu_chunk_seqlens", "last_chunk_indices", "seq_idx"):
        d[k] = torch.from_numpy(np.asarray(c[k])).to(dev)
    d["init"] = None if c.get("initial_states") is None else G.dev(c["initial_states"], sd, dev)
    for k in ("A", "D", "dt_bias"):
        d[k] = None if c.get(k) is None else torch.from_numpy(c[k]).to(dev)
    return d


def _run(c, d, noalloc, intermediate=False):
    """One prefill; returns (y, states) on the host."""
    io, sd = c["io_dtype"], c["state_dtype"]
    nchunks = len(c["seq_idx"])
    rows = nchunks if intermediate else len(c["last_chunk_indices"])
    out = torch.full(np.shape(c["x"]), float("nan"), dtype=G.TORCH[io], device="cuda:0")
    states = torch.full((rows,) + tuple(np.shape(c["x"])[1:]) + (np.shape(c["B"])[2],), float("nan"),
                        dtype=G.TORCH[sd], device="cuda:0")
    a = G.ssu.make_ssd_args(d["x"], d["dt"], d["A"], d["B"], d["C"], c["chunk_size"], d["cu_seqlens"],
                            d["cu_chunk_seqlens"], d["last_chunk_indices"], d["seq_idx"], out, states,
                            D=d["D"], z=d["z"], dt_bias=d["dt_bias"], dt_softplus=c["dt_softplus"],
                            dt_limit=c["dt_limit"], initial_states=d["init"],
                            return_intermediate_states=intermediate)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        G.ssu.ssu_ssd_prefill_noalloc(a, stream)
    else:
        nbytes = G.ssu.ssu_ssd_workspace_bytes(np.shape(c["x"])[1], 64, np.shape(c["B"])[2], nchunks)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda:0")
        G.ssu.ssu_ssd_prefill(a, ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    return G.host(out, io), G.host(states, sd)


def test_ssd_noalloc_matches_workspace_entry_point():
    big = W.ssd(seed=21, lengths=(700, 256, 1, 513, 1200), heads=16, dim=64, dstate=128, groups=2,
                chunk_size=256, io="bf16", state_dtype="f32", initial_states=True)
    small = W.ssd(seed=22, lengths=(90, 200), heads=8, dim=64, dstate=64, groups=2, chunk_size=64,
                  io="bf16", state_dtype="f32", initial_states=True)
    for name, c, inter in (("first, 13 chunks x 16 heads", big, False),
                           ("second, smaller: 5 chunks x 8 heads", small, True)):
        assert G.ssu.ssu_ssd_workspace_bytes(np.shape(c["x"])[1], 64, np.shape(c["B"])[2],
                                             len(c["seq_idx"])) <= G.ssu.SSD_SCRATCH_BYTES
        G.say("[gpu] ssd noalloc %s: launching both entry points" % name)
        d = _device(c)
        y_ws, s_ws = _run(c, d, noalloc=False, intermediate=inter)
        y_na, s_na = _run(c, d, noalloc=True, intermediate=inter)
        # the same kernels on the same inputs: the same bytes
        assert np.array_equal(y_na, y_ws), name
        assert np.array_equal(s_na, s_ws), name
        ref = ssu_oracle.run_ssd(c)
        io, sd = c["io_dtype"], c["state_dtype"]
        ry = G.brute64.to_f64(ref["y"], io)
        ey = float(np.abs(G.brute64.to_f64(y_na, io) - ry).max())
        want = ref["chunk_states"] if inter else ref["states"]
        rs = G.brute64.to_f64(want, sd)
        es = float(np.abs(G.brute64.to_f64(s_na, sd) - rs).max())
        assert ey <= 2e-2 * np.abs(ry).max() and es <= 2e-2 * np.abs(rs).max(), (name, ey, es)
        G.say("[gpu] ssd noalloc %s: ok (identical to the workspace entry point)" % name)
