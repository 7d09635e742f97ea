"""memmove-safe Mamba state copies on the GPU (ssu_batch_memcpy,
ssu_conv_state_shift) against the CPU oracle and against slices of the
untouched snapshot, each case repeated 10 times (vLLM PR #50729 digest,
"测试配套": the race is intermittent, so a single pass proves little)."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import workloads as W
from oracle import ssu_oracle

pytestmark = pytest.mark.gpu
REPEAT = 10


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


def run_memcpy(c, repeat=REPEAT, max_size=None):
    """Device copies of c["buf"] per c's offsets; checks every repetition
    against the snapshot's slices and the oracle."""
    buf = torch.from_numpy(c["buf"]).to("cuda:0")
    snap = buf.clone()
    base = buf.data_ptr()
    src = (torch.from_numpy(np.asarray(c["src_off"], np.int64)) + base).to("cuda:0")
    dst = (torch.from_numpy(np.asarray(c["dst_off"], np.int64)) + base).to("cuda:0")
    sizes = torch.from_numpy(np.asarray(c["sizes"])).to("cuda:0")
    want = c["buf"].copy()
    for s, d, n in zip(c["src_off"], c["dst_off"], c["sizes"]):
        if n > 0:
            want[d:d + n] = c["buf"][s:s + n]
    ref = ssu_oracle.run_batch_memmove(c["buf"], c["src_off"], c["dst_off"], np.maximum(c["sizes"], 0))
    assert np.array_equal(ref, want)
    for r in range(repeat):
        buf.copy_(snap)
        G.ssu.batch_memcpy(src, dst, sizes, max_size)
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        assert np.array_equal(got, want), "repetition %d" % r


@pytest.mark.parametrize("direction", ["left", "right", "apart"])
@pytest.mark.parametrize("shift", [16, 1, 6, 4096])
def test_batch_memcpy_rows(direction, shift):
    """The PR's regression case (128 rows x 32 KiB shifted left by 16 bytes,
    a mod-251 pattern) and its mirror and misaligned variants."""
    G.say("[gpu] batch memcpy %s shift %d" % (direction, shift))
    run_memcpy(W.memmove_rows(rows=128, row_bytes=32 * 1024, shift=shift, direction=direction))


@pytest.mark.parametrize("direction", ["left", "right"])
def test_batch_memcpy_partial_second_chunk(direction):
    """Overlapping rows of 24 KiB + 48 bytes in 16-byte words: one full
    chunk of 256 lanes x 4 words and a partial one, read whole before any
    store."""
    G.say("[gpu] batch memcpy partial second chunk %s" % direction)
    run_memcpy(W.memmove_rows(rows=64, row_bytes=24 * 1024 + 48, shift=32, direction=direction))


def test_batch_memcpy_large_and_empty():
    """One 8 MiB copy shifted onto itself (many ordered chunks), large disjoint
    copies beyond the max_size hint (tiles loop), and zero / negative sizes."""
    G.say("[gpu] batch memcpy large")
    c = W.memmove_rows(rows=1, row_bytes=8 << 20, shift=4096 + 8, direction="left")
    run_memcpy(c, repeat=3)
    c = W.memmove_rows(rows=1, row_bytes=8 << 20, shift=12, direction="right")
    run_memcpy(c, repeat=3)
    c = W.memmove_rows(rows=4, row_bytes=1 << 20, direction="apart")
    run_memcpy(c, repeat=2, max_size=4096)
    c = W.memmove_rows(rows=6, row_bytes=4096, shift=16, direction="left")
    c["sizes"][[1, 4]] = [0, -5]
    run_memcpy(c, repeat=2)


def run_shift(c, repeat=REPEAT):
    pool = c["pool"]
    dev = torch.from_numpy(pool.view(np.uint8)).to("cuda:0").view(
        {1: torch.uint8, 2: torch.float16, 4: torch.float32, 8: torch.float64}[pool.itemsize])
    dev = dev.reshape(pool.shape)
    snap = dev.clone()
    idx = {k: torch.from_numpy(np.asarray(c[k])).to("cuda:0") for k in ("src_blk", "dst_blk", "bias")}
    ref = ssu_oracle.run_conv_shift(pool, c["layout"], c["src_blk"], c["dst_blk"], c["bias"])
    want = pool.copy()
    Wd = pool.shape[1] if c["layout"] == "SD" else pool.shape[2]
    for s, d, b in zip(c["src_blk"], c["dst_blk"], c["bias"]):
        if 0 <= b <= Wd and 0 <= s < pool.shape[0] and 0 <= d < pool.shape[0]:
            if c["layout"] == "SD":
                want[d, :Wd - b] = pool[s, b:].copy()
            else:
                want[d, :, :Wd - b] = pool[s, :, b:].copy()
    assert np.array_equal(ref.view(np.uint8), want.view(np.uint8))
    for r in range(repeat):
        dev.copy_(snap)
        G.ssu.conv_state_shift(dev, idx["src_blk"], idx["dst_blk"], idx["bias"], c["layout"])
        torch.cuda.synchronize()
        got = dev.cpu().numpy().view(np.uint8).reshape(want.view(np.uint8).shape)
        assert np.array_equal(got, want.view(np.uint8)), "repetition %d" % r


@pytest.mark.parametrize("layout", ["SD", "DS"])
@pytest.mark.parametrize("dtype", [np.float16, np.float32, np.float64])
def test_conv_shift(layout, dtype):
    """Same and distinct blocks, biases 1..3 (the PR's accept-token biases),
    fp16 / fp32 / fp64 conv states, both layouts."""
    G.say("[gpu] conv shift %s %s" % (layout, np.dtype(dtype).name))
    c = W.conv_shift(seed=3, requests=48, width=4, inner=1000, dtype=dtype, layout=layout)
    run_shift(c)


def test_conv_shift_edges():
    """Bias 0 and W, width 3 and 7, inner sizes not a multiple of a chunk,
    byte elements, and out-of-range requests (written nowhere)."""
    G.say("[gpu] conv shift edges")
    for layout in ("SD", "DS"):
        for width, inner in ((3, 37), (7, 300), (4, 8192)):
            c = W.conv_shift(seed=width, requests=12, width=width, inner=inner, dtype=np.uint8,
                             layout=layout)
            c["bias"][:4] = [0, width, 1, width - 1]
            run_shift(c, repeat=3)
        c = W.conv_shift(seed=5, requests=6, width=4, inner=64, dtype=np.float32, layout=layout)
        c["bias"][0] = 5
        c["bias"][1] = -1
        c["src_blk"][2] = 999
        c["dst_blk"][3] = -2
        run_shift(c, repeat=2)


# ---------------------------------------------------------------- full sizes

def test_memcpy_left_full_workload():
    """The benchmark's memcpy_left workload (4096 rows of 32 KiB, each moved
    onto itself 16 bytes to the left) with its max_size, twice, every byte
    against the snapshot and the oracle."""
    import bench
    c, _ = bench.workload("memcpy_left")
    G.say("[gpu] memcpy_left full: launching")
    run_memcpy(c, repeat=2, max_size=int(np.max(c["sizes"])))
    G.say("[gpu] memcpy_left full: ok")


@pytest.mark.parametrize("config", ["conv_shift_sd", "conv_shift_ds"])
def test_conv_shift_full_workload(config):
    """The benchmark's convolution-state shift workloads (6144 shifts of
    64 KiB fp16 blocks, half inside one block), twice, every byte against
    the snapshot and the oracle."""
    import bench
    c, _ = bench.workload(config)
    G.say("[gpu] %s full: launching" % config)
    run_shift(c, repeat=2)
    G.say("[gpu] %s full: ok" % config)


def test_temporal_state_copy():
    """Temporal (SSM) state copies of a speculative step (vLLM PR #50729
    digest, "功能与动机" and the temporal-copy test it names): each sequence
    b holds its per-position states in blocks bt[b, 0..K-1] of a pool of
    [heads, dim, dstate] fp32 states; after acceptance, the state of the
    last accepted position bt[b, bias] moves whole into bt[b, 0] (bias =
    accepted - 1, copies only for bias >= 1, biases up to K - 1 >= 2). The
    reading: whole-block copies between distinct blocks, which the batched
    copy serves (no layout-aware kernel of its own); checked against the
    snapshot's slices and the oracle, 10 repetitions."""
    rng = np.random.default_rng(77)
    batch, K, heads, dim, dstate = 24, 4, 8, 64, 128
    block = heads * dim * dstate * 4
    slots = batch * K + 8
    perm = rng.permutation(slots)[:batch * K].reshape(batch, K)
    bias = rng.integers(0, K, batch)
    bias[:3] = [0, 2, K - 1]
    pool = rng.standard_normal(slots * heads * dim * dstate).astype(np.float32).view(np.uint8)
    src = [int(perm[b, bias[b]]) * block for b in range(batch) if bias[b] >= 1]
    dst = [int(perm[b, 0]) * block for b in range(batch) if bias[b] >= 1]
    c = {"buf": pool.copy(), "src_off": np.asarray(src, np.int64), "dst_off": np.asarray(dst, np.int64),
         "sizes": np.full(len(src), block, np.int64)}
    G.say("[gpu] temporal state copy: %d blocks of %d bytes" % (len(src), block))
    run_memcpy(c, max_size=block)
