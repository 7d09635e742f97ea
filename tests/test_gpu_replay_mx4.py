"""ReplaySSM decode with an MXFP4 read copy of the checkpoint
(ssu_replay_mx4_update, ssu_mx4_quantize) against the CPU oracle (ReplaySSM
article, section "数据与边界", which measures a 4-bit copy; OCP Microscaling
v1.0, MXFP4 with E2M1 elements).

As for the MXFP8 copy: output-only steps read the copy, so y is compared with
the oracle run on the same copy bytes; a flush stores the fp32 checkpoint and
rewrites the copy, whose bytes are the quantization of the stored state,
exactly."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import workloads as W
from oracle import ssu_oracle
import mamba_selective_state_amd as ssu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


# ---------------------------------------------------------------- quantizer

def gpu_quantize(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")
    codes, scales = ssu.mx4_quantize(t)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def special_blocks():
    """Blocks that exercise every branch of the conversion: the midpoints
    between neighbouring E2M1 values (ties go to the even code) and points
    just beside them, at several scales, saturation, zeros, NaN, fp32
    subnormals (the clamped scale exponent) and the largest fp32
    magnitudes."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    rows = []
    for k in (-120, -20, -3, 0, 7, 100):
        # amax 4 * 2^k gives the scale 2^k exactly
        X = 2.0 ** k
        vals = []
        for m in mids:
            vals += [m, m * (1 + 2.0 ** -20), m * (1 - 2.0 ** -20)]
        vals += grid
        v = np.array(vals, np.float64) * X
        sgn = np.where(np.arange(v.size) % 3 == 1, -1.0, 1.0)
        v = (v * sgn).astype(np.float32)
        v = np.concatenate([v, np.zeros((-v.size) % 32, np.float32)])
        v[2 + 32 * np.arange(v.size // 32)] = 4.0 * X  # each block keeps amax 4 * 2^k
        rows.append(v.reshape(-1, 32))
    sat = np.full(32, 1.0, np.float32)
    sat[0] = 7.9  # scale 2^0: 7.9 and -7 saturate to 6
    sat[1] = -7.0
    sat[2] = 6.99
    rows.append(sat[None])
    rows.append(np.zeros((1, 32), np.float32))
    nan = np.linspace(-1, 1, 32).astype(np.float32)
    nan[4] = np.nan
    nan[9] = -np.nan
    rows.append(nan[None])
    tiny = (np.arange(32) * 1e-41).astype(np.float32)  # fp32 subnormals: scale 2^-126
    rows.append(tiny[None])
    huge = np.full(32, 3.0e38, np.float32)             # the largest scale an fp32 block reaches
    huge[::2] = -1.0e38
    rows.append(huge[None])
    return np.concatenate(rows).ravel()


def test_mx4_quantize_special_values():
    x = special_blocks()
    G.say("[gpu] mx4 quantize, %d special values: launching" % x.size)
    codes, scales = gpu_quantize(x)
    rc, rs = ssu_oracle.mx4_quantize(x)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)
    G.say("[gpu] mx4 quantize special: ok")


@pytest.mark.parametrize("nblocks", [1, 3, 64, 4095, 20001])
def test_mx4_quantize_random(nblocks):
    rng = np.random.default_rng(nblocks + 7)
    x = (rng.standard_normal(nblocks * 32) *
         np.repeat(np.exp2(rng.integers(-30, 30, nblocks)), 32)).astype(np.float32)
    G.say("[gpu] mx4 quantize %d blocks: launching" % nblocks)
    codes, scales = gpu_quantize(x)
    rc, rs = ssu_oracle.mx4_quantize(x)
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)


def test_mx4_quantize_pool_size():
    """More blocks than the grid has lanes for (the grid-stride loop runs more
    than once) with a ragged tail; the replay benchmark's pool is this
    large."""
    nblocks = 65536 * 64 + 17
    rng = np.random.default_rng(4)
    x = rng.standard_normal(nblocks * 32, dtype=np.float32)
    G.say("[gpu] mx4 quantize %d blocks: launching" % nblocks)
    codes, scales = gpu_quantize(x)
    rc, rs = ssu_oracle.mx4_quantize(x)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)
    G.say("[gpu] mx4 quantize pool size: ok")


# ---------------------------------------------------------------- replay

CASES = [
    # (io, L, dt per head, dstate, dim)
    ("bf16", 16, False, 128, 64),
    ("bf16", 4, True, 128, 40),
    ("f16", 8, False, 64, 64),
    ("f32", 5, False, 32, 28),
    ("bf16", 16, False, 256, 64),
    ("f16", 33, True, 64, 64),
]


@pytest.mark.parametrize("io,L,per_head,N,P", CASES,
                         ids=["%s-L%d-%s-n%d-p%d" % (a, b, "ph" if c else "full", d, e)
                              for a, b, c, d, e in CASES])
def test_replay_mx4_small(io, L, per_head, N, P):
    c = W.replay(seed=60 + L + N, batch=24, heads=8, dim=P, dstate=N, groups=2, slots=40, L=L,
                 io=io, dt_per_head=per_head)
    c["buf_len"][:] = np.arange(24) % L
    c["buf_len"][:3] = [0, L - 1, L // 2]
    G.check_replay_lp(G.with_copy(c, fmt="mx4"), "replay mx4 %s L=%d n=%d" % (io, L, N))


def test_replay_mx4_reads_the_copy():
    """A copy that differs from the checkpoint (here: of half the pool): the
    output-only steps follow the copy, the flushes the checkpoint."""
    c = W.replay(seed=61, batch=32, heads=8, dim=64, dstate=128, groups=2, slots=48, L=8)
    c["buf_len"][:] = np.arange(32) % 8
    half = np.asarray(c["state"], np.float32) * 0.5
    G.check_replay_lp(G.with_copy(c, half, fmt="mx4"), "replay mx4, stale copy")
    plain = ssu_oracle.run_replay(c)
    lp = ssu_oracle.run_replay(G.with_copy(c, half, fmt="mx4"))
    assert not np.array_equal(plain["y"], lp["y"])


def test_replay_mx4_pad_and_disable():
    c = W.replay(seed=62, batch=12, heads=8, dim=64, dstate=128, groups=2, slots=20, L=4)
    tab = c["state_batch_indices"].copy()
    tab[[1, 5]] = -1
    c["state_batch_indices"] = tab
    c["buf_len"][:] = [3, 3, 1, 3, 0, 2, 3, 1, 2, 3, 0, 3]
    c = G.with_copy(c, fmt="mx4")
    G.check_replay_lp(c, "replay mx4 with pad rows")
    G.check_replay_lp(dict(c, disable_state_update=True), "replay mx4 disabled")


def test_replay_mx4_sequence_of_steps():
    """Twenty steps of a caller's loop (buf_len advanced, reset after a fold),
    the copy carried on the GPU: every step's y and the final pool, buffers
    and copy equal the oracle's chain."""
    L = 4
    c = G.with_copy(W.replay(seed=63, batch=16, heads=8, dim=64, dstate=64, groups=2, slots=24,
                             L=L), fmt="mx4")
    d = G.device_replay_lp(c)
    rng = np.random.default_rng(64)
    cur = dict(c)
    for step in range(20):
        if step:
            fresh = W.replay(seed=200 + step, batch=16, heads=8, dim=64, dstate=64, groups=2,
                             slots=24, L=L)
            for k in ("x", "dt", "B", "C", "z"):
                cur[k] = fresh[k]
                dtype = c.get("dt_dtype", c["io_dtype"]) if k == "dt" else c["io_dtype"]
                d[k] = G.dev(fresh[k], dtype, "cuda:0")
        ref = ssu_oracle.run_replay(cur)
        got = G.run_gpu_replay_lp(cur, d=d)
        G.compare_replay(cur, got, ref, "mx4 step %d" % step)
        G.compare_copy(cur, got, ref, "mx4 step %d" % step)
        for k in ("state", "buf_x", "buf_dt", "buf_B", "lp", "lp_scale"):
            cur[k] = got[k]
        blen = np.asarray(cur["buf_len"]) + 1
        blen[blen == L] = 0
        skip = rng.random(16) < 0.2
        blen[skip] = np.asarray(cur["buf_len"])[skip]
        cur["buf_len"] = blen.astype(np.int32)
        d["buf_len"] = torch.from_numpy(cur["buf_len"]).to("cuda:0")
    G.say("[gpu] replay mx4 20 steps: ok")


def test_replay_mx4_full_workload():
    """The replay benchmark's workload with its MXFP4 copy made on the GPU:
    the copy equals the oracle's quantization of the pool; then every
    sequence of the step against the oracle's whole step (pool, y, buffers,
    copy)."""
    c = W.replay()
    G.say("[gpu] replay mx4 full: quantizing")
    d = G.device_replay(c)
    d["lp"], d["lp_scale"] = ssu.mx4_quantize(d["state"])
    torch.cuda.synchronize()
    lp0, lps0 = d["lp"].cpu().numpy(), d["lp_scale"].cpu().numpy()
    rc, rs = ssu_oracle.mx4_quantize(np.asarray(c["state"], np.float32))
    assert np.array_equal(lps0, rs) and np.array_equal(lp0, rc)
    c = dict(c, lp=lp0, lp_scale=lps0, lp_format="mx4")
    G.say("[gpu] replay mx4 full: oracle")
    ref = ssu_oracle.run_replay(c)
    G.say("[gpu] replay mx4 full: launching")
    got = G.run_gpu_replay_lp(c, d=d)
    stats = G.compare_replay(c, got, ref, "replay mx4 full")
    stats["copy_mismatch"] = G.compare_copy(c, got, ref, "replay mx4 full")
    G.say("[gpu] replay mx4 full: ok %s" % {k: "%.3g" % v for k, v in stats.items()})
