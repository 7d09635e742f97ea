"""ReplaySSM decode on the GPU (ssu_replay_update) against its CPU oracle,
and against the plain update it must reproduce (ReplaySSM article, section
"核心做法": with L = 1 the step is the baseline; a flush folds the buffered
inputs into the checkpoint)."""
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


CASES = [
    # (state, io, L, dt per head, dstate, dim)
    ("f32", "bf16", 16, False, 128, 64),
    ("f32", "bf16", 4, True, 128, 64),
    ("bf16", "bf16", 8, False, 128, 40),
    ("f16", "f16", 3, True, 64, 64),
    ("f32", "f32", 5, False, 32, 28),
    ("f32", "bf16", 2, False, 256, 64),
    # long windows for each split of a dim row's window into runs of steps
    # (8 runs: fp32 state, dstate 256; 4: fp32, dstate 128; 2: 16-bit state)
    ("f32", "bf16", 16, False, 256, 64),
    ("bf16", "bf16", 16, True, 128, 64),
    ("f32", "f16", 33, False, 64, 64),
]


@pytest.mark.parametrize("sd,io,L,per_head,N,P", CASES,
                         ids=["%s-%s-L%d-%s-n%d-p%d" % (a, b, c, "ph" if d else "full", e, f)
                              for a, b, c, d, e, f in CASES])
def test_replay_small(sd, io, L, per_head, N, P):
    c = W.replay(seed=20 + L + N, batch=24, heads=8, dim=P, dstate=N, groups=2, slots=40, L=L,
                 state_dtype=sd, io=io, dt_per_head=per_head)
    # make sure both kinds of step occur, and every window length up to L
    c["buf_len"][:] = np.arange(24) % L
    c["buf_len"][:3] = [0, L - 1, L // 2]
    G.check_replay(c, "replay %s %s L=%d" % (sd, io, L))


@pytest.mark.parametrize("batch", [100, 513])
def test_replay_fill_order(batch):
    """Sequences that fill their buffer are taken first when the batch is at
    most 512 (a scan of every count), in batch order otherwise: a batch over
    several 64-sequence blocks with a partial last one, and one past the
    scan's limit, each with fills scattered through it."""
    L = 6
    c = W.replay(seed=30 + batch, batch=batch, heads=4, dim=64, dstate=64, groups=2,
                 slots=batch + 8, L=L)
    rng = np.random.default_rng(batch)
    c["buf_len"][:] = rng.integers(0, L, batch)
    c["buf_len"][rng.random(batch) < 0.2] = L - 1
    G.check_replay(c, "replay fill order, batch %d" % batch)


def test_replay_L1_equals_plain_kernel():
    """L = 1: every step is a fill of one step, whose state update is the
    plain one-token kernel's arithmetic: the pools agree bit for bit. y is the
    same dot product S . C summed in another order (4 values a lane over 32
    lanes against 8 over 16), so the two bf16 outputs are at most one
    rounding apart."""
    for sd in ("f32", "bf16"):
        c = W.replay(seed=7, batch=32, heads=16, dim=64, dstate=128, groups=4, slots=48, L=1,
                     state_dtype=sd, buf_len=0)
        G.say("[gpu] replay L=1 vs plain (%s): launching" % sd)
        got = G.run_gpu_replay(c)
        plain = {k: v for k, v in c.items() if not k.startswith("buf") and k != "L"}
        y, s = G.run_gpu(plain)
        assert np.array_equal(got["state"], s), sd
        gy = G.brute64.to_f64(got["y"], c["io_dtype"])
        py = G.brute64.to_f64(y, c["io_dtype"])
        # one bf16 step (8 significant bits) of the larger magnitude
        assert (np.abs(gy - py) <= np.maximum(np.abs(gy), np.abs(py)) * 2.0 ** -7).all(), sd


def test_replay_window_equals_chain():
    """A window of L steps from an empty buffer (the caller moves the
    pointer 0..L-1): outputs match the plain kernel's chained calls, and the
    checkpoint after the flush equals the plain kernel's pool bit for bit."""
    L = 6
    c = W.replay(seed=8, batch=16, heads=8, dim=64, dstate=128, groups=2, slots=24, L=L,
                 buf_len=0)
    plain = {k: v for k, v in c.items() if not k.startswith("buf") and k != "L"}
    d = G.device_replay(c)
    dp = G.device_case(plain)
    rng = np.random.default_rng(9)
    G.say("[gpu] replay window of %d steps: launching" % L)
    for t in range(L):
        for k in ("x", "dt", "B", "C", "z"):
            a = W.to_storage(rng.standard_normal(np.shape(c[k]), dtype=np.float32),
                             c["io_dtype"])
            c[k] = plain[k] = a
            d[k] = dp[k] = G.dev(a, c["io_dtype"], "cuda:0")
        d["buf_len"].fill_(t)
        got = G.run_gpu_replay(c, d=d)
        y, s = G.run_gpu(plain, d=dp)
        scale = np.abs(G.brute64.to_f64(y, "bf16")).max()
        err = np.abs(G.brute64.to_f64(got["y"], "bf16") - G.brute64.to_f64(y, "bf16")).max()
        assert err <= 2e-2 * scale, (t, err, scale)
        live = np.asarray(c["state_batch_indices"])
        if t < L - 1:
            assert np.array_equal(got["state"], c["state"]), t  # checkpoint untouched
        else:
            assert np.array_equal(got["state"][live], s[live])  # the fold is the chain


def test_replay_pad_and_disable():
    c = W.replay(seed=10, batch=12, heads=8, dim=64, dstate=128, groups=2, slots=20, L=4)
    tab = c["state_batch_indices"].copy()
    tab[[1, 5]] = -1
    c["state_batch_indices"] = tab
    c["buf_len"][[1, 5]] = [3, 2]  # ignored for pad rows
    G.check_replay(c, "replay with pad rows")
    G.check_replay(dict(c, disable_state_update=True), "replay disabled")


def test_replay_full_workload():
    """The benchmark's replay workload (decode layer, batch 256, L = 16):
    every sequence against the oracle's whole step (pool, y and the three
    buffers, bit for bit where they are raw copies)."""
    c = W.replay()
    G.say("[gpu] replay full: oracle")
    ref = ssu_oracle.run_replay(c)
    G.say("[gpu] replay full: launching")
    got = G.run_gpu_replay(c)
    stats = G.compare_replay(c, got, ref, "replay full")
    G.say("[gpu] replay full: ok %s" % {k: "%.3g" % v for k, v in stats.items()})


def test_replay_out_of_range_counts():
    """buf_len outside [0, L) for a live slot: that sequence's y is NaN and
    nothing of it is written; the other sequences are unaffected."""
    L = 8
    c = W.replay(seed=11, batch=12, heads=8, dim=64, dstate=128, groups=2, slots=20, L=L)
    bad = [2, 7, 9]
    c["buf_len"][bad] = [L, -1, L + 5]
    G.say("[gpu] replay out-of-range counts: launching")
    got = G.run_gpu_replay(c)
    assert np.isnan(G.brute64.to_f64(got["y"][bad], c["io_dtype"])).all()
    tab = np.asarray(c["state_batch_indices"])
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(got[k][tab[bad]], np.asarray(c[k])[tab[bad]]), k
    good = [b for b in range(12) if b not in bad]
    sub, used = G.replay_subcase(c, good)
    ref = ssu_oracle.run_replay(sub)
    sub_got = {"y": got["y"][good], "state": got["state"][used]}
    for k in ("buf_x", "buf_dt", "buf_B"):
        sub_got[k] = got[k][used]
    G.compare_replay(sub, sub_got, ref, "replay, valid rows")
