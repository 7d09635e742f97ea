"""ReplaySSM speculative step on the GPU (ssu_replay_spec_update) against its
CPU oracle (ReplaySSM article, section "投机解码回滚变成挪指针": T drafts read
out under a causal mask against one checkpoint and buffer window, appended to
the buffer; the fold comes at h + 2T > L)."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


CASES = [
    # (state, io, L, T, dt per head, dstate, dim)
    ("f32", "bf16", 16, 4, False, 128, 64),
    ("f32", "bf16", 16, 3, True, 128, 64),
    ("f32", "bf16", 9, 7, False, 128, 64),    # two draft groups
    ("bf16", "bf16", 12, 2, False, 128, 40),
    ("f16", "f16", 8, 1, True, 64, 64),
    ("f32", "f32", 10, 5, False, 32, 28),
    ("f32", "bf16", 16, 4, False, 256, 64),
]


@pytest.mark.parametrize("sd,io,L,T,per_head,N,P", CASES,
                         ids=["%s-%s-L%d-T%d-%s-n%d-p%d" % (a, b, c, d, "ph" if e else "full", f, g)
                              for a, b, c, d, e, f, g in CASES])
def test_replay_spec_small(sd, io, L, T, per_head, N, P):
    c = W.replay_spec(seed=40 + L + T + N, batch=24, T=T, heads=8, dim=P, dstate=N, groups=2,
                      slots=40, L=L, state_dtype=sd, io=io, dt_per_head=per_head)
    c["buf_len"][:] = np.arange(24) % (L + 1)  # every pointer 0..L, folding or not
    G.check_replay(c, "replay spec %s %s L=%d T=%d" % (sd, io, L, T))


def test_replay_spec_pad_and_disable():
    c = W.replay_spec(seed=41, batch=12, T=3, heads=8, dim=64, dstate=128, groups=2, slots=20, L=8)
    tab = c["state_batch_indices"].copy()
    tab[[1, 5]] = -1
    c["state_batch_indices"] = tab
    c["buf_len"][[1, 5]] = [7, 2]  # ignored for pad rows
    G.check_replay(c, "replay spec with pad rows")
    G.check_replay(dict(c, disable_state_update=True), "replay spec disabled")


def test_replay_spec_commit_sequence():
    """Several speculative steps with the caller committing accepted prefixes
    (pointer + accepted, from 0 after a fold): every step matches the oracle.
    Each step starts both sides from the oracle's pool and buffers (the GPU's
    folds may differ from the oracle's in the last bits)."""
    L, T = 10, 3
    c = W.replay_spec(seed=42, batch=16, T=T, heads=8, dim=64, dstate=128, groups=2, slots=24, L=L,
                      buf_len=0)
    d = G.device_replay(c)
    rng = np.random.default_rng(43)
    for step in range(6):
        ref = G.oracle_replay(c)
        G.say("[gpu] replay spec step %d: launching" % step)
        got = G.run_gpu_replay(c, d=d)
        G.compare_replay(c, got, ref, "spec step %d" % step)
        # commit on the oracle's side and the device's side alike
        fold = np.asarray(c["buf_len"]) + 2 * T > L
        acc = rng.integers(1, T + 1, len(c["buf_len"]))
        new_len = np.where(fold, 0, c["buf_len"]) + acc
        c.update(state=ref["state"], buf_x=ref["buf_x"], buf_dt=ref["buf_dt"], buf_B=ref["buf_B"])
        d["state"].copy_(G.dev(c["state"], c["state_dtype"], "cuda:0"))
        for k in ("buf_x", "buf_B"):
            d[k].copy_(G.dev(c[k], c["io_dtype"], "cuda:0"))
        d["buf_dt"].copy_(G.dev(c["buf_dt"], c.get("dt_dtype", c["io_dtype"]), "cuda:0"))
        c["buf_len"] = new_len.astype(np.int32)
        d["buf_len"].copy_(torch.from_numpy(c["buf_len"]))
        for k in ("x", "dt", "B", "C", "z"):
            a = W.to_storage(rng.standard_normal(np.shape(c[k]), dtype=np.float32), c["io_dtype"])
            c[k] = a
            d[k] = G.dev(a, c["io_dtype"], "cuda:0")


def test_replay_spec_out_of_range_counts():
    """buf_len outside [0, L] for a live slot: that sequence's y is NaN and
    nothing of it is written; the others are unaffected."""
    L = 8
    c = W.replay_spec(seed=44, batch=12, T=2, heads=8, dim=64, dstate=128, groups=2, slots=20, L=L)
    bad = [2, 7, 9]
    c["buf_len"][bad] = [L + 1, -1, L + 5]
    G.say("[gpu] replay spec out-of-range counts: launching")
    got = G.run_gpu_replay(c)
    assert np.isnan(G.brute64.to_f64(got["y"][bad], c["io_dtype"])).all()
    tab = np.asarray(c["state_batch_indices"])
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(got[k][tab[bad]], np.asarray(c[k])[tab[bad]]), k
    good = [b for b in range(12) if b not in bad]
    sub, used = G.replay_subcase(c, good)
    ref = G.oracle_replay(sub)
    sub_got = {"y": got["y"][good], "state": got["state"][used]}
    for k in ("buf_x", "buf_dt", "buf_B"):
        sub_got[k] = got[k][used]
    G.compare_replay(sub, sub_got, ref, "replay spec, valid rows")


def test_replay_spec_full_workload():
    """The speculative benchmark workload (batch 512, T = 4, L = 16): every
    sequence, folding or not, against the oracle's whole step (pool, y and
    the three buffers bit for bit)."""
    c = W.replay_spec()
    G.say("[gpu] replay spec full: oracle")
    ref = G.oracle_replay(c)
    G.say("[gpu] replay spec full: launching")
    got = G.run_gpu_replay(c)
    stats = G.compare_replay(c, got, ref, "replay spec full")
    G.say("[gpu] replay spec full: ok %s" % {k: "%.3g" % v for k, v in stats.items()})


@pytest.mark.parametrize("dt_per_head", [False, True])
def test_replay_spec_fold_across_workgroups(dt_per_head):
    """Every sequence folds while its drafts go to the entries the folds read
    (h = 6, T = 4, L = 8: entries 0..5 read, 0..3 written), 64 heads share
    one group's B rows and a per-head dt is shared by a head's dim tiles, on
    a grid far larger than what can be resident at once (512 x 64 x dim
    tiles). Every folded checkpoint, y and buffer entry against the oracle:
    a fold that saw a draft's B or dt would differ."""
    c = W.replay_spec(seed=61, batch=512, T=4, heads=64, dim=64, dstate=128, groups=1,
                      slots=520, L=8, buf_len=6, dt_per_head=dt_per_head)
    G.say("[gpu] replay spec fold across workgroups (per-head dt %s): oracle" % dt_per_head)
    ref = G.oracle_replay(c)
    assert ref["written"].sum() == 512
    G.say("[gpu] replay spec fold across workgroups: launching")
    got = G.run_gpu_replay(c)
    stats = G.compare_replay(c, got, ref, "replay spec fold across workgroups")
    G.say("[gpu] replay spec fold across workgroups: ok %s"
          % {k: "%.3g" % v for k, v in stats.items()})
