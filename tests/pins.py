"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, none of which retypes the oracle's own loop.

Each pin takes an oracle instance (oracle.ssu_oracle.Oracle) and raises
AssertionError (or the oracle's own error) when the oracle is wrong, so the
same pins run against the real oracle and against copies of it with a planted
mistake (tests/test_oracle_mutants.py).

Sources:
  MATE  = MATE docs, "Mamba / SSU" (table "SSU at a glance", the minimal, MTP
          and flat-table examples, the API reference)
  RSSM  = ReplaySSM article (lpnh.cn): section "三个瓶颈其实来自同一个动作"
          (the Mamba-2 step and readout) and section "核心做法" (the unrolled
          window S_h = g_h S_ckpt + sum_j g_{j+1:h} v_j k_j^T, and output-only
          decode from a zero state, o = (v k^T) q = v (k^T q))
"""
import math

import numpy as np
import torch

import workloads as W
from oracle import brute64

U32 = 2.0 ** -24  # unit roundoff of fp32


def f64(a, dtype):
    return brute64.to_f64(a, dtype)


def ulp16(v, dtype):
    """Spacing of the 16-bit format at |v| (bounded below by its subnormal step)."""
    mant = 10 if dtype == "f16" else 7
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))
    return np.maximum(2.0 ** (e - mant), 2.0 ** -24 if dtype == "f16" else 2.0 ** -133)


def processed_dt(case):
    """dt' = softplus(dt + dt_bias) in float64, broadcast to [R, H, P]."""
    x = np.asarray(case["x"])
    R = x.shape[0] * (x.shape[1] if x.ndim == 4 else 1)
    H, P = x.shape[-2], x.shape[-1]
    dt = f64(case["dt"], case.get("dt_dtype", case["io_dtype"]))
    dt = dt.reshape(R, H, 1) if dt.size == R * H else dt.reshape(R, H, P)
    dt = np.broadcast_to(dt, (R, H, P)).copy()
    if case.get("dt_bias") is not None:
        dt = dt + np.asarray(case["dt_bias"], np.float64)[None, :, None]
    if case.get("dt_softplus"):
        dt = np.where(dt > 20, dt, np.log1p(np.exp(np.minimum(dt, 20))))
    return dt


def small(kind, **kw):
    return W.BUILDERS[kind](**kw)


# ---------------------------------------------------------------- formats

def pin_f16_decode_exhaustive(orc):
    """Every binary16 bit pattern widens to NumPy's float16 -> float32 value."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(b) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_samples(n=60000, seed=0):
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    special = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24,
                        2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -15 * 1.5, 1 + 2.0 ** -11,
                        1 + 3 * 2.0 ** -11, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.0e38, np.inf,
                        -np.inf, 1e-40], dtype=np.float32)
    # values near binary16 / bfloat16 rounding boundaries
    near = rng.standard_normal(20000).astype(np.float32) * np.float32(100)
    near16 = near.astype(np.float16).astype(np.float32)
    tie = (near16.view(np.uint32) + np.uint32(1 << 12)).view(np.float32)
    return np.concatenate([u.view(np.float32), special, near, tie])


def pin_f16_encode(orc):
    """float32 -> binary16 rounds to nearest even, as NumPy's cast does."""
    v = _f32_samples()
    with np.errstate(over="ignore", invalid="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(x) for x in v], dtype=np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all(got[nan] & 0x3FF)


def pin_bf16_roundtrip(orc):
    """float32 -> bfloat16 rounds to nearest even, as PyTorch's cast does;
    bfloat16 -> float32 is the top half of the binary32 pattern."""
    v = _f32_samples(seed=1)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(x) for x in v], dtype=np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x7F)
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    back = np.array([orc.bf16_to_f32(b) for b in bits], dtype=np.float32)
    ref_back = (bits.astype(np.uint32) << 16).view(np.float32)
    ok = ~np.isnan(ref_back)
    assert np.array_equal(back[ok].view(np.uint32), ref_back[ok].view(np.uint32))


def pin_softplus(orc):
    """softplus(0) = ln 2; softplus(v) = log(1 + e^v) to fp32 accuracy; and
    above 20 the value itself (the difference is below half an ulp)."""
    assert abs(orc.softplus(0.0) - math.log(2.0)) <= math.log(2.0) * U32 * 2
    for v in np.linspace(-30, 30, 241):
        v = float(np.float32(v))
        ref = float(np.logaddexp(0.0, v))
        assert abs(orc.softplus(v) - ref) <= 4 * U32 * max(ref, 1e-30), v
    assert orc.softplus(25.5) == 25.5


# ---------------------------------------------------------------- recurrence

def pin_dt_zero_keeps_state(orc):
    """dt = 0 without bias or softplus: the decay is exp(0) = 1 and the rank-1
    term vanishes, so every stored tile equals the tile read, bit for bit."""
    for sd in ("f32", "f16", "bf16"):
        c = small("decode", batch=5, heads=4, dim=12, dstate=16, groups=2, slots=12,
                  state_dtype=sd, io="bf16")
        c["dt"] = np.zeros_like(c["dt"])
        c["dt_bias"], c["dt_softplus"] = None, False
        o = orc.run(c)
        assert np.array_equal(o["state"], c["state"]), sd
        assert o["written"].sum() == 5


def pin_b_zero_pure_decay(orc):
    """B = 0: each element becomes S * exp(dt * A[h]) (RSSM's step with a zero
    rank-1 term); checked in float64 against the fp32 error bound."""
    c = small("decode", batch=6, heads=4, dim=8, dstate=16, groups=2, slots=12, state_dtype="f32",
              io="f32")
    c["B"] = np.zeros_like(c["B"])
    c["dt_bias"], c["dt_softplus"] = None, False
    c["dt"] = np.abs(c["dt"]).astype(np.float32) * np.float32(0.5)
    o = orc.run(c)
    A = np.asarray(c["A"], np.float64)
    rt = np.asarray(c["state_batch_indices"])
    for b in range(6):
        S0 = c["state"][rt[b]].astype(np.float64)
        dt = np.asarray(c["dt"][b], np.float64)
        arg = dt * A[:, None]
        ref = S0 * np.exp(arg)[:, :, None]
        bound = np.abs(ref) * (np.abs(arg)[:, :, None] * U32 + 3 * U32) * 1.5 + 1e-38
        assert np.all(np.abs(o["state"][rt[b]] - ref) <= bound)


def _zero_state_expected(case, rows):
    """RSSM output-only decode from a zero state: S = dt' x B^T, so
    y[d] = dt'[d] x[d] (B . C) + D x[d], times silu(z[d])."""
    io = case["io_dtype"]
    dtp = processed_dt(case)
    X = f64(case["x"], io)
    H = X.shape[1]
    Bm, Cm = f64(case["B"], io), f64(case["C"], io)
    G = Bm.shape[1]
    out, scale = [], []
    for r in rows:
        bc = np.array([Bm[r, h // (H // G)] @ Cm[r, h // (H // G)] for h in range(H)])
        babs = np.array([np.abs(Bm[r, h // (H // G)]) @ np.abs(Cm[r, h // (H // G)])
                         for h in range(H)])
        y = dtp[r] * X[r] * bc[:, None]
        s = np.abs(dtp[r] * X[r]) * babs[:, None]
        if case.get("D") is not None:
            y = y + np.asarray(case["D"], np.float64)[:, None] * X[r]
            s = s + np.abs(np.asarray(case["D"], np.float64)[:, None] * X[r])
        if case.get("z") is not None:
            Z = f64(case["z"], io)[r]
            g = Z / (1 + np.exp(-Z))
            y, s = y * g, s * np.abs(g)
        out.append(y)
        scale.append(s)
    return np.array(out), np.array(scale)


def pin_zero_state_closed_form(orc):
    """Rows whose read slot is the pad id start from a zero state (MATE slot
    semantics); their y must equal RSSM's output-only closed form."""
    for io in ("f32", "bf16"):
        c = small("decode_pad", batch=20, heads=4, dim=8, dstate=32, groups=2, slots=40,
                  state_dtype="f32", io=io, pad_frac=0.25, pad_slot_id=0)
        o = orc.run(c)
        rows = c["pad_rows"]
        ref, scale = _zero_state_expected(c, rows)
        got = f64(o["y"], io)[rows]
        tol = 40 * U32 * scale + 1e-30
        if io != "f32":
            tol = tol + ulp16(ref, io)
        assert np.all(np.abs(got - ref) <= tol), io


def pin_c_zero_and_z_zero(orc):
    """C = 0 leaves y = D x silu(z); z = 0 makes y exactly 0 (silu(0) = 0)."""
    c = small("decode", batch=4, heads=4, dim=8, dstate=16, groups=2, slots=8, state_dtype="f32",
              io="f32")
    c["C"] = np.zeros_like(c["C"])
    o = orc.run(c)
    X, Z = c["x"].astype(np.float64), c["z"].astype(np.float64)
    ref = np.asarray(c["D"], np.float64)[None, :, None] * X * (Z / (1 + np.exp(-Z)))
    assert np.all(np.abs(o["y"] - ref) <= 6 * U32 * np.abs(ref) + 1e-38)
    c2 = small("decode", batch=4, heads=4, dim=8, dstate=16, groups=2, slots=8, state_dtype="f32",
               io="f32")
    c2["z"] = np.zeros_like(c2["z"])
    assert np.all(orc.run(c2)["y"] == 0.0)


def _chained(orc, case):
    """The same sequences as T one-token calls: call t takes row bos+t of every
    sequence with more than t tokens; call 0 reads the read slot, call t > 0
    reads the slot call t-1 wrote; each call writes the token's destination."""
    cu = np.asarray(case["cu_seqlens"], np.int64)
    lens = np.diff(cu)
    acc = case.get("num_accepted_tokens")
    rt = np.asarray(case["state_batch_indices"])
    wt = case.get("dst_state_batch_indices")
    wt = rt if wt is None else np.asarray(wt)
    two_d = rt.ndim == 2

    def entry(tab, b, t):
        return int(tab[b, t]) if two_d else int(tab[cu[b] + t])

    pool = case["state"].copy()
    y = np.zeros_like(case["x"])
    for t in range(int(lens.max())):
        seqs = [b for b in range(len(lens)) if lens[b] > t]
        rows = np.array([cu[b] + t for b in seqs])
        start = [0 if acc is None else max(int(acc[b]) - 1, 0) for b in seqs]
        rd = np.array([entry(rt, b, s) if t == 0 else entry(wt, b, t - 1)
                       for b, s in zip(seqs, start)], np.int64)
        wr = np.array([entry(wt, b, t) for b in seqs], np.int64)
        one = dict(case, state=pool, x=case["x"][rows], dt=case["dt"][rows], B=case["B"][rows],
                   C=case["C"][rows], z=None if case.get("z") is None else case["z"][rows],
                   state_batch_indices=rd, dst_state_batch_indices=wr, cu_seqlens=None,
                   num_accepted_tokens=None)
        o = orc.run(one)
        pool = o["state"]
        y[rows] = o["y"]
    return y, pool


def pin_mtp_equals_chained_calls(orc):
    """A T-token MTP call equals T chained one-token calls, bit for bit, in
    every state dtype (the carried state is the stored value)."""
    for sd in ("f32", "f16", "bf16"):
        c = small("mtp", nseq=5, steps=4, heads=4, dim=8, dstate=16, groups=2, state_dtype=sd,
                  pad_slot_id=-1)
        o = orc.run(c)
        y, pool = _chained(orc, c)
        assert np.array_equal(o["y"], y), sd
        assert np.array_equal(o["state"], pool), sd
    c = small("varlen", nseq=9, max_len=4, heads=4, dim=8, dstate=16, state_dtype="bf16", dst=False)
    o = orc.run(c)
    y, pool = _chained(orc, c)
    assert np.array_equal(o["y"], y) and np.array_equal(o["state"], pool)


def pin_unrolled_window(orc):
    """RSSM's unrolled window: after T steps from S_0,
    S_T = (prod_i a_i) S_0 + sum_j (prod_{i>j} a_i) dt_j x_j B_j^T, in float64."""
    c = small("mtp", nseq=3, steps=6, heads=2, dim=8, dstate=16, groups=1, state_dtype="f32",
              io="f32", pad_slot_id=-1)
    c["num_accepted_tokens"] = np.ones(3, np.int32)
    o = orc.run(c)
    dtp = processed_dt(c)
    A = np.asarray(c["A"], np.float64)
    X, Bm = c["x"].astype(np.float64), c["B"].astype(np.float64)
    rt, wt = c["state_batch_indices"], c["dst_state_batch_indices"]
    for b in range(3):
        for h in range(2):
            S0 = c["state"][rt[b, 0], h].astype(np.float64)
            rows = range(b * 6, b * 6 + 6)
            alpha = [np.exp(dtp[r, h] * A[h]) for r in rows]
            ST = np.prod(alpha, axis=0)[:, None] * S0
            mag = np.abs(ST).copy()
            for j, r in enumerate(rows):
                tail = np.prod(alpha[j + 1:], axis=0) if j < 5 else np.ones(8)
                term = (tail * dtp[r, h] * X[r, h])[:, None] * Bm[r, 0][None, :]
                ST += term
                mag += np.abs(term)
            got = o["state"][wt[b, 5], h]
            assert np.all(np.abs(got - ST) <= 6 * 8 * U32 * (mag + np.abs(S0)) + 1e-30)


# ---------------------------------------------------------------- slots

def pin_pad_slot_untouched(orc):
    """pad_slot_id = 0 with slot 0 holding data: slot 0 stays byte-identical,
    every other untouched slot too (MATE: pad is never written)."""
    for sd in ("f32", "bf16"):
        c = small("decode_pad", batch=24, heads=2, dim=8, dstate=16, groups=1, slots=48,
                  state_dtype=sd, pad_frac=0.2, pad_slot_id=0)
        assert np.any(c["state"][0] != 0)
        o = orc.run(c)
        assert not o["written"][0]
        assert np.array_equal(o["state"][~o["written"]], c["state"][~o["written"]])
        live = np.asarray(c["state_batch_indices"])
        live = live[live != 0]
        assert set(np.flatnonzero(o["written"])) == set(live.tolist())


def pin_disable_keeps_pool(orc):
    """disable_state_update leaves the whole pool byte-identical; y is the
    same as with the update enabled."""
    c = small("varlen", nseq=10, max_len=5, heads=2, dim=8, dstate=16)
    o1 = orc.run(c)
    o2 = orc.run(dict(c, disable_state_update=True))
    assert np.array_equal(o2["state"], c["state"]) and not o2["written"].any()
    assert np.array_equal(o1["y"], o2["y"])


def pin_flat_equals_2d(orc):
    """A 2-D [sequences, steps] table and the flat [rows] table name the same
    entries for one sequence (MATE flat-table example) and, 1-D tables being
    row-indexed, for uniform lengths."""
    c = small("mtp", nseq=1, steps=7, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=0)
    c["num_accepted_tokens"] = np.array([1], np.int32)
    o2 = orc.run(c)
    flat = dict(c, state_batch_indices=c["state_batch_indices"].ravel(),
                dst_state_batch_indices=c["dst_state_batch_indices"].ravel())
    o1 = orc.run(flat)
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])
    c = small("mtp", nseq=4, steps=3, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=-1)
    o2 = orc.run(c)
    o1 = orc.run(dict(c, state_batch_indices=c["state_batch_indices"].ravel(),
                      dst_state_batch_indices=c["dst_state_batch_indices"].ravel()))
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])
    assert np.array_equal(o1["written"], o2["written"])


def pin_strided_literal(orc):
    """A [rows, 1] view with strides (1, 1) addresses entry b + t (MATE slot
    semantics, "addressed by strides"); with one sequence that is row t."""
    c = small("mtp", nseq=1, steps=5, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=-1)
    c["num_accepted_tokens"] = np.array([3], np.int32)
    o2 = orc.run(c)
    view = dict(c, state_batch_indices=W.Strided(c["state_batch_indices"].ravel(), (5, 1), (1, 1)),
                dst_state_batch_indices=W.Strided(c["dst_state_batch_indices"].ravel(), (5, 1),
                                                  (1, 1)))
    o1 = orc.run(view)
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])
    assert o1["read_slot"][0] == c["state_batch_indices"][0, 2]


def pin_default_destination(orc):
    """No destination table: each token publishes to its own entry of the read
    table (MATE: the default the Triton kernel applies)."""
    c = small("varlen", nseq=8, max_len=4, heads=2, dim=8, dstate=16, dst=False)
    o1 = orc.run(c)
    o2 = orc.run(dict(c, dst_state_batch_indices=c["state_batch_indices"].copy()))
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])
    rows = int(np.asarray(c["cu_seqlens"])[-1])
    assert set(np.flatnonzero(o1["written"])) == set(c["state_batch_indices"][:rows].tolist())


def pin_empty_sequences(orc):
    """Empty sequences are skipped: with a 2-D table their row of entries is
    neither read nor written."""
    c = small("mtp", nseq=4, steps=3, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=-1)
    # sequence 1 becomes empty: its rows are dropped from the packed inputs
    keep = np.r_[0:3, 6:12]
    c2 = dict(c, x=c["x"][keep], dt=c["dt"][keep], B=c["B"][keep], C=c["C"][keep],
              z=c["z"][keep], cu_seqlens=np.array([0, 3, 3, 6, 9], np.int32))
    o = orc.run(c2)
    assert o["read_slot"][1] == np.iinfo(np.int64).min
    for slot in list(c["state_batch_indices"][1]) + list(c["dst_state_batch_indices"][1]):
        assert not o["written"][slot]
    assert np.array_equal(o["state"][~o["written"]], c["state"][~o["written"]])


def pin_accepted_floor(orc):
    """num_accepted_tokens seeds the read at count - 1, floored at 0: 0 and 1
    read the same entry; k reads entry k - 1."""
    c = small("mtp", nseq=3, steps=4, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=-1)
    a0 = orc.run(dict(c, num_accepted_tokens=np.array([0, 0, 0], np.int32)))
    a1 = orc.run(dict(c, num_accepted_tokens=np.array([1, 1, 1], np.int32)))
    assert np.array_equal(a0["y"], a1["y"]) and np.array_equal(a0["state"], a1["state"])
    a3 = orc.run(dict(c, num_accepted_tokens=np.array([3, 4, 2], np.int32)))
    rt = c["state_batch_indices"]
    assert list(a3["read_slot"]) == [rt[0, 2], rt[1, 3], rt[2, 1]]


def pin_pad_destination_mid_sequence(orc):
    """A pad destination skips that store only; later tokens continue from the
    carried state, so y is unchanged and the pad slot keeps its bytes."""
    c = small("mtp", nseq=2, steps=4, heads=2, dim=8, dstate=16, groups=1, pad_slot_id=-1)
    w = c["dst_state_batch_indices"].copy()
    # slot 0 is sequence 0's first read-table entry, which accepted count 2
    # leaves unread
    w[0, 1] = 0
    c2 = dict(c, dst_state_batch_indices=w, pad_slot_id=0,
              num_accepted_tokens=np.array([2, 2], np.int32))
    ref = orc.run(dict(c, num_accepted_tokens=np.array([2, 2], np.int32)))
    o = orc.run(c2)
    assert np.array_equal(o["y"], ref["y"])
    assert not o["written"][0] and np.array_equal(o["state"][0], c["state"][0])


def pin_dt_per_head_broadcast(orc):
    """dt with one value per head equals the same values repeated over dim."""
    c = small("varlen", nseq=6, max_len=3, heads=4, dim=8, dstate=16)
    o1 = orc.run(c)
    P = c["x"].shape[-1]
    o2 = orc.run(dict(c, dt=np.repeat(c["dt"][:, :, None], P, axis=2)))
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])


def pin_groups(orc):
    """groups = 1 equals B, C replicated to groups = heads; and with two groups
    heads 0..H/2-1 use group 0 (a zero B, C there means pure decay)."""
    c = small("decode", batch=3, heads=4, dim=8, dstate=16, groups=1, slots=6)
    o1 = orc.run(c)
    o2 = orc.run(dict(c, B=np.repeat(c["B"], 4, axis=1), C=np.repeat(c["C"], 4, axis=1)))
    assert np.array_equal(o1["y"], o2["y"]) and np.array_equal(o1["state"], o2["state"])
    c = small("decode", batch=3, heads=4, dim=8, dstate=16, groups=2, slots=6, state_dtype="f32",
              io="f32")
    c["B"][:, 0] = 0
    c["C"][:, 0] = 0
    o = orc.run(c)
    X, Z = c["x"].astype(np.float64), c["z"].astype(np.float64)
    ydz = np.asarray(c["D"], np.float64)[None, :, None] * X * (Z / (1 + np.exp(-Z)))
    assert np.allclose(o["y"][:, :2], ydz[:, :2], rtol=1e-6, atol=0)
    assert not np.allclose(o["y"][:, 2:], ydz[:, 2:], rtol=1e-3, atol=0)


def pin_brute_force(orc, combos=48, seed=7):
    """Whole oracle against the independent float64 brute force on tiny shapes
    over the option space (layouts, tables, dtypes, bias/softplus, D, z, pad,
    disable, accepted counts)."""
    rng = np.random.default_rng(seed)
    for k in range(combos):
        kind = ["decode", "decode_pad", "mtp", "varlen"][k % 4]
        sd = ["f32", "f16", "bf16"][rng.integers(3)]
        io = ["bf16", "f16", "f32"][rng.integers(3)]
        s = int(rng.integers(1 << 30))
        if kind == "decode":
            c = W.decode(seed=s, batch=3, heads=4, dim=4, dstate=8, groups=2, slots=8,
                         state_dtype=sd, io=io)
        elif kind == "decode_pad":
            c = W.decode_pad(seed=s, batch=5, heads=2, dim=4, dstate=8, groups=1, slots=9,
                             state_dtype=sd, io=io, pad_frac=0.4,
                             pad_slot_id=int(rng.choice([0, -1])))
        elif kind == "mtp":
            c = W.mtp(seed=s, nseq=2, steps=3, heads=2, dim=4, dstate=8, groups=2, state_dtype=sd,
                      io=io, pad_slot_id=int(rng.choice([0, -1])))
        else:
            c = W.varlen(seed=s, nseq=4, max_len=3, heads=2, dim=4, dstate=8, state_dtype=sd,
                         io=io, dst=bool(rng.integers(2)), disable=bool(rng.integers(2)))
        if rng.integers(2):
            # without softplus dt must stay a non-negative step: U[0, 0.1) as
            # in the MATE minimal example
            c["dt_bias"], c["dt_softplus"] = None, False
            dtd = c.get("dt_dtype", io)
            c["dt"] = W.to_storage(rng.random(np.shape(c["dt"]), dtype=np.float32) * 0.1, dtd)
        if rng.integers(3) == 0:
            c["D"] = None
        if rng.integers(3) == 0:
            c["z"] = None
        o = orc.run(c)
        b = brute64.run(c)
        assert np.array_equal(o["written"], b["written"]), k
        S_o, S_b = f64(o["state"], sd), f64(b["state"], sd)
        if sd == "f32":
            tol = 64 * U32 * (np.abs(S_b) + 1)
        else:
            tol = 2 * ulp16(S_b, sd) + 64 * U32 * (np.abs(S_b) + 1)
        assert np.all(np.abs(S_o - S_b) <= tol), (k, kind, sd)
        y_o = f64(o["y"], io)
        tol = 64 * U32 * (np.abs(b["y64"]) + 8) * 8
        if io != "f32":
            tol = tol + 2 * ulp16(b["y64"], io)
        assert np.all(np.abs(y_o - b["y64"]) <= tol), (k, kind, io)


# ---------------------------------------------------------------- golden

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden",
                                    "mate_examples.json")


def golden_case(spec, seed=11):
    """A call shaped like one of the MATE page's examples, with random layer
    data (x, B, C bf16 N(0,1), dt fp32 U[0, 0.1), A = -U[0, 1))."""
    import json
    shape = json.load(open(GOLDEN))["shape"]
    H, P, N, G = shape["heads"], shape["dim"], shape["dstate"], shape["groups"]
    rng = np.random.default_rng(seed)
    R = spec["x_rows"]
    c = {"state_dtype": "f16", "io_dtype": "bf16", "dt_dtype": "f32"}
    c["state"] = W.to_storage(rng.standard_normal((spec["slots"], H, P, N), dtype=np.float32), "f16")
    c["x"] = W.to_storage(rng.standard_normal((R, H, P), dtype=np.float32), "bf16")
    c["dt"] = rng.random((R, H, P), dtype=np.float32) * np.float32(0.1)
    c["A"] = (-rng.random(H, dtype=np.float32)).astype(np.float32)
    c["B"] = W.to_storage(rng.standard_normal((R, G, N), dtype=np.float32), "bf16")
    c["C"] = W.to_storage(rng.standard_normal((R, G, N), dtype=np.float32), "bf16")
    c.update(D=None, z=None, dt_bias=None, dt_softplus=False, disable_state_update=False,
             pad_slot_id=spec["pad_slot_id"])
    for k in ("state_batch_indices", "dst_state_batch_indices", "cu_seqlens",
              "num_accepted_tokens"):
        c[k] = None if spec[k] is None else np.array(spec[k], dtype=np.int32)
    return c


def pin_golden_mate_examples(orc):
    """The MATE page's three examples: read and written slots as the page's
    slot rules fix them (tests/golden/mate_examples.json)."""
    import json
    for spec in json.load(open(GOLDEN))["cases"]:
        c = golden_case(spec)
        o = orc.run(c)
        assert list(o["read_slot"]) == spec["expected_read_slots"], spec["name"]
        assert sorted(np.flatnonzero(o["written"]).tolist()) == spec["expected_written_slots"], \
            spec["name"]
        untouched = ~o["written"]
        assert np.array_equal(o["state"][untouched], c["state"][untouched]), spec["name"]


# ---------------------------------------------------------------- ReplaySSM

def _replay_case(L, buf_len, sd="f32", io="f32", **kw):
    base = dict(batch=4, heads=4, dim=8, dstate=16, groups=2, slots=8)
    base.update(kw)
    return W.replay(L=L, buf_len=buf_len, state_dtype=sd, io=io, **base)


def _as_ssu(case):
    return {k: v for k, v in case.items() if k not in ("L", "buf_x", "buf_dt", "buf_B", "buf_len")}


def pin_replay_L1_is_plain_update(orc):
    """L = 1: every step is a flush with an empty buffer, so the step is the
    plain update bit for bit (ReplaySSM article, "核心做法": the kernel
    degenerates to the baseline) - y, checkpoint, and untouched buffers."""
    from oracle import ssu_oracle
    for sd in ("f32", "bf16"):
        c = _replay_case(1, 0, sd=sd, io="bf16")
        r = ssu_oracle.run_replay(c, orc)
        p = orc.run(_as_ssu(c))
        assert np.array_equal(r["y"], p["y"]) and np.array_equal(r["state"], p["state"]), sd
        assert np.array_equal(r["buf_x"], c["buf_x"]) and np.array_equal(r["buf_B"], c["buf_B"])


def _replay_window(orc, L, sd, io, steps_inputs, case0):
    """Run a window of L replay steps from an empty buffer (the caller moves
    the pointer 0, 1, .., L-1) and the same steps as chained plain updates."""
    from oracle import ssu_oracle
    c = dict(case0)
    plain = _as_ssu(case0)
    ys_r, ys_p = [], []
    for t, inp in enumerate(steps_inputs):
        c.update(inp)
        c["buf_len"] = np.full(len(c["buf_len"]), t, np.int32)
        r = ssu_oracle.run_replay(c, orc)
        c.update(state=r["state"], buf_x=r["buf_x"], buf_dt=r["buf_dt"], buf_B=r["buf_B"])
        ys_r.append(r["y"])
        plain.update(inp)
        p = orc.run(plain)
        plain["state"] = p["state"]
        ys_p.append(p["y"])
    return c, plain, ys_r, ys_p


def _fresh_inputs(case, seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        inp = {}
        for k in ("x", "dt", "B", "C", "z"):
            a = case[k]
            dtype = case.get("dt_dtype", case["io_dtype"]) if k == "dt" else case["io_dtype"]
            inp[k] = W.to_storage(rng.standard_normal(a.shape, dtype=np.float32), dtype)
        out.append(inp)
    return out


def pin_replay_flush_is_chain(orc):
    """A window of L steps: after the flush the checkpoint equals L chained
    plain updates bit for bit (the fold replays the same steps); before it,
    the checkpoint is untouched and each step's y (from checkpoint + buffer,
    the unrolled window of "核心做法") equals the plain update's y to fp32
    accuracy."""
    for sd in ("f32", "f16"):
        L = 5
        c0 = _replay_case(L, 0, sd=sd, io="f32")
        inputs = _fresh_inputs(c0, 3, L)
        c, plain, ys_r, ys_p = _replay_window(orc, L, sd, "f32", inputs, c0)
        live = np.asarray(c0["state_batch_indices"])
        assert np.array_equal(c["state"][live], plain["state"][live]), sd
        for t in range(L):
            scale = np.abs(ys_p[t]).max() + 1.0
            tol = 1e-5 if sd == "f32" else 2e-2
            assert np.abs(ys_r[t].astype(np.float64) - ys_p[t]).max() <= tol * scale, (sd, t)


def pin_replay_nonflush_writes_entry_only(orc):
    """A step that does not fill the buffer leaves the checkpoint pool
    byte-identical and writes exactly entry h of its slot's buffer with the
    step's raw inputs."""
    from oracle import ssu_oracle
    c = _replay_case(6, [0, 2, 4, 1], sd="bf16", io="bf16")
    r = ssu_oracle.run_replay(c, orc)
    assert np.array_equal(r["state"], c["state"]) and not r["written"].any()
    bx, bB, bdt = c["buf_x"].copy(), c["buf_B"].copy(), c["buf_dt"].copy()
    for b, s in enumerate(c["state_batch_indices"]):
        h = c["buf_len"][b]
        bx[s, h] = c["x"][b]
        bdt[s, h] = c["dt"][b]
        bB[s, h] = c["B"][b]
    assert np.array_equal(r["buf_x"], bx) and np.array_equal(r["buf_B"], bB)
    assert np.array_equal(r["buf_dt"], bdt)


def pin_replay_zero_checkpoint(orc):
    """Pad slot (zero checkpoint) and an empty buffer: y is the output-only
    closed form dt' x (B . C) + D x, gated, and nothing is written."""
    from oracle import ssu_oracle
    c = _replay_case(4, [0, 3, 0, 2], sd="f32", io="f32")
    c["state_batch_indices"] = np.array([0, -1, 2, -1], np.int32)  # pad rows' pointers ignored
    r = ssu_oracle.run_replay(c, orc)
    ref, scale = _zero_state_expected(_as_ssu(c), [1, 3])
    assert np.all(np.abs(r["y"][[1, 3]] - ref) <= 40 * U32 * scale + 1e-30)
    for s in (1, 3, 4, 5, 6, 7):
        assert np.array_equal(r["buf_x"][s], c["buf_x"][s])


def pin_replay_disable(orc):
    """disable_state_update writes neither the checkpoint nor the buffer; y
    is unchanged."""
    from oracle import ssu_oracle
    c = _replay_case(3, [2, 1, 0, 2], sd="f32", io="bf16")
    r1 = ssu_oracle.run_replay(c, orc)
    r2 = ssu_oracle.run_replay(dict(c, disable_state_update=True), orc)
    assert np.array_equal(r1["y"], r2["y"])
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(r2[k], c[k if k != "state" else "state"]), k


def pin_replay_brute_force(orc, combos=24, seed=11):
    """The replay step against the independent float64 version on tiny
    shapes over L, buffer pointers, dtypes and options."""
    from oracle import ssu_oracle
    rng = np.random.default_rng(seed)
    for k in range(combos):
        L = int(rng.choice([1, 2, 3, 5]))
        sd = ["f32", "f16", "bf16"][rng.integers(3)]
        io = ["f32", "bf16"][rng.integers(2)]
        c = W.replay(seed=int(rng.integers(1 << 30)), batch=3, heads=2, dim=4, dstate=8, groups=1,
                     slots=5, L=L, state_dtype=sd, io=io, dt_per_head=bool(rng.integers(2)),
                     buf_len=rng.integers(0, L, 3))
        if rng.integers(2):
            c["dt_bias"], c["dt_softplus"] = None, False
            dtd = c.get("dt_dtype", io)
            c["dt"] = W.to_storage(rng.random(np.shape(c["dt"]), dtype=np.float32) * 0.1, dtd)
            c["buf_dt"] = W.to_storage(rng.random(np.shape(c["buf_dt"]), dtype=np.float32) * 0.1,
                                       dtd)
        if rng.integers(3) == 0:
            c["z"] = None
        o = ssu_oracle.run_replay(c, orc)
        b = brute64.run_replay(c)
        for key in ("buf_x", "buf_dt", "buf_B"):
            assert np.array_equal(o[key], b[key]), (k, key)
        assert np.array_equal(o["written"], b["written"]), k
        S_o, S_b = f64(o["state"], sd), f64(b["state"], sd)
        tol = (64 * U32 * (np.abs(S_b) + 1)) if sd == "f32" else \
            (2 * ulp16(S_b, sd) + 64 * U32 * (np.abs(S_b) + 1))
        assert np.all(np.abs(S_o - S_b) <= tol), (k, sd, L)
        y_o = f64(o["y"], io)
        tol = 64 * U32 * (np.abs(b["y64"]) + 8) * 8 * L
        if io != "f32":
            tol = tol + 2 * ulp16(b["y64"], io)
        assert np.all(np.abs(y_o - b["y64"]) <= tol), (k, io, L)


# ------------------------------------------------ ReplaySSM, speculative step

def _spec_case(L, T, buf_len, sd="f32", io="f32", **kw):
    base = dict(batch=4, heads=4, dim=8, dstate=16, groups=2, slots=8)
    base.update(kw)
    return W.replay_spec(L=L, T=T, buf_len=buf_len, state_dtype=sd, io=io, **base)


def _spec_chain(orc, c, b, entries):
    """Plain update over one sequence: from slot s's checkpoint, the buffer
    entries `entries` of the slot and then the T drafts of sequence b, one
    token after the other (dense [1, steps] form). Returns (y [steps, H, P],
    pool after the first len(entries) steps, pool after all)."""
    s = int(np.asarray(c["state_batch_indices"])[b])
    T = np.shape(c["x"])[1]
    per_head = np.ndim(c["dt"]) == 3
    rows = {}
    for k, buf in (("x", "buf_x"), ("dt", "buf_dt"), ("B", "buf_B")):
        rows[k] = np.concatenate([np.asarray(c[buf])[s, list(entries)],
                                  np.asarray(c[k])[b]], axis=0)[None]
    rows["C"] = np.concatenate([np.asarray(c["C"])[b][:1].repeat(len(entries), 0),
                                np.asarray(c["C"])[b]], axis=0)[None]
    if c.get("z") is not None:
        rows["z"] = np.concatenate([np.asarray(c["z"])[b][:1].repeat(len(entries), 0),
                                    np.asarray(c["z"])[b]], axis=0)[None]
    plain = {k: v for k, v in c.items()
             if k not in ("L", "buf_x", "buf_dt", "buf_B", "buf_len")}
    plain.update(rows)
    plain["state_batch_indices"] = np.array([[s] * (len(entries) + T)], np.int64)
    plain["dst_state_batch_indices"] = np.array([list(range(len(entries) + T))], np.int64) + \
        np.shape(c["state"])[0]
    pool = np.asarray(c["state"])
    plain["state"] = np.concatenate([pool, np.zeros((len(entries) + T,) + pool.shape[1:],
                                                    pool.dtype)], axis=0)
    o = orc.run(plain)
    nslots = pool.shape[0]
    after_entries = o["state"][nslots + len(entries) - 1] if entries else pool[s]
    return o["y"][0], after_entries, per_head


def pin_replay_spec_is_chain(orc):
    """Speculative step (ReplaySSM article, "投机解码回滚变成挪指针"): draft t's
    y equals the plain update's y after the committed entries and drafts
    0..t (the causal mask), to fp32 accuracy; a folding step (h + 2T > L)
    stores the checkpoint the plain update reaches after the committed entries
    bit for bit, and the drafts go to entries w..w+T-1 (w = 0 after a fold)."""
    from oracle import ssu_oracle
    for sd, io in (("f32", "f32"), ("bf16", "f32")):
        L, T = 8, 3
        c = _spec_case(L, T, [0, 2, 3, 5], sd=sd, io=io)  # folds: h > L - 2T = 2
        r = ssu_oracle.run_replay_spec(c, orc)
        for b, h in enumerate(c["buf_len"]):
            s = int(c["state_batch_indices"][b])
            fold = h + 2 * T > L
            w = 0 if fold else h
            y, after, _ = _spec_chain(orc, c, b, range(h))
            scale = np.abs(y).max() + 1.0
            tol = 1e-5 if sd == "f32" else 2e-2
            got = r["y"][b].astype(np.float64)
            assert np.abs(got - y[h:]).max() <= tol * scale, (sd, b)
            if fold:
                assert r["written"][s] and np.array_equal(r["state"][s], after), (sd, b)
            else:
                assert not r["written"][s] and np.array_equal(r["state"][s], c["state"][s])
            for k, buf in (("x", "buf_x"), ("dt", "buf_dt"), ("B", "buf_B")):
                want = np.asarray(c[buf])[s].copy()
                want[w:w + T] = np.asarray(c[k])[b]
                assert np.array_equal(r[buf][s], want), (sd, b, buf)


def pin_replay_spec_rollback(orc):
    """Rejected drafts cost nothing: after a step whose drafts were appended
    at h.., the caller accepts a prefix (pointer h + a); the next step's
    drafts overwrite the rejected entries and read out exactly as the plain
    update over the committed entries, the accepted drafts and the new ones."""
    from oracle import ssu_oracle
    L, T = 12, 3
    c = _spec_case(L, T, [1, 0, 2, 4])
    r = ssu_oracle.run_replay_spec(c, orc)
    acc = [2, 3, 1, 2]
    c2 = dict(c, buf_x=r["buf_x"], buf_dt=r["buf_dt"], buf_B=r["buf_B"], state=r["state"])
    c2.update(_fresh_inputs_spec(c, 5))
    c2["buf_len"] = np.asarray(c["buf_len"]) + np.asarray(acc, np.int32)
    r2 = ssu_oracle.run_replay_spec(c2, orc)
    for b in range(4):
        h2 = int(c2["buf_len"][b])
        y, _, _ = _spec_chain(orc, c2, b, range(h2))
        scale = np.abs(y).max() + 1.0
        assert np.abs(r2["y"][b].astype(np.float64) - y[h2:]).max() <= 1e-5 * scale, b


def _fresh_inputs_spec(case, seed):
    rng = np.random.default_rng(seed)
    inp = {}
    for k in ("x", "dt", "B", "C", "z"):
        a = case[k]
        dtype = case.get("dt_dtype", case["io_dtype"]) if k == "dt" else case["io_dtype"]
        inp[k] = W.to_storage(rng.standard_normal(a.shape, dtype=np.float32), dtype)
    return inp


def pin_replay_spec_fold_boundary(orc):
    """The fold comes one window early: at h + 2T > L, not at h + T > L
    (L = 8, T = 2: h = 4 keeps the window, h = 5 folds although its drafts
    would still fit)."""
    from oracle import ssu_oracle
    c = _spec_case(8, 2, [4, 5, 0, 6], sd="f32", io="bf16")
    r = ssu_oracle.run_replay_spec(c, orc)
    tab = c["state_batch_indices"]
    assert [bool(r["written"][s]) for s in tab] == [False, True, False, True]
    for b, w in enumerate([4, 0, 0, 0]):
        s = tab[b]
        assert np.array_equal(r["buf_x"][s, w:w + 2], c["x"][b]), b


def pin_replay_spec_pad_and_disable(orc):
    """The pad id reads a zero checkpoint with no buffer (its pointer is
    ignored) and writes nothing: its drafts read out as the plain update's
    chain from a zero state; disable_state_update writes nothing and leaves
    y unchanged."""
    from oracle import ssu_oracle
    c = _spec_case(6, 2, [1, 3, 4, 0], sd="f32", io="f32")
    tab = c["state_batch_indices"].copy()
    tab[2] = -1
    c["state_batch_indices"] = tab
    r = ssu_oracle.run_replay_spec(c, orc)
    live = set(int(v) for v in tab[[0, 1, 3]])
    others = [s for s in range(8) if s not in live]
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(r[k][others], c[k][others]), k
    zero = dict(c)
    zero["state"] = np.zeros_like(c["state"])
    zero["state_batch_indices"] = np.where(tab < 0, 7, tab)  # an all-zero slot instead of the pad
    y, _, _ = _spec_chain(orc, zero, 2, [])
    scale = np.abs(y).max() + 1.0
    assert np.abs(r["y"][2].astype(np.float64) - y).max() <= 1e-5 * scale
    d = ssu_oracle.run_replay_spec(dict(c, disable_state_update=True), orc)
    assert np.array_equal(d["y"], r["y"])
    for k in ("state", "buf_x", "buf_dt", "buf_B"):
        assert np.array_equal(d[k], c[k]), k


def pin_replay_spec_brute_force(orc, combos=20, seed=12):
    """The speculative step against the independent float64 version on tiny
    shapes over L, T, pointers (folding or not), dtypes and options."""
    from oracle import ssu_oracle
    rng = np.random.default_rng(seed)
    for k in range(combos):
        L = int(rng.choice([1, 2, 4, 7]))
        T = int(rng.integers(1, L + 1))
        sd = ["f32", "f16", "bf16"][rng.integers(3)]
        io = ["f32", "bf16"][rng.integers(2)]
        c = W.replay_spec(seed=int(rng.integers(1 << 30)), batch=3, T=T, heads=2, dim=4, dstate=8,
                          groups=1, slots=5, L=L, state_dtype=sd, io=io,
                          dt_per_head=bool(rng.integers(2)), buf_len=rng.integers(0, L + 1, 3))
        if rng.integers(2):
            c["dt_bias"], c["dt_softplus"] = None, False
            dtd = c.get("dt_dtype", io)
            c["dt"] = W.to_storage(rng.random(np.shape(c["dt"]), dtype=np.float32) * 0.1, dtd)
            c["buf_dt"] = W.to_storage(rng.random(np.shape(c["buf_dt"]), dtype=np.float32) * 0.1,
                                       dtd)
        if rng.integers(3) == 0:
            c["z"] = None
        if rng.integers(4) == 0:
            tab = c["state_batch_indices"].copy()
            tab[1] = -1
            c["state_batch_indices"] = tab
        if rng.integers(5) == 0:
            c["disable_state_update"] = True
        o = ssu_oracle.run_replay_spec(c, orc)
        b = brute64.run_replay_spec(c)
        for key in ("buf_x", "buf_dt", "buf_B"):
            assert np.array_equal(o[key], b[key]), (k, key)
        assert np.array_equal(o["written"], b["written"]), k
        S_o, S_b = f64(o["state"], sd), f64(b["state"], sd)
        tol = (64 * U32 * (np.abs(S_b) + 1)) if sd == "f32" else \
            (2 * ulp16(S_b, sd) + 64 * U32 * (np.abs(S_b) + 1))
        assert np.all(np.abs(S_o - S_b) <= tol), (k, sd, L)
        y_o = f64(o["y"], io)
        tol = 64 * U32 * (np.abs(b["y64"]) + 8) * 8 * (L + T)
        if io != "f32":
            tol = tol + 2 * ulp16(b["y64"], io)
        assert np.all(np.abs(y_o - b["y64"]) <= tol), (k, io, L, T)


# ------------------------------------------------------------ state copies

def pin_memmove_matches_snapshot(orc):
    """Batched copies with memmove semantics (vLLM PR #50729 digest, "测试配套":
    expected values come from slicing the untouched snapshot): rows copied
    onto themselves shifted left (the PR's regression case, scaled down) and
    right, copies to other rows, and empty copies."""
    from oracle import ssu_oracle
    for direction in ("left", "right", "apart"):
        for shift in (1, 16, 2000):
            c = W.memmove_rows(rows=6, row_bytes=4096, shift=shift, direction=direction)
            snap = c["buf"].copy()
            got = ssu_oracle.run_batch_memmove(c["buf"], c["src_off"], c["dst_off"], c["sizes"], orc)
            want = snap.copy()
            for s, d, n in zip(c["src_off"], c["dst_off"], c["sizes"]):
                want[d:d + n] = snap[s:s + n]
            assert np.array_equal(got, want), (direction, shift)
    buf = np.arange(64, dtype=np.uint8)
    got = ssu_oracle.run_batch_memmove(buf, [3], [9], [0], orc)
    assert np.array_equal(got, buf)


def pin_conv_shift_matches_snapshot(orc):
    """Convolution-state shift (vLLM PR #50729 digest, "实现拆解": state[dst][:W -
    bias] = state[src][bias:]), both layouts, the same or another block, every
    bias 0..W, element sizes 2/4/8 (the PR's fp16/fp32/fp64 cases), against
    slices of the untouched snapshot; the two layouts agree after a
    transpose; out-of-range requests write nothing."""
    from oracle import ssu_oracle
    for dt in (np.float16, np.float32, np.float64):
        for width in (4, 3):
            for bias in range(width + 1):
                sd = W.conv_shift(seed=bias, requests=4, width=width, inner=6, dtype=dt,
                                  layout="SD", same_frac=0.5)
                sd["bias"][:] = bias
                got = ssu_oracle.run_conv_shift(sd["pool"], "SD", sd["src_blk"], sd["dst_blk"],
                                                sd["bias"], orc)
                want = sd["pool"].copy()
                for s, d in zip(sd["src_blk"], sd["dst_blk"]):
                    want[d, :width - bias] = sd["pool"][s, bias:].copy()
                assert np.array_equal(got, want), (dt, width, bias)
                ds_pool = np.ascontiguousarray(sd["pool"].transpose(0, 2, 1))
                got_ds = ssu_oracle.run_conv_shift(ds_pool, "DS", sd["src_blk"], sd["dst_blk"],
                                                   sd["bias"], orc)
                assert np.array_equal(got_ds, np.ascontiguousarray(want.transpose(0, 2, 1)))
    c = W.conv_shift(seed=1, requests=3, width=4, inner=5, dtype=np.float32, layout="DS")
    c["bias"][:] = [5, -1, 1]
    c["src_blk"][2] = 99
    got = ssu_oracle.run_conv_shift(c["pool"], "DS", c["src_blk"], c["dst_blk"], c["bias"], orc)
    assert np.array_equal(got, c["pool"])


# ------------------------------------------------------------ SSD prefill

def _ssd_case(**kw):
    base = dict(seed=1, lengths=(70, 16, 1, 33), heads=4, dim=8, dstate=16, groups=2,
                chunk_size=16)
    base.update(kw)
    return W.ssd(**base)


def pin_ssd_matches_chunked_float64(orc):
    """SSD prefill (MATE "SSD packed prefill"): the token-by-token oracle
    against an independent float64 implementation of the chunked algorithm
    (decay cumsum, chunk states, state passing, intra-chunk causal sum plus
    the decayed entering state), over chunk sizes, dtypes, initial states,
    dt_limit and softplus on and off."""
    from oracle import ssu_oracle
    combos = [dict(io="f32", state_dtype="f32"), dict(io="bf16", state_dtype="f32", chunk_size=8),
              dict(io="bf16", state_dtype="bf16", initial_states=False),
              dict(io="f32", state_dtype="f32", softplus=False),            # negative dt' floored at 0
              dict(io="f32", state_dtype="f16", dt_limit=(0.01, 0.05)),
              dict(io="f32", state_dtype="f32", z=False, D=False, lengths=(5, 40, 17))]
    for kw in combos:
        c = _ssd_case(**kw)
        r = ssu_oracle.run_ssd(c, orc)
        q = brute64.run_ssd_chunked(c)
        io, sd = c["io_dtype"], c["state_dtype"]
        scale_y = np.abs(q["y64"]).max() + 1.0
        tol_y = (1e-5 if io == "f32" else 8e-3) * scale_y
        assert np.abs(f64(r["y"], io) - q["y64"]).max() <= tol_y, kw
        scale_s = np.abs(q["chunk_states64"]).max() + 1.0
        tol_s = (1e-5 if sd == "f32" else 8e-3) * scale_s
        assert np.abs(f64(r["chunk_states"], sd) - q["chunk_states64"]).max() <= tol_s, kw
        assert np.array_equal(r["states"], r["chunk_states"][c["last_chunk_indices"]])


def _ssd_as_decode(c, b):
    """Sequence b of an SSD case as a dense [1, len] plain-update case from
    its initial state (slot 0 of a one-slot pool)."""
    cu = np.asarray(c["cu_seqlens"])
    t0, t1 = int(cu[b]), int(cu[b + 1])
    H, P = np.shape(c["x"])[1:]
    N = np.shape(c["B"])[2]
    pool = (np.asarray(c["initial_states"])[b:b + 1] if c.get("initial_states") is not None
            else np.zeros((1, H, P, N), np.float32 if c["state_dtype"] == "f32" else np.uint16))
    d = {"state": pool.copy(), "state_dtype": c["state_dtype"], "io_dtype": c["io_dtype"],
         "dt_dtype": c["dt_dtype"], "A": c["A"], "D": c["D"], "dt_bias": c["dt_bias"],
         "dt_softplus": c["dt_softplus"], "pad_slot_id": -1, "disable_state_update": False,
         "cu_seqlens": None, "num_accepted_tokens": None,
         "state_batch_indices": np.zeros((1, t1 - t0), np.int64),
         "dst_state_batch_indices": np.zeros((1, t1 - t0), np.int64)}
    for k in ("x", "dt", "B", "C", "z"):
        d[k] = None if c.get(k) is None else np.asarray(c[k])[t0:t1][None]
    return d, t0, t1


def pin_ssd_equals_decode_chain(orc):
    """Each sequence of a prefill equals the plain update applied to its
    tokens one after the other from its initial state (dt' stays positive, so
    the default dt_limit is inactive), y and final state bit for bit."""
    from oracle import ssu_oracle
    c = _ssd_case(io="bf16", state_dtype="f32")
    r = ssu_oracle.run_ssd(c, orc)
    for b in (0, 1, 3):
        d, t0, t1 = _ssd_as_decode(c, b)
        p = orc.run(d)
        assert np.array_equal(r["y"][t0:t1], p["y"][0]), b
        assert np.array_equal(r["states"][b], p["state"][0]), b


def pin_ssd_chunking_invariance(orc):
    """Chunk boundaries change nothing: the same sequences split into chunks
    of 5, 16 or 64 tokens give the same outputs and final states bit for bit."""
    from oracle import ssu_oracle
    outs = [ssu_oracle.run_ssd(_ssd_case(chunk_size=k), orc) for k in (5, 16, 64)]
    for o in outs[1:]:
        assert np.array_equal(o["y"], outs[0]["y"]) and np.array_equal(o["states"], outs[0]["states"])


def pin_ssd_empty_chunks(orc):
    """A chunk of zero tokens (cu_chunk_seqlens repeating an entry) changes
    nothing, inside a sequence, opening one or ending one: outputs and final
    states equal the case without them bit for bit, and the empty chunk's
    own intermediate state is the state before it."""
    from oracle import ssu_oracle
    c = _ssd_case(lengths=(40, 30), initial_states=True)
    cu, seq = np.asarray(c["cu_chunk_seqlens"]), np.asarray(c["seq_idx"])
    out = []
    first1 = int(np.argmax(seq == 1))
    for k in range(len(seq)):
        if k == first1:
            out.append((int(cu[k]), int(cu[k]), 1))          # opens sequence 1
        out.append((int(cu[k]), int(cu[k + 1]), int(seq[k])))
        if k == 0:
            out.append((int(cu[1]), int(cu[1]), int(seq[0])))  # inside sequence 0
    out.append((int(cu[-1]), int(cu[-1]), int(seq[-1])))        # ends the last sequence
    e = dict(c, cu_chunk_seqlens=np.asarray([0] + [q[1] for q in out], np.int64),
             seq_idx=np.asarray([q[2] for q in out], np.int64),
             last_chunk_indices=np.asarray([max(k for k, q in enumerate(out) if q[2] == b) for b in (0, 1)],
                                           np.int64))
    r0 = ssu_oracle.run_ssd(c, orc)
    r = ssu_oracle.run_ssd(e, orc)
    assert np.array_equal(r["y"], r0["y"]) and np.array_equal(r["states"], r0["states"])
    # the empty chunk inside sequence 0 (chunk 1) passes chunk 0's state on
    assert np.array_equal(r["chunk_states"][1], r["chunk_states"][0])


def pin_ssd_seq_idx_authority(orc):
    """seq_idx decides where a sequence opens: relabelling the second
    sequence's chunks as the first's makes them continue its state (the same
    as one sequence of both token ranges), whatever last_chunk_indices says."""
    from oracle import ssu_oracle
    c = _ssd_case(lengths=(40, 30), initial_states=False)
    merged = dict(c, seq_idx=np.zeros_like(c["seq_idx"]), last_chunk_indices=c["last_chunk_indices"])
    one = dict(_ssd_case(lengths=(70,), initial_states=False), x=c["x"], dt=c["dt"], B=c["B"],
               C=c["C"], z=c["z"], A=c["A"], D=c["D"], dt_bias=c["dt_bias"])
    r = ssu_oracle.run_ssd(merged, orc)
    o = ssu_oracle.run_ssd(one, orc)
    assert np.array_equal(r["y"], o["y"])
    assert np.array_equal(r["chunk_states"][-1], o["chunk_states"][-1])
    s = ssu_oracle.run_ssd(c, orc)  # the proper labels reset at the second sequence
    assert not np.array_equal(s["y"][40:], r["y"][40:])


def pin_ssd_dt_limit_zero(orc):
    """dt_limit = (0, 0) clamps every dt' to 0: the state never moves from its
    initial value and y = S_init . C + D x, gated (closed form)."""
    from oracle import ssu_oracle
    c = _ssd_case(io="f32", state_dtype="f32", dt_limit=(0.0, 0.0))
    r = ssu_oracle.run_ssd(c, orc)
    init = np.asarray(c["initial_states"], np.float64)
    for b in range(len(c["last_chunk_indices"])):
        assert np.array_equal(r["states"][b], c["initial_states"][b]), b
    cu = c["cu_seqlens"]
    G = c["B"].shape[1]
    H = c["x"].shape[1]
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            for h in range(H):
                g = h // (H // G)
                y = init[b, h] @ c["C"][t, g].astype(np.float64) + c["D"][h] * c["x"][t, h]
                zz = c["z"][t, h].astype(np.float64)
                y = y * zz / (1 + np.exp(-zz))
                assert np.allclose(r["y"][t, h], y, rtol=1e-5, atol=1e-5), (b, t, h)


# ---------------------------------------------------- MXFP8 read copy (R30-R32)

def pin_e4m3_codec(orc):
    """FP8 E4M3 (OCP): decoding every one of the 256 codes and encoding
    in-range values (ties to even included) agree with PyTorch's float8_e4m3fn
    (a library implementation); every finite code round-trips; magnitudes
    above 448 saturate (R31)."""
    import torch
    from oracle import ssu_oracle
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib_vals = codes.view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        v = ssu_oracle.e4m3_decode(c, orc)
        assert (np.isnan(v) and np.isnan(lib_vals[c])) or v == lib_vals[c], c
        if not np.isnan(v):
            assert ssu_oracle.e4m3_encode(v, orc) == c or (v == 0.0 and c in (0, 0x80)), c
    finite = np.sort(lib_vals[np.isfinite(lib_vals) & (lib_vals >= 0)])
    finite = np.unique(finite)
    mids = (finite[:-1] + finite[1:]) / 2            # ties
    rng = np.random.default_rng(3)
    probes = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                             rng.uniform(0, 463.9, 4000), rng.uniform(0, 2 ** -5, 2000)]).astype(np.float32)
    probes = np.concatenate([probes, -probes])
    want = torch.from_numpy(probes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([ssu_oracle.e4m3_encode(v, orc) for v in probes], np.uint8)
    assert np.array_equal(got, want)
    for v in (464.0, 500.0, 1e30, -480.0):
        assert ssu_oracle.e4m3_encode(v, orc) == (0x7E if v > 0 else 0xFE), v


def pin_mx8_blocks(orc):
    """MXFP8 blocks (R30) against the OCP MX definition, with the formats
    decoded by a library (PyTorch's float8_e8m0fnu and float8_e4m3fn): the
    scale byte decodes to X = 2^k with the block's largest magnitude in
    [2^emax, 2^(emax+1)) X, emax being the exponent of E4M3's largest finite
    value (8); so the largest code of every block sits in E4M3's top binade
    (clipped to its largest value above it). Away from the exponent clamp,
    every unclipped element decodes within half an E4M3 step (1/16 relative,
    2^-10 X below the normal range), and an already decoded block is a fixed
    point. A block of zeros has zero codes (and byte 1, k = -126)."""
    import torch
    from oracle import ssu_oracle
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-12, 12, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    x[5] *= np.float32(1e-38)                      # scale exponent clamped at -126
    codes, scales = ssu_oracle.mx8_quantize(x, orc)
    X = torch.from_numpy(scales[:, 0].copy()).view(torch.float8_e8m0fnu).double().numpy()
    e4 = torch.from_numpy(codes.reshape(-1).copy()).view(torch.float8_e4m3fn).double().numpy()
    e4 = e4.reshape(codes.shape)
    fmax = float(torch.finfo(torch.float8_e4m3fn).max)
    emax = math.floor(math.log2(fmax))
    amax = np.abs(x).max(axis=1).astype(np.float64)
    live = (amax > 0) & (np.arange(64) != 5)
    ratio = amax[live] / X[live]
    assert np.all(ratio >= 2.0 ** emax) and np.all(ratio < 2.0 ** (emax + 1)), ratio
    top = np.abs(e4[live]).max(axis=1)
    assert np.all((top >= 2.0 ** emax) & (top <= fmax)), top
    assert scales[3, 0] == 1 and not codes[3].any()
    assert scales[5, 0] == 1                     # 2^-126, the smallest scale R30 allows
    deq = ssu_oracle.mx8_dequantize(codes, scales, orc).astype(np.float64)
    assert np.array_equal(deq, e4 * X[:, None])  # decode = E4M3 value x E8M0 scale
    sc = np.broadcast_to(X[:, None], x.shape)
    clipped = np.abs(x) / sc >= fmax + 16        # beyond the rounding edge (464)
    assert np.all(np.abs(deq[clipped]) == (fmax * sc)[clipped])
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) / 16, sc * 2.0 ** -10)
    assert np.all(err[~clipped] <= bound[~clipped])
    c2, s2 = ssu_oracle.mx8_quantize(deq.astype(np.float32), orc)
    assert np.array_equal(ssu_oracle.mx8_dequantize(c2, s2, orc), deq.astype(np.float32))


# ---------------------------------------------------- MXFP4 read copy (R33, R34)

# FP4 E2M1 magnitudes as the OCP Microscaling v1.0 specification tabulates
# them (codes 0..7; codes 8..15 are their negatives)
E2M1_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def pin_e2m1_codec(orc):
    """FP4 E2M1 (R34): the 16 codes decode to the OCP table (and each value is
    exact in PyTorch's float8_e4m3fn, a library check of the literals); every
    code round-trips; encoding any value below 6 gives the table's nearest
    value, ties to the even code (brute force over the table); values of 6
    and above saturate to 6."""
    import torch
    from oracle import ssu_oracle
    want = list(E2M1_TABLE) + [-v for v in E2M1_TABLE]
    got = [ssu_oracle.e2m1_decode(c, orc) for c in range(16)]
    assert got == want and all(math.copysign(1, g) == (-1 if c >= 8 else 1) for c, g in enumerate(got))
    t = torch.tensor(want, dtype=torch.float32)
    assert torch.equal(t.to(torch.float8_e4m3fn).float(), t)
    for c in range(16):
        assert ssu_oracle.e2m1_encode(got[c], orc) == c, c
    rng = np.random.default_rng(5)
    mags = np.asarray(E2M1_TABLE)
    mids = (mags[:-1] + mags[1:]) / 2
    probes = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                             rng.uniform(0, 6, 3000)]).astype(np.float32)
    for v in probes:
        d = np.abs(mags - float(v))
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])  # ties: the even code
        assert ssu_oracle.e2m1_encode(float(v), orc) == code, v
        assert ssu_oracle.e2m1_encode(-float(v), orc) == code | 8, v
    for v in (6.0, 6.5, 7.0, 1e30):
        assert ssu_oracle.e2m1_encode(v, orc) == 7 and ssu_oracle.e2m1_encode(-v, orc) == 15, v


def pin_mx4_blocks(orc):
    """MXFP4 blocks (R33, R34) against the OCP MX definition with the scale
    decoded by PyTorch's float8_e8m0fnu: max |x| / X lies in
    [2^emax, 2^(emax+1)), emax = 2 being the exponent of E2M1's largest
    value (6); every block's largest code sits in E2M1's top binade [4, 6];
    unclipped elements decode within half a step (|x| / 4, X / 4 below 1 X),
    clipped ones to 6 X; element 2i is the low nibble of byte i; a decoded
    block is a fixed point; a block of zeros has zero codes."""
    import torch
    from oracle import ssu_oracle
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-12, 12, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    x[7, :] = 0.0
    x[7, 0] = 5.0
    codes, scales = ssu_oracle.mx4_quantize(x, orc)
    assert codes.shape == (64, 16) and scales.shape == (64, 1)
    X = torch.from_numpy(scales[:, 0].copy()).view(torch.float8_e8m0fnu).double().numpy()
    emax = math.floor(math.log2(max(E2M1_TABLE)))
    amax = np.abs(x).max(axis=1).astype(np.float64)
    live = amax > 0
    ratio = amax[live] / X[live]
    assert np.all(ratio >= 2.0 ** emax) and np.all(ratio < 2.0 ** (emax + 1)), ratio
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(64, 32)  # element 2i low, 2i + 1 high
    vals = np.where(nib >= 8, -1.0, 1.0) * np.asarray(E2M1_TABLE)[nib & 7]
    top = np.abs(vals[live]).max(axis=1)
    assert np.all((top >= 4.0) & (top <= 6.0)), top
    assert not codes[3].any() and scales[3, 0] == 1
    assert codes[7, 0] == ssu_oracle.e2m1_encode(5.0 / X[7], orc)  # the low nibble of byte 0
    deq = ssu_oracle.mx4_dequantize(codes, scales, orc).astype(np.float64)
    assert np.array_equal(deq, vals * X[:, None])
    sc = np.broadcast_to(X[:, None], x.shape)
    clipped = np.abs(x) / sc >= 6.0
    assert np.all(np.abs(deq[clipped]) == (6.0 * sc)[clipped])
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) / 4, sc / 4)
    assert np.all(err[~clipped] <= bound[~clipped])
    c2, s2 = ssu_oracle.mx4_quantize(deq.astype(np.float32), orc)
    assert np.array_equal(ssu_oracle.mx4_dequantize(c2, s2, orc), deq.astype(np.float32))


def pin_replay_read_copy_mx4(orc):
    """ReplaySSM with an MXFP4 read copy (R32 with R33, R34): an output-only
    step equals the plain replay step run on the copy's decoded values; a
    fold ignores the copy, matches the plain step bit for bit and rewrites
    exactly the folded slot's copy."""
    from oracle import ssu_oracle
    c = _replay_case(6, [0, 5, 3, 5], sd="f32", io="bf16", dstate=64)  # sequences 1 and 3 fold
    c["lp"], c["lp_scale"] = ssu_oracle.mx4_quantize(np.asarray(c["state"], np.float32) * np.float32(1.7), orc)
    c["lp_format"] = "mx4"
    r = ssu_oracle.run_replay(c, orc)
    plain_c = {k: v for k, v in c.items() if not k.startswith("lp")}
    deq = ssu_oracle.mx4_dequantize(c["lp"], c["lp_scale"], orc)
    plain_deq = ssu_oracle.run_replay(dict(plain_c, state=deq), orc)
    plain = ssu_oracle.run_replay(plain_c, orc)
    tab = c["state_batch_indices"]
    for b in (0, 2):
        assert np.array_equal(r["y"][b], plain_deq["y"][b]), b
    for b in (1, 3):
        assert np.array_equal(r["y"][b], plain["y"][b]), b
    assert np.array_equal(r["state"], plain["state"])
    for b in range(4):
        s = tab[b]
        if b in (1, 3):
            qc, qs = ssu_oracle.mx4_quantize(plain["state"][s], orc)
            assert np.array_equal(r["lp"][s], qc) and np.array_equal(r["lp_scale"][s], qs), b
        else:
            assert np.array_equal(r["lp"][s], c["lp"][s]), b


def pin_threads_byte_identical(orc):
    """Sequences are independent (the oracle refuses shared slots), so the
    oracle threaded over sequences gives the serial result byte for byte:
    the update on every sequence layout, the replay step and the speculative
    step."""
    from oracle import ssu_oracle
    cases = [("ssu", small("varlen", nseq=13, heads=4, dim=8, dstate=16)),
             ("ssu", small("mtp", nseq=7, steps=3, heads=4, dim=8, dstate=16, groups=2)),
             ("ssu", small("decode", batch=9, heads=4, dim=8, dstate=16, groups=2, slots=12)),
             ("replay", _replay_case(4, [0, 3, 1, 2, 3, 0, 2], batch=7, slots=9)),
             ("spec", _spec_case(8, 2, [0, 5, 7, 8, 2, 6], batch=6, slots=8))]
    before = orc.threads()
    try:
        for kind, c in cases:
            fn = {"ssu": ssu_oracle.run, "replay": ssu_oracle.run_replay,
                  "spec": ssu_oracle.run_replay_spec}[kind]
            orc.set_threads(1)
            one = fn(c, orc)
            for n in (3, 8):
                orc.set_threads(n)
                many = fn(c, orc)
                for k in one:
                    assert np.array_equal(np.asarray(one[k]), np.asarray(many[k])), (kind, n, k)
    finally:
        orc.set_threads(before)


def _lp_case(L, buf_len, **kw):
    from oracle import ssu_oracle
    c = _replay_case(L, buf_len, sd="f32", io="bf16", dstate=64, **kw)
    c["lp"], c["lp_scale"] = ssu_oracle.mx8_quantize(
        np.asarray(c["state"], np.float32) * np.float32(1.7), orc_default())
    return c


def orc_default():
    from oracle import ssu_oracle
    return ssu_oracle.default()


def pin_replay_read_copy(orc):
    """ReplaySSM with an MXFP8 read copy (R32): an output-only step equals the
    plain replay step run on the copy's decoded values (the high-precision
    pool is not read); a fold ignores the copy, matches the plain replay step
    bit for bit, and rewrites exactly the folded slot's copy with the
    quantized new checkpoint."""
    from oracle import ssu_oracle
    c = _lp_case(6, [0, 5, 3, 5])                  # sequences 1 and 3 fold
    r = ssu_oracle.run_replay(c, orc)
    deq = ssu_oracle.mx8_dequantize(c["lp"], c["lp_scale"], orc)
    plain_deq = ssu_oracle.run_replay(dict({k: v for k, v in c.items() if not k.startswith("lp")},
                                           state=deq), orc)
    plain = ssu_oracle.run_replay({k: v for k, v in c.items() if not k.startswith("lp")}, orc)
    tab = c["state_batch_indices"]
    for b in (0, 2):
        assert np.array_equal(r["y"][b], plain_deq["y"][b]), b
    for b in (1, 3):
        assert np.array_equal(r["y"][b], plain["y"][b]), b
    assert np.array_equal(r["state"], plain["state"])
    for b in range(4):
        s = tab[b]
        if b in (1, 3):
            qc, qs = ssu_oracle.mx8_quantize(plain["state"][s], orc)
            assert np.array_equal(r["lp"][s], qc) and np.array_equal(r["lp_scale"][s], qs), b
        else:
            assert np.array_equal(r["lp"][s], c["lp"][s]), b
    d = ssu_oracle.run_replay(dict(c, disable_state_update=True), orc)
    assert np.array_equal(d["lp"], c["lp"]) and np.array_equal(d["lp_scale"], c["lp_scale"])


ALL = [pin_golden_mate_examples, pin_f16_decode_exhaustive, pin_f16_encode, pin_bf16_roundtrip, pin_softplus,
       pin_dt_zero_keeps_state, pin_b_zero_pure_decay, pin_zero_state_closed_form,
       pin_c_zero_and_z_zero, pin_mtp_equals_chained_calls, pin_unrolled_window,
       pin_pad_slot_untouched, pin_disable_keeps_pool, pin_flat_equals_2d, pin_strided_literal,
       pin_default_destination, pin_empty_sequences, pin_accepted_floor,
       pin_pad_destination_mid_sequence, pin_dt_per_head_broadcast, pin_groups, pin_brute_force,
       pin_replay_L1_is_plain_update, pin_replay_flush_is_chain,
       pin_replay_nonflush_writes_entry_only, pin_replay_zero_checkpoint, pin_replay_disable,
       pin_replay_brute_force, pin_replay_spec_is_chain, pin_replay_spec_rollback,
       pin_replay_spec_fold_boundary, pin_replay_spec_pad_and_disable, pin_replay_spec_brute_force,
       pin_memmove_matches_snapshot, pin_conv_shift_matches_snapshot,
       pin_ssd_matches_chunked_float64, pin_ssd_equals_decode_chain, pin_ssd_chunking_invariance,
       pin_ssd_seq_idx_authority, pin_ssd_empty_chunks, pin_ssd_dt_limit_zero, pin_e4m3_codec, pin_mx8_blocks,
       pin_replay_read_copy, pin_e2m1_codec, pin_mx4_blocks, pin_replay_read_copy_mx4,
       pin_threads_byte_identical]
