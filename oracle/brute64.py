"""Float64 brute force of the selective state update, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). It exists to pin the C
oracle: it is written separately (Python over rows and heads, NumPy over the
[dim, dstate] tile, float64 arithmetic), from the same pages:
  - MATE docs, "Mamba / SSU", table "SSU at a glance" (layouts, slot rules,
    variable-length and MTP decode) and the API reference's argument list;
  - ReplaySSM article (lpnh.cn), section "三个瓶颈其实来自同一个动作": the
    step S_t = a_t S_{t-1} + dt_t x_t B_t^T with the readout y_t = S_t C_t.
Same readings as the C oracle (R1..R12 in its header). Rounding happens only
where the method stores a value: the carried/stored state in the state dtype
and y in the io dtype. Library routines do the dtype casts (NumPy for half,
PyTorch for bfloat16).
"""
import numpy as np
import torch


def to_f64(a, dtype):
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def from_f64(v, dtype):
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rows_of_sequences(case, R):
    """[(first row, length)] per sequence, from the call's layout."""
    x = np.asarray(case["x"])
    cu = case.get("cu_seqlens")
    if cu is not None:
        cu = [int(v) for v in np.asarray(cu)]
        return [(cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]
    if x.ndim == 4:
        T = x.shape[1]
        return [(b * T, T) for b in range(x.shape[0])]
    return [(r, 1) for r in range(R)]


def _lookup(table, b, first_row, t):
    """Slot named by sequence b's position t (1-D tables are row-indexed)."""
    if hasattr(table, "base") and not isinstance(table, np.ndarray):
        base = np.asarray(table.base).ravel()
        if len(table.shape) == 1:
            return int(base[first_row + t])
        return int(base[b * table.strides[0] + t * table.strides[1]])
    table = np.asarray(table)
    if table.ndim == 1:
        return int(table[first_row + t])
    return int(table[b, t])


def run(case):
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    pool = np.asarray(case["state"])
    slots, H, P, N = pool.shape
    x = np.asarray(case["x"])
    R = x.shape[0] * (x.shape[1] if x.ndim == 4 else 1)
    X = to_f64(x, io).reshape(R, H, P)
    dt = np.asarray(case["dt"])
    if dt.ndim == x.ndim - 1:  # one value per head, broadcast over dim
        DT = np.repeat(to_f64(dt, dtd).reshape(R, H, 1), P, axis=2)
    else:
        DT = to_f64(dt, dtd).reshape(R, H, P)
    G = np.asarray(case["B"]).shape[-2]
    Bm = to_f64(case["B"], io).reshape(R, G, N)
    Cm = to_f64(case["C"], io).reshape(R, G, N)
    Z = None if case.get("z") is None else to_f64(case["z"], io).reshape(R, H, P)
    A = np.asarray(case["A"], dtype=np.float64)
    Dv = None if case.get("D") is None else np.asarray(case["D"], dtype=np.float64)
    bias = None if case.get("dt_bias") is None else np.asarray(case["dt_bias"], dtype=np.float64)
    pad = int(case.get("pad_slot_id", -1))
    disable = bool(case.get("disable_state_update", False))
    rtab = case.get("state_batch_indices")
    wtab = case.get("dst_state_batch_indices")
    acc = case.get("num_accepted_tokens")

    new_pool = pool.copy()
    Y = np.zeros((R, H, P), dtype=np.float64)
    written = np.zeros(slots, dtype=bool)
    per_group = H // G
    for b, (first, length) in enumerate(_rows_of_sequences(case, R)):
        if length == 0:
            continue
        start = 0 if acc is None else max(int(np.asarray(acc)[b]) - 1, 0)
        src = b if rtab is None else _lookup(rtab, b, first, start)
        for h in range(H):
            g = h // per_group
            if src == pad:
                S = np.zeros((P, N))
            else:
                S = to_f64(pool[src, h], sd)
            for t in range(length):
                r = first + t
                step = DT[r, h].copy()
                if bias is not None:
                    step = step + bias[h]
                if case.get("dt_softplus", False):
                    step = np.where(step > 20.0, step, np.log1p(np.exp(np.minimum(step, 20.0))))
                S = S * np.exp(step * A[h])[:, None] + np.outer(step * X[r, h], Bm[r, g])
                y = S @ Cm[r, g]
                if Dv is not None:
                    y = y + Dv[h] * X[r, h]
                if Z is not None:
                    y = y * (Z[r, h] / (1.0 + np.exp(-Z[r, h])))
                Y[r, h] = y
                S = to_f64(from_f64(S, sd), sd)
                if disable:
                    continue
                if wtab is not None:
                    dst = _lookup(wtab, b, first, t)
                elif rtab is not None:
                    dst = _lookup(rtab, b, first, t)
                else:
                    dst = b
                if dst == pad:
                    continue
                new_pool[dst, h] = from_f64(S, sd)
                written[dst] = True
    y = from_f64(Y, io).reshape(x.shape)
    return {"y": y, "y64": Y.reshape(x.shape), "state": new_pool, "written": written}


def run_replay(case):
    """ReplaySSM decode step in float64 (readings R16..R19 of the C oracle):
    a flush (h + 1 == L) folds the buffered steps and the current one into the
    checkpoint one plain update after the other; any other step computes y
    from the checkpoint and the buffer with the unrolled window and appends
    its inputs at entry h."""
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    pool = np.asarray(case["state"])
    slots, H, P, N = pool.shape
    L = int(case["L"])
    X = to_f64(case["x"], io)
    R = X.shape[0]
    dt = np.asarray(case["dt"])
    per_head = dt.ndim == 2
    DT = to_f64(dt, dtd)
    Bm, Cm = to_f64(case["B"], io), to_f64(case["C"], io)
    G = Bm.shape[1]
    Z = None if case.get("z") is None else to_f64(case["z"], io)
    A = np.asarray(case["A"], np.float64)
    Dv = None if case.get("D") is None else np.asarray(case["D"], np.float64)
    bias = None if case.get("dt_bias") is None else np.asarray(case["dt_bias"], np.float64)
    pad = int(case.get("pad_slot_id", -1))
    disable = bool(case.get("disable_state_update", False))
    tab = case.get("state_batch_indices")
    bx, bdt, bB = (np.asarray(case["buf_x"]), np.asarray(case["buf_dt"]),
                   np.asarray(case["buf_B"]))
    out = {"state": pool.copy(), "buf_x": bx.copy(), "buf_dt": bdt.copy(), "buf_B": bB.copy(),
           "written": np.zeros(slots, dtype=bool)}
    Y = np.zeros((R, H, P))

    def proc(v, h):
        if bias is not None:
            v = v + bias[h]
        if case.get("dt_softplus", False):
            v = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
        return v

    for b in range(R):
        s = b if tab is None else int(np.asarray(tab)[b])
        hb = 0 if s == pad else int(np.asarray(case["buf_len"])[b])  # the pad id has no buffer
        for h in range(H):
            g = h // (H // G)
            # the steps' inputs: buffered entries, then the current step
            xs = [to_f64(bx[s, j, h], io) for j in range(hb)] + [X[b, h]]
            if per_head:
                dts = [np.full(P, to_f64(bdt[s, j, h], dtd)) for j in range(hb)] + \
                      [np.full(P, DT[b, h])]
            else:
                dts = [to_f64(bdt[s, j, h], dtd) for j in range(hb)] + [DT[b, h]]
            Bs = [to_f64(bB[s, j, g], io) for j in range(hb)] + [Bm[b, g]]
            steps = [proc(d, h) for d in dts]
            alphas = [np.exp(st * A[h]) for st in steps]
            S = np.zeros((P, N)) if s == pad else to_f64(pool[s, h], sd)
            if hb + 1 == L:
                for j in range(hb + 1):
                    S = S * alphas[j][:, None] + np.outer(steps[j] * xs[j], Bs[j])
                    if j == hb:
                        y = S @ Cm[b, g]
                    S = to_f64(from_f64(S, sd), sd)
                if s != pad and not disable:
                    out["state"][s, h] = from_f64(S, sd)
                    out["written"][s] = True
            else:
                gamma = np.prod(alphas, axis=0)
                y = gamma * (S @ Cm[b, g])
                for j in range(hb + 1):
                    tail = np.prod(alphas[j + 1:], axis=0) if j < hb else np.ones(P)
                    y = y + steps[j] * xs[j] * tail * (Bs[j] @ Cm[b, g])
                if s != pad and not disable:
                    out["buf_x"][s, hb, h] = np.asarray(case["x"])[b, h]
                    out["buf_dt"][s, hb, h] = dt[b, h]
                    out["buf_B"][s, hb, g] = np.asarray(case["B"])[b, g]
            if Dv is not None:
                y = y + Dv[h] * X[b, h]
            if Z is not None:
                y = y * (Z[b, h] / (1.0 + np.exp(-Z[b, h])))
            Y[b, h] = y
    out["y"] = from_f64(Y, io)
    out["y64"] = Y
    return out


def run_replay_spec(case):
    """ReplaySSM speculative step in float64 (readings R21..R23 of the C
    oracle): T drafts per sequence; when h + 2T > L the h committed entries
    are first applied to the checkpoint (stored), and the window restarts
    empty; draft t is read out over the window's committed entries and drafts
    0..t; the drafts are appended after the window's committed entries."""
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    pool = np.asarray(case["state"])
    slots, H, P, N = pool.shape
    L = int(case["L"])
    x = np.asarray(case["x"])
    Bt, T = x.shape[:2]
    X = to_f64(x, io)
    dt = np.asarray(case["dt"])
    per_head = dt.ndim == 3
    DT = to_f64(dt, dtd)
    Bm, Cm = to_f64(case["B"], io), to_f64(case["C"], io)
    G = Bm.shape[2]
    Z = None if case.get("z") is None else to_f64(case["z"], io)
    A = np.asarray(case["A"], np.float64)
    Dv = None if case.get("D") is None else np.asarray(case["D"], np.float64)
    bias = None if case.get("dt_bias") is None else np.asarray(case["dt_bias"], np.float64)
    pad = int(case.get("pad_slot_id", -1))
    disable = bool(case.get("disable_state_update", False))
    tab = case.get("state_batch_indices")
    bx, bdt, bB = (np.asarray(case["buf_x"]), np.asarray(case["buf_dt"]),
                   np.asarray(case["buf_B"]))
    out = {"state": pool.copy(), "buf_x": bx.copy(), "buf_dt": bdt.copy(), "buf_B": bB.copy(),
           "written": np.zeros(slots, dtype=bool)}
    Y = np.zeros((Bt, T, H, P))

    def proc(v, h):
        if bias is not None:
            v = v + bias[h]
        if case.get("dt_softplus", False):
            v = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
        return v

    for b in range(Bt):
        s = b if tab is None else int(np.asarray(tab)[b])
        hc = 0 if s == pad else int(np.asarray(case["buf_len"])[b])
        fold = hc + 2 * T > L
        w = 0 if fold else hc
        for h in range(H):
            g = h // (H // G)

            def entry(j):  # (dt' over dim, x, B) of buffer entry j
                d = np.full(P, to_f64(bdt[s, j, h], dtd)) if per_head else to_f64(bdt[s, j, h], dtd)
                return proc(d, h), to_f64(bx[s, j, h], io), to_f64(bB[s, j, g], io)

            def draft(t):
                d = np.full(P, DT[b, t, h]) if per_head else DT[b, t, h]
                return proc(d, h), X[b, t, h], Bm[b, t, g]

            S = np.zeros((P, N)) if s == pad else to_f64(pool[s, h], sd)
            if fold:
                for j in range(hc):
                    st, xv, Bv = entry(j)
                    S = S * np.exp(st * A[h])[:, None] + np.outer(st * xv, Bv)
                    S = to_f64(from_f64(S, sd), sd)
                if s != pad and not disable:
                    out["state"][s, h] = from_f64(S, sd)
                    out["written"][s] = True
            steps = [entry(j) for j in range(w)] + [draft(t) for t in range(T)]
            for t in range(T):
                C = Cm[b, t, g]
                window = steps[:w + t + 1]
                alphas = [np.exp(st * A[h]) for st, _, _ in window]
                y = np.prod(alphas, axis=0) * (S @ C)
                for j, (st, xv, Bv) in enumerate(window):
                    tail = np.prod(alphas[j + 1:], axis=0) if j + 1 < len(window) else np.ones(P)
                    y = y + st * xv * tail * (Bv @ C)
                if Dv is not None:
                    y = y + Dv[h] * X[b, t, h]
                if Z is not None:
                    y = y * (Z[b, t, h] / (1.0 + np.exp(-Z[b, t, h])))
                Y[b, t, h] = y
            if s != pad and not disable:
                for t in range(T):
                    out["buf_x"][s, w + t, h] = x[b, t, h]
                    out["buf_dt"][s, w + t, h] = dt[b, t, h]
                    out["buf_B"][s, w + t, g] = np.asarray(case["B"])[b, t, g]
    out["y"] = from_f64(Y, io)
    out["y64"] = Y
    return out


def run_ssd_chunked(case):
    """SSD prefill in float64 by the chunked algorithm (not the token loop of
    the C oracle): per chunk, the decay cumsum, the chunk's own state from a
    zero start, the state passed in from the previous chunk (or the initial
    state where seq_idx opens a sequence), and each token's output as the
    intra-chunk causal sum plus the decayed entering state read out by C."""
    io, sd = case["io_dtype"], case["state_dtype"]
    dtd = case.get("dt_dtype", io)
    X = to_f64(case["x"], io)
    T, H, P = X.shape
    DT = to_f64(case["dt"], dtd)
    Bm, Cm = to_f64(case["B"], io), to_f64(case["C"], io)
    G, N = Bm.shape[1:]
    Z = None if case.get("z") is None else to_f64(case["z"], io)
    A = np.asarray(case["A"], np.float64)
    Dv = None if case.get("D") is None else np.asarray(case["D"], np.float64)
    bias = None if case.get("dt_bias") is None else np.asarray(case["dt_bias"], np.float64)
    lo, hi = case.get("dt_limit", (0.0, float("inf")))
    init = None if case.get("initial_states") is None else to_f64(case["initial_states"], sd)
    cu = np.asarray(case["cu_chunk_seqlens"])
    seq = np.asarray(case["seq_idx"])
    nch = len(seq)
    Y = np.zeros((T, H, P))
    states = np.zeros((nch, H, P, N))
    for h in range(H):
        g = h // (H // G)
        S_prev = None
        for c in range(nch):
            t0, t1 = int(cu[c]), int(cu[c + 1])
            v = DT[t0:t1, h].copy()
            if bias is not None:
                v = v + bias[h]
            if case.get("dt_softplus", False):
                v = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
            v = np.clip(v, lo, hi)
            acum = np.cumsum(v * A[h])                      # decay cumsum in the chunk
            x, Bc, Cc = X[t0:t1, h], Bm[t0:t1, g], Cm[t0:t1, g]
            if c == 0 or seq[c] != seq[c - 1]:
                S_in = init[seq[c], h] if init is not None else np.zeros((P, N))
            else:
                S_in = S_prev
            # the chunk's own state from zero: sum_t exp(acum[-1] - acum[t]) dt'_t x_t B_t^T
            w = np.exp(acum[-1] - acum) * v if len(v) else v
            S_own = (x * w[:, None]).T @ Bc
            S_out = np.exp(acum[-1] if len(v) else 0.0) * S_in + S_own
            # outputs: causal intra-chunk sum plus the entering state
            L = t1 - t0
            CB = Cc @ Bc.T
            decay = np.exp(acum[:, None] - acum[None, :]) * np.tril(np.ones((L, L)))
            y = (CB * decay * v[None, :]) @ x + np.exp(acum)[:, None] * (Cc @ S_in.T)
            if Dv is not None:
                y = y + Dv[h] * x
            if Z is not None:
                zz = Z[t0:t1, h]
                y = y * (zz / (1.0 + np.exp(-zz)))
            Y[t0:t1, h] = y
            states[c, h] = S_out
            S_prev = S_out
    last = np.asarray(case["last_chunk_indices"])
    return {"y64": Y, "chunk_states64": states, "states64": states[last],
            "y": from_f64(Y, io), "chunk_states": from_f64(states, sd)}
