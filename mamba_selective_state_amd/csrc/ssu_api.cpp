// Host entry points of libssu: argument validation, kernel selection and the
// single launch of ssu_update; ssu_plan (the prewarm of the MATE API).
//
// Validation only looks at shapes, strides, dtypes and pointer alignment; it
// never reads device memory, so ssu_update makes no host/device copy and no
// synchronisation (MATE docs, "Mamba / SSU", section "Graph capture").
// Anything outside the supported contract is an error naming the rule or the
// capability (MATE, the paragraph after "dt_limit": NotImplementedError or
// ValueError rather than silently narrowing semantics).
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace {

thread_local std::string g_error;

ssu_status_t fail(ssu_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

}  // namespace

ssu_status_t ssu::report_error(ssu_status_t st, const char *msg) {
    g_error = msg;
    return st;
}

namespace {

bool is_float(int d) { return d == SSU_F32 || d == SSU_F16 || d == SSU_BF16; }
bool is_index(int d) { return d == SSU_I32 || d == SSU_I64; }
int64_t elem_bytes(int d) {
    return (d == SSU_F16 || d == SSU_BF16) ? 2 : (d == SSU_I64 || d == SSU_F64) ? 8 : d == SSU_U8 ? 1 : 4;
}
bool known_dtype(int d) { return d >= SSU_F32 && d <= SSU_U8; }
bool present(const ssu_tensor_t &t) { return t.data != nullptr; }
bool dstate_supported(int64_t n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
bool aligned(const void *p, int64_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

const char *dtype_str(int d) {
    switch (d) {
    case SSU_F32: return "f32";
    case SSU_F16: return "f16";
    case SSU_BF16: return "bf16";
    case SSU_I32: return "i32";
    case SSU_I64: return "i64";
    case SSU_F64: return "f64";
    case SSU_U8: return "u8";
    }
    return "unknown";
}

// The row structure every per-row tensor shares with x.
struct Rows {
    int32_t ndim;   // 3 (rows, ...) or 4 (batch, steps, ...)
    int64_t lead0;  // rows, or batch
    int64_t lead1;  // steps (4-D only)
    int64_t rows;   // total rows
};

// Checks that `t` is [lead..., M, K] (K omitted when k < 0) matching the row
// structure, with strides >= 0, and returns the row stride and the strides
// of the M and K axes. A 4-D tensor must be addressable as rows: its batch
// stride equals steps * its step stride (or one of the two axes has size 1).
ssu_status_t row_tensor(const char *name, const ssu_tensor_t &t, const Rows &rw, int64_t m,
                        int64_t k, int64_t *sr, int64_t *sm, int64_t *sk) {
    const int lead = rw.ndim - 2;
    const int want = lead + 1 + (k >= 0 ? 1 : 0);
    if (t.ndim != want)
        return fail(SSU_ERR_VALUE, "%s must have %d dimensions, got %d", name, want, t.ndim);
    for (int i = 0; i < t.ndim; i++)
        if (t.stride[i] < 0)
            return fail(SSU_ERR_VALUE, "%s has a negative stride", name);
    if (t.size[0] != rw.lead0 || (lead == 2 && t.size[1] != rw.lead1))
        return fail(SSU_ERR_VALUE, "%s leading shape does not match x", name);
    if (t.size[lead] != m)
        return fail(SSU_ERR_VALUE, "%s axis %d is %lld, expected %lld", name, lead,
                    (long long)t.size[lead], (long long)m);
    if (k >= 0 && t.size[lead + 1] != k)
        return fail(SSU_ERR_VALUE, "%s last axis is %lld, expected %lld", name,
                    (long long)t.size[lead + 1], (long long)k);
    if (lead == 1) {
        *sr = t.stride[0];
    } else if (rw.lead1 == 1) {
        *sr = t.stride[0];
    } else {
        if (rw.lead0 > 1 && t.stride[0] != rw.lead1 * t.stride[1])
            return fail(SSU_ERR_NOT_IMPLEMENTED,
                        "%s: a [batch, steps, ...] tensor must have batch stride = steps * step "
                        "stride",
                        name);
        *sr = t.stride[1];
    }
    *sm = t.stride[lead];
    *sk = k >= 0 ? t.stride[lead + 1] : 0;
    return SSU_OK;
}

// Per-head fp32 vector: [heads], or [heads, ...] with stride 0 on the other
// axes (a broadcast view).
ssu_status_t head_vector(const char *name, const ssu_tensor_t &t, int64_t H, bool required,
                         const float **ptr, int64_t *stride) {
    if (!present(t)) {
        if (required)
            return fail(SSU_ERR_VALUE, "%s is required", name);
        *ptr = nullptr;
        *stride = 0;
        return SSU_OK;
    }
    if (t.dtype != SSU_F32)
        return fail(SSU_ERR_VALUE, "%s must be f32 per head, got %s", name, dtype_str(t.dtype));
    if (t.ndim < 1 || t.ndim > 4 || t.size[0] != H)
        return fail(SSU_ERR_VALUE, "%s must be [heads] (heads = %lld)", name, (long long)H);
    for (int i = 1; i < t.ndim; i++)
        if (t.stride[i] != 0 && t.size[i] != 1)
            return fail(SSU_ERR_VALUE, "%s must be per head: axes after the first need stride 0",
                        name);
    if (t.stride[0] < 0 || !aligned(t.data, 4))
        return fail(SSU_ERR_VALUE, "%s: bad stride or alignment", name);
    *ptr = static_cast<const float *>(t.data);
    *stride = t.stride[0];
    return SSU_OK;
}

ssu_status_t slot_table(const char *name, const ssu_tensor_t &t, const Rows &rw, int64_t nseq,
                        int32_t layout, int64_t steps, const void **ptr, int64_t *s0, int64_t *s1,
                        bool *two_d, bool *i64) {
    *ptr = nullptr;
    *s0 = *s1 = 0;
    *two_d = *i64 = false;
    if (!present(t))
        return SSU_OK;
    if (!is_index(t.dtype))
        return fail(SSU_ERR_VALUE, "%s must be i32 or i64, got %s", name, dtype_str(t.dtype));
    if (!aligned(t.data, elem_bytes(t.dtype)))
        return fail(SSU_ERR_VALUE, "%s is not aligned to its element size", name);
    if (t.ndim == 1) {
        if (t.size[0] != rw.rows)
            return fail(SSU_ERR_VALUE,
                        "%s is 1-D (one entry per row) with %lld entries; the call has %lld rows",
                        name, (long long)t.size[0], (long long)rw.rows);
        if (t.stride[0] < 0)
            return fail(SSU_ERR_VALUE, "%s has a negative stride", name);
        *s0 = t.stride[0];
    } else if (t.ndim == 2) {
        if (t.size[0] < nseq)
            return fail(SSU_ERR_VALUE, "%s is 2-D with %lld rows; the call has %lld sequences",
                        name, (long long)t.size[0], (long long)nseq);
        if (layout == ssu::kDense && t.size[1] < steps)
            return fail(SSU_ERR_VALUE, "%s has %lld columns; the call has %lld steps", name,
                        (long long)t.size[1], (long long)steps);
        if (t.stride[0] < 0 || t.stride[1] < 0)
            return fail(SSU_ERR_VALUE, "%s has a negative stride", name);
        *s0 = t.stride[0];
        *s1 = t.stride[1];
        *two_d = true;
    } else {
        return fail(SSU_ERR_VALUE, "%s must be 1-D [rows] or 2-D [sequences, steps]", name);
    }
    *ptr = t.data;
    *i64 = t.dtype == SSU_I64;
    return SSU_OK;
}

ssu_status_t meta_vector(const char *name, const ssu_tensor_t &t, int64_t want, const void **ptr,
                         int64_t *stride, bool *i64) {
    *ptr = nullptr;
    *stride = 0;
    *i64 = false;
    if (!present(t))
        return SSU_OK;
    if (!is_index(t.dtype))
        return fail(SSU_ERR_VALUE, "%s must be i32 or i64, got %s", name, dtype_str(t.dtype));
    if (t.ndim != 1 || (want >= 0 && t.size[0] != want))
        return fail(SSU_ERR_VALUE, "%s must be 1-D with %lld entries", name, (long long)want);
    if (t.stride[0] < 0 || !aligned(t.data, elem_bytes(t.dtype)))
        return fail(SSU_ERR_VALUE, "%s: bad stride or alignment", name);
    *ptr = t.data;
    *stride = t.stride[0];
    *i64 = t.dtype == SSU_I64;
    return SSU_OK;
}

// Largest element offset a strided view reaches (0 when it is empty).
int64_t max_offset(const ssu_tensor_t &t) {
    int64_t m = 0;
    for (int i = 0; i < t.ndim; i++) {
        if (t.size[i] <= 0)
            return 0;
        m += (t.size[i] - 1) * t.stride[i];
    }
    return m;
}

struct Geometry {
    int32_t block, rows_per_block, dim_tiles;
};

Geometry geometry(int64_t P, int64_t N, int state_dtype, int kind) {
    const int passes =
        ssu::passes_for(static_cast<int>(N), static_cast<int>(elem_bytes(state_dtype)), kind);
    const int64_t rows_per_wave = ssu::kRowsPerPass * passes;
    int64_t waves = (P + rows_per_wave - 1) / rows_per_wave;
    if (waves > ssu::kMaxWaves)
        waves = ssu::kMaxWaves;
    if (waves < 1)
        waves = 1;
    Geometry g;
    g.block = static_cast<int32_t>(waves * ssu::kWaveLanes);
    g.rows_per_block = static_cast<int32_t>(waves * rows_per_wave);
    g.dim_tiles = static_cast<int32_t>((P + g.rows_per_block - 1) / g.rows_per_block);
    return g;
}

const char *unsupported_option(uint32_t bits) {
    if (bits & SSU_OPT_STATE_SCALE) return "state_scale";
    if (bits & SSU_OPT_INTERMEDIATE_STATES) return "intermediate_states_buffer / intermediate_state_indices / intermediate_state_scales";
    if (bits & SSU_OPT_RAND_SEED) return "rand_seed (stochastic rounding)";
    if (bits & SSU_OPT_CACHE_STEPS) return "cache_steps";
    if (bits & SSU_OPT_ALGORITHM) return "algorithm other than 'auto'";
    if (bits & SSU_OPT_BACKEND) return "backend other than 'auto'";
    return nullptr;
}

// Vector width (elements) of the kernel's dstate accesses for a state dtype.
int64_t access_vec(int state_dtype, int64_t N) {
    const int64_t per16 = 16 / elem_bytes(state_dtype);
    const int64_t e = N / ssu::kLanesPerRow;
    return per16 < e ? per16 : e;
}

// Everything ssu_update and ssu_replay_update check and derive from the
// common arguments, without touching the device.
struct Prepared {
    ssu::Params p;
    bool empty;        // no rows or no sequences: nothing to launch
    bool multi;        // the multi-token kernel is needed
    int state_dtype, io, dt_dtype;
    int64_t slots, H, P, N, G, nseq;
    int32_t layout;
    bool rtab_2d;
    int64_t dt_sp;     // dt's stride over dim (0: one value per head)
    Geometry geo;
    int64_t grid;
};

ssu_status_t prepare(const ssu_args_t *a, Prepared *out) {
    out->empty = false;
    if (!a)
        return fail(SSU_ERR_VALUE, "args is NULL");
    if (const char *opt = unsupported_option(a->unsupported))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "%s is not implemented", opt);

    // state pool [slots, heads, dim, dstate], contiguous
    const ssu_tensor_t &st = a->state;
    if (!present(st))
        return fail(SSU_ERR_VALUE, "state is required");
    if (!is_float(st.dtype))
        return fail(SSU_ERR_VALUE, "state must be f32, f16 or bf16, got %s", dtype_str(st.dtype));
    if (st.ndim != 4)
        return fail(SSU_ERR_VALUE, "state must be [slots, heads, dim, dstate]");
    const int64_t slots = st.size[0], H = st.size[1], P = st.size[2], N = st.size[3];
    if (slots <= 0 || H <= 0 || P <= 0 || N <= 0)
        return fail(SSU_ERR_VALUE, "state has an empty axis");
    if (st.stride[3] != 1 || st.stride[2] != N || st.stride[1] != P * N || st.stride[0] != H * P * N)
        return fail(SSU_ERR_VALUE, "state must be contiguous");
    if (!aligned(st.data, 16))
        return fail(SSU_ERR_VALUE, "state must be 16-byte aligned");
    if (!dstate_supported(N))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "dstate %lld is not supported (16, 32, 64, 128, 256)",
                    (long long)N);
    if (H > INT32_MAX || P > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "heads or dim too large");

    // x and the row structure
    const ssu_tensor_t &x = a->x;
    if (!present(x))
        return fail(SSU_ERR_VALUE, "x is required");
    if (!is_float(x.dtype))
        return fail(SSU_ERR_VALUE, "x must be f32, f16 or bf16, got %s", dtype_str(x.dtype));
    const int io = x.dtype;
    Rows rw;
    rw.ndim = x.ndim;
    if (x.ndim == 3) {
        rw.lead0 = x.size[0];
        rw.lead1 = 1;
        rw.rows = x.size[0];
    } else if (x.ndim == 4) {
        rw.lead0 = x.size[0];
        rw.lead1 = x.size[1];
        rw.rows = x.size[0] * x.size[1];
    } else {
        return fail(SSU_ERR_VALUE,
                    "x must be [batch, heads, dim], [rows, heads, dim] or [batch, steps, heads, dim]");
    }
    if (rw.lead0 < 0 || rw.lead1 < 0)
        return fail(SSU_ERR_VALUE, "x has a negative size");
    ssu::Params p;
    memset(&p, 0, sizeof p);
    int64_t sk = 0;
    // element strides, narrowed to 32 bits once every span is known to fit
    int64_t x_sr = 0, x_sh = 0, dt_sr = 0, dt_sh = 0, dt_sp = 0, A_sh = 0, D_sh = 0, bias_sh = 0;
    int64_t B_sr = 0, B_sg = 0, C_sr = 0, C_sg = 0, z_sr = 0, z_sh = 0, out_sr = 0, out_sh = 0;
    int64_t r_s0 = 0, r_s1 = 0, w_s0 = 0, w_s1 = 0, cu_s = 0, acc_s = 0;
    ssu_status_t s;
    if ((s = row_tensor("x", x, rw, H, P, &x_sr, &x_sh, &sk)) != SSU_OK)
        return s;
    if (sk != 1)
        return fail(SSU_ERR_VALUE, "x must have unit stride over dim");
    if (!aligned(x.data, elem_bytes(io)))
        return fail(SSU_ERR_VALUE, "x is not aligned to its element size");

    // sequences
    int64_t nseq = 0, steps = 0;
    int32_t layout;
    if (present(a->cu_seqlens)) {
        if (x.ndim != 3)
            return fail(SSU_ERR_VALUE, "cu_seqlens goes with the packed [rows, heads, dim] x");
        if (a->cu_seqlens.ndim != 1 || a->cu_seqlens.size[0] < 1)
            return fail(SSU_ERR_VALUE, "cu_seqlens must be 1-D [nseq + 1]");
        nseq = a->cu_seqlens.size[0] - 1;
        layout = ssu::kCuSeqlens;
    } else if (x.ndim == 4) {
        nseq = rw.lead0;
        steps = rw.lead1;
        layout = ssu::kDense;
    } else {
        nseq = rw.rows;
        layout = ssu::kOneToken;
    }
    bool cu_i64 = false, acc_i64 = false;
    if ((s = meta_vector("cu_seqlens", a->cu_seqlens, nseq + 1, &p.cu, &cu_s, &cu_i64)) != SSU_OK)
        return s;
    if ((s = meta_vector("num_accepted_tokens", a->num_accepted_tokens, nseq, &p.acc, &acc_s,
                         &acc_i64)) != SSU_OK)
        return s;
    const bool multi = layout != ssu::kOneToken || p.acc != nullptr;

    // dt: full [.., heads, dim] (any strides) or one value per head
    const ssu_tensor_t &dt = a->dt;
    if (!present(dt))
        return fail(SSU_ERR_VALUE, "dt is required");
    if (dt.dtype != SSU_F32 && dt.dtype != io)
        return fail(SSU_ERR_VALUE, "dt must be f32 or the x dtype, got %s", dtype_str(dt.dtype));
    if (!aligned(dt.data, elem_bytes(dt.dtype)))
        return fail(SSU_ERR_VALUE, "dt is not aligned to its element size");
    if (dt.ndim == x.ndim) {
        if ((s = row_tensor("dt", dt, rw, H, P, &dt_sr, &dt_sh, &dt_sp)) != SSU_OK)
            return s;
    } else if (dt.ndim == x.ndim - 1) {
        if ((s = row_tensor("dt", dt, rw, H, -1, &dt_sr, &dt_sh, &sk)) != SSU_OK)
            return s;
        dt_sp = 0;
    } else {
        return fail(SSU_ERR_VALUE, "dt must be shaped like x, or like x without its last axis");
    }

    // per-head vectors
    if ((s = head_vector("A", a->A, H, true, &p.A, &A_sh)) != SSU_OK)
        return s;
    if ((s = head_vector("D", a->D, H, false, &p.D, &D_sh)) != SSU_OK)
        return s;
    if ((s = head_vector("dt_bias", a->dt_bias, H, false, &p.dt_bias, &bias_sh)) != SSU_OK)
        return s;

    // B and C: [.., groups, dstate] in the x dtype
    if (!present(a->B) || !present(a->C))
        return fail(SSU_ERR_VALUE, "B and C are required");
    if (a->B.dtype != io || a->C.dtype != io)
        return fail(SSU_ERR_VALUE, "B and C must have the x dtype");
    const int64_t G = a->B.ndim >= 2 ? a->B.size[a->B.ndim - 2] : 0;
    if (G <= 0 || H % G != 0)
        return fail(SSU_ERR_VALUE, "heads (%lld) must be divisible by groups (%lld)", (long long)H,
                    (long long)G);
    if ((s = row_tensor("B", a->B, rw, G, N, &B_sr, &B_sg, &sk)) != SSU_OK)
        return s;
    if (sk != 1)
        return fail(SSU_ERR_VALUE, "B must have unit stride over dstate");
    if ((s = row_tensor("C", a->C, rw, G, N, &C_sr, &C_sg, &sk)) != SSU_OK)
        return s;
    if (sk != 1)
        return fail(SSU_ERR_VALUE, "C must have unit stride over dstate");
    {
        const int64_t vec = access_vec(st.dtype, N);
        const int64_t bytes = vec * elem_bytes(io);
        if (!aligned(a->B.data, bytes) || !aligned(a->C.data, bytes) || B_sr % vec || B_sg % vec ||
            C_sr % vec || C_sg % vec)
            return fail(SSU_ERR_VALUE,
                        "B and C rows must start on %lld-byte boundaries (base and strides)",
                        (long long)bytes);
    }

    // z and out
    if (present(a->z)) {
        if (a->z.dtype != io)
            return fail(SSU_ERR_VALUE, "z must have the x dtype");
        if ((s = row_tensor("z", a->z, rw, H, P, &z_sr, &z_sh, &sk)) != SSU_OK)
            return s;
        if (sk != 1)
            return fail(SSU_ERR_VALUE, "z must have unit stride over dim");
        if (!aligned(a->z.data, elem_bytes(io)))
            return fail(SSU_ERR_VALUE, "z is not aligned to its element size");
        p.z = a->z.data;
    }
    if (!present(a->out))
        return fail(SSU_ERR_VALUE, "out is required");
    if (a->out.dtype != io)
        return fail(SSU_ERR_VALUE, "out must have the x dtype");
    if ((s = row_tensor("out", a->out, rw, H, P, &out_sr, &out_sh, &sk)) != SSU_OK)
        return s;
    if (sk != 1)
        return fail(SSU_ERR_VALUE, "out must have unit stride over dim");
    if (!aligned(a->out.data, elem_bytes(io)))
        return fail(SSU_ERR_VALUE, "out is not aligned to its element size");

    // slot tables
    bool r2d, ri64, w2d, wi64;
    if ((s = slot_table("state_batch_indices", a->state_batch_indices, rw, nseq, layout, steps,
                        &p.rtab, &r_s0, &r_s1, &r2d, &ri64)) != SSU_OK)
        return s;
    if ((s = slot_table("dst_state_batch_indices", a->dst_state_batch_indices, rw, nseq, layout,
                        steps, &p.wtab, &w_s0, &w_s1, &w2d, &wi64)) != SSU_OK)
        return s;

    out->state_dtype = st.dtype;
    out->io = io;
    out->dt_dtype = dt.dtype;
    out->slots = slots;
    out->H = H;
    out->P = P;
    out->N = N;
    out->G = G;
    out->nseq = nseq;
    out->layout = layout;
    out->multi = multi;
    out->rtab_2d = r2d;
    out->dt_sp = dt_sp;
    if (nseq <= 0 || rw.rows <= 0) {
        out->empty = true;  // nothing to do
        return SSU_OK;
    }

    // every tensor but the pool is addressed with 32-bit element offsets
    {
        const ssu_tensor_t *spans[] = {&x, &dt, &a->A, &a->B, &a->C, &a->D, &a->z, &a->dt_bias,
                                       &a->out, &a->cu_seqlens, &a->num_accepted_tokens};
        const char *names[] = {"x", "dt", "A", "B", "C", "D", "z", "dt_bias", "out",
                               "cu_seqlens", "num_accepted_tokens"};
        for (int i = 0; i < 11; i++)
            if (present(*spans[i]) && max_offset(*spans[i]) >= INT32_MAX)
                return fail(SSU_ERR_NOT_IMPLEMENTED, "%s spans 2^31 elements or more", names[i]);
        // a 2-D table may be addressed past its declared extent (a strided
        // view): bound what the kernel can reach
        const int64_t reach_r = (nseq + rw.rows) * (r_s0 > r_s1 ? r_s0 : r_s1);
        const int64_t reach_w = (nseq + rw.rows) * (w_s0 > w_s1 ? w_s0 : w_s1);
        if (reach_r >= INT32_MAX || reach_w >= INT32_MAX)
            return fail(SSU_ERR_NOT_IMPLEMENTED, "slot tables span 2^31 entries or more");
        if (rw.rows >= INT32_MAX || max_offset(x) >= INT32_MAX)
            return fail(SSU_ERR_NOT_IMPLEMENTED, "too many rows");
    }
    p.x_sr = static_cast<int32_t>(x_sr);
    p.x_sh = static_cast<int32_t>(x_sh);
    p.dt_sr = static_cast<int32_t>(dt_sr);
    p.dt_sh = static_cast<int32_t>(dt_sh);
    p.dt_sp = static_cast<int32_t>(dt_sp);
    p.A_sh = static_cast<int32_t>(A_sh);
    p.D_sh = static_cast<int32_t>(D_sh);
    p.bias_sh = static_cast<int32_t>(bias_sh);
    p.B_sr = static_cast<int32_t>(B_sr);
    p.B_sg = static_cast<int32_t>(B_sg);
    p.C_sr = static_cast<int32_t>(C_sr);
    p.C_sg = static_cast<int32_t>(C_sg);
    p.z_sr = static_cast<int32_t>(z_sr);
    p.z_sh = static_cast<int32_t>(z_sh);
    p.out_sr = static_cast<int32_t>(out_sr);
    p.out_sh = static_cast<int32_t>(out_sh);
    p.r_s0 = static_cast<int32_t>(r_s0);
    p.r_s1 = static_cast<int32_t>(r_s1);
    p.w_s0 = static_cast<int32_t>(w_s0);
    p.w_s1 = static_cast<int32_t>(w_s1);
    p.cu_s = static_cast<int32_t>(cu_s);
    p.acc_s = static_cast<int32_t>(acc_s);
    if (nseq > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "too many sequences");

    const Geometry geo = geometry(P, N, st.dtype, multi ? ssu::kTileMulti : ssu::kTileOneToken);
    const int64_t grid = nseq * H * geo.dim_tiles;
    if (grid > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "grid of %lld workgroups is too large",
                    (long long)grid);

    p.state = const_cast<void *>(st.data);
    p.slot_stride = H * P * N;
    p.x = x.data;
    p.dt = dt.data;
    p.B = a->B.data;
    p.C = a->C.data;
    p.out = const_cast<void *>(a->out.data);
    p.pad = a->pad_slot_id;
    p.nseq = static_cast<int32_t>(nseq);
    p.H = static_cast<int32_t>(H);
    p.P = static_cast<int32_t>(P);
    p.heads_per_group = static_cast<int32_t>(H / G);
    p.steps = static_cast<int32_t>(steps);
    p.layout = layout;
    p.dim_tiles = geo.dim_tiles;
    p.rows_per_block = geo.rows_per_block;
    p.flags = (dt.dtype == SSU_F32 ? ssu::kDtF32 : 0) | (a->dt_softplus ? ssu::kSoftplus : 0) |
              (a->disable_state_update ? ssu::kDisable : 0) | (r2d ? ssu::kRead2D : 0) |
              (ri64 ? ssu::kReadI64 : 0) | (w2d ? ssu::kWrite2D : 0) |
              (wi64 ? ssu::kWriteI64 : 0) | (cu_i64 ? ssu::kCuI64 : 0) |
              (acc_i64 ? ssu::kAccI64 : 0);

    out->p = p;
    out->geo = geo;
    out->grid = grid;
    return SSU_OK;
}


}  // namespace

extern "C" {

int ssu_abi_version(void) { return SSU_ABI_VERSION; }

// ---- memmove-safe state copies

// Workgroups that share one non-overlapping copy of up to `bytes` bytes:
// one per 16 KiB (256 lanes x 4 words of 16 bytes), between 1 and 64.
static int32_t copy_tiles_for(int64_t bytes) {
    const int64_t tile = static_cast<int64_t>(ssu::kCopyThreads) * 4 * 16;
    int64_t t = (bytes + tile - 1) / tile;
    return static_cast<int32_t>(t < 1 ? 1 : (t > 64 ? 64 : t));
}

ssu_status_t ssu_batch_memcpy(const ssu_tensor_t *src_ptrs, const ssu_tensor_t *dst_ptrs,
                              const ssu_tensor_t *sizes, int64_t max_size, void *stream) {
    if (!src_ptrs || !dst_ptrs || !sizes)
        return fail(SSU_ERR_VALUE, "ssu_batch_memcpy: NULL argument");
    const ssu_tensor_t *ptrs[] = {src_ptrs, dst_ptrs};
    const char *names[] = {"src_ptrs", "dst_ptrs"};
    for (int k = 0; k < 2; k++) {
        const ssu_tensor_t &t = *ptrs[k];
        if (!present(t) || t.dtype != SSU_I64 || t.ndim != 1)
            return fail(SSU_ERR_VALUE, "%s must be a 1-D i64 array of device addresses", names[k]);
        if (t.stride[0] < 0 || !aligned(t.data, 8))
            return fail(SSU_ERR_VALUE, "%s: bad stride or alignment", names[k]);
    }
    const int64_t n = src_ptrs->size[0];
    if (dst_ptrs->size[0] != n)
        return fail(SSU_ERR_VALUE, "src_ptrs and dst_ptrs differ in length");
    ssu::CopyParams cp;
    memset(&cp, 0, sizeof cp);
    int64_t sizes_s = 0;
    bool sizes_i64 = false;
    if (!present(*sizes))
        return fail(SSU_ERR_VALUE, "sizes is required");
    ssu_status_t s = meta_vector("sizes", *sizes, n, &cp.sizes, &sizes_s, &sizes_i64);
    if (s != SSU_OK)
        return s;
    if (n == 0)
        return g_error.clear(), SSU_OK;
    cp.src_ptrs = src_ptrs->data;
    cp.dst_ptrs = dst_ptrs->data;
    cp.src_s = src_ptrs->stride[0];
    cp.dst_s = dst_ptrs->stride[0];
    cp.sizes_s = sizes_s;
    cp.sizes_i64 = sizes_i64;
    cp.tiles = copy_tiles_for(max_size);
    const int64_t grid = n * cp.tiles;
    if (grid > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "too many copies");
    const int e = ssu::launch_batch_memcpy(cp, static_cast<unsigned>(grid), stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

// ---- SSD packed prefill

// Workspace: the state each chunk leaves to the next [nchunks, H, P, N] f32,
// the chain flags [nchunks, H * P / kSsdDim] and the chunk-to-sequence map
// [nchunks] (int32), the 8 ticket counters; each part 256-byte aligned.
struct SsdWorkspace {
    int64_t state, flags, owner, tickets, total;  // byte offsets and the total
};
static SsdWorkspace ssd_ws_parts(int64_t H, int64_t P, int64_t N, int64_t nchunks) {
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t parts = (P + ssu::kSsdDim - 1) / ssu::kSsdDim;  // kSsdDim-wide parts of a head
    SsdWorkspace w;
    w.state = 0;
    w.flags = up(nchunks * H * P * N * 4);
    w.owner = w.flags + up(nchunks * H * parts * 4);
    w.tickets = w.owner + up(nchunks * 4);
    w.total = w.tickets + 256;
    return w;
}

int64_t ssu_ssd_workspace_bytes(int64_t heads, int64_t dim, int64_t dstate, int64_t nchunks) {
    if (heads < 0 || dim < 0 || dstate < 0 || nchunks < 0)
        return -1;
    return ssd_ws_parts(heads, dim, dstate, nchunks).total;
}

// A [rows, a, b] tensor with unit stride on the last axis; returns its row
// and second-axis strides.
static ssu_status_t ssd_rows(const char *name, const ssu_tensor_t &t, int64_t rows, int64_t a, int64_t b,
                             int dtype, bool vec16, int64_t *st, int64_t *s1) {
    if (t.ndim != 3 || t.size[0] != rows || t.size[1] != a || t.size[2] != b)
        return fail(SSU_ERR_VALUE, "%s must be [%lld, %lld, %lld]", name, (long long)rows, (long long)a,
                    (long long)b);
    if (t.dtype != dtype)
        return fail(SSU_ERR_VALUE, "%s must have the x dtype", name);
    if (t.stride[2] != 1 || t.stride[0] < 0 || t.stride[1] < 0)
        return fail(SSU_ERR_VALUE, "%s must have unit stride on its last axis", name);
    if (vec16 && (!aligned(t.data, 16) || t.stride[0] % 8 || t.stride[1] % 8))
        return fail(SSU_ERR_VALUE, "%s rows must start on 16-byte boundaries", name);
    if (!aligned(t.data, 2))
        return fail(SSU_ERR_VALUE, "%s is misaligned", name);
    *st = t.stride[0];
    *s1 = t.stride[1];
    return SSU_OK;
}

static bool contiguous4(const ssu_tensor_t &t) {
    return t.ndim == 4 && t.stride[3] == 1 && t.stride[2] == t.size[3] &&
           t.stride[1] == t.size[2] * t.size[3] && t.stride[0] == t.size[1] * t.size[2] * t.size[3];
}

ssu_status_t ssu_ssd_plan(const ssu_ssd_plan_desc_t *d, ssu_ssd_plan_info_t *info) {
    if (!d)
        return fail(SSU_ERR_VALUE, "ssu_ssd_plan: desc is NULL");
    if (d->heads <= 0 || d->groups <= 0 || d->dim <= 0 || d->dstate <= 0)
        return fail(SSU_ERR_VALUE, "heads, groups, dim and dstate must be positive");
    if (d->heads % d->groups != 0)
        return fail(SSU_ERR_VALUE, "heads (%d) must be divisible by groups (%d)", d->heads, d->groups);
    if (d->io_dtype != SSU_BF16 && d->io_dtype != SSU_F16)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill takes bf16 or f16 x, got %s", dtype_str(d->io_dtype));
    if (!is_float(d->state_dtype))
        return fail(SSU_ERR_VALUE, "state_dtype must be f32, f16 or bf16");
    if (d->dt_dtype != SSU_F32 && d->dt_dtype != d->io_dtype)
        return fail(SSU_ERR_VALUE, "dt_dtype must be f32 or the x dtype");
    if (d->dim % ssu::kSsdDim != 0)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill supports head dims that are multiples of %d, got %d",
                    ssu::kSsdDim, d->dim);
    if (d->dstate != 64 && d->dstate != 128)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill supports dstate 64 or 128, got %d", d->dstate);
    if (d->chunk_size < 1 || d->chunk_size > ssu::kSsdMaxChunk)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "chunk_size must be 1..%d, got %d", ssu::kSsdMaxChunk, d->chunk_size);
    const char *names[2] = {"", ""};
    int vgprs[2] = {0, 0};
    const int e = ssu::ssd_kernel_attributes(d->io_dtype, d->state_dtype, d->dstate, names, vgprs);
    if (e != 0)
        return fail(SSU_ERR_HIP, "loading the SSD kernels failed: %s", ssu::hip_error_string(e));
    if (info) {
        memset(info, 0, sizeof *info);
        info->launches = 2;
        for (int i = 0; i < 2; i++) {
            snprintf(info->kernels[i], sizeof info->kernels[i], "%s", names[i]);
            info->vgprs[i] = vgprs[i];
        }
        info->workspace_bytes_per_chunk = ssu_ssd_workspace_bytes(d->heads, d->dim, d->dstate, 1);
    }
    g_error.clear();
    return SSU_OK;
}

ssu_status_t ssu_ssd_prefill(const ssu_ssd_args_t *a, void *workspace, int64_t workspace_bytes, void *stream) {
    if (!a)
        return fail(SSU_ERR_VALUE, "ssu_ssd_prefill: args is NULL");
    if (a->unsupported & SSU_OPT_SSD_CHECKPOINT)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "checkpoint_token_indices / checkpoint_state_slots / "
                                             "checkpoint_states are not implemented");
    if (a->unsupported & ~static_cast<uint32_t>(SSU_OPT_SSD_CHECKPOINT))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "unknown option bits");
    const ssu_tensor_t &x = a->x;
    if (!present(x) || x.ndim != 3)
        return fail(SSU_ERR_VALUE, "x must be [tokens, heads, dim]");
    if (x.dtype != SSU_BF16 && x.dtype != SSU_F16)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill takes bf16 or f16 x, got %s", dtype_str(x.dtype));
    const int64_t T = x.size[0], H = x.size[1], P = x.size[2];
    if (P <= 0 || P % ssu::kSsdDim != 0)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill supports head dims that are multiples of %d, got %lld",
                    ssu::kSsdDim, (long long)P);
    ssu::SsdParams sp;
    memset(&sp, 0, sizeof sp);
    ssu_status_t s;
    if ((s = ssd_rows("x", x, T, H, P, x.dtype, true, &sp.x_st, &sp.x_sh)) != SSU_OK)
        return s;
    if (!present(a->B) || !present(a->C) || a->B.ndim != 3)
        return fail(SSU_ERR_VALUE, "B and C [tokens, groups, dstate] are required");
    const int64_t G = a->B.size[1], N = a->B.size[2];
    if (G <= 0 || H % G)
        return fail(SSU_ERR_VALUE, "heads (%lld) must be divisible by groups (%lld)", (long long)H, (long long)G);
    if (N != 64 && N != 128)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "SSD prefill supports dstate 64 or 128, got %lld", (long long)N);
    if ((s = ssd_rows("B", a->B, T, G, N, x.dtype, true, &sp.B_st, &sp.B_sg)) != SSU_OK)
        return s;
    if ((s = ssd_rows("C", a->C, T, G, N, x.dtype, true, &sp.C_st, &sp.C_sg)) != SSU_OK)
        return s;
    if (present(a->z) && (s = ssd_rows("z", a->z, T, H, P, x.dtype, true, &sp.z_st, &sp.z_sh)) != SSU_OK)
        return s;
    if (!present(a->out))
        return fail(SSU_ERR_VALUE, "out is required");
    if ((s = ssd_rows("out", a->out, T, H, P, x.dtype, true, &sp.out_st, &sp.out_sh)) != SSU_OK)
        return s;
    const ssu_tensor_t &dt = a->dt;
    if (!present(dt) || dt.ndim != 2 || dt.size[0] != T || dt.size[1] != H || (dt.dtype != SSU_F32 && dt.dtype != x.dtype))
        return fail(SSU_ERR_VALUE, "dt must be [tokens, heads], f32 or the x dtype");
    if (dt.stride[0] < 0 || dt.stride[1] < 0 || !aligned(dt.data, elem_bytes(dt.dtype)))
        return fail(SSU_ERR_VALUE, "dt: bad stride or alignment");
    sp.dt_st = dt.stride[0];
    sp.dt_sh = dt.stride[1];
    if ((s = head_vector("A", a->A, H, true, &sp.A, &sp.A_sh)) != SSU_OK)
        return s;
    if ((s = head_vector("D", a->D, H, false, &sp.D, &sp.D_sh)) != SSU_OK)
        return s;
    if ((s = head_vector("dt_bias", a->dt_bias, H, false, &sp.dt_bias, &sp.bias_sh)) != SSU_OK)
        return s;
    if (a->chunk_size < 1 || a->chunk_size > ssu::kSsdMaxChunk)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "chunk_size must be 1..%d, got %lld", ssu::kSsdMaxChunk,
                    (long long)a->chunk_size);
    if (!(a->dt_limit_lo <= a->dt_limit_hi))
        return fail(SSU_ERR_VALUE, "dt_limit must be (lo, hi) with lo <= hi");
    // chunk metadata
    if (!present(a->cu_chunk_seqlens) || a->cu_chunk_seqlens.ndim != 1 || a->cu_chunk_seqlens.size[0] < 1)
        return fail(SSU_ERR_VALUE, "cu_chunk_seqlens must be 1-D [nchunks + 1]");
    const int64_t nchunks = a->cu_chunk_seqlens.size[0] - 1;
    bool i64 = false;
    if ((s = meta_vector("cu_chunk_seqlens", a->cu_chunk_seqlens, nchunks + 1, &sp.cu_chunk, &sp.cu_chunk_s, &i64)) != SSU_OK)
        return s;
    sp.cu_chunk_i64 = i64;
    if (!present(a->seq_idx))
        return fail(SSU_ERR_VALUE, "seq_idx is required");
    if ((s = meta_vector("seq_idx", a->seq_idx, nchunks, &sp.seq_idx, &sp.seq_idx_s, &i64)) != SSU_OK)
        return s;
    sp.seq_idx_i64 = i64;
    if (!present(a->last_chunk_indices) || a->last_chunk_indices.ndim != 1)
        return fail(SSU_ERR_VALUE, "last_chunk_indices must be 1-D [batch]");
    const int64_t batch = a->last_chunk_indices.size[0];
    if ((s = meta_vector("last_chunk_indices", a->last_chunk_indices, batch, &sp.last_chunk, &sp.last_chunk_s, &i64)) != SSU_OK)
        return s;
    sp.last_chunk_i64 = i64;
    if (present(a->cu_seqlens) && (a->cu_seqlens.ndim != 1 || a->cu_seqlens.size[0] != batch + 1))
        return fail(SSU_ERR_VALUE, "cu_seqlens must be 1-D [batch + 1]");
    // states
    const ssu_tensor_t &st = a->states;
    const int64_t srows = a->return_intermediate_states ? nchunks : batch;
    if (!present(st) || !contiguous4(st) || st.size[0] != srows || st.size[1] != H || st.size[2] != P ||
        st.size[3] != N || !is_float(st.dtype) || !aligned(st.data, 16))
        return fail(SSU_ERR_VALUE, "states must be contiguous [%s, heads, dim, dstate] (f32/f16/bf16)",
                    a->return_intermediate_states ? "nchunks" : "batch");
    if (present(a->initial_states)) {
        const ssu_tensor_t &in = a->initial_states;
        if (!contiguous4(in) || in.size[0] != batch || in.size[1] != H || in.size[2] != P || in.size[3] != N ||
            in.dtype != st.dtype)
            return fail(SSU_ERR_VALUE, "initial_states must be contiguous [batch, heads, dim, dstate] in the states dtype");
        sp.init = in.data;
    }
    if (nchunks == 0 || T == 0 || H == 0)
        return g_error.clear(), SSU_OK;
    const int64_t hsplit = P / ssu::kSsdDim;
    if (nchunks * H * hsplit > INT32_MAX / 8)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "grid too large");
    const SsdWorkspace wp = ssd_ws_parts(H, P, N, nchunks);
    if (!workspace || workspace_bytes < wp.total || !aligned(workspace, 256))
        return fail(SSU_ERR_VALUE, "workspace must be 256-byte aligned with at least %lld bytes", (long long)wp.total);
    char *ws = static_cast<char *>(workspace);
    sp.ws_state = reinterpret_cast<float *>(ws + wp.state);
    sp.ws_flags = reinterpret_cast<int *>(ws + wp.flags);
    sp.ws_owner = reinterpret_cast<int *>(ws + wp.owner);
    sp.ws_tickets = reinterpret_cast<int *>(ws + wp.tickets);
    sp.x = x.data;
    sp.dt = dt.data;
    sp.B = a->B.data;
    sp.C = a->C.data;
    sp.z = a->z.data;
    sp.out = const_cast<void *>(a->out.data);
    sp.states = const_cast<void *>(st.data);
    sp.T = T;
    sp.H = H * hsplit;  // the kernels see heads of dim kSsdDim
    sp.hsplit = static_cast<int32_t>(hsplit);
    sp.N = N;
    sp.nchunks = nchunks;
    sp.batch = batch;
    sp.chunk_size = a->chunk_size;
    sp.hpg = static_cast<int32_t>(H / G * hsplit);
    sp.nhb = (sp.hpg + ssu::kSsdHeads - 1) / ssu::kSsdHeads;        // blocks of heads
    const int64_t nstream = G * sp.nhb;
    sp.streams_per_xcd = static_cast<int32_t>((nstream + 7) / 8);   // streams per virtual XCD
    sp.dt_f32 = dt.dtype == SSU_F32;
    sp.softplus = a->dt_softplus != 0;
    sp.intermediate = a->return_intermediate_states != 0;
    sp.dt_lo = a->dt_limit_lo;
    sp.dt_hi = a->dt_limit_hi;
    const int e = ssu::launch_ssd(sp, x.dtype, st.dtype, stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

ssu_status_t ssu_conv_state_shift(const ssu_conv_shift_args_t *a, void *stream) {
    if (!a)
        return fail(SSU_ERR_VALUE, "ssu_conv_state_shift: args is NULL");
    const ssu_tensor_t &st = a->state;
    if (!present(st) || st.ndim != 3 || !known_dtype(st.dtype))
        return fail(SSU_ERR_VALUE, "state must be a 3-D conv-state pool");
    if (a->layout != SSU_CONV_TOKEN_MAJOR && a->layout != SSU_CONV_DIM_MAJOR)
        return fail(SSU_ERR_VALUE, "layout must be SSU_CONV_TOKEN_MAJOR or SSU_CONV_DIM_MAJOR");
    const int64_t es = elem_bytes(st.dtype);
    if (st.stride[2] != 1 || st.stride[1] != st.size[2] || st.stride[0] != st.size[1] * st.size[2] ||
        !aligned(st.data, 16))
        return fail(SSU_ERR_VALUE, "state must be contiguous and 16-byte aligned");
    ssu::ConvParams cv;
    memset(&cv, 0, sizeof cv);
    const bool dim_major = a->layout == SSU_CONV_DIM_MAJOR;
    cv.state = const_cast<void *>(st.data);
    cv.blocks = st.size[0];
    cv.W = dim_major ? st.size[2] : st.size[1];
    cv.inner = dim_major ? st.size[1] : st.size[2];
    cv.elem = es;
    const int64_t n = present(a->src_block) ? a->src_block.size[0] : -1;
    if (!present(a->src_block) || !present(a->dst_block) || !present(a->bias))
        return fail(SSU_ERR_VALUE, "src_block, dst_block and bias are required");
    bool i64 = false;
    ssu_status_t s;
    if ((s = meta_vector("src_block", a->src_block, n, &cv.src, &cv.src_s, &i64)) != SSU_OK)
        return s;
    cv.src_i64 = i64;
    if ((s = meta_vector("dst_block", a->dst_block, n, &cv.dst, &cv.dst_s, &i64)) != SSU_OK)
        return s;
    cv.dst_i64 = i64;
    if ((s = meta_vector("bias", a->bias, n, &cv.bias, &cv.bias_s, &i64)) != SSU_OK)
        return s;
    cv.bias_i64 = i64;
    if (n == 0 || cv.blocks == 0 || cv.W == 0 || cv.inner == 0)
        return g_error.clear(), SSU_OK;
    // dim-major: a workgroup per 8 rows a lane; token-major: one workgroup a
    // request (it loops over the block's 16 KiB tiles)
    cv.tiles = dim_major ? static_cast<int32_t>(std::min<int64_t>(
                               64, (cv.inner + 8 * ssu::kCopyThreads - 1) / (8 * ssu::kCopyThreads)))
                         : 1;
    const int64_t grid = n * cv.tiles;
    if (grid > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "too many requests");
    const int e = ssu::launch_conv_shift(cv, dim_major, static_cast<unsigned>(grid), stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

const char *ssu_last_error(void) { return g_error.c_str(); }

ssu_status_t ssu_plan(const ssu_plan_desc_t *desc, ssu_plan_info_t *info) {
    if (!desc)
        return fail(SSU_ERR_VALUE, "ssu_plan: desc is NULL");
    if (!is_float(desc->state_dtype))
        return fail(SSU_ERR_VALUE, "state_dtype must be f32, f16 or bf16");
    if (!is_float(desc->io_dtype))
        return fail(SSU_ERR_VALUE, "io_dtype must be f32, f16 or bf16");
    if (desc->dt_dtype != SSU_F32 && desc->dt_dtype != desc->io_dtype)
        return fail(SSU_ERR_VALUE, "dt_dtype must be f32 or the io dtype");
    if (!is_index(desc->slot_dtype) || !is_index(desc->meta_dtype))
        return fail(SSU_ERR_VALUE, "slot_dtype and meta_dtype must be i32 or i64");
    if (desc->heads <= 0 || desc->dim <= 0 || desc->groups <= 0)
        return fail(SSU_ERR_VALUE, "heads, dim and groups must be positive");
    if (desc->heads % desc->groups != 0)
        return fail(SSU_ERR_VALUE, "heads (%d) must be divisible by groups (%d)", desc->heads,
                    desc->groups);
    if (!dstate_supported(desc->dstate))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "dstate %d is not supported (16, 32, 64, 128, 256)",
                    desc->dstate);
    if (desc->dt_dim != 1 && desc->dt_dim != desc->dim)
        return fail(SSU_ERR_VALUE, "dt_dim must be 1 or dim");
    ssu::KernelRef k;
    const bool multi = desc->packed != 0;
    // packed calls with disable_state_update take the output-only variant
    // where one exists (the choice ssu_update makes)
    const bool yonly = multi && desc->disable_state_update &&
                       ssu::find_yonly_kernel(desc->state_dtype, desc->io_dtype, desc->dstate, &k);
    if (!yonly && !ssu::find_kernel(desc->state_dtype, desc->io_dtype, desc->dstate, multi, &k))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "no kernel for this dtype combination");
    int vgprs = 0, sgprs = 0;
    const int e = ssu::kernel_attributes(k, &vgprs, &sgprs);
    if (e != 0)
        return fail(SSU_ERR_HIP, "loading the kernel failed: %s", ssu::hip_error_string(e));
    if (info) {
        const Geometry g = geometry(desc->dim, desc->dstate, desc->state_dtype,
                                    yonly ? k.tile : multi ? ssu::kTileMulti : ssu::kTileOneToken);
        memset(info, 0, sizeof *info);
        if (yonly)
            snprintf(info->kernel, sizeof info->kernel, "ssu_packed_output_only_%s_%s_n%d",
                     dtype_str(desc->state_dtype), dtype_str(desc->io_dtype), desc->dstate);
        else
            ssu::kernel_name(desc->state_dtype, desc->io_dtype, desc->dstate, multi, info->kernel,
                             sizeof info->kernel);
        info->block_threads = g.block;
        info->rows_per_block = g.rows_per_block;
        info->blocks_per_seq_head = g.dim_tiles;
        info->vgprs = vgprs;
        info->sgprs = sgprs;
    }
    g_error.clear();
    return SSU_OK;
}

ssu_status_t ssu_update(const ssu_args_t *a, void *stream) {
    Prepared pr;
    ssu_status_t s = prepare(a, &pr);
    if (s != SSU_OK)
        return s;
    if (pr.empty)
        return g_error.clear(), SSU_OK;
    ssu::KernelRef k;
    // with disable_state_update nothing is stored: the multi-token path's
    // output-only variant where it applies
    const bool yonly = pr.multi && (pr.p.flags & ssu::kDisable) &&
                       ssu::find_yonly_kernel(pr.state_dtype, pr.io, static_cast<int>(pr.N), &k);
    if (!yonly && !ssu::find_kernel(pr.state_dtype, pr.io, static_cast<int>(pr.N), pr.multi, &k))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "no kernel for state %s / io %s / dstate %lld",
                    dtype_str(pr.state_dtype), dtype_str(pr.io), (long long)pr.N);
    ssu::Params p = pr.p;
    Geometry geo = pr.geo;
    int64_t grid = pr.grid;
    if (yonly) {  // the output-only variant's own tile
        geo = geometry(pr.P, pr.N, pr.state_dtype, k.tile);
        p.dim_tiles = geo.dim_tiles;
        p.rows_per_block = geo.rows_per_block;
        grid = pr.nseq * pr.H * geo.dim_tiles;
        if (grid > INT32_MAX)
            return fail(SSU_ERR_NOT_IMPLEMENTED, "grid of %lld workgroups is too large", (long long)grid);
    }
    const int e = ssu::launch(k, p, static_cast<unsigned>(grid), static_cast<unsigned>(geo.block), stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

// Both ReplaySSM entry points: validate, then launch the one-token or the
// speculative kernel.
// lp_bits: the read copy's format for the LP entry points (8 MXFP8, 4 MXFP4).
static ssu_status_t replay_common(const ssu_replay_args_t *ra, bool spec, void *stream,
                                  const ssu_replay_lp_args_t *lpa = nullptr, int lp_bits = 8) {
    const char *fn = lpa ? (lp_bits == 4 ? "ssu_replay_mx4_update" : "ssu_replay_lp_update")
                     : spec ? "ssu_replay_spec_update"
                            : "ssu_replay_update";
    if (!ra)
        return fail(SSU_ERR_VALUE, "%s: args is NULL", fn);
    const ssu_args_t *a = &ra->base;
    if (present(a->dst_state_batch_indices) || present(a->cu_seqlens) ||
        present(a->num_accepted_tokens))
        return fail(SSU_ERR_NOT_IMPLEMENTED,
                    "replay decode takes one slot table and no dst_state_batch_indices, "
                    "cu_seqlens or num_accepted_tokens");
    if (a->x.ndim != (spec ? 4 : 3))
        return fail(SSU_ERR_NOT_IMPLEMENTED, spec ? "speculative replay takes x [batch, T, heads, dim]"
                                                  : "replay decode takes x [batch, heads, dim]");
    // The speculative step names one slot per sequence: its 1-D table is
    // viewed as [batch, T] with a zero step stride for the shared checks.
    ssu_args_t view = *a;
    const ssu_tensor_t &tab = a->state_batch_indices;
    if (spec && present(tab)) {
        if (tab.ndim != 1 || tab.size[0] != a->x.size[0])
            return fail(SSU_ERR_VALUE, "state_batch_indices must be 1-D [batch]");
        view.state_batch_indices.ndim = 2;
        view.state_batch_indices.size[1] = a->x.size[1];
        view.state_batch_indices.stride[1] = 0;
    }
    Prepared pr;
    ssu_status_t s = prepare(&view, &pr);
    if (s != SSU_OK)
        return s;
    if (!spec && pr.rtab_2d)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "replay decode takes a 1-D slot table");

    // buffers: contiguous, shaped after the pool
    const ssu_tensor_t &bx = ra->buf_x, &bdt = ra->buf_dt, &bB = ra->buf_B;
    if (!present(bx) || !present(bdt) || !present(bB))
        return fail(SSU_ERR_VALUE, "buf_x, buf_dt and buf_B are required");
    if (bx.ndim != 4 || bx.size[0] != pr.slots || bx.size[1] < 1 || bx.size[2] != pr.H ||
        bx.size[3] != pr.P)
        return fail(SSU_ERR_VALUE, "buf_x must be [slots, L, heads, dim]");
    const int64_t L = bx.size[1];
    if (bx.dtype != pr.io || bB.dtype != pr.io)
        return fail(SSU_ERR_VALUE, "buf_x and buf_B must have the x dtype");
    if (bB.ndim != 4 || bB.size[0] != pr.slots || bB.size[1] != L || bB.size[2] != pr.G ||
        bB.size[3] != pr.N)
        return fail(SSU_ERR_VALUE, "buf_B must be [slots, L, groups, dstate]");
    if (bdt.dtype != pr.dt_dtype)
        return fail(SSU_ERR_VALUE, "buf_dt must have the dt dtype");
    const bool dt_per_head = bdt.ndim == 3;
    if (dt_per_head ? (bdt.size[0] != pr.slots || bdt.size[1] != L || bdt.size[2] != pr.H)
                    : (bdt.ndim != 4 || bdt.size[0] != pr.slots || bdt.size[1] != L ||
                       bdt.size[2] != pr.H || bdt.size[3] != pr.P))
        return fail(SSU_ERR_VALUE, "buf_dt must be [slots, L, heads, dim] or [slots, L, heads]");
    if (dt_per_head && pr.dt_sp != 0)
        return fail(SSU_ERR_VALUE, "a per-head buf_dt needs dt with one value per head");
    const ssu_tensor_t *bufs[] = {&bx, &bdt, &bB};
    for (const ssu_tensor_t *t : bufs) {
        int64_t want = 1;
        for (int i = t->ndim - 1; i >= 0; i--) {
            if (t->stride[i] != want && t->size[i] != 1)
                return fail(SSU_ERR_VALUE, "replay buffers must be contiguous");
            want *= t->size[i];
        }
    }
    if (!aligned(bx.data, elem_bytes(pr.io)) || !aligned(bdt.data, elem_bytes(pr.dt_dtype)) ||
        !aligned(bB.data, 16))
        return fail(SSU_ERR_VALUE, "replay buffers are misaligned (buf_B needs 16 bytes)");
    const int64_t T = spec ? a->x.size[1] : 1;
    if (spec && T > L)
        return fail(SSU_ERR_VALUE, "T = %lld drafts do not fit a buffer of L = %lld entries",
                    (long long)T, (long long)L);
    ssu::ReplayParams rp;
    memset(&rp, 0, sizeof rp);
    int64_t len_s = 0;
    bool len_i64 = false;
    if (!present(ra->buf_len))
        return fail(SSU_ERR_VALUE, "buf_len is required");
    if ((s = meta_vector("buf_len", ra->buf_len, pr.nseq, &rp.buf_len, &len_s, &len_i64)) !=
        SSU_OK)
        return s;
    if (lpa) {
        // the copy mirrors the pool's [slots, heads, dim, dstate], one byte a
        // value (MXFP8) or two values a byte (MXFP4)
        const char *fmt = lp_bits == 4 ? "MXFP4" : "MXFP8";
        if (pr.state_dtype != SSU_F32)
            return fail(SSU_ERR_NOT_IMPLEMENTED, "the %s read copy needs an f32 checkpoint", fmt);
        if (pr.N % 32 != 0)
            return fail(SSU_ERR_VALUE, "the %s read copy needs dstate a multiple of 32", fmt);
        const ssu_tensor_t &lp = lpa->lp, &lps = lpa->lp_scale;
        if (!present(lp) || !present(lps))
            return fail(SSU_ERR_VALUE, "lp and lp_scale are required");
        if (lp.dtype != SSU_U8 || lps.dtype != SSU_U8)
            return fail(SSU_ERR_VALUE, "lp and lp_scale must be u8");
        const int64_t want_lp[4] = {pr.slots, pr.H, pr.P, lp_bits == 4 ? pr.N / 2 : pr.N};
        const int64_t want_sc[4] = {pr.slots, pr.H, pr.P, pr.N / 32};
        const ssu_tensor_t *ts[2] = {&lp, &lps};
        const int64_t *wants[2] = {want_lp, want_sc};
        for (int i = 0; i < 2; i++) {
            const ssu_tensor_t *t = ts[i];
            if (t->ndim != 4)
                return fail(SSU_ERR_VALUE, "lp and lp_scale must be 4-D");
            int64_t want = 1;
            for (int j = 3; j >= 0; j--) {
                if (t->size[j] != wants[i][j])
                    return fail(SSU_ERR_VALUE, i                ? "lp_scale must be [slots, heads, dim, dstate / 32]"
                                               : lp_bits == 4 ? "lp must be [slots, heads, dim, dstate / 2]"
                                                              : "lp must be [slots, heads, dim, dstate]");
                if (t->stride[j] != want && t->size[j] != 1)
                    return fail(SSU_ERR_VALUE, "lp and lp_scale must be contiguous");
                want *= t->size[j];
            }
        }
        if (!aligned(lp.data, 16) || !aligned(lps.data, 8))
            return fail(SSU_ERR_VALUE, "lp must be 16-byte and lp_scale 8-byte aligned");
        rp.lp = static_cast<uint8_t *>(const_cast<void *>(lp.data));
        rp.lp_scale = static_cast<uint8_t *>(const_cast<void *>(lps.data));
    }
    if (pr.empty)
        return g_error.clear(), SSU_OK;
    // the kernel addresses one slot's buffer entries with 32-bit offsets
    if (L * pr.H * pr.P >= INT32_MAX || L * pr.G * pr.N >= INT32_MAX ||
        pr.nseq * len_s >= INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "buffer per slot or buf_len too large");
    rp.buf_x = const_cast<void *>(bx.data);
    rp.buf_dt = const_cast<void *>(bdt.data);
    rp.buf_B = const_cast<void *>(bB.data);
    rp.L = static_cast<int32_t>(L);
    rp.len_s = static_cast<int32_t>(len_s);
    rp.len_i64 = len_i64;
    rp.dt_per_head = dt_per_head;
    rp.G = static_cast<int32_t>(pr.G);

    ssu::KernelRef k;
    if (lpa ? !ssu::find_replay_lp_kernel(pr.io, static_cast<int>(pr.N), lp_bits, &k)
            : !ssu::find_replay_kernel(pr.state_dtype, pr.io, static_cast<int>(pr.N), spec, &k))
        return fail(SSU_ERR_NOT_IMPLEMENTED, "no replay kernel for state %s / io %s / dstate %lld",
                    dtype_str(pr.state_dtype), dtype_str(pr.io), (long long)pr.N);
    ssu::Params p = pr.p;
    int64_t grid, block;
    if (spec) {
        const Geometry geo = geometry(pr.P, pr.N, pr.state_dtype, ssu::kTileReplay);
        p.dim_tiles = geo.dim_tiles;
        p.rows_per_block = geo.rows_per_block;
        grid = pr.nseq * pr.H * geo.dim_tiles;
        block = geo.block;
    } else {
        // one wave per kReplayRows dim rows of a (sequence, head)
        p.dim_tiles = static_cast<int32_t>((pr.P + ssu::kReplayRows - 1) / ssu::kReplayRows);
        if (pr.nseq <= ssu::kReplayScanMax && rp.L > 1)
            p.flags |= ssu::kFillFirst;
        p.rows_per_block = ssu::kReplayRows;
        const int64_t waves = pr.nseq * pr.H * p.dim_tiles;
        if (waves > INT32_MAX)
            return fail(SSU_ERR_NOT_IMPLEMENTED, "grid too large");
        grid = (waves + ssu::kReplayWaves - 1) / ssu::kReplayWaves;
        block = ssu::kReplayWaves * ssu::kWaveLanes;
    }
    if (grid > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "grid too large");
    if (spec && pr.nseq * T > INT32_MAX)
        return fail(SSU_ERR_NOT_IMPLEMENTED, "batch * T too large");
    int e = ssu::launch_replay(k, p, rp, static_cast<unsigned>(grid), static_cast<unsigned>(block),
                               stream);
    // the speculative step's shared appends run after the step (same stream)
    if (e == 0 && spec)
        e = ssu::launch_replay_spec_append(p, rp, static_cast<int>(elem_bytes(pr.io)),
                                           static_cast<int>(elem_bytes(pr.dt_dtype)),
                                           static_cast<unsigned>(pr.nseq * T), stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

ssu_status_t ssu_replay_update(const ssu_replay_args_t *ra, void *stream) {
    return replay_common(ra, false, stream);
}

ssu_status_t ssu_replay_spec_update(const ssu_replay_args_t *ra, void *stream) {
    return replay_common(ra, true, stream);
}

ssu_status_t ssu_replay_lp_update(const ssu_replay_lp_args_t *la, void *stream) {
    if (!la)
        return fail(SSU_ERR_VALUE, "ssu_replay_lp_update: args is NULL");
    return replay_common(&la->base, false, stream, la, 8);
}

ssu_status_t ssu_replay_mx4_update(const ssu_replay_lp_args_t *la, void *stream) {
    if (!la)
        return fail(SSU_ERR_VALUE, "ssu_replay_mx4_update: args is NULL");
    return replay_common(&la->base, false, stream, la, 4);
}

// a contiguous tensor of `dtype` read as flat; returns its element count or -1
static int64_t flat_count(const ssu_tensor_t &t, int dtype) {
    if (!present(t) || t.dtype != dtype || t.ndim < 1 || t.ndim > 4)
        return -1;
    int64_t want = 1;
    for (int j = t.ndim - 1; j >= 0; j--) {
        if (t.size[j] < 0 || (t.stride[j] != want && t.size[j] != 1))
            return -1;
        want *= t.size[j];
    }
    return want;
}

// MXFP8 (bits 8) or MXFP4 (bits 4) quantization of a flat fp32 tensor.
static ssu_status_t mx_quantize(const char *fn, int bits, const ssu_tensor_t *src,
                                const ssu_tensor_t *codes, const ssu_tensor_t *scales, void *stream) {
    if (!src || !codes || !scales)
        return fail(SSU_ERR_VALUE, "%s: a tensor is NULL", fn);
    const int64_t n = flat_count(*src, SSU_F32);
    if (n < 0)
        return fail(SSU_ERR_VALUE, "src must be a contiguous f32 tensor");
    if (n % 32 != 0)
        return fail(SSU_ERR_VALUE, "src holds %lld values, not a multiple of 32", (long long)n);
    const int64_t ncodes = bits == 4 ? n / 2 : n;
    if (flat_count(*codes, SSU_U8) != ncodes)
        return fail(SSU_ERR_VALUE, "codes must be a contiguous u8 tensor of %lld bytes", (long long)ncodes);
    if (flat_count(*scales, SSU_U8) != n / 32)
        return fail(SSU_ERR_VALUE, "scales must be a contiguous u8 tensor of %lld values",
                    (long long)(n / 32));
    if (n == 0)
        return g_error.clear(), SSU_OK;
    if (!aligned(src->data, 16) || !aligned(codes->data, bits == 4 ? 4 : 8))
        return fail(SSU_ERR_VALUE, bits == 4 ? "src must be 16-byte and codes 4-byte aligned"
                                             : "src must be 16-byte and codes 8-byte aligned");
    const float *sp = static_cast<const float *>(src->data);
    uint8_t *cp = static_cast<uint8_t *>(const_cast<void *>(codes->data));
    uint8_t *scp = static_cast<uint8_t *>(const_cast<void *>(scales->data));
    const int e = bits == 4 ? ssu::launch_mx4_quantize(sp, cp, scp, n / 32, stream)
                            : ssu::launch_mx8_quantize(sp, cp, scp, n / 32, stream);
    if (e != 0)
        return fail(SSU_ERR_HIP, "kernel launch failed: %s", ssu::hip_error_string(e));
    g_error.clear();
    return SSU_OK;
}

ssu_status_t ssu_mx8_quantize(const ssu_tensor_t *src, const ssu_tensor_t *codes,
                              const ssu_tensor_t *scales, void *stream) {
    return mx_quantize("ssu_mx8_quantize", 8, src, codes, scales, stream);
}

ssu_status_t ssu_mx4_quantize(const ssu_tensor_t *src, const ssu_tensor_t *codes,
                              const ssu_tensor_t *scales, void *stream) {
    return mx_quantize("ssu_mx4_quantize", 4, src, codes, scales, stream);
}

}  // extern "C"
