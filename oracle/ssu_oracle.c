/*
 * ssu_oracle.c -- plain, slow CPU reference of the Mamba-2 selective state
 * update (SSU) decode step.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package entry's smoke check
 * and the benchmark's CPU-baseline leg are the only code that loads this
 * library. The GPU library never calls it and shares no source with it: the
 * dtype codes, the half/bfloat16 conversions and every formula below are
 * written here on their own.
 *
 * What it computes (the pages it follows):
 *  - MATE docs, "Mamba / SSU": the table "SSU at a glance" fixes the state
 *    pool [slots, heads, dim, dstate] updated in place through destination
 *    slots; A / D / dt_bias per head in fp32; B / C [rows, groups, dstate] in
 *    the x dtype with heads divisible by groups; the output [rows, heads, dim]
 *    in the x dtype; the slot semantics (flat or 2-D tables, pad_slot_id reads
 *    as a zero state and is never written, disable_state_update leaves the
 *    pool unchanged); variable-length and MTP decode (cu_seqlens splits the
 *    rows, num_accepted_tokens seeds the read slot at count-1 floored at 0,
 *    every token publishes to its own destination entry, defaulting to its
 *    own entry of the read table; empty sequences are skipped). The
 *    "SSU toolchain requirements" list says the recurrence runs in fp32 and
 *    the state is kept in the state dtype.
 *  - ReplaySSM article (lpnh.cn), section "三个瓶颈其实来自同一个动作" (the
 *    three bottlenecks): the Mamba-2 step S_t = a_t * S_{t-1} + D_t * v_t k_t^T
 *    with the readout y_t = S_t q_t. With v = x, k = B, q = C, D_t = dt and
 *    a_t = exp(dt * A[h]), one step on a [dim, dstate] tile is
 *        S[d][n] = S[d][n] * exp(dt'[d] A[h]) + (dt'[d] x[d]) B[n]
 *        y[d]    = sum_n S[d][n] C[n] + D[h] x[d],  times silu(z[d]) if z.
 *
 * Readings taken where the pages leave a step open (each one is listed with
 * its justification in the design notes of the repository):
 *  R1  a 1-D slot table is row-indexed: sequence b, position t names entry
 *      bos(b) + t; a 2-D table is addressed by its strides, b*s0 + t*s1.
 *      Both name the same entries for one sequence, as the MATE page says.
 *  R2  head h uses group h / (heads / groups) (consecutive heads share one).
 *  R3  dt' = softplus(dt + dt_bias): bias first, then softplus; no clamp.
 *  R4  softplus(v) = log1p(exp(v)), and v itself for v > 20.
 *  R5  y is computed from the fp32 updated state; the state carried to the
 *      next token of a sequence is the value stored in the state dtype.
 *  R6  y uses the post-update state, and is (C.S + D x) * silu(z).
 *  R7  16-bit stores and outputs round to nearest even.
 *  R8  without num_accepted_tokens the read position is 0.
 *  R9  a row whose read slot is the pad id is computed from a zero state and
 *      its y is written.
 *  R10 a pad destination skips that store only; the carry goes on.
 *  R11 with no read table the slot is the sequence index for the read and
 *      for every write.
 *  R12 a slot written by one sequence and read or written by another has no
 *      defined result; this oracle refuses such inputs.
 *
 * Precision: every product and sum is rounded to fp32 on its own (the build
 * uses -O2 -ffp-contract=off, no fast-math); the readout sums n in order.
 *
 * Parity pins: every function here is pinned by the CPU test suite against
 * values the mathematics fixes (library conversions, closed forms, invariants
 * and a float64 brute force). The one convention the pages do not fix at all
 * is R2's head-to-group order: the code's implementation of R2 is pinned, the
 * convention itself is parity unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* ---- sequences in parallel
 *
 * Sequences are independent: every function below that loops over them has
 * already refused inputs where two sequences share a slot, so each sequence
 * reads only the input pool and its own inputs and writes only its own
 * slots, buffer entries and output rows. Running them on several threads
 * therefore gives the same bytes as one thread (the CPU suite checks it).
 * The thread count is process-wide, 1 unless set. */
static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_get_threads(void) { return g_threads; }

typedef void (*oracle_seq_fn)(const void *args, int64_t b, void *scratch);
typedef struct {
    const void *args;
    oracle_seq_fn fn;
    int64_t nseq, first, step;
    size_t scratch_bytes;
} oracle_job;

static void *oracle_worker(void *p)
{
    const oracle_job *j = (const oracle_job *)p;
    void *scratch = malloc(j->scratch_bytes ? j->scratch_bytes : 1);
    for (int64_t b = j->first; b < j->nseq; b += j->step)
        j->fn(j->args, b, scratch);
    free(scratch);
    return NULL;
}

/* fn(args, b, scratch) for b = 0..nseq-1, sequence b on thread b mod n */
static void for_each_sequence(const void *args, oracle_seq_fn fn, int64_t nseq, size_t scratch_bytes)
{
    int n = g_threads;
    if (n > nseq)
        n = nseq < 1 ? 1 : (int)nseq;
    oracle_job *jobs = (oracle_job *)malloc((size_t)n * sizeof(oracle_job));
    pthread_t *tid = (pthread_t *)malloc((size_t)n * sizeof(pthread_t));
    int started = 0;
    for (int i = 0; i < n; i++) {
        jobs[i].args = args;
        jobs[i].fn = fn;
        jobs[i].nseq = nseq;
        jobs[i].first = i;
        jobs[i].step = n;
        jobs[i].scratch_bytes = scratch_bytes;
    }
    if (n > 1)
        for (; started < n - 1; started++)
            if (pthread_create(&tid[started], NULL, oracle_worker, &jobs[started + 1]))
                break;
    /* thread 0 is this one; a worker that could not start runs here too */
    oracle_worker(&jobs[0]);
    for (int i = started + 1; i < n; i++)
        oracle_worker(&jobs[i]);
    for (int i = 0; i < started; i++)
        pthread_join(tid[i], NULL);
    free(jobs);
    free(tid);
}

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_ONE_TOKEN = 0, OR_DENSE = 1, OR_CU = 2 };

typedef struct {
    const int64_t *data; /* NULL: no table */
    int64_t len;         /* number of int64 elements data may be indexed at */
    int32_t ndim;        /* 1 (row-indexed, R1) or 2 (strided) */
    int64_t s0, s1;      /* element strides of a 2-D table */
} oracle_table;

typedef struct {
    /* state pool [slots, H, P, N]: read from pool_in, stores go to pool_out
     * (the caller initialises pool_out as a copy of pool_in) */
    const void *pool_in;
    void *pool_out;
    int32_t state_dtype;
    int64_t slots, H, P, N, G;
    /* packed rows */
    int64_t R;
    int32_t io_dtype;   /* dtype of x, B, C, z and out */
    const void *x;      /* [R, H, P] */
    const void *dt;     /* [R, H, P], or [R, H] when dt_per_head */
    int32_t dt_dtype;
    int32_t dt_per_head;
    const float *A;     /* [H] */
    const void *B;      /* [R, G, N] */
    const void *C;      /* [R, G, N] */
    const float *D;     /* [H] or NULL */
    const void *z;      /* [R, H, P] or NULL */
    const float *dt_bias; /* [H] or NULL */
    int32_t dt_softplus;
    /* sequences */
    int32_t layout;     /* OR_ONE_TOKEN, OR_DENSE, OR_CU */
    int64_t steps;      /* OR_DENSE: tokens per sequence */
    const int64_t *cu;  /* OR_CU: [nseq + 1] */
    int64_t nseq;       /* OR_CU: number of sequences */
    const int64_t *acc; /* [nseq] or NULL */
    oracle_table rtab, wtab;
    int64_t pad;
    int32_t disable;
    void *out;          /* [R, H, P] */
    uint8_t *written;   /* [slots] or NULL: set to 1 for every slot stored */
    int64_t *read_slot; /* [nseq] or NULL: resolved read slot (INT64_MIN if empty) */
} oracle_args;

/* ---- scalar formats (IEEE 754 binary16; bfloat16 = top half of binary32) */

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t e = (h >> 10) & 0x1F;
    uint32_t m = h & 0x3FF;
    uint32_t u;
    if (e == 0x1F) {
        u = sign | 0x7F800000u | (m << 13); /* inf / nan, payload kept */
    } else if (e != 0) {
        u = sign | ((e - 15 + 127) << 23) | (m << 13);
    } else if (m == 0) {
        u = sign;
    } else {
        /* subnormal: value m * 2^-24, renormalise */
        int k = 0;
        while (!(m & 0x400)) { m <<= 1; k++; }
        m &= 0x3FF;
        u = sign | ((uint32_t)(127 - 15 + 1 - k) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* round q + rem / 2^shift to nearest, ties to even */
static uint32_t round_shift(uint32_t v, int shift)
{
    uint32_t q = v >> shift;
    uint32_t rem = v & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q++;
    return q;
}

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    int32_t exp = (int32_t)((u >> 23) & 0xFF);
    uint32_t man = u & 0x7FFFFFu;
    if (exp == 0xFF) {
        if (man == 0)
            return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | (man >> 13)); /* quiet nan */
    }
    int32_t e = exp - 127 + 15; /* binary16 biased exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);
    if (e <= 0) {
        /* subnormal result: value / 2^-24 = (man | 1<<23) * 2^(exp - 126) */
        if (exp == 0)
            return (uint16_t)sign; /* fp32 subnormals are far below 2^-25 */
        int shift = 126 - exp;     /* >= 14 */
        if (shift > 24)
            return (uint16_t)sign;
        return (uint16_t)(sign | round_shift(man | 0x800000u, shift));
    }
    /* normal: 10 mantissa bits kept, 13 rounded away; a carry may roll the
     * exponent up, to infinity at the top, which is the right result */
    uint32_t q = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u)))
        q++;
    return (uint16_t)(sign | q);
}

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x40u); /* quiet nan, sign kept */
    return (uint16_t)(round_shift(u, 16) & 0xFFFFu);
}

static float load_as_f32(const void *p, int32_t dtype, int64_t i)
{
    switch (dtype) {
    case OR_F32: return ((const float *)p)[i];
    case OR_F16: return oracle_f16_to_f32(((const uint16_t *)p)[i]);
    default:     return oracle_bf16_to_f32(((const uint16_t *)p)[i]);
    }
}

static void store_from_f32(void *p, int32_t dtype, int64_t i, float v)
{
    switch (dtype) {
    case OR_F32: ((float *)p)[i] = v; break;
    case OR_F16: ((uint16_t *)p)[i] = oracle_f32_to_f16(v); break;
    default:     ((uint16_t *)p)[i] = oracle_f32_to_bf16(v); break;
    }
}

/* value after a store in `dtype` and a load back (R5's carried state) */
static float through_dtype(int32_t dtype, float v)
{
    switch (dtype) {
    case OR_F32: return v;
    case OR_F16: return oracle_f16_to_f32(oracle_f32_to_f16(v));
    default:     return oracle_bf16_to_f32(oracle_f32_to_bf16(v));
    }
}

/* R4 */
float oracle_softplus(float v)
{
    if (v > 20.0f)
        return v;
    return log1pf(expf(v));
}

static float silu(float v) { return v / (1.0f + expf(-v)); }

/* ---- sequences and slots */

static void seq_span(const oracle_args *a, int64_t b, int64_t *bos, int64_t *len)
{
    if (a->layout == OR_ONE_TOKEN) {
        *bos = b;
        *len = 1;
    } else if (a->layout == OR_DENSE) {
        *bos = b * a->steps;
        *len = a->steps;
    } else {
        *bos = a->cu[b];
        *len = a->cu[b + 1] - a->cu[b];
    }
}

static int64_t num_seqs(const oracle_args *a)
{
    if (a->layout == OR_ONE_TOKEN)
        return a->R;
    if (a->layout == OR_DENSE)
        return a->steps > 0 ? a->R / a->steps : 0;
    return a->nseq;
}

static void set_err(char *err, int errlen, const char *msg, long long v1, long long v2)
{
    if (err && errlen > 0)
        snprintf(err, (size_t)errlen, msg, v1, v2);
}

/* resolve sequence b's read slot (R8, R11 and the count-1 floor); returns 0
 * and the slot, or -1 when the entry lies outside the table */
static int read_slot_of(const oracle_args *a, int64_t b, int64_t bos, int64_t *slot)
{
    int64_t pos0 = 0;
    if (a->acc) {
        pos0 = a->acc[b] - 1;
        if (pos0 < 0)
            pos0 = 0;
    }
    if (!a->rtab.data) {
        *slot = b;
        return 0;
    }
    int64_t i = a->rtab.ndim == 1 ? bos + pos0 : b * a->rtab.s0 + pos0 * a->rtab.s1;
    if (i < 0 || i >= a->rtab.len)
        return -1;
    *slot = a->rtab.data[i];
    return 0;
}

/* destination of sequence b's token t: its own entry of the destination
 * table, else of the read table, else the sequence index (R11) */
static int write_slot_of(const oracle_args *a, int64_t b, int64_t bos, int64_t t, int64_t *slot)
{
    const oracle_table *tb = a->wtab.data ? &a->wtab : (a->rtab.data ? &a->rtab : NULL);
    if (!tb) {
        *slot = b;
        return 0;
    }
    int64_t i = tb->ndim == 1 ? bos + t : b * tb->s0 + t * tb->s1;
    if (i < 0 || i >= tb->len)
        return -1;
    *slot = tb->data[i];
    return 0;
}

/* checks the oracle makes so that a result it returns is well defined */
static int check_inputs(const oracle_args *a, char *err, int errlen)
{
    if (a->H <= 0 || a->P <= 0 || a->N <= 0 || a->G <= 0 || a->H % a->G != 0) {
        set_err(err, errlen, "bad heads/groups %lld/%lld", (long long)a->H, (long long)a->G);
        return 1;
    }
    int64_t nseq = num_seqs(a);
    if (a->layout == OR_DENSE && a->steps > 0 && a->R % a->steps != 0) {
        set_err(err, errlen, "rows %lld not a multiple of steps %lld", (long long)a->R,
                (long long)a->steps);
        return 1;
    }
    if (a->layout == OR_CU) {
        if (a->cu[0] != 0 || a->cu[nseq] != a->R) {
            set_err(err, errlen, "cu_seqlens must run from 0 to rows (%lld), ends at %lld",
                    (long long)a->R, (long long)a->cu[nseq]);
            return 1;
        }
        for (int64_t b = 0; b < nseq; b++)
            if (a->cu[b + 1] < a->cu[b]) {
                set_err(err, errlen, "cu_seqlens decreases at %lld%lld", (long long)b, 0);
                return 1;
            }
    }
    int64_t *writer = (int64_t *)malloc((size_t)(a->slots > 0 ? a->slots : 1) * sizeof(int64_t));
    for (int64_t s = 0; s < a->slots; s++)
        writer[s] = -1;
    int rc = 0;
    /* every slot named must be the pad id or inside the pool; a slot written
     * by one sequence must not be read or written by another (R12) */
    for (int64_t b = 0; b < nseq && !rc; b++) {
        int64_t bos, len, s;
        seq_span(a, b, &bos, &len);
        if (len == 0)
            continue;
        if (read_slot_of(a, b, bos, &s)) {
            set_err(err, errlen, "read entry of sequence %lld outside the table%lld", (long long)b, 0);
            rc = 1;
            break;
        }
        if (s != a->pad && (s < 0 || s >= a->slots)) {
            set_err(err, errlen, "read slot %lld of sequence %lld outside the pool", (long long)s,
                    (long long)b);
            rc = 1;
            break;
        }
        if (a->disable)
            continue;
        for (int64_t t = 0; t < len; t++) {
            if (write_slot_of(a, b, bos, t, &s)) {
                set_err(err, errlen, "write entry of sequence %lld token %lld outside the table",
                        (long long)b, (long long)t);
                rc = 1;
                break;
            }
            if (s == a->pad)
                continue;
            if (s < 0 || s >= a->slots) {
                set_err(err, errlen, "write slot %lld of sequence %lld outside the pool",
                        (long long)s, (long long)b);
                rc = 1;
                break;
            }
            if (writer[s] != -1 && writer[s] != b) {
                set_err(err, errlen, "slot %lld written by two sequences (second: %lld)",
                        (long long)s, (long long)b);
                rc = 1;
                break;
            }
            writer[s] = b;
        }
    }
    for (int64_t b = 0; b < nseq && !rc; b++) {
        int64_t bos, len, s;
        seq_span(a, b, &bos, &len);
        if (len == 0)
            continue;
        read_slot_of(a, b, bos, &s);
        if (s != a->pad && writer[s] != -1 && writer[s] != b) {
            set_err(err, errlen, "slot %lld read by sequence %lld and written by another",
                    (long long)s, (long long)b);
            rc = 1;
        }
    }
    free(writer);
    return rc;
}

/* ---- the update */

/* sequence b of the update; S: scratch of P * N floats */
static void ssu_sequence(const void *args, int64_t b, void *scratch)
{
    const oracle_args *a = (const oracle_args *)args;
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G;
    const int64_t heads_per_group = H / G;
    const int64_t tile = P * N;
    float *S = (float *)scratch;
    {
        int64_t bos, len;
        seq_span(a, b, &bos, &len);
        if (a->read_slot)
            a->read_slot[b] = INT64_MIN;
        if (len == 0)
            return; /* empty sequences are skipped */
        int64_t rslot;
        read_slot_of(a, b, bos, &rslot);
        if (a->read_slot)
            a->read_slot[b] = rslot;

        for (int64_t h = 0; h < H; h++) {
            const int64_t g = h / heads_per_group; /* R2 */
            /* the tile this sequence starts from; the pad id reads as zeros */
            for (int64_t e = 0; e < tile; e++)
                S[e] = rslot == a->pad
                           ? 0.0f
                           : load_as_f32(a->pool_in, a->state_dtype, (rslot * H + h) * tile + e);

            for (int64_t t = 0; t < len; t++) {
                const int64_t r = bos + t;
                for (int64_t d = 0; d < P; d++) {
                    const int64_t xi = (r * H + h) * P + d;
                    float v = a->dt_per_head ? load_as_f32(a->dt, a->dt_dtype, r * H + h)
                                             : load_as_f32(a->dt, a->dt_dtype, xi);
                    if (a->dt_bias)
                        v = v + a->dt_bias[h]; /* R3 */
                    if (a->dt_softplus)
                        v = oracle_softplus(v);
                    const float xv = load_as_f32(a->x, a->io_dtype, xi);
                    const float decay = expf(v * a->A[h]);
                    const float dtx = v * xv;
                    float *Sd = S + d * N;
                    for (int64_t n = 0; n < N; n++) {
                        const float bn = load_as_f32(a->B, a->io_dtype, (r * G + g) * N + n);
                        Sd[n] = Sd[n] * decay + dtx * bn;
                    }
                    float y = 0.0f;
                    for (int64_t n = 0; n < N; n++) {
                        const float cn = load_as_f32(a->C, a->io_dtype, (r * G + g) * N + n);
                        y = y + Sd[n] * cn;
                    }
                    if (a->D)
                        y = y + a->D[h] * xv;
                    if (a->z)
                        y = y * silu(load_as_f32(a->z, a->io_dtype, xi)); /* R6 */
                    store_from_f32(a->out, a->io_dtype, xi, y);
                }
                /* R5: carry what the state dtype holds */
                for (int64_t e = 0; e < tile; e++)
                    S[e] = through_dtype(a->state_dtype, S[e]);
                if (a->disable)
                    continue;
                int64_t wslot;
                write_slot_of(a, b, bos, t, &wslot);
                if (wslot == a->pad)
                    continue; /* R10 */
                for (int64_t e = 0; e < tile; e++)
                    store_from_f32(a->pool_out, a->state_dtype, (wslot * H + h) * tile + e, S[e]);
                if (a->written)
                    a->written[wslot] = 1;
            }
        }
    }
}

int oracle_ssu(const oracle_args *a, char *err, int errlen)
{
    if (check_inputs(a, err, errlen))
        return 1;
    for_each_sequence(a, ssu_sequence, num_seqs(a), (size_t)(a->P * a->N) * sizeof(float));
    return 0;
}

/* ---- MXFP8 (E4M3) block format: the low-precision read copy
 *
 * ReplaySSM article, section "数据与边界" (and the low-precision paragraph
 * after it): output-only steps can read a low-precision copy of the
 * checkpoint while the recurrence stays high precision; only the fold reads
 * and writes the high-precision state, and rewrites the copy. The pages use
 * NVFP4 on NVIDIA parts; on this hardware the copy is the OCP Microscaling
 * (MX) v1.0 format MXFP8: blocks of 32 consecutive dstate elements sharing
 * a power-of-two scale (E8M0) with elements in FP8 E4M3 (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; no infinities; 0x7F / 0xFF are NaN;
 * largest magnitude 448; subnormals m x 2^-9).
 *
 * Readings:
 *  R30 block scale exponent = floor(log2(max |x|)) - 8 (8 = the exponent of
 *      E4M3's largest power of two, so the largest element lands in
 *      [256, 512)), clamped to [-126, 127]; a block of zeros gets -126; the
 *      scale byte is exponent + 127;
 *  R31 elements: x / 2^exponent (exact) rounded to nearest, ties to even, in
 *      E4M3; magnitudes above 448 saturate to 448 (the MX rule for FP8
 *      element types); decoding multiplies the E4M3 value by 2^exponent.
 */
float oracle_e4m3_decode(uint8_t b)
{
    const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7)
        return NAN;
    const float mag = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v))
        return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const float a = fabsf(v);
    if (a >= 448.0f)
        return sign | 0x7E; /* R31: saturate */
    if (a < ldexpf(1.0f, -6)) {
        /* subnormal range: multiples of 2^-9 (q = 8 is the smallest normal) */
        const float q = nearbyintf(ldexpf(a, 9));
        return sign | (uint8_t)q;
    }
    int ex;
    frexpf(a, &ex); /* a = f 2^ex, f in [0.5, 1) */
    int e = ex - 1; /* floor(log2 a), -6 .. 8 */
    float q = nearbyintf((ldexpf(a, -e) - 1.0f) * 8.0f); /* 0 .. 8 */
    if (q == 8.0f) {
        q = 0.0f;
        e = e + 1;
    }
    if (e > 8 || (e == 8 && q == 7.0f))
        return sign | 0x7E; /* rounded past 448 */
    return sign | (uint8_t)(((e + 7) << 3) | (int)q);
}

/* one block of 32 values -> 32 codes and the scale byte */
void oracle_mx8_block(const float *x, uint8_t *codes, uint8_t *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++)
        if (fabsf(x[i]) > amax)
            amax = fabsf(x[i]);
    int k = -126;
    if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);
        k = (ex - 1) - 8; /* R30 */
        if (k < -126)
            k = -126;
        if (k > 127)
            k = 127;
    }
    *scale = (uint8_t)(k + 127);
    for (int i = 0; i < 32; i++)
        codes[i] = oracle_e4m3_encode(ldexpf(x[i], -k));
}

float oracle_mx8_value(uint8_t code, uint8_t scale)
{
    return ldexpf(oracle_e4m3_decode(code), (int)scale - 127);
}

/* ---- MXFP4 (E2M1) block format: a 4-bit read copy
 *
 * The same read copy as MXFP8 above with 4-bit elements (the ReplaySSM
 * article measures a 4-bit copy; OCP Microscaling v1.0's MXFP4 is the 4-bit
 * format with power-of-two block scales): blocks of 32 consecutive dstate
 * elements share an E8M0 scale, elements are FP4 E2M1 (1 sign, 2 exponent
 * bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * no infinities, no NaN).
 *
 * Readings:
 *  R33 two elements per byte: element 2i in the low nibble, 2i+1 in the high
 *      nibble; a copy row of dstate values takes dstate / 2 bytes;
 *  R34 block scale exponent = floor(log2(max |x|)) - 2 (2 = the exponent of
 *      E2M1's largest power of two, so the largest element lands in [4, 8)),
 *      clamped to [-126, 127], -126 for a block of zeros (as R30); elements
 *      x / 2^exponent rounded to nearest, ties to the even code, in E2M1;
 *      magnitudes above 6 saturate to 6; a NaN element gets code 0 (E2M1
 *      has no NaN; checkpoints are finite).
 */
float oracle_e2m1_decode(uint8_t nib)
{
    const int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

uint8_t oracle_e2m1_encode(float v)
{
    if (isnan(v))
        return 0; /* R34 */
    const uint8_t sign = signbit(v) ? 8 : 0;
    const float a = fabsf(v);
    if (a >= 6.0f)
        return sign | 7; /* R34: saturate */
    int code;
    if (a < 2.0f) /* 0, 0.5, 1, 1.5, 2: codes 0..4, steps of 0.5 */
        code = (int)nearbyintf(a * 2.0f);
    else if (a < 4.0f) /* 2, 3, 4: codes 4, 5, 6 */
        code = 4 + ((int)nearbyintf(a) - 2);
    else /* 4, 6: codes 6, 7 */
        code = 6 + ((int)nearbyintf(a * 0.5f) - 2);
    return sign | (uint8_t)code;
}

/* one block of 32 values -> 16 bytes of codes and the scale byte */
void oracle_mx4_block(const float *x, uint8_t *codes, uint8_t *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++)
        if (fabsf(x[i]) > amax)
            amax = fabsf(x[i]);
    int k = -126;
    if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);
        k = (ex - 1) - 2; /* R34 */
        if (k < -126)
            k = -126;
        if (k > 127)
            k = 127;
    }
    *scale = (uint8_t)(k + 127);
    for (int i = 0; i < 16; i++)
        codes[i] = (uint8_t)(oracle_e2m1_encode(ldexpf(x[2 * i], -k)) |
                             (oracle_e2m1_encode(ldexpf(x[2 * i + 1], -k)) << 4)); /* R33 */
}

/* element i of a row of codes (R33), times its block scale */
float oracle_mx4_value(const uint8_t *codes, int64_t i, uint8_t scale)
{
    const uint8_t nib = (uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 15);
    return ldexpf(oracle_e2m1_decode(nib), (int)scale - 127);
}

/* ---- ReplaySSM decode: checkpoint plus input buffer
 *
 * ReplaySSM article (lpnh.cn), section "核心做法" (core method) and its
 * minimal pseudocode: the state is kept as a checkpoint plus a buffer of the
 * last steps' inputs. A step appends its inputs (v, Δ, k) = (x, dt, B) to the
 * buffer and computes its output from the checkpoint and the buffer without
 * writing the state; once every L steps a flush folds the buffer into the
 * checkpoint and writes it back. With L = 1 every step is a flush and the step
 * is the plain update ("the kernel degenerates to the baseline").
 *
 * Readings (the pages leave them open):
 *  R16 the buffer holds the raw step inputs (x, dt and B in their own
 *      dtypes); the step that fills it (h + 1 == L, h = entries before the
 *      step) is the flush: the buffered steps and the current one are applied
 *      to the checkpoint one after the other exactly as the plain update
 *      does (state rounded to the state dtype after each), y comes from the
 *      folded state, and the checkpoint is stored;
 *  R17 any other step writes its inputs to entry h of the slot's buffer and
 *      computes, per dim row d, with a_i = exp(dt'_i A[h]) and j, i over the
 *      buffered steps and the current one (index h):
 *        y = (prod_i a_i) (S_ckpt . C) + sum_j dt'_j x_j (prod_{i>j} a_i) (B_j . C)
 *            + D x, times silu(z)
 *      (the unrolled window of the same section; output-only decode);
 *  R18 h is the caller's per-sequence buffer pointer (the article moves a
 *      buffer pointer on commit); the caller resets it after a flush;
 *  R32 with an MXFP8 read copy (R30, R31), an output-only step takes the
 *      checkpoint from the copy (the high-precision pool is not read); a fold
 *      reads and writes the high-precision checkpoint as before and then
 *      rewrites the copy of that slot from the folded state;
 *  R19 one token per sequence, the checkpoint slot is read and written in
 *      place; the pad id reads a zero checkpoint, has no buffer (its pointer
 *      is taken as 0) and writes nothing; disable_state_update writes neither
 *      checkpoint nor buffer.
 */
typedef struct {
    oracle_args base; /* one token per sequence; rtab 1-D or NULL; no wtab */
    int64_t L;
    const void *bx_in;  /* [slots, L, H, P] io dtype */
    void *bx_out;
    const void *bdt_in; /* [slots, L, H, P] (or [slots, L, H] when dt is per head), dt dtype */
    void *bdt_out;
    const void *bB_in;  /* [slots, L, G, N] io dtype */
    void *bB_out;
    const int64_t *buf_len; /* [nseq] entries in each sequence's buffer */
    /* optional MXFP8 read copy of the checkpoint pool (one-token step only):
     * codes [slots, H, P, N], scales [slots, H, P, N / 32] */
    const uint8_t *lp_in, *lps_in;
    uint8_t *lp_out, *lps_out;
    int32_t lp_bits; /* 8: MXFP8 codes [slots, H, P, N]; 4: MXFP4 codes [slots, H, P, N / 2] */
} oracle_replay_args;

/* dt' of one buffered or current step, one dim row */
static float processed_dt(const oracle_args *a, float raw, int64_t h)
{
    float v = raw;
    if (a->dt_bias)
        v = v + a->dt_bias[h];
    if (a->dt_softplus)
        v = oracle_softplus(v);
    return v;
}

static void copy_elem(void *dst, const void *src, int32_t dtype, int64_t di, int64_t si)
{
    if (dtype == OR_F32)
        ((float *)dst)[di] = ((const float *)src)[si];
    else
        ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
}

static void replay_sequence(const void *args, int64_t b, void *scratch);
static void replay_spec_sequence(const void *args, int64_t b, void *scratch);

int oracle_replay(const oracle_replay_args *ra, char *err, int errlen)
{
    const oracle_args *a = &ra->base;
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G, L = ra->L;
    const int64_t tile = P * N;
    if (a->layout != OR_ONE_TOKEN || a->wtab.data || a->acc || L < 1 || H % G) {
        set_err(err, errlen, "replay takes one token per sequence, no destination table, L >= 1%lld%lld", 0, 0);
        return 1;
    }
    if (a->rtab.data && a->rtab.ndim != 1) {
        set_err(err, errlen, "replay takes a 1-D slot table%lld%lld", 0, 0);
        return 1;
    }
    if ((ra->lp_in || ra->lp_out) && N % 32) {
        set_err(err, errlen, "a read copy needs dstate divisible by 32%lld%lld", 0, 0);
        return 1;
    }
    const int64_t nseq = a->R;
    /* slots in range, at most one sequence per slot, 0 <= h < L */
    for (int64_t b = 0; b < nseq; b++) {
        const int64_t s = a->rtab.data ? a->rtab.data[b] : b;
        const int64_t h = ra->buf_len[b];
        if (s != a->pad && (h < 0 || h >= L)) {
            set_err(err, errlen, "buffer length %lld of sequence %lld outside [0, L)", (long long)h, (long long)b);
            return 1;
        }
        if (s == a->pad)
            continue;
        if (s < 0 || s >= a->slots) {
            set_err(err, errlen, "slot %lld of sequence %lld outside the pool", (long long)s, (long long)b);
            return 1;
        }
        for (int64_t b2 = 0; b2 < b; b2++)
            if ((a->rtab.data ? a->rtab.data[b2] : b2) == s) {
                set_err(err, errlen, "slot %lld used by two sequences (second: %lld)", (long long)s, (long long)b);
                return 1;
            }
    }
    for_each_sequence(ra, replay_sequence, nseq, (size_t)(tile + 3 * L) * sizeof(float));
    return 0;
}

/* sequence b of the replay step; scratch: the tile, then alpha, dt' and x
 * of up to L steps */
static void replay_sequence(const void *args, int64_t b, void *scratch)
{
    const oracle_replay_args *ra = (const oracle_replay_args *)args;
    const oracle_args *a = &ra->base;
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G, L = ra->L;
    const int64_t per_group = H / G, tile = P * N;
    const int64_t dtw = a->dt_per_head ? 1 : P; /* dt values per (step, head) */
    float *S = (float *)scratch;
    float *alpha = S + tile;
    float *dtp = alpha + L;
    float *xs = dtp + L;
    {
        const int64_t s = a->rtab.data ? a->rtab.data[b] : b;
        const int pad = s == a->pad;
        const int64_t h = pad ? 0 : ra->buf_len[b]; /* R19 */
        if (a->read_slot)
            a->read_slot[b] = s;
        for (int64_t hd = 0; hd < H; hd++) {
            const int64_t g = hd / per_group;
            /* inputs of step j (j < h buffered, j == h current) */
#define RX(j, d) ((j) < h ? load_as_f32(ra->bx_in, a->io_dtype, ((s * L + (j)) * H + hd) * P + (d)) \
                          : load_as_f32(a->x, a->io_dtype, (b * H + hd) * P + (d)))
#define RDT(j, d) ((j) < h ? load_as_f32(ra->bdt_in, a->dt_dtype, ((s * L + (j)) * H + hd) * dtw + (a->dt_per_head ? 0 : (d))) \
                           : load_as_f32(a->dt, a->dt_dtype, (b * H + hd) * dtw + (a->dt_per_head ? 0 : (d))))
#define RB(j, n) ((j) < h ? load_as_f32(ra->bB_in, a->io_dtype, ((s * L + (j)) * G + g) * N + (n)) \
                          : load_as_f32(a->B, a->io_dtype, (b * G + g) * N + (n)))
            /* R32: an output-only step reads the read copy when there is one */
            const int from_copy = ra->lp_in && h + 1 != L && !pad;
            for (int64_t e = 0; e < tile; e++) {
                const int64_t at = (s * H + hd) * tile + e; /* element of the pool */
                S[e] = pad         ? 0.0f
                       : !from_copy ? load_as_f32(a->pool_in, a->state_dtype, at)
                       : ra->lp_bits == 4 ? oracle_mx4_value(ra->lp_in, at, ra->lps_in[at / 32])
                                          : oracle_mx8_value(ra->lp_in[at], ra->lps_in[at / 32]);
            }
            if (h + 1 == L) {
                /* flush: fold the buffered steps and the current one into the
                 * checkpoint, one plain update after the other */
                for (int64_t j = 0; j <= h; j++) {
                    for (int64_t d = 0; d < P; d++) {
                        const float v = processed_dt(a, RDT(j, d), hd);
                        const float xv = RX(j, d);
                        const float decay = expf(v * a->A[hd]);
                        const float dtx = v * xv;
                        float *Sd = S + d * N;
                        for (int64_t n = 0; n < N; n++)
                            Sd[n] = Sd[n] * decay + dtx * RB(j, n);
                        if (j == h) {
                            float y = 0.0f;
                            for (int64_t n = 0; n < N; n++)
                                y = y + Sd[n] * load_as_f32(a->C, a->io_dtype, (b * G + g) * N + n);
                            if (a->D)
                                y = y + a->D[hd] * xv;
                            if (a->z)
                                y = y * silu(load_as_f32(a->z, a->io_dtype, (b * H + hd) * P + d));
                            store_from_f32(a->out, a->io_dtype, (b * H + hd) * P + d, y);
                        }
                    }
                    for (int64_t e = 0; e < tile; e++)
                        S[e] = through_dtype(a->state_dtype, S[e]);
                }
                if (!pad && !a->disable) {
                    for (int64_t e = 0; e < tile; e++)
                        store_from_f32(a->pool_out, a->state_dtype, (s * H + hd) * tile + e, S[e]);
                    if (a->written)
                        a->written[s] = 1;
                    if (ra->lp_out) /* R32: the fold rewrites the read copy */
                        for (int64_t e = 0; e < tile; e += 32) {
                            const int64_t at = (s * H + hd) * tile + e;
                            if (ra->lp_bits == 4)
                                oracle_mx4_block(S + e, ra->lp_out + at / 2, ra->lps_out + at / 32);
                            else
                                oracle_mx8_block(S + e, ra->lp_out + at, ra->lps_out + at / 32);
                        }
                }
            } else {
                /* output-only: y from the checkpoint and the buffer */
                for (int64_t d = 0; d < P; d++) {
                    for (int64_t j = 0; j <= h; j++) {
                        dtp[j] = processed_dt(a, RDT(j, d), hd);
                        alpha[j] = expf(dtp[j] * a->A[hd]);
                        xs[j] = RX(j, d);
                    }
                    float u = 0.0f; /* S_ckpt . C */
                    for (int64_t n = 0; n < N; n++)
                        u = u + S[d * N + n] * load_as_f32(a->C, a->io_dtype, (b * G + g) * N + n);
                    float gamma = 1.0f;
                    for (int64_t j = 0; j <= h; j++)
                        gamma = gamma * alpha[j];
                    float y = gamma * u;
                    for (int64_t j = 0; j <= h; j++) {
                        float tail = 1.0f; /* prod_{i > j} a_i */
                        for (int64_t i = j + 1; i <= h; i++)
                            tail = tail * alpha[i];
                        float w = 0.0f; /* B_j . C */
                        for (int64_t n = 0; n < N; n++)
                            w = w + RB(j, n) * load_as_f32(a->C, a->io_dtype, (b * G + g) * N + n);
                        y = y + dtp[j] * xs[j] * tail * w;
                    }
                    if (a->D)
                        y = y + a->D[hd] * xs[h];
                    if (a->z)
                        y = y * silu(load_as_f32(a->z, a->io_dtype, (b * H + hd) * P + d));
                    store_from_f32(a->out, a->io_dtype, (b * H + hd) * P + d, y);
                }
                /* append the step's inputs at entry h */
                if (!pad && !a->disable) {
                    for (int64_t d = 0; d < P; d++)
                        copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + h) * H + hd) * P + d,
                                  (b * H + hd) * P + d);
                    for (int64_t d = 0; d < dtw; d++)
                        copy_elem(ra->bdt_out, a->dt, a->dt_dtype, ((s * L + h) * H + hd) * dtw + d,
                                  (b * H + hd) * dtw + d);
                    for (int64_t n = 0; n < N; n++)
                        copy_elem(ra->bB_out, a->B, a->io_dtype, ((s * L + h) * G + g) * N + n,
                                  (b * G + g) * N + n);
                }
            }
#undef RX
#undef RDT
#undef RB
        }
    }
}

/* ---- ReplaySSM speculative step: T draft tokens per sequence
 *
 * ReplaySSM article (lpnh.cn), section "投机解码回滚变成挪指针" (speculative
 * decoding: rollback becomes moving a pointer). The inputs of all T draft
 * tokens are appended to the same buffer and the caller commits the accepted
 * prefix by advancing the buffer pointer; every draft query is evaluated
 * against the same checkpoint and buffer window, the drafts differing only by
 * the causal mask; the fold is triggered one window early, at h + 2T > L
 * instead of the natural h + T > L, so that a step always has T free entries.
 *
 * Readings (the page gives the rule, not the layout of a folding step):
 *  R21 x, dt, z are [batch, T, H, P] (dt [batch, T, H] per head), B and C
 *      [batch, T, G, N]; h = buf_len[b] committed entries, 0 <= h <= L,
 *      1 <= T <= L. If h + 2T > L the step folds first: the h committed
 *      entries are applied to the checkpoint one plain update after the other
 *      (rounded to the state dtype after each) and the checkpoint is stored;
 *      the window then starts empty (w = 0). Otherwise w = h and the
 *      checkpoint is only read;
 *  R22 draft t's output, with the steps k of the window being the w committed
 *      entries followed by drafts 0..t, a_k = exp(dt'_k A[h]) and S the
 *      checkpoint (folded or not):
 *        y_t = (prod_k a_k) (S . C_t) + sum_j dt'_j x_j (prod_{k>j} a_k) (B_j . C_t)
 *              + D x_t, times silu(z_t)
 *      (the unrolled window of "核心做法" with the causal mask);
 *  R23 the drafts' raw inputs are written to entries w .. w+T-1; the caller
 *      then sets the pointer to w + the accepted count. The pad id reads a
 *      zero checkpoint, has no buffer (h taken as 0) and writes nothing;
 *      disable_state_update writes neither checkpoint nor buffer.
 */
int oracle_replay_spec(const oracle_replay_args *ra, char *err, int errlen)
{
    const oracle_args *a = &ra->base;
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G, L = ra->L, T = a->steps;
    const int64_t tile = P * N;
    if (a->layout != OR_DENSE || T < 1 || T > L || a->R % T || a->wtab.data || a->acc || H % G) {
        set_err(err, errlen, "speculative replay takes [batch, T, ...] inputs with 1 <= T <= L%lld%lld", 0, 0);
        return 1;
    }
    if (a->rtab.data && a->rtab.ndim != 1) {
        set_err(err, errlen, "replay takes a 1-D slot table%lld%lld", 0, 0);
        return 1;
    }
    if (ra->lp_in || ra->lp_out) {
        set_err(err, errlen, "the speculative step takes no read copy%lld%lld", 0, 0);
        return 1;
    }
    const int64_t nseq = a->R / T;
    for (int64_t b = 0; b < nseq; b++) {
        const int64_t s = a->rtab.data ? a->rtab.data[b] : b;
        const int64_t h = ra->buf_len[b];
        if (s == a->pad)
            continue;
        if (h < 0 || h > L) {
            set_err(err, errlen, "buffer length %lld of sequence %lld outside [0, L]", (long long)h, (long long)b);
            return 1;
        }
        if (s < 0 || s >= a->slots) {
            set_err(err, errlen, "slot %lld of sequence %lld outside the pool", (long long)s, (long long)b);
            return 1;
        }
        for (int64_t b2 = 0; b2 < b; b2++)
            if ((a->rtab.data ? a->rtab.data[b2] : b2) == s) {
                set_err(err, errlen, "slot %lld used by two sequences (second: %lld)", (long long)s, (long long)b);
                return 1;
            }
    }
    for_each_sequence(ra, replay_spec_sequence, nseq, (size_t)(tile + 3 * (L + T)) * sizeof(float));
    return 0;
}

/* sequence b of the speculative step; scratch: the tile, then alpha, dt'
 * and x of up to L + T steps */
static void replay_spec_sequence(const void *args, int64_t b, void *scratch)
{
    const oracle_replay_args *ra = (const oracle_replay_args *)args;
    const oracle_args *a = &ra->base;
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G, L = ra->L, T = a->steps;
    const int64_t per_group = H / G, tile = P * N;
    const int64_t dtw = a->dt_per_head ? 1 : P;
    float *S = (float *)scratch;
    float *alpha = S + tile;
    float *dtp = alpha + (L + T);
    float *xs = dtp + (L + T);
    {
        const int64_t s = a->rtab.data ? a->rtab.data[b] : b;
        const int pad = s == a->pad;
        const int64_t h = pad ? 0 : ra->buf_len[b]; /* R23 */
        const int fold = h + 2 * T > L;               /* R21: one window early */
        const int64_t w = fold ? 0 : h;
        if (a->read_slot)
            a->read_slot[b] = s;
        for (int64_t hd = 0; hd < H; hd++) {
            const int64_t g = hd / per_group;
            /* buffer entry j of this slot */
#define BX(j, d) load_as_f32(ra->bx_in, a->io_dtype, ((s * L + (j)) * H + hd) * P + (d))
#define BDT(j, d) load_as_f32(ra->bdt_in, a->dt_dtype, ((s * L + (j)) * H + hd) * dtw + (a->dt_per_head ? 0 : (d)))
#define BB(j, n) load_as_f32(ra->bB_in, a->io_dtype, ((s * L + (j)) * G + g) * N + (n))
            /* draft t of this sequence: packed row b*T + t */
#define DX(t, d) load_as_f32(a->x, a->io_dtype, ((b * T + (t)) * H + hd) * P + (d))
#define DDT(t, d) load_as_f32(a->dt, a->dt_dtype, ((b * T + (t)) * H + hd) * dtw + (a->dt_per_head ? 0 : (d)))
#define DB(t, n) load_as_f32(a->B, a->io_dtype, ((b * T + (t)) * G + g) * N + (n))
#define DC(t, n) load_as_f32(a->C, a->io_dtype, ((b * T + (t)) * G + g) * N + (n))
            for (int64_t e = 0; e < tile; e++)
                S[e] = pad ? 0.0f : load_as_f32(a->pool_in, a->state_dtype, (s * H + hd) * tile + e);
            if (fold) {
                /* apply the committed entries to the checkpoint */
                for (int64_t j = 0; j < h; j++) {
                    for (int64_t d = 0; d < P; d++) {
                        const float v = processed_dt(a, BDT(j, d), hd);
                        const float decay = expf(v * a->A[hd]);
                        const float dtx = v * BX(j, d);
                        for (int64_t n = 0; n < N; n++)
                            S[d * N + n] = S[d * N + n] * decay + dtx * BB(j, n);
                    }
                    for (int64_t e = 0; e < tile; e++) /* R21: rounded after each */
                        S[e] = through_dtype(a->state_dtype, S[e]);
                }
                if (!pad && !a->disable) {
                    for (int64_t e = 0; e < tile; e++)
                        store_from_f32(a->pool_out, a->state_dtype, (s * H + hd) * tile + e, S[e]);
                    if (a->written)
                        a->written[s] = 1;
                }
            }
            for (int64_t d = 0; d < P; d++) {
                /* the window: w committed entries, then the T drafts */
                for (int64_t k = 0; k < w + T; k++) {
                    const float raw = k < w ? BDT(k, d) : DDT(k - w, d);
                    dtp[k] = processed_dt(a, raw, hd);
                    alpha[k] = expf(dtp[k] * a->A[hd]);
                    xs[k] = k < w ? BX(k, d) : DX(k - w, d);
                }
                for (int64_t t = 0; t < T; t++) {
                    const int64_t last = w + t; /* draft t's place in the window */
                    float u = 0.0f;             /* S . C_t */
                    for (int64_t n = 0; n < N; n++)
                        u = u + S[d * N + n] * DC(t, n);
                    float gamma = 1.0f;
                    for (int64_t k = 0; k <= last; k++)
                        gamma = gamma * alpha[k];
                    float y = gamma * u;
                    for (int64_t j = 0; j <= last; j++) {
                        float tail = 1.0f; /* prod_{j < k <= last} a_k */
                        for (int64_t k = j + 1; k <= last; k++)
                            tail = tail * alpha[k];
                        float wj = 0.0f; /* B_j . C_t */
                        for (int64_t n = 0; n < N; n++)
                            wj = wj + (j < w ? BB(j, n) : DB(j - w, n)) * DC(t, n);
                        y = y + dtp[j] * xs[j] * tail * wj;
                    }
                    if (a->D)
                        y = y + a->D[hd] * xs[last];
                    if (a->z)
                        y = y * silu(load_as_f32(a->z, a->io_dtype, ((b * T + t) * H + hd) * P + d));
                    store_from_f32(a->out, a->io_dtype, ((b * T + t) * H + hd) * P + d, y);
                }
            }
            /* append the drafts at entries w .. w+T-1 */
            if (!pad && !a->disable) {
                for (int64_t t = 0; t < T; t++) {
                    for (int64_t d = 0; d < P; d++)
                        copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + w + t) * H + hd) * P + d,
                                  ((b * T + t) * H + hd) * P + d);
                    for (int64_t d = 0; d < dtw; d++)
                        copy_elem(ra->bdt_out, a->dt, a->dt_dtype, ((s * L + w + t) * H + hd) * dtw + d,
                                  ((b * T + t) * H + hd) * dtw + d);
                    for (int64_t n = 0; n < N; n++)
                        copy_elem(ra->bB_out, a->B, a->io_dtype, ((s * L + w + t) * G + g) * N + n,
                                  ((b * T + t) * G + g) * N + n);
                }
            }
#undef BX
#undef BDT
#undef BB
#undef DX
#undef DDT
#undef DB
#undef DC
        }
    }
}

/* ---- memmove-safe Mamba state copies
 *
 * vLLM PR #50729 digest (prhub), sections "实现拆解" (implementation) and
 * "关键源码片段" (key source excerpts): speculative decoding shifts a sequence's
 * convolution state left inside one physical block, so a parallel copy whose
 * source and destination ranges overlap must still behave like memmove; the
 * generic batched copy needs the same guarantee whenever a destination starts
 * below its source inside the copied range.
 *
 * Readings:
 *  R24 batched copy: copy i moves sizes[i] bytes from src_off[i] to
 *      dst_off[i] (byte offsets into one buffer here; device addresses on the
 *      GPU) with memmove semantics in both directions (the page's fix covers a
 *      destination below its source; a destination above it is the mirror
 *      case). Two different copies may not touch the same bytes (that would
 *      make the result depend on their order): this oracle refuses it.
 *  R25 convolution-state shift: a pool of blocks, each conv_width tokens of
 *      `inner` elements of elem_size bytes, token-major ([blocks, W, inner],
 *      "SD") or dim-major ([blocks, inner, W], "DS"). Request r writes
 *      state[dst][:W - bias] = state[src][bias:] (the page's
 *      state[bt[src_col], token_bias:] -> state[bt[dst_col], :conv_width -
 *      token_bias]) and leaves the rest of the destination block alone; bias
 *      in [0, W]. Two requests may not write the same block or write a block
 *      another reads (refused here). A request whose block ids or bias are out
 *      of range writes nothing (the GPU library checks them on the device).
 */
int oracle_batch_memmove(uint8_t *buf, int64_t buf_len, const int64_t *src_off,
                         const int64_t *dst_off, const int64_t *sizes, int64_t n,
                         char *err, int errlen)
{
    for (int64_t i = 0; i < n; i++) {
        if (sizes[i] < 0 || src_off[i] < 0 || dst_off[i] < 0 || src_off[i] + sizes[i] > buf_len ||
            dst_off[i] + sizes[i] > buf_len) {
            set_err(err, errlen, "copy %lld outside the buffer (size %lld)", (long long)i, (long long)sizes[i]);
            return 1;
        }
        for (int64_t j = 0; j < i; j++) {
            /* copy i's bytes (source or destination) against copy j's */
            const int64_t ai[2] = {src_off[i], dst_off[i]}, aj[2] = {src_off[j], dst_off[j]};
            for (int u = 0; u < 2; u++)
                for (int v = 0; v < 2; v++) {
                    if (u == 0 && v == 0)
                        continue; /* two reads of the same bytes are fine */
                    if (ai[u] < aj[v] + sizes[j] && aj[v] < ai[u] + sizes[i] && sizes[i] && sizes[j]) {
                        set_err(err, errlen, "copies %lld and %lld touch the same bytes", (long long)j, (long long)i);
                        return 1;
                    }
                }
        }
    }
    for (int64_t i = 0; i < n; i++)
        memmove(buf + dst_off[i], buf + src_off[i], (size_t)sizes[i]); /* R24 */
    return 0;
}

enum { OR_CONV_SD = 0, OR_CONV_DS = 1 };

int oracle_conv_shift(uint8_t *pool, int64_t blocks, int32_t layout, int64_t W, int64_t inner,
                      int64_t elem_size, const int64_t *src_blk, const int64_t *dst_blk,
                      const int64_t *bias, int64_t n, char *err, int errlen)
{
    const int64_t block_bytes = W * inner * elem_size;
    for (int64_t r = 0; r < n; r++)
        for (int64_t q = 0; q < r; q++) {
            const int ok_r = src_blk[r] >= 0 && src_blk[r] < blocks && dst_blk[r] >= 0 &&
                             dst_blk[r] < blocks && bias[r] >= 0 && bias[r] <= W;
            const int ok_q = src_blk[q] >= 0 && src_blk[q] < blocks && dst_blk[q] >= 0 &&
                             dst_blk[q] < blocks && bias[q] >= 0 && bias[q] <= W;
            if (ok_r && ok_q && (dst_blk[r] == dst_blk[q] || dst_blk[r] == src_blk[q] ||
                                 src_blk[r] == dst_blk[q])) {
                set_err(err, errlen, "requests %lld and %lld share a written block", (long long)q, (long long)r);
                return 1;
            }
        }
    for (int64_t r = 0; r < n; r++) {
        if (src_blk[r] < 0 || src_blk[r] >= blocks || dst_blk[r] < 0 || dst_blk[r] >= blocks ||
            bias[r] < 0 || bias[r] > W)
            continue; /* R25: out of range, nothing written */
        uint8_t *src = pool + src_blk[r] * block_bytes;
        uint8_t *dst = pool + dst_blk[r] * block_bytes;
        const int64_t keep = W - bias[r]; /* tokens moved */
        if (layout == OR_CONV_SD) {
            /* tokens bias..W-1 of the source become tokens 0..W-bias-1 */
            memmove(dst, src + bias[r] * inner * elem_size, (size_t)(keep * inner * elem_size));
        } else {
            /* each of the inner rows shifts left by bias tokens */
            for (int64_t d = 0; d < inner; d++)
                memmove(dst + d * W * elem_size, src + (d * W + bias[r]) * elem_size,
                        (size_t)(keep * elem_size));
        }
    }
    return 0;
}

/* ---- SSD packed variable-length prefill
 *
 * MATE docs, "Mamba / SSU", section "SSD packed prefill" and the API entry of
 * ssd_combined_fwd_varlen: one packed call over a variable-length batch runs
 * the same recurrence as the decode step over every token of every sequence
 * (the five SSD stages are a chunked way to compute it), with x [tokens,
 * heads, dim], one dt per (token, head), dt' = softplus(dt + dt_bias) (or
 * dt + dt_bias) clamped to dt_limit = (lo, hi) (default (0, inf): floored at
 * zero), optional initial states, D and z; it returns the state after each
 * sequence's last chunk, or after every chunk.
 *
 * Readings:
 *  R26 the oracle is the recurrence itself, token by token in chunk order:
 *      S = S * exp(dt' A[h]) + (dt' x) B^T, y = S . C + D x, times silu(z);
 *      the state is carried in fp32 and rounded to the state dtype only where
 *      it is returned;
 *  R27 chunk c covers tokens cu_chunk_seqlens[c] .. cu_chunk_seqlens[c+1]-1
 *      (the only authority for that mapping); chunk c opens a sequence when
 *      c = 0 or seq_idx[c] != seq_idx[c-1], and then starts from
 *      initial_states[seq_idx[c]] (or zeros); any other chunk continues from
 *      the previous chunk's state;
 *  R28 the state recorded for chunk c is the state after its last token; the
 *      returned states are those of chunks last_chunk_indices[b] (or all
 *      chunks when intermediate states are asked for);
 *  R29 D is one value per head; z gates after D, as in the decode step.
 */
typedef struct {
    int64_t T, H, P, N, G, nchunks, batch, chunk_size;
    int32_t io_dtype, dt_dtype, state_dtype;
    const void *x;            /* [T, H, P] io dtype */
    const void *dt;           /* [T, H] dt dtype */
    const float *A;           /* [H] */
    const void *B, *C;        /* [T, G, N] io dtype */
    const float *D;           /* [H] or NULL */
    const void *z;            /* [T, H, P] or NULL */
    const float *dt_bias;     /* [H] or NULL */
    int32_t dt_softplus;
    float dt_lo, dt_hi;
    const int64_t *cu_chunk;  /* [nchunks + 1] */
    const int64_t *seq_idx;   /* [nchunks] */
    const void *init;         /* [batch, H, P, N] state dtype, or NULL */
    void *out;                /* [T, H, P] io dtype */
    void *chunk_states;       /* [nchunks, H, P, N] state dtype */
} oracle_ssd_args;

int oracle_ssd(const oracle_ssd_args *a, char *err, int errlen)
{
    const int64_t H = a->H, P = a->P, N = a->N, G = a->G, tile = P * N;
    if (G <= 0 || H % G || a->nchunks < 0 || a->chunk_size < 1) {
        set_err(err, errlen, "bad shape%lld%lld", 0, 0);
        return 1;
    }
    if (a->nchunks > 0 && (a->cu_chunk[0] != 0 || a->cu_chunk[a->nchunks] != a->T)) {
        set_err(err, errlen, "cu_chunk_seqlens must run from 0 to the token count (%lld)%lld", (long long)a->T, 0);
        return 1;
    }
    for (int64_t c = 0; c < a->nchunks; c++) {
        const int64_t len = a->cu_chunk[c + 1] - a->cu_chunk[c];
        if (len < 0 || len > a->chunk_size) {
            set_err(err, errlen, "chunk %lld has %lld tokens", (long long)c, (long long)len);
            return 1;
        }
        if (a->seq_idx[c] < 0 || a->seq_idx[c] >= a->batch) {
            set_err(err, errlen, "seq_idx[%lld] = %lld outside the batch", (long long)c, (long long)a->seq_idx[c]);
            return 1;
        }
    }
    const int64_t per_group = H / G;
    float *S = (float *)malloc((size_t)(H * tile) * sizeof(float));
    for (int64_t c = 0; c < a->nchunks; c++) {
        const int opens = c == 0 || a->seq_idx[c] != a->seq_idx[c - 1]; /* R27 */
        for (int64_t h = 0; h < H; h++) {
            float *Sh = S + h * tile;
            const int64_t g = h / per_group;
            if (opens)
                for (int64_t e = 0; e < tile; e++)
                    Sh[e] = a->init ? load_as_f32(a->init, a->state_dtype, (a->seq_idx[c] * H + h) * tile + e) : 0.0f;
            for (int64_t t = a->cu_chunk[c]; t < a->cu_chunk[c + 1]; t++) {
                float v = load_as_f32(a->dt, a->dt_dtype, t * H + h);
                if (a->dt_bias)
                    v = v + a->dt_bias[h];
                if (a->dt_softplus)
                    v = oracle_softplus(v);
                if (v < a->dt_lo) /* dt_limit, after softplus */
                    v = a->dt_lo;
                if (v > a->dt_hi)
                    v = a->dt_hi;
                const float decay = expf(a->A[h] * v); /* R26 */
                for (int64_t d = 0; d < P; d++) {
                    const float xv = load_as_f32(a->x, a->io_dtype, (t * H + h) * P + d);
                    const float dtx = v * xv;
                    float y = 0.0f;
                    for (int64_t n = 0; n < N; n++) {
                        float *s = Sh + d * N + n;
                        *s = *s * decay + dtx * load_as_f32(a->B, a->io_dtype, (t * G + g) * N + n);
                        y = y + *s * load_as_f32(a->C, a->io_dtype, (t * G + g) * N + n);
                    }
                    if (a->D) /* R29 */
                        y = y + xv * a->D[h];
                    if (a->z)
                        y = y * silu(load_as_f32(a->z, a->io_dtype, (t * H + h) * P + d));
                    store_from_f32(a->out, a->io_dtype, (t * H + h) * P + d, y);
                }
            }
            for (int64_t e = 0; e < tile; e++) /* R28 */
                store_from_f32(a->chunk_states, a->state_dtype, (c * H + h) * tile + e, Sh[e]);
        }
    }
    free(S);
    return 0;
}

/* bulk MXFP8: nblocks consecutive blocks of 32 values */
void oracle_mx8_quantize(const float *x, int64_t nblocks, uint8_t *codes, uint8_t *scales)
{
    for (int64_t b = 0; b < nblocks; b++)
        oracle_mx8_block(x + 32 * b, codes + 32 * b, scales + b);
}

void oracle_mx4_quantize(const float *x, int64_t nblocks, uint8_t *codes, uint8_t *scales)
{
    for (int64_t b = 0; b < nblocks; b++)
        oracle_mx4_block(x + 32 * b, codes + 16 * b, scales + b);
}

void oracle_mx4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t nblocks, float *x)
{
    for (int64_t i = 0; i < nblocks * 32; i++)
        x[i] = oracle_mx4_value(codes, i, scales[i / 32]);
}

void oracle_mx8_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t nblocks, float *x)
{
    for (int64_t i = 0; i < 32 * nblocks; i++)
        x[i] = oracle_mx8_value(codes[i], scales[i / 32]);
}
