// SSD packed variable-length prefill for gfx950 (MATE docs, "Mamba / SSU",
// section "SSD packed prefill"): the same recurrence as the decode step over
// every token of a packed batch, computed chunk by chunk. Three launches:
//   ssd_chunk_state_kernel   per (chunk, group, 8 heads): dt' (softplus,
//                            dt_limit), the decay cumsum, and the chunk's own
//                            state sum_t exp(A_end - A_t) dt'_t x_t B_t^T (MFMA);
//   ssd_state_pass_kernel    per (head, state slice): walks the chunks in
//                            order, resetting where seq_idx opens a sequence;
//                            writes each chunk's entering state (in the x
//                            dtype) to the workspace and the returned states;
//   ssd_chunk_scan_kernel    per (chunk, group, 4 heads): y_t = sum_{s<=t}
//                            (C_t . B_s) exp(A_t - A_s) dt'_s x_s
//                            + exp(A_t) C_t . S_in + D x_t, gated by
//                            silu(z_t) (MFMA).
// MFMA operands are bf16 / f16 (the x dtype): 16x16x32 tiles with fp32
// accumulation; the scaled operands (w_t x_t, the scaled C.B^T, the entering
// state) are rounded to the x dtype before they enter a product. Every
// kernel works on heads of dim 64; wider heads (a multiple of 64) are split
// into several of those (head_off).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename IT> struct Mfma;
template <> struct Mfma<__bf16> {
    using V = bf16x8;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    using V = f16x8;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kP = kSsdDim;        // head dim
constexpr int kL = kSsdMaxChunk;   // largest chunk
constexpr int kPad = 8;            // LDS row padding (elements)

__device__ __forceinline__ float exp_f(float v) { return __builtin_amdgcn_exp2f(v * 1.44269504088896341f); }

__device__ __forceinline__ float softplus_f(float v) {
    const float u = exp_f(v);
    const float w = 1.0f + u;
    const float l = __builtin_amdgcn_logf(w) * 0.693147180559945309f;
    const float r = w == 1.0f ? u : l * (u * __builtin_amdgcn_rcpf(w - 1.0f));
    return v > 20.0f ? v : r;
}

__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + exp_f(-z)); }

template <typename T>
__device__ __forceinline__ float to_f(T v) { return static_cast<float>(v); }

__device__ __forceinline__ int64_t idx_at(const void *base, bool i64, int64_t i) {
    return i64 ? static_cast<const int64_t *>(base)[i] : static_cast<int64_t>(static_cast<const int32_t *>(base)[i]);
}

// A head of dim kP * hsplit runs as hsplit heads of dim kP ("virtual"
// heads, numbered hsplit * head + part): each part is dims part * kP .. of
// the head's rows of x, z and out, and takes the head's dt, A, D, dt_bias
// (the recurrence never mixes dim rows); the contiguous state and workspace
// layouts [.., heads, dim, dstate] are the same memory as [.., virtual
// heads, kP, dstate]. Element offset of virtual head v in a row of x, z or out:
__device__ __forceinline__ int64_t head_off(const SsdParams &sp, int v, int64_t head_stride) {
    return static_cast<int64_t>(v / sp.hsplit) * head_stride + static_cast<int64_t>(v % sp.hsplit) * kP;
}

// Token range of chunk c; an inconsistent entry (outside the tokens, or
// longer than the chunk size) makes the chunk empty.
__device__ __forceinline__ void chunk_range(const SsdParams &sp, int64_t c, int64_t *t0, int *len) {
    const int64_t a = idx_at(sp.cu_chunk, sp.cu_chunk_i64, c * sp.cu_chunk_s);
    const int64_t b = idx_at(sp.cu_chunk, sp.cu_chunk_i64, (c + 1) * sp.cu_chunk_s);
    const bool ok = a >= 0 && b >= a && b <= sp.T && b - a <= sp.chunk_size;
    *t0 = ok ? a : 0;
    *len = ok ? static_cast<int>(b - a) : 0;
}

// dt' of token t, head h: softplus(dt + dt_bias) (or dt + dt_bias), then the
// dt_limit clamp; the load and the arithmetic apart, so that the load can be
// issued early
// (the raw bits: converted at use, so that no wait follows the load)
template <typename IT>
__device__ __forceinline__ uint32_t raw_dt(const SsdParams &sp, int64_t t, int h) {
    const int64_t i = t * sp.dt_st + static_cast<int64_t>(h) * sp.dt_sh;
    return sp.dt_f32 ? static_cast<const uint32_t *>(sp.dt)[i] : static_cast<const uint16_t *>(sp.dt)[i];
}
template <typename IT>
__device__ __forceinline__ float dt_value(const SsdParams &sp, uint32_t bits) {
    return sp.dt_f32 ? __builtin_bit_cast(float, bits)
                     : to_f(__builtin_bit_cast(IT, static_cast<uint16_t>(bits)));
}
// bias: dt_bias of the head, 0 without one
__device__ __forceinline__ float processed_dt(const SsdParams &sp, float v, float bias) {
    v += bias;
    if (sp.softplus)
        v = softplus_f(v);
    v = v < sp.dt_lo ? sp.dt_lo : v;
    return v > sp.dt_hi ? sp.dt_hi : v;
}

// Inclusive prefix sum over a wave's 64 lanes (log-step shuffles)
__device__ __forceinline__ float wave_inclusive_sum(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(v, off, 64);
        v += lane >= off ? u : 0.0f;
    }
    return v;
}

// Workgroup ids go to the 8 XCDs round robin; consecutive logical ids in
// groups of 16 are placed on one XCD, so the workgroups of one (chunk, group)
// read that chunk's B (and C) through one L2.
__device__ __forceinline__ int32_t xcd_grouped(int32_t id, int32_t n) {
    constexpr int32_t kXcd = 8, K = 16, block = kXcd * K;
    const int32_t m = id / block;
    if ((m + 1) * block > n)
        return id;
    const int32_t r = id % block;
    return m * block + (r % kXcd) * K + r / kXcd;
}

// ---- stage 1: dt', the decay cumsum, and the chunk's own state
//
// One workgroup per (chunk, group, block of kStateHeads heads of the group),
// 512 lanes in two halves of 256 (lane t % 256 = token of the chunk; each
// half stages half of the token's x and B rows): B^T is staged in LDS once
// for the heads, and the heads' dt' and cumsums (wave scans plus the wave
// totals through LDS) are formed together behind one barrier; then per head
// (w x)^T with w_t = exp(A_end - A_t) dt'_t goes to one of two LDS buffers
// and the chunk's own state [64 x N] = sum_t (w_t x_t) B_t^T is formed as
// MFMA tiles (wave w: p tile w / 2, half of the n tiles): one barrier per
// head. The next head's x rows are requested during the current head's
// products.

constexpr int kStateHeads = 8;
constexpr int kStateThreads = 512;  // two halves of 256 lanes, lane t % 256 = token

template <typename IT, int N>
__global__ __launch_bounds__(kStateThreads) void ssd_chunk_state_kernel(const SsdParams sp) {
    using M = Mfma<IT>;
    using V = typename M::V;
    constexpr int kHalfP = kP / 2, kHalfN = N / 2;  // each half stages half of a token's x and B rows
    __shared__ float wave_tot[kStateHeads][kL / 64];
    __shared__ __attribute__((aligned(16))) IT Xs[2][kP][kL + kPad];  // (w x)^T: [p][t], two heads in turn
    __shared__ __attribute__((aligned(16))) IT Bs[N][kL + kPad];      // B^T: [n][t]

    const int ngroups = static_cast<int>(sp.H / sp.hpg);
    const int nhb = (sp.hpg + kStateHeads - 1) / kStateHeads;
    const int32_t wg = xcd_grouped(blockIdx.x, gridDim.x);  // a (chunk, group)'s workgroups share an L2
    const int64_t c = wg / (ngroups * nhb);
    const int g = (wg / nhb) % ngroups;
    const int hb = wg % nhb;
    const int h0 = g * sp.hpg + hb * kStateHeads;
    const int nh = sp.hpg - hb * kStateHeads < kStateHeads ? sp.hpg - hb * kStateHeads : kStateHeads;
    const int t = threadIdx.x;
    const int tk = t & (kL - 1), half = t / kL;  // token in the chunk, which half of its rows
    const int lane = t & 63, wv = t >> 6, wq = wv & 3;  // wq: the wave within its half
    int64_t t0;
    int len;
    chunk_range(sp, c, &t0, &len);
    // lanes past the chunk read token 0 (always present) and contribute zeros
    const int64_t tok = tk < len ? t0 + tk : 0;

    auto load_x = [&](int h, V (&xv)[kHalfP / 8]) {
        const IT *xrow = static_cast<const IT *>(sp.x) + (tok * sp.x_st + head_off(sp, h, sp.x_sh)) + half * kHalfP;
#pragma unroll
        for (int p0 = 0; p0 < kHalfP / 8; p0++)
            xv[p0] = *reinterpret_cast<const V *>(xrow + 8 * p0);
    };
    // loads in the order they are waited on: the heads' A, dt_bias and dt,
    // then B, then the first head's x row
    float Ah[kStateHeads], biash[kStateHeads];
    uint32_t dtr[kStateHeads];
#pragma unroll
    for (int hk = 0; hk < kStateHeads; hk++) {
        const int h = hk < nh ? h0 + hk : h0;
        Ah[hk] = sp.A[(h / sp.hsplit) * sp.A_sh];
        biash[hk] = sp.dt_bias ? sp.dt_bias[(h / sp.hsplit) * sp.bias_sh] : 0.0f;
        dtr[hk] = raw_dt<IT>(sp, tok, h / sp.hsplit);
    }
    V bv[kHalfN / 8];
    {
        const IT *brow = static_cast<const IT *>(sp.B) + (tok * sp.B_st + g * sp.B_sg) + half * kHalfN;
#pragma unroll
        for (int n0 = 0; n0 < kHalfN / 8; n0++)
            bv[n0] = *reinterpret_cast<const V *>(brow + 8 * n0);
    }
    V xv[kHalfP / 8];
    load_x(h0, xv);
#pragma unroll
    for (int n0 = 0; n0 < kHalfN / 8; n0++)
#pragma unroll
        for (int k = 0; k < 8; k++)
            Bs[half * kHalfN + 8 * n0 + k][tk] = tk < len ? bv[n0][k] : static_cast<IT>(0.0f);

    // every head's dt' and inclusive prefix sum of dt' A over the chunk:
    // within each wave, then the wave totals through LDS (both halves compute
    // the same sums; the first half publishes them), one barrier for all heads
    float dtp[kStateHeads], acum[kStateHeads];
#pragma unroll
    for (int hk = 0; hk < kStateHeads; hk++) {
        dtp[hk] = tk < len ? processed_dt(sp, dt_value<IT>(sp, dtr[hk]), biash[hk]) : 0.0f;
        acum[hk] = wave_inclusive_sum(dtp[hk] * Ah[hk], lane);
        if (lane == 63 && half == 0)
            wave_tot[hk][wq] = acum[hk];
    }
    __syncthreads();  // the wave totals, B^T
    float w[kStateHeads];
#pragma unroll
    for (int hk = 0; hk < kStateHeads; hk++) {
        // the chunk's total, summed in the order of the last lane's cumsum
        // (padding adds nothing)
        float total = wave_tot[hk][kL / 64 - 1];
#pragma unroll
        for (int k = 0; k < kL / 64; k++) {
            const float wt = wave_tot[hk][k];
            acum[hk] += k < wq ? wt : 0.0f;
            total += k < kL / 64 - 1 ? wt : 0.0f;
        }
        if (half == 0 && hk < nh) {
            const int64_t wrow = (c * sp.H + h0 + hk) * kL;
            sp.ws_dtp[wrow + tk] = dtp[hk];
            sp.ws_acum[wrow + tk] = acum[hk];
        }
        w[hk] = tk < len ? exp_f(total - acum[hk]) * dtp[hk] : 0.0f;
    }

    const int r = lane & 15, k8 = 8 * (lane >> 4);
    const int ksteps = (len + 31) / 32;
    // products: wave wv takes p tile wv / 2 and half of the n tiles
    constexpr int kNT = N / 32;  // n tiles per wave
    const int ptile = wv >> 1, nt0 = (wv & 1) * kNT;
#pragma unroll
    for (int hk = 0; hk < kStateHeads; hk++) {
        if (hk >= nh)
            break;  // uniform
        const int h = h0 + hk;
        // (w x)^T into this head's buffer: the other one's products may still
        // run; the barrier of the head before ended the products that read
        // this buffer
        IT(*const X)[kL + kPad] = Xs[hk & 1];
#pragma unroll
        for (int p0 = 0; p0 < kHalfP / 8; p0++)
#pragma unroll
            for (int k = 0; k < 8; k++)
                X[half * kHalfP + 8 * p0 + k][tk] = static_cast<IT>(to_f(xv[p0][k]) * w[hk]);
        __syncthreads();
        if (hk + 1 < nh)  // the next head's x row, in flight during the products
            load_x(h + 1, xv);

        // state^T[n][p] = sum_t Bs[n][t] X[p][t]: formed transposed, a lane
        // ends with 4 consecutive columns n of one row p (16-byte stores)
        f32x4 acc[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; nt++)
            acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = 0; k < ksteps; k++) {
            const V a = *reinterpret_cast<const V *>(&X[16 * ptile + r][32 * k + k8]);
#pragma unroll
            for (int nt = 0; nt < kNT; nt++) {
                const V b = *reinterpret_cast<const V *>(&Bs[16 * (nt0 + nt) + r][32 * k + k8]);
                acc[nt] = M::run(b, a, acc[nt]);
            }
        }
        float *dst = sp.ws_state + (c * sp.H + h) * static_cast<int64_t>(kP * N) + (16 * ptile + r) * N;
#pragma unroll
        for (int nt = 0; nt < kNT; nt++)
            *reinterpret_cast<f32x4 *>(dst + 16 * (nt0 + nt) + 4 * (lane >> 4)) = acc[nt];
    }
}

// ---- stage 2: state passing
//
// One workgroup of 256 lanes per (head, slice of 1024 state elements), 4
// consecutive elements per lane (16-byte loads). The walk over the chunks is
// sequential; what each step needs besides the chunk's own state -- its decay
// factor exp(total cumsum) and its sequence -- is staged in LDS for a segment
// of kPassSeg chunks at a time, so that a step waits on nothing but the own
// states, which are requested kPassAhead chunks ahead.

constexpr int kPassThreads = 256;
constexpr int kPassVec = 4;      // elements per lane
constexpr int kPassAhead = 4;    // own states in flight per lane
constexpr int kPassSeg = 1024;   // chunks whose decay and sequence are staged at a time

template <typename T> struct alignas(4 * sizeof(T)) Vec4 { T v[4]; };  // one 8- or 16-byte access

template <typename ST, typename IT>
__global__ __launch_bounds__(kPassThreads) void ssd_state_pass_kernel(const SsdParams sp) {
    extern __shared__ int owner[];  // owner[c]: the sequence whose state chunk c returns, or -1
    __shared__ float decay_s[kPassSeg];
    __shared__ int64_t seq_s[kPassSeg];
    constexpr int kSlice = kPassThreads * kPassVec;
    const int64_t PN = static_cast<int64_t>(kP) * sp.N;
    const int64_t slices = (PN + kSlice - 1) / kSlice;
    const int h = static_cast<int>(blockIdx.x / slices);
    const int64_t e = (blockIdx.x % slices) * kSlice + threadIdx.x * kPassVec;  // first element of the lane
    if (!sp.intermediate) {
        for (int64_t c = threadIdx.x; c < sp.nchunks; c += kPassThreads)
            owner[c] = -1;
        __syncthreads();
        for (int64_t b = threadIdx.x; b < sp.batch; b += kPassThreads) {
            const int64_t c = idx_at(sp.last_chunk, sp.last_chunk_i64, b * sp.last_chunk_s);
            if (c >= 0 && c < sp.nchunks)
                owner[c] = static_cast<int>(b);
        }
    }
    const bool live = e < PN;  // PN is a multiple of 4: a lane's 4 elements are all in or all out
    ST *outs = static_cast<ST *>(sp.states);
    const ST *init = static_cast<const ST *>(sp.init);
    const int64_t step = sp.H * PN;  // between one chunk's states and the next's
    const float *own_p = sp.ws_state + h * PN + (live ? e : 0);
    auto load_own = [&](int64_t c) {
        return c < sp.nchunks ? *reinterpret_cast<const f32x4 *>(own_p + c * step) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    f32x4 own[kPassAhead];
#pragma unroll
    for (int j = 0; j < kPassAhead; j++)
        own[j] = load_own(j);
    f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t prev = -1;
    for (int64_t c0 = 0; c0 < sp.nchunks; c0 += kPassSeg) {
        const int64_t nseg = sp.nchunks - c0 < kPassSeg ? sp.nchunks - c0 : kPassSeg;
        __syncthreads();  // the previous segment's entries are read; the owner map is written
        for (int64_t k = threadIdx.x; k < nseg; k += kPassThreads) {
            const int64_t c = c0 + k;
            decay_s[k] = exp_f(sp.ws_acum[(c * sp.H + h) * kL + kL - 1]);
            seq_s[k] = idx_at(sp.seq_idx, sp.seq_idx_i64, c * sp.seq_idx_s);
        }
        __syncthreads();
        // kPassAhead chunks per trip (the register ring's index is a constant)
        for (int64_t k0 = 0; k0 < nseg; k0 += kPassAhead) {
#pragma unroll
            for (int j = 0; j < kPassAhead; j++) {
                const int64_t k = k0 + j;
                if (k < nseg) {  // uniform
                    const int64_t c = c0 + k;
                    const int64_t seq = seq_s[k];
                    if (c == 0 || seq != prev) {  // a chunk opens a sequence: its entering state
                        const bool has = init && seq >= 0 && seq < sp.batch && live;
                        const ST *ip = init + ((has ? seq : 0) * sp.H + h) * PN + (live ? e : 0);
#pragma unroll
                        for (int i = 0; i < kPassVec; i++)
                            S[i] = has ? static_cast<float>(ip[i]) : 0.0f;
                    }
                    prev = seq;
                    const f32x4 o = own[j];
                    own[j] = load_own(c + kPassAhead);
                    const int64_t at = (c * sp.H + h) * PN + e;
                    const float d = decay_s[k];
                    if (live) {
                        Vec4<IT> sv;
#pragma unroll
                        for (int i = 0; i < kPassVec; i++)
                            sv.v[i] = static_cast<IT>(S[i]);  // the entering state, as the scan reads it
                        *reinterpret_cast<Vec4<IT> *>(static_cast<IT *>(sp.ws_sin) + at) = sv;
                    }
#pragma unroll
                    for (int i = 0; i < kPassVec; i++)
                        S[i] = d * S[i] + o[i];
                    const int b = sp.intermediate ? 0 : owner[c];
                    if (live && (sp.intermediate || b >= 0)) {
                        Vec4<ST> ov;
#pragma unroll
                        for (int i = 0; i < kPassVec; i++)
                            ov.v[i] = static_cast<ST>(S[i]);
                        ST *dst = sp.intermediate ? outs + at : outs + (static_cast<int64_t>(b) * sp.H + h) * PN + e;
                        *reinterpret_cast<Vec4<ST> *>(dst) = ov;
                    }
                }
            }
        }
    }
}

// ---- stage 3: the chunk scan
//

// y_t = exp(A_t) C_t . S_in + sum_{s<=t} (C_t . B_s) exp(A_t - A_s) dt'_s x_s
//       + D x_t, gated by silu(z_t);   A = the decay cumsum of the chunk.
// One workgroup of 8 waves per (chunk, group, block of kScanHeads heads of
// the group). Rows t in 16-row tiles (wave w takes tiles w and 15-w: equal
// work under the causal mask), columns s in 32-column blocks J. C . B^T does
// not depend on the head: each wave forms its part once, for its 9 (block,
// tile) pairs, and keeps it in registers (fp32) for all heads of the
// workgroup; per head only the decay scaling and the products with x and the
// entering state remain. Per head, x^T, the entering state and the cumsums
// are staged in LDS, the next head's requested while the current one
// computes. Both products are formed transposed, so that a lane owns one
// token t:
//   (B_J C^T)[s][t]: the lane holds t and the 8 columns s = 32J + 4g + i,
//   32J + 16 + 4g + i (g = lane / 16, i < 4), which after scaling is the
//   B operand of y^T += x_J^T (...)^T with that k order (the x side reads
//   the same columns); nothing goes back through LDS;
//   y^T[p][t]: MFMA row m of p tile pt is p = 16 (m / 4) + 4 pt + m % 4, so
//   the lane ends with the 16 consecutive p = 16g .. 16g + 15 of its token
//   (two 16-byte stores, loads of x and z alike).
// Dim p is stored at LDS row 4 (p % 16) + p / 16 of x^T and of the entering
// state: the 16 rows an operand read touches are then consecutive, and with
// 142-word x^T rows the 16 lanes of an 8-byte read pass hit distinct banks
// of the 32.
// Below the diagonal block the decay factors into a row and a column term,
// exp(A_t - A_s) dt'_s = exp(A_t - A_J) * exp(A_J - A_s) dt'_s with A_J the
// cumsum at the block's last token; both are at most 1 there (the cumsum
// does not increase). The diagonal block takes the exact factor per element
// under the causal mask.
constexpr int kScanThreads = 512;
constexpr int kScanTiles = 2;   // 16-token tiles per wave
constexpr int kScanHeads = 4;   // heads per workgroup
constexpr int kScanSlots = 9;   // (block, tile) pairs of a wave: (w / 2 + 1) + ((15 - w) / 2 + 1)
constexpr int kXsRow = kL + 28; // x^T row stride (elements): 142 words, 14 banks past a multiple of 32

__device__ __forceinline__ int dim_row(int p) { return 4 * (p & 15) + (p >> 4); }

template <typename IT, int N>
__global__ __launch_bounds__(kScanThreads) void ssd_chunk_scan_kernel(const SsdParams sp) {
    using M = Mfma<IT>;
    using V = typename M::V;
    constexpr int KN = N / 32;                      // k steps over dstate
    constexpr int kSinSeg = kP * N / kScanThreads;  // entering-state elements a lane stages
    constexpr int kRowPieces = N / 8;               // 16-byte pieces of a B row
    constexpr int kBPass = kL * kRowPieces / kScanThreads;
    static_assert(kSinSeg == 8 || kSinSeg == 16, "whole 16-byte LDS stores");
    static_assert(kP == 64, "a lane's 16 consecutive p per g; the dim-row map");
    static_assert(kL == 256 && kScanThreads == 512, "8 waves of two 16-token tiles");
    __shared__ __attribute__((aligned(16))) float acum_s[kL];
    __shared__ __attribute__((aligned(16))) float dtp_s[kL];
    __shared__ __attribute__((aligned(16))) float q_s[kL];          // column factors
    __shared__ __attribute__((aligned(16))) IT Xs[kP][kXsRow];      // x^T: [dim row][s]
    __shared__ __attribute__((aligned(16))) IT Bs[kL][N + kPad];    // B rows [s][n]
    __shared__ __attribute__((aligned(16))) IT Sin[kP][N + kPad];   // entering state [dim row][n]

    const int ngroups = static_cast<int>(sp.H / sp.hpg);
    const int nhb = (sp.hpg + kScanHeads - 1) / kScanHeads;
    const int32_t wg = xcd_grouped(blockIdx.x, gridDim.x);
    const int64_t c = wg / (ngroups * nhb);
    const int g = (wg / nhb) % ngroups;
    const int hb = wg % nhb;
    const int h0 = g * sp.hpg + hb * kScanHeads;
    const int nh = sp.hpg - hb * kScanHeads < kScanHeads ? sp.hpg - hb * kScanHeads : kScanHeads;
    const int t = threadIdx.x;
    int64_t t0;
    int len;
    chunk_range(sp, c, &t0, &len);
    // the same for every lane: keep them (and what depends on them) scalar
    len = __builtin_amdgcn_readfirstlane(len);
    t0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(t0 >> 32))) << 32 |
         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(t0)));
    if (len == 0)
        return;  // uniform
    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform per wave
    const int r = lane & 15, gq = lane >> 4, g4 = 4 * gq, k8 = 8 * gq;
    const int ntiles = (len + 15) / 16;
    const int rts[kScanTiles] = {wv, 15 - wv};

    // per head: x^T pieces (lane t: the 16-byte dim piece t % 8 of tokens 2j,
    // 2j + 1, j = t / 8 and j + 64), the entering state (kSinSeg consecutive
    // elements) and, for t < 256, token t's cumsum, dt' and block-end cumsum
    struct HeadIn {
        V xv[2][2];
        V sv[kSinSeg / 8];
        float at, dt, aj;
    };
    const int pc = 8 * (t & 7);
    auto load_head = [&](int h, HeadIn &in) {
        const IT *xs = static_cast<const IT *>(sp.x) + head_off(sp, h, sp.x_sh) + pc;
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int v = 0; v < 2; v++) {
                const int tok = 2 * ((t >> 3) + 64 * u) + v;
                in.xv[u][v] = *reinterpret_cast<const V *>(xs + (t0 + (tok < len ? tok : 0)) * sp.x_st);
            }
        const IT *sin = static_cast<const IT *>(sp.ws_sin) + (c * sp.H + h) * static_cast<int64_t>(kP * N) + t * kSinSeg;
#pragma unroll
        for (int k = 0; k < kSinSeg / 8; k++)
            in.sv[k] = *reinterpret_cast<const V *>(sin + 8 * k);
        const int64_t wrow = (c * sp.H + h) * kL;
        const int tc = t & (kL - 1);
        in.at = sp.ws_acum[wrow + tc];
        in.dt = sp.ws_dtp[wrow + tc];
        in.aj = sp.ws_acum[wrow + (tc | 31)];
    };
    auto store_head = [&](const HeadIn &in) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int j2 = 2 * ((t >> 3) + 64 * u);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const IT lo = j2 < len ? in.xv[u][0][e] : static_cast<IT>(0.0f);
                const IT hi = j2 + 1 < len ? in.xv[u][1][e] : static_cast<IT>(0.0f);
                *reinterpret_cast<uint32_t *>(&Xs[dim_row(pc + e)][j2]) =
                    static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                    (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
        }
        const int sp0 = (t * kSinSeg) / N, sn0 = (t * kSinSeg) % N;
#pragma unroll
        for (int k = 0; k < kSinSeg / 8; k++)
            *reinterpret_cast<V *>(&Sin[dim_row(sp0)][sn0 + 8 * k]) = in.sv[k];
        if (t < kL) {
            acum_s[t] = in.at;
            dtp_s[t] = in.dt;
            q_s[t] = exp_f(in.aj - in.at) * in.dt;  // exp(A_J - A_t) dt'_t, J = t / 32
        }
    };

    // shared by the heads: B rows (16-byte pieces, consecutive lanes along a
    // row; rows past the chunk repeat its last row) and the C operands
    {
        const IT *Bg = static_cast<const IT *>(sp.B) + g * sp.B_sg;
        V bv[kBPass];
#pragma unroll
        for (int k = 0; k < kBPass; k++) {
            const int piece = k * kScanThreads + t, srow = piece / kRowPieces;
            bv[k] = *reinterpret_cast<const V *>(Bg + (t0 + (srow < len ? srow : len - 1)) * sp.B_st +
                                                 (piece % kRowPieces) * 8);
        }
        HeadIn first;
        load_head(h0, first);
#pragma unroll
        for (int k = 0; k < kBPass; k++) {
            const int piece = k * kScanThreads + t;
            *reinterpret_cast<V *>(&Bs[piece / kRowPieces][(piece % kRowPieces) * 8]) = bv[k];
        }
        store_head(first);
    }
    V ac[kScanTiles][KN];  // the C row of the lane's token in each tile
#pragma unroll
    for (int i = 0; i < kScanTiles; i++) {
        const int tr = 16 * rts[i] + r;
        const int64_t tok = t0 + (tr < len ? tr : len - 1);
        const IT *crow = static_cast<const IT *>(sp.C) + g * sp.C_sg + tok * sp.C_st;
#pragma unroll
        for (int k = 0; k < KN; k++)
            ac[i][k] = *reinterpret_cast<const V *>(crow + 32 * k + k8);
    }
    __syncthreads();

    // The wave's (block, tile) slots: tile rt0 = wv keeps block J in slot J
    // (J = 0 .. nj0, its diagonal block nj0 = rt0 / 2 <= 3), tile
    // rt1 = 15 - wv block J in slot 8 - J (J = 0 .. nj1, nj1 = rt1 / 2 =
    // 7 - nj0): slots nj0 + 1 .. 8, and every slot index a constant.
    const int rt0 = rts[0], rt1 = rts[1];
    const int nj0 = rt0 >> 1, nj1 = rt1 >> 1;
    const bool act0 = rt0 < ntiles, act1 = rt1 < ntiles;  // uniform; act1 implies act0
    const int tt0 = 16 * rt0 + r, tt1 = 16 * rt1 + r;     // the lane's tokens
    // (B_J C^T) of one tile: the lane's token, columns s_lo + i, s_lo + 16 + i
    auto bc = [&](int J, const V (&acv)[KN], f32x4 (&d)[2]) {
        d[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        d[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KN; k++) {
            d[0] = M::run(*reinterpret_cast<const V *>(&Bs[32 * J + r][32 * k + k8]), acv[k], d[0]);
            d[1] = M::run(*reinterpret_cast<const V *>(&Bs[32 * J + 16 + r][32 * k + k8]), acv[k], d[1]);
        }
    };
    f32x4 cb[kScanSlots][2];
#pragma unroll
    for (int q = 0; q < kScanSlots; q++)
        cb[q][0] = cb[q][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (act0) {
#pragma unroll
        for (int J = 0; J < 4; J++)
            if (J <= nj0)
                bc(J, ac[0], cb[J]);
    }
    if (act1) {
#pragma unroll
        for (int J = 0; J < 8; J++)
            if (J <= nj1)
                bc(J, ac[1], cb[8 - J]);
    }
    // B is no longer needed: its rows take the C rows (row = token), the B
    // operands of the entering-state product, read back per head by the
    // lanes that wrote them
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanTiles; i++)
#pragma unroll
        for (int k = 0; k < KN; k++)
            *reinterpret_cast<V *>(&Bs[16 * rts[i] + r][32 * k + k8]) = ac[i][k];
    IT(*const Cs)[N + kPad] = Bs;

    IT *outp = static_cast<IT *>(sp.out);
    const IT *zs = static_cast<const IT *>(sp.z);
    const int pr = 16 * (r >> 2) + (r & 3);  // p of MFMA row r in p tile 0 (+ 4 pt)
    int xrow[kP / 16];                       // LDS row of p = pr + 4 pt
#pragma unroll
    for (int pt = 0; pt < kP / 16; pt++)
        xrow[pt] = dim_row(pr + 4 * pt);

    // D of the workgroup's heads, read once (a per-head load in the loop would
    // be waited on together with every load issued before it)
    float Dh[kScanHeads];
#pragma unroll
    for (int hk = 0; hk < kScanHeads; hk++)
        Dh[hk] = sp.D ? sp.D[((hk < nh ? h0 + hk : h0) / sp.hsplit) * sp.D_sh] : 0.0f;

    for (int hk = 0; hk < nh; hk++) {
        const int h = h0 + hk;
        float dh = Dh[0];
#pragma unroll
        for (int k = 1; k < kScanHeads; k++)
            dh = hk == k ? Dh[k] : dh;
        // z of the lane's token (16 consecutive p), for the gate
        auto load_z = [&](int tt, V (&zv2)[2]) {
            const int64_t tok = t0 + (tt < len ? tt : len - 1);
            const IT *zg = zs + tok * sp.z_st + head_off(sp, h, sp.z_sh) + 16 * gq;
#pragma unroll
            for (int k = 0; k < 2; k++)
                zv2[k] = zs ? *reinterpret_cast<const V *>(zg + 8 * k) : V{};
        };
        // the entering state's contribution, y^T = S_in C^T, scaled by exp(A_t)
        auto init = [&](int tt, float at, f32x4 (&y)[kP / 16]) {
            const float rs = exp_f(at);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < KN; k++)
                    acc = M::run(*reinterpret_cast<const V *>(&Sin[xrow[pt]][32 * k + k8]),
                                 *reinterpret_cast<const V *>(&Cs[tt][32 * k + k8]), acc);
#pragma unroll
                for (int ii = 0; ii < 4; ii++)
                    acc[ii] *= rs;
                y[pt] = acc;
            }
        };
        // below the diagonal: the row factor exp(A_t - A_J) and the columns' factors
        auto scale_off = [&](int J, float at, const f32x4 (&d)[2]) {
            const int s_lo = 32 * J + g4;
            const float rf = exp_f(at - acum_s[32 * J + 31]);
            const f32x4 q_lo = *reinterpret_cast<const f32x4 *>(&q_s[s_lo]);
            const f32x4 q_hi = *reinterpret_cast<const f32x4 *>(&q_s[s_lo + 16]);
            V a;
#pragma unroll
            for (int ii = 0; ii < 4; ii++) {
                a[ii] = static_cast<IT>(d[0][ii] * (rf * q_lo[ii]));
                a[4 + ii] = static_cast<IT>(d[1][ii] * (rf * q_hi[ii]));
            }
            return a;
        };
        // the diagonal block: exact factor, causal mask (a select, no branch;
        // A_t - A_s <= 0 for s <= t, the clamp only keeps the masked-out
        // factors finite)
        auto scale_diag = [&](int J, int tt, float at, const f32x4 (&d)[2]) {
            const int s_lo = 32 * J + g4;
            const f32x4 a_lo = *reinterpret_cast<const f32x4 *>(&acum_s[s_lo]);
            const f32x4 a_hi = *reinterpret_cast<const f32x4 *>(&acum_s[s_lo + 16]);
            const f32x4 w_lo = *reinterpret_cast<const f32x4 *>(&dtp_s[s_lo]);
            const f32x4 w_hi = *reinterpret_cast<const f32x4 *>(&dtp_s[s_lo + 16]);
            // the compares are made here, per head: hoisted out of the head
            // loop their masks would hold 2 SGPRs each for the whole loop
            int lim = tt - s_lo;
            asm volatile("" : "+v"(lim));
            V a;
#pragma unroll
            for (int ii = 0; ii < 4; ii++) {
                const float m0 = d[0][ii] * (exp_f(fminf(at - a_lo[ii], 0.0f)) * w_lo[ii]);
                const float m1 = d[1][ii] * (exp_f(fminf(at - a_hi[ii], 0.0f)) * w_hi[ii]);
                a[ii] = static_cast<IT>(ii <= lim ? m0 : 0.0f);
                a[4 + ii] = static_cast<IT>(16 + ii <= lim ? m1 : 0.0f);
            }
            return a;
        };
        auto xop = [&](int J, int pt) {
            const int s_lo = 32 * J + g4;
            const uint2 lo = *reinterpret_cast<const uint2 *>(&Xs[xrow[pt]][s_lo]);
            const uint2 hi = *reinterpret_cast<const uint2 *>(&Xs[xrow[pt]][s_lo + 16]);
            return __builtin_bit_cast(V, (uint4{lo.x, lo.y, hi.x, hi.y}));
        };
        // block J of a tile: scaled, then y^T += x_J^T (...)^T
        auto block = [&](int J, bool diag, int tt, float at, const f32x4 (&d)[2], f32x4 (&y)[kP / 16]) {
            const V a = diag ? scale_diag(J, tt, at, d) : scale_off(J, at, d);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
                y[pt] = M::run(xop(J, pt), a, y[pt]);
        };
        // D x (x from its LDS copy: p = 16 gq + e sits at row 4 e + gq), the
        // gate, the store: y[pt][ii] is p = 16 gq + 4 pt + ii of the token
        auto finish = [&](const f32x4 (&y)[kP / 16], const V (&zv2)[2], int tt) {
            if (tt >= len)
                return;
            const int64_t tok = t0 + tt;
            V o[2];
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    const int e = 4 * pt + ii;  // 0..15
                    float v = y[pt][ii] + dh * to_f(Xs[4 * e + gq][tt]);
                    if (zs)
                        v *= silu_f(to_f(zv2[e / 8][e % 8]));
                    o[e / 8][e % 8] = static_cast<IT>(v);
                }
            IT *orow = outp + tok * sp.out_st + head_off(sp, h, sp.out_sh) + 16 * gq;
            *reinterpret_cast<V *>(orow) = o[0];
            *reinterpret_cast<V *>(orow + 8) = o[1];
        };

        // the two tiles one after the other: one tile's accumulators and z
        // row are live at a time. Loads are issued in the order they are
        // waited on: tile 0's z, then tile 1's, then the next head's inputs
        // (in flight during tile 1 and until the head's end)
        if (act0) {  // uniform per wave
            V zv2[2];
            load_z(tt0, zv2);
            const float at0 = acum_s[tt0];
            f32x4 y[kP / 16];
            init(tt0, at0, y);
#pragma unroll
            for (int J = 0; J < 4; J++)
                if (J <= nj0)  // uniform
                    block(J, J == nj0, tt0, at0, cb[J], y);
            finish(y, zv2, tt0);
        }
        V zv1[2];
        if (act1)
            load_z(tt1, zv1);
        HeadIn next;
        if (hk + 1 < nh)
            load_head(h + 1, next);
        if (act1) {
            const V (&zv2)[2] = zv1;
            const float at1 = acum_s[tt1];
            f32x4 y[kP / 16];
            init(tt1, at1, y);
#pragma unroll
            for (int J = 0; J < 8; J++)
                if (J <= nj1)  // uniform; nj1 >= 4
                    block(J, J == nj1, tt1, at1, cb[8 - J], y);
            finish(y, zv2, tt1);
        }
        if (hk + 1 < nh) {  // uniform: the next head's inputs replace this one's
            __syncthreads();
            store_head(next);
            __syncthreads();
        }
    }
}

template <typename IT, int N>
int launch_ssd_typed(const SsdParams &sp, int state_dtype, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SsdParams p = sp;
    void *args[] = {&p};
    const unsigned state_grid = static_cast<unsigned>(sp.nchunks * (sp.H / sp.hpg) *
                                                      ((sp.hpg + kStateHeads - 1) / kStateHeads));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_chunk_state_kernel<IT, N>), dim3(state_grid),
                                   dim3(kStateThreads), args, 0, s);
    if (e != hipSuccess)
        return static_cast<int>(e);
    const unsigned pass_grid =
        static_cast<unsigned>(sp.H * ((static_cast<int64_t>(kP) * N + kPassThreads * kPassVec - 1) / (kPassThreads * kPassVec)));
    const size_t owner_bytes = sp.intermediate ? 0 : static_cast<size_t>(sp.nchunks) * sizeof(int);
    const void *pass = state_dtype == SSU_F32    ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<float, IT>)
                       : state_dtype == SSU_F16  ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<_Float16, IT>)
                                                 : reinterpret_cast<const void *>(&ssd_state_pass_kernel<__bf16, IT>);
    e = hipLaunchKernel(pass, dim3(pass_grid), dim3(kPassThreads), args, owner_bytes, s);
    if (e != hipSuccess)
        return static_cast<int>(e);
    const unsigned scan_grid = static_cast<unsigned>(sp.nchunks * (sp.H / sp.hpg) *
                                                     ((sp.hpg + kScanHeads - 1) / kScanHeads));
    e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_chunk_scan_kernel<IT, N>), dim3(scan_grid),
                        dim3(kScanThreads), args, 0, s);
    return static_cast<int>(e);
}

template <typename IT, int N>
int attributes_typed(int state_dtype, const char *names[3], int vgprs[3]) {
    const void *fns[3] = {
        reinterpret_cast<const void *>(&ssd_chunk_state_kernel<IT, N>),
        state_dtype == SSU_F32   ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<float, IT>)
        : state_dtype == SSU_F16 ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<_Float16, IT>)
                                 : reinterpret_cast<const void *>(&ssd_state_pass_kernel<__bf16, IT>),
        reinterpret_cast<const void *>(&ssd_chunk_scan_kernel<IT, N>)};
    names[0] = "ssd_chunk_state_kernel";
    names[1] = "ssd_state_pass_kernel";
    names[2] = "ssd_chunk_scan_kernel";
    for (int i = 0; i < 3; i++) {
        hipFuncAttributes attr;
        const hipError_t e = hipFuncGetAttributes(&attr, fns[i]);
        if (e != hipSuccess)
            return static_cast<int>(e);
        vgprs[i] = attr.numRegs;
    }
    return 0;
}

}  // namespace

int ssd_kernel_attributes(int io_dtype, int state_dtype, int dstate, const char *names[3], int vgprs[3]) {
    if (io_dtype == SSU_BF16)
        return dstate == 64 ? attributes_typed<__bf16, 64>(state_dtype, names, vgprs)
                            : attributes_typed<__bf16, 128>(state_dtype, names, vgprs);
    return dstate == 64 ? attributes_typed<_Float16, 64>(state_dtype, names, vgprs)
                        : attributes_typed<_Float16, 128>(state_dtype, names, vgprs);
}

int launch_ssd(const SsdParams &sp, int io_dtype, int state_dtype, void *stream) {
    if (io_dtype == SSU_BF16)
        return sp.N == 64 ? launch_ssd_typed<__bf16, 64>(sp, state_dtype, stream)
                          : launch_ssd_typed<__bf16, 128>(sp, state_dtype, stream);
    return sp.N == 64 ? launch_ssd_typed<_Float16, 64>(sp, state_dtype, stream)
                      : launch_ssd_typed<_Float16, 128>(sp, state_dtype, stream);
}

}  // namespace ssu
