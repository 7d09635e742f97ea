// SSD packed variable-length prefill for gfx950 (MATE docs, "Mamba / SSU",
// section "SSD packed prefill"): the same recurrence as the decode step over
// every token of a packed batch, computed chunk by chunk. Three launches:
//   ssd_chunk_state_kernel   per (chunk, head): dt' (softplus, dt_limit),
//                            the decay cumsum, and the chunk's own state
//                            sum_t exp(A_end - A_t) dt'_t x_t B_t^T (MFMA);
//   ssd_state_pass_kernel    per (head, state slice): walks the chunks in
//                            order, resetting where seq_idx opens a sequence;
//                            leaves each chunk's entering state in the
//                            workspace and writes the returned states;
//   ssd_chunk_scan_kernel    per (chunk, head): y_t = sum_{s<=t} (C_t . B_s)
//                            exp(A_t - A_s) dt'_s x_s + exp(A_t) C_t . S_in
//                            + D x_t, gated by silu(z_t) (MFMA).
// MFMA operands are bf16 / f16 (the x dtype): 16x16x32 tiles with fp32
// accumulation; the scaled operands (w_t B_t, the masked C.B^T, the entering
// state) are rounded to the x dtype before they enter a product.

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
// dt_limit clamp
template <typename IT>
__device__ __forceinline__ float processed_dt(const SsdParams &sp, int64_t t, int h) {
    const int64_t i = t * sp.dt_st + static_cast<int64_t>(h) * sp.dt_sh;
    float v = sp.dt_f32 ? static_cast<const float *>(sp.dt)[i] : to_f(static_cast<const IT *>(sp.dt)[i]);
    if (sp.dt_bias)
        v += sp.dt_bias[h * sp.bias_sh];
    if (sp.softplus)
        v = softplus_f(v);
    v = v < sp.dt_lo ? sp.dt_lo : v;
    return v > sp.dt_hi ? sp.dt_hi : v;
}

// ---- stage 1: dt', the decay cumsum, and the chunk's own state

template <typename IT, int N>
__global__ __launch_bounds__(256) void ssd_chunk_state_kernel(const SsdParams sp) {
    using M = Mfma<IT>;
    using V = typename M::V;
    __shared__ float scan[kL];
    __shared__ __attribute__((aligned(16))) IT Xs[kP][kL + kPad];  // x^T:  [p][t]
    __shared__ __attribute__((aligned(16))) IT Bs[N][kL + kPad];   // (w B)^T: [n][t]

    const int64_t c = blockIdx.x / sp.H;
    const int h = blockIdx.x % sp.H;
    const int g = h / sp.hpg;
    const int t = threadIdx.x;  // token in the chunk (kL threads)
    int64_t t0;
    int len;
    chunk_range(sp, c, &t0, &len);

    const float dtp = t < len ? processed_dt<IT>(sp, t0 + t, h) : 0.0f;
    scan[t] = dtp * sp.A[h * sp.A_sh];
    __syncthreads();
    for (int off = 1; off < kL; off <<= 1) {  // inclusive prefix sum
        const float add = t >= off ? scan[t - off] : 0.0f;
        __syncthreads();
        scan[t] += add;
        __syncthreads();
    }
    const float acum = scan[t];
    const float total = scan[kL - 1];  // padding adds nothing
    const int64_t wrow = (c * sp.H + h) * kL;
    sp.ws_dtp[wrow + t] = dtp;
    sp.ws_acum[wrow + t] = acum;
    const float w = t < len ? exp_f(total - acum) * dtp : 0.0f;

    // token t's x row and scaled B row, transposed into LDS (lanes past the
    // chunk read token 0, always present, and store zeros)
    const int64_t tok = t < len ? t0 + t : 0;
    const IT *xrow = static_cast<const IT *>(sp.x) + (tok * sp.x_st + h * sp.x_sh);
    const IT *brow = static_cast<const IT *>(sp.B) + (tok * sp.B_st + g * sp.B_sg);
#pragma unroll
    for (int p0 = 0; p0 < kP; p0 += 8) {
        const V v = *reinterpret_cast<const V *>(xrow + p0);
#pragma unroll
        for (int k = 0; k < 8; k++)
            Xs[p0 + k][t] = t < len ? v[k] : static_cast<IT>(0.0f);
    }
#pragma unroll
    for (int n0 = 0; n0 < N; n0 += 8) {
        const V v = *reinterpret_cast<const V *>(brow + n0);
#pragma unroll
        for (int k = 0; k < 8; k++)
            Bs[n0 + k][t] = static_cast<IT>(to_f(v[k]) * w);
    }
    __syncthreads();

    // state[p][n] = sum_t Xs[p][t] Bs[n][t]; wave wv takes rows p = 16 wv ..
    const int lane = t & 63, wv = t >> 6;
    f32x4 acc[N / 16];
#pragma unroll
    for (int nt = 0; nt < N / 16; nt++)
        acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int ksteps = (len + 31) / 32;
    const int r = lane & 15, k8 = 8 * (lane >> 4);
    for (int k = 0; k < ksteps; k++) {
        const V a = *reinterpret_cast<const V *>(&Xs[16 * wv + r][32 * k + k8]);
#pragma unroll
        for (int nt = 0; nt < N / 16; nt++) {
            const V b = *reinterpret_cast<const V *>(&Bs[16 * nt + r][32 * k + k8]);
            acc[nt] = M::run(a, b, acc[nt]);
        }
    }
    float *dst = sp.ws_state + (c * sp.H + h) * static_cast<int64_t>(kP * N);
#pragma unroll
    for (int nt = 0; nt < N / 16; nt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            dst[(16 * wv + 4 * (lane >> 4) + i) * N + 16 * nt + r] = acc[nt][i];
}

// ---- stage 2: state passing

template <typename ST>
__global__ __launch_bounds__(256) void ssd_state_pass_kernel(const SsdParams sp) {
    extern __shared__ int owner[];  // owner[c]: the sequence whose state chunk c returns, or -1
    const int64_t tiles = (static_cast<int64_t>(kP) * sp.N + 255) / 256;
    const int h = static_cast<int>(blockIdx.x / tiles);
    const int64_t e = (blockIdx.x % tiles) * 256 + threadIdx.x;  // element of the [P, N] tile
    const int64_t PN = static_cast<int64_t>(kP) * sp.N;
    if (!sp.intermediate) {
        for (int64_t c = threadIdx.x; c < sp.nchunks; c += 256)
            owner[c] = -1;
        __syncthreads();
        for (int64_t b = threadIdx.x; b < sp.batch; b += 256) {
            const int64_t c = idx_at(sp.last_chunk, sp.last_chunk_i64, b * sp.last_chunk_s);
            if (c >= 0 && c < sp.nchunks)
                owner[c] = static_cast<int>(b);
        }
        __syncthreads();
    }
    if (e >= PN)
        return;
    ST *outs = static_cast<ST *>(sp.states);
    const ST *init = static_cast<const ST *>(sp.init);
    float S = 0.0f;
    int64_t prev = -1;
    float own = sp.nchunks > 0 ? sp.ws_state[h * PN + e] : 0.0f;
    for (int64_t c = 0; c < sp.nchunks; c++) {
        const int64_t seq = idx_at(sp.seq_idx, sp.seq_idx_i64, c * sp.seq_idx_s);
        if (c == 0 || seq != prev)  // a chunk opens a sequence: its entering state
            S = (init && seq >= 0 && seq < sp.batch) ? static_cast<float>(init[(seq * sp.H + h) * PN + e]) : 0.0f;
        prev = seq;
        const int64_t at = (c * sp.H + h) * PN + e;
        // next chunk's own state requested before this one is overwritten
        const float own_next = c + 1 < sp.nchunks ? sp.ws_state[at + sp.H * PN] : 0.0f;
        const float total = sp.ws_acum[(c * sp.H + h) * kL + kL - 1];
        sp.ws_state[at] = S;  // the entering state, read by the scan
        S = exp_f(total) * S + own;
        if (sp.intermediate) {
            outs[at] = static_cast<ST>(S);
        } else {
            const int b = owner[c];
            if (b >= 0)
                outs[(static_cast<int64_t>(b) * sp.H + h) * PN + e] = static_cast<ST>(S);
        }
        own = own_next;
    }
}

// ---- stage 3: the chunk scan

template <typename IT, int N>
__global__ __launch_bounds__(256) void ssd_chunk_scan_kernel(const SsdParams sp) {
    using M = Mfma<IT>;
    using V = typename M::V;
    __shared__ float acum_s[kL], dtp_s[kL];
    __shared__ __attribute__((aligned(16))) IT Xs[kP][kL + kPad];      // x^T: [p][s]
    __shared__ __attribute__((aligned(16))) IT Sin[kP][N + kPad];      // entering state [p][n]
    __shared__ __attribute__((aligned(16))) IT Ms[4][16][32 + kPad];   // per wave: masked C.B^T slice

    const int64_t c = blockIdx.x / sp.H;
    const int h = blockIdx.x % sp.H;
    const int g = h / sp.hpg;
    const int t = threadIdx.x;
    int64_t t0;
    int len;
    chunk_range(sp, c, &t0, &len);
    if (len == 0)
        return;  // uniform
    const int64_t wrow = (c * sp.H + h) * kL;
    acum_s[t] = sp.ws_acum[wrow + t];
    dtp_s[t] = sp.ws_dtp[wrow + t];
    {
        const IT *xrow = static_cast<const IT *>(sp.x) + ((t0 + (t < len ? t : 0)) * sp.x_st + h * sp.x_sh);
#pragma unroll
        for (int p0 = 0; p0 < kP; p0 += 8) {
            const V v = *reinterpret_cast<const V *>(xrow + p0);
#pragma unroll
            for (int k = 0; k < 8; k++)
                Xs[p0 + k][t] = t < len ? v[k] : static_cast<IT>(0.0f);
        }
        const float *sin = sp.ws_state + (c * sp.H + h) * static_cast<int64_t>(kP * N);
        for (int i = t; i < kP * N; i += 256)
            Sin[i / N][i % N] = static_cast<IT>(sin[i]);
    }
    __syncthreads();

    const int lane = t & 63, wv = t >> 6;
    const int r = lane & 15, k8 = 8 * (lane >> 4), q4 = 4 * (lane >> 4);
    const IT *Cs = static_cast<const IT *>(sp.C);
    const int ntiles = (len + 15) / 16;
    for (int rt = wv; rt < ntiles; rt += 4) {  // 16-row tiles, round robin over the waves
        // this lane's A operands: C of row 16 rt + r (rows past the chunk read its last row)
        const int trow = 16 * rt + r < len ? 16 * rt + r : len - 1;
        const IT *crow = Cs + ((t0 + trow) * sp.C_st + g * sp.C_sg);
        V ac[N / 32];
#pragma unroll
        for (int k = 0; k < N / 32; k++)
            ac[k] = *reinterpret_cast<const V *>(crow + 32 * k + k8);
        // the entering state's contribution, scaled per row by exp(A_t)
        f32x4 y[kP / 16];
#pragma unroll
        for (int pt = 0; pt < kP / 16; pt++) {
            f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < N / 32; k++)
                a = M::run(ac[k], *reinterpret_cast<const V *>(&Sin[16 * pt + r][32 * k + k8]), a);
            y[pt] = a;
        }
        float rowscale[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int tr = 16 * rt + q4 + i;
            rowscale[i] = exp_f(acum_s[tr < len ? tr : len - 1]);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
                y[pt][i] *= rowscale[i];
        }
        // the causal intra-chunk sum, 32 columns s at a time; the B operands
        // of the next 32 columns are requested one step ahead
        float at[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int tr = 16 * rt + q4 + i;
            at[i] = acum_s[tr < len ? tr : len - 1];
        }
        const IT *Bsrc = static_cast<const IT *>(sp.B) + g * sp.B_sg;
        auto fetch_b = [&](int sb, V (&bo)[2][N / 32]) {
#pragma unroll
            for (int s16 = 0; s16 < 2; s16++) {
                const int scol = 32 * sb + 16 * s16 + r;
                const IT *brow = Bsrc + (t0 + (scol < len ? scol : len - 1)) * sp.B_st;
#pragma unroll
                for (int k = 0; k < N / 32; k++)
                    bo[s16][k] = *reinterpret_cast<const V *>(brow + 32 * k + k8);
            }
        };
        const int scols = (16 * rt + 15) / 32 + 1;
        V bcur[2][N / 32], bnext[2][N / 32];
        fetch_b(0, bcur);
        for (int sb = 0; sb < scols; sb++) {
            fetch_b(sb + 1 < scols ? sb + 1 : sb, bnext);
#pragma unroll
            for (int s16 = 0; s16 < 2; s16++) {
                const int scol = 32 * sb + 16 * s16 + r;  // this lane's column of C.B^T
                const int sr = scol < len ? scol : len - 1;
                f32x4 cb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < N / 32; k++)
                    cb = M::run(ac[k], bcur[s16][k], cb);
                const float as = acum_s[sr], ds = dtp_s[sr];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int tr = 16 * rt + q4 + i;
                    const bool keep = scol <= tr && scol < len;
                    const float m = keep ? cb[i] * exp_f(at[i] - as) * ds : 0.0f;
                    Ms[wv][q4 + i][16 * s16 + r] = static_cast<IT>(m);
                }
            }
            // wave-private slice: ds_write then ds_read, in order within the wave
            const V am = *reinterpret_cast<const V *>(&Ms[wv][r][k8]);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
                y[pt] = M::run(am, *reinterpret_cast<const V *>(&Xs[16 * pt + r][32 * sb + k8]), y[pt]);
#pragma unroll
            for (int s16 = 0; s16 < 2; s16++)
#pragma unroll
                for (int k = 0; k < N / 32; k++)
                    bcur[s16][k] = bnext[s16][k];
        }
        // D x, the gate, the store
        IT *outp = static_cast<IT *>(sp.out);
        const IT *zs = static_cast<const IT *>(sp.z);
        const float dh = sp.D ? sp.D[h * sp.D_sh] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int tr = 16 * rt + q4 + i;
            if (tr >= len)
                continue;
            const int64_t tok = t0 + tr;
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++) {
                const int p = 16 * pt + r;
                float v = y[pt][i] + dh * to_f(Xs[p][tr]);
                if (zs)
                    v *= silu_f(to_f(zs[tok * sp.z_st + h * sp.z_sh + p]));
                outp[tok * sp.out_st + h * sp.out_sh + p] = static_cast<IT>(v);
            }
        }
    }
}

template <typename IT, int N>
int launch_ssd_typed(const SsdParams &sp, int state_dtype, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SsdParams p = sp;
    void *args[] = {&p};
    const unsigned chunk_grid = static_cast<unsigned>(sp.nchunks * sp.H);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_chunk_state_kernel<IT, N>), dim3(chunk_grid),
                                   dim3(256), args, 0, s);
    if (e != hipSuccess)
        return static_cast<int>(e);
    const unsigned pass_grid = static_cast<unsigned>(sp.H * ((static_cast<int64_t>(kP) * N + 255) / 256));
    const size_t owner_bytes = sp.intermediate ? 0 : static_cast<size_t>(sp.nchunks) * sizeof(int);
    const void *pass = state_dtype == SSU_F32    ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<float>)
                       : state_dtype == SSU_F16  ? reinterpret_cast<const void *>(&ssd_state_pass_kernel<_Float16>)
                                                 : reinterpret_cast<const void *>(&ssd_state_pass_kernel<__bf16>);
    e = hipLaunchKernel(pass, dim3(pass_grid), dim3(256), args, owner_bytes, s);
    if (e != hipSuccess)
        return static_cast<int>(e);
    e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_chunk_scan_kernel<IT, N>), dim3(chunk_grid), dim3(256),
                        args, 0, s);
    return static_cast<int>(e);
}

}  // namespace

int launch_ssd(const SsdParams &sp, int io_dtype, int state_dtype, void *stream) {
    if (io_dtype == SSU_BF16)
        return sp.N == 64 ? launch_ssd_typed<__bf16, 64>(sp, state_dtype, stream)
                          : launch_ssd_typed<__bf16, 128>(sp, state_dtype, stream);
    return sp.N == 64 ? launch_ssd_typed<_Float16, 64>(sp, state_dtype, stream)
                      : launch_ssd_typed<_Float16, 128>(sp, state_dtype, stream);
}

}  // namespace ssu
