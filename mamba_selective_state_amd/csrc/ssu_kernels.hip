// gfx950 kernels of the Mamba-2 selective state update (SSU).
//
// What one workgroup computes (MATE docs, "Mamba / SSU", API reference and
// table "SSU at a glance"; ReplaySSM article, section "三个瓶颈其实来自同一个动作"
// for the step S_t = a_t S_{t-1} + dt_t x_t B_t^T and readout y_t = S_t C_t):
// one (sequence, head, dim tile). It resolves the sequence's read slot, loads
// its [rows, dstate] part of the state tile into registers once, then for each
// of the sequence's tokens applies the decay and the rank-1 term in fp32,
// reduces y = C.S across the 16 lanes of each dim row with DPP, adds D.x, gates
// by silu(z), and stores the tile through the token's destination slot.
//
// Layout in registers: lane l of a wave serves dim row 4*pass + l/16 of the
// wave's rows and the dstate columns c*16*VEC + (l%16)*VEC + [0, VEC) of it,
// VEC being the elements of one 16-byte access (4 fp32 or 8 16-bit values).
// A wave's access of one chunk therefore covers whole 64..256-byte runs of
// consecutive rows: every state byte moves in 16-byte coalesced accesses, and
// the tile, contiguous in the pool, is read and written exactly once per call
// (plus once per extra token on the multi-token path, as each token publishes
// its state).
//
// Read-before-write: each lane stores only the elements it loaded itself,
// after loading them, and different lanes, waves and workgroups own disjoint
// elements, so a destination slot equal to the read slot (in-place decode, or
// a token writing the entry the sequence read) is safe without barriers.
//
// No matrix cores: the step is a rank-1 update and a matrix-vector product
// per token, far below the HBM ridge point; the kernel is bandwidth-bound.

#include <hip/hip_runtime.h>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(_Float16 v) { return (float)v; }
__device__ __forceinline__ float widen(__bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T narrow(float v) { return (T)v; }  // round to nearest even

// Raw bits of one element, zero-extended; the conversion to fp32 is a separate
// step so that a load is not followed by a wait inside a branch.
template <typename T>
__device__ __forceinline__ uint32_t load_bits(const T *p) {
    if constexpr (sizeof(T) == 4)
        return *reinterpret_cast<const uint32_t *>(p);
    else
        return *reinterpret_cast<const uint16_t *>(p);
}
__device__ __forceinline__ float bits_f32(uint32_t b, float *) { return __uint_as_float(b); }
__device__ __forceinline__ float bits_f32(uint32_t b, __bf16 *) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bits_f32(uint32_t b, _Float16 *) {
    return (float)__builtin_bit_cast(_Float16, static_cast<uint16_t>(b));
}
template <typename T>
__device__ __forceinline__ float from_bits(uint32_t b) { return bits_f32(b, static_cast<T *>(nullptr)); }

// One 16-byte (or smaller) access of VEC consecutive elements.
template <typename T, int VEC>
struct alignas(sizeof(T) * VEC) Pack {
    T v[VEC];
};

__device__ __forceinline__ int64_t load_index(const void *base, bool i64, int64_t i) {
    return i64 ? static_cast<const int64_t *>(base)[i]
               : static_cast<int64_t>(static_cast<const int32_t *>(base)[i]);
}

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15); every lane of the
// row receives the sum. Needs all lanes of the row active.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// Entry of a slot table naming sequence b's position t.
__device__ __forceinline__ int64_t table_slot(const void *tab, bool two_d, bool i64, int64_t s0,
                                              int64_t s1, int64_t b, int64_t first_row, int64_t t) {
    const int64_t i = two_d ? b * s0 + t * s1 : (first_row + t) * s0;
    return load_index(tab, i64, i);
}

template <typename ST, typename IT, int N, bool MULTI>
__global__ __launch_bounds__(kMaxWaves *kWaveLanes) void ssu_kernel(const Params p) {
    constexpr int E = N / kLanesPerRow;  // state elements per lane per row
    constexpr int VEC = (16 / (int)sizeof(ST)) < E ? (16 / (int)sizeof(ST)) : E;
    constexpr int NCH = E / VEC;         // accesses per lane per row
    constexpr int PASSES = passes_for(N);
    constexpr int IVEC = VEC;            // B / C are read with the same column split
    static_assert(E * kLanesPerRow == N && NCH * VEC == E, "dstate split");

    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int wave = threadIdx.x / kWaveLanes;
    const int col = lane & (kLanesPerRow - 1);
    const int rsub = lane / kLanesPerRow;
    const int flags = p.flags;

    // workgroup -> (sequence, head, dim tile)
    const int64_t wg = blockIdx.x;
    const int tile = static_cast<int>(wg % p.dim_tiles);
    const int64_t sh = wg / p.dim_tiles;
    const int h = static_cast<int>(sh % p.H);
    const int64_t b = sh / p.H;
    const int g = h / p.heads_per_group;
    const int d0 = tile * p.rows_per_block + wave * (kRowsPerPass * PASSES) + rsub;

    // the sequence's rows
    int64_t first_row = b, len = 1;
    if (MULTI) {
        if (p.layout == kCuSeqlens) {
            first_row = load_index(p.cu, flags & kCuI64, b * p.cu_s);
            len = load_index(p.cu, flags & kCuI64, (b + 1) * p.cu_s) - first_row;
        } else if (p.layout == kDense) {
            first_row = b * p.steps;
            len = p.steps;
        }
        if (len <= 0)
            return;  // empty sequence: nothing to read or write
    }

    // read slot: entry num_accepted_tokens[b] - 1 (floored at 0) of the read
    // table, or the sequence index without a table
    int64_t start = 0;
    if (MULTI && p.acc) {
        start = load_index(p.acc, flags & kAccI64, b * p.acc_s) - 1;
        start = start < 0 ? 0 : start;
    }
    const int64_t rslot = p.rtab ? table_slot(p.rtab, flags & kRead2D, flags & kReadI64, p.r_s0,
                                              p.r_s1, b, first_row, start)
                                 : b;

    const int64_t tile_off = static_cast<int64_t>(h) * p.P * N;
    ST *const pool = static_cast<ST *>(p.state);

    // load the state tile (zeros for the pad id)
    float S[PASSES][E];
    const bool read_pad = rslot == p.pad;
#pragma unroll
    for (int q = 0; q < PASSES; q++) {
        const int d = d0 + q * kRowsPerPass;
        if (!read_pad && d < p.P) {
            const ST *src = pool + rslot * p.slot_stride + tile_off + static_cast<int64_t>(d) * N;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const Pack<ST, VEC> v =
                    *reinterpret_cast<const Pack<ST, VEC> *>(src + c * kLanesPerRow * VEC + col * VEC);
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    S[q][c * VEC + k] = widen(v.v[k]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; e++)
                S[q][e] = 0.0f;
        }
    }

    const float a_h = p.A[h * p.A_sh];
    const float d_h = p.D ? p.D[h * p.D_sh] : 0.0f;
    const float bias_h = p.dt_bias ? p.dt_bias[h * p.bias_sh] : 0.0f;
    const IT *const xs = static_cast<const IT *>(p.x);
    const IT *const zs = static_cast<const IT *>(p.z);
    const IT *const Bs = static_cast<const IT *>(p.B);
    const IT *const Cs = static_cast<const IT *>(p.C);
    IT *const ys = static_cast<IT *>(p.out);
    const void *const wtab = p.wtab ? p.wtab : p.rtab;
    const bool w2d = p.wtab ? (flags & kWrite2D) : (flags & kRead2D);
    const bool wi64 = p.wtab ? (flags & kWriteI64) : (flags & kReadI64);
    const int64_t ws0 = p.wtab ? p.w_s0 : p.r_s0;
    const int64_t ws1 = p.wtab ? p.w_s1 : p.r_s1;

    for (int64_t t = 0; t < len; t++) {
        const int64_t r = first_row + t;

        // this lane's dstate columns of B and C
        float Bv[E], Cv[E];
        {
            const IT *bsrc = Bs + r * p.B_sr + static_cast<int64_t>(g) * p.B_sg;
            const IT *csrc = Cs + r * p.C_sr + static_cast<int64_t>(g) * p.C_sg;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const Pack<IT, IVEC> bv =
                    *reinterpret_cast<const Pack<IT, IVEC> *>(bsrc + c * kLanesPerRow * IVEC + col * IVEC);
                const Pack<IT, IVEC> cv =
                    *reinterpret_cast<const Pack<IT, IVEC> *>(csrc + c * kLanesPerRow * IVEC + col * IVEC);
#pragma unroll
                for (int k = 0; k < IVEC; k++) {
                    Bv[c * IVEC + k] = widen(bv.v[k]);
                    Cv[c * IVEC + k] = widen(cv.v[k]);
                }
            }
        }

        // this token's per-row inputs for all of the lane's rows, issued
        // together before any of them is used
        uint32_t xb[PASSES], dtb[PASSES], zb[PASSES];
        const bool dt_f32 = flags & kDtF32;
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d = d0 + q * kRowsPerPass;
            xb[q] = dtb[q] = zb[q] = 0u;
            if (d < p.P) {
                xb[q] = load_bits(xs + r * p.x_sr + h * p.x_sh + d);
                const int64_t di = r * p.dt_sr + h * p.dt_sh + static_cast<int64_t>(d) * p.dt_sp;
                dtb[q] = dt_f32 ? load_bits(static_cast<const float *>(p.dt) + di)
                                : load_bits(static_cast<const IT *>(p.dt) + di);
                if (zs)
                    zb[q] = load_bits(zs + r * p.z_sr + h * p.z_sh + d);
            }
        }
        float xv[PASSES], dtv[PASSES], zv[PASSES];
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            xv[q] = from_bits<IT>(xb[q]);
            dtv[q] = dt_f32 ? __uint_as_float(dtb[q]) : from_bits<IT>(dtb[q]);
            zv[q] = from_bits<IT>(zb[q]);
        }

#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d = d0 + q * kRowsPerPass;
            float v = dtv[q] + bias_h;
            if (flags & kSoftplus)
                v = softplus(v);
            const float decay = expf(v * a_h);
            const float dtx = v * xv[q];
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < E; e++) {
                S[q][e] = fmaf(S[q][e], decay, dtx * Bv[e]);
                acc = fmaf(S[q][e], Cv[e], acc);
            }
            float y = row16_sum(acc) + d_h * xv[q];
            if (zs)
                y *= zv[q] / (1.0f + expf(-zv[q]));
            if (d < p.P && col == 0)
                ys[r * p.out_sr + h * p.out_sh + d] = narrow<IT>(y);
        }

        // store through the token's destination (its own entry of the
        // destination table, else of the read table, else slot b)
        const int64_t wslot =
            wtab ? table_slot(wtab, w2d, wi64, ws0, ws1, b, first_row, t) : b;
        const bool store = !(flags & kDisable) && wslot != p.pad;
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d = d0 + q * kRowsPerPass;
            ST *dst = pool + wslot * p.slot_stride + tile_off + static_cast<int64_t>(d) * N;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                Pack<ST, VEC> v;
#pragma unroll
                for (int k = 0; k < VEC; k++) {
                    v.v[k] = narrow<ST>(S[q][c * VEC + k]);
                    if (MULTI)
                        S[q][c * VEC + k] = widen(v.v[k]);  // carry the stored value
                }
                if (store && d < p.P)
                    *reinterpret_cast<Pack<ST, VEC> *>(dst + c * kLanesPerRow * VEC + col * VEC) = v;
            }
        }
    }
}

template <typename ST, typename IT, bool M>
bool pick_n(int n, KernelRef *k) {
    switch (n) {
#define SSU_CASE(NN)                                                                     \
    case NN:                                                                             \
        k->fn = reinterpret_cast<const void *>(&ssu_kernel<ST, IT, NN, M>);             \
        return true;
        SSU_CASE(16)
        SSU_CASE(32)
        SSU_CASE(64)
        SSU_CASE(128)
        SSU_CASE(256)
#undef SSU_CASE
    }
    return false;
}

template <typename ST>
bool pick_io(int io, int n, bool multi, KernelRef *k) {
    switch (io) {
    case SSU_F32: return multi ? pick_n<ST, float, true>(n, k) : pick_n<ST, float, false>(n, k);
    case SSU_F16: return multi ? pick_n<ST, _Float16, true>(n, k) : pick_n<ST, _Float16, false>(n, k);
    case SSU_BF16: return multi ? pick_n<ST, __bf16, true>(n, k) : pick_n<ST, __bf16, false>(n, k);
    }
    return false;
}

const char *dtype_name(int d) {
    switch (d) {
    case SSU_F32: return "f32";
    case SSU_F16: return "f16";
    case SSU_BF16: return "bf16";
    }
    return "?";
}

}  // namespace

bool find_kernel(int state_dtype, int io_dtype, int dstate, bool multi, KernelRef *out) {
    switch (state_dtype) {
    case SSU_F32: return pick_io<float>(io_dtype, dstate, multi, out);
    case SSU_F16: return pick_io<_Float16>(io_dtype, dstate, multi, out);
    case SSU_BF16: return pick_io<__bf16>(io_dtype, dstate, multi, out);
    }
    return false;
}

void kernel_name(int state_dtype, int io_dtype, int dstate, bool multi, char *buf, int len) {
    snprintf(buf, static_cast<size_t>(len), "%s_%s_%s_n%d", multi ? "ssu_packed" : "ssu_onetoken",
             dtype_name(state_dtype), dtype_name(io_dtype), dstate);
}

const char *hip_error_string(int e) { return hipGetErrorString(static_cast<hipError_t>(e)); }

int launch(const KernelRef &k, const Params &p, unsigned grid, unsigned block, void *stream) {
    Params copy = p;
    void *args[] = {&copy};
    return static_cast<int>(hipLaunchKernel(k.fn, dim3(grid), dim3(block), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

int kernel_attributes(const KernelRef &k, int *vgprs, int *sgprs) {
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, k.fn);
    if (e != hipSuccess)
        return static_cast<int>(e);
    // hipFuncAttributes reports registers per thread as numRegs
    *vgprs = attr.numRegs;
    *sgprs = 0;
    return 0;
}

}  // namespace ssu
