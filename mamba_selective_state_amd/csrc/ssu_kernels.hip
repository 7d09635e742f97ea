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

#include <type_traits>

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

// Streaming accesses of the state pool. Each state byte is touched once per
// call, so the pool's loads and stores carry the non-temporal hint and do not
// displace the per-row inputs (B and C are shared by a group's heads) from
// the caches.
#ifndef SSU_NT_STATE
#define SSU_NT_STATE 1
#endif
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int BYTES> struct RawOf;
template <> struct RawOf<2> { using T = unsigned short; };
template <> struct RawOf<4> { using T = unsigned int; };
template <> struct RawOf<8> { using T = u32x2; };
template <> struct RawOf<16> { using T = u32x4; };

template <typename P>
__device__ __forceinline__ P load_state(const P *src) {
    using R = typename RawOf<sizeof(P)>::T;
    R r = SSU_NT_STATE ? __builtin_nontemporal_load(reinterpret_cast<const R *>(src))
                       : *reinterpret_cast<const R *>(src);
    return __builtin_bit_cast(P, r);
}

template <typename P>
__device__ __forceinline__ void store_state(P *dst, const P &v) {
    using R = typename RawOf<sizeof(P)>::T;
    const R r = __builtin_bit_cast(R, v);
    if (SSU_NT_STATE)
        __builtin_nontemporal_store(r, reinterpret_cast<R *>(dst));
    else
        *reinterpret_cast<R *>(dst) = r;
}

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

// Value of lane Q of the caller's DPP row (lanes 16k .. 16k+15), in every
// lane of that row.
template <int Q>
__device__ __forceinline__ float row16_bcast(float v) {
    static_assert(Q >= 0 && Q < 16, "lane within a row");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + Q, 0xF, 0xF, false));  // row_newbcast
}

__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// Entry of a slot table naming sequence b's position t.
__device__ __forceinline__ int64_t table_slot(const void *tab, bool two_d, bool i64, int64_t s0,
                                              int64_t s1, int64_t b, int64_t first_row, int64_t t) {
    const int64_t i = two_d ? b * s0 + t * s1 : (first_row + t) * s0;
    return load_index(tab, i64, i);
}

// Inputs of one token for the lane: its dstate columns of B and C (raw, in
// the x dtype) and x, dt and z of the dim row whose scalars the lane computes.
template <typename IT, int NCH, int IVEC>
struct TokenInputs {
    Pack<IT, IVEC> b[NCH], c[NCH];
    uint32_t x, dt, z;
};

// Unrolled loop over the passes with the pass index as a constant (DPP
// controls must be immediates).
template <int Q, int PASSES, typename F>
__device__ __forceinline__ void for_passes(F &&f) {
    if constexpr (Q < PASSES) {
        f(std::integral_constant<int, Q>());
        for_passes<Q + 1, PASSES>(f);
    }
}

template <typename ST, typename IT, int N, bool MULTI>
__global__ __launch_bounds__(kMaxWaves *kWaveLanes) void ssu_kernel(const Params p) {
    constexpr int E = N / kLanesPerRow;  // state elements per lane per row
    constexpr int VEC = (16 / (int)sizeof(ST)) < E ? (16 / (int)sizeof(ST)) : E;
    constexpr int NCH = E / VEC;         // accesses per lane per row
    constexpr int PASSES = passes_for(N, sizeof(ST), MULTI);
    constexpr int IVEC = VEC;            // B / C are read with the same column split
    static_assert(E * kLanesPerRow == N && NCH * VEC == E, "dstate split");
    static_assert(PASSES <= kLanesPerRow, "one scalar-owning lane per pass");
    using SPack = Pack<ST, VEC>;
    using Inputs = TokenInputs<IT, NCH, IVEC>;

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
    // Pass q covers dim rows dw + 4q + rsub. The per-row scalars of pass q
    // (decay, dt' x, the gate and y) are computed once, by lane col == q of
    // each row group: the lane's "own" row is dw + 4 col + rsub.
    const int dw = tile * p.rows_per_block + wave * (kRowsPerPass * PASSES);
    const int d_own = dw + col * kRowsPerPass + rsub;
    const bool owner = col < PASSES && d_own < p.P;

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

    // The lane's part of the tile, kept in the state dtype: what is stored is
    // also what the next token starts from. The pad id reads as zeros.
    SPack S[PASSES][NCH];
    const bool read_pad = rslot == p.pad;
    const ST *const rbase = pool + rslot * p.slot_stride + tile_off;
#pragma unroll
    for (int q = 0; q < PASSES; q++) {
        const int d = dw + q * kRowsPerPass + rsub;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            if (!read_pad && d < p.P) {
                S[q][c] = load_state(reinterpret_cast<const SPack *>(
                    rbase + static_cast<int64_t>(d) * N + c * kLanesPerRow * VEC + col * VEC));
            } else {
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    S[q][c].v[k] = narrow<ST>(0.0f);
            }
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
    const bool dt_f32 = flags & kDtF32;
    const void *const wtab = p.wtab ? p.wtab : p.rtab;
    const bool w2d = p.wtab ? (flags & kWrite2D) : (flags & kRead2D);
    const bool wi64 = p.wtab ? (flags & kWriteI64) : (flags & kReadI64);
    const int64_t ws0 = p.wtab ? p.w_s0 : p.r_s0;
    const int64_t ws1 = p.wtab ? p.w_s1 : p.r_s1;

    // issue the loads of row r's inputs (no use before the next wait)
    auto fetch = [&](int64_t r, Inputs &in) {
        const IT *bsrc = Bs + r * p.B_sr + static_cast<int64_t>(g) * p.B_sg + col * IVEC;
        const IT *csrc = Cs + r * p.C_sr + static_cast<int64_t>(g) * p.C_sg + col * IVEC;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            in.b[c] = *reinterpret_cast<const Pack<IT, IVEC> *>(bsrc + c * kLanesPerRow * IVEC);
            in.c[c] = *reinterpret_cast<const Pack<IT, IVEC> *>(csrc + c * kLanesPerRow * IVEC);
        }
        in.x = in.dt = in.z = 0u;
        if (owner) {
            in.x = load_bits(xs + r * p.x_sr + h * p.x_sh + d_own);
            const int64_t di = r * p.dt_sr + h * p.dt_sh + static_cast<int64_t>(d_own) * p.dt_sp;
            in.dt = dt_f32 ? load_bits(static_cast<const float *>(p.dt) + di)
                           : load_bits(static_cast<const IT *>(p.dt) + di);
            if (zs)
                in.z = load_bits(zs + r * p.z_sr + h * p.z_sh + d_own);
        }
    };

    Inputs cur;
    fetch(first_row, cur);
    for (int64_t t = 0; t < len; t++) {
        const int64_t r = first_row + t;
        // the next token's inputs are requested before this token's stores,
        // so waiting for them later does not wait for the stores
        Inputs nxt;
        if (MULTI && t + 1 < len)
            fetch(r + 1, nxt);

        float Bv[E], Cv[E];
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int k = 0; k < IVEC; k++) {
                Bv[c * IVEC + k] = widen(cur.b[c].v[k]);
                Cv[c * IVEC + k] = widen(cur.c[c].v[k]);
            }

        // scalars of the lane's own row
        const float xv = from_bits<IT>(cur.x);
        float v = (dt_f32 ? __uint_as_float(cur.dt) : from_bits<IT>(cur.dt)) + bias_h;
        if (flags & kSoftplus)
            v = softplus(v);
        const float decay = expf(v * a_h);
        const float dtx = v * xv;

        // destination: the token's own entry of the destination table, else
        // of the read table, else slot b
        const int64_t wslot =
            wtab ? table_slot(wtab, w2d, wi64, ws0, ws1, b, first_row, t) : b;
        const bool store = !(flags & kDisable) && wslot != p.pad;
        ST *const wbase = pool + wslot * p.slot_stride + tile_off;

        float ysum = 0.0f;
        for_passes<0, PASSES>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int d = dw + q * kRowsPerPass + rsub;
            const float dq = row16_bcast<q>(decay);
            const float tq = row16_bcast<q>(dtx);
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
#pragma unroll
                for (int k = 0; k < VEC; k++) {
                    const int e = c * VEC + k;
                    const float s = fmaf(widen(S[q][c].v[k]), dq, tq * Bv[e]);
                    acc = fmaf(s, Cv[e], acc);
                    S[q][c].v[k] = narrow<ST>(s);  // the stored and carried value
                }
            }
            const float sum = row16_sum(acc);
            ysum = col == q ? sum : ysum;
            if (store && d < p.P) {
                ST *dst = wbase + static_cast<int64_t>(d) * N + col * VEC;
#pragma unroll
                for (int c = 0; c < NCH; c++)
                    store_state(reinterpret_cast<SPack *>(dst + c * kLanesPerRow * VEC), S[q][c]);
            }
        });

        // y of the lane's own row
        if (owner) {
            float y = ysum + d_h * xv;
            if (zs) {
                const float zv = from_bits<IT>(cur.z);
                y *= zv / (1.0f + expf(-zv));
            }
            ys[r * p.out_sr + h * p.out_sh + d_own] = narrow<IT>(y);
        }
        if (MULTI)
            cur = nxt;
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
