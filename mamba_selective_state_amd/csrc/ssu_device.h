// Device helpers shared by the gfx950 kernels of libssu (ssu_kernels.hip and
// ssu_replay.hip): element conversions, 16-byte state accesses, DPP row
// reductions and broadcasts, the per-row transcendentals, the XCD-aware
// workgroup order, slot-table reads, raw input words and the MXFP8 and
// MXFP4 codecs.
#pragma once

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
// call, so the pool's loads carry the non-temporal hint and do not displace
// the per-row inputs (B and C are shared by a group's heads) from the caches.
// The store hint is chosen per kernel: measured on this part, non-temporal
// stores win for in-place read-modify-write streams, and plain stores for
// write-mostly streams.
#ifndef SSU_NT_LOAD
#define SSU_NT_LOAD 1
#endif
#ifndef SSU_NT_STORE
#define SSU_NT_STORE 1
#endif
#ifndef SSU_NT_STORE_MULTI
#define SSU_NT_STORE_MULTI 1
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
    R r = SSU_NT_LOAD ? __builtin_nontemporal_load(reinterpret_cast<const R *>(src))
                      : *reinterpret_cast<const R *>(src);
    return __builtin_bit_cast(P, r);
}

template <bool NT, typename P>
__device__ __forceinline__ void store_state(P *dst, const P &v) {
    using R = typename RawOf<sizeof(P)>::T;
    const R r = __builtin_bit_cast(R, v);
    if constexpr (NT)
        __builtin_nontemporal_store(r, reinterpret_cast<R *>(dst));
    else
        *reinterpret_cast<R *>(dst) = r;
}

__device__ __forceinline__ int64_t load_index(const void *base, bool i64, int32_t i) {
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

// Largest value over each aligned group of LANES lanes (2, 4, 8 or 16) of a
// DPP row, in every lane of the group (same steps as row16_sum).
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
    static_assert(LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "a DPP row splits in powers of two");
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    if constexpr (LANES >= 4)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    if constexpr (LANES >= 8)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    if constexpr (LANES >= 16)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// Value of lane Q of the caller's DPP row (lanes 16k .. 16k+15), in every
// lane of that row.
template <int Q>
__device__ __forceinline__ float row16_bcast(float v) {
    static_assert(Q >= 0 && Q < 16, "lane within a row");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + Q, 0xF, 0xF, false));  // row_newbcast
}

// Per-row scalars use the hardware base-2 exponential, logarithm and
// reciprocal (a few ulps each). Their errors stay far inside the update's
// error budget: a relative error e in dt' or in the decay moves
// S * exp(dt' A) by at most |S| x exp(-x) e <= 0.37 |S| e (x = |dt' A|), and
// the rank-1 term by e |dt' x B|. exp(0) is exactly 1, so dt = 0 keeps the
// state bit for bit.
__device__ __forceinline__ float exp_hw(float v) {
    return __builtin_amdgcn_exp2f(v * 1.44269504088896341f);
}

// log(1 + e^v), e^v itself above v = 20 (the difference is below half an
// ulp there). log1p(u) = log(w) * u / (w - 1) with w = 1 + u keeps the
// relative accuracy for small u (w - 1 is exact).
__device__ __forceinline__ float softplus(float v) {
    const float u = exp_hw(v);
    const float w = 1.0f + u;
    const float l = __builtin_amdgcn_logf(w) * 0.693147180559945309f;
    const float r = w == 1.0f ? u : l * (u * __builtin_amdgcn_rcpf(w - 1.0f));
    return v > 20.0f ? v : r;
}

// z * sigmoid(z)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + exp_hw(-z)); }

// Workgroups are dispatched to the 8 XCDs round-robin (id % 8), each XCD with
// its own L2. Consecutive logical work units (the dim tiles of one head, the
// heads of one group) read the same lines of x, dt, z, B and C. With a
// cluster size K > 0, each block of 8K consecutive ids gives XCD x the K
// consecutive logical units K x .. K x + K - 1 of that block (the last,
// partial block maps to itself), so such units share an L2 while the grid
// still sweeps the pool in order.
#ifndef SSU_XCD_CLUSTER
#define SSU_XCD_CLUSTER 16
#endif
constexpr int kXcds = 8;
__device__ __forceinline__ int32_t xcd_clustered_index(int32_t id, int32_t n) {
    constexpr int32_t K = SSU_XCD_CLUSTER;
    if constexpr (K == 0) {
        return id;
    } else {
        constexpr int32_t block = kXcds * K;
        const int32_t m = id / block;
        if ((m + 1) * block > n)
            return id;
        const int32_t r = id % block;
        return m * block + (r % kXcds) * K + r / kXcds;
    }
}

// Entry of a slot table naming sequence b's position t.
__device__ __forceinline__ int64_t table_slot(const void *tab, bool two_d, bool i64, int32_t s0,
                                              int32_t s1, int32_t b, int32_t first_row, int32_t t) {
    const int32_t i = two_d ? b * s0 + t * s1 : (first_row + t) * s0;
    return load_index(tab, i64, i);
}

// Inputs of one token for the lane: its dstate columns of B and C (raw, in
// the x dtype) and x, dt and z of the dim row whose scalars the lane computes.
// Raw 32-bit words of one B or C access (IVEC elements of the x dtype), kept
// unconverted until they are used.
template <typename IT, int IVEC>
struct RawWords {
    static constexpr int kBytes = IVEC * (int)sizeof(IT);
    static constexpr int kWords = kBytes < 4 ? 1 : kBytes / 4;
    uint32_t w[kWords];
};

template <typename IT, int IVEC>
__device__ __forceinline__ RawWords<IT, IVEC> load_words(const IT *src) {
    RawWords<IT, IVEC> r;
    constexpr int kBytes = RawWords<IT, IVEC>::kBytes;
    if constexpr (kBytes <= 2) {
        r.w[0] = *reinterpret_cast<const uint16_t *>(src);
    } else if constexpr (kBytes <= 16) {
        using R = typename RawOf<kBytes>::T;
        const R v = *reinterpret_cast<const R *>(src);
        r = __builtin_bit_cast(RawWords<IT, IVEC>, v);
    } else {
#pragma unroll
        for (int i = 0; i < kBytes / 16; i++) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(src)[i];
            r.w[4 * i] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    }
    return r;
}

// Stores a RawWords block as loaded (exactly IVEC elements).
template <typename IT, int IVEC>
__device__ __forceinline__ void store_words(IT *dst, const RawWords<IT, IVEC> &r) {
    constexpr int kBytes = RawWords<IT, IVEC>::kBytes;
    if constexpr (kBytes <= 2) {
        *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(r.w[0]);
    } else if constexpr (kBytes <= 16) {
        using R = typename RawOf<kBytes>::T;
        *reinterpret_cast<R *>(dst) = __builtin_bit_cast(R, r);
    } else {
#pragma unroll
        for (int i = 0; i < kBytes / 16; i++)
            reinterpret_cast<u32x4 *>(dst)[i] = u32x4{r.w[4 * i], r.w[4 * i + 1], r.w[4 * i + 2], r.w[4 * i + 3]};
    }
}

// element k of a RawWords block, widened to fp32
template <typename IT, int IVEC>
__device__ __forceinline__ float word_elem(const RawWords<IT, IVEC> &r, int k) {
    if constexpr (sizeof(IT) == 4)
        return __uint_as_float(r.w[k]);
    else {
        const uint32_t word = r.w[k / 2];
        return from_bits<IT>((k & 1) ? (word >> 16) : (word & 0xFFFFu));
    }
}

// Inputs of one token for the lane, as loaded (raw bits): its dstate columns
// of B and C, and x, z, dt of the dim row whose scalars it computes (dt in
// two 16-bit halves, the high one used for fp32 dt), and the destination
// table entry (two words, the high one used for i64 tables).
template <typename IT, int NCH, int IVEC>
struct TokenInputs {
    using Bits = std::conditional_t<sizeof(IT) == 2, uint16_t, uint32_t>;
    RawWords<IT, IVEC> b[NCH], c[NCH];
    Bits x, z;
    uint16_t dt_lo, dt_hi;
    uint32_t ws_lo, ws_hi;
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


// MXFP8 (OCP Microscaling, E4M3 elements, E8M0 scale per 32 values) for the
// checkpoint's read copy. A block's scale is 2^k with k = floor(log2 max|x|)
// - 8 clamped to [-126, 127] (-126 for a block of zeros); elements x 2^-k
// round to nearest even in E4M3 and saturate at 448.
__device__ __forceinline__ float mx8_scale(uint32_t byte) {
    return byte ? __uint_as_float(byte << 23) : 0x1p-127f;
}

// Two E4M3 codes (bytes 2*HI and 2*HI + 1 of `codes`) times the scale: the
// conversion unit decodes the OCP format (NaN codes to NaN) and applies the
// power-of-two scale exactly, fp32 subnormal results included.
template <bool HI>
__device__ __forceinline__ float2 e4m3_pair(uint32_t codes, float scale) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, scale, HI);
    return float2{v[0], v[1]};
}

// E4M3 codes of v[0..3] / 2^k, packed byte i = value i. The conversion unit
// divides by the power-of-two scale and rounds to nearest even; it turns a
// quotient beyond the largest finite value into NaN, so the inputs are first
// clamped to +-448 * 2^k (saturation), and a NaN input is given code 0x7F.
__device__ __forceinline__ uint32_t e4m3_codes4(const float v[4], int k) {
    const float X = __uint_as_float(static_cast<uint32_t>(k + 127) << 23);
    const float lim = 448.0f * X;  // infinite for k = 127: no value reaches it
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        c[i] = v[i] != v[i] ? 0.0f : fminf(fmaxf(v[i], -lim), lim);
    typedef short short2_t __attribute__((ext_vector_type(2)));
    short2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c[0], c[1], X, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c[2], c[3], X, true);
    uint32_t codes = static_cast<uint32_t>(static_cast<uint16_t>(r[0])) |
                     (static_cast<uint32_t>(static_cast<uint16_t>(r[1])) << 16);
#pragma unroll
    for (int i = 0; i < 4; i++)
        codes = v[i] != v[i] ? (codes & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i)) : codes;
    return codes;
}

// scale exponent of a block from its largest magnitude
__device__ __forceinline__ int mx8_exponent(float amax) {
    const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
    if (ex == 0)
        return -126;  // zero or subnormal
    const int k = ex - 127 - 8;
    return k < -126 ? -126 : (k > 127 ? 127 : k);
}

// MXFP4 (OCP Microscaling, FP4 E2M1 elements two a byte -- the even
// element in the low nibble -- and an E8M0 scale per 32 values) for the
// checkpoint's 4-bit read copy. A block's scale is 2^k with k =
// floor(log2 max|x|) - 2 clamped to [-126, 127] (-126 for a block of zeros);
// elements x 2^-k round to nearest even in E2M1 and saturate at 6.

// The two E2M1 elements of byte BYTE of `codes`, times the scale (the
// conversion unit decodes the low nibble first and applies the power-of-two
// scale exactly).
template <int BYTE>
__device__ __forceinline__ float2 e2m1_pair(uint32_t codes, float scale) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, BYTE);
    return float2{v[0], v[1]};
}

// E2M1 codes of v[0..3] / 2^k in the low 16 bits: byte 0 holds v[0] (low
// nibble) and v[1], byte 1 v[2] and v[3]. The conversion unit divides by the
// power-of-two scale, rounds to nearest even and saturates at 6 (checked on
// the device at scale exponents from -126 to 127 against a plain E2M1
// rounding); it gives a NaN input the code of 6, which is set to 0 here.
__device__ __forceinline__ uint32_t e2m1_codes4(const float v[4], int k) {
    const float X = __uint_as_float(static_cast<uint32_t>(k + 127) << 23);
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], X, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], X, 1);
#pragma unroll
    for (int i = 0; i < 4; i++)
        r = v[i] != v[i] ? r & ~(0xFu << (4 * i)) : r;
    return r & 0xFFFFu;
}

// scale exponent of an MXFP4 block from its largest magnitude
__device__ __forceinline__ int mx4_exponent(float amax) {
    const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
    if (ex == 0)
        return -126;  // zero or subnormal
    const int k = ex - 127 - 2;
    return k < -126 ? -126 : (k > 127 ? 127 : k);
}

}  // namespace
}  // namespace ssu
