// SSD packed variable-length prefill for gfx950 (MATE docs, "Mamba / SSU",
// section "SSD packed prefill"): the same recurrence as the decode step over
// every token of a packed batch, computed chunk by chunk. The page's five
// stages (dt' and the decay cumsum, the chunks' own states, the state
// passing, C.B^T and the chunk scan) run in one kernel, after a small one
// that clears its synchronisation words:
//   ssd_prep_kernel   clears the ticket counters and the chain flags and
//                     maps each chunk to the sequence whose returned state
//                     it gives (last_chunk_indices);
//   ssd_fused_kernel  per (chunk, group, 4 heads): dt' (softplus,
//                     dt_limit), the cumsum, C.B^T, the chunk's own state
//                     sum_t exp(A_end - A_t) dt'_t x_t B_t^T, and
//                     y_t = sum_{s<=t} (C_t . B_s) exp(A_t - A_s) dt'_s x_s
//                           + exp(A_t) C_t . S_in + D x_t, gated by
//                     silu(z_t) (MFMA). The entering state S_in is the
//                     state the chunk before in the sequence leaves,
//                     S_out = exp(A_end) S_in + own state: that chunk's
//                     workgroup publishes it (fp32) with a flag, this one
//                     waits for the flag. The state passing is a chain
//                     through the workgroups of one (group, 4 heads) stream
//                     in chunk order; nothing else of a chunk leaves its
//                     workgroup.
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


// ---- synchronisation of the chain
//
// Order of work: the workgroups of virtual XCD v (blockIdx % 8: the
// hardware's round-robin placement, so that a stream's chunks share one L2)
// take tickets from counter v in the order they start; ticket k is chunk
// k / n_v of stream lo_v + k % n_v, the streams lo_v .. lo_v + n_v - 1 being
// v's. The chunk a workgroup waits for is of its own stream, so it holds a
// smaller ticket of the same counter: its workgroup has started, and by
// induction on the ticket every wait ends (a chunk that opens its sequence
// waits for nothing). The spin is bounded besides: after kSpinMax polls a
// workgroup goes on without the state.
//
// Publication: the chain state is written and read with device-scope (sc1)
// buffer accesses, coherent across the XCDs' L2s. Every wave waits for its
// stores to complete before the workgroup barrier, after which one lane
// writes the flag with a device-scope store. A waiting workgroup's first lane
// polls the flag with device-scope loads; the barrier after the poll orders
// every wave's state loads after it.

constexpr int kXcds = 8;
constexpr int kSpinMax = 1 << 20;
constexpr int kDeviceScope = 16;      // buffer cache policy: sc1
constexpr int kWaitStores = 0x0F70;   // s_waitcnt vmcnt(0)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// One workgroup maps chunks to the sequences whose returned state they give
// and clears the ticket counters; the others clear the chain flags.
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void ssd_prep_kernel(const SsdParams sp) {
    if (blockIdx.x == 0) {
        if (threadIdx.x < kXcds)
            sp.ws_tickets[threadIdx.x] = 0;
        if (!sp.intermediate) {
            for (int64_t c = threadIdx.x; c < sp.nchunks; c += kPrepThreads)
                sp.ws_owner[c] = -1;
            __syncthreads();
            for (int64_t b = threadIdx.x; b < sp.batch; b += kPrepThreads) {
                const int64_t c = idx_at(sp.last_chunk, sp.last_chunk_i64, b * sp.last_chunk_s);
                if (c >= 0 && c < sp.nchunks)
                    sp.ws_owner[c] = static_cast<int>(b);
            }
        }
        return;
    }
    const int64_t nflags = sp.nchunks * sp.H;
    for (int64_t i = (blockIdx.x - 1) * static_cast<int64_t>(kPrepThreads) + threadIdx.x; i < nflags;
         i += (gridDim.x - 1) * static_cast<int64_t>(kPrepThreads))
        sp.ws_flags[i] = 0;
}

// ---- the fused kernel
//
// One workgroup of 8 waves per (chunk, group, block of kFHeads heads of the
// group). Phases:
//  1. loads: B rows (lane items: a pair of rows, one 16-byte piece), the C
//     row of each of the lane's two tokens, dt of the lane's heads for token
//     t % 256, the first head's x; dt' and the cumsums of all heads (wave
//     scans, the wave totals through LDS); B rows and x^T to LDS.
//  2. C.B^T: rows t in 16-row tiles (wave w takes tiles w and 15 - w: equal
//     work under the causal mask), columns s in 32-column blocks J; each wave
//     forms its 9 (block, tile) pairs once, in registers (fp32), for all
//     heads. Meanwhile the per-head factors go to LDS.
//  3. B^T replaces the B rows in LDS (the chunk state's operand).
//  4. per head: the own state^T [n][p] = B^T (w x)^T (wave w: p tile w / 2,
//     half of the n tiles; lane: 4 consecutive n of one p); the part of y
//     within the chunk (the scaled C.B^T times x) plus D x; then the wait for
//     the entering state, the chain step (S_out stored for the next chunk,
//     or as a returned state), the entering state to LDS, its part of y
//     (S_in C^T scaled by exp(A_t)), the gate and the store.
// Both products of y are formed transposed, so that a lane owns one token t:
//   (B_J C^T)[s][t]: the lane holds t and the 8 columns s = 32J + 4g + i,
//   32J + 16 + 4g + i (g = lane / 16, i < 4), which after scaling is the
//   B operand of y^T += x_J^T (...)^T with that k order (the x side reads
//   the same columns); nothing goes back through LDS;
//   y^T[p][t]: MFMA row m of p tile pt is p = 16 (m / 4) + 4 pt + m % 4, so
//   the lane ends with the 16 consecutive p = 16g .. 16g + 15 of its token
//   (two 16-byte stores, loads of z alike).
// The own state uses the same k order over tokens and the same p map (its
// MFMA column r is p = 16 (r / 4) + r % 4 + 4 pt).
// Dim p is stored at LDS row 4 (p % 16) + p / 16 of x^T (the entering state
// in MFMA-row order, sin_row): the 16 rows an operand read touches are then
// consecutive; with 142-word x^T rows and 130-word B^T rows the 16 lanes of
// an 8-byte read pass hit distinct banks of the 32.
// Below the diagonal block the decay factors into a row and a column term,
// exp(A_t - A_s) dt'_s = exp(A_t - A_J) * exp(A_J - A_s) dt'_s with A_J the
// cumsum at the block's last token; both are at most 1 there (the cumsum
// does not increase). The diagonal block takes the exact factor per element
// under the causal mask.
constexpr int kFThreads = 512;
constexpr int kFHeads = kSsdHeads;  // heads per workgroup
constexpr int kHPL = kFHeads > 1 ? kFHeads / 2 : 1;  // heads whose dt' a lane forms (two halves of 256 lanes)
// head j of the lane's heads; with one head both halves form it (and store the same values)
__device__ __forceinline__ int lane_head(int half, int j) { return kFHeads > 1 ? kHPL * half + j : 0; }
constexpr int kFTiles = 2;      // 16-token tiles per wave
constexpr int kFSlots = 9;      // (block, tile) pairs of a wave: (w / 2 + 1) + ((15 - w) / 2 + 1)
constexpr int kXsRow = kL + 28; // x^T row stride (elements): 142 words
constexpr int kBtRow = kL + 4;  // B^T row stride (elements): 130 words

__device__ __forceinline__ int dim_row(int p) { return 4 * (p & 15) + (p >> 4); }
// Row of dim p in the entering state's LDS copy: 16 pt + r for p = 16 (r / 4)
// + r % 4 + 4 pt, so that the 16 rows of an operand read are in MFMA-row
// order (16-byte reads by 8 lanes hit distinct banks with 68-word rows)
__device__ __forceinline__ int sin_row(int p) { return 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

template <typename T> struct alignas(4 * sizeof(T)) Vec4 { T v[4]; };  // one 8- or 16-byte access

template <typename IT, typename ST, int N>
__global__ __launch_bounds__(kFThreads) void ssd_fused_kernel(const SsdParams sp) {
    using M = Mfma<IT>;
    using V = typename M::V;
    constexpr int KN = N / 32;                                // k steps over dstate
    constexpr int KNT = N / 32;                               // n tiles per wave of the own state
    constexpr int kPieces = N / 8;                            // 16-byte pieces of a B row
    constexpr int kPairs = kL / 2;                            // pairs of B rows
    constexpr int kBItems = kPairs * kPieces / kFThreads;     // (row pair, piece) items per lane
    // Item i: pieces i % 8 + 8 ((i / 8) / kPairs) of row pair (i / 8) % kPairs,
    // so 8 consecutive lanes read a row's whole 128-byte line (consecutive
    // pairs per lane read 64 rows per load instruction: 3.8% slower), and
    // the B^T stores of a pass meet at most 2 to a bank.
    static_assert(kPieces % 8 == 0, "whole lines of 8 pieces");
    auto b_pair = [](int i) { return (i / 8) % kPairs; };
    auto b_piece = [](int i) { return i % 8 + 8 * ((i / 8) / kPairs); };
    constexpr int kBRowsElems = kL * (N + kPad), kBtElems = N * kBtRow;
    constexpr int64_t PN = static_cast<int64_t>(kP) * N;
    static_assert(kP == 64 && kL == 256 && kFThreads == 512, "8 waves of two 16-token tiles, 4 p tiles");
    static_assert(kBItems * kFThreads == kPairs * kPieces, "whole items per lane");
    __shared__ float wave_tot[kFHeads][kL / 64];
    __shared__ float total_s[kFHeads];
    __shared__ __attribute__((aligned(16))) float acum_s[kFHeads][kL];
    __shared__ __attribute__((aligned(16))) float dtp_s[kFHeads][kL];
    __shared__ __attribute__((aligned(16))) float q_s[kFHeads][kL];  // exp(A_J - A_t) dt'_t, J = t / 32
    __shared__ __attribute__((aligned(16))) float w_s[kFHeads][kL];  // exp(A_end - A_t) dt'_t
    __shared__ __attribute__((aligned(16))) IT Xs[kP][kXsRow];       // x^T of the current head: [dim row][s]
    __shared__ __attribute__((aligned(16))) IT Bm[kBRowsElems > kBtElems ? kBRowsElems : kBtElems];
    __shared__ __attribute__((aligned(16))) IT Sin[kP][N + kPad];    // the entering state: [dim row][n]
    __shared__ int ticket_s;
    IT(*const Bs)[N + kPad] = reinterpret_cast<IT(*)[N + kPad]>(Bm);  // B rows [s][n]
    IT(*const Bt)[kBtRow] = reinterpret_cast<IT(*)[kBtRow]>(Bm);      // B^T [n][s], after C.B^T

    const int t = threadIdx.x;
    const int vx = blockIdx.x % kXcds;
    if (t == 0)
        ticket_s = atomicAdd(sp.ws_tickets + vx, 1);
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(ticket_s);
    const int nstream = static_cast<int>(sp.H / sp.hpg) * sp.nhb;
    const int lo = vx * sp.streams_per_xcd;
    const int cnt = nstream - lo < sp.streams_per_xcd ? nstream - lo : sp.streams_per_xcd;
    if (cnt <= 0 || ticket >= sp.nchunks * cnt)
        return;  // uniform
    const int64_t c = ticket / cnt;
    const int stream = lo + ticket % cnt;
    const int g = stream / sp.nhb, hb = stream % sp.nhb;
    const int h0 = g * sp.hpg + hb * kFHeads;
    const int nh = sp.hpg - hb * kFHeads < kFHeads ? sp.hpg - hb * kFHeads : kFHeads;

    int64_t t0;
    int len;
    chunk_range(sp, c, &t0, &len);
    // the same for every lane: keep them (and what depends on them) scalar
    len = __builtin_amdgcn_readfirstlane(len);
    t0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(t0 >> 32))) << 32 |
         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(t0)));
    // where the entering state comes from, and who takes the leaving one:
    // seq_idx decides which chunks open a sequence
    const int64_t seq = idx_at(sp.seq_idx, sp.seq_idx_i64, c * sp.seq_idx_s);
    const bool opens = c == 0 || idx_at(sp.seq_idx, sp.seq_idx_i64, (c - 1) * sp.seq_idx_s) != seq;
    const bool feeds = c + 1 < sp.nchunks && idx_at(sp.seq_idx, sp.seq_idx_i64, (c + 1) * sp.seq_idx_s) == seq;
    const int owner = sp.intermediate ? -1 : sp.ws_owner[c];
    const bool has_init = sp.init && seq >= 0 && seq < sp.batch;

    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform per wave
    const int r = lane & 15, gq = lane >> 4, g4 = 4 * gq, k8 = 8 * gq;
    const int ntiles = (len + 15) / 16;
    const int rts[kFTiles] = {wv, 15 - wv};
    // a B or C row past the chunk repeats its last row (token 0 for an empty chunk)
    auto row_tok = [&](int i) -> int64_t { return len == 0 ? 0 : t0 + (i < len ? i : len - 1); };

    // ---- 1. loads in the order they are waited on: dt, B, the first head's x, C
    // the wave's heads kHPL half + j (uniform per wave), token t % 256
    const int tk = t & (kL - 1), half = wv >> 2, wq = wv & 3;
    float Ah[kHPL], biash[kHPL];
    uint32_t dtr[kHPL];
#pragma unroll
    for (int j = 0; j < kHPL; j++) {
        const int hk = lane_head(half, j);
        const int hh = (hk < nh ? h0 + hk : h0) / sp.hsplit;
        Ah[j] = sp.A[hh * sp.A_sh];
        biash[j] = sp.dt_bias ? sp.dt_bias[hh * sp.bias_sh] : 0.0f;
        dtr[j] = raw_dt<IT>(sp, tk < len ? t0 + tk : 0, hh);
    }
    V bv[kBItems][2];
    {
        const IT *Bg = static_cast<const IT *>(sp.B) + g * sp.B_sg;
#pragma unroll
        for (int u = 0; u < kBItems; u++) {
            const int item = u * kFThreads + t, pair = b_pair(item), pc = b_piece(item);
#pragma unroll
            for (int v = 0; v < 2; v++)
                bv[u][v] = *reinterpret_cast<const V *>(Bg + row_tok(2 * pair + v) * sp.B_st + 8 * pc);
        }
    }
    // x^T of a head: lane t holds the 16-byte dim piece t % 8 of tokens 2j,
    // 2j + 1, j = t / 8 and j + 64
    struct XIn {
        V xv[2][2];
    };
    const int pc8 = 8 * (t & 7);
    auto load_x = [&](int h, XIn &in) {
        const IT *xs = static_cast<const IT *>(sp.x) + head_off(sp, h, sp.x_sh) + pc8;
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int v = 0; v < 2; v++) {
                const int tok = 2 * ((t >> 3) + 64 * u) + v;
                in.xv[u][v] = *reinterpret_cast<const V *>(xs + (tok < len ? t0 + tok : 0) * sp.x_st);
            }
    };
    auto store_x = [&](const XIn &in) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int j2 = 2 * ((t >> 3) + 64 * u);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const IT lo_ = j2 < len ? in.xv[u][0][e] : static_cast<IT>(0.0f);
                const IT hi_ = j2 + 1 < len ? in.xv[u][1][e] : static_cast<IT>(0.0f);
                *reinterpret_cast<uint32_t *>(&Xs[dim_row(pc8 + e)][j2]) =
                    static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo_)) |
                    (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi_)) << 16);
            }
        }
    };
    {
        XIn first;
        load_x(h0, first);
#pragma unroll
        for (int u = 0; u < kBItems; u++) {
            const int item = u * kFThreads + t, pair = b_pair(item), pc = b_piece(item);
#pragma unroll
            for (int v = 0; v < 2; v++)
                *reinterpret_cast<V *>(&Bs[2 * pair + v][8 * pc]) = bv[u][v];
        }
        store_x(first);
    }
    V ac[kFTiles][KN];  // the C row of the lane's token in each tile
#pragma unroll
    for (int i = 0; i < kFTiles; i++) {
        const IT *crow = static_cast<const IT *>(sp.C) + g * sp.C_sg + row_tok(16 * rts[i] + r) * sp.C_st;
#pragma unroll
        for (int k = 0; k < KN; k++)
            ac[i][k] = *reinterpret_cast<const V *>(crow + 32 * k + k8);
    }
    // dt' and the inclusive prefix sum of dt' A of the lane's two heads:
    // within each wave, then the wave totals through LDS
    float dtp2[kHPL], acum2[kHPL];
#pragma unroll
    for (int j = 0; j < kHPL; j++) {
        const int hk = lane_head(half, j);
        dtp2[j] = tk < len ? processed_dt(sp, dt_value<IT>(sp, dtr[j]), biash[j]) : 0.0f;
        acum2[j] = wave_inclusive_sum(dtp2[j] * Ah[j], lane);
        if (lane == 63)
            wave_tot[hk][wq] = acum2[j];
    }
    __syncthreads();  // B rows, x^T, the wave totals

    // ---- 2. the per-head factors, and C.B^T
#pragma unroll
    for (int j = 0; j < kHPL; j++) {
        const int hk = lane_head(half, j);
        // the chunk's total, summed in the order of the last token's cumsum
        // (padding adds nothing)
        float a = acum2[j];
        float total = wave_tot[hk][kL / 64 - 1];
#pragma unroll
        for (int k = 0; k < kL / 64; k++) {
            const float wt = wave_tot[hk][k];
            a += k < wq ? wt : 0.0f;
            total += k < kL / 64 - 1 ? wt : 0.0f;
        }
        const float aj = __shfl(a, lane | 31, 64);  // the cumsum at the token's 32-block end
        acum_s[hk][tk] = a;
        dtp_s[hk][tk] = dtp2[j];
        q_s[hk][tk] = exp_f(aj - a) * dtp2[j];
        w_s[hk][tk] = tk < len ? exp_f(total - a) * dtp2[j] : 0.0f;
        if (tk == 0)
            total_s[hk] = total;
    }
    const int rt0 = rts[0], rt1 = rts[1];
    const int nj0 = rt0 >> 1, nj1 = rt1 >> 1;
    const bool act0 = rt0 < ntiles, act1 = rt1 < ntiles;  // uniform; act1 implies act0
    const int tt0 = 16 * rt0 + r, tt1 = 16 * rt1 + r;     // the lane's tokens
    // The wave's (block, tile) slots: tile rt0 = wv keeps block J in slot J
    // (J = 0 .. nj0, its diagonal block nj0 = rt0 / 2 <= 3), tile
    // rt1 = 15 - wv block J in slot 8 - J (J = 0 .. nj1, nj1 = rt1 / 2 =
    // 7 - nj0): slots nj0 + 1 .. 8, and every slot index a constant.
    auto bc = [&](int J, const V (&acv)[KN], f32x4 (&d)[2]) {
        d[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        d[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KN; k++) {
            d[0] = M::run(*reinterpret_cast<const V *>(&Bs[32 * J + r][32 * k + k8]), acv[k], d[0]);
            d[1] = M::run(*reinterpret_cast<const V *>(&Bs[32 * J + 16 + r][32 * k + k8]), acv[k], d[1]);
        }
    };
    f32x4 cb[kFSlots][2];
#pragma unroll
    for (int q = 0; q < kFSlots; q++)
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
    __syncthreads();  // every read of the B rows is done; the factors are in LDS

    // ---- 3. B^T over the B rows: pairs of tokens per 32-bit store
#pragma unroll
    for (int u = 0; u < kBItems; u++) {
        const int item = u * kFThreads + t, pair = b_pair(item), pc = b_piece(item);
#pragma unroll
        for (int e = 0; e < 8; e++) {
            // the elements by value: a bit cast of a vector element in place
            // reads element 0
            const IT lo_ = bv[u][0][e], hi_ = bv[u][1][e];
            *reinterpret_cast<uint32_t *>(&Bt[8 * pc + e][2 * pair]) =
                static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo_)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi_)) << 16);
        }
    }
    __syncthreads();

    // ---- 4. per head
    IT *outp = static_cast<IT *>(sp.out);
    const IT *zs = static_cast<const IT *>(sp.z);
    ST *outs = static_cast<ST *>(sp.states);
    const ST *init = static_cast<const ST *>(sp.init);
    const int pr = 16 * (r >> 2) + (r & 3);  // p of MFMA row / column r in p tile 0 (+ 4 pt)
    int xrow[kP / 16];                       // LDS row of p = pr + 4 pt
#pragma unroll
    for (int pt = 0; pt < kP / 16; pt++)
        xrow[pt] = dim_row(pr + 4 * pt);
    const int ptile = wv >> 1, ntb = (wv & 1) * KNT;  // the wave's part of the own state
    const int p_own = pr + 4 * ptile;                  // the lane's state row
    const int ksteps = (len + 31) / 32;

    for (int hk = 0; hk < nh; hk++) {
        const int h = h0 + hk;
        const float dh = sp.D ? sp.D[(h / sp.hsplit) * sp.D_sh] : 0.0f;
        const float *acum_h = acum_s[hk];
        const float *dtp_h = dtp_s[hk];
        const float *q_h = q_s[hk];
        const float *w_h = w_s[hk];

        // the own state^T: lane (r, g) ends with n = 16 (ntb + nt) + 4 g + i,
        // p = p_own
        f32x4 own[KNT];
#pragma unroll
        for (int nt = 0; nt < KNT; nt++)
            own[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = 0; k < ksteps; k++) {
            const int s_lo = 32 * k + g4;
            const uint2 xl = *reinterpret_cast<const uint2 *>(&Xs[xrow[ptile]][s_lo]);
            const uint2 xh = *reinterpret_cast<const uint2 *>(&Xs[xrow[ptile]][s_lo + 16]);
            const f32x4 wl = *reinterpret_cast<const f32x4 *>(&w_h[s_lo]);
            const f32x4 wh = *reinterpret_cast<const f32x4 *>(&w_h[s_lo + 16]);
            const V xr = __builtin_bit_cast(V, (uint4{xl.x, xl.y, xh.x, xh.y}));
            V b;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                b[i] = static_cast<IT>(to_f(xr[i]) * wl[i]);
                b[4 + i] = static_cast<IT>(to_f(xr[4 + i]) * wh[i]);
            }
#pragma unroll
            for (int nt = 0; nt < KNT; nt++) {
                const uint2 bl = *reinterpret_cast<const uint2 *>(&Bt[16 * (ntb + nt) + r][s_lo]);
                const uint2 bh = *reinterpret_cast<const uint2 *>(&Bt[16 * (ntb + nt) + r][s_lo + 16]);
                own[nt] = M::run(__builtin_bit_cast(V, (uint4{bl.x, bl.y, bh.x, bh.y})), b, own[nt]);
            }
        }

        // below the diagonal: the row factor exp(A_t - A_J) and the columns' factors
        auto scale_off = [&](int J, float at, const f32x4 (&d)[2]) {
            const int s_lo = 32 * J + g4;
            const float rf = exp_f(at - acum_h[32 * J + 31]);
            const f32x4 q_lo = *reinterpret_cast<const f32x4 *>(&q_h[s_lo]);
            const f32x4 q_hi = *reinterpret_cast<const f32x4 *>(&q_h[s_lo + 16]);
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
            const f32x4 a_lo = *reinterpret_cast<const f32x4 *>(&acum_h[s_lo]);
            const f32x4 a_hi = *reinterpret_cast<const f32x4 *>(&acum_h[s_lo + 16]);
            const f32x4 w_lo = *reinterpret_cast<const f32x4 *>(&dtp_h[s_lo]);
            const f32x4 w_hi = *reinterpret_cast<const f32x4 *>(&dtp_h[s_lo + 16]);
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
            const uint2 lo_ = *reinterpret_cast<const uint2 *>(&Xs[xrow[pt]][s_lo]);
            const uint2 hi_ = *reinterpret_cast<const uint2 *>(&Xs[xrow[pt]][s_lo + 16]);
            return __builtin_bit_cast(V, (uint4{lo_.x, lo_.y, hi_.x, hi_.y}));
        };
        // block J of a tile: scaled, then y^T += x_J^T (...)^T
        auto block = [&](int J, bool diag, int tt, float at, const f32x4 (&d)[2], f32x4 (&y)[kP / 16]) {
            const V a = diag ? scale_diag(J, tt, at, d) : scale_off(J, at, d);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
                y[pt] = M::run(xop(J, pt), a, y[pt]);
        };
        // D x from the x^T copy: y[pt][ii] is p = 16 gq + 4 pt + ii of the
        // token, which sits at row 4 (4 pt + ii) + gq
        auto add_dx = [&](int tt, f32x4 (&y)[kP / 16]) {
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
#pragma unroll
                for (int ii = 0; ii < 4; ii++)
                    y[pt][ii] += dh * to_f(Xs[4 * (4 * pt + ii) + gq][tt]);
        };
        // the part of y within the chunk, D x included
        f32x4 y0[kP / 16], y1[kP / 16];
#pragma unroll
        for (int pt = 0; pt < kP / 16; pt++)
            y0[pt] = y1[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (act0) {  // uniform per wave
            const float at0 = acum_h[tt0];
#pragma unroll
            for (int J = 0; J < 4; J++)
                if (J <= nj0)  // uniform
                    block(J, J == nj0, tt0, at0, cb[J], y0);
            add_dx(tt0, y0);
        }
        if (act1) {
            const float at1 = acum_h[tt1];
#pragma unroll
            for (int J = 0; J < 8; J++)
                if (J <= nj1)  // uniform; nj1 >= 4
                    block(J, J == nj1, tt1, at1, cb[8 - J], y1);
            add_dx(tt1, y1);
        }
        // z of the lane's tokens (16 consecutive p), and the next head's x,
        // in flight during the wait
        auto load_z = [&](int tt, V (&zv2)[2]) {
            const int64_t tok = row_tok(tt);
            const IT *zg = zs + tok * sp.z_st + head_off(sp, h, sp.z_sh) + 16 * gq;
#pragma unroll
            for (int k = 0; k < 2; k++)
                zv2[k] = zs ? *reinterpret_cast<const V *>(zg + 8 * k) : V{};
        };
        V zv0[2], zv1[2];
        if (act0)
            load_z(tt0, zv0);
        if (act1)
            load_z(tt1, zv1);
        XIn nx;
        if (hk + 1 < nh)
            load_x(h + 1, nx);

        // the entering state: published by the chunk before, unless this
        // chunk opens its sequence
        if (!opens && t == 0) {
            const int *flag = sp.ws_flags + (c - 1) * sp.H + h;
            for (int spins = 0;
                 __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 && spins < kSpinMax;
                 spins++)
                __builtin_amdgcn_s_sleep(2);
        }
        __syncthreads();  // the flag is seen; every wave is done with x^T and the entering state's LDS copy
        if (hk + 1 < nh)
            store_x(nx);
        // The chain's fp32 state is kept in the workspace in the lanes' own
        // order (16 bytes of lane l of wave w at (w KNT + nt) 64 + l): the
        // next chunk's lanes hold the same (p, n) and read it back, each
        // load or store instruction covering 1 KiB (in [p][n] order one
        // covered 16 rows x 64 bytes, 5% slower over the prefill).
        static_assert(kFThreads / 64 * KNT * 64 * 16 == PN * 4, "the lanes' order covers the state");
        const uint32_t chain_off = static_cast<uint32_t>(wv * KNT * 64 + lane) * 16;
        f32x4 sin[KNT];
        if (!opens) {
            const __amdgpu_buffer_rsrc_t src =
                buffer_of(sp.ws_state + ((c - 1) * sp.H + h) * PN, static_cast<uint32_t>(PN * 4));
#pragma unroll
            for (int nt = 0; nt < KNT; nt++)
                sin[nt] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               src, chain_off + nt * 64 * 16, 0, kDeviceScope));
        } else if (has_init) {
            const ST *ip = init + (seq * sp.H + h) * PN + p_own * N + g4;
#pragma unroll
            for (int nt = 0; nt < KNT; nt++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    sin[nt][i] = static_cast<float>(ip[16 * (ntb + nt) + i]);
        } else {
#pragma unroll
            for (int nt = 0; nt < KNT; nt++)
                sin[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // the state the chunk leaves: to the next chunk, and / or returned
        const float decay = exp_f(total_s[hk]);
        f32x4 so[KNT];
#pragma unroll
        for (int nt = 0; nt < KNT; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                so[nt][i] = fmaf(decay, sin[nt][i], own[nt][i]);
        if (feeds) {
            const __amdgpu_buffer_rsrc_t dst =
                buffer_of(sp.ws_state + (c * sp.H + h) * PN, static_cast<uint32_t>(PN * 4));
#pragma unroll
            for (int nt = 0; nt < KNT; nt++)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, so[nt]), dst,
                                                       chain_off + nt * 64 * 16, 0, kDeviceScope);
        }
        if (sp.intermediate || owner >= 0) {
            ST *dst = outs + ((sp.intermediate ? c : owner) * sp.H + h) * PN + p_own * N + g4;
#pragma unroll
            for (int nt = 0; nt < KNT; nt++) {
                Vec4<ST> ov;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    ov.v[i] = static_cast<ST>(so[nt][i]);
                *reinterpret_cast<Vec4<ST> *>(dst + 16 * (ntb + nt)) = ov;
            }
        }
        // the entering state, as the products read it
#pragma unroll
        for (int nt = 0; nt < KNT; nt++) {
            Vec4<IT> sv;
#pragma unroll
            for (int i = 0; i < 4; i++)
                sv.v[i] = static_cast<IT>(sin[nt][i]);
            *reinterpret_cast<Vec4<IT> *>(&Sin[sin_row(p_own)][16 * (ntb + nt) + g4]) = sv;
        }
        if (feeds)
            __builtin_amdgcn_s_waitcnt(kWaitStores);  // the state's stores are complete
        __syncthreads();  // the entering state's LDS copy and the next head's x^T
        if (feeds && t == 0)
            __hip_atomic_store(sp.ws_flags + c * sp.H + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

        // the entering state's part, y^T += exp(A_t) S_in C^T, both tiles
        // from one read of each operand of S_in
        {
            const float rs0 = exp_f(acum_h[tt0]), rs1 = exp_f(acum_h[tt1]);
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++) {
                f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < KN; k++) {
                    const V sa = *reinterpret_cast<const V *>(&Sin[16 * pt + r][32 * k + k8]);
                    if (act0)
                        acc0 = M::run(sa, ac[0][k], acc0);
                    if (act1)
                        acc1 = M::run(sa, ac[1][k], acc1);
                }
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    y0[pt][ii] = fmaf(rs0, acc0[ii], y0[pt][ii]);
                    y1[pt][ii] = fmaf(rs1, acc1[ii], y1[pt][ii]);
                }
            }
        }
        // the gate and the store: y[pt][ii] is p = 16 gq + 4 pt + ii of the token
        auto finish = [&](int tt, const V (&zv2)[2], const f32x4 (&y)[kP / 16]) {
            if (tt >= len)
                return;
            V o[2];
#pragma unroll
            for (int pt = 0; pt < kP / 16; pt++)
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    const int e = 4 * pt + ii;  // 0..15
                    float v = y[pt][ii];
                    if (zs)
                        v *= silu_f(to_f(zv2[e / 8][e % 8]));
                    o[e / 8][e % 8] = static_cast<IT>(v);
                }
            IT *orow = outp + (t0 + tt) * sp.out_st + head_off(sp, h, sp.out_sh) + 16 * gq;
            *reinterpret_cast<V *>(orow) = o[0];
            *reinterpret_cast<V *>(orow + 8) = o[1];
        };
        if (act0)
            finish(tt0, zv0, y0);
        if (act1)
            finish(tt1, zv1, y1);
    }
}

template <typename IT, typename ST, int N>
int launch_ssd_typed(const SsdParams &sp, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SsdParams p = sp;
    void *args[] = {&p};
    const int64_t nflags = sp.nchunks * sp.H;
    const int64_t flag_wgs = (nflags + kPrepThreads - 1) / kPrepThreads;
    const unsigned prep_grid = static_cast<unsigned>(1 + (flag_wgs < 256 ? flag_wgs : 256));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_prep_kernel), dim3(prep_grid),
                                   dim3(kPrepThreads), args, 0, s);
    if (e != hipSuccess)
        return static_cast<int>(e);
    const unsigned grid = static_cast<unsigned>(kXcds * sp.nchunks * sp.streams_per_xcd);
    e = hipLaunchKernel(reinterpret_cast<const void *>(&ssd_fused_kernel<IT, ST, N>), dim3(grid),
                        dim3(kFThreads), args, 0, s);
    return static_cast<int>(e);
}

template <typename IT, typename ST>
int launch_ssd_n(const SsdParams &sp, void *stream) {
    return sp.N == 64 ? launch_ssd_typed<IT, ST, 64>(sp, stream) : launch_ssd_typed<IT, ST, 128>(sp, stream);
}

template <typename IT>
int launch_ssd_st(const SsdParams &sp, int state_dtype, void *stream) {
    return state_dtype == SSU_F32   ? launch_ssd_n<IT, float>(sp, stream)
           : state_dtype == SSU_F16 ? launch_ssd_n<IT, _Float16>(sp, stream)
                                    : launch_ssd_n<IT, __bf16>(sp, stream);
}

template <typename IT, typename ST>
const void *fused_fn(int dstate) {
    return dstate == 64 ? reinterpret_cast<const void *>(&ssd_fused_kernel<IT, ST, 64>)
                        : reinterpret_cast<const void *>(&ssd_fused_kernel<IT, ST, 128>);
}

template <typename IT>
const void *fused_fn_st(int state_dtype, int dstate) {
    return state_dtype == SSU_F32   ? fused_fn<IT, float>(dstate)
           : state_dtype == SSU_F16 ? fused_fn<IT, _Float16>(dstate)
                                    : fused_fn<IT, __bf16>(dstate);
}

}  // namespace

int ssd_kernel_attributes(int io_dtype, int state_dtype, int dstate, const char *names[2], int vgprs[2]) {
    const void *fns[2] = {reinterpret_cast<const void *>(&ssd_prep_kernel),
                          io_dtype == SSU_BF16 ? fused_fn_st<__bf16>(state_dtype, dstate)
                                               : fused_fn_st<_Float16>(state_dtype, dstate)};
    names[0] = "ssd_prep_kernel";
    names[1] = "ssd_fused_kernel";
    for (int i = 0; i < 2; i++) {
        hipFuncAttributes attr;
        const hipError_t e = hipFuncGetAttributes(&attr, fns[i]);
        if (e != hipSuccess)
            return static_cast<int>(e);
        vgprs[i] = attr.numRegs;
    }
    return 0;
}

int launch_ssd(const SsdParams &sp, int io_dtype, int state_dtype, void *stream) {
    return io_dtype == SSU_BF16 ? launch_ssd_st<__bf16>(sp, state_dtype, stream)
                                : launch_ssd_st<_Float16>(sp, state_dtype, stream);
}

}  // namespace ssu
