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


#include "ssu_device.h"

namespace ssu {
namespace {

// Output-only variant of the multi-token kernel (YONLY), for
// disable_state_update: nothing is stored, so a sequence of at most kYMax
// tokens gets each y_t from the read tile and the unrolled window (ReplaySSM
// article, section "核心做法"):
//   y_t = (prod_{i<=t} a_i)(S_0 . C_t) + sum_{j<=t} (prod_{j<i<=t} a_i) dt'_j x_j (B_j . C_t) + D x_t,
// gated: one multiply-add per state element and token in place of the
// update, the readout and the rounding of the carried state. The carry is
// therefore not rounded to the state dtype between tokens, which moves y by
// far less than the tolerance of 16-bit outputs; the variant is used with
// fp32 outputs only for fp32 state, where nothing is rounded. All the
// tokens' inputs are requested at once, with the tile: their B and C rows go
// to LDS, the own row's x, z and dt to registers. Each DPP row forms the dots
// B_j . C_t with j = its row (mod 4) and hands them to the row owners through
// LDS (a workgroup is one wave, whose LDS accesses complete in order).
// Longer sequences take the update path.
constexpr int kYMax = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// D += A B on a 16 x 16 x 32 tile: A row m = lane % 16 with k = 8 (lane / 16)
// .. +7, B column n = lane % 16 with the same k, D[4 (lane / 16) + i][lane % 16]
// in register i.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
constexpr int kYRound = 4;  // tokens whose per-row inputs are requested together

// The output-only variant forms every S_0 . C_t on the matrix cores where
// the products are exact in an MFMA input type: a bf16 state with bf16 C, an
// fp16 state with fp16 C, or with bf16 C taken into fp16 by a power-of-two
// scale per token (bf16's 8 significant bits fit fp16's 11).
template <typename ST, typename IT, int N, bool YONLY>
constexpr bool yonly_mfma() {
    return YONLY && N % 32 == 0 && (kRowsPerPass * passes_for(N, sizeof(ST), kTileYonlyMfma)) % 16 == 0 &&
           ((std::is_same_v<ST, __bf16> && std::is_same_v<IT, __bf16>) ||
            (std::is_same_v<ST, _Float16> && !std::is_same_v<IT, float>));
}
template <typename ST, int N>
constexpr int yonly_mfma_waves_per_eu() {
    return kRowsPerPass * passes_for(N, sizeof(ST), kTileYonlyMfma) > 32 ? SSU_WAVES_PER_EU_YMFMA
                                                                         : SSU_WAVES_PER_EU_YMFMA_32;
}

template <typename ST, typename IT, int N, bool MULTI, bool YONLY = false>
__global__ __launch_bounds__(kMaxWaves *kWaveLanes,
                             (yonly_mfma<ST, IT, N, YONLY>() ? yonly_mfma_waves_per_eu<ST, N>()
                              : YONLY && sizeof(ST) == 2      ? SSU_WAVES_PER_EU_YVALU16
                              : MULTI                         ? SSU_WAVES_PER_EU_MULTI
                                                              : SSU_WAVES_PER_EU)) void ssu_kernel(const Params p) {
    static_assert(!YONLY || MULTI, "the output-only path is a multi-token path");
    constexpr int E = N / kLanesPerRow;  // state elements per lane per row
    constexpr int VEC = (16 / (int)sizeof(ST)) < E ? (16 / (int)sizeof(ST)) : E;
    constexpr int NCH = E / VEC;         // accesses per lane per row
    constexpr int PASSES = passes_for(N, sizeof(ST),
                                      yonly_mfma<ST, IT, N, YONLY>() ? kTileYonlyMfma
                                      : YONLY                         ? kTileYonly
                                      : MULTI                         ? kTileMulti
                                                                      : kTileOneToken);
    constexpr int IVEC = VEC;            // B / C are read with the same column split
    static_assert(E * kLanesPerRow == N && NCH * VEC == E, "dstate split");
    static_assert(PASSES <= kLanesPerRow, "one scalar-owning lane per pass");
    using SPack = Pack<ST, VEC>;
    using Inputs = TokenInputs<IT, NCH, IVEC>;
    constexpr int kRowsWave = kRowsPerPass * PASSES;
    constexpr bool YMFMA = yonly_mfma<ST, IT, N, YONLY>();

    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int wave = threadIdx.x / kWaveLanes;
    const int col = lane & (kLanesPerRow - 1);
    const int rsub = lane / kLanesPerRow;
    const int flags = p.flags;

    // workgroup -> (sequence, head, dim tile)
    const int32_t wg = xcd_clustered_index(blockIdx.x, gridDim.x);
    const int tile = wg % p.dim_tiles;
    const int32_t sh = wg / p.dim_tiles;
    const int h = sh % p.H;
    const int32_t b = sh / p.H;
    const int g = h / p.heads_per_group;
    // Pass q covers dim rows dw + 4q + rsub. The per-row scalars of pass q
    // (decay, dt' x, the gate and y) are computed once, by lane col == q of
    // each row group: the lane's "own" row is dw + 4 col + rsub.
    const int dw = tile * p.rows_per_block + wave * (kRowsPerPass * PASSES);
    const int d_own = dw + col * kRowsPerPass + rsub;
    const bool owner = col < PASSES && d_own < p.P;

    // the sequence's rows
    int32_t first_row = b, len = 1;
    if (MULTI) {
        if (p.layout == kCuSeqlens) {
            first_row = static_cast<int32_t>(load_index(p.cu, flags & kCuI64, b * p.cu_s));
            len = static_cast<int32_t>(load_index(p.cu, flags & kCuI64, (b + 1) * p.cu_s)) - first_row;
        } else if (p.layout == kDense) {
            first_row = b * p.steps;
            len = p.steps;
        }
        if (len <= 0)
            return;  // empty sequence: nothing to read or write
    }

    // read slot: entry num_accepted_tokens[b] - 1 (floored at 0) of the read
    // table, or the sequence index without a table
    int32_t start = 0;
    if (MULTI && p.acc) {
        start = static_cast<int32_t>(load_index(p.acc, flags & kAccI64, b * p.acc_s)) - 1;
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
    auto load_tile = [&]() {
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
    };
    // (the output-only variant on the matrix cores reads the tile in its own
    // layout, and this one only for a sequence too long for it)
    if constexpr (!YMFMA)
        load_tile();

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
    const int32_t ws0 = p.wtab ? p.w_s0 : p.r_s0;
    const int32_t ws1 = p.wtab ? p.w_s1 : p.r_s1;

    // Issue the loads of token t's inputs; nothing here waits. Every load is
    // unconditional and in bounds (a lane that owns no row reads its row
    // group's first row; absent z reads x; a 16-bit dt or an i32 table reads
    // the same address twice), so no branch joins pending loads; the values
    // are selected where they are used.
    const int d_fetch = owner ? d_own : 0;
    const IT *const zsrc = zs ? zs : xs;
    const int32_t z_sr = zs ? p.z_sr : p.x_sr, z_sh = zs ? p.z_sh : p.x_sh;
    const int dt_bytes = dt_f32 ? 4 : 2;
    const unsigned char *const dts = static_cast<const unsigned char *>(p.dt);
    const unsigned char *const wtb =
        static_cast<const unsigned char *>(wtab ? wtab : static_cast<const void *>(p.A));
    const int w_bytes = wi64 ? 8 : 4;
    auto fetch = [&](int32_t t, Inputs &in) {
        const int32_t r = first_row + t;
        const IT *bsrc = Bs + (r * p.B_sr + g * p.B_sg + col * IVEC);
        const IT *csrc = Cs + (r * p.C_sr + g * p.C_sg + col * IVEC);
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            in.b[c] = load_words<IT, IVEC>(bsrc + c * kLanesPerRow * IVEC);
            in.c[c] = load_words<IT, IVEC>(csrc + c * kLanesPerRow * IVEC);
        }
        const IT *xp = xs + (r * p.x_sr + h * p.x_sh + d_fetch);
        const IT *zp = zsrc + (r * z_sr + h * z_sh + d_fetch);
        in.x = *reinterpret_cast<const typename Inputs::Bits *>(xp);
        in.z = *reinterpret_cast<const typename Inputs::Bits *>(zp);
        const unsigned char *dp =
            dts + static_cast<int64_t>(r * p.dt_sr + h * p.dt_sh + d_fetch * p.dt_sp) * dt_bytes;
        in.dt_lo = *reinterpret_cast<const uint16_t *>(dp);
        in.dt_hi = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        // destination entry (the sequence index when there is no table)
        const int32_t wi = wtab ? (w2d ? b * ws0 + t * ws1 : (first_row + t) * ws0) : 0;
        const unsigned char *wp = wtb + static_cast<int64_t>(wi) * w_bytes;
        in.ws_lo = *reinterpret_cast<const uint32_t *>(wp);
        in.ws_hi = *reinterpret_cast<const uint32_t *>(wp + (wi64 ? 4 : 0));
    };

    // one token: update the tile with the inputs in `in`, store it, write y
    auto process = [&](int32_t t, const Inputs &in) {
        const int32_t r = first_row + t;
        float Bv[E], Cv[E];
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int k = 0; k < IVEC; k++) {
                Bv[c * IVEC + k] = word_elem(in.b[c], k);
                Cv[c * IVEC + k] = word_elem(in.c[c], k);
            }

        // scalars of the lane's own row
        const float xv = from_bits<IT>(in.x);
        const float zv = from_bits<IT>(in.z);
        const float dtv = dt_f32 ? __uint_as_float(uint32_t(in.dt_lo) | (uint32_t(in.dt_hi) << 16))
                                 : from_bits<IT>(in.dt_lo);
        float v = dtv + bias_h;
        if (flags & kSoftplus)
            v = softplus(v);
        const float decay = exp_hw(v * a_h);
        const float dtx = v * xv;

        // destination: the token's own entry of the destination table, else
        // of the read table, else slot b
        const uint32_t wlo = __builtin_amdgcn_readfirstlane(in.ws_lo);
        const uint32_t whi = __builtin_amdgcn_readfirstlane(in.ws_hi);
        const int64_t wslot = !wtab ? b
                              : wi64 ? static_cast<int64_t>((uint64_t(whi) << 32) | wlo)
                                     : static_cast<int64_t>(static_cast<int32_t>(wlo));
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
                    store_state<MULTI ? SSU_NT_STORE_MULTI : SSU_NT_STORE>(
                        reinterpret_cast<SPack *>(dst + c * kLanesPerRow * VEC), S[q][c]);
            }
        });

        // y of the lane's own row
        if (owner) {
            float y = ysum + d_h * xv;
            if (zs)
                y *= silu(zv);
            ys[r * p.out_sr + h * p.out_sh + d_own] = narrow<IT>(y);
        }
    };

    if constexpr (YONLY) {
        if (len <= kYMax) {  // uniform
            // (rows padded by 16 bytes, and Ul's by a word: the tokens' rows,
            // read by one 16-byte operand load each, and the wave's 64 rows
            // of Ul, read column-wise, fall in distinct banks)
            __shared__ __attribute__((aligned(16))) IT Bl[kYMax][N + 8];  // B rows of the tokens
            __shared__ __attribute__((aligned(16))) IT Cl[kYMax][N + 8];  // C rows of the tokens
            __shared__ float Wl[kYMax][kYMax];                        // Wl[j][t] = B_j . C_t
            // (matrix cores) the tile as A operands: lane l takes row
            // 16 mt + l % 16 and columns 32 kb + 8 (l / 16) .. +7 (16 bytes);
            // rows past the dim and the pad id read a valid row, then zeros
            constexpr int MT = YMFMA ? kRowsWave / 16 : 1, KB = YMFMA ? N / 32 : 1;
            using MV = std::conditional_t<std::is_same_v<ST, __bf16>, bf16x8, f16x8>;
            u32x4 sa[MT][KB];
            constexpr int kCpr = YMFMA ? N * (int)sizeof(ST) / 16 : 1;  // 16-byte pieces of a row
            static_assert(!YMFMA || kCpr == 4 * KB, "a row is KB operand columns of 4 pieces");
            // (64-row tiles; a one-tile wave reads in operand order, as its
            // LDS copy would cost it a wave per SIMD)
            constexpr bool kReorder = YMFMA && MT > 1;
            if constexpr (YMFMA) {
                // read in whole contiguous KiB: load (mt, kb) gives lane l the
                // 16-byte piece c = 64 (KB mt + kb) + l of the wave's rows
                // (row c / kCpr, piece c % kCpr), and the 16-row tile mt is
                // put in operand order through LDS before its products (an
                // operand-order read touches 16 rows x 64 bytes per load
                // instruction, which was 15% slower)
                const ST *abase = read_pad ? pool + tile_off : rbase;
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
#pragma unroll
                    for (int kb = 0; kb < KB; kb++) {
                        const int c = 64 * (KB * mt + kb) + lane;
                        const int d = dw + (kReorder ? c / kCpr : 16 * mt + (lane & 15));
                        const int dl = d < p.P ? d : p.P - 1;
                        const int piece = kReorder ? c % kCpr : 4 * kb + (lane >> 4);
                        sa[mt][kb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                            abase + static_cast<int64_t>(dl) * N + 8 * piece));
                    }
                }
            }
            // Every token's inputs in one round of loads, in flight with the
            // tile: DPP row rsub copies the B and C rows of tokens rsub,
            // rsub + 4 into LDS (tokens past the last reload the last), and
            // the own row's x, z and dt of each token go to registers.
            constexpr int kRounds = kYMax / kRowsPerPass;
            RawWords<IT, IVEC> bst[kRounds][NCH], cst[kRounds][NCH];
#pragma unroll
            for (int i = 0; i < kRounds; i++) {
                const int j = rsub + i * kRowsPerPass;
                const int32_t r = first_row + (j < len ? j : len - 1);
                const IT *bsrc = Bs + (r * p.B_sr + g * p.B_sg + col * IVEC);
                const IT *csrc = Cs + (r * p.C_sr + g * p.C_sg + col * IVEC);
#pragma unroll
                for (int c = 0; c < NCH; c++) {
                    bst[i][c] = load_words<IT, IVEC>(bsrc + c * kLanesPerRow * IVEC);
                    cst[i][c] = load_words<IT, IVEC>(csrc + c * kLanesPerRow * IVEC);
                }
            }
            // the own row's x, z and dt, kRound tokens at a time (the first
            // round now, the next when its first token comes; one round of 8
            // was not faster on the matrix-core variant)
            constexpr int kRound = kYRound;
            typename Inputs::Bits xb[kRound], zb[kRound];
            uint16_t dlo[kRound], dhi[kRound];
            auto fetch_round = [&](int t0) {
#pragma unroll
                for (int u = 0; u < kRound; u++) {
                    const int32_t r = first_row + (t0 + u < len ? t0 + u : len - 1);
                    xb[u] = *reinterpret_cast<const typename Inputs::Bits *>(xs + (r * p.x_sr + h * p.x_sh + d_fetch));
                    zb[u] = *reinterpret_cast<const typename Inputs::Bits *>(zsrc + (r * z_sr + h * z_sh + d_fetch));
                    const unsigned char *dp =
                        dts + static_cast<int64_t>(r * p.dt_sr + h * p.dt_sh + d_fetch * p.dt_sp) * dt_bytes;
                    dlo[u] = *reinterpret_cast<const uint16_t *>(dp);
                    dhi[u] = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
                }
            };
            fetch_round(0);
#pragma unroll
            for (int i = 0; i < kRounds; i++) {
                const int j = rsub + i * kRowsPerPass;
                if (j < len) {
#pragma unroll
                    for (int c = 0; c < NCH; c++) {
                        store_words<IT, IVEC>(&Bl[j][c * kLanesPerRow * IVEC + col * IVEC], bst[i][c]);
                        store_words<IT, IVEC>(&Cl[j][c * kLanesPerRow * IVEC + col * IVEC], cst[i][c]);
                    }
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // u_t = S_0 . C_t of every row of the wave and token, on the matrix cores
            __shared__ float Ul[YMFMA ? kRowsWave : 1][kYMax + 1];
            if constexpr (YMFMA) {
                // bf16 C into fp16: token j scaled by 2^-e_j, e_j = floor(log2 max |C_j|) - 14,
                // so its values down to 2^-28 of the largest are exact fp16 normals
                constexpr bool kScaled = std::is_same_v<ST, _Float16> && std::is_same_v<IT, __bf16>;
                // (and B the same way, for W = B C^T)
                __shared__ int El[2][kYMax];
                if constexpr (kScaled) {
#pragma unroll
                    for (int i = 0; i < kRounds; i++) {
                        float mc = 0.0f, mb = 0.0f;
#pragma unroll
                        for (int c = 0; c < NCH; c++)
#pragma unroll
                            for (int k = 0; k < IVEC; k++) {
                                mc = fmaxf(mc, fabsf(word_elem(cst[i][c], k)));
                                mb = fmaxf(mb, fabsf(word_elem(bst[i][c], k)));
                            }
                        mc = group_max<16>(mc);
                        mb = group_max<16>(mb);
                        const int j = rsub + i * kRowsPerPass;
                        auto expo = [](float m) {
                            const int ex = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu);
                            return m == 0.0f ? 0 : (ex == 0 ? -126 : ex - 127) - 14;
                        };
                        if (col == 0 && j < len) {
                            El[0][j] = expo(mc);
                            El[1][j] = expo(mb);
                        }
                    }
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
                // one token a lane: the B operand's column (C_n) and the W
                // product's A row (B_n)
                const int n = lane & 15;
                const int nr = n < len ? n : len - 1;
                const int ec = kScaled ? El[0][nr] : 0, eb = kScaled ? El[1][nr] : 0;
                auto operand = [&](const IT *src, int e) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
                    MV v;
                    if constexpr (kScaled) {
                        const bf16x8 x = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                        for (int k = 0; k < 8; k++)
                            v[k] = static_cast<_Float16>(ldexpf(static_cast<float>(x[k]), -e));
                    } else {
                        v = __builtin_bit_cast(MV, w);
                    }
                    return n < len ? v : MV{};
                };
                f32x4 D[MT], Dw = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                // the C operands, kept for the tiles when there are several
                MV bvs[MT > 1 ? KB : 1];
                auto c_op = [&](int kb) { return operand(&Cl[nr][32 * kb + 8 * (lane >> 4)], ec); };
                auto b_op = [&](int kb) { return operand(&Bl[nr][32 * kb + 8 * (lane >> 4)], eb); };
                if constexpr (MT > 1) {
#pragma unroll
                    for (int kb = 0; kb < KB; kb++) {
                        bvs[kb] = c_op(kb);
                        Dw = mfma16x16x32(b_op(kb), bvs[kb], Dw);
                    }
                }
                // the 16-row tile mt in operand order: lane l takes row l % 16
                // and piece 4 kb + l / 16 (rows padded by a piece: the 16
                // lanes of a pass hit distinct banks both ways)
                __shared__ __attribute__((aligned(16))) u32x4 Tl[kReorder ? 16 : 1][kReorder ? kCpr + 1 : 1];
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    if constexpr (kReorder) {
#pragma unroll
                        for (int kb = 0; kb < KB; kb++) {
                            const int c = 64 * kb + lane;
                            Tl[c / kCpr][c % kCpr] = sa[mt][kb];
                        }
                    }
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    D[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    const bool live = !read_pad && dw + 16 * mt + (lane & 15) < p.P;
#pragma unroll
                    for (int kb = 0; kb < KB; kb++) {
                        MV bv;
                        if constexpr (MT > 1) {
                            bv = bvs[kb];
                        } else {
                            bv = c_op(kb);
                            Dw = mfma16x16x32(b_op(kb), bv, Dw);
                        }
                        u32x4 t;
                        if constexpr (kReorder)
                            t = Tl[lane & 15][4 * kb + (lane >> 4)];
                        else
                            t = sa[mt][kb];
                        const u32x4 a = live ? t : u32x4{0u, 0u, 0u, 0u};
                        D[mt] = mfma16x16x32(__builtin_bit_cast(MV, a), bv, D[mt]);
                    }
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
                if (n < kYMax) {
#pragma unroll
                    for (int mt = 0; mt < MT; mt++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            Ul[16 * mt + 4 * (lane >> 4) + i][n] = ldexpf(D[mt][i], ec);
                    // Dw[i] = W[j][n] with j = 4 (lane / 16) + i, scaled by 2^-(eb_j + ec_n)
                    if ((lane >> 4) < kYMax / 4) {
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int j = 4 * (lane >> 4) + i;
                            const int ebj = kScaled ? El[1][j < len ? j : len - 1] : 0;
                            Wl[j][n] = ldexpf(Dw[i], ec + ebj);
                        }
                    }
                }
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            float av[kYMax], dxv[kYMax];  // the own row's decay and dt' x per token
            float G = 1.0f;               // prod of the decays so far
#pragma unroll
            for (int t = 0; t < kYMax; t++) {
                if (t >= len)
                    break;  // uniform
                if (t > 0 && t % kRound == 0)
                    fetch_round(t);
                const int u = t % kRound;
                const int32_t r = first_row + t;
                float Cv[E];
                if constexpr (!YMFMA) {
#pragma unroll
                    for (int c = 0; c < NCH; c++) {
                        const RawWords<IT, IVEC> cw =
                            *reinterpret_cast<const RawWords<IT, IVEC> *>(&Cl[t][c * kLanesPerRow * IVEC + col * IVEC]);
#pragma unroll
                        for (int k = 0; k < IVEC; k++)
                            Cv[c * IVEC + k] = word_elem(cw, k);
                    }
                }
                // scalars of the lane's own row
                const float xv = from_bits<IT>(xb[u]);
                const float zv = from_bits<IT>(zb[u]);
                const float dtv = dt_f32 ? __uint_as_float(uint32_t(dlo[u]) | (uint32_t(dhi[u]) << 16))
                                         : from_bits<IT>(dlo[u]);
                float v = dtv + bias_h;
                if (flags & kSoftplus)
                    v = softplus(v);
                av[t] = exp_hw(v * a_h);
                dxv[t] = v * xv;
                G *= av[t];
                // u = S_0 . C_t of the own row
                float usum = 0.0f;
                if constexpr (YMFMA) {
                    const int lr = d_own - dw;  // < kRowsWave for an owner
                    usum = Ul[lr < kRowsWave ? lr : kRowsWave - 1][t];
                } else {
                    for_passes<0, PASSES>([&](auto qc) {
                        constexpr int q = decltype(qc)::value;
                        float acc = 0.0f;
#pragma unroll
                        for (int c = 0; c < NCH; c++)
#pragma unroll
                            for (int k = 0; k < VEC; k++)
                                acc = fmaf(widen(S[q][c].v[k]), Cv[c * VEC + k], acc);
                        const float sum = row16_sum(acc);
                        usum = col == q ? sum : usum;
                    });
                }
                // B_j . C_t for j = rsub, rsub + 4, ... up to t (rows past t
                // repeat token t and write nothing); on the matrix cores, all
                // of them before the loop
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
                for (int jj = 0; jj < (YMFMA ? 0 : kYMax); jj += kRowsPerPass) {
                    if (jj > t)
                        break;  // uniform
                    const int j = jj + rsub;
                    const int jr = j <= t ? j : t;
                    float part = 0.0f;
#pragma unroll
                    for (int c = 0; c < NCH; c++) {
                        const RawWords<IT, IVEC> bw =
                            *reinterpret_cast<const RawWords<IT, IVEC> *>(&Bl[jr][c * kLanesPerRow * IVEC + col * IVEC]);
#pragma unroll
                        for (int k = 0; k < IVEC; k++)
                            part = fmaf(word_elem(bw, k), Cv[c * IVEC + k], part);
                    }
                    const float dot = row16_sum(part);
                    if (col == 0 && j <= t)
                        Wl[j][t] = dot;
                }
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                // the window of the own row, Horner over j
                float R = 0.0f;
#pragma unroll
                for (int j = 0; j < kYMax; j++) {
                    if (j > t)
                        break;
                    R = fmaf(R, av[j], dxv[j] * Wl[j][t]);
                }
                if (owner) {
                    float y = fmaf(G, usum, R) + d_h * xv;
                    if (zs)
                        y *= silu(zv);
                    ys[r * p.out_sr + h * p.out_sh + d_own] = narrow<IT>(y);
                }
            }
            return;
        }
    }

    if constexpr (YMFMA) {
        // a sequence longer than kYMax: the update path without stores, one
        // token at a time (the double-buffered loop below would set this
        // kernel's registers for a case its callers rarely reach)
        load_tile();
        for (int32_t t = 0; t < len; t++) {
            Inputs in;
            fetch(t, in);
            process(t, in);
        }
        return;
    }

    // Tokens alternate between two input buffers: the next token's inputs are
    // requested before the current token's stores, and no register copy joins
    // the two, so waiting for one buffer never waits for the other or for the
    // stores issued in between.
    Inputs in0, in1;
    fetch(0, in0);
    if (!MULTI) {
        process(0, in0);
        return;
    }
    // The vector-memory counter is in order: the scheduling barriers keep a
    // buffer's loads issued after everything the current token waits for.
    // The prefetch is unconditional (past the last token it reloads the last
    // token's inputs, which stay unused), so no branch joins pending loads.
    const int32_t last = len - 1;
    for (int32_t t = 0; t < len; t += 2) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(t + 1 < len ? t + 1 : last, in1);
        __builtin_amdgcn_sched_barrier(0);
        process(t, in0);
        if (t + 1 >= len)
            break;
        __builtin_amdgcn_sched_barrier(0);
        fetch(t + 2 < len ? t + 2 : last, in0);
        __builtin_amdgcn_sched_barrier(0);
        process(t + 1, in1);
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

template <typename ST, typename IT>
bool pick_yonly_n(int n, KernelRef *k) {
    switch (n) {
#define SSU_CASE(NN)                                                                     \
    case NN:                                                                             \
        k->fn = reinterpret_cast<const void *>(&ssu_kernel<ST, IT, NN, true, true>);    \
        k->tile = yonly_mfma<ST, IT, NN, true>() ? kTileYonlyMfma : kTileYonly;           \
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

bool find_yonly_kernel(int state_dtype, int io_dtype, int dstate, KernelRef *out) {
    // the carry is not rounded between tokens: with fp32 outputs only for
    // fp32 state
    switch (state_dtype) {
    case SSU_F32:
        return io_dtype == SSU_F32    ? pick_yonly_n<float, float>(dstate, out)
               : io_dtype == SSU_F16  ? pick_yonly_n<float, _Float16>(dstate, out)
               : io_dtype == SSU_BF16 ? pick_yonly_n<float, __bf16>(dstate, out)
                                      : false;
    case SSU_F16:
        return io_dtype == SSU_F16    ? pick_yonly_n<_Float16, _Float16>(dstate, out)
               : io_dtype == SSU_BF16 ? pick_yonly_n<_Float16, __bf16>(dstate, out)
                                      : false;
    case SSU_BF16:
        return io_dtype == SSU_F16    ? pick_yonly_n<__bf16, _Float16>(dstate, out)
               : io_dtype == SSU_BF16 ? pick_yonly_n<__bf16, __bf16>(dstate, out)
                                      : false;
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
