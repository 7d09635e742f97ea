// gfx950 kernels of ReplaySSM (ReplaySSM article, sections "核心做法" and
// "投机解码回滚变成挪指针"): the one-token replay step over a checkpoint and a
// buffer of past raw inputs, its variants with an MXFP8 or MXFP4 read copy
// of the checkpoint, the speculative step over T draft tokens, and the
// quantizers that make the first copy of a pool.

#include "ssu_device.h"

namespace ssu {
namespace {

// ReplaySSM decode (ReplaySSM article, section "核心做法"): one wave per 64
// dim rows of a (sequence, head). With h buffered entries, the steps j = 0..h
// (j = h is the current token) and w_j = B_j . C (C the current token's),
// each dim row runs
//   R <- R a_j + dt'_j x_j w_j,   G <- G a_j,
// and y = G (S_ckpt . C) + R + D x, gated: an output-only step, which writes
// nothing else but its raw inputs at buffer entry h. A step with h + 1 == L
// folds the steps into the checkpoint instead, a pass of up to KW steps at a
// time over the tile, each step the plain update's arithmetic exactly,
//   S <- fma(S, a_j, (dt'_j x_j) B_j)   (a 16-bit state rounded between steps),
// so that a fill equals the chain of plain updates bit for bit; its y is
// S . C of the folded rows. Lane r owns row r of the wave's
// rows (its scalars, x, z, dt, the recurrence and y). The tile is streamed in
// slices, 16 values a lane (N / 16 lanes a row) for the output-only read and
// 4 (N / 4 lanes) for the fold; slice i gives lane group k the row k LPR + i,
// so that lane r finds the row sum of its own row in its group at slice
// r % LPR. The fold's per-row (a_j, dt'_j x_j) go through a per-wave table in LDS. An
// entry count outside [0, L) (not for the pad id) makes the sequence's y NaN
// and writes nothing. LPF: the read copy's format -- 0 none, 8 MXFP8 (a byte
// a value), 4 MXFP4 (two values a byte); a copy is read in place of the
// checkpoint by output-only steps that are not a fill of the buffer.
constexpr int kReplayWin = SSU_REPLAY_WIN;  // window steps per round of the output-only path
constexpr int kReplayTab = 36;  // floats per row of the fold table (a_0 .. a_15, dt'x_0 .. dt'x_15; 16-byte rows)

// Sum over aligned groups of L lanes (1 .. 64), in every lane of the group.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 2)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (L >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if constexpr (L >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (L >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    if constexpr (L >= 32)
        v += __shfl_xor(v, 16);
    if constexpr (L >= 64)
        v += __shfl_xor(v, 32);
    return v;
}

// K consecutive elements of the x dtype as raw words, read AV elements at a
// time (the alignment the host guarantees for B and C rows).
template <typename IT, int K, int AV>
__device__ __forceinline__ RawWords<IT, K> load_run(const IT *src) {
    static_assert(K % AV == 0, "whole accesses");
    RawWords<IT, K> r;
    constexpr int kAcc = RawWords<IT, AV>::kBytes;
    if constexpr (kAcc >= 4) {
        constexpr int kw = kAcc / 4;
#pragma unroll
        for (int a = 0; a < K / AV; a++) {
            const RawWords<IT, AV> w = load_words<IT, AV>(src + a * AV);
#pragma unroll
            for (int k = 0; k < kw; k++)
                r.w[a * kw + k] = w.w[k];
        }
    } else {  // 2-byte accesses, two to a word
#pragma unroll
        for (int a = 0; a < K; a += 2) {
            const uint32_t lo = load_words<IT, 1>(src + a).w[0], hi = load_words<IT, 1>(src + a + 1).w[0];
            r.w[a / 2] = lo | (hi << 16);
        }
    }
    return r;
}

template <typename ST, typename IT, int N, int LPF>
__global__ __launch_bounds__(kReplayWaves *kWaveLanes, replay_waves_per_eu()) void ssu_replay_kernel(
    const Params p, const ReplayParams rp) {
    constexpr bool LP = LPF != 0;
    constexpr int LPR = N / 16;        // lanes per row, output-only read
    constexpr int RPI = kWaveLanes / LPR;
    constexpr int NS = LPR;            // slices over the wave's rows
    constexpr int LPRF = N / 4;        // lanes per row, fold
    constexpr int NSF = LPRF;
    constexpr int KW = sizeof(IT) == 4 ? 8 : 16;  // fold steps per pass
    // B and C accesses: the element alignment the host checks for the pool's dtype
    constexpr int AV = (16 / (int)sizeof(ST)) < N / 16 ? 16 / (int)sizeof(ST) : N / 16;
    constexpr int AVF = AV < 4 ? AV : 4;
    static_assert(N % 16 == 0 && N <= 256, "dstate 16 .. 256");
    static_assert(!LP || (sizeof(ST) == 4 && N % 32 == 0), "MX blocks of 32 values of an fp32 checkpoint");
    static_assert(LPF == 0 || LPF == 8 || LPF == 4, "copy formats");
    static_assert(KW <= 16 && KW % 4 == 0 && kReplayTab >= 32, "the fold table holds a pass");
    using Bits = std::conditional_t<sizeof(IT) == 2, uint16_t, uint32_t>;
    using SPack = Pack<ST, 4>;
    __shared__ __attribute__((aligned(16))) float tab[kReplayWaves][kReplayRows][kReplayTab];

    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int wave = threadIdx.x / kWaveLanes;
    int32_t item =
        __builtin_amdgcn_readfirstlane(xcd_clustered_index(blockIdx.x, gridDim.x) * kReplayWaves + wave);
    if (item >= p.nseq * p.H * p.dim_tiles)
        return;  // the last workgroup's spare waves
    if (p.flags & kFillFirst) {
        // Any order of the (sequence, head, rows) items is correct. A fill
        // moves several times a step's bytes, so the sequences whose step
        // fills the buffer (buf_len + 1 == L) are taken first, then the
        // others, each in batch order: no long wave starts last.
        constexpr int kBlocks = kReplayScanMax / kWaveLanes;
        const int32_t per = p.H * p.dim_tiles;
        uint32_t bits = 0;  // bit m: sequence 64 m + lane fills
#pragma unroll
        for (int m = 0; m < kBlocks; m++) {
            const int32_t bm = m * kWaveLanes + lane;
            if (m * kWaveLanes < p.nseq && bm < p.nseq)
                bits |= static_cast<uint32_t>(load_index(rp.buf_len, rp.len_i64, bm * rp.len_s) + 1 == rp.L) << m;
        }
        int32_t fills = 0;
#pragma unroll
        for (int m = 0; m < kBlocks; m++)
            fills += __popcll(__ballot((bits >> m) & 1u));
        const bool take_fill = item < fills * per;
        int32_t k = take_fill ? item / per : (item - fills * per) / per;  // rank in its kind
        int32_t bsel = 0;
        bool found = false;
#pragma unroll
        for (int m = 0; m < kBlocks; m++) {
            const int32_t live = p.nseq - m * kWaveLanes;  // sequences in block m
            if (live <= 0 || found)
                continue;
            uint64_t mask = __ballot((bits >> m) & 1u);
            if (!take_fill)
                mask = ~mask & (live >= kWaveLanes ? ~0ull : (1ull << live) - 1);
            const int32_t c = __popcll(mask);
            if (k < c) {
                // position of the k-th set bit
                int pos = 0;
#pragma unroll
                for (int w = 32; w >= 1; w >>= 1) {
                    const int32_t lo = __popcll((mask >> pos) & ((1ull << w) - 1));
                    if (k >= lo) {
                        k -= lo;
                        pos += w;
                    }
                }
                bsel = m * kWaveLanes + pos;
                found = true;
            } else {
                k -= c;
            }
        }
        item = __builtin_amdgcn_readfirstlane(bsel * per + item % per);
    }
    const int chunk = item % p.dim_tiles;
    const int32_t sh = item / p.dim_tiles;
    const int h = sh % p.H;
    const int32_t b = sh / p.H;
    const int g = h / p.heads_per_group;
    const int flags = p.flags;
    const int P = p.P, H = p.H;
    const int row0 = chunk * kReplayRows;
    const int nrow = P - row0 < kReplayRows ? P - row0 : kReplayRows;
    const bool own = lane < nrow;
    const int dr = row0 + (own ? lane : nrow - 1);  // the lane's row for its row loads
    // absolute row of wave row r (rows past the dim read the last one; their results are never stored)
    auto arow = [&](int r) { return row0 + (r < nrow ? r : nrow - 1); };

    const int64_t s = p.rtab ? load_index(p.rtab, flags & kReadI64, b * p.r_s0) : b;
    const int64_t h_raw = load_index(rp.buf_len, rp.len_i64, b * rp.len_s);
    const bool pad = s == p.pad;  // no checkpoint and no buffer: h is taken as 0
    const int64_t h_in = pad ? 0 : h_raw;
    IT *const ys = static_cast<IT *>(p.out) + (static_cast<int64_t>(b) * p.out_sr + static_cast<int64_t>(h) * p.out_sh);
    if (h_in < 0 || h_in >= rp.L) {
        if (own)
            ys[row0 + lane] = narrow<IT>(__builtin_nanf(""));
        return;
    }
    const int32_t hb = static_cast<int32_t>(h_in);
    const bool flush = hb + 1 == rp.L;
    const bool write = !pad && !(flags & kDisable);
    const bool dt_f32 = flags & kDtF32;
    const int dt_bytes = dt_f32 ? 4 : 2;

    const int64_t slot = pad ? 0 : s;
    const int64_t tile_off = static_cast<int64_t>(h) * P * N;
    ST *const sbase = static_cast<ST *>(p.state) + slot * p.slot_stride + tile_off;
    const int64_t lp_tile = slot * (static_cast<int64_t>(H) * P * N) + tile_off;  // element offset in the copy
    const int64_t sl = slot * rp.L;  // first buffer entry of the slot
    const IT *const xs = static_cast<const IT *>(p.x);
    const IT *const zs = static_cast<const IT *>(p.z);
    const unsigned char *const dts = static_cast<const unsigned char *>(p.dt);
    const IT *const Brow = static_cast<const IT *>(p.B) + (static_cast<int64_t>(b) * p.B_sr + static_cast<int64_t>(g) * p.B_sg);
    const IT *const Crow = static_cast<const IT *>(p.C) + (static_cast<int64_t>(b) * p.C_sr + static_cast<int64_t>(g) * p.C_sg);
    IT *const bxs = static_cast<IT *>(rp.buf_x);
    IT *const bBs = static_cast<IT *>(rp.buf_B);
    unsigned char *const bdts = static_cast<unsigned char *>(rp.buf_dt);

    const float a_h = p.A[h * p.A_sh];
    const float d_h = p.D ? p.D[h * p.D_sh] : 0.0f;
    const float bias_h = p.dt_bias ? p.dt_bias[h * p.bias_sh] : 0.0f;

    // Buffer entry j of the lane's row (x, dt) or of the group (B): a
    // uniform base plus a 32-bit offset (one slot's buffer spans fewer than
    // 2^31 elements). Step j < hb reads entry j; step hb is the current token,
    // whose values are selected in place of an entry read (entry min(j, hb - 1)
    // of the slot, always in bounds, is read and dropped).
    const int32_t hb1 = hb > 0 ? hb - 1 : 0;
    const IT *const bx0 = bxs + (sl * H + h) * P;
    const unsigned char *const bdt0 = bdts + (rp.dt_per_head ? sl * H + h : (sl * H + h) * P) * dt_bytes;
    const IT *const bB0 = bBs + (sl * rp.G + g) * N;
    const uint32_t HP = static_cast<uint32_t>(H * P), GN = static_cast<uint32_t>(rp.G * N);
    const uint32_t dt_row = rp.dt_per_head ? 0u : static_cast<uint32_t>(dr);
    const uint32_t dt_entry = rp.dt_per_head ? static_cast<uint32_t>(H) : HP;
    auto entry = [&](int32_t j) { return static_cast<uint32_t>(j < hb1 ? j : hb1); };
    // dt as two 16-bit halves (the high one used for fp32 dt), loaded unconditionally
    auto dt_bits = [&](const unsigned char *q) {
        const uint32_t lo = *reinterpret_cast<const uint16_t *>(q);
        const uint32_t hi = *reinterpret_cast<const uint16_t *>(q + (dt_f32 ? 2 : 0));
        return lo | (hi << 16);
    };
    auto step_dt = [&](uint32_t bits) {
        float v = (dt_f32 ? __uint_as_float(bits) : from_bits<IT>(bits & 0xFFFFu)) + bias_h;
        if (flags & kSoftplus)
            v = softplus(v);
        return v;
    };

    // the current step's x, z and dt of the lane's row
    const int64_t xo = static_cast<int64_t>(b) * p.x_sr + static_cast<int64_t>(h) * p.x_sh + dr;
    const Bits x_bits = *reinterpret_cast<const Bits *>(xs + xo);
    const Bits z_bits = *reinterpret_cast<const Bits *>(
        zs ? zs + (static_cast<int64_t>(b) * p.z_sr + static_cast<int64_t>(h) * p.z_sh + dr) : xs + xo);
    const uint32_t dt_cur = dt_bits(dts + ((static_cast<int64_t>(b) * p.dt_sr + static_cast<int64_t>(h) * p.dt_sh) +
                                           static_cast<int64_t>(dr) * p.dt_sp) * dt_bytes);
    // step j's x and dt bits for the lane's row, from loads of entry(j)
    auto x_step = [&](int32_t j) { return *reinterpret_cast<const Bits *>(bx0 + (entry(j) * HP + dr)); };
    auto dt_step = [&](int32_t j) { return dt_bits(bdt0 + (entry(j) * dt_entry + dt_row) * dt_bytes); };

    float ysum = 0.0f;
    if (flush && write) {
        // ---- fold: the checkpoint tile, 4 values a lane, KW steps a pass
        const int colf = (lane % LPRF) * 4;
        const RawWords<IT, 4> cfw = load_run<IT, 4, AVF>(Crow + colf);
        float Cf[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
            Cf[k] = word_elem(cfw, k);
        float (*const trow)[kReplayTab] = tab[wave];
        const int grp = (lane / LPRF) * LPRF;  // slice i gives the lane row grp + i
        constexpr int DF = NSF < SSU_REPLAY_FOLD_DEPTH ? NSF : SSU_REPLAY_FOLD_DEPTH;  // slices in flight
        for (int32_t j0 = 0; j0 <= hb; j0 += KW) {
            const bool last = j0 + KW > hb;
            // the first slices of the tile are requested before the table is formed
            SPack ring[DF];
            auto issue = [&](int i, SPack &dst) {
                dst = load_state(reinterpret_cast<const SPack *>(sbase + static_cast<int64_t>(arow(grp + i)) * N + colf));
            };
#pragma unroll
            for (int u = 0; u < DF; u++)
                issue(u, ring[u]);
            {
                // the pass's decays and dt'x of the lane's own row
                Bits xv[KW];
                uint32_t dv[KW];
#pragma unroll
                for (int t = 0; t < KW; t++) {
                    xv[t] = x_step(j0 + t);
                    dv[t] = dt_step(j0 + t);
                }
#pragma unroll
                for (int t = 0; t < KW; t++) {
                    const bool cur = j0 + t == hb;
                    const float v = step_dt(cur ? dt_cur : dv[t]);
                    trow[lane][t] = exp_hw(v * a_h);
                    trow[lane][16 + t] = v * from_bits<IT>(cur ? x_bits : xv[t]);
                }
            }
            __builtin_amdgcn_wave_barrier();
            RawWords<IT, 4> bq[KW];  // the pass's B at the lane's columns
#pragma unroll
            for (int t = 0; t < KW; t++)
                bq[t] = load_run<IT, 4, AVF>((j0 + t < hb ? bB0 + entry(j0 + t) * GN : Brow) + colf);
            for (int i0 = 0; i0 < NSF; i0 += DF) {
#pragma unroll
                for (int u = 0; u < DF; u++) {
                    const int i = i0 + u;
                    SPack S = ring[u];
                    if (i + DF < NSF)
                        issue(i + DF, ring[u]);
                    // the B words are unpacked per slice, not held unpacked
                    // across the loop (64 more registers)
#pragma unroll
                    for (int t = 0; t < KW; t++)
#pragma unroll
                        for (int k = 0; k < RawWords<IT, 4>::kWords; k++)
                            asm volatile("" : "+v"(bq[t].w[k]));
                    const int r = grp + i;
                    const float4 *tr = reinterpret_cast<const float4 *>(trow[r]);
                    // the pass's steps in order (the last value unrounded, for y)
                    float sv[4];
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        sv[k] = widen(S.v[k]);
#pragma unroll
                    for (int q = 0; q < KW / 4; q++) {
                        if (j0 + 4 * q > hb)  // uniform
                            break;
                        const float4 a4 = tr[q], d4 = tr[4 + q];
                        const float aq[4] = {a4.x, a4.y, a4.z, a4.w}, dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                        for (int tt = 0; tt < 4; tt++) {
                            if (j0 + 4 * q + tt > hb)  // uniform
                                break;
#pragma unroll
                            for (int k = 0; k < 4; k++)
                                sv[k] = fmaf(widen(narrow<ST>(sv[k])), aq[tt], dq[tt] * word_elem(bq[4 * q + tt], k));
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        S.v[k] = narrow<ST>(sv[k]);
                    const bool in = r < nrow;
                    const int64_t at = static_cast<int64_t>(row0 + r) * N + colf;
                    if (in)
                        store_state<SSU_NT_STORE>(reinterpret_cast<SPack *>(sbase + at), S);
                    if (last) {
                        float part = 0.0f;
#pragma unroll
                        for (int k = 0; k < 4; k++)
                            part = fmaf(sv[k], Cf[k], part);
                        const float sum = group_sum<LPRF>(part);
                        ysum = lane % LPRF == i ? sum : ysum;
                        if constexpr (LP) {
                            // the stored values into the read copy: 8 lanes a block
                            float v4[4], amax = 0.0f;
#pragma unroll
                            for (int k = 0; k < 4; k++) {
                                v4[k] = widen(S.v[k]);
                                amax = fmaxf(amax, fabsf(v4[k]));
                            }
                            amax = group_max<8>(amax);
                            const int kexp = LPF == 4 ? mx4_exponent(amax) : mx8_exponent(amax);
                            const uint32_t codes = LPF == 4 ? e2m1_codes4(v4, kexp) : e4m3_codes4(v4, kexp);
                            if (in) {
                                const int64_t e = lp_tile + at;
                                if constexpr (LPF == 4)
                                    *reinterpret_cast<uint16_t *>(rp.lp + e / 2) = static_cast<uint16_t>(codes);
                                else
                                    *reinterpret_cast<uint32_t *>(rp.lp + e) = codes;
                                if (lane % 8 == 0)
                                    rp.lp_scale[e / 32] = static_cast<uint8_t>(kexp + 127);
                            }
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        // ---- output-only: u = S . C from the copy or the checkpoint, and the window
        // A lane's 16 columns of a row: for a copy, 16 consecutive ones (one
        // access); for the checkpoint, SQ runs of VV (16 bytes each), the row
        // split so that every access of a wave is lane-contiguous.
        constexpr int VV = LP ? 16 : 16 / (int)sizeof(ST);
        constexpr int SQ = 16 / VV;
        auto col_of = [&](int k) { return (lane % LPR) * VV + k * (LPR * VV); };  // start of run k
        const int grp = (lane / LPR) * LPR;  // slice i gives the lane row grp + i
        float Cv[16];
#pragma unroll
        for (int k = 0; k < SQ; k++) {
            const RawWords<IT, VV> cw = load_run<IT, VV, (AV < VV ? AV : VV)>(Crow + col_of(k));
#pragma unroll
            for (int e = 0; e < VV; e++)
                Cv[k * VV + e] = word_elem(cw, e);
        }
        // the copy's slices: 16 codes (MXFP8) or 8 bytes of code pairs
        // (MXFP4) and the block's scale byte; the checkpoint's: 16 values
        constexpr int kCopyWords = LPF == 4 ? 2 : 4;
        constexpr int kCkptWords = 16 * (int)sizeof(ST) / 4;
        constexpr int kDC = LPF == 4 ? SSU_REPLAY_COPY4_DEPTH : SSU_REPLAY_COPY8_DEPTH;
        constexpr int kDS = (SSU_REPLAY_CKPT_WORDS) / kCkptWords < 1 ? 1 : (SSU_REPLAY_CKPT_WORDS) / kCkptWords;
        constexpr int DC = NS < kDC ? NS : kDC;  // copy slices in flight
        constexpr int DS = NS < kDS ? NS : kDS;  // checkpoint slices in flight
        // (an LP kernel reads the checkpoint only for a fill with
        // disable_state_update, after the window and without a prefetch)
        const bool from_copy = LP && !flush && !pad;
        const bool from_ckpt = !pad && !from_copy;
        struct CopySlice {
            uint32_t w[kCopyWords];
            uint32_t scale;
        };
        struct CkptSlice {
            uint32_t w[kCkptWords];
        };
        CopySlice cring[LP ? DC : 1];
        CkptSlice sring[LP ? 1 : DS];
        auto issue_copy = [&](int i, CopySlice &dst) {
            if constexpr (LP) {
                const int64_t e = lp_tile + static_cast<int64_t>(arow(grp + i)) * N + col_of(0);
                if constexpr (LPF == 4) {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(rp.lp + e / 2);
                    dst.w[0] = v.x;
                    dst.w[1] = v.y;
                } else {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(rp.lp + e);
                    dst.w[0] = v.x;
                    dst.w[1] = v.y;
                    dst.w[2] = v.z;
                    dst.w[3] = v.w;
                }
                dst.scale = rp.lp_scale[e / 32];
            }
        };
        auto issue_ckpt = [&](int i, CkptSlice &dst) {
            const ST *rowp = sbase + static_cast<int64_t>(arow(grp + i)) * N;
#pragma unroll
            for (int k = 0; k < kCkptWords / 4; k++) {
                // (an LP kernel's lanes read 16 consecutive values, the copy's columns)
                const u32x4 *q = reinterpret_cast<const u32x4 *>(rowp + (LP ? col_of(0) + k * (16 / (int)sizeof(ST)) : col_of(k)));
                const u32x4 v = SSU_NT_LOAD ? __builtin_nontemporal_load(q) : *q;
                dst.w[4 * k] = v.x;
                dst.w[4 * k + 1] = v.y;
                dst.w[4 * k + 2] = v.z;
                dst.w[4 * k + 3] = v.w;
            }
        };
        if (from_copy) {
#pragma unroll
            for (int u = 0; u < DC; u++)
                issue_copy(u, cring[u]);
        } else if (!LP && from_ckpt) {
#pragma unroll
            for (int u = 0; u < DS; u++)
                issue_ckpt(u, sring[u]);
        }

        // window: rounds of kReplayWin steps; w_j = B_j . C by lane groups
        // (RPI dots a load), then each row's recurrence
        constexpr int NQ = RPI >= kReplayWin ? 1 : kReplayWin / RPI;
        float R = 0.0f, G = 1.0f;
        for (int32_t j0 = 0; j0 <= hb; j0 += kReplayWin) {
            RawWords<IT, 16> bw[NQ];
#pragma unroll
            for (int q = 0; q < NQ; q++) {
                const int t = q * RPI + lane / LPR;
                const int32_t j = j0 + (t < kReplayWin ? t : kReplayWin - 1);
                const IT *brow = j < hb ? bB0 + entry(j) * GN : Brow;
#pragma unroll
                for (int k = 0; k < SQ; k++) {
                    const RawWords<IT, VV> w = load_run<IT, VV, (AV < VV ? AV : VV)>(brow + col_of(k));
#pragma unroll
                    for (int e = 0; e < RawWords<IT, VV>::kWords; e++)
                        bw[q].w[k * RawWords<IT, VV>::kWords + e] = w.w[e];
                }
            }
            Bits xv[kReplayWin];
            uint32_t dv[kReplayWin];
#pragma unroll
            for (int t = 0; t < kReplayWin; t++) {
                xv[t] = x_step(j0 + t);
                dv[t] = dt_step(j0 + t);
            }
            float wq[NQ];
#pragma unroll
            for (int q = 0; q < NQ; q++) {
                float part = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; k++)
                    part = fmaf(word_elem(bw[q], k), Cv[k], part);
                wq[q] = group_sum<LPR>(part);
            }
#pragma unroll
            for (int t = 0; t < kReplayWin; t++) {
                const int32_t j = j0 + t;
                if (j <= hb) {  // uniform
                    const bool cur = j == hb;
                    const float w = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(wq[t / RPI]), (t % RPI) * LPR));
                    const float v = step_dt(cur ? dt_cur : dv[t]);
                    const float a = exp_hw(v * a_h);
                    R = fmaf(R, a, v * from_bits<IT>(cur ? x_bits : xv[t]) * w);
                    G *= a;
                }
            }
        }

        // u of the lane's own row
        float u = 0.0f;
        if (from_copy) {
            if constexpr (LP) {
                for (int i0 = 0; i0 < NS; i0 += DC) {
#pragma unroll
                    for (int uu = 0; uu < DC; uu++) {
                        const int i = i0 + uu;
                        const CopySlice cs = cring[uu];
                        if (i + DC < NS)
                            issue_copy(i + DC, cring[uu]);
                        const float sc = mx8_scale(cs.scale);
                        float v[16];
#pragma unroll
                        for (int k = 0; k < kCopyWords; k++) {
                            if constexpr (LPF == 4) {
                                const float2 a = e2m1_pair<0>(cs.w[k], sc), b2 = e2m1_pair<1>(cs.w[k], sc);
                                const float2 c2 = e2m1_pair<2>(cs.w[k], sc), d2 = e2m1_pair<3>(cs.w[k], sc);
                                v[8 * k] = a.x;
                                v[8 * k + 1] = a.y;
                                v[8 * k + 2] = b2.x;
                                v[8 * k + 3] = b2.y;
                                v[8 * k + 4] = c2.x;
                                v[8 * k + 5] = c2.y;
                                v[8 * k + 6] = d2.x;
                                v[8 * k + 7] = d2.y;
                            } else {
                                const float2 lo = e4m3_pair<false>(cs.w[k], sc), hi = e4m3_pair<true>(cs.w[k], sc);
                                v[4 * k] = lo.x;
                                v[4 * k + 1] = lo.y;
                                v[4 * k + 2] = hi.x;
                                v[4 * k + 3] = hi.y;
                            }
                        }
                        float part = 0.0f;
#pragma unroll
                        for (int k = 0; k < 16; k++)
                            part = fmaf(v[k], Cv[k], part);
                        const float sum = group_sum<LPR>(part);
                        u = lane % LPR == i ? sum : u;
                    }
                }
            }
        } else if (from_ckpt) {
            constexpr int D = LP ? 1 : DS;
            for (int i0 = 0; i0 < NS; i0 += D) {
#pragma unroll
                for (int uu = 0; uu < D; uu++) {
                    const int i = i0 + uu;
                    if (LP)
                        issue_ckpt(i, sring[0]);
                    const CkptSlice cs = sring[uu];
                    if (!LP && i + D < NS)
                        issue_ckpt(i + D, sring[uu]);
                    float part = 0.0f;
#pragma unroll
                    for (int k = 0; k < 16; k++) {
                        float v;
                        if constexpr (sizeof(ST) == 4)
                            v = __uint_as_float(cs.w[k]);
                        else
                            v = from_bits<ST>((k & 1) ? cs.w[k / 2] >> 16 : cs.w[k / 2] & 0xFFFFu);
                        part = fmaf(v, Cv[k], part);
                    }
                    const float sum = group_sum<LPR>(part);
                    u = lane % LPR == i ? sum : u;
                }
            }
        }
        ysum = fmaf(G, u, R);

        // append the step's raw inputs at entry hb
        if (write && !flush) {
            const int64_t e = sl + hb;
            auto put_dt = [&](unsigned char *dst) {
                if (dt_f32)
                    *reinterpret_cast<uint32_t *>(dst) = dt_cur;
                else
                    *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(dt_cur);
            };
            if (own) {
                *reinterpret_cast<Bits *>(bxs + (e * H + h) * P + dr) = x_bits;
                if (!rp.dt_per_head)
                    put_dt(bdts + ((e * H + h) * P + dr) * dt_bytes);
            }
            if (rp.dt_per_head && chunk == 0 && lane == 0)
                put_dt(bdts + (e * H + h) * dt_bytes);
            if (h % p.heads_per_group == 0 && chunk == 0) {
                const Bits *src = reinterpret_cast<const Bits *>(Brow);
                Bits *dst = reinterpret_cast<Bits *>(bBs + (e * rp.G + g) * N);
                for (int n = lane; n < N; n += kWaveLanes)
                    dst[n] = src[n];
            }
        }
    }

    // y of the lane's own row
    if (own) {
        float y = ysum + d_h * from_bits<IT>(x_bits);
        if (zs)
            y *= silu(from_bits<IT>(z_bits));
        ys[row0 + lane] = narrow<IT>(y);
    }
}

// ReplaySSM speculative step (ReplaySSM article, section "投机解码回滚变成挪指针"):
// T draft tokens per sequence, packed as rows b*T + t. One workgroup per
// (sequence, head, dim tile), the checkpoint tile in ssu_kernel's layout. If
// h + 2T > L (the fold one window early), the h committed entries are first
// applied to the tile with the plain update's arithmetic (no readout) and the
// tile is stored; the window then starts empty (w = 0), else w = h. Drafts
// are read out kSpecGroup at a time: the window (w committed entries, then
// the drafts up to the group's last) is split into NSEG contiguous runs of
// steps: lane col of a DPP row takes dim row col % PASSES and run
// col / PASSES, and the runs' pairs are joined in step order ((R0, G0)
// followed by (R1, G1) is (R0 G1 + R1, G0 G1)); every run keeps one (R, G)
// pair per draft of the group,
// updated only at steps that draft can see (the causal mask), and each
// B_j . C_t is formed once per DPP row and draft. The drafts' raw inputs go
// to entries w .. w+T-1: x and a per-dim dt here, by the lane that owns the
// dim row; B and a per-head dt by ssu_replay_spec_append_kernel, launched
// after this kernel on the same stream. An entry count outside [0, L] (not
// for the pad id) makes the sequence's y NaN and writes nothing.
//
// Ordering: a fold reads committed entries 0..h-1 and its drafts go to
// entries 0..T-1, so a folding sequence's appends overwrite entries its fold
// reads. An entry's B row is read by every dim tile of every head of the
// group and a per-head dt by every dim tile of the head, across workgroups
// that run in no fixed order, so those two are written only once this
// launch has ended. x and a per-dim dt of row d are read (fold) and written
// (append) by the one lane that owns row d, in that order; other lanes read
// no buffer row they do not own. A sequence that does not fold reads entries
// below w and writes entries w and above.
constexpr int kSpecGroup = 4;

template <typename ST, typename IT, int N>
__global__ __launch_bounds__(kMaxWaves *kWaveLanes, replay_spec_waves_per_eu(sizeof(ST), N)) void ssu_replay_spec_kernel(
    const Params p, const ReplayParams rp) {
    constexpr int E = N / kLanesPerRow;
    constexpr int VEC = (16 / (int)sizeof(ST)) < E ? (16 / (int)sizeof(ST)) : E;
    constexpr int NCH = E / VEC;
    constexpr int PASSES = passes_for(N, sizeof(ST), kTileReplay);
    constexpr int IVEC = VEC;
    constexpr int NSEG = kLanesPerRow / PASSES;
    constexpr int NDOT = NSEG < kRowsPerPass ? 1 : NSEG / kRowsPerPass;
    constexpr int TG = kSpecGroup;
    static_assert(PASSES <= kLanesPerRow && kLanesPerRow % PASSES == 0, "runs tile the row");
    using SPack = Pack<ST, VEC>;
    using Bits = typename TokenInputs<IT, NCH, IVEC>::Bits;

    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int wave = threadIdx.x / kWaveLanes;
    const int col = lane & (kLanesPerRow - 1);
    const int rsub = lane / kLanesPerRow;
    const int flags = p.flags;

    const int32_t wg = xcd_clustered_index(blockIdx.x, gridDim.x);
    const int tile = wg % p.dim_tiles;
    const int32_t sh = wg / p.dim_tiles;
    const int h = sh % p.H;
    const int32_t b = sh / p.H;
    const int g = h / p.heads_per_group;
    const int dw = tile * p.rows_per_block + wave * (kRowsPerPass * PASSES);
    const int d_own = dw + col * kRowsPerPass + rsub;
    const bool owner = col < PASSES && d_own < p.P;
    const int d_fetch = owner ? d_own : 0;
    const int32_t T = p.steps;

    const int64_t s = p.rtab ? load_index(p.rtab, flags & kReadI64, b * p.r_s0) : b;
    const bool pad = s == p.pad;  // no checkpoint and no buffer: h is taken as 0
    const int64_t h_in = pad ? 0 : load_index(rp.buf_len, rp.len_i64, b * rp.len_s);
    const bool bad = h_in < 0 || h_in > rp.L;
    const int32_t hc = bad ? 0 : static_cast<int32_t>(h_in);
    const bool fold = !bad && hc + 2 * T > rp.L;
    const int32_t w = fold ? 0 : hc;
    const bool write = !pad && !bad && !(flags & kDisable);
    const bool dt_f32 = flags & kDtF32;
    const int dt_bytes = dt_f32 ? 4 : 2;

    const int P = p.P, H = p.H;
    const int64_t tile_off = static_cast<int64_t>(h) * P * N;
    ST *const sbase = static_cast<ST *>(p.state) + (pad ? 0 : s) * p.slot_stride + tile_off;
    const int64_t sl = (pad ? 0 : s) * rp.L;
    const IT *const xs = static_cast<const IT *>(p.x);
    const IT *const zs = static_cast<const IT *>(p.z);
    const IT *const Bs = static_cast<const IT *>(p.B);
    const IT *const Cs = static_cast<const IT *>(p.C);
    IT *const ys = static_cast<IT *>(p.out);
    const unsigned char *const dts = static_cast<const unsigned char *>(p.dt);
    IT *const bxs = static_cast<IT *>(rp.buf_x);
    IT *const bBs = static_cast<IT *>(rp.buf_B);
    unsigned char *const bdts = static_cast<unsigned char *>(rp.buf_dt);

    const float a_h = p.A[h * p.A_sh];
    const float d_h = p.D ? p.D[h * p.D_sh] : 0.0f;
    const float bias_h = p.dt_bias ? p.dt_bias[h * p.bias_sh] : 0.0f;

    // buffer entry k of the slot (32-bit lane offsets from per-slot bases),
    // draft t (row b*T + t), and step k of the window (k < w: entry k, else
    // draft k - w), each for a dim row d in range
    const IT *const bx0 = bxs + (sl * H + h) * P;
    const unsigned char *const bdt0 = bdts + (rp.dt_per_head ? sl * H + h : (sl * H + h) * P) * dt_bytes;
    const IT *const bB0 = bBs + (sl * rp.G + g) * N + col * IVEC;
    const uint32_t HP = static_cast<uint32_t>(H * P), GN = static_cast<uint32_t>(rp.G * N);
    const uint32_t entry_dt = rp.dt_per_head ? static_cast<uint32_t>(H) : HP;
    auto row = [&](int32_t t) { return b * T + t; };
    auto entry_x = [&](int32_t k, int d) { return bx0 + (static_cast<uint32_t>(k) * HP + d); };
    auto entry_dt_p = [&](int32_t k, int d) {
        return bdt0 + (static_cast<uint32_t>(k) * entry_dt + (rp.dt_per_head ? 0u : static_cast<uint32_t>(d))) * dt_bytes;
    };
    auto entry_B = [&](int32_t k) { return bB0 + static_cast<uint32_t>(k) * GN; };
    auto draft_x = [&](int32_t t, int d) { return xs + (row(t) * p.x_sr + h * p.x_sh + d); };
    auto draft_dt_p = [&](int32_t t, int d) {
        return dts + static_cast<int64_t>(row(t) * p.dt_sr + h * p.dt_sh + d * p.dt_sp) * dt_bytes;
    };
    auto draft_B = [&](int32_t t) { return Bs + (row(t) * p.B_sr + g * p.B_sg + col * IVEC); };
    auto x_at = [&](int32_t k, int d) -> const Bits * {
        return reinterpret_cast<const Bits *>(k < w ? entry_x(k, d) : draft_x(k - w, d));
    };
    auto dt_at = [&](int32_t k, int d) { return k < w ? entry_dt_p(k, d) : draft_dt_p(k - w, d); };
    auto B_at = [&](int32_t k) { return k < w ? entry_B(k) : draft_B(k - w); };
    auto step_dt = [&](uint16_t lo, uint16_t hi) {
        float v = (dt_f32 ? __uint_as_float(uint32_t(lo) | (uint32_t(hi) << 16)) : from_bits<IT>(lo)) + bias_h;
        if (flags & kSoftplus)
            v = softplus(v);
        return v;
    };

    // the checkpoint tile (zeros for the pad id; rows past the dim read the
    // last row, their results are never stored)
    SPack S[PASSES][NCH];
    if (pad) {  // uniform
#pragma unroll
        for (int q = 0; q < PASSES; q++)
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    S[q][c].v[k] = narrow<ST>(0.0f);
    } else {
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d0 = dw + q * kRowsPerPass + rsub;
            const uint32_t d = d0 < P ? d0 : P - 1;
#pragma unroll
            for (int c = 0; c < NCH; c++)
                S[q][c] = load_state(reinterpret_cast<const SPack *>(
                    sbase + (d * N + static_cast<uint32_t>(c * kLanesPerRow * VEC + col * VEC))));
        }
    }

    if (fold) {
        // the committed entries, one plain update after the other, one entry
        // ahead in loads
        struct StepIn {
            RawWords<IT, IVEC> b[NCH];
            Bits x;
            uint16_t dt_lo, dt_hi;
        };
        auto fetch_entry = [&](int32_t j, StepIn &in) {
#pragma unroll
            for (int c = 0; c < NCH; c++)
                in.b[c] = load_words<IT, IVEC>(entry_B(j) + c * kLanesPerRow * IVEC);
            // a lane that owns no row reads the first draft's x and dt (read
            // only, unused) rather than a buffer row another lane appends to
            in.x = *reinterpret_cast<const Bits *>(owner ? entry_x(j, d_own) : draft_x(0, 0));
            const unsigned char *dp =
                owner || rp.dt_per_head ? entry_dt_p(j, owner ? d_own : 0) : draft_dt_p(0, 0);
            in.dt_lo = *reinterpret_cast<const uint16_t *>(dp);
            in.dt_hi = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        };
        auto apply = [&](const StepIn &in) {
            const float v = step_dt(in.dt_lo, in.dt_hi);
            const float decay = exp_hw(v * a_h);
            const float dtx = v * from_bits<IT>(in.x);
            float Bv[E];
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int k = 0; k < IVEC; k++)
                    Bv[c * IVEC + k] = word_elem(in.b[c], k);
            for_passes<0, PASSES>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const float dq = row16_bcast<q>(decay);
                const float tq = row16_bcast<q>(dtx);
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < VEC; k++)
                        S[q][c].v[k] = narrow<ST>(fmaf(widen(S[q][c].v[k]), dq, tq * Bv[c * VEC + k]));
            });
        };
        if (hc > 0) {
            StepIn in0, in1;
            fetch_entry(0, in0);
            for (int32_t j = 0; j < hc; j += 2) {
                __builtin_amdgcn_sched_barrier(0);
                fetch_entry(j + 1 < hc ? j + 1 : hc - 1, in1);
                __builtin_amdgcn_sched_barrier(0);
                apply(in0);
                if (j + 1 >= hc)
                    break;
                __builtin_amdgcn_sched_barrier(0);
                fetch_entry(j + 2 < hc ? j + 2 : hc - 1, in0);
                __builtin_amdgcn_sched_barrier(0);
                apply(in1);
            }
        }
        if (write) {
#pragma unroll
            for (int q = 0; q < PASSES; q++) {
                const int d = dw + q * kRowsPerPass + rsub;
                if (d < P) {
                    ST *dst = sbase + static_cast<int64_t>(d) * N + col * VEC;
#pragma unroll
                    for (int c = 0; c < NCH; c++)
                        store_state<SSU_NT_STORE>(
                            reinterpret_cast<SPack *>(dst + c * kLanesPerRow * VEC), S[q][c]);
                }
            }
        }
    }

    // the drafts, kSpecGroup at a time
    const int kseg = col / PASSES;
    const int d_win = dw + (col % PASSES) * kRowsPerPass + rsub;
    const int d_wf = d_win < P ? d_win : 0;
    for (int32_t t0 = 0; t0 < T; t0 += TG) {
        const int32_t W = w + (T < t0 + TG ? T : t0 + TG);  // window steps this group sees
        const int32_t SL = (W + NSEG - 1) / NSEG;
        // the group's C (the lane's columns, raw) and the owner row's x, z, dt
        RawWords<IT, IVEC> cw[TG][NCH];
        Bits xo[TG], zo[TG];
        uint16_t dlo[TG], dhi[TG];
#pragma unroll
        for (int i = 0; i < TG; i++) {
            const int32_t t = t0 + i < T ? t0 + i : T - 1;
            const IT *cp = Cs + (row(t) * p.C_sr + g * p.C_sg + col * IVEC);
#pragma unroll
            for (int c = 0; c < NCH; c++)
                cw[i][c] = load_words<IT, IVEC>(cp + c * kLanesPerRow * IVEC);
            xo[i] = *reinterpret_cast<const Bits *>(draft_x(t, d_fetch));
            zo[i] = *reinterpret_cast<const Bits *>(
                zs ? zs + (row(t) * p.z_sr + h * p.z_sh + d_fetch) : draft_x(t, d_fetch));
            const unsigned char *dp = draft_dt_p(t, d_fetch);
            dlo[i] = *reinterpret_cast<const uint16_t *>(dp);
            dhi[i] = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        }

        struct WinIn {
            RawWords<IT, IVEC> b[NDOT][NCH];
            Bits x;
            uint16_t dt_lo, dt_hi;
        };
        auto fetch_win = [&](int32_t st, WinIn &in) {
#pragma unroll
            for (int rr = 0; rr < NDOT; rr++) {
                const int kd = NSEG < kRowsPerPass ? rsub % NSEG : rr * kRowsPerPass + rsub;
                const int32_t jd = kd * SL + st;
                const IT *src = B_at(jd < W ? jd : W - 1);
#pragma unroll
                for (int c = 0; c < NCH; c++)
                    in.b[rr][c] = load_words<IT, IVEC>(src + c * kLanesPerRow * IVEC);
            }
            const int32_t j = kseg * SL + st;
            const int32_t jc = j < W ? j : W - 1;
            in.x = *x_at(jc, d_wf);
            const unsigned char *dp = dt_at(jc, d_wf);
            in.dt_lo = *reinterpret_cast<const uint16_t *>(dp);
            in.dt_hi = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        };
        float R[TG], Gp[TG];
#pragma unroll
        for (int i = 0; i < TG; i++) {
            R[i] = 0.0f;
            Gp[i] = 1.0f;
        }
        auto run_win = [&](int32_t st, const WinIn &in) {
            float wv[TG];
#pragma unroll
            for (int i = 0; i < TG; i++)
                wv[i] = 0.0f;
#pragma unroll
            for (int rr = 0; rr < NDOT; rr++) {
                float Bd[E];
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < IVEC; k++)
                        Bd[c * IVEC + k] = word_elem(in.b[rr][c], k);
                const int src = ((kseg % kRowsPerPass) * kLanesPerRow + col) * 4;
#pragma unroll
                for (int i = 0; i < TG; i++) {
                    float part = 0.0f;
#pragma unroll
                    for (int c = 0; c < NCH; c++)
#pragma unroll
                        for (int k = 0; k < IVEC; k++)
                            part = fmaf(Bd[c * IVEC + k], word_elem(cw[i][c], k), part);
                    const float dot = row16_sum(part);
                    const float got = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dot)));
                    wv[i] = kseg / kRowsPerPass == rr ? got : wv[i];
                }
            }
            const int32_t j = kseg * SL + st;
            const float v = step_dt(in.dt_lo, in.dt_hi);
            const float alpha = exp_hw(v * a_h);
            const float cx = v * from_bits<IT>(in.x);
#pragma unroll
            for (int i = 0; i < TG; i++) {
                const bool vis = j < W && j <= w + t0 + i;  // causal mask
                R[i] = vis ? fmaf(R[i], alpha, cx * wv[i]) : R[i];
                Gp[i] = vis ? Gp[i] * alpha : Gp[i];
            }
        };
        constexpr int kWinWords = NDOT * NCH * RawWords<IT, IVEC>::kWords + 2;
        constexpr int T0 = 2 < 32 / kWinWords ? 2 : (32 / kWinWords < 1 ? 1 : 32 / kWinWords);
        WinIn wb[T0];
        fetch_win(0, wb[0]);
#pragma unroll
        for (int i = 1; i < T0; i++)
            if (i < SL)  // uniform
                fetch_win(i, wb[i]);
#pragma unroll
        for (int i = 0; i < T0; i++)
            if (i < SL)
                run_win(i, wb[i]);
        WinIn w0, w1;
        if (SL > T0) {
            fetch_win(T0, w0);
            for (int32_t st = T0; st < SL; st += 2) {
                __builtin_amdgcn_sched_barrier(0);
                fetch_win(st + 1 < SL ? st + 1 : SL - 1, w1);
                __builtin_amdgcn_sched_barrier(0);
                run_win(st, w0);
                if (st + 1 >= SL)
                    break;
                __builtin_amdgcn_sched_barrier(0);
                fetch_win(st + 2 < SL ? st + 2 : SL - 1, w0);
                __builtin_amdgcn_sched_barrier(0);
                run_win(st + 1, w1);
            }
        }
        // join the runs in step order, per draft
        for_passes<0, 4>([&](auto lc) {
            constexpr int span = PASSES << decltype(lc)::value;
            if constexpr (span < kLanesPerRow) {
                constexpr int ctrl = 0x120 + (kLanesPerRow - span);  // row_ror: lane i reads lane i + span
#pragma unroll
                for (int i = 0; i < TG; i++) {
                    const float Rn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R[i]), ctrl, 0xF, 0xF, false));
                    const float Gn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(Gp[i]), ctrl, 0xF, 0xF, false));
                    R[i] = fmaf(R[i], Gn, Rn);
                    Gp[i] = Gp[i] * Gn;
                }
            }
        });
        // u_t = S . C_t of the owner rows: all drafts of the group in one
        // sweep over the tile when their decoded C fits in about 32
        // registers, else one draft at a time
        float u[TG];
        auto sweep = [&](auto ni_c, int i0) {
            constexpr int NI = decltype(ni_c)::value;
            float Cd[NI][E];
#pragma unroll
            for (int i = 0; i < NI; i++)
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < IVEC; k++)
                        Cd[i][c * IVEC + k] = word_elem(cw[i0 + i][c], k);
            float uu[NI];
#pragma unroll
            for (int i = 0; i < NI; i++)
                uu[i] = 0.0f;
            for_passes<0, PASSES>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                float acc[NI];
#pragma unroll
                for (int i = 0; i < NI; i++)
                    acc[i] = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < VEC; k++) {
                        const float sv = widen(S[q][c].v[k]);
#pragma unroll
                        for (int i = 0; i < NI; i++)
                            acc[i] = fmaf(sv, Cd[i][c * VEC + k], acc[i]);
                    }
#pragma unroll
                for (int i = 0; i < NI; i++) {
                    const float sum = row16_sum(acc[i]);
                    uu[i] = col == q ? sum : uu[i];
                }
            });
#pragma unroll
            for (int i = 0; i < NI; i++)
                u[i0 + i] = uu[i];
        };
        if constexpr (TG * E <= 32)
            sweep(std::integral_constant<int, TG>(), 0);
        // y of each draft: G u + R + D x, gated
#pragma unroll
        for (int i = 0; i < TG; i++) {
            if constexpr (TG * E > 32) {
                u[i] = 0.0f;
                for_passes<0, PASSES>([&](auto qc) {
                    constexpr int q = decltype(qc)::value;
                    float acc = 0.0f;
#pragma unroll
                    for (int c = 0; c < NCH; c++)
#pragma unroll
                        for (int k = 0; k < VEC; k++)
                            acc = fmaf(widen(S[q][c].v[k]), word_elem(cw[i][c], k), acc);
                    const float sum = row16_sum(acc);
                    u[i] = col == q ? sum : u[i];
                });
            }
            if (owner && t0 + i < T) {
                float y = fmaf(Gp[i], u[i], R[i]) + d_h * from_bits<IT>(xo[i]);
                if (zs)
                    y *= silu(from_bits<IT>(zo[i]));
                ys[row(t0 + i) * p.out_sr + h * p.out_sh + d_own] = narrow<IT>(bad ? __builtin_nanf("") : y);
            }
        }
        // append the group's drafts at entries w + t: the owner rows' x and
        // per-dim dt (B and a per-head dt: ssu_replay_spec_append_kernel)
        if (write && owner) {
#pragma unroll
            for (int i = 0; i < TG; i++) {
                if (t0 + i >= T)
                    break;
                const int64_t e = sl + w + t0 + i;
                *reinterpret_cast<Bits *>(bxs + (e * H + h) * P + d_own) = xo[i];
                if (!rp.dt_per_head) {
                    unsigned char *dst = bdts + ((e * H + h) * P + d_own) * dt_bytes;
                    if (dt_f32)
                        *reinterpret_cast<uint32_t *>(dst) = uint32_t(dlo[i]) | (uint32_t(dhi[i]) << 16);
                    else
                        *reinterpret_cast<uint16_t *>(dst) = dlo[i];
                }
            }
        }
    }
}

// The speculative step's appends that other workgroups of the step read:
// the drafts' B rows (every head of a group) and a per-head dt (every dim
// tile of a head), written to entries w .. w+T-1 after the step's kernel has
// ended (same stream). One workgroup per (sequence, draft); the sequence's
// slot, pointer, fold decision and write rule are those of the step.
// IO_BYTES / DT_BYTES: element sizes of the x dtype and the dt dtype.
template <int IO_BYTES, int DT_BYTES>
__global__ __launch_bounds__(kSpecAppendThreads) void ssu_replay_spec_append_kernel(const Params p,
                                                                                   const ReplayParams rp) {
    using IOW = std::conditional_t<IO_BYTES == 2, uint16_t, uint32_t>;
    using DTW = std::conditional_t<DT_BYTES == 2, uint16_t, uint32_t>;
    const int32_t T = p.steps;
    const int32_t b = blockIdx.x / T;
    const int32_t t = blockIdx.x % T;
    const int flags = p.flags;
    const int64_t s = p.rtab ? load_index(p.rtab, flags & kReadI64, b * p.r_s0) : b;
    if (s == p.pad || (flags & kDisable))
        return;
    const int64_t h_in = load_index(rp.buf_len, rp.len_i64, b * rp.len_s);
    if (h_in < 0 || h_in > rp.L)
        return;
    const int32_t hc = static_cast<int32_t>(h_in);
    const int32_t w = hc + 2 * T > rp.L ? 0 : hc;
    const int64_t e = s * rp.L + w + t;  // the buffer entry
    const int32_t r = b * T + t;         // the draft's row
    const int32_t N = p.P == 0 ? 0 : static_cast<int32_t>(p.slot_stride / (static_cast<int64_t>(p.H) * p.P));
    const IOW *const Bs = static_cast<const IOW *>(p.B);
    IOW *const bB = static_cast<IOW *>(rp.buf_B) + e * rp.G * N;
    for (int32_t i = threadIdx.x; i < rp.G * N; i += blockDim.x) {
        const int32_t g = i / N, n = i - g * N;
        bB[i] = Bs[r * p.B_sr + g * p.B_sg + n];
    }
    if (rp.dt_per_head) {
        const DTW *const dts = static_cast<const DTW *>(p.dt);
        DTW *const bdt = static_cast<DTW *>(rp.buf_dt) + e * p.H;
        for (int32_t h = threadIdx.x; h < p.H; h += blockDim.x)
            bdt[h] = dts[r * p.dt_sr + h * p.dt_sh];
    }
}

template <typename ST, typename IT, bool SPEC>
bool pick_replay_n(int n, KernelRef *k) {
    switch (n) {
#define SSU_CASE(NN)                                                                     \
    case NN:                                                                             \
        k->fn = SPEC ? reinterpret_cast<const void *>(&ssu_replay_spec_kernel<ST, IT, NN>) \
                     : reinterpret_cast<const void *>(&ssu_replay_kernel<ST, IT, NN, 0>);      \
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

template <typename ST, bool SPEC>
bool pick_replay_io(int io, int n, KernelRef *k) {
    switch (io) {
    case SSU_F32: return pick_replay_n<ST, float, SPEC>(n, k);
    case SSU_F16: return pick_replay_n<ST, _Float16, SPEC>(n, k);
    case SSU_BF16: return pick_replay_n<ST, __bf16, SPEC>(n, k);
    }
    return false;
}


}  // namespace

bool find_replay_kernel(int state_dtype, int io_dtype, int dstate, bool spec, KernelRef *out) {
    switch (state_dtype) {
    case SSU_F32:
        return spec ? pick_replay_io<float, true>(io_dtype, dstate, out)
                    : pick_replay_io<float, false>(io_dtype, dstate, out);
    case SSU_F16:
        return spec ? pick_replay_io<_Float16, true>(io_dtype, dstate, out)
                    : pick_replay_io<_Float16, false>(io_dtype, dstate, out);
    case SSU_BF16:
        return spec ? pick_replay_io<__bf16, true>(io_dtype, dstate, out)
                    : pick_replay_io<__bf16, false>(io_dtype, dstate, out);
    }
    return false;
}

template <typename IT, int LPF>
bool pick_replay_lp_n(int n, KernelRef *k) {
    switch (n) {
    case 32: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 32, LPF>); return true;
    case 64: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 64, LPF>); return true;
    case 128: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 128, LPF>); return true;
    case 256: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 256, LPF>); return true;
    }
    return false;
}

bool find_replay_lp_kernel(int io_dtype, int dstate, int bits, KernelRef *out) {
    if (bits == 4) {
        switch (io_dtype) {
        case SSU_F32: return pick_replay_lp_n<float, 4>(dstate, out);
        case SSU_F16: return pick_replay_lp_n<_Float16, 4>(dstate, out);
        case SSU_BF16: return pick_replay_lp_n<__bf16, 4>(dstate, out);
        }
        return false;
    }
    switch (io_dtype) {
    case SSU_F32: return pick_replay_lp_n<float, 8>(dstate, out);
    case SSU_F16: return pick_replay_lp_n<_Float16, 8>(dstate, out);
    case SSU_BF16: return pick_replay_lp_n<__bf16, 8>(dstate, out);
    }
    return false;
}

// MXFP8 quantization: 4 lanes per block of 32 values (8 each), grid-stride
__global__ __launch_bounds__(256) void mx8_quantize_kernel(const float *src, uint8_t *codes, uint8_t *scales,
                                                           int64_t nblocks) {
    const int64_t lanes = static_cast<int64_t>(gridDim.x) * blockDim.x;
    // every lane of a wave runs the same number of iterations (the shuffles need all lanes)
    const int64_t total = (nblocks * 4 + 63) / 64 * 64;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (total + lanes - 1) / lanes * lanes;
         i += lanes) {
        const bool live = i < nblocks * 4;
        const int64_t at = (live ? i : 0) * 8;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(src + at);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(src + at + 4);
        float v[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w),
                      __uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++)
            amax = fmaxf(amax, fabsf(v[k]));
        amax = group_max<4>(amax);
        const int kexp = mx8_exponent(amax);
        const uint32_t lo = e4m3_codes4(v, kexp);
        const uint32_t hi = e4m3_codes4(v + 4, kexp);
        if (live) {
            *reinterpret_cast<u32x2 *>(codes + at) = u32x2{lo, hi};
            if ((i & 3) == 0)
                scales[i / 4] = static_cast<uint8_t>(kexp + 127);
        }
    }
}

// MXFP4 quantization: 4 lanes per block of 32 values (8 each: 4 bytes of
// codes), grid-stride
__global__ __launch_bounds__(256) void mx4_quantize_kernel(const float *src, uint8_t *codes, uint8_t *scales,
                                                           int64_t nblocks) {
    const int64_t lanes = static_cast<int64_t>(gridDim.x) * blockDim.x;
    // every lane of a wave runs the same number of iterations (the shuffles need all lanes)
    const int64_t total = (nblocks * 4 + 63) / 64 * 64;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (total + lanes - 1) / lanes * lanes;
         i += lanes) {
        const bool live = i < nblocks * 4;
        const int64_t at = (live ? i : 0) * 8;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(src + at);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(src + at + 4);
        float v[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w),
                      __uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++)
            amax = fmaxf(amax, fabsf(v[k]));
        amax = group_max<4>(amax);
        const int kexp = mx4_exponent(amax);
        const uint32_t lo = e2m1_codes4(v, kexp);
        const uint32_t hi = e2m1_codes4(v + 4, kexp);
        if (live) {
            *reinterpret_cast<uint32_t *>(codes + at / 2) = lo | (hi << 16);
            if ((i & 3) == 0)
                scales[i / 4] = static_cast<uint8_t>(kexp + 127);
        }
    }
}

int launch_mx4_quantize(const float *src, uint8_t *codes, uint8_t *scales, int64_t nblocks, void *stream) {
    int64_t blocks = (nblocks * 4 + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks);
    void *args[] = {const_cast<float **>(&src), &codes, &scales, &nblocks};
    return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void *>(&mx4_quantize_kernel),
                                            dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

int launch_mx8_quantize(const float *src, uint8_t *codes, uint8_t *scales, int64_t nblocks, void *stream) {
    int64_t blocks = (nblocks * 4 + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks);
    void *args[] = {const_cast<float **>(&src), &codes, &scales, &nblocks};
    return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void *>(&mx8_quantize_kernel),
                                            dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

int launch_replay(const KernelRef &k, const Params &p, const ReplayParams &rp, unsigned grid,
                  unsigned block, void *stream) {
    Params pc = p;
    ReplayParams rc = rp;
    void *args[] = {&pc, &rc};
    return static_cast<int>(hipLaunchKernel(k.fn, dim3(grid), dim3(block), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

int launch_replay_spec_append(const Params &p, const ReplayParams &rp, int io_bytes, int dt_bytes,
                              unsigned grid, void *stream) {
    const void *fn = io_bytes == 2 ? (dt_bytes == 2 ? reinterpret_cast<const void *>(&ssu_replay_spec_append_kernel<2, 2>)
                                                    : reinterpret_cast<const void *>(&ssu_replay_spec_append_kernel<2, 4>))
                                   : (dt_bytes == 2 ? reinterpret_cast<const void *>(&ssu_replay_spec_append_kernel<4, 2>)
                                                    : reinterpret_cast<const void *>(&ssu_replay_spec_append_kernel<4, 4>));
    Params pc = p;
    ReplayParams rc = rp;
    void *args[] = {&pc, &rc};
    return static_cast<int>(hipLaunchKernel(fn, dim3(grid), dim3(kSpecAppendThreads), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace ssu
