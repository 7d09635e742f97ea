// gfx950 kernels of ReplaySSM (ReplaySSM article, sections "核心做法" and
// "投机解码回滚变成挪指针"): the one-token replay step over a checkpoint and a
// buffer of past raw inputs, its variant with an MXFP8 read copy of the
// checkpoint, the speculative step over T draft tokens, and the MXFP8
// quantizer that makes the first copy of a pool.

#include "ssu_device.h"

namespace ssu {
namespace {

// ReplaySSM decode (ReplaySSM article, section "核心做法"): one workgroup per
// (sequence, head, dim tile), the checkpoint tile in ssu_kernel's lane
// layout. A step with h buffered entries either fills the buffer (h + 1 == L:
// replay the buffered steps and the current one through the update, exactly
// as ssu_kernel applies a token, then y and the checkpoint store) or is
// output-only: the checkpoint tile is streamed once for u = S_ckpt . C and
// each dim row's window term over the steps j = 0..h,
//   R <- R a_j + dt'_j x_j (B_j . C),   G <- G a_j,
// gives y = G u + R + D x, gated; the step's raw inputs go to buffer entry h.
// The output-only window is split into NSEG contiguous runs of steps: lane
// col of a DPP row takes dim row col % PASSES and run col / PASSES, and the
// runs' (R, G) pairs are then joined in step order ((R0, G0) followed by
// (R1, G1) is (R0 G1 + R1, G0 G1)). Each B_j . C is formed once per DPP row
// and handed to the lanes whose step it is. An entry count outside [0, L)
// (not for the pad id) makes the sequence's y NaN and writes nothing.
template <typename ST, typename IT, int N, bool LP>
__global__ __launch_bounds__(kMaxWaves *kWaveLanes, replay_waves_per_eu(sizeof(ST), N)) void ssu_replay_kernel(
    const Params p, const ReplayParams rp) {
    constexpr int E = N / kLanesPerRow;
    constexpr int VEC = (16 / (int)sizeof(ST)) < E ? (16 / (int)sizeof(ST)) : E;
    constexpr int NCH = E / VEC;
    constexpr int PASSES = passes_for(N, sizeof(ST), kTileReplay);
    constexpr int IVEC = VEC;
    // window runs per dim row, and B . C rounds (one per DPP row) per window step
    constexpr int NSEG = kLanesPerRow / PASSES;
    constexpr int NDOT = NSEG < kRowsPerPass ? 1 : NSEG / kRowsPerPass;
    static_assert(PASSES <= kLanesPerRow && kLanesPerRow % PASSES == 0, "runs tile the row");
    static_assert(!LP || (sizeof(ST) == 4 && VEC >= 2 && N % 32 == 0), "MX blocks span whole lanes of a row");
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

    const int64_t s = p.rtab ? load_index(p.rtab, flags & kReadI64, b * p.r_s0) : b;
    const bool pad = s == p.pad;  // no checkpoint and no buffer: h is taken as 0
    const int64_t h_in = pad ? 0 : load_index(rp.buf_len, rp.len_i64, b * rp.len_s);
    const bool bad = h_in < 0 || h_in >= rp.L;
    const int32_t hb = bad ? 0 : static_cast<int32_t>(h_in);
    const bool flush = !bad && hb + 1 == rp.L;
    const bool write = !pad && !bad && !(flags & kDisable);
    const bool dt_f32 = flags & kDtF32;
    const int dt_bytes = dt_f32 ? 4 : 2;

    const int P = p.P, H = p.H;
    const int64_t tile_off = static_cast<int64_t>(h) * P * N;
    ST *const sbase = static_cast<ST *>(p.state) + (pad ? 0 : s) * p.slot_stride + tile_off;
    const int64_t sl = (pad ? 0 : s) * rp.L;  // first buffer entry of the slot
    const IT *const xs = static_cast<const IT *>(p.x);
    const IT *const zs = static_cast<const IT *>(p.z);
    IT *const ys = static_cast<IT *>(p.out);
    const unsigned char *const dts = static_cast<const unsigned char *>(p.dt);
    const IT *const Bcur = static_cast<const IT *>(p.B) + (b * p.B_sr + g * p.B_sg + col * IVEC);
    const IT *const Ccur = static_cast<const IT *>(p.C) + (b * p.C_sr + g * p.C_sg + col * IVEC);
    IT *const bxs = static_cast<IT *>(rp.buf_x);
    IT *const bBs = static_cast<IT *>(rp.buf_B);
    unsigned char *const bdts = static_cast<unsigned char *>(rp.buf_dt);

    const float a_h = p.A[h * p.A_sh];
    const float d_h = p.D ? p.D[h * p.D_sh] : 0.0f;
    const float bias_h = p.dt_bias ? p.dt_bias[h * p.bias_sh] : 0.0f;

    // Inputs of step j (j < hb: buffer entry j; j == hb: the current step)
    // for dim row d, which must be in range: a uniform base (the slot's
    // entry 0 at this head or group, or the current row) plus a 32-bit lane
    // offset (one slot's buffer spans fewer than 2^31 elements).
    const IT *const bx0 = bxs + (sl * H + h) * P;
    const unsigned char *const bdt0 = bdts + (rp.dt_per_head ? sl * H + h : (sl * H + h) * P) * dt_bytes;
    const IT *const bB0 = bBs + (sl * rp.G + g) * N + col * IVEC;
    const IT *const xcur0 = xs + (b * p.x_sr + h * p.x_sh);
    const unsigned char *const dtcur0 = dts + static_cast<int64_t>(b * p.dt_sr + h * p.dt_sh) * dt_bytes;
    const uint32_t HP = static_cast<uint32_t>(H * P), GN = static_cast<uint32_t>(rp.G * N);
    auto x_at = [&](int32_t j, int d) -> const Bits * {
        const IT *q = j < hb ? bx0 + (static_cast<uint32_t>(j) * HP + d) : xcur0 + static_cast<uint32_t>(d);
        return reinterpret_cast<const Bits *>(q);
    };
    auto dt_at = [&](int32_t j, int d) -> const unsigned char * {
        return j < hb ? bdt0 + (static_cast<uint32_t>(j) * (rp.dt_per_head ? H : HP) +
                                (rp.dt_per_head ? 0u : static_cast<uint32_t>(d))) * dt_bytes
                      : dtcur0 + static_cast<uint32_t>(d * p.dt_sp * dt_bytes);
    };
    auto B_at = [&](int32_t j) -> const IT * {
        return j < hb ? bB0 + static_cast<uint32_t>(j) * GN : Bcur;
    };
    auto step_dt = [&](uint16_t lo, uint16_t hi) {
        float v = (dt_f32 ? __uint_as_float(uint32_t(lo) | (uint32_t(hi) << 16)) : from_bits<IT>(lo)) + bias_h;
        if (flags & kSoftplus)
            v = softplus(v);
        return v;
    };

    // the lane's columns of C, the owner row's x and z (z read from x when
    // there is no gate, to keep the load unconditional), the checkpoint tile
    RawWords<IT, IVEC> cw[NCH];
    Bits x_bits, z_bits;
    uint16_t dto_lo, dto_hi;  // the owner row's dt, for the append
    SPack S[PASSES][NCH];
    auto load_current = [&]() {
#pragma unroll
        for (int c = 0; c < NCH; c++)
            cw[c] = load_words<IT, IVEC>(Ccur + c * kLanesPerRow * IVEC);
        const int64_t xo = b * p.x_sr + h * p.x_sh + d_fetch;
        x_bits = *reinterpret_cast<const Bits *>(xs + xo);
        z_bits = *reinterpret_cast<const Bits *>(zs ? zs + (b * p.z_sr + h * p.z_sh + d_fetch) : xs + xo);
    };
    // The read copy: lanes of one 32-value block (32 / VEC lanes of a row)
    // read VEC codes each and the block's scale byte.
    const int64_t lp_tile = (pad ? 0 : s) * (static_cast<int64_t>(p.H) * P * N) + tile_off;  // byte offset of the tile
    // A row's N / 32 scale bytes (at most 8) come in one load per pass.
    auto load_copy = [&]() {
        if constexpr (LP) {  // compiled for the copy kernels only (their rows hold >= 2 values per lane)
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d0 = dw + q * kRowsPerPass + rsub;
            const int64_t d = d0 < P ? d0 : P - 1;
            const int64_t row = lp_tile + d * N;
            uint64_t sw;
            if constexpr (N / 32 > 4) {
                const uint2 w = *reinterpret_cast<const uint2 *>(rp.lp_scale + row / 32);
                sw = w.x | (static_cast<uint64_t>(w.y) << 32);
            } else if constexpr (N / 32 == 4) {
                sw = *reinterpret_cast<const uint32_t *>(rp.lp_scale + row / 32);
            } else if constexpr (N / 32 == 2) {
                sw = *reinterpret_cast<const uint16_t *>(rp.lp_scale + row / 32);
            } else {
                sw = rp.lp_scale[row / 32];
            }
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const int n0 = c * kLanesPerRow * VEC + col * VEC;
                uint32_t codes;
                if constexpr (VEC == 4)
                    codes = *reinterpret_cast<const uint32_t *>(rp.lp + row + n0);
                else
                    codes = *reinterpret_cast<const uint16_t *>(rp.lp + row + n0);
                const float sc = mx8_scale(static_cast<uint32_t>(sw >> (8 * (n0 / 32))) & 0xFFu);
                const float2 lo = e4m3_pair<false>(codes, sc);
                S[q][c].v[0] = narrow<ST>(lo.x);
                S[q][c].v[1] = narrow<ST>(lo.y);
                if constexpr (VEC == 4) {
                    const float2 hi = e4m3_pair<true>(codes, sc);
                    S[q][c].v[2] = narrow<ST>(hi.x);
                    S[q][c].v[3] = narrow<ST>(hi.y);
                }
            }
        }
        }
    };
    // the folded tile into the read copy (after its fp32 store)
    auto store_copy = [&]() {
        constexpr int kBlockLanes = LP ? 32 / VEC : 2;  // lanes sharing a block
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d = dw + q * kRowsPerPass + rsub;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                float amax = 0.0f;
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    amax = fmaxf(amax, fabsf(widen(S[q][c].v[k])));
                amax = group_max<kBlockLanes>(amax);
                const int kexp = mx8_exponent(amax);
                float v4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    v4[k] = widen(S[q][c].v[k]);
                const uint32_t codes = e4m3_codes4(v4, kexp);
                if (d < P) {
                    const int64_t n0 = c * kLanesPerRow * VEC + col * VEC;
                    const int64_t at = lp_tile + static_cast<int64_t>(d) * N + n0;
                    if constexpr (VEC == 4)
                        *reinterpret_cast<uint32_t *>(rp.lp + at) = codes;
                    else
                        *reinterpret_cast<uint16_t *>(rp.lp + at) = static_cast<uint16_t>(codes);
                    if (col % kBlockLanes == 0)
                        rp.lp_scale[at / 32] = static_cast<uint8_t>(kexp + 127);
                }
            }
        }
    };
    // (rows past the dim read the last row; their results are never stored)
    auto load_checkpoint = [&]() {
        if (pad) {  // uniform
#pragma unroll
            for (int q = 0; q < PASSES; q++)
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < VEC; k++)
                        S[q][c].v[k] = narrow<ST>(0.0f);
            return;
        }
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int d0 = dw + q * kRowsPerPass + rsub;
            const uint32_t d = d0 < P ? d0 : P - 1;
#pragma unroll
            for (int c = 0; c < NCH; c++)
                S[q][c] = load_state(reinterpret_cast<const SPack *>(
                    sbase + (d * N + static_cast<uint32_t>(c * kLanesPerRow * VEC + col * VEC))));
        }
    };
    float Cv[E];
    auto decode_C = [&]() {
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int k = 0; k < IVEC; k++)
                Cv[c * IVEC + k] = word_elem(cw[c], k);
    };

    float ysum = 0.0f;
    if (flush) {
        // Replay the buffered steps and the current one through the update,
        // one step ahead in loads (two buffers, scheduling barriers: the
        // vector-memory counter is in order; the prefetch past the last step
        // reloads the last step, so no branch joins pending loads).
        struct StepIn {
            RawWords<IT, IVEC> b[NCH];
            Bits x;
            uint16_t dt_lo, dt_hi;
        };
        auto fetch_step = [&](int32_t j, StepIn &in) {
            const IT *bsrc = B_at(j);
#pragma unroll
            for (int c = 0; c < NCH; c++)
                in.b[c] = load_words<IT, IVEC>(bsrc + c * kLanesPerRow * IVEC);
            in.x = *x_at(j, d_fetch);
            const unsigned char *dp = dt_at(j, d_fetch);
            in.dt_lo = *reinterpret_cast<const uint16_t *>(dp);
            in.dt_hi = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        };
        auto run = [&](int32_t j, const StepIn &in) {
            const float v = step_dt(in.dt_lo, in.dt_hi);
            const float decay = exp_hw(v * a_h);
            const float dtx = v * from_bits<IT>(in.x);
            const bool last = j == hb;
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
                float acc = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; c++) {
#pragma unroll
                    for (int k = 0; k < VEC; k++) {
                        const int e = c * VEC + k;
                        const float sv = fmaf(widen(S[q][c].v[k]), dq, tq * Bv[e]);
                        acc = fmaf(sv, Cv[e], acc);
                        S[q][c].v[k] = narrow<ST>(sv);
                    }
                }
                if (last) {
                    const float sum = row16_sum(acc);
                    ysum = col == q ? sum : ysum;
                }
            });
        };
        StepIn in0, in1;
        fetch_step(0, in0);
        load_current();
        load_checkpoint();
        decode_C();
        for (int32_t j = 0; j <= hb; j += 2) {
            __builtin_amdgcn_sched_barrier(0);
            fetch_step(j + 1 <= hb ? j + 1 : hb, in1);
            __builtin_amdgcn_sched_barrier(0);
            run(j, in0);
            if (j + 1 > hb)
                break;
            __builtin_amdgcn_sched_barrier(0);
            fetch_step(j + 2 <= hb ? j + 2 : hb, in0);
            __builtin_amdgcn_sched_barrier(0);
            run(j + 1, in1);
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
            if constexpr (LP)
                store_copy();
        }
    } else {
        // the lane's window row and run; run k holds steps k*SL .. k*SL+SL-1
        const int kseg = col / PASSES;
        const int d_win = dw + (col % PASSES) * kRowsPerPass + rsub;
        const int d_wf = d_win < P ? d_win : 0;
        const int32_t SL = (hb + NSEG) / NSEG;  // ceil((hb + 1) / NSEG)
        struct WinIn {
            RawWords<IT, IVEC> b[NDOT][NCH];  // B rows this DPP row dots with C
            Bits x;
            uint16_t dt_lo, dt_hi;
        };
        // loads for the t-th step of every run (steps past hb reload step hb)
        auto fetch_win = [&](int32_t t, WinIn &in) {
#pragma unroll
            for (int rr = 0; rr < NDOT; rr++) {
                const int kd = NSEG < kRowsPerPass ? rsub % NSEG : rr * kRowsPerPass + rsub;
                const int32_t jd = kd * SL + t;
                const IT *src = B_at(jd < hb ? jd : hb);
#pragma unroll
                for (int c = 0; c < NCH; c++)
                    in.b[rr][c] = load_words<IT, IVEC>(src + c * kLanesPerRow * IVEC);
            }
            const int32_t j = kseg * SL + t;
            const int32_t jc = j < hb ? j : hb;
            in.x = *x_at(jc, d_wf);
            const unsigned char *dp = dt_at(jc, d_wf);
            in.dt_lo = *reinterpret_cast<const uint16_t *>(dp);
            in.dt_hi = *reinterpret_cast<const uint16_t *>(dp + (dt_f32 ? 2 : 0));
        };
        float R = 0.0f, G = 1.0f;
        auto run_win = [&](int32_t t, const WinIn &in) {
            // B_jd . C for this DPP row's steps, then the lane's own one:
            // run k's value sits in DPP row k % 4 of round k / 4
            float w = 0.0f;
#pragma unroll
            for (int rr = 0; rr < NDOT; rr++) {
                float part = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; c++)
#pragma unroll
                    for (int k = 0; k < IVEC; k++)
                        part = fmaf(word_elem(in.b[rr][c], k), Cv[c * IVEC + k], part);
                const float dot = row16_sum(part);
                const int src = ((kseg % kRowsPerPass) * kLanesPerRow + col) * 4;
                const float got = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dot)));
                w = kseg / kRowsPerPass == rr ? got : w;
            }
            const int32_t j = kseg * SL + t;
            const bool valid = j <= hb;
            const float v = step_dt(in.dt_lo, in.dt_hi);
            const float alpha = valid ? exp_hw(v * a_h) : 1.0f;
            const float term = valid ? v * from_bits<IT>(in.x) * w : 0.0f;
            R = fmaf(R, alpha, term);
            G = G * alpha;
        };
        // the first T0 steps of every run are requested before the tile
        // (as many as about 32 registers hold)
        constexpr int kWinWords = NDOT * NCH * RawWords<IT, IVEC>::kWords + 2;
        constexpr int T0 = SSU_REPLAY_PREFETCH < 32 / kWinWords ? SSU_REPLAY_PREFETCH
                           : (32 / kWinWords < 1 ? 1 : 32 / kWinWords);
        WinIn wb[T0];
        fetch_win(0, wb[0]);
#pragma unroll
        for (int i = 1; i < T0; i++)
            if (i < SL)  // uniform
                fetch_win(i, wb[i]);
        load_current();
        const unsigned char *dpo = dt_at(hb, d_fetch);
        dto_lo = *reinterpret_cast<const uint16_t *>(dpo);
        dto_hi = *reinterpret_cast<const uint16_t *>(dpo + (dt_f32 ? 2 : 0));
        if constexpr (LP) {
            if (pad)
                load_checkpoint();  // zeros
            else
                load_copy();
        } else {
            load_checkpoint();
        }
        decode_C();
#pragma unroll
        for (int i = 0; i < T0; i++)
            if (i < SL)
                run_win(i, wb[i]);
        // longer runs: one step ahead in loads, as in the fold
        WinIn w0, w1;
        if (SL > T0) {
            fetch_win(T0, w0);
            for (int32_t t = T0; t < SL; t += 2) {
                __builtin_amdgcn_sched_barrier(0);
                fetch_win(t + 1 < SL ? t + 1 : SL - 1, w1);
                __builtin_amdgcn_sched_barrier(0);
                run_win(t, w0);
                if (t + 1 >= SL)
                    break;
                __builtin_amdgcn_sched_barrier(0);
                fetch_win(t + 2 < SL ? t + 2 : SL - 1, w0);
                __builtin_amdgcn_sched_barrier(0);
                run_win(t + 1, w1);
            }
        }
        // join the runs in step order: the run PASSES lanes up follows
        for_passes<0, 4>([&](auto lc) {
            constexpr int span = PASSES << decltype(lc)::value;
            if constexpr (span < kLanesPerRow) {
                constexpr int ctrl = 0x120 + (kLanesPerRow - span);  // row_ror: lane i reads lane i + span
                const float Rn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), ctrl, 0xF, 0xF, false));
                const float Gn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(G), ctrl, 0xF, 0xF, false));
                R = fmaf(R, Gn, Rn);
                G = G * Gn;
            }
        });
        // u = S_ckpt . C of the lane's own row (run 0 lanes are the owners)
        float u = 0.0f;
        for_passes<0, PASSES>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int k = 0; k < VEC; k++)
                    acc = fmaf(widen(S[q][c].v[k]), Cv[c * VEC + k], acc);
            const float sum = row16_sum(acc);
            u = col == q ? sum : u;
        });
        ysum = fmaf(G, u, R);
        // append the step's raw inputs at entry hb
        if (write) {
            const int64_t e = sl + hb;
            auto put_dt = [&](unsigned char *dst) {
                if (dt_f32)
                    *reinterpret_cast<uint32_t *>(dst) = uint32_t(dto_lo) | (uint32_t(dto_hi) << 16);
                else
                    *reinterpret_cast<uint16_t *>(dst) = dto_lo;
            };
            if (owner) {
                *reinterpret_cast<Bits *>(bxs + (e * H + h) * P + d_own) = x_bits;
                if (!rp.dt_per_head)
                    put_dt(bdts + ((e * H + h) * P + d_own) * dt_bytes);
            }
            if (rp.dt_per_head && tile == 0 && threadIdx.x == 0)
                put_dt(bdts + (e * H + h) * dt_bytes);  // lane 0 owns a row; dt is the head's
            if (h % p.heads_per_group == 0 && tile == 0 && wave == 0 && rsub == 0) {
                IT *dst = bBs + (e * rp.G + g) * N + col * IVEC;
#pragma unroll
                for (int c = 0; c < NCH; c++) {
                    store_words<IT, IVEC>(dst + c * kLanesPerRow * IVEC,
                                          load_words<IT, IVEC>(Bcur + c * kLanesPerRow * IVEC));
                }
            }
        }
    }

    // y of the lane's own row
    if (owner) {
        float y = ysum + d_h * from_bits<IT>(x_bits);
        if (zs)
            y *= silu(from_bits<IT>(z_bits));
        ys[b * p.out_sr + h * p.out_sh + d_own] = narrow<IT>(bad ? __builtin_nanf("") : y);
    }
}

// ReplaySSM speculative step (ReplaySSM article, section "投机解码回滚变成挪指针"):
// T draft tokens per sequence, packed as rows b*T + t. One workgroup per
// (sequence, head, dim tile), the checkpoint tile in ssu_kernel's layout. If
// h + 2T > L (the fold one window early), the h committed entries are first
// applied to the tile with the plain update's arithmetic (no readout) and the
// tile is stored; the window then starts empty (w = 0), else w = h. Drafts
// are read out kSpecGroup at a time: the window (w committed entries, then
// the drafts up to the group's last) is split into runs as in
// ssu_replay_kernel, every run keeps one (R, G) pair per draft of the group,
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
                     : reinterpret_cast<const void *>(&ssu_replay_kernel<ST, IT, NN, false>);  \
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

template <typename IT>
bool pick_replay_lp_n(int n, KernelRef *k) {
    switch (n) {
    case 32: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 32, true>); return true;
    case 64: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 64, true>); return true;
    case 128: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 128, true>); return true;
    case 256: k->fn = reinterpret_cast<const void *>(&ssu_replay_kernel<float, IT, 256, true>); return true;
    }
    return false;
}

bool find_replay_lp_kernel(int io_dtype, int dstate, KernelRef *out) {
    switch (io_dtype) {
    case SSU_F32: return pick_replay_lp_n<float>(dstate, out);
    case SSU_F16: return pick_replay_lp_n<_Float16>(dstate, out);
    case SSU_BF16: return pick_replay_lp_n<__bf16>(dstate, out);
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
