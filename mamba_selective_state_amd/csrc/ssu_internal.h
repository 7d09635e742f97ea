// Internal interface between the host entry points (ssu_api.cpp) and the
// gfx950 kernels (ssu_kernels.hip) of libssu.
#pragma once

#include <stdint.h>

#include "../../include/ssu.h"

namespace ssu {

// Sets the thread's last-error message (ssu_last_error) and returns `st`.
ssu_status_t report_error(ssu_status_t st, const char *msg);

// How rows are grouped into sequences.
enum Layout : int32_t {
    kOneToken = 0,  // x [batch, heads, dim]: sequence b is row b
    kDense = 1,     // x [batch, steps, heads, dim]: sequence b is rows b*steps ..
    kCuSeqlens = 2  // x [rows, heads, dim] split by cu_seqlens
};

enum Flags : int32_t {
    kDtF32 = 1 << 0,     // dt is f32 (else the x dtype)
    kSoftplus = 1 << 1,  // dt' = softplus(dt + dt_bias)
    kDisable = 1 << 2,   // disable_state_update
    kRead2D = 1 << 3,    // read table is 2-D (else 1-D, row-indexed)
    kReadI64 = 1 << 4,
    kWrite2D = 1 << 5,
    kWriteI64 = 1 << 6,
    kCuI64 = 1 << 7,
    kAccI64 = 1 << 8,
    kFillFirst = 1 << 9  // replay: sequences that fill their buffer are taken first
};

// Geometry of one workgroup: 16 lanes share a dim row (one DPP row), so a
// 64-lane wave covers 4 dim rows per pass; each lane keeps dstate/16 state
// elements of each of its rows in registers.
constexpr int kWaveLanes = 64;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerPass = kWaveLanes / kLanesPerRow;
#ifndef SSU_MAX_WAVES
#define SSU_MAX_WAVES 1
#endif
constexpr int kMaxWaves = SSU_MAX_WAVES;
// Minimum resident waves per SIMD the register allocation must allow, for the
// one-token and the multi-token kernel.
#ifndef SSU_WAVES_PER_EU
#define SSU_WAVES_PER_EU 1
#endif
// The one-token replay kernel: workgroups of kReplayWaves independent waves,
// each on kReplayRows dim rows of one (sequence, head), and the waves per
// SIMD its register allocation must allow.
constexpr int kReplayRows = 64;
constexpr int kReplayWaves = 4;
// Batches up to this size take the filling sequences first (each wave scans
// the buffer counts of the whole batch).
constexpr int kReplayScanMax = 512;
#ifndef SSU_WAVES_PER_EU_REPLAY
#define SSU_WAVES_PER_EU_REPLAY 4
#endif
constexpr int replay_waves_per_eu() { return SSU_WAVES_PER_EU_REPLAY; }
// Window steps per round of the output-only path; slices in flight per
// wave: of the fold, of the output-only read's MXFP8 and MXFP4 copies, and
// 32-bit words of its checkpoint slices.
#ifndef SSU_REPLAY_COPY8_DEPTH
#define SSU_REPLAY_COPY8_DEPTH 4
#endif
#ifndef SSU_REPLAY_COPY4_DEPTH
#define SSU_REPLAY_COPY4_DEPTH 4
#endif
#ifndef SSU_REPLAY_WIN
#define SSU_REPLAY_WIN 8
#endif
#ifndef SSU_REPLAY_FOLD_DEPTH
#define SSU_REPLAY_FOLD_DEPTH 4
#endif
#ifndef SSU_REPLAY_CKPT_WORDS
#define SSU_REPLAY_CKPT_WORDS 32
#endif
// The speculative replay kernel also holds a group of drafts' C and their
// per-draft accumulators.
constexpr int replay_spec_waves_per_eu(int state_bytes, int dstate) {
    return state_bytes == 4 && dstate <= 128 ? 3 : 2;
}
#ifndef SSU_WAVES_PER_EU_MULTI
#define SSU_WAVES_PER_EU_MULTI 4
#endif
// the multi-token kernel's output-only variant on the matrix cores: its
// 64-row tiles (dstate up to 128) need more registers than 4 waves leave
// (3 waves); its tiles of 32 rows or fewer (dstate 256: 16) fit 4
// (SSU_WAVES_PER_EU_YMFMA_32)
#ifndef SSU_WAVES_PER_EU_YMFMA
#define SSU_WAVES_PER_EU_YMFMA 3
#endif
// its VALU form with a 16-bit state (it spills at 4 waves: 159 against 191 us
// with bf16 state and fp16 outputs); with an fp32 state the spilling 4-wave
// build was the faster one (95 against 101 us on MTP)
#ifndef SSU_WAVES_PER_EU_YVALU16
#define SSU_WAVES_PER_EU_YVALU16 3
#endif
#ifndef SSU_WAVES_PER_EU_YMFMA_32
#define SSU_WAVES_PER_EU_YMFMA_32 4
#endif

// Passes (dim rows per lane): enough rows that each lane keeps about
// `lane_bytes` of state in flight (dstate/16 elements per row, in the state
// dtype), between 1 and 8 rows (separate budgets for the one-token and the
// multi-token kernel, which also holds the next token's inputs); up to 16
// for the output-only variant on the matrix cores up to dstate 128, whose
// wave shares its tokens' B and C rows and their products over all of its
// rows (a larger dstate keeps the 16-row tile its A operands fit in at 4
// waves per SIMD).
#ifndef SSU_LANE_BYTES
#define SSU_LANE_BYTES 128
#endif
#ifndef SSU_LANE_BYTES_MULTI
#define SSU_LANE_BYTES_MULTI 128
#endif
#ifndef SSU_LANE_BYTES_REPLAY
#define SSU_LANE_BYTES_REPLAY 128
#endif
// the multi-token kernel's output-only variant, which also holds its tokens'
// per-row inputs
#ifndef SSU_LANE_BYTES_YONLY
#define SSU_LANE_BYTES_YONLY 128
#endif
#ifndef SSU_LANE_BYTES_YMFMA
#define SSU_LANE_BYTES_YMFMA 256
#endif
enum TileKind { kTileOneToken = 0, kTileMulti = 1, kTileReplay = 2, kTileYonly = 3, kTileYonlyMfma = 4 };
constexpr int passes_for(int dstate, int state_bytes, int kind) {
    const int per_row = (dstate / kLanesPerRow) * state_bytes;
    const int budget = kind == kTileMulti       ? SSU_LANE_BYTES_MULTI
                       : kind == kTileReplay    ? SSU_LANE_BYTES_REPLAY
                       : kind == kTileYonly     ? SSU_LANE_BYTES_YONLY
                       : kind == kTileYonlyMfma ? (dstate <= 128 ? SSU_LANE_BYTES_YMFMA : SSU_LANE_BYTES_YONLY)
                                                : SSU_LANE_BYTES;
    const int cap = kind == kTileYonlyMfma ? 16 : 8;
    const int rows = budget / per_row;
    return rows < 1 ? 1 : (rows > cap ? cap : rows);
}

// Kernel arguments. Strides are in elements. The pool is contiguous
// [slots, heads, dim, dstate] and addressed with 64-bit offsets; every other
// tensor spans fewer than 2^31 elements (checked on the host) and is
// addressed with 32-bit offsets: row * sr + head (or group) * sh + d (last
// stride 1, except dt's sp).
struct Params {
    void *state;
    int64_t slot_stride;  // heads * dim * dstate
    int64_t pad;
    const void *x;
    const void *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;        // may be null
    const void *z;         // may be null
    const float *dt_bias;  // may be null
    void *out;
    const void *rtab;      // may be null
    const void *wtab;      // may be null (then rtab, then the sequence index)
    const void *cu;        // kCuSeqlens only
    const void *acc;       // may be null
    int32_t x_sr, x_sh;
    int32_t dt_sr, dt_sh, dt_sp;
    int32_t A_sh, D_sh, bias_sh;
    int32_t B_sr, B_sg, C_sr, C_sg;
    int32_t z_sr, z_sh;
    int32_t out_sr, out_sh;
    int32_t r_s0, r_s1, w_s0, w_s1;
    int32_t cu_s, acc_s;
    int32_t nseq, H, P, heads_per_group;
    int32_t steps;          // kDense: tokens per sequence
    int32_t layout;         // Layout
    int32_t dim_tiles;      // workgroups per (sequence, head)
    int32_t rows_per_block; // dim rows per workgroup
    int32_t flags;          // Flags
};

// ReplaySSM decode: the per-slot input buffers (contiguous) and the caller's
// per-sequence buffer pointers.
struct ReplayParams {
    void *buf_x;        // [slots, L, H, P]
    void *buf_dt;       // [slots, L, H, P] or [slots, L, H]
    void *buf_B;        // [slots, L, G, N]
    const void *buf_len;
    int32_t L;
    int32_t len_s;      // element stride of buf_len
    int32_t len_i64;    // buf_len is i64
    int32_t dt_per_head;  // buf_dt is [slots, L, H]
    int32_t G;
    // read copy of the checkpoint pool (LP kernels): E4M3 codes
    // [slots, H, P, N] (MXFP8) or E2M1 codes [slots, H, P, N / 2] (MXFP4),
    // and E8M0 scales [slots, H, P, N / 32]
    uint8_t *lp;
    uint8_t *lp_scale;
};

// Selected kernel variant for (state dtype, io dtype, dstate, multi-token).
struct KernelRef {
    const void *fn;
    int tile = kTileOneToken;  // TileKind of its dim tile (set by find_yonly_kernel)
};

// Returns false if no variant exists for the combination.
bool find_kernel(int state_dtype, int io_dtype, int dstate, bool multi, KernelRef *out);
// The multi-token kernel's output-only variant for disable_state_update;
// false where it does not apply (16-bit state with fp32 outputs). Sets
// out->tile to kTileYonlyMfma for the matrix-core form, else kTileYonly.
bool find_yonly_kernel(int state_dtype, int io_dtype, int dstate, KernelRef *out);

// "ssu_onetoken_<state>_<io>_n<dstate>" or "ssu_packed_...".
void kernel_name(int state_dtype, int io_dtype, int dstate, bool multi, char *buf, int len);

const char *hip_error_string(int e);

// Launches `k` with `p`; returns the hipError_t value as int.
int launch(const KernelRef &k, const Params &p, unsigned grid, unsigned block, void *stream);

// The ReplaySSM decode kernel for (state dtype, io dtype, dstate).
// memmove-safe state copies (ssu_copy.hip): workgroup size, the batched
// copy's and the convolution shift's arguments (strides in elements).
constexpr int kCopyThreads = 256;
struct CopyParams {
    const void *src_ptrs, *dst_ptrs, *sizes;
    int64_t src_s, dst_s, sizes_s;
    int32_t sizes_i64;
    int32_t tiles;  // workgroups per copy
};
struct ConvParams {
    void *state;
    int64_t blocks, W, inner, elem;
    const void *src, *dst, *bias;
    int64_t src_s, dst_s, bias_s;
    int32_t src_i64, dst_i64, bias_i64;
    int32_t tiles;  // workgroups per request
};
int launch_batch_memcpy(const CopyParams &cp, unsigned grid, void *stream);

// SSD packed prefill (ssu_ssd.hip): head dim, largest chunk, arguments
// (strides in elements; the workspace holds dt' and the decay cumsum per
// [chunk, head, token] and one fp32 state per [chunk, head]).
constexpr int kSsdDim = 64;
constexpr int kSsdMaxChunk = 256;
// Heads per workgroup of the fused prefill kernel (the host derives the
// grid from it): its B rows, C.B^T and cumsum pass serve them all; 8 took
// 557 against 567 us for 4 (and 619 for 2), with 156 KB of LDS
#ifndef SSU_SSD_HEADS
#define SSU_SSD_HEADS 8
#endif
constexpr int kSsdHeads = SSU_SSD_HEADS;
struct SsdParams {
    const void *x, *dt, *B, *C, *z;
    void *out, *states;
    const void *init;
    const float *A, *D, *dt_bias;
    const void *cu_chunk, *seq_idx, *last_chunk;
    float *ws_state;  // the state each chunk leaves to the next [nchunks, H, P, N] (fp32)
    int *ws_flags;    // [nchunks, H]: 1 once ws_state of (chunk, head) is published
    int *ws_tickets;  // [8]: start-order counters, one per virtual XCD
    int *ws_owner;    // [nchunks]: the sequence whose returned state the chunk gives, or -1
    int64_t T, H, N, nchunks, batch, chunk_size;
    int64_t x_st, x_sh, dt_st, dt_sh, B_st, B_sg, C_st, C_sg, z_st, z_sh, out_st, out_sh;
    int64_t A_sh, D_sh, bias_sh;
    int64_t cu_chunk_s, seq_idx_s, last_chunk_s;
    int32_t cu_chunk_i64, seq_idx_i64, last_chunk_i64;
    int32_t hpg, dt_f32, softplus, intermediate;
    int32_t hsplit;  // kSsdDim-wide parts per head: H and hpg count the parts
    int32_t nhb;              // blocks of kSsdHeads heads per group
    int32_t streams_per_xcd;  // (group, block) streams per virtual XCD
    float dt_lo, dt_hi;
};
int launch_ssd(const SsdParams &sp, int io_dtype, int state_dtype, void *stream);
// Loads the prefill's two kernels for (io dtype, state dtype, dstate) on
// the current device; fills their names (launch order) and registers.
// Returns the hipError_t value as int.
int ssd_kernel_attributes(int io_dtype, int state_dtype, int dstate, const char *names[2], int vgprs[2]);
int launch_conv_shift(const ConvParams &cv, bool dim_major, unsigned grid, void *stream);

bool find_replay_kernel(int state_dtype, int io_dtype, int dstate, bool spec, KernelRef *out);
// The one-token replay kernel with an MXFP8 (bits 8) or MXFP4 (bits 4) read
// copy (fp32 checkpoints).
bool find_replay_lp_kernel(int io_dtype, int dstate, int bits, KernelRef *out);
// MXFP8 / MXFP4 quantization of `nblocks` blocks of 32 fp32 values.
int launch_mx8_quantize(const float *src, uint8_t *codes, uint8_t *scales, int64_t nblocks, void *stream);
int launch_mx4_quantize(const float *src, uint8_t *codes, uint8_t *scales, int64_t nblocks, void *stream);
int launch_replay(const KernelRef &k, const Params &p, const ReplayParams &rp, unsigned grid,
                  unsigned block, void *stream);
// The speculative step's second launch: the drafts' B rows and per-head dt
// appended once the step's kernel has ended. One workgroup per (sequence,
// draft): grid = batch * T.
constexpr int kSpecAppendThreads = 256;
int launch_replay_spec_append(const Params &p, const ReplayParams &rp, int io_bytes, int dt_bytes,
                              unsigned grid, void *stream);

// Loads the kernel's code object on the current device and reports its
// registers; returns the hipError_t value as int.
int kernel_attributes(const KernelRef &k, int *vgprs, int *sgprs);

}  // namespace ssu
