/*
 * ssu.h -- C ABI of libssu: the Mamba-2 selective state update (SSU) decode
 * step on AMD Instinct MI355X (gfx950).
 *
 * The operation (MATE docs, "Mamba / SSU": the API reference of
 * selective_state_update and the table "SSU at a glance"; ReplaySSM article,
 * section "三个瓶颈其实来自同一个动作" for the step itself): for every sequence
 * b and head h, with g = h / (heads / groups),
 *
 *   S      = state[read_slot(b), h]            ([dim, dstate]; zeros for the pad id)
 *   for each token t of the sequence (row r):
 *     dt'  = dt[r, h, d] (+ dt_bias[h]), then softplus if dt_softplus
 *     S[d][n] = S[d][n] * exp(dt'[d] * A[h]) + dt'[d] * x[r, h, d] * B[r, g, n]
 *     y[r, h, d] = (sum_n S[d][n] * C[r, g, n] + D[h] * x[r, h, d]) * silu(z[r, h, d])
 *     state[write_slot(b, t), h] = S            (unless pad or disable_state_update)
 *
 * The recurrence runs in fp32; the state is stored in the state dtype (and
 * the state carried to the next token is that stored value); 16-bit values
 * round to nearest even.
 *
 * Slots (MATE, "SSU at a glance", rows "Slot semantics" and "Variable-length
 * and MTP decode"):
 *   - sequences: x [batch, heads, dim] is one token per sequence; x
 *     [rows, heads, dim] with cu_seqlens [nseq + 1] is packed (sequence b owns
 *     rows cu[b] .. cu[b+1]-1, empty sequences are skipped); x
 *     [batch, steps, heads, dim] is the dense form (steps tokens each);
 *   - read position: num_accepted_tokens[b] - 1, floored at 0 (0 without it);
 *   - a 1-D table is row-indexed: sequence b's position t is entry
 *     first_row(b) + t; a 2-D table is addressed by its strides,
 *     b * stride[0] + t * stride[1]; without a read table the slot is b;
 *   - every token stores to its own destination entry, or to its own entry of
 *     the read table when no destination table is given;
 *   - pad_slot_id reads as a zero state and is never written;
 *     disable_state_update leaves the pool unchanged.
 *
 * Memory: every pointer in ssu_tensor_t is DEVICE memory owned by the caller.
 * The library allocates nothing per call and keeps no pointer after a call
 * returns. ssu_update is asynchronous on the given stream (a hipStream_t,
 * NULL for the null stream) and performs no host/device synchronisation and
 * no device-to-host copy, so it may be captured into a HIP graph.
 *
 * Device-resident values (slot ids, cu_seqlens, num_accepted_tokens) are never
 * read on the host. Slot ids outside [0, slots) other than the pad id,
 * decreasing cu_seqlens, read positions outside the table, or a slot written
 * by one sequence and read or written by another are caller contract
 * violations with undefined results.
 *
 * Errors: every entry point returns an ssu_status_t; ssu_last_error() gives a
 * message (thread-local) naming the violated rule or the missing capability.
 */
#ifndef SSU_H
#define SSU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSU_ABI_VERSION 4

#ifndef SSU_API
#define SSU_API __attribute__((visibility("default")))
#endif

typedef enum {
    SSU_F32 = 0,
    SSU_F16 = 1,
    SSU_BF16 = 2,
    SSU_I32 = 3,
    SSU_I64 = 4,
    SSU_F64 = 5, /* state copies only */
    SSU_U8 = 6   /* state copies only */
} ssu_dtype_t;

typedef enum {
    SSU_OK = 0,
    SSU_ERR_VALUE = 1,           /* wrong shape, dtype, stride, alignment, or missing tensor */
    SSU_ERR_NOT_IMPLEMENTED = 2, /* an option or size the library does not support */
    SSU_ERR_HIP = 3              /* the HIP runtime reported an error (launch, attributes) */
} ssu_status_t;

/* A strided view of caller-owned device memory. data == NULL means "absent"
 * (None). size[] and stride[] hold ndim entries; strides are in elements. */
typedef struct {
    const void *data;
    int32_t dtype; /* ssu_dtype_t */
    int32_t ndim;
    int64_t size[4];
    int64_t stride[4];
} ssu_tensor_t;

/* Bits of ssu_args_t.unsupported: options of the MATE API that this library
 * does not implement; a set bit makes ssu_update return
 * SSU_ERR_NOT_IMPLEMENTED naming the option. */
enum {
    SSU_OPT_STATE_SCALE = 1u << 0,
    SSU_OPT_INTERMEDIATE_STATES = 1u << 1, /* intermediate_states_buffer / indices / scales */
    SSU_OPT_RAND_SEED = 1u << 2,           /* stochastic rounding (not implemented on the MATE page either) */
    SSU_OPT_CACHE_STEPS = 1u << 3,         /* cache_steps != 0 */
    SSU_OPT_ALGORITHM = 1u << 4,           /* algorithm != "auto" */
    SSU_OPT_BACKEND = 1u << 5,             /* backend != "auto" */
    SSU_OPT_SSD_CHECKPOINT = 1u << 6       /* ssu_ssd_prefill: checkpoint_* arguments */
};

/* Arguments of one update (MATE selective_state_update, same names).
 *   state   [slots, heads, dim, dstate], contiguous, f32 / f16 / bf16, updated in place;
 *           base 16-byte aligned.
 *   x       [batch, heads, dim] | [rows, heads, dim] (with cu_seqlens) |
 *           [batch, steps, heads, dim]; f32 / f16 / bf16; last stride 1.
 *   dt      same leading shape as x with last axis dim (any strides, stride 0
 *           over dim for one value per head), or without the last axis (one
 *           value per head); f32 or the x dtype.
 *   A       [heads] f32 (or more axes with stride 0: broadcast over dim/dstate).
 *   B, C    [rows, groups, dstate] (or [batch, steps, groups, dstate]), x dtype,
 *           last stride 1; heads % groups == 0.
 *   D, dt_bias  [heads] f32 or absent (broadcast axes with stride 0 allowed).
 *   z       like x or absent.
 *   state_batch_indices, dst_state_batch_indices
 *           absent, [rows] / [batch] (1-D, row-indexed), or 2-D [nseq, steps];
 *           i32 / i64.
 *   cu_seqlens          [nseq + 1] i32 / i64, with x [rows, heads, dim].
 *   num_accepted_tokens [nseq] i32 / i64.
 *   out     required at this level; same shape as x, x dtype, last stride 1.
 *           Every row of out is written. */
typedef struct {
    ssu_tensor_t state, x, dt, A, B, C, D, z, dt_bias;
    ssu_tensor_t state_batch_indices, dst_state_batch_indices;
    ssu_tensor_t cu_seqlens, num_accepted_tokens;
    ssu_tensor_t out;
    int32_t dt_softplus;
    int32_t disable_state_update;
    int64_t pad_slot_id; /* default -1 */
    uint32_t unsupported; /* SSU_OPT_* bits */
} ssu_args_t;

/* Configuration to prepare ahead of graph capture (MATE
 * prewarm_selective_state_update). dt_dim is 1 for one dt value per head,
 * else dim. packed selects the multi-token kernel (cu_seqlens, dense
 * [batch, steps, ...], or num_accepted_tokens); slot_dtype and meta_dtype are
 * accepted for compatibility (both index widths run in the same kernels).
 * disable_state_update (nonzero) with packed selects the output-only variant
 * those calls take where one exists for the dtypes (as ssu_update does), and
 * reports its tiling. */
typedef struct {
    int32_t state_dtype, io_dtype, dt_dtype, slot_dtype, meta_dtype; /* ssu_dtype_t */
    int32_t heads, dim, dstate, groups, dt_dim, packed;
    int64_t max_rows; /* informational; 0 if unknown */
    int32_t disable_state_update;
} ssu_plan_desc_t;

/* What ssu_plan selected (for logging and tests). */
typedef struct {
    char kernel[64];       /* name of the selected kernel variant ("ssu_onetoken_...",
                              "ssu_packed_..." or "ssu_packed_output_only_...") */
    int32_t block_threads; /* threads per workgroup */
    int32_t rows_per_block;/* dim rows one workgroup covers */
    int32_t blocks_per_seq_head; /* workgroups per (sequence, head) */
    int32_t vgprs, sgprs;  /* registers of the selected kernel (0 if unknown) */
} ssu_plan_info_t;

/* Validate a configuration, select its kernel and load it onto the current
 * device, so a later ssu_update of that shape launches with no first-use
 * cost. Idempotent and thread-safe; info may be NULL. Errors: SSU_ERR_VALUE,
 * SSU_ERR_NOT_IMPLEMENTED, SSU_ERR_HIP. */
SSU_API ssu_status_t ssu_plan(const ssu_plan_desc_t *desc, ssu_plan_info_t *info);

/* Validate the arguments on the host and enqueue exactly one kernel on
 * `stream` (none when there are no rows). Asynchronous; allocates nothing;
 * never reads device memory on the host. Works without a prior ssu_plan. */
SSU_API ssu_status_t ssu_update(const ssu_args_t *args, void *stream);

/* ReplaySSM decode (ReplaySSM article, lpnh.cn, section "核心做法" and its
 * minimal pseudocode): the state of a slot is its checkpoint (the pool entry)
 * plus a buffer of up to L past steps' inputs. For each sequence b with slot
 * s and h = buf_len[b] entries already buffered (0 <= h < L):
 *   - if h + 1 == L (the step fills the buffer: a flush), the buffered steps
 *     and the current one are applied to the checkpoint one after the other
 *     exactly as ssu_update applies a token (state rounded to the state dtype
 *     after each), y is computed from the result, and the checkpoint is
 *     stored; the buffer is not touched (the caller resets h to 0);
 *   - otherwise (output only) the checkpoint is read but not written; with
 *     a_i = exp(dt'_i A[h]) over the buffered steps i < h and the current
 *     step i = h, for every dim row d:
 *       y = (prod_i a_i) (S_ckpt . C) + sum_j dt'_j x_j (prod_{i>j} a_i) (B_j . C)
 *           + D x, times silu(z)
 *     and the current step's raw x, dt and B are written to buffer entry h
 *     (the caller then advances h by one).
 * With L = 1 every step is a flush and equals ssu_update bit for bit.
 * base: as for ssu_update with x [batch, heads, dim] (one token per
 * sequence), state_batch_indices 1-D or absent (slot b), and no
 * dst_state_batch_indices, cu_seqlens or num_accepted_tokens; the pad id
 * reads a zero checkpoint and writes nothing; disable_state_update writes
 * neither checkpoint nor buffer.
 *   buf_x   [slots, L, heads, dim], x dtype, contiguous
 *   buf_dt  [slots, L, heads, dim], or [slots, L, heads] when dt is one value
 *           per head, dt dtype, contiguous
 *   buf_B   [slots, L, groups, dstate], x dtype, contiguous
 *   buf_len [batch] i32 / i64 (device): entries buffered per sequence; a
 *           value outside [0, L) for a slot other than the pad id makes
 *           that sequence's y NaN and writes nothing for it (the kernel
 *           checks it; nothing outside the buffers is read)
 * All DEVICE memory owned by the caller; buffers are updated in place. Same
 * error, stream and allocation conventions as ssu_update. */
typedef struct {
    ssu_args_t base;
    ssu_tensor_t buf_x, buf_dt, buf_B, buf_len;
} ssu_replay_args_t;

SSU_API ssu_status_t ssu_replay_update(const ssu_replay_args_t *args, void *stream);

/* ReplaySSM speculative step (ReplaySSM article, lpnh.cn, section
 * "投机解码回滚变成挪指针"): T draft tokens per sequence are read out against
 * the same checkpoint and buffer window under a causal mask and appended to
 * the buffer; the caller commits the accepted prefix by moving the pointer.
 * For each sequence b with slot s and h = buf_len[b] committed entries:
 *   - if h + 2T > L (the fold, one window early), the h committed entries
 *     are applied to the checkpoint one after the other exactly as
 *     ssu_update applies tokens (state rounded to the state dtype after each)
 *     and the checkpoint is stored; the window then starts empty (w = 0);
 *     otherwise w = h and the checkpoint is only read;
 *   - draft t (t = 0..T-1) reads out, with the steps i, j of the window being
 *     the w committed entries followed by drafts 0..t and a_i = exp(dt'_i A):
 *       y_t = (prod_i a_i) (S . C_t) + sum_j dt'_j x_j (prod_{i>j} a_i) (B_j . C_t)
 *             + D x_t, times silu(z_t)       (S: the checkpoint, folded or not)
 *   - the drafts' raw x, dt and B are written to entries w .. w+T-1; the
 *     caller then sets the pointer to w + the number of accepted drafts.
 * base: as for ssu_update with x [batch, T, heads, dim] (dt [batch, T,
 * heads, dim] or [batch, T, heads], B and C [batch, T, groups, dstate], z
 * and out like x), state_batch_indices 1-D [batch] or absent (slot b), and no
 * dst_state_batch_indices, cu_seqlens or num_accepted_tokens; 1 <= T <= L.
 * Buffers as for ssu_replay_update; buf_len values lie in [0, L] (a value
 * outside for a slot other than the pad id makes that sequence's y NaN and
 * writes nothing). The pad id reads a zero checkpoint, has no buffer and
 * writes nothing; disable_state_update writes neither checkpoint nor buffer.
 * Enqueues two kernels on `stream`: the step, then the append of the drafts'
 * B rows and per-head dt, which a folding sequence's group-mates still read
 * while the step runs. Otherwise the same error, stream and allocation
 * conventions as ssu_update. */
SSU_API ssu_status_t ssu_replay_spec_update(const ssu_replay_args_t *args, void *stream);

/* ---- ReplaySSM with a low-precision read copy (ReplaySSM article, lpnh.cn,
 * section "数据与边界": the checkpoint is a read-mostly value that a
 * low-precision copy can stand in for on the steps that only read it).
 * Format: OCP Microscaling (MX) v1.0, MXFP8 with E4M3 elements: every 32
 * consecutive dstate values of a checkpoint row form a block with one E8M0
 * scale byte X = 2^(e - 127), where e - 127 = floor(log2 max|v|) - 8 clamped
 * to [-126, 127] (-126 for an all-zero block); each element is v / X rounded
 * to nearest even in E4M3 (bias 7, subnormals, largest finite 448, codes
 * 0x7F / 0xFF are NaN), saturating to +-448. A value decodes as code * X. */

/* Quantize fp32 values to MXFP8:
 *   src     [n] f32 (device), n a multiple of 32, 16-byte aligned; blocks
 *           are consecutive runs of 32 values
 *   codes   [n] u8 (device), 8-byte aligned: E4M3 codes
 *   scales  [n / 32] u8 (device): E8M0 scale bytes
 * A NaN element becomes code 0x7F and does not count toward the block's
 * largest magnitude; a block holding an infinity has no defined scale and
 * its bytes are unspecified (a checkpoint is finite). One kernel on
 * `stream`, asynchronous, allocates nothing; n = 0 launches nothing. All
 * three must be contiguous (of any shape: they are read as flat); a rule
 * broken returns SSU_ERR_VALUE naming it. */
SSU_API ssu_status_t ssu_mx8_quantize(const ssu_tensor_t *src, const ssu_tensor_t *codes,
                                      const ssu_tensor_t *scales, void *stream);

/* ssu_replay_update with the checkpoint's MXFP8 copy: output-only steps read
 * the copy (codes * scale, decoded to fp32) in place of the fp32 checkpoint;
 * a flush reads the fp32 checkpoint, folds and stores it as ssu_replay_update
 * does, and then writes the copy of the stored state (the format above) into
 * lp and lp_scale. The pad id reads zeros and writes nothing;
 * disable_state_update writes neither checkpoint, copy nor buffer.
 * base: as for ssu_replay_update, with an f32 state pool whose [heads, dim,
 * dstate] part is contiguous, and dstate a multiple of 32.
 *   lp        [slots, heads, dim, dstate] u8, contiguous, 16-byte aligned (device)
 *   lp_scale  [slots, heads, dim, dstate / 32] u8, contiguous, 8-byte aligned (device)
 * The caller keeps the copy in step with the checkpoint (ssu_mx8_quantize
 * of the pool makes a first copy). Same error, stream and allocation
 * conventions as ssu_update. */
typedef struct {
    ssu_replay_args_t base;
    ssu_tensor_t lp, lp_scale;
} ssu_replay_lp_args_t;

SSU_API ssu_status_t ssu_replay_lp_update(const ssu_replay_lp_args_t *args, void *stream);

/* The same read copy in MXFP4 (OCP Microscaling v1.0, FP4 with E2M1
 * elements), a quarter of the fp32 checkpoint's bytes plus the scales:
 * blocks of 32 consecutive dstate values with one E8M0 scale byte
 * X = 2^(e - 127), e - 127 = floor(log2 max|v|) - 2 clamped to [-126, 127]
 * (-126 for an all-zero block); each element is v / X rounded to nearest
 * even among the E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6 (sign in bit 3),
 * saturating to +-6. Two elements a byte, the even-indexed one in the low
 * nibble. A value decodes as code * X. */

/* Quantize fp32 values to MXFP4:
 *   src     [n] f32 (device), n a multiple of 32, 16-byte aligned; blocks
 *           are consecutive runs of 32 values
 *   codes   [n / 2] u8 (device), 4-byte aligned: E2M1 code pairs
 *   scales  [n / 32] u8 (device): E8M0 scale bytes
 * A NaN element becomes code 0 and does not count toward the block's
 * largest magnitude; a block holding an infinity has no defined scale and
 * its bytes are unspecified (a checkpoint is finite). Otherwise as
 * ssu_mx8_quantize. */
SSU_API ssu_status_t ssu_mx4_quantize(const ssu_tensor_t *src, const ssu_tensor_t *codes,
                                      const ssu_tensor_t *scales, void *stream);

/* ssu_replay_lp_update with the MXFP4 copy:
 *   lp        [slots, heads, dim, dstate / 2] u8, contiguous, 16-byte aligned (device)
 *   lp_scale  [slots, heads, dim, dstate / 32] u8, contiguous, 8-byte aligned (device)
 * Everything else as ssu_replay_lp_update (ssu_mx4_quantize of the pool
 * makes a first copy). */
SSU_API ssu_status_t ssu_replay_mx4_update(const ssu_replay_lp_args_t *args, void *stream);

/* ---- memmove-safe Mamba state copies (vLLM PR #50729 digest, prhub:
 * sections "实现拆解" and "关键源码片段"). Speculative decoding shifts a
 * convolution state left inside one physical block; a parallel copy whose
 * destination overlaps its own source must still end as if the whole source
 * had been read first (memmove). */

/* Batched byte copy with memmove semantics: copy i moves sizes[i] bytes from
 * address src_ptrs[i] to dst_ptrs[i]. A copy whose destination overlaps its
 * own source (on either side) is done by one workgroup in source order away
 * from the overlap, each chunk read completely before any of it is written;
 * other copies are split over several workgroups.
 *   src_ptrs, dst_ptrs  [n] i64 (device): device byte addresses
 *   sizes               [n] i32 / i64 (device): byte counts (<= 0: nothing)
 *   max_size            the caller's bound on the sizes; it only sets how many
 *                       workgroups share one copy (larger sizes are still
 *                       copied in full)
 * Two different copies must not touch the same bytes (the result would
 * depend on their order). DEVICE memory owned by the caller; one kernel on
 * `stream`, asynchronous, allocates nothing; n = 0 launches nothing. */
SSU_API ssu_status_t ssu_batch_memcpy(const ssu_tensor_t *src_ptrs, const ssu_tensor_t *dst_ptrs,
                                      const ssu_tensor_t *sizes, int64_t max_size, void *stream);

/* Convolution-state layouts: token-major [blocks, W, inner] ("SD") and
 * dim-major [blocks, inner, W] ("DS"). */
typedef enum { SSU_CONV_TOKEN_MAJOR = 0, SSU_CONV_DIM_MAJOR = 1 } ssu_conv_layout_t;

typedef struct {
    ssu_tensor_t state;      /* [blocks, W, inner] or [blocks, inner, W], contiguous,
                                16-byte aligned, any dtype (only its element size
                                matters) */
    int32_t layout;          /* ssu_conv_layout_t */
    ssu_tensor_t src_block;  /* [n] i32 / i64 (device) */
    ssu_tensor_t dst_block;  /* [n] i32 / i64 (device) */
    ssu_tensor_t bias;       /* [n] i32 / i64 (device): tokens dropped, 0..W */
} ssu_conv_shift_args_t;

/* Convolution-state shift: request r writes
 *   state[dst_block[r]][:W - bias[r]] = state[src_block[r]][bias[r]:]
 * (token rows for the token-major layout, each of the inner rows for the
 * dim-major one) and leaves the rest of the destination block as it was; a
 * request with src == dst shifts a block inside itself. A request whose block
 * ids or bias are out of range writes nothing (checked on the device). Two
 * requests must not write the same block or one that another reads. One
 * kernel on `stream`, asynchronous, allocates nothing. */
SSU_API ssu_status_t ssu_conv_state_shift(const ssu_conv_shift_args_t *args, void *stream);

/* ---- SSD packed variable-length prefill (MATE docs, "Mamba / SSU",
 * section "SSD packed prefill" and the API entry of ssd_combined_fwd_varlen):
 * the decode step's recurrence run over every token of a packed batch,
 * chunk by chunk, from each sequence's initial state (or zeros):
 *   dt' = clamp(softplus(dt + dt_bias) or dt + dt_bias, dt_limit)
 *   S   = S exp(dt' A[h]) + dt' x B^T,   y = (S . C + D x) silu(z)
 * Chunk c covers tokens cu_chunk_seqlens[c] .. cu_chunk_seqlens[c+1]-1 (the
 * only authority for that mapping; at most chunk_size tokens); it opens a
 * sequence when c = 0 or seq_idx[c] != seq_idx[c-1], and then starts from
 * initial_states[seq_idx[c]]. The state is carried in fp32; `states`
 * receives, in its dtype, the state after chunk last_chunk_indices[b] for
 * every sequence b, or the state after every chunk when
 * return_intermediate_states is set. The products run on bf16 / f16 matrix
 * cores (the x dtype) with fp32 accumulation.
 * Supported: head dims that are multiples of 64, dstate 64 or 128,
 * chunk_size <= 256, x bf16 or f16,
 * states f32 / f16 / bf16. A chunk whose cu_chunk_seqlens entries are out of
 * range or longer than chunk_size is taken as empty (checked on the device). */
typedef struct {
    ssu_tensor_t x;                  /* [tokens, heads, dim], dim contiguous, rows 16-byte aligned */
    ssu_tensor_t dt;                 /* [tokens, heads], f32 or the x dtype */
    ssu_tensor_t A;                  /* [heads] f32 */
    ssu_tensor_t B, C;               /* [tokens, groups, dstate], x dtype, rows 16-byte aligned */
    ssu_tensor_t D;                  /* [heads] f32, or absent */
    ssu_tensor_t z;                  /* like x (dim contiguous, rows 16-byte aligned), or absent */
    ssu_tensor_t dt_bias;            /* [heads] f32, or absent */
    ssu_tensor_t cu_seqlens;         /* [batch + 1] i32 / i64, or absent (not read) */
    ssu_tensor_t cu_chunk_seqlens;   /* [nchunks + 1] i32 / i64 (device) */
    ssu_tensor_t last_chunk_indices; /* [batch] i32 / i64 (device) */
    ssu_tensor_t seq_idx;            /* [nchunks] i32 / i64 (device) */
    ssu_tensor_t initial_states;     /* [batch, heads, dim, dstate] contiguous, the state dtype, or absent */
    ssu_tensor_t out;                /* like x (dim contiguous, rows 16-byte aligned): y, written */
    ssu_tensor_t states;             /* [batch or nchunks, heads, dim, dstate] contiguous: written */
    int64_t chunk_size;
    int32_t dt_softplus;
    int32_t return_intermediate_states;
    float dt_limit_lo, dt_limit_hi;  /* (0, +inf) by default */
    uint32_t unsupported;            /* SSU_OPT_SSD_CHECKPOINT: the checkpoint_* arguments */
} ssu_ssd_args_t;

/* Bytes of device workspace ssu_ssd_prefill needs for `nchunks` chunks. */
SSU_API int64_t ssu_ssd_workspace_bytes(int64_t heads, int64_t dim, int64_t dstate, int64_t nchunks);

/* Two kernels on `stream` (none when there are no chunks); asynchronous;
 * allocates nothing: the caller passes `workspace` (DEVICE memory, 256-byte
 * aligned, at least ssu_ssd_workspace_bytes) and keeps it for the call's
 * duration. The workspace carries each chunk's state to the next chunk of
 * its sequence and the words that order that hand-over; the call clears
 * them itself, so the workspace needs no clearing, but two calls that
 * overlap (other streams) must not share one. Errors as for ssu_update. */
SSU_API ssu_status_t ssu_ssd_prefill(const ssu_ssd_args_t *args, void *workspace, int64_t workspace_bytes,
                                     void *stream);

/* ---- SSD prewarm (MATE docs, "Mamba / SSU", the API entry of
 * prewarm_ssd_combined_fwd_varlen): validate one prefill configuration --
 * the shape parameters, the dtypes and chunk_size; token and chunk counts
 * are runtime sizes -- and load its kernels onto the current device, before
 * any graph capture, so a later ssu_ssd_prefill of that configuration has
 * no first-use cost. block_M is accepted and ignored (the gfx950 kernels fix
 * their own tiling). Idempotent and thread-safe; info may be NULL. Errors:
 * SSU_ERR_VALUE (bad shape or dtype), SSU_ERR_NOT_IMPLEMENTED (a supported
 * set is left: head dims a multiple of 64, dstate 64 or 128, chunk_size <=
 * 256, x bf16 or f16), SSU_ERR_HIP (loading failed). */
typedef struct {
    int32_t heads, groups, dim, dstate, chunk_size;
    int32_t io_dtype, state_dtype, dt_dtype; /* ssu_dtype_t */
    int32_t block_M;
} ssu_ssd_plan_desc_t;

typedef struct {
    int32_t launches;            /* kernels one prefill call enqueues */
    char kernels[3][64];         /* their names, in launch order */
    int32_t vgprs[3];            /* their registers per lane */
    int64_t workspace_bytes_per_chunk; /* ssu_ssd_workspace_bytes(heads, dim, dstate, 1) */
} ssu_ssd_plan_info_t;

SSU_API ssu_status_t ssu_ssd_plan(const ssu_ssd_plan_desc_t *desc, ssu_ssd_plan_info_t *info);

/* ---- SSD prefill that allocates nothing and takes no workspace argument.
 * For callers that cannot allocate device memory or pass one: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, kernels and results as ssu_ssd_prefill; its workspace is a
 * device array of SSU_SSD_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's load until the process ends (its address on a
 * GPU is looked up on the first call made with that GPU current). A call
 * whose workspace (ssu_ssd_workspace_bytes) exceeds that size fails with
 * SSU_ERR_VALUE before anything is enqueued. `stream` must belong to the
 * current device. Every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other threads) race on it; calls on one
 * stream are ordered. Nothing in the array needs clearing between calls. */
#define SSU_SSD_SCRATCH_BYTES (64ll << 20)
SSU_API ssu_status_t ssu_ssd_prefill_noalloc(const ssu_ssd_args_t *args, void *stream);

/* Message of the last failing call on this thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
SSU_API const char *ssu_last_error(void);

/* SSU_ABI_VERSION of the library. */
SSU_API int ssu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSU_H */
