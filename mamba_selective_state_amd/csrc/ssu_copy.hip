// memmove-safe Mamba state copies for gfx950 (vLLM PR #50729 digest, prhub,
// sections "实现拆解" and "关键源码片段"): a batched byte copy whose copies may
// overlap their own source, and the convolution-state shift in token-major
// and dim-major layouts.
//
// A copy that does not overlap its own source is split over workgroups and
// moves 16-byte words (or the widest word its addresses and size allow). A
// copy whose destination overlaps its source is done by one workgroup in
// chunks, walking away from the overlap (ascending when the destination lies
// below the source, descending when above): every lane loads its words of
// the chunk, the workgroup waits for all of its loads and meets at a barrier,
// and only then stores. A chunk's stores never reach source bytes a later
// chunk still reads, so the result is that of reading the whole source first
// (a copy of up to 2 chunks is read whole, then written).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssu_internal.h"

namespace ssu {
namespace {

typedef unsigned int cu32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int cu32x4 __attribute__((ext_vector_type(4)));
template <int B> struct WordOf;
template <> struct WordOf<1> { using T = uint8_t; };
template <> struct WordOf<2> { using T = uint16_t; };
template <> struct WordOf<4> { using T = uint32_t; };
template <> struct WordOf<8> { using T = cu32x2; };
template <> struct WordOf<16> { using T = cu32x4; };

constexpr int kUnroll = 4;  // words per lane per chunk

// The copies' addresses come from pointer tables: as generic pointers their
// accesses would be flat ones, which count against the LDS counter too (a
// barrier's LDS wait would then wait for every load in flight). Every
// address here is device global memory.
template <typename T> using Global = __attribute__((address_space(1))) T;
template <typename T> __device__ __forceinline__ Global<T> *global_ptr(void *p) {
    return (Global<T> *)p;
}
template <typename T> __device__ __forceinline__ const Global<T> *global_ptr(const void *p) {
    return (const Global<T> *)p;
}

// Widest word (16, 8, 4, 2 or 1 bytes) that divides both addresses and the size.
__device__ __forceinline__ int word_bytes(uintptr_t dst, uintptr_t src, int64_t size) {
    const uint64_t m = static_cast<uint64_t>(dst | src | static_cast<uintptr_t>(size));
    return (m & 15) == 0 ? 16 : (m & 7) == 0 ? 8 : (m & 3) == 0 ? 4 : (m & 1) == 0 ? 2 : 1;
}

// Words [first, first + count) of the copy in tiles of blockDim.x * kUnroll
// words, tile t0, t0 + tstride, ... (no ordering between tiles).
template <int WB>
__device__ void copy_tiles(uint8_t *dst, const uint8_t *src, int64_t nwords, int64_t t0, int64_t tstride) {
    using T = typename WordOf<WB>::T;
    Global<T> *d = global_ptr<T>(dst);
    const Global<T> *s = global_ptr<T>(src);
    const int64_t tile = static_cast<int64_t>(blockDim.x) * kUnroll;
    for (int64_t t = t0; t * tile < nwords; t += tstride) {
        const int64_t base = t * tile + threadIdx.x;
        T v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < nwords)
                v[u] = s[i];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < nwords)
                d[i] = v[u];
        }
    }
}

constexpr int kWholeChunks = 2;  // copies up to this many chunks are loaded whole before any store

// The whole copy by this workgroup. Up to kWholeChunks chunks: every lane
// loads all of its words, the workgroup waits for them and meets at a
// barrier, then stores (one round trip). Longer: chunk by chunk away from the
// overlap, each chunk loaded by every lane, waited for and fenced by a
// barrier before any lane stores it.
template <int WB>
__device__ void copy_ordered(uint8_t *dst, const uint8_t *src, int64_t nwords, bool descending) {
    using T = typename WordOf<WB>::T;
    Global<T> *d = global_ptr<T>(dst);
    const Global<T> *s = global_ptr<T>(src);
    const int64_t chunk = static_cast<int64_t>(blockDim.x) * kUnroll;
    const int64_t chunks = (nwords + chunk - 1) / chunk;
    if (chunks <= kWholeChunks) {  // uniform
        T v[kWholeChunks][kUnroll];
#pragma unroll
        for (int c = 0; c < kWholeChunks; c++)
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const int64_t i = c * chunk + u * static_cast<int64_t>(blockDim.x) + threadIdx.x;
                if (i < nwords)
                    v[c][u] = s[i];
            }
        __builtin_amdgcn_s_waitcnt(0);  // this lane's loads have returned
        __syncthreads();                // ... and every other lane's
#pragma unroll
        for (int c = 0; c < kWholeChunks; c++)
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const int64_t i = c * chunk + u * static_cast<int64_t>(blockDim.x) + threadIdx.x;
                if (i < nwords)
                    d[i] = v[c][u];
            }
        return;
    }
    for (int64_t c = 0; c < chunks; c++) {
        const int64_t base = (descending ? chunks - 1 - c : c) * chunk + threadIdx.x;
        T v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < nwords)
                v[u] = s[i];
        }
        __builtin_amdgcn_s_waitcnt(0);  // this lane's loads have returned
        __syncthreads();                // ... and every other lane's
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < nwords)
                d[i] = v[u];
        }
    }
}

// One memmove-safe copy of `size` bytes; tile t of `tiles` workgroups that
// share it (an overlapping copy is done by tile 0 alone).
__device__ void copy_one(uint8_t *dst, const uint8_t *src, int64_t size, int64_t t, int64_t tiles) {
    if (size <= 0 || dst == src)
        return;
    const bool overlap = dst < src + size && src < dst + size;
    const int wb = word_bytes(reinterpret_cast<uintptr_t>(dst), reinterpret_cast<uintptr_t>(src), size);
    if (overlap) {
        if (t != 0)
            return;
        const bool descending = dst > src;
        switch (wb) {
        case 16: copy_ordered<16>(dst, src, size / 16, descending); break;
        case 8: copy_ordered<8>(dst, src, size / 8, descending); break;
        case 4: copy_ordered<4>(dst, src, size / 4, descending); break;
        case 2: copy_ordered<2>(dst, src, size / 2, descending); break;
        default: copy_ordered<1>(dst, src, size, descending); break;
        }
        return;
    }
    switch (wb) {
    case 16: copy_tiles<16>(dst, src, size / 16, t, tiles); break;
    case 8: copy_tiles<8>(dst, src, size / 8, t, tiles); break;
    case 4: copy_tiles<4>(dst, src, size / 4, t, tiles); break;
    case 2: copy_tiles<2>(dst, src, size / 2, t, tiles); break;
    default: copy_tiles<1>(dst, src, size, t, tiles); break;
    }
}

__device__ __forceinline__ int64_t index_at(const void *base, bool i64, int64_t i) {
    return i64 ? static_cast<const int64_t *>(base)[i] : static_cast<int64_t>(static_cast<const int32_t *>(base)[i]);
}

// grid = n * tiles workgroups: copy blockIdx / tiles, tile blockIdx % tiles
__global__ __launch_bounds__(kCopyThreads) void batch_memcpy_kernel(const CopyParams cp) {
    const int64_t i = blockIdx.x / cp.tiles;
    const int64_t t = blockIdx.x % cp.tiles;
    uint8_t *dst = reinterpret_cast<uint8_t *>(static_cast<const uint64_t *>(cp.dst_ptrs)[i * cp.dst_s]);
    const uint8_t *src = reinterpret_cast<const uint8_t *>(static_cast<const uint64_t *>(cp.src_ptrs)[i * cp.src_s]);
    const int64_t size = index_at(cp.sizes, cp.sizes_i64, i * cp.sizes_s);
    copy_one(dst, src, size, t, cp.tiles);
}

// Token-major conv state: request r moves tokens bias..W-1 of the source
// block (one contiguous range) to tokens 0..W-bias-1 of the destination.
__global__ __launch_bounds__(kCopyThreads) void conv_shift_token_major_kernel(const ConvParams cv) {
    const int64_t r = blockIdx.x / cv.tiles;
    const int64_t t = blockIdx.x % cv.tiles;
    const int64_t s = index_at(cv.src, cv.src_i64, r * cv.src_s);
    const int64_t d = index_at(cv.dst, cv.dst_i64, r * cv.dst_s);
    const int64_t b = index_at(cv.bias, cv.bias_i64, r * cv.bias_s);
    if (s < 0 || s >= cv.blocks || d < 0 || d >= cv.blocks || b < 0 || b > cv.W)
        return;  // out of range: nothing written
    uint8_t *pool = static_cast<uint8_t *>(cv.state);
    const int64_t row = cv.inner * cv.elem;  // bytes per token
    copy_one(pool + d * cv.W * row, pool + s * cv.W * row + b * row, (cv.W - b) * row, t, cv.tiles);
}

// Dim-major conv state, rows of 2, 4 or 8 bytes: a lane loads its whole rows
// (a wave's access covers 64 consecutive rows), shifts each in a register,
// and stores either the whole row with its own tail merged back (a shift
// inside one block) or just the kept elements (another block, whose tail is
// left alone).
template <typename R>
__device__ void shift_rows_word(const ConvParams &cv, int64_t s, int64_t d, int64_t b, int64_t row0,
                                int64_t rstride) {
    R *pool = static_cast<R *>(cv.state);
    const int bits_per = static_cast<int>(cv.elem) * 8;
    const int keep_bits = static_cast<int>(cv.W - b) * bits_per;  // 1 .. row bits
    const uint64_t lo = keep_bits >= 64 ? ~0ull : ((1ull << keep_bits) - 1);
    const int sh = static_cast<int>(b) * bits_per;                 // < row bits
    // a lane's rows are its own: all of them are loaded before any is stored
    constexpr int kRows = 8;
    for (int64_t r0 = row0; r0 < cv.inner; r0 += kRows * rstride) {
        uint64_t v[kRows];
#pragma unroll
        for (int k = 0; k < kRows; k++) {
            const int64_t row = r0 + k * rstride;
            v[k] = row < cv.inner ? static_cast<uint64_t>(pool[s * cv.inner + row]) : 0;
        }
#pragma unroll
        for (int k = 0; k < kRows; k++) {
            const int64_t row = r0 + k * rstride;
            if (row >= cv.inner)
                break;
            if (s == d) {
                // inside one block: the row's own tail is merged back, one store
                pool[d * cv.inner + row] = static_cast<R>(((v[k] >> sh) & lo) | (v[k] & ~lo));
            } else {
                // another block: only the kept elements are stored
                const uint64_t w = v[k] >> sh;
                unsigned char *dst = reinterpret_cast<unsigned char *>(pool + d * cv.inner + row);
                for (int64_t e = 0; e < cv.W - b; e++) {
                    const uint64_t ev = w >> (e * bits_per);
                    switch (cv.elem) {
                    case 4: reinterpret_cast<uint32_t *>(dst)[e] = static_cast<uint32_t>(ev); break;
                    case 2: reinterpret_cast<uint16_t *>(dst)[e] = static_cast<uint16_t>(ev); break;
                    default: dst[e] = static_cast<unsigned char>(ev); break;
                    }
                }
            }
        }
    }
}

// Dim-major conv state, any row: each lane shifts its rows element by element,
// ascending (the load of element e + bias precedes the store of element e,
// and later loads lie further right, so nothing is overwritten before it is
// read).
template <typename E>
__device__ void shift_rows(const ConvParams &cv, int64_t s, int64_t d, int64_t b, int64_t row0,
                           int64_t rstride) {
    E *pool = static_cast<E *>(cv.state);
    const int64_t keep = cv.W - b;
    for (int64_t row = row0; row < cv.inner; row += rstride) {
        const E *sp = pool + (s * cv.inner + row) * cv.W + b;
        E *dp = pool + (d * cv.inner + row) * cv.W;
        for (int64_t e = 0; e < keep; e++)
            dp[e] = sp[e];
    }
}

__global__ __launch_bounds__(kCopyThreads) void conv_shift_dim_major_kernel(const ConvParams cv) {
    const int64_t r = blockIdx.x / cv.tiles;
    const int64_t t = blockIdx.x % cv.tiles;
    const int64_t s = index_at(cv.src, cv.src_i64, r * cv.src_s);
    const int64_t d = index_at(cv.dst, cv.dst_i64, r * cv.dst_s);
    const int64_t b = index_at(cv.bias, cv.bias_i64, r * cv.bias_s);
    if (s < 0 || s >= cv.blocks || d < 0 || d >= cv.blocks || b < 0 || b >= cv.W)
        return;  // out of range, or bias W: nothing written
    const int64_t row0 = t * blockDim.x + threadIdx.x;
    const int64_t rstride = static_cast<int64_t>(cv.tiles) * blockDim.x;
    switch (cv.W * cv.elem) {  // whole rows of 2, 4 or 8 bytes (the pool is aligned to them)
    case 8: shift_rows_word<uint64_t>(cv, s, d, b, row0, rstride); return;
    case 4: shift_rows_word<uint32_t>(cv, s, d, b, row0, rstride); return;
    case 2: shift_rows_word<uint16_t>(cv, s, d, b, row0, rstride); return;
    }
    switch (cv.elem) {
    case 8: shift_rows<uint64_t>(cv, s, d, b, row0, rstride); break;
    case 4: shift_rows<uint32_t>(cv, s, d, b, row0, rstride); break;
    case 2: shift_rows<uint16_t>(cv, s, d, b, row0, rstride); break;
    default: shift_rows<uint8_t>(cv, s, d, b, row0, rstride); break;
    }
}

}  // namespace

int launch_batch_memcpy(const CopyParams &cp, unsigned grid, void *stream) {
    CopyParams c = cp;
    void *args[] = {&c};
    return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void *>(&batch_memcpy_kernel), dim3(grid),
                                            dim3(kCopyThreads), args, 0, static_cast<hipStream_t>(stream)));
}

int launch_conv_shift(const ConvParams &cv, bool dim_major, unsigned grid, void *stream) {
    ConvParams c = cv;
    void *args[] = {&c};
    const void *fn = dim_major ? reinterpret_cast<const void *>(&conv_shift_dim_major_kernel)
                               : reinterpret_cast<const void *>(&conv_shift_token_major_kernel);
    return static_cast<int>(hipLaunchKernel(fn, dim3(grid), dim3(kCopyThreads), args, 0,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace ssu
