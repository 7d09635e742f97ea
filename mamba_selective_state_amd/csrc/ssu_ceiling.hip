// Streaming ceilings of the device: plain kernels that move a buffer through
// HBM in the access patterns of the state update (16-byte accesses, with or
// without the non-temporal hint), so that a measured kernel can be read
// against what this part sustains for the same read/write mix. They are a
// measurement aid for bench.py (libssu_ceiling.so), not part of libssu's
// interface.
//
// Patterns (n 16-byte words per buffer):
//   0 read-modify-write in place   p[i] = p[i] * 0.5 + 1
//   1 copy                         d[i] = s[i]
//   2 write only                   d[i] = constant
//   3 read only                    one sum per workgroup written at the end
// Each lane handles WORDS words spaced one wave apart (every wave access
// covers 1 KiB of consecutive bytes); workgroups of 64 or 256 lanes walk the
// buffer grid-stride (a grid that covers it in one pass does no stride).

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxThreads = 256;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4 *p, u32x4 v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

__device__ __forceinline__ u32x4 rmw(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; k++)
        r[k] = __float_as_uint(__uint_as_float(v[k]) * 0.5f + 1.0f);
    return r;
}

template <int KIND, bool NT, int WORDS>
__global__ __launch_bounds__(kMaxThreads) void ceiling_kernel(const u32x4 *src, u32x4 *dst, int64_t n,
                                                              float *sink) {
    constexpr int kWordsPerLane = WORDS;
    const int64_t span = static_cast<int64_t>(blockDim.x) * kWordsPerLane;  // words per workgroup pass
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc = 0.0f;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span; base < n;
         base += static_cast<int64_t>(gridDim.x) * span) {
        // wave w takes words base + w * 256 + k * 64 + lane
        const int64_t w0 = base + static_cast<int64_t>(wave) * 64 * kWordsPerLane + lane;
        if constexpr (KIND == 2) {
#pragma unroll
            for (int k = 0; k < kWordsPerLane; k++)
                if (w0 + 64 * k < n)
                    st<NT>(dst + w0 + 64 * k, u32x4{1u, 2u, 3u, 4u});
        } else {
            u32x4 v[kWordsPerLane];
#pragma unroll
            for (int k = 0; k < kWordsPerLane; k++)
                v[k] = w0 + 64 * k < n ? ld<NT>(src + w0 + 64 * k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < kWordsPerLane; k++) {
                if (w0 + 64 * k >= n)
                    continue;
                if constexpr (KIND == 0)
                    st<NT>(dst + w0 + 64 * k, rmw(v[k]));
                else if constexpr (KIND == 1)
                    st<NT>(dst + w0 + 64 * k, v[k]);
                else
                    acc += __uint_as_float(v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3]);
            }
        }
    }
    if constexpr (KIND == 3) {
        __shared__ float part[kMaxThreads];
        part[threadIdx.x] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float s = 0.0f;
            for (int i = 0; i < static_cast<int>(blockDim.x); i++)
                s += part[i];
            sink[blockIdx.x] = s;
        }
    }
}

template <int KIND, int WORDS>
const void *pick_nt(bool nt) {
    return nt ? reinterpret_cast<const void *>(&ceiling_kernel<KIND, true, WORDS>)
              : reinterpret_cast<const void *>(&ceiling_kernel<KIND, false, WORDS>);
}
template <int KIND>
const void *pick(bool nt, int words) {
    return words == 8 ? pick_nt<KIND, 8>(nt) : words == 2 ? pick_nt<KIND, 2>(nt) : pick_nt<KIND, 4>(nt);
}

}  // namespace

// Runs pattern `kind` over `bytes` (a multiple of 16; src/dst 16-byte aligned;
// for kind 0 src == dst; for kind 3 `sink` holds `grid` floats) with `grid`
// workgroups of `threads` lanes (64 or 256), `words` 16-byte words per lane
// per pass (2, 4 or 8), on `stream`. Returns the hipError_t value.
extern "C" __attribute__((visibility("default"))) int ssu_ceiling_run(int kind, int nt, const void *src, void *dst,
                                                                     int64_t bytes, void *sink, int grid,
                                                                     int threads, int words, void *stream) {
    if (kind < 0 || kind > 3 || bytes % 16 || grid < 1 || (threads != 64 && threads != 256) ||
        (words != 2 && words != 4 && words != 8))
        return static_cast<int>(hipErrorInvalidValue);
    const void *fn = kind == 0   ? pick<0>(nt, words)
                     : kind == 1 ? pick<1>(nt, words)
                     : kind == 2 ? pick<2>(nt, words)
                                 : pick<3>(nt, words);
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    int64_t n = bytes / 16;
    float *k = static_cast<float *>(sink);
    void *args[] = {&s, &d, &n, &k};
    return static_cast<int>(hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(static_cast<unsigned>(threads)),
                                            args, 0, static_cast<hipStream_t>(stream)));
}
