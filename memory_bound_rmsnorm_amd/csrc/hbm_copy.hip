// A plain device-to-device copy with 16-byte vector accesses: the bandwidth
// ceiling that a one-read/one-write kernel can reach on this GPU, and the
// known-size reference for scaling the HBM byte counters.  Declared in
// include/hbm_copy.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hbm_copy.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 512 lanes x 2 vectors per lane: the fastest copy shape measured on MI355X.
constexpr int kThreads = 512;
constexpr int kUnroll = 2;

__global__ void __launch_bounds__(kThreads) hbm_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t nvec, const unsigned char* __restrict__ src_tail,
                                                            unsigned char* __restrict__ dst_tail, int tail) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < nvec;
         base += stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t i = base + static_cast<int64_t>(k) * kThreads;
            if (i < nvec) v[k] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t i = base + static_cast<int64_t>(k) * kThreads;
            if (i < nvec) __builtin_nontemporal_store(v[k], dst + i);
        }
    }
    if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

}  // namespace

extern "C" HBM_COPY_API int hbm_copy(const void* src, void* dst, int64_t bytes, int32_t max_blocks, void* stream) {
    if (bytes < 0 || max_blocks < 0) return 1;
    if (bytes == 0) return 0;
    if (!src || !dst) return 1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return 1;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + static_cast<uintptr_t>(bytes) && d < s + static_cast<uintptr_t>(bytes)) return 1;
    const int64_t nvec = bytes / 16;
    const int tail = static_cast<int>(bytes % 16);
    int64_t blocks = (nvec + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    if (blocks < 1) blocks = 1;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL(hbm_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                       nvec, static_cast<const unsigned char*>(src) + nvec * 16,
                       static_cast<unsigned char*>(dst) + nvec * 16, tail);
    if (hipGetLastError() != hipSuccess) return 3;
    return 0;
}
