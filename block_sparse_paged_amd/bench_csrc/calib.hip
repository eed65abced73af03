// Measurement-only kernels for bench.py (built into libmsa_bench.so, not into
// libmsa): a streaming HBM read that gives the attainable read bandwidth of
// the GPU it runs on, and an empty kernel whose graph-replayed launches give
// the fixed cost of one launch boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;          // 16-byte loads in flight per lane

// Workgroup b reads 16-byte units b*kThreads*kUnroll + ... in grid-stride
// rounds with non-temporal loads, folds them with XOR and stores one word.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t units,
                                                               uint32_t *__restrict__ sink) {
    const int64_t per_round = (int64_t)gridDim.x * kThreads * kUnroll;
    uint32_t acc = 0u;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < units;
         base += per_round) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            v[u] = i < units ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one word per workgroup: the XOR of its lanes' folds
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `src` (16-byte aligned) with `grid`
// workgroups; sink needs `grid` words.  Returns a hipError_t.
int msab_stream_read(const void *src, size_t bytes, uint32_t *sink, int grid, hipStream_t stream) {
    if (!src || !sink || grid < 1 || (bytes & 15) || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, stream, (const u32x4 *)src,
                       (int64_t)(bytes / 16), sink);
    return (int)hipGetLastError();
}

// One launch of an empty kernel of `grid` one-wave workgroups.
int msab_empty(int grid, hipStream_t stream) {
    if (grid < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(64), 0, stream);
    return (int)hipGetLastError();
}

}  // extern "C"
