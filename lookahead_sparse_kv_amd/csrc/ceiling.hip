// ceiling.hip -- measured HBM ceilings for the benchmark's roofline fractions.
//
// Not part of the LSA C ABI (include/lsa.h) and not used by it: a separate
// small library (libceiling.so) that bench.py loads to measure, in the same
// run as the kernels it rates, what this GPU's memory system delivers for
//   * a contiguous streaming read (the pattern of the index score),
//   * a contiguous copy (read + write), and
//   * a gather of whole rows at random row indices (the pattern of the
//     sparse attention over top-k rows).
// Each kernel reads every byte it is given exactly once with 16-byte loads
// and folds what it read into one value per workgroup (written to `sink`),
// so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;      // 16-byte loads in flight per thread

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup g reads 16-byte words g*per .. (g+1)*per-1 (per = kThreads*kUnroll*iters),
// consecutive threads on consecutive words.
__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = min(lo + per, n16);
    uint32_t acc = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            v[u] = j < hi ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

__global__ __launch_bounds__(kThreads) void k_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = min(lo + per, n16);
    for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            if (j < hi) v[u] = __builtin_nontemporal_load(src + j);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            if (j < hi) __builtin_nontemporal_store(v[u], dst + j);
        }
    }
}

// Rows of row16 16-byte words, rows idx[r] for r in the wave's share, kUnroll
// row groups in flight.  A row of at least 64 words is read by the whole wave
// (64 words per instruction); a shorter one (64 a multiple of row16) shares an
// instruction with 64 / row16 - 1 others, lane l reading word l % row16 of row
// l / row16 of the group.
__global__ __launch_bounds__(kThreads) void k_gather(const u32x4* __restrict__ src,
                                                     const int32_t* __restrict__ idx,
                                                     int64_t nrows, int row16,
                                                     uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
    const int rpi = row16 < 64 ? 64 / row16 : 1;          // rows per instruction
    const int sub = row16 < 64 ? lane / row16 : 0;
    const int c0 = row16 < 64 ? lane % row16 : lane;
    uint32_t acc = 0;
    for (int64_t r0 = wave * kUnroll * rpi; r0 < nrows; r0 += nwaves * kUnroll * rpi) {
        int32_t rr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) rr[u] = idx[min(r0 + u * rpi + sub, nrows - 1)];
        for (int c = c0; c < row16; c += 64) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                v[u] = r0 + u * rpi + sub < nrows
                           ? __builtin_nontemporal_load(src + (int64_t)rr[u] * row16 + c)
                           : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    if (lane == 0) atomicXor(sink + blockIdx.x, acc);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

// All pointers are device pointers; byte counts are multiples of 16.  `sink`
// holds one uint32 per workgroup (grid entries).  Return 0, or -1 on a bad
// argument, -4 if the launch failed.
extern "C" int ceiling_read(const void* src, int64_t bytes, int grid, uint32_t* sink,
                            void* stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 || grid <= 0) return -1;
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, bytes / 16, sink);
    return status(hipGetLastError());
}

extern "C" int ceiling_copy(const void* src, void* dst, int64_t bytes, int grid, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 || grid <= 0) return -1;
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, bytes / 16);
    return status(hipGetLastError());
}

// Rows of row_bytes at src + idx[r] * row_bytes, r < nrows (indices must be valid
// rows); below 1 KiB, row_bytes must divide 1 KiB.
extern "C" int ceiling_gather(const void* src, const int32_t* idx, int64_t nrows,
                              int64_t row_bytes, int grid, uint32_t* sink, void* stream) {
    if (!src || !idx || !sink || nrows <= 0 || row_bytes <= 0 || row_bytes % 16 || grid <= 0 ||
        (row_bytes < 1024 && 1024 % row_bytes))
        return -1;
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, idx, nrows, (int)(row_bytes / 16), sink);
    return status(hipGetLastError());
}
