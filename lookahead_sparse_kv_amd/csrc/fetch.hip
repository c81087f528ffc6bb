// fetch.hip -- lsa_fetch_rows: just-in-time fetch of the kept entries into a hot buffer.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Dynamic Fetching": the
// entries whose score reaches 0.5 are fetched from the CPU-side cold pool into
// GPU memory, which then holds only this critical subset.
//
// A zero-copy gather: the kernel reads the source rows itself (pinned host
// memory mapped into the device's address space, or device memory) and writes
// them packed, in list order, into the destination.  Bound by the host link
// (or HBM for a device source): each thread keeps kFetchUnroll 16-byte loads in
// flight, and consecutive lanes move consecutive 16-byte segments of a row, so
// both the reads and the writes are whole 64-byte (or larger) runs.
#include "common.hpp"

namespace lsa {

constexpr int kFetchRows = 32;      // destination rows per workgroup
constexpr int kFetchUnroll = 8;     // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void k_fetch_rows(
    const u32x4* __restrict__ src, int segs, const int64_t* __restrict__ src_row_start,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ idx_start,
    const int32_t* __restrict__ count, int64_t max_count, u32x4* __restrict__ dst,
    const int64_t* __restrict__ dst_row_start) {
    const int b = blockIdx.y;
    const int64_t cnt = min((int64_t)count[b], max_count);
    const int64_t r0 = (int64_t)blockIdx.x * kFetchRows;
    if (r0 >= cnt) return;
    const int rows = (int)min(cnt - r0, (int64_t)kFetchRows);
    const int total = rows * segs;                      // 16-byte segments of this tile
    const int64_t sbase = src_row_start[b];
    const int64_t dbase = dst_row_start[b] + r0;
    const int32_t* ib = idx + idx_start[b] + r0;
    for (int e0 = threadIdx.x; e0 < total; e0 += 256 * kFetchUnroll) {
        u32x4 v[kFetchUnroll];
        int64_t dofs[kFetchUnroll];
#pragma unroll
        for (int u = 0; u < kFetchUnroll; ++u) {
            const int e = e0 + 256 * u;
            if (e < total) {
                const int r = e / segs, sg = e - (e / segs) * segs;
                const int64_t row = sbase + ib[r];
                v[u] = src[row * segs + sg];
                dofs[u] = (int64_t)r * segs + sg;
            }
        }
#pragma unroll
        for (int u = 0; u < kFetchUnroll; ++u)
            if (e0 + 256 * u < total) dst[dbase * segs + dofs[u]] = v[u];
    }
}

// The address the device reads p through: device (or managed) memory as it is,
// pinned host memory through its mapping.  Pageable host memory is refused --
// a kernel that touched it would fault.
static int device_view(const void* p, bool host_ok, const void** out, const char* what) {
    hipPointerAttribute_t a;
    const hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: %s is not memory the device can read",
                    what);
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *out = p;
        return LSA_OK;
    }
    if (host_ok && a.type == hipMemoryTypeHost && a.devicePointer) {
        // hostPointer and devicePointer name the same byte of the allocation
        const char* hp = a.hostPointer ? (const char*)a.hostPointer : (const char*)p;
        *out = (const char*)a.devicePointer + ((const char*)p - hp);
        return LSA_OK;
    }
    return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: %s must be %s", what,
                host_ok ? "device memory or pinned host memory" : "device memory");
}

}  // namespace lsa

using namespace lsa;

extern "C" int lsa_fetch_rows(const void* src, int64_t row_bytes, const int64_t* src_row_start,
                              const int32_t* idx, const int64_t* idx_start, const int32_t* count,
                              int B, int64_t max_count, void* dst, const int64_t* dst_row_start,
                              void* stream) {
    clear_error();
    if (!src || !src_row_start || !idx || !idx_start || !count || !dst || !dst_row_start)
        return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: a required pointer is NULL");
    if (B <= 0 || max_count < 0 || row_bytes <= 0 || row_bytes % 16 != 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: B=%d max_count=%lld row_bytes=%lld", B,
                    (long long)max_count, (long long)row_bytes);
    if (!aligned16(src) || !aligned16(dst))
        return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: src and dst must be 16-byte aligned");
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "lsa_fetch_rows: B=%d > 65535", B);
    // a tile's segment count must fit an int
    if (row_bytes / 16 > ((int64_t)1 << 31) / kFetchRows)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_fetch_rows: row_bytes=%lld too large",
                    (long long)row_bytes);
    if (max_count > (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_fetch_rows: max_count too large");
    int rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    const void* src_dev = nullptr;
    const void* dst_dev = nullptr;
    if ((rc = device_view(src, true, &src_dev, "src")) != LSA_OK) return rc;
    if ((rc = device_view(dst, false, &dst_dev, "dst")) != LSA_OK) return rc;
    if (!aligned16(src_dev)) return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: src mapping unaligned");
    if (max_count == 0) return LSA_OK;
    dim3 grid((unsigned)ceil_div(max_count, kFetchRows), (unsigned)B);
    hipLaunchKernelGGL(k_fetch_rows, grid, dim3(256), 0, (hipStream_t)stream, (const u32x4*)src_dev,
                       (int)(row_bytes / 16), src_row_start, idx, idx_start, count, max_count,
                       (u32x4*)dst, dst_row_start);
    return launch_status("fetch_rows");
}
