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
//
// From host memory a few workgroups already keep the link busy (each has
// kFetchThreads * kFetchUnroll * 16 bytes in flight), so the grid is capped at
// kFetchHostWGs and each workgroup takes a long run of its sequence's list: the
// fetch then holds a few CUs while it waits on the link, and the decode steps
// it overlaps keep the rest.  From device memory every workgroup takes
// kFetchRows rows, as HBM needs far more in flight.
#include "common.hpp"

#ifndef LSA_FETCH_HOST_WGS
#define LSA_FETCH_HOST_WGS 32
#endif
#ifndef LSA_FETCH_UNROLL
#define LSA_FETCH_UNROLL 8
#endif

namespace lsa {

constexpr int kFetchThreads = 256;
constexpr int kFetchRows = 32;      // fewest rows per workgroup
constexpr int kFetchUnroll = LSA_FETCH_UNROLL;      // 16-byte loads in flight per thread
constexpr int kFetchHostWGs = LSA_FETCH_HOST_WGS;   // grid cap for a host source

// Workgroup (x, b) copies a contiguous run of sequence b's list, at least
// kFetchRows rows long, as one flat range of 16-byte segments: every step
// moves kFetchThreads * kFetchUnroll segments whatever the row length.  A
// thread's (row, segment) position advances by constant strides, so no
// division sits in the loop.
__global__ __launch_bounds__(kFetchThreads) void k_fetch_rows(
    const u32x4* __restrict__ src, int segs, const int64_t* __restrict__ src_row_start,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ idx_start,
    const int32_t* __restrict__ count, int64_t max_count, u32x4* __restrict__ dst,
    const int64_t* __restrict__ dst_row_start) {
    const int b = blockIdx.y;
    const int64_t cnt = min((int64_t)count[b], max_count);
    const int64_t per = max((int64_t)kFetchRows, (cnt + gridDim.x - 1) / gridDim.x);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    if (r0 >= cnt) return;
    const int rows = (int)min(cnt - r0, per);
    const int64_t sbase = src_row_start[b];
    const int32_t* ib = idx + idx_start[b] + r0;
    u32x4* db = dst + (dst_row_start[b] + r0) * segs;
    // strides of one unroll slot and of one whole step, as (rows, segments)
    constexpr int kStep = kFetchThreads * kFetchUnroll;
    const int slot_r = kFetchThreads / segs, slot_s = kFetchThreads % segs;
    const int step_r = kStep / segs, step_s = kStep % segs;
    int r = threadIdx.x / segs, sg = threadIdx.x % segs;
    while (r < rows) {
        u32x4 v[kFetchUnroll];
        int ru[kFetchUnroll], su[kFetchUnroll];
        int rr = r, ss = sg;
#pragma unroll
        for (int u = 0; u < kFetchUnroll; ++u) {
            ru[u] = rr;
            su[u] = ss;
            if (rr < rows) v[u] = src[(sbase + ib[rr]) * segs + ss];
            ss += slot_s;
            rr += slot_r;
            if (ss >= segs) {
                ss -= segs;
                ++rr;
            }
        }
#pragma unroll
        for (int u = 0; u < kFetchUnroll; ++u)
            if (ru[u] < rows) db[(int64_t)ru[u] * segs + su[u]] = v[u];
        sg += step_s;
        r += step_r;
        if (sg >= segs) {
            sg -= segs;
            ++r;
        }
    }
}

// The address the device reads p through: device (or managed) memory as it is,
// pinned host memory through its mapping.  Pageable host memory is refused --
// a kernel that touched it would fault.
static int device_view(const void* p, bool host_ok, const void** out, bool* is_host,
                       const char* what) {
    *is_host = false;
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
        *is_host = true;
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
    bool src_host = false, dst_host = false;
    if ((rc = device_view(src, true, &src_dev, &src_host, "src")) != LSA_OK) return rc;
    if ((rc = device_view(dst, false, &dst_dev, &dst_host, "dst")) != LSA_OK) return rc;
    if (!aligned16(src_dev)) return fail(LSA_ERR_INVALID_ARG, "lsa_fetch_rows: src mapping unaligned");
    if (max_count == 0) return LSA_OK;
    int64_t gx = ceil_div(max_count, kFetchRows);            // runs of the longest list
    if (src_host) gx = std::min(gx, std::max<int64_t>(1, ceil_div(kFetchHostWGs, B)));
    dim3 grid((unsigned)gx, (unsigned)B);
    hipLaunchKernelGGL(k_fetch_rows, grid, dim3(kFetchThreads), 0, (hipStream_t)stream, (const u32x4*)src_dev,
                       (int)(row_bytes / 16), src_row_start, idx, idx_start, count, max_count,
                       (u32x4*)dst, dst_row_start);
    return launch_status("fetch_rows");
}
