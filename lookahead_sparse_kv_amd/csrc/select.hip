// select.hip -- lsa_select_compact: keep every entry whose index score reaches 0.5.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Dynamic Fetching": all
// entries with I >= 0.5 are fetched, with no fixed count.  I >= 0.5 exactly
// when the logit z >= 0, so the gate compares the fp32 logit.
//
// Two passes over the logits of each sequence, both HBM-streaming:
//   count:   one workgroup per tile of kTile entries writes the tile's count;
//   scatter: each tile adds the counts of the tiles before it (a few dozen
//            values, from L2), then writes its kept indices in ascending
//            order through a workgroup-wide exclusive scan.
// The order of the output never depends on scheduling.
#include "common.hpp"

namespace lsa {

constexpr int kSelThreads = 256;
constexpr int kSelPer = 8;                              // entries per thread
constexpr int kTile = kSelThreads * kSelPer;            // 2048 entries per workgroup

__device__ __forceinline__ bool gate(float v, float thr) { return v >= thr; }  // NaN fails

// Loads this thread's 8 consecutive logits (two 16-byte loads when aligned).
__device__ __forceinline__ void load_tile8(const float* __restrict__ zb, int64_t s0, int64_t S,
                                           float (&v)[kSelPer]) {
    if (s0 + kSelPer <= S && ((reinterpret_cast<uintptr_t>(zb + s0) & 15u) == 0)) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(zb + s0);
        const f32x4 c = *reinterpret_cast<const f32x4*>(zb + s0 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = c[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) v[j] = (s0 + j < S) ? zb[s0 + j] : -INFINITY;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_select_count(
    const float* __restrict__ z, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ seq_len, int64_t max_len, float thr, int ntiles,
    int32_t* __restrict__ tile_count) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int64_t s0 = (int64_t)tile * kTile + (int64_t)threadIdx.x * kSelPer;
    int c = 0;
    if ((int64_t)tile * kTile < S) {
        float v[kSelPer];
        load_tile8(z + entry_start[b], s0, S, v);
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) c += (s0 + j < S && gate(v[j], thr)) ? 1 : 0;
    }
    // workgroup sum
    __shared__ int red[kSelThreads / kWave];
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int i = 0; i < kSelThreads / kWave; ++i) t += red[i];
        tile_count[(int64_t)b * ntiles + tile] = t;
    }
}

// Inclusive scan over a wave (64 lanes) with shuffles.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

__global__ __launch_bounds__(kSelThreads) void k_select_scatter(
    const float* __restrict__ z, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ seq_len, int64_t max_len, float thr, int ntiles,
    const int32_t* __restrict__ tile_count, int32_t* __restrict__ cand_idx,
    int32_t* __restrict__ cand_count) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int64_t tiles_b = (S + kTile - 1) / kTile;
    if (tile > 0 && tile >= tiles_b) return;

    __shared__ int wsum[kSelThreads / kWave];
    __shared__ int base_sh;
    // The tile's logits load first, so they are in flight with the counts of the
    // tiles before it (the barriers below wait for LDS only, not for them).
    const int64_t s0 = (int64_t)tile * kTile + (int64_t)threadIdx.x * kSelPer;
    float v[kSelPer];
    const bool live = (int64_t)tile * kTile < S;
    if (live) load_tile8(z + entry_start[b], s0, S, v);
    // offset of this tile = counts of the tiles before it
    int pre = 0;
    for (int i = threadIdx.x; i < tile; i += kSelThreads) pre += tile_count[(int64_t)b * ntiles + i];
    for (int off = 32; off > 0; off >>= 1) pre += __shfl_xor(pre, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = pre;
    lds_barrier();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int i = 0; i < kSelThreads / kWave; ++i) t += wsum[i];
        base_sh = t;
    }
    lds_barrier();
    const int base = base_sh;

    bool keep[kSelPer];
    int c = 0;
    if (live) {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            keep[j] = s0 + j < S && gate(v[j], thr);
            c += keep[j] ? 1 : 0;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) keep[j] = false;
    }
    const int incl = wave_incl_scan(c);
    lds_barrier();  // wsum reuse
    if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
    lds_barrier();
    int wpre = 0;
    const int w = threadIdx.x >> 6;
    for (int i = 0; i < w; ++i) wpre += wsum[i];
    int pos = base + wpre + incl - c;
    int32_t* out = cand_idx + entry_start[b];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j)
        if (keep[j]) out[pos++] = (int32_t)(s0 + j);
    const bool last_tile = tiles_b == 0 ? (tile == 0) : (tile == tiles_b - 1);
    if (last_tile && threadIdx.x == kSelThreads - 1) {
        int tot = 0;
        for (int i = 0; i < kSelThreads / kWave; ++i) tot += wsum[i];
        cand_count[b] = base + tot;
    }
}

}  // namespace lsa

using namespace lsa;

static int64_t select_tiles(int64_t max_len) {
    const int64_t t = ceil_div(max_len, kTile);
    return t < 1 ? 1 : t;
}

size_t lsa_select_workspace(int B, int64_t max_len) {
    return sizeof(int32_t) * (size_t)B * (size_t)select_tiles(max_len);
}

extern "C" int lsa_select_compact(const float* z, const int64_t* entry_start,
                                  const int32_t* seq_len, int B, int64_t max_len, float threshold,
                                  int32_t* cand_idx, int32_t* cand_count, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    clear_error();
    if (!z || !entry_start || !seq_len || !cand_idx || !cand_count)
        return fail(LSA_ERR_INVALID_ARG, "lsa_select_compact: a required pointer is NULL");
    if (B <= 0 || max_len < 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_select_compact: B=%d max_len=%lld", B,
                    (long long)max_len);
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "lsa_select_compact: B=%d > 65535", B);
    if (max_len > (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_select_compact: max_len too large");
    const size_t need = lsa_select_workspace(B, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(LSA_ERR_WORKSPACE, "lsa_select_compact: workspace %zu < %zu bytes",
                    workspace_bytes, need);
    int rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int ntiles = (int)select_tiles(max_len);
    dim3 grid((unsigned)ntiles, (unsigned)B);
    int32_t* tc = (int32_t*)workspace;
    hipLaunchKernelGGL(k_select_count, grid, dim3(kSelThreads), 0, st, z, entry_start, seq_len,
                       max_len, threshold, ntiles, tc);
    rc = launch_status("select_count");
    if (rc != LSA_OK) return rc;
    hipLaunchKernelGGL(k_select_scatter, grid, dim3(kSelThreads), 0, st, z, entry_start, seq_len,
                       max_len, threshold, ntiles, tc, cand_idx, cand_count);
    return launch_status("select_scatter");
}
