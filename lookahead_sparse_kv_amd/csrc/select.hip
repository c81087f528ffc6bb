// select.hip -- lsa_select_compact: keep every entry whose index score reaches 0.5.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Dynamic Fetching": all
// entries with I >= 0.5 are fetched, with no fixed count.  I >= 0.5 exactly
// when the logit z >= 0, so the gate compares the fp32 logit.
//
// From the logits: two passes over each sequence, both HBM-streaming:
//   count:   one workgroup per tile of kTile entries writes the tile's count;
//   scatter: each tile adds the counts of the tiles before it (a few dozen
//            values, from L2), then writes its kept indices in ascending
//            order through a workgroup-wide exclusive scan.
// From gate bits (one 16-bit word per 16 entries, set by the score kernels in
// the launch that computes the logits): one pass; each tile of kBitTile
// entries counts the set bits of all earlier tiles itself (1/128 of the
// logits' bytes), so no count pass runs.
// The order of the output never depends on scheduling.
#include <mutex>

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

constexpr int kBitTile = 8192;                          // entries per workgroup (bit form)
constexpr int kBitWords = kBitTile / 16;                // gate words per tile (512)
static_assert(kBitWords == 2 * kSelThreads, "two words per thread");

// Bit form: thread t of tile `tile` owns words 2t, 2t+1 of the tile (32 entries).
// Every load is issued at once, before the sequence length arrives: the words
// read are below gstride (a multiple of 8 that covers max_len), so in the
// caller's rows whatever S is, and bits past S are masked off afterwards.
__global__ __launch_bounds__(kSelThreads) void k_select_bits(
    const uint16_t* __restrict__ gate_bits, int64_t gstride,
    const int64_t* __restrict__ entry_start, const int32_t* __restrict__ seq_len,
    int64_t max_len, int32_t* __restrict__ cand_idx, int32_t* __restrict__ cand_count) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* row = gate_bits + (int64_t)b * gstride;   // 16-byte aligned
    const int len_b = seq_len[b];
    const int64_t eo = entry_start[b];

    // this thread's two words (w0 even, gstride a multiple of 8: both or neither)
    const int64_t w0 = (int64_t)tile * kBitWords + 2 * tid;
    uint32_t bits = w0 < gstride ? *reinterpret_cast<const uint32_t*>(row + w0) : 0u;
    // the words of the tiles before this one (below tile * kBitWords < gstride)
    const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
    const int nq = tile * (kBitWords / 8);                    // 16-byte words before the tile
    int pre = 0;
    for (int i0 = tid; i0 < nq; i0 += 4 * kSelThreads) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kSelThreads;
            v[u] = i < nq ? r4[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            pre += __popc(v[u][0]) + __popc(v[u][1]) + __popc(v[u][2]) + __popc(v[u][3]);
    }
    const int64_t S = min((int64_t)len_b, max_len);
    const int64_t tiles_b = (S + kBitTile - 1) / kBitTile;
    if (tile > 0 && tile >= tiles_b) return;
    // earlier tiles are whole (tile < tiles_b), so all their words count; here,
    // entries past S are masked off (a word holding entry S-1 need not be clean)
    const int64_t e0 = 16 * w0;
    const int64_t left = S - e0;
    if (left < 32) bits &= left > 0 ? (1u << left) - 1u : 0u;
    const int c = __popc(bits);
    // one pass of two wave scans: the earlier tiles' total and this tile's
    // exclusive positions
    __shared__ int wpre[kSelThreads / kWave];
    __shared__ int wcnt[kSelThreads / kWave];
    for (int off = 32; off > 0; off >>= 1) pre += __shfl_xor(pre, off);
    const int incl = wave_incl_scan(c);
    const int lane = tid & 63, w = tid >> 6;
    if (lane == 63) {
        wpre[w] = pre;
        wcnt[w] = incl;
    }
    lds_barrier();
    int base = 0, wbefore = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelThreads / kWave; ++i) {
        base += wpre[i];
        wbefore += i < w ? wcnt[i] : 0;
        tot += wcnt[i];
    }
    int pos = base + wbefore + incl - c;
    int32_t* out = cand_idx + eo;
    while (bits) {
        const int j = __ffs(bits) - 1;
        out[pos++] = (int32_t)(e0 + j);
        bits &= bits - 1u;
    }
    const bool last_tile = tiles_b == 0 ? (tile == 0) : (tile == tiles_b - 1);
    if (last_tile && tid == 0) cand_count[b] = base + tot;
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

// The two launches (count, then scatter), with the per-tile counts in `tc`.
static int select_launch(const char* who, const float* z, const int64_t* entry_start,
                         const int32_t* seq_len, int B, int64_t max_len, float threshold,
                         int32_t* cand_idx, int32_t* cand_count, int32_t* tc, hipStream_t st) {
    const int ntiles = (int)select_tiles(max_len);
    dim3 grid((unsigned)ntiles, (unsigned)B);
    hipLaunchKernelGGL(k_select_count, grid, dim3(kSelThreads), 0, st, z, entry_start, seq_len,
                       max_len, threshold, ntiles, tc);
    int rc = launch_status(who);
    if (rc != LSA_OK) return rc;
    hipLaunchKernelGGL(k_select_scatter, grid, dim3(kSelThreads), 0, st, z, entry_start, seq_len,
                       max_len, threshold, ntiles, tc, cand_idx, cand_count);
    return launch_status(who);
}

static int select_validate_sizes(const char* who, int B, int64_t max_len);

static int select_validate(const char* who, const float* z, const int64_t* entry_start,
                           const int32_t* seq_len, int B, int64_t max_len,
                           const int32_t* cand_idx, const int32_t* cand_count) {
    if (!z || !entry_start || !seq_len || !cand_idx || !cand_count)
        return fail(LSA_ERR_INVALID_ARG, "%s: a required pointer is NULL", who);
    return select_validate_sizes(who, B, max_len);
}

static int select_validate_sizes(const char* who, int B, int64_t max_len) {
    if (B <= 0 || max_len < 0)
        return fail(LSA_ERR_INVALID_ARG, "%s: B=%d max_len=%lld", who, B, (long long)max_len);
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "%s: B=%d > 65535", who, B);
    if (max_len > (int64_t)1 << 31) return fail(LSA_ERR_UNSUPPORTED, "%s: max_len too large", who);
    return LSA_OK;
}

extern "C" int lsa_select_compact(const float* z, const uint16_t* gate_bits,
                                  const int64_t* entry_start, const int32_t* seq_len, int B,
                                  int64_t max_len, float threshold, int32_t* cand_idx,
                                  int32_t* cand_count, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    clear_error();
    if (gate_bits) {
        if (!entry_start || !seq_len || !cand_idx || !cand_count)
            return fail(LSA_ERR_INVALID_ARG, "lsa_select_compact: a required pointer is NULL");
        if (!aligned16(gate_bits))
            return fail(LSA_ERR_INVALID_ARG, "lsa_select_compact: gate_bits must be 16-byte aligned");
        int rc = select_validate_sizes("lsa_select_compact", B, max_len);
        if (rc != LSA_OK) return rc;
        rc = check_device(nullptr);
        if (rc != LSA_OK) return rc;
        const int64_t t = ceil_div(max_len, kBitTile);
        dim3 grid((unsigned)(t < 1 ? 1 : t), (unsigned)B);
        hipLaunchKernelGGL(k_select_bits, grid, dim3(kSelThreads), 0, (hipStream_t)stream,
                           gate_bits, lsa_gate_words(max_len), entry_start, seq_len, max_len,
                           cand_idx, cand_count);
        return launch_status("lsa_select_compact");
    }
    int rc = select_validate("lsa_select_compact", z, entry_start, seq_len, B, max_len, cand_idx,
                             cand_count);
    if (rc != LSA_OK) return rc;
    const size_t need = lsa_select_workspace(B, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(LSA_ERR_WORKSPACE, "lsa_select_compact: workspace %zu < %zu bytes",
                    workspace_bytes, need);
    rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    return select_launch("lsa_select_compact", z, entry_start, seq_len, B, max_len, threshold,
                         cand_idx, cand_count, (int32_t*)workspace, (hipStream_t)stream);
}

// ------------------------------------------------- no-allocation variant
// The per-tile counts of lsa_select_compact_noalloc live in this file-scope
// device array (one copy per GPU, held until the process ends).  Its name is
// a host-side stand-in in host code: kernels get its device address, taken
// once per device with hipGetSymbolAddress.  Every tile count a call reads
// is written earlier in the same call, so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
namespace lsa {
constexpr int64_t kSelScratchTiles = (int64_t)1 << 18;   // 1 MiB of int32 tile counts
static __device__ __align__(256) int32_t scratch[kSelScratchTiles];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

// The device address of `scratch` on the current device (set up on first use).
static int scratch_address(const char* who, int32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(LSA_ERR_UNSUPPORTED, "%s: device id %d", who, dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(LSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = (int32_t*)ptr;
    }
    *out = g_scratch_ptr[dev];
    return LSA_OK;
}
}  // namespace lsa

extern "C" int lsa_select_compact_noalloc(const float* z, const int64_t* entry_start,
                                          const int32_t* seq_len, int B, int64_t max_len,
                                          float threshold, int32_t* cand_idx,
                                          int32_t* cand_count, void* stream) {
    clear_error();
    const char* who = "lsa_select_compact_noalloc";
    int rc = select_validate(who, z, entry_start, seq_len, B, max_len, cand_idx, cand_count);
    if (rc != LSA_OK) return rc;
    const int64_t tiles = (int64_t)B * select_tiles(max_len);
    if (tiles > kSelScratchTiles)
        return fail(LSA_ERR_UNSUPPORTED,
                    "%s: B * ceil(max_len / %d) = %lld tiles exceed the built-in scratch of %lld "
                    "(use lsa_select_compact with a workspace)",
                    who, kTile, (long long)tiles, (long long)kSelScratchTiles);
    rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    int32_t* tc = nullptr;
    rc = scratch_address(who, &tc);
    if (rc != LSA_OK) return rc;
    return select_launch(who, z, entry_start, seq_len, B, max_len, threshold, cand_idx,
                         cand_count, tc, (hipStream_t)stream);
}
