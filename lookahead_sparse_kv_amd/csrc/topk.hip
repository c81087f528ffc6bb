// topk.hip -- lsa_topk: fine-grained top-k inside the kept subset.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Tiered Selection": once
// the critical subset is resident, a top-k inside it picks the entries for the
// core attention.  Ranking: larger key first, equal keys by smaller entry
// index, NaN last, -0.0 == +0.0.  The kept set is returned in ascending index.
//
// One workgroup (1024 threads) per sequence.  Keys are mapped to
// order-preserving uint32, staged in LDS (up to kCap candidates; larger sets
// use a global scratch area), and a radix select over 8-bit digits -- starting
// below the bits every candidate shares -- finds the k-th key U and how many
// keys equal to U to take.  A last ordered pass
// keeps every key > U and the first `need` keys == U (the smallest indices,
// since candidates are in ascending order), compacted with workgroup scans.
#include "common.hpp"

namespace lsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kCap = 32768;                      // candidates held in LDS
constexpr int kCapPadded = kCap + kCap / 32;     // one pad word per 32 (bank spread)
constexpr int kHistCopies = 16;                  // lane-spread copies of each radix bin

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;                 // NaN ranks below every number
    if (u == 0x80000000u) u = 0u;          // -0.0 ranks with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread across the workgroup; returns the total in *total.
__device__ __forceinline__ int block_excl_scan(int x, int* scratch, int* total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    __syncthreads();
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int i = 0; i < kTkWaves; ++i) {
        const int s = scratch[i];
        pre += (i < w) ? s : 0;
        tot += s;
    }
    *total = tot;
    return pre + incl - x;
}

template <bool IN_LDS>
__device__ void topk_body(const float* __restrict__ rb, const int32_t* __restrict__ cand, int n,
                          int k, uint32_t* keys, int32_t* __restrict__ out, unsigned* hist,
                          int* scratch, int* sh) {
    auto P = [](int j) { return IN_LDS ? j + (j >> 5) : j; };
    const int tid = threadIdx.x;
    // Gather the keys, 8 independent loads in flight per thread (indices are
    // clamped instead of branched on, so no load waits for the previous one).
    // The AND and OR of all keys give the bits every candidate shares.
    uint32_t kand = ~0u, kor = 0u;
    for (int j0 = tid; j0 < n; j0 += 8 * kTkThreads) {
        int c[8];
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cand[min(j0 + u * kTkThreads, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = rb[c[u]];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * kTkThreads;
            const uint32_t key = order_key(v[u]);
            kand &= key;
            kor |= key;
            if (j < n) keys[P(j)] = key;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kand &= (uint32_t)__shfl_xor((int)kand, off);
        kor |= (uint32_t)__shfl_xor((int)kor, off);
    }
    if ((tid & 63) == 0) {
        scratch[tid >> 6] = (int)kand;
        scratch[kTkWaves + (tid >> 6)] = (int)kor;
    }
    __syncthreads();
    kand = ~0u;
    kor = 0u;
    for (int i = 0; i < kTkWaves; ++i) {
        kand &= (uint32_t)scratch[i];
        kor |= (uint32_t)scratch[kTkWaves + i];
    }

    // Radix select over the bits where candidates differ, most significant
    // first, 8 bits per pass: histogram the digit among keys that match the
    // prefix fixed so far, then keep the digit holding the need-th largest key.
    const uint32_t diff = kand ^ kor;
    const int top = diff ? 31 - __clz(diff) : -1;          // highest differing bit
    uint32_t pmask = top >= 31 ? 0u : (~0u << (top + 1));
    uint32_t prefix = kand & pmask;
    int need = k;
    for (int hi = top + 1; hi > 0;) {
        const int lo = max(hi - 8, 0);
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        __syncthreads();                                   // previous pass done with hist/sh
        for (int i = tid; i < 256 * kHistCopies; i += kTkThreads) hist[i] = 0;
        __syncthreads();
        // kHistCopies copies of every bin, picked by lane, so lanes counting the
        // same digit hit different banks instead of serialising on one word
        const int copy = tid & (kHistCopies - 1);
        for (int j = tid; j < n; j += kTkThreads) {
            const uint32_t u = keys[P(j)];
            if ((u & pmask) == prefix) atomicAdd(&hist[((u >> lo) & dmask) * kHistCopies + copy], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 4l..4l+3; find the digit d with
            // (#keys with digit > d) < need <= (#keys with digit >= d).
            int cnt[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4* hq = reinterpret_cast<const u32x4*>(&hist[(4 * tid + q) * kHistCopies]);
                int t = 0;
#pragma unroll
                for (int i = 0; i < kHistCopies / 4; ++i) {
                    const u32x4 v = hq[i];
                    t += (int)(v[0] + v[1] + v[2] + v[3]);
                }
                cnt[q] = t;
            }
            const int c0 = cnt[0], c1 = cnt[1], c2 = cnt[2], c3 = cnt[3];
            const int tot = c0 + c1 + c2 + c3;
            int suf = tot;  // inclusive suffix sum over lanes >= tid
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_down(suf, off);
                if (tid + off < 64) suf += y;
            }
            const int above = suf - tot;  // keys with a digit in higher lanes
            if (above < need && need <= suf) {
                int acc = above, d = 4 * tid + 3;
                const int cs[4] = {c0, c1, c2, c3};
                for (int q = 3; q >= 0; --q) {
                    if (acc + cs[q] >= need) {
                        d = 4 * tid + q;
                        break;
                    }
                    acc += cs[q];
                }
                sh[0] = d;
                sh[1] = need - acc;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh[0] << lo;
        pmask |= dmask << lo;
        need = sh[1];
        hi = lo;
    }
    const uint32_t U = prefix;

    // Ordered compaction: thread t walks candidates [t*per, (t+1)*per).  The
    // first 16 candidate indices of the run are fetched now, so their latency
    // hides behind the counting and the two workgroup scans.
    const int per = (n + kTkThreads - 1) / kTkThreads;
    const int j0 = min(tid * per, n), j1 = min(j0 + per, n);
    int cpre[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) cpre[u] = cand[min(j0 + u, n - 1)];
    int gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t u = keys[P(j)];
        gt += u > U;
        eq += u == U;
    }
    int tot;
    const int eq_base = block_excl_scan(eq, scratch, &tot);
    const int take_eq = max(0, min(need - eq_base, eq));
    int pos = block_excl_scan(gt + take_eq, scratch, &tot);
    int eq_seen = eq_base;
    auto emit = [&](int j, int cj) {
        const uint32_t key = keys[P(j)];
        if (key > U) {
            out[pos++] = cj;
        } else if (key == U) {
            if (eq_seen < need) out[pos++] = cj;
            ++eq_seen;
        }
    };
#pragma unroll
    for (int u = 0; u < 16; ++u)
        if (j0 + u < j1) emit(j0 + u, cpre[u]);
    for (int jb = j0 + 16; jb < j1; jb += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cand[min(jb + u, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (jb + u < j1) emit(jb + u, c[u]);
    }
}

__global__ __launch_bounds__(kTkThreads) void k_topk(
    const float* __restrict__ r, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ seq_len, int64_t max_len, const int32_t* __restrict__ cand_idx,
    const int32_t* __restrict__ cand_count, int k, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ topk_count, uint32_t* __restrict__ gkeys) {
    __shared__ uint32_t skeys[kCapPadded];
    __shared__ __attribute__((aligned(16))) unsigned hist[256 * kHistCopies];
    __shared__ int scratch[2 * kTkWaves];
    __shared__ int sh[2];
    const int b = blockIdx.x;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int n = (int)max((int64_t)0, min((int64_t)cand_count[b], S));
    const int64_t eo = entry_start[b];
    const int32_t* cand = cand_idx + eo;
    int32_t* out = topk_idx + (int64_t)b * k;
    if (n <= k) {
        for (int j = threadIdx.x; j < n; j += kTkThreads) out[j] = cand[j];
        if (threadIdx.x == 0) topk_count[b] = n;
        return;
    }
    if (n <= kCap)
        topk_body<true>(r + eo, cand, n, k, skeys, out, hist, scratch, sh);
    else
        topk_body<false>(r + eo, cand, n, k, gkeys + (int64_t)b * max_len, out, hist, scratch, sh);
    if (threadIdx.x == 0) topk_count[b] = k;
}

}  // namespace lsa

using namespace lsa;

size_t lsa_topk_workspace(int B, int64_t max_len) {
    return max_len > kCap ? sizeof(uint32_t) * (size_t)B * (size_t)max_len : 0;
}

extern "C" int lsa_topk(const float* rank_key, const int64_t* entry_start, const int32_t* seq_len,
                        int B, int64_t max_len, const int32_t* cand_idx, const int32_t* cand_count,
                        int k, int32_t* topk_idx, int32_t* topk_count, void* workspace,
                        size_t workspace_bytes, void* stream) {
    clear_error();
    if (!rank_key || !entry_start || !seq_len || !cand_idx || !cand_count || !topk_idx ||
        !topk_count)
        return fail(LSA_ERR_INVALID_ARG, "lsa_topk: a required pointer is NULL");
    if (B <= 0 || max_len < 0 || k <= 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_topk: B=%d max_len=%lld k=%d", B,
                    (long long)max_len, k);
    if (k > 65536) return fail(LSA_ERR_UNSUPPORTED, "lsa_topk: k=%d > 65536", k);
    if (B > 1 << 20) return fail(LSA_ERR_UNSUPPORTED, "lsa_topk: B=%d too large", B);
    if (max_len > (int64_t)1 << 31) return fail(LSA_ERR_UNSUPPORTED, "lsa_topk: max_len too large");
    const size_t need = lsa_topk_workspace(B, max_len);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(LSA_ERR_WORKSPACE, "lsa_topk: workspace %zu < %zu bytes", workspace_bytes,
                    need);
    int rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)B), dim3(kTkThreads), 0, (hipStream_t)stream,
                       rank_key, entry_start, seq_len, max_len, cand_idx, cand_count, k, topk_idx,
                       topk_count, (uint32_t*)workspace);
    return launch_status("topk");
}
