// topk.hip -- lsa_topk: fine-grained top-k inside the kept subset.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Tiered Selection": once
// the critical subset is resident, a top-k inside it picks the entries for the
// core attention.  Ranking: larger key first, equal keys by smaller entry
// index, NaN last, -0.0 == +0.0.  The kept set is returned in ascending index,
// as entry indices or (out_positions) as positions in the candidate list -- the
// rows of a hot buffer that holds the candidates' rows in list order.
//
// One workgroup (1024 threads) per sequence.  Keys are mapped to
// order-preserving uint32.  The k-th largest key U is found digit by digit,
// most significant first; the keys sharing the digits fixed so far shrink with
// every step, and once at most kShort remain they are copied to a short list,
// once at most kRank remain they are ranked exactly (count of larger and of
// equal keys).  A last ordered pass keeps every key > U and the first `need`
// keys == U (the smallest indices: candidates arrive in ascending order).
//
//   n <= kRegCap: every candidate stays in registers from the gather to the
//     output (wave w holds a contiguous run of 64-candidate chunks, key and
//     index); the first digit is the fixed top 12 bits (sign, exponent, 3
//     mantissa bits), histogrammed during the gather; the ordered pass uses
//     ballots per chunk and one scan over the 16 waves.
//   n >  kRegCap: keys in a global scratch area; 8-bit digits starting below
//     the bits every candidate shares; the ordered pass walks per-thread runs.
#include "common.hpp"

namespace lsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kRunChunks = 32;                   // most 64-candidate chunks per wave in registers
constexpr int kRegCap = kTkWaves * kRunChunks * kWave;  // 32768 candidates
constexpr int kHistCopies = 16;                  // lane-spread copies of each 8-bit radix bin
constexpr int kShort = 2048;                     // longest digit list copied to the short list
constexpr int kRank = 256;                       // longest list ranked by direct counting
constexpr int kD0 = 12;                          // first digit of the register path (bits 31..20)
constexpr int kBins0 = 1 << kD0;
constexpr int kCopies0 = 8;                      // lane-spread copies of each first-digit bin
constexpr int kHistWords = kBins0 * kCopies0;    // 128 KiB; the 8-bit passes use the first 4096
static_assert(kBins0 == 4 * kTkThreads && 256 * kHistCopies <= kHistWords, "histogram layout");

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

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Counts of four consecutive bins of COPIES lane-spread copies each (the
// 16 COPIES bytes at `bins`, one thread's block).  A block is a whole number of
// 128-byte bank rows and the threads' blocks are adjacent, so reading them in
// the same order would put every lane of a 16-byte load on the same banks; lane
// l starts at 16-byte chunk l instead and walks its block round robin.
template <int COPIES>
__device__ __forceinline__ void sum_bins4(const unsigned* bins, int lane, int (&c4)[4]) {
    constexpr int CH = COPIES;                 // 16-byte chunks per block (4 bins x COPIES/4)
    constexpr int CPB = COPIES / 4;            // chunks per bin
#pragma unroll
    for (int q = 0; q < 4; ++q) c4[q] = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = (i + lane) & (CH - 1);
        const u32x4 v = reinterpret_cast<const u32x4*>(bins)[c];
        const int t = (int)(v[0] + v[1] + v[2] + v[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) c4[q] += (c / CPB == q) ? t : 0;
    }
}

// Search state: the need-th largest key among those with (key & pmask) == prefix
// is the k-th key overall; m keys match; bits below hi are still open.
struct RadixState {
    uint32_t prefix, pmask;
    int hi, m, need;
};

// Narrow the search until every bit is fixed (prefix = U, need = how many keys
// equal to U to take).  Workgroup-wide; hist holds >= 256 * kHistCopies words.
// Global-path refinement over keys[0..n) (IN_LDS selects the padded LDS layout):
// narrow the search until every bit is fixed (prefix = U, need = how many keys
// equal to U to take).  Workgroup-wide; hist holds >= 256 * kHistCopies words.
template <bool IN_LDS>
__device__ void radix_refine(const uint32_t* keys, int n, RadixState& st, unsigned* hist,
                             uint32_t* shortl, int* sh);

// The 8-bit digit search shared by both refinements: lane l of wave 0 owns
// digits 4l..4l+3 of the histogram; writes (digit, need within it, its count).
__device__ __forceinline__ void digit_search(const unsigned* hist, int need, int* sh) {
    const int tid = threadIdx.x;
    int c4[4];
    // (one wave; reading the blocks round robin as in the first digit measured slower here)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4* hq = reinterpret_cast<const u32x4*>(&hist[(4 * tid + q) * kHistCopies]);
        int t = 0;
#pragma unroll
        for (int i = 0; i < kHistCopies / 4; ++i) {
            const u32x4 v = hq[i];
            t += (int)(v[0] + v[1] + v[2] + v[3]);
        }
        c4[q] = t;
    }
    const int tot = c4[0] + c4[1] + c4[2] + c4[3];
    int suf = tot;  // inclusive suffix sum over lanes >= tid
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(suf, off);
        if (tid + off < 64) suf += y;
    }
    const int above = suf - tot;  // keys with a digit in higher lanes
    if (above < need && need <= suf) {
        int acc = above, q = 3;
        for (; q > 0; --q) {
            if (acc + c4[q] >= need) break;
            acc += c4[q];
        }
        sh[0] = 4 * tid + q;
        sh[1] = need - acc;
        sh[2] = c4[q];
    }
}

// Exact rank of the k-th key among the m keys in list[0..m): the key with
// (#larger) < need <= (#larger + #equal); every thread holding such a key writes
// the same answer to sh[4], sh[5].
__device__ __forceinline__ void rank_list(const uint32_t* list, int m, int need, int* sh) {
    const int tid = threadIdx.x;
    if (tid < m) {
        const uint32_t x = list[tid];
        int gt = 0, eq = 0;
        for (int i = 0; i < (m & ~3); i += 4) {
            const u32x4 y = *reinterpret_cast<const u32x4*>(&list[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gt += y[e] > x;
                eq += y[e] == x;
            }
        }
        for (int i = m & ~3; i < m; ++i) {
            gt += list[i] > x;
            eq += list[i] == x;
        }
        if (gt < need && need <= gt + eq) {
            sh[4] = (int)x;
            sh[5] = need - gt;
        }
    }
}

// n <= kRegCap: candidates in registers.  Wave w holds chunks [w*cpw, (w+1)*cpw)
// of 64 consecutive candidates; lane l of chunk u is candidate (w*cpw + u)*64 + l.
// RC >= cpw is the register window: every per-chunk loop is unrolled RC times
// and the code runs once per workgroup, so the caller picks the smallest RC
// that fits (instruction fetch of unused chunk bodies costs real time).
template <int RC, bool POS>
__device__ void topk_regs(const float* __restrict__ rb, const int32_t* __restrict__ cand, int n,
                          int k, int32_t* __restrict__ out, unsigned* hist, uint32_t* shortl,
                          int* scratch, int* sh) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cpw = (n + kTkWaves * kWave - 1) / (kTkWaves * kWave);
    const int wb = wave * cpw * kWave;
    uint32_t kr[RC];
    int cr[RC];
    // gather: candidate indices, then their keys (every load of the run in flight);
    // the histogram is cleared meanwhile
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        cr[u] = 0;
        if (u < cpw) cr[u] = cand[min(wb + kWave * u + lane, n - 1)];
    }
    for (int i = tid; i < kHistWords / 4; i += kTkThreads)
        reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
    float v[RC];
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        v[u] = 0.0f;
        if (u < cpw) v[u] = rb[cr[u]];
    }
    __syncthreads();                                       // histogram cleared
    const int copy = lane & (kCopies0 - 1);
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        kr[u] = 0u;
        if (u < cpw) {
            const bool in = wb + kWave * u + lane < n;
            kr[u] = in ? order_key(v[u]) : 0u;
            if (in) atomicAdd(&hist[(kr[u] >> (32 - kD0)) * kCopies0 + copy], 1u);
        }
    }
    auto valid = [&](int u) { return u < cpw && wb + kWave * u + lane < n; };
    __syncthreads();
    // First digit: thread t owns bins 4(1023-t) .. +3, so the exclusive scan over
    // threads counts the keys in higher bins.
    {
        const int bb = 4 * (kTkThreads - 1 - tid);
        int c4[4];
        sum_bins4<kCopies0>(hist + bb * kCopies0, lane, c4);
        const int tot4 = c4[0] + c4[1] + c4[2] + c4[3];
        int total;
        const int above = block_excl_scan(tot4, scratch, &total);
        if (above < k && k <= above + tot4) {
            int acc = above, q = 3;
            for (; q > 0; --q) {
                if (acc + c4[q] >= k) break;
                acc += c4[q];
            }
            sh[0] = bb + q;
            sh[1] = k - acc;
            sh[2] = c4[q];
        }
    }
    __syncthreads();
    uint32_t prefix = (uint32_t)sh[0] << (32 - kD0);
    uint32_t pmask = ~0u << (32 - kD0);
    int hi = 32 - kD0, m = sh[2], need = sh[1];

    // Refine until every bit of U is fixed.
    bool in_short = false;
    while (hi > 0) {
        if (m <= kRank) {
            // gather the m matching keys into the (free) histogram area and rank them
            __syncthreads();                               // hist and sh are free
            if (tid == 0) sh[3] = 0;
            __syncthreads();
            if (in_short) {
                for (int j = tid; j < sh[6]; j += kTkThreads) {
                    const uint32_t x = shortl[j];
                    if ((x & pmask) == prefix) hist[atomicAdd(&sh[3], 1)] = x;
                }
            } else {
#pragma unroll
                for (int u = 0; u < RC; ++u)
                    if (valid(u) && (kr[u] & pmask) == prefix) hist[atomicAdd(&sh[3], 1)] = kr[u];
            }
            __syncthreads();
            rank_list(hist, m, need, sh);
            __syncthreads();
            prefix = (uint32_t)sh[4];
            need = sh[5];
            break;
        }
        if (!in_short && m <= kShort) {
            // copy the matching keys (any order) to the short list; later steps scan it
            __syncthreads();                               // every thread has read sh
            if (tid == 0) sh[3] = 0;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < RC; ++u)
                if (valid(u) && (kr[u] & pmask) == prefix) shortl[atomicAdd(&sh[3], 1)] = kr[u];
            __syncthreads();
            if (tid == 0) sh[6] = sh[3];                   // list length
            in_short = true;
        }
        // one pass over the next (up to) 8 bits
        const int lo = max(hi - 8, 0);
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        __syncthreads();                                   // previous step done with hist/sh
        for (int i = tid; i < 256 * kHistCopies; i += kTkThreads) hist[i] = 0;
        __syncthreads();
        const int hcopy = tid & (kHistCopies - 1);
        if (in_short) {
            for (int j = tid; j < sh[6]; j += kTkThreads) {
                const uint32_t x = shortl[j];
                if ((x & pmask) == prefix) atomicAdd(&hist[((x >> lo) & dmask) * kHistCopies + hcopy], 1u);
            }
        } else {
#pragma unroll
            for (int u = 0; u < RC; ++u)
                if (valid(u) && (kr[u] & pmask) == prefix)
                    atomicAdd(&hist[((kr[u] >> lo) & dmask) * kHistCopies + hcopy], 1u);
        }
        __syncthreads();
        if (tid < 64) digit_search(hist, need, sh);
        __syncthreads();
        prefix |= (uint32_t)sh[0] << lo;
        pmask |= dmask << lo;
        need = sh[1];
        m = sh[2];
        hi = lo;
    }
    const uint32_t U = prefix;

    // Ordered compaction: counts per wave by ballots, one scan over the waves,
    // then every chunk writes its selected candidates contiguously.
    int gt_w = 0, eq_w = 0;
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        if (u < cpw) {
            const bool in = valid(u);
            gt_w += __popcll(__ballot(in && kr[u] > U));
            eq_w += __popcll(__ballot(in && kr[u] == U));
        }
    }
    __syncthreads();                                       // scratch and sh are free
    if (lane == 0) {
        scratch[wave] = gt_w;
        scratch[kTkWaves + wave] = eq_w;
    }
    __syncthreads();
    // output slot and equal keys before this wave: lane j < 16 holds wave j's
    // counts; one shuffle scan gives each wave's share of the equal keys
    int pos, eqs;
    {
        const bool lw = lane < kTkWaves;
        const int gtj = lw ? scratch[lane] : 0;
        const int eqj = lw ? scratch[kTkWaves + lane] : 0;
        int eq_incl = eqj;
#pragma unroll
        for (int off = 1; off < kTkWaves; off <<= 1) {
            const int y = __shfl_up(eq_incl, off);
            if (lane >= off) eq_incl += y;
        }
        const int eq_before = eq_incl - eqj;
        int term = gtj + max(0, min(need - eq_before, eqj));   // wave j's selected keys
#pragma unroll
        for (int off = 1; off < kTkWaves; off <<= 1) {
            const int y = __shfl_up(term, off);
            if (lane >= off) term += y;
        }
        const int term_excl = __shfl(term, max(wave - 1, 0));
        pos = wave > 0 ? term_excl : 0;
        eqs = __shfl(eq_before, wave);
    }
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        if (u < cpw) {                                     // uniform
            const bool in = valid(u);
            const bool g = in && kr[u] > U;
            const bool e = in && kr[u] == U;
            const uint64_t be = __ballot(e);
            const bool sel = g || (e && eqs + lanes_below(be) < need);
            const uint64_t bs = __ballot(sel);
            if (sel) out[pos + lanes_below(bs)] = POS ? wb + kWave * u + lane : cr[u];
            pos += __popcll(bs);
            eqs += __popcll(be);
        }
    }
}

template <bool IN_LDS>
__device__ void radix_refine(const uint32_t* keys, int n, RadixState& st, unsigned* hist,
                             uint32_t* shortl, int* sh) {
    auto P = [](int j) { return IN_LDS ? j + (j >> 5) : j; };
    const int tid = threadIdx.x;
    bool in_short = false;
    int cnt = n;                                           // keys scanned per step
    while (st.hi > 0) {
        if (st.m <= kRank) {
            __syncthreads();                               // hist and sh are free
            if (tid == 0) sh[3] = 0;
            __syncthreads();
            for (int j = tid; j < cnt; j += kTkThreads) {
                const uint32_t u = in_short ? shortl[j] : keys[P(j)];
                if ((u & st.pmask) == st.prefix) hist[atomicAdd(&sh[3], 1)] = u;
            }
            __syncthreads();
            rank_list(hist, st.m, st.need, sh);
            __syncthreads();
            st.prefix = (uint32_t)sh[4];
            st.need = sh[5];
            st.hi = 0;
            return;
        }
        if (!in_short && st.m <= kShort) {
            __syncthreads();                               // every thread has read sh
            if (tid == 0) sh[3] = 0;
            __syncthreads();
            for (int j = tid; j < n; j += kTkThreads) {
                const uint32_t u = keys[P(j)];
                if ((u & st.pmask) == st.prefix) shortl[atomicAdd(&sh[3], 1)] = u;
            }
            in_short = true;
            cnt = st.m;
        }
        const int lo = max(st.hi - 8, 0);
        const uint32_t dmask = (1u << (st.hi - lo)) - 1u;
        __syncthreads();                                   // previous step done with hist/sh
        for (int i = tid; i < 256 * kHistCopies; i += kTkThreads) hist[i] = 0;
        __syncthreads();
        // kHistCopies copies of every bin, picked by lane, so lanes counting the
        // same digit hit different banks instead of serialising on one word
        const int copy = tid & (kHistCopies - 1);
        for (int j = tid; j < cnt; j += kTkThreads) {
            const uint32_t u = in_short ? shortl[j] : keys[P(j)];
            if ((u & st.pmask) == st.prefix)
                atomicAdd(&hist[((u >> lo) & dmask) * kHistCopies + copy], 1u);
        }
        __syncthreads();
        if (tid < 64) digit_search(hist, st.need, sh);
        __syncthreads();
        st.prefix |= (uint32_t)sh[0] << lo;
        st.pmask |= dmask << lo;
        st.need = sh[1];
        st.m = sh[2];
        st.hi = lo;
    }
}

// n > kRegCap: keys in the global scratch area (plain layout).
template <bool IN_LDS, bool POS>
__device__ void topk_global(const float* __restrict__ rb, const int32_t* __restrict__ cand, int n,
                            int k, uint32_t* keys, int32_t* __restrict__ out, unsigned* hist,
                            uint32_t* shortl, int* scratch, int* sh) {
    auto P = [](int j) { return IN_LDS ? j + (j >> 5) : j; };
    const int tid = threadIdx.x;
    // Gather the keys, 8 independent loads in flight per thread.  The AND and OR
    // of all keys give the bits every candidate shares.
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
    const uint32_t diff = kand ^ kor;
    const int top = diff ? 31 - __clz(diff) : -1;          // highest differing bit
    const uint32_t pmask = top >= 31 ? 0u : (~0u << (top + 1));
    RadixState st{kand & pmask, pmask, top + 1, n, k};
    radix_refine<IN_LDS>(keys, n, st, hist, shortl, sh);
    const uint32_t U = st.prefix;
    const int need = st.need;

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
            out[pos++] = POS ? j : cj;
        } else if (key == U) {
            if (eq_seen < need) out[pos++] = POS ? j : cj;
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

template <bool POS>
__global__ __launch_bounds__(kTkThreads) void k_topk(
    const float* __restrict__ r, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ seq_len, int64_t max_len, const int32_t* __restrict__ cand_idx,
    const int32_t* __restrict__ cand_count, int k, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ topk_count, uint32_t* __restrict__ gkeys) {
    __shared__ __attribute__((aligned(16))) unsigned hist[kHistWords];
    __shared__ __attribute__((aligned(16))) uint32_t shortl[kShort];
    __shared__ int scratch[2 * kTkWaves];
    __shared__ int sh[8];
    const int b = blockIdx.x;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int n = (int)max((int64_t)0, min((int64_t)cand_count[b], S));
    const int64_t eo = entry_start[b];
    const int32_t* cand = cand_idx + eo;
    int32_t* out = topk_idx + (int64_t)b * k;
    if (n <= k) {
        for (int j = threadIdx.x; j < n; j += kTkThreads) out[j] = POS ? j : cand[j];
        if (threadIdx.x == 0) topk_count[b] = n;
        return;
    }
    const int cpw = (n + kTkWaves * kWave - 1) / (kTkWaves * kWave);   // chunks per wave
#define LSA_TK_REGS(rc)                                                        \
    else if (cpw <= rc) topk_regs<rc, POS>(r + eo, cand, n, k, out, hist, shortl, scratch, sh);
    if (false) {
    }
    // steps of 8 chunks: finer steps make workgroups of one launch run different
    // bodies, which then share fewer instruction-cache lines (measured slower)
    LSA_TK_REGS(8) LSA_TK_REGS(16) LSA_TK_REGS(24) LSA_TK_REGS(kRunChunks)
#undef LSA_TK_REGS
    else
        topk_global<false, POS>(r + eo, cand, n, k, gkeys + (int64_t)b * max_len, out, hist,
                                shortl, scratch, sh);
    if (threadIdx.x == 0) topk_count[b] = k;
}

}  // namespace lsa

using namespace lsa;

size_t lsa_topk_workspace(int B, int64_t max_len) {
    return max_len > kRegCap ? sizeof(uint32_t) * (size_t)B * (size_t)max_len : 0;
}

extern "C" int lsa_topk(const float* rank_key, const int64_t* entry_start, const int32_t* seq_len,
                        int B, int64_t max_len, const int32_t* cand_idx, const int32_t* cand_count,
                        int k, int32_t* topk_idx, int32_t* topk_count, int out_positions,
                        void* workspace, size_t workspace_bytes, void* stream) {
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
    if (out_positions)
        hipLaunchKernelGGL(k_topk<true>, dim3((unsigned)B), dim3(kTkThreads), 0,
                           (hipStream_t)stream, rank_key, entry_start, seq_len, max_len, cand_idx,
                           cand_count, k, topk_idx, topk_count, (uint32_t*)workspace);
    else
        hipLaunchKernelGGL(k_topk<false>, dim3((unsigned)B), dim3(kTkThreads), 0,
                           (hipStream_t)stream, rank_key, entry_start, seq_len, max_len, cand_idx,
                           cand_count, k, topk_idx, topk_count, (uint32_t*)workspace);
    return launch_status("topk");
}
