// encode.hip -- lsa_query_encode: the Memory Indexer's query encoder.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Memory Indexer" (the query
// token's hidden state h_t is mapped into low-rank indexer queries) and 2.3
// "Query Optimization" (the encoder's low-rank projection matrices).  Per token m:
//     c[m]    = W_down h[m]            rank r, kept in bf16 between the products
//     q[m, h] = W_up[h] c[m]           bf16: the score's per-head queries
//     w[m, h] = W_gate[h] . h[m]       fp32: the score's per-head gate weights
//
// Two launches of one product D = A B^T, A [M, K] activations and B [N, K]
// weight rows, both bf16 with K contiguous, fp32 accumulation on the matrix
// cores:
//     1) A = h, B = [W_down ; W_gate] (N = r + H): columns < r go to c (bf16),
//        the others to w (fp32) -- the gate rides along the down projection;
//     2) A = c, B = W_up (N = H*D): q (bf16).
// Few tokens (decode: one per sequence) make each product a stream of the
// weights, bound by HBM: k_encode_skinny gives every workgroup 16 weight rows
// and splits K over its waves, each wave holding all the tokens' rows in
// registers, so every weight byte is read once; for up to 8 tokens and a long
// K, k_encode_rows gives a workgroup 4 rows (vector dot products) so that
// more workgroups stream at once; one token, k_encode_stream, an equal share of
// the rows per CU with every load in flight.  Many tokens (a burst of tau positions):
// k_encode_tiled, an LDS-tiled product bound by the matrix cores.
#include "common.hpp"

// LDS stages of the tiled product per tile shape
#ifndef LSA_ENC_NS22
#define LSA_ENC_NS22 2
#endif
#ifndef LSA_ENC_NS21
#define LSA_ENC_NS21 4
#endif
#ifndef LSA_ENC_NS11
#define LSA_ENC_NS11 4
#endif
// K depth of one stage per tile shape (64 or 32)
#ifndef LSA_ENC_BK22
#define LSA_ENC_BK22 64
#endif
#ifndef LSA_ENC_BK21
#define LSA_ENC_BK21 64
#endif
#ifndef LSA_ENC_BK11
#define LSA_ENC_BK11 64
#endif
// 128x64 tiles are taken when they fill at least this percentage of the CUs
#ifndef LSA_ENC_FILL21
#define LSA_ENC_FILL21 75
#endif

namespace lsa {

// D = A B^T with column routing: weight row n < nsplit comes from b0 (row n)
// and its output goes to out0 (bf16); row n >= nsplit comes from b1 (row
// n - nsplit) and goes to out1 (fp32, column n - nsplit).
struct EncGemm {
    const bf16* a;
    int64_t lda;
    const bf16* b0;
    const bf16* b1;
    int M, N, K, nsplit;
    bf16* out0;
    int64_t ld0;
    float* out1;
    int64_t ld1;
};

__device__ __forceinline__ const bf16* enc_brow(const EncGemm& g, int n) {
    return n < g.nsplit ? g.b0 + (int64_t)n * g.K : g.b1 + (int64_t)(n - g.nsplit) * g.K;
}

__device__ __forceinline__ void enc_store(const EncGemm& g, int m, int n, float v) {
    if (n < g.nsplit)
        g.out0[(int64_t)m * g.ld0 + n] = (bf16)v;
    else
        g.out1[(int64_t)m * g.ld1 + (n - g.nsplit)] = v;
}

// ------------------------------------------------------------- few tokens
// Workgroup: weight rows n0 .. n0+15; wave w takes an even share of the K
// steps (32 deep) and keeps U steps of loads in flight; MT tiles of 16 token
// rows share each weight fragment.  The waves' partial sums meet in LDS and are
// added in wave order (deterministic).  Rows past M or N are computed on a
// clamped row and never stored.
template <int MT, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void k_encode_skinny(EncGemm g) {
    __shared__ float red[WAVES][MT][4][kWave];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const bf16* brow = enc_brow(g, min(n0 + (lane & 15), g.N - 1));
    const bf16* arow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) arow[t] = g.a + (int64_t)min(16 * t + (lane & 15), g.M - 1) * g.lda;
    const int kq = 8 * (lane >> 4);
    const int steps = g.K / 32;
    const int s0 = steps * wave / WAVES, s1 = steps * (wave + 1) / WAVES;
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; s += U) {
        bf16x8 bv[U], av[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < s1) {
                const int k = 32 * (s + u) + kq;
                bv[u] = load8(brow + k);
#pragma unroll
                for (int t = 0; t < MT; ++t) av[u][t] = load8(arow[t] + k);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < s1) {
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = mfma16(av[u][t], bv[u], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][t][v][lane] = acc[t][v];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * 4 * kWave; e += WAVES * kWave) {
        const int t = e / (4 * kWave), v = (e / kWave) & 3, l = e & 63;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += red[w][t][v][l];
        const int m = 16 * t + 4 * (l >> 4) + v, n = n0 + (l & 15);
        if (m < g.M && n < g.N) enc_store(g, m, n, sum);
    }
}

// ---------------------------------------------------------- fewest tokens
// M <= 8 (decode: one token per sequence): a plain vector product, as the
// matrix cores would idle on 8 token rows.  Workgroup = R weight rows, so the
// down product's 1600 rows give 400 workgroups and every CU streams weights
// (16-row blocks gave 100).  Thread t takes the 8-element K chunks t, t + 256,
// ... of all R rows and all MT token rows (U chunks in flight) and keeps R x MT
// fp32 sums, accumulated with bf16 pair dot products (the products of two bf16
// values are exact in fp32); the 256 threads' sums meet through LDS in a fixed
// order (deterministic): 8 slices of 32 threads each, then the 8 slice sums.
// Token rows past M are computed on row M-1 and never stored; weight rows past
// N likewise.
template <int R, int MT, int U>
__global__ __launch_bounds__(256) void k_encode_rows(EncGemm g) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    constexpr int NV = R * MT;                   // sums per thread
    constexpr int SL = 256 / NV;                 // slices of the first reduction step
    static_assert(NV * SL == 256 && NV <= 64, "reduction layout");
    // row stride NV + 1: the 64 lanes of a read fall on 64 distinct banks
    __shared__ float part[256][NV + 1];
    __shared__ float slice[SL][NV];
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * R;
    const bf16* brow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) brow[r] = enc_brow(g, min(n0 + r, g.N - 1));
    const bf16* arow[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) arow[m] = g.a + (int64_t)min(m, g.M - 1) * g.lda;
    const int nch = g.K / 8;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
    for (int c0 = tid; c0 < nch; c0 += 256 * U) {
        bf16x8 bw[U][R], av[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(c0 + 256 * u, nch - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) bw[u][r] = load8(brow[r] + 8 * c);
#pragma unroll
            for (int m = 0; m < MT; ++m) av[u][m] = load8(arow[m] + 8 * c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + 256 * u < nch) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const bf16x2 x = {bw[u][r][2 * j], bw[u][r][2 * j + 1]};
                            const bf16x2 y = {av[u][m][2 * j], av[u][m][2 * j + 1]};
                            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc[r][m], false);
                        }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) part[tid][r * MT + m] = acc[r][m];
    __syncthreads();
    {
        // thread t adds sum v = t % NV of the NV threads of slice t / NV, in order
        const int v = tid % NV, sl = tid / NV;
        float x = 0.0f;
#pragma unroll 8
        for (int j = 0; j < NV; ++j) x += part[NV * sl + j][v];
        slice[sl][v] = x;
    }
    __syncthreads();
    if (tid < NV) {
        float x = 0.0f;
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) x += slice[sl][tid];
        const int r = tid / MT, m = tid % MT;
        if (m < g.M && n0 + r < g.N) enc_store(g, m, n0 + r, x);
    }
}

// The 64 lanes' sums of v[0 .. NV-1] (NV a power of two, at most 64): exchanges
// that halve the values a lane carries over lane distances 32, 16, .., 64/NV,
// then plain exchanges over the distances left.  Lane l ends with the sum of
// value l / (64 / NV) over all 64 lanes, added in an order fixed by the lane
// pattern alone.
// 16 bytes at byte offset off of a buffer (zeros past its range).
__device__ __forceinline__ bf16x8 buffer_load8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int HALF, int OFF>
__device__ __forceinline__ void wave_halve(float* v, int lane) {
    const bool up = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const float keep = up ? v[i + HALF] : v[i];
        const float send = up ? v[i] : v[i + HALF];
        v[i] = keep + __shfl_xor(send, OFF);
    }
    if constexpr (HALF > 1) wave_halve<HALF / 2, OFF / 2>(v, lane);
}

template <int NV>
__device__ __forceinline__ float wave_sum_each(float (&v)[NV], int lane) {
    if constexpr (NV > 1) wave_halve<NV / 2, 32>(v, lane);
    float x = v[0];
#pragma unroll
    for (int off = 32 / NV; off >= 1; off /= 2) x += __shfl_xor(x, off);
    return x;
}

// ------------------------------------------------------ few tokens, streamed
// Up to MT token rows against weight rows that stream through the registers,
// each weight byte read once.  Workgroup i of G takes rows N i / G .. N (i+1) /
// G - 1, so every CU streams the same number of rows (the grid holds at least
// one workgroup per CU).  Its waves form NG row groups of WPG waves; group g
// takes the workgroup's rows g, g + NG, .. (RPT at most), and its threads the
// 8-element K chunks t, t + 64 WPG, .. (CPT at most).  A thread loads its
// chunks of the MT token rows once, then its chunks of every row (all RPT x
// CPT loads in flight), and accumulates RPT x MT fp32 sums with bf16 pair dot
// products (bf16 products are exact in fp32).  The sums meet across the
// group's lanes by wave_sum_each, then across its waves through LDS in wave
// order, so the result does not depend on scheduling.  Token rows past M and
// rows past the workgroup's range are computed on a clamped row and never
// stored.
template <int MT, int NG, int WPG, int CPT, int RPT>
__global__ __launch_bounds__(NG * WPG * kWave) void k_encode_stream(EncGemm g) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    constexpr int TG = WPG * kWave;              // threads of a row group
    constexpr int NV = RPT * MT;                 // sums per thread
    constexpr int LPV = kWave / NV;              // lanes that end with the same sum
    static_assert((NV & (NV - 1)) == 0 && NV <= kWave, "butterfly layout");
    __shared__ float red[NG][WPG][kWave];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / WPG, wv = wave - grp * WPG;
    const int t = wv * kWave + lane;
    const int r0 = (int)((int64_t)g.N * blockIdx.x / gridDim.x);
    const int r1 = (int)((int64_t)g.N * (blockIdx.x + 1) / gridDim.x);
    if (r1 <= r0) return;                        // no rows (the host keeps G <= N)
    // Buffer loads with the row's byte range: chunks past the row's end read
    // zeros, so the products below need no branch (a branch would let the
    // compiler sink the first weight load behind the others and wait for all).
    const int range = g.K * 2;
    bf16x8 av[CPT][MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(g.a + (int64_t)min(m, g.M - 1) * g.lda), (short)0, range, kBufferWord3);
#pragma unroll
        for (int j = 0; j < CPT; ++j) av[j][m] = buffer_load8(ar, 16 * (t + TG * j));
    }
    bf16x8 bw[RPT][CPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            (void*)enc_brow(g, min(r0 + grp + NG * r, r1 - 1)), (short)0, range, kBufferWord3);
#pragma unroll
        for (int j = 0; j < CPT; ++j) bw[r][j] = buffer_load8(br, 16 * (t + TG * j));
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first product
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int j = 0; j < CPT; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bf16x2 x = {bw[r][j][2 * p], bw[r][j][2 * p + 1]};
                    const bf16x2 y = {av[j][m][2 * p], av[j][m][2 * p + 1]};
                    acc[r * MT + m] = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc[r * MT + m], false);
                }
    float s = wave_sum_each<NV>(acc, lane);
    if constexpr (WPG > 1) {
        red[grp][wv][lane] = s;
        __syncthreads();
        if (wv != 0) return;
#pragma unroll
        for (int w = 1; w < WPG; ++w) s += red[grp][w][lane];
    }
    if (lane % LPV == 0) {
        const int i = lane / LPV, r = i / MT, m = i - r * MT;
        const int n = r0 + grp + NG * r;
        if (m < g.M && n < r1) enc_store(g, m, n, s);
    }
}

// ------------------------------------------------------------ many tokens
// Workgroup tile (64 WM) x (64 WN), four waves in a 2 x 2 grid, each owning a
// (32 WM) x (32 WN) block of 32x32x16 matrix-core tiles.  K advances BK at a
// time through a ring of NS LDS stages that buffer loads fill directly
// (`buffer_load ... lds`, no register staging): while stage kt is multiplied,
// stages kt+1 .. kt+NS-2 are in flight and kt+NS-1 is issued.  One LDS-only
// barrier per stage.  Each copy instruction writes 1 KiB of whole stage rows
// and picks per lane which logical slot to fetch, so that slot s of row r sits
// at s ^ swz(r) and the sixteen rows one fragment read touches at a time fall
// in sixteen distinct 4-bank groups (measured: no bank conflicts).  Every
// copy's buffer is settled before the loop, so the loop holds no branches
// (a branch per copy costs the compiler's precise load counting and a third
// of the speed).  Copies past the last stage use an empty range and read
// nothing.  Tiles are dealt to XCDs in contiguous ranges, token tiles fastest,
// so the workgroups of one XCD share their activation and weight rows in L2.
// Measured at 1024 tokens (7168 -> 1536 -> 64 x 128): 64-deep stages beat
// 32-deep ones; two stages and two workgroups per CU beat deeper rings with
// one workgroup per CU on 128 x 128 tiles.
template <int SLOTS>
__device__ __forceinline__ int enc_swz(int row) {
    return (row >> (SLOTS == 8 ? 1 : 2)) & (SLOTS - 1);
}

template <int WM, int WN, int NS, int BK>
__global__ __launch_bounds__(256) void k_encode_tiled(EncGemm g, int tiles_m, int tiles_n) {
    constexpr int BM = 64 * WM, BN = 64 * WN;
    constexpr int SLOTS = BK / 8;                  // 16-byte slots per stage row
    constexpr int RPI = 64 / SLOTS;                // stage rows per copy instruction
    constexpr int AL = BM / (4 * RPI), BL = BN / (4 * RPI);   // copies per wave per stage
    static_assert(BK == 32 || BK == 64, "stage depth");
    static_assert(AL >= 1 && BL >= 1, "tile too small for the copy layout");
    static_assert((NS - 2) * (AL + BL) < 64 && NS >= 2, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) bf16 ring[NS][(BM + BN) * BK];

    const int n_tiles = tiles_m * tiles_n;
    const int per_xcd = (n_tiles + 7) / 8;
    const int slot = blockIdx.x >> 3;
    const int tile = (blockIdx.x & 7) * per_xcd + slot;
    if (slot >= per_xcd || tile >= n_tiles) return;
    const int m0 = (tile % tiles_m) * BM, n0 = (tile / tiles_m) * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave & 1) * 32 * WM, wn = (wave >> 1) * 32 * WN;
    const int nk = g.K / BK;

    // Wave w copies stage rows RPI (AL w + i) .. of A (i < AL) and RPI (BL w + j)
    // .. of B (j < BL), one instruction each.  Per lane: the row's byte offset
    // (clamped rows re-read the last one) at the logical slot it fetches.  Per
    // B instruction: its buffer (weight rows below nsplit, or from nsplit; the
    // first row decides, as nsplit is a multiple of RPI) and byte range, set
    // once here so that the copies themselves hold no branches.
    const int range_a = (int)min((int64_t)g.M * g.lda * 2, (int64_t)0x7fffffff);
    uint32_t aoff[AL], boff[BL];
    const bf16* bbase[BL];
    int brange[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = RPI * (AL * wave + i) + lane / SLOTS;
        const int m = min(m0 + r, g.M - 1);
        aoff[i] = (uint32_t)(((int64_t)m * g.lda + 8 * ((lane % SLOTS) ^ enc_swz<SLOTS>(r))) * 2);
    }
#pragma unroll
    for (int j = 0; j < BL; ++j) {
        const int r8 = RPI * (BL * wave + j);
        const int r = r8 + lane / SLOTS;
        const bool hi = min(n0 + r8, g.N - 1) >= g.nsplit;
        const int n = min(n0 + r, g.N - 1) - (hi ? g.nsplit : 0);
        boff[j] = (uint32_t)(((int64_t)n * g.K + 8 * ((lane % SLOTS) ^ enc_swz<SLOTS>(BM + r))) * 2);
        bbase[j] = hi ? g.b1 : g.b0;
        brange[j] = (int)min((int64_t)(hi ? g.N - g.nsplit : g.nsplit) * g.K * 2,
                             (int64_t)0x7fffffff);
    }
    auto issue = [&](int kt) {
        const bool live = kt < nk;
        const int soff = live ? kt * BK * 2 : 0;
        bf16* st = ring[kt % NS];
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)g.a, (short)0, live ? range_a : 0, kBufferWord3);
            // read into a scalar first: passed as an array element, the host pass
            // drops the kernel's launch stub
            const uint32_t vo = aoff[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(st + RPI * (AL * wave + i) * BK),
                16, vo, soff, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < BL; ++j) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)bbase[j], (short)0, live ? brange[j] : 0, kBufferWord3);
            const uint32_t vo = boff[j];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs,
                (__attribute__((address_space(3))) void*)(st + (BM + RPI * (BL * wave + j)) * BK),
                16, vo, soff, 0, 0);
        }
    };

    f32x16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int fr = lane & 31, fk = lane >> 5;      // fragment row; which half of 16 k
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt<(NS - 2) * (AL + BL)>();        // this wave's copies of stage kt landed
        lds_barrier();                             // everyone's, and stage kt-1 is read
        issue(kt + NS - 1);
        const bf16* st = ring[kt % NS];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[WM], bfr[WN];
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const int r = wm + 32 * i + fr;
                af[i] = *reinterpret_cast<const bf16x8*>(st + r * BK +
                                                         8 * ((2 * ks + fk) ^ enc_swz<SLOTS>(r)));
            }
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const int r = BM + wn + 32 * j + fr;
                bfr[j] = *reinterpret_cast<const bf16x8*>(st + r * BK +
                                                          8 * ((2 * ks + fk) ^ enc_swz<SLOTS>(r)));
            }
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    }
    wait_vmcnt<0>();                               // no copy lands after the workgroup ends

    // lane l holds rows 8(v/4) + 4(l/32) + v%4, column l%32 of each 32x32 block
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int n = n0 + wn + 32 * j + (lane & 31);
                if (m < g.M && n < g.N) enc_store(g, m, n, acc[i][j][v]);
            }
}

constexpr int kEncSkinnyMaxM = 32;   // token rows the few-token kernel keeps in registers

#ifndef LSA_ENC_STREAM
#define LSA_ENC_STREAM 1
#endif

// One token row (batch-1 decode), if K is in the streamed kernel's range: up
// to 256 chunks per row on single-wave row groups of 4 rows (8 groups per
// workgroup), up to 1024 chunks on one 8-wave group of 8 rows; one workgroup
// per CU, or more when the rows would not fit.  15.1 -> 13.4 us per call at
// 7168 -> 1536 -> 64 x 128 in one A/B.  With 4 or 8 token rows the products
// (4 x 4 dot products per chunk per row) finish after the last rows land and
// the call was slower (15.8 -> 17.8 and 17.4 -> 18.0 us), as was a matrix-core
// form with the token rows staged in LDS (17.5 us at 8 rows, 14.6 at one):
// every workgroup then reads the whole token block, 29 MB over the chip at 8
// rows against 23 MB of weights.
static bool launch_stream(const EncGemm& g, int num_cus, hipStream_t st) {
    const int nch = g.K / 8;
    if (nch <= 4 * kWave) {
        constexpr int NG = 8, RPT = 4;
        const dim3 grid((unsigned)std::min<int64_t>(
            g.N, std::max<int64_t>(num_cus, ceil_div(g.N, NG * RPT))));
        const dim3 block(NG * kWave);
        switch ((nch + kWave - 1) / kWave) {
            case 1: hipLaunchKernelGGL((k_encode_stream<1, NG, 1, 1, RPT>), grid, block, 0, st, g); break;
            case 2: hipLaunchKernelGGL((k_encode_stream<1, NG, 1, 2, RPT>), grid, block, 0, st, g); break;
            case 3: hipLaunchKernelGGL((k_encode_stream<1, NG, 1, 3, RPT>), grid, block, 0, st, g); break;
            default: hipLaunchKernelGGL((k_encode_stream<1, NG, 1, 4, RPT>), grid, block, 0, st, g); break;
        }
        return true;
    }
    if (nch <= 2 * 8 * kWave) {
        constexpr int WPG = 8, RPT = 8;
        const dim3 grid((unsigned)std::min<int64_t>(g.N, std::max<int64_t>(num_cus, ceil_div(g.N, RPT))));
        hipLaunchKernelGGL((k_encode_stream<1, 1, WPG, 2, RPT>), grid, dim3(WPG * kWave), 0, st, g);
        return true;
    }
    return false;
}

constexpr int kEncRowsMaxM = 8;      // token rows the vector kernel takes
constexpr int kEncRows = 4;          // weight rows per workgroup of the vector kernel
constexpr int kEncRowsMinK = 4096;   // depth from which it beats the 16-row kernel

static int launch_product(const EncGemm& g, int num_cus, hipStream_t st) {
    if (LSA_ENC_STREAM && g.M == 1 && launch_stream(g, num_cus, st)) return launch_status("query_encode");
    // Up to 8 tokens and a long K (the down product, 7168 deep): 4-row
    // workgroups, 21.8 -> 17.0 us per 8-token call at 7168 -> 1536 -> 64 x 128
    // in one A/B (the up product, 1536 deep, stays on the 16-row kernel: its
    // 8192 rows already give 512 workgroups).
    if (g.M <= kEncRowsMaxM && g.K >= kEncRowsMinK) {
        const dim3 grid((unsigned)ceil_div(g.N, kEncRows));
        hipLaunchKernelGGL((k_encode_rows<kEncRows, kEncRowsMaxM, 1>), grid, dim3(256), 0, st, g);
        return launch_status("query_encode");
    }
    if (g.M <= kEncSkinnyMaxM) {
        const dim3 grid((unsigned)ceil_div(g.N, 16));
        // long K: 16 waves share it, so more weight loads are in flight per row block
        if (g.M <= 16) {
            if (g.K >= 4096)
                hipLaunchKernelGGL((k_encode_skinny<1, 16, 8>), grid, dim3(16 * kWave), 0, st, g);
            else
                hipLaunchKernelGGL((k_encode_skinny<1, 8, 8>), grid, dim3(8 * kWave), 0, st, g);
        } else {
            if (g.K >= 4096)
                hipLaunchKernelGGL((k_encode_skinny<2, 16, 8>), grid, dim3(16 * kWave), 0, st, g);
            else
                hipLaunchKernelGGL((k_encode_skinny<2, 8, 8>), grid, dim3(8 * kWave), 0, st, g);
        }
        return launch_status("query_encode");
    }
    // the largest tile whose count still fills the CUs: 128x128, 128x64, else 64x64
    const int tm2 = (int)ceil_div(g.M, 128), tn2 = (int)ceil_div(g.N, 128);
    const int tn1 = (int)ceil_div(g.N, 64), tm1 = (int)ceil_div(g.M, 64);
    if ((int64_t)tm2 * tn2 >= num_cus) {
        const unsigned grid = (unsigned)(8 * ceil_div((int64_t)tm2 * tn2, 8));
        hipLaunchKernelGGL((k_encode_tiled<2, 2, LSA_ENC_NS22, LSA_ENC_BK22>), dim3(grid), dim3(256), 0, st, g,
                           tm2, tn2);
    } else if ((int64_t)tm2 * tn1 * 100 >= (int64_t)LSA_ENC_FILL21 * num_cus) {
        const unsigned grid = (unsigned)(8 * ceil_div((int64_t)tm2 * tn1, 8));
        hipLaunchKernelGGL((k_encode_tiled<2, 1, LSA_ENC_NS21, LSA_ENC_BK21>), dim3(grid), dim3(256), 0, st, g,
                           tm2, tn1);
    } else {
        const unsigned grid = (unsigned)(8 * ceil_div((int64_t)tm1 * tn1, 8));
        hipLaunchKernelGGL((k_encode_tiled<1, 1, LSA_ENC_NS11, LSA_ENC_BK11>), dim3(grid), dim3(256), 0, st, g,
                           tm1, tn1);
    }
    return launch_status("query_encode");
}

}  // namespace lsa

using namespace lsa;

extern "C" int lsa_query_encode(const void* h, int M, int d_model, int rank, int H, int D,
                                const void* w_down, const void* w_up, const void* w_gate,
                                void* c_buf, void* q_out, float* w_out, void* stream) {
    clear_error();
    if (!h || !w_down || !w_up || !w_gate || !c_buf || !q_out || !w_out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_query_encode: a required pointer is NULL");
    if (M <= 0 || d_model <= 0 || rank <= 0 || H <= 0 || D <= 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_query_encode: M=%d d_model=%d rank=%d H=%d D=%d", M,
                    d_model, rank, H, D);
    if (!aligned16(h) || !aligned16(w_down) || !aligned16(w_up) || !aligned16(w_gate) ||
        !aligned16(c_buf))
        return fail(LSA_ERR_INVALID_ARG,
                    "lsa_query_encode: h, the weights and c_buf must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(q_out) & 1u) || (reinterpret_cast<uintptr_t>(w_out) & 3u))
        return fail(LSA_ERR_INVALID_ARG, "lsa_query_encode: q_out or w_out misaligned");
    if (d_model % 64 != 0 || rank % 64 != 0)
        return fail(LSA_ERR_UNSUPPORTED,
                    "lsa_query_encode: d_model=%d and rank=%d must be multiples of 64", d_model,
                    rank);
    if ((int64_t)H * D > (1 << 20) || (int64_t)rank + H > (1 << 20) || d_model > (1 << 20))
        return fail(LSA_ERR_UNSUPPORTED, "lsa_query_encode: projection too large");
    // the tiled product addresses every operand with 32-bit byte offsets
    const int64_t lim = 0x7fffffff;
    if ((int64_t)M * d_model * 2 > lim || (int64_t)M * rank * 2 > lim ||
        (int64_t)rank * d_model * 2 > lim || (int64_t)H * D * rank * 2 > lim ||
        (int64_t)H * d_model * 2 > lim)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_query_encode: an operand exceeds 2 GiB");
    int num_cus = 0;
    int rc = check_device(&num_cus);
    if (rc != LSA_OK) return rc;
    const hipStream_t st = (hipStream_t)stream;
    const EncGemm down{(const bf16*)h,   d_model,         (const bf16*)w_down, (const bf16*)w_gate,
                       M,                rank + H,        d_model,             rank,
                       (bf16*)c_buf,     rank,            w_out,               H};
    const EncGemm up{(const bf16*)c_buf, rank,  (const bf16*)w_up, (const bf16*)w_up,
                     M,                  H * D, rank,              H * D,
                     (bf16*)q_out,       H * D, nullptr,           0};
    if ((rc = launch_product(down, num_cus, st)) != LSA_OK) return rc;
    return launch_product(up, num_cus, st);
}
