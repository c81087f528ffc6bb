// attend.hip -- lsa_sparse_attend: core attention over the chosen entries plus every HCA entry.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1: the heavily compressed
// (HCA, 128:1) entries are all retained, and the final core attention runs
// over the top-k entries chosen inside the fetched subset.  Each compressed
// entry carries one latent row that serves as key and value for all query
// heads (multi-query form over a shared latent).
//
// Matrix-core kernel (bf16, Dl in {128, 256, 512}).  Every query head of every
// position of sequence b attends to the same rows, so the (position, head)
// pairs of b are flattened into M = T * Hq query rows.  A workgroup of eight
// waves takes one (b, group of 64 query rows, row split) and walks its rows in
// chunks of 32, each row passing through LDS once:
//   1. the four score waves copy the chunk's rows from HBM straight into an
//      LDS ring slot (buffer loads into LDS, NB-1 chunks ahead);
//   2. S^T = K Q^T: score wave w owns query rows 16w.. against all 32 chunk
//      rows over the full latent depth, Q held in registers, and runs the
//      online softmax of its rows alone (base 2, running max moved lazily);
//      P (bf16) goes to LDS;
//   3. O[:, dims_u] += P C[:, dims_u]: value wave u owns Dl/4 latent dims of
//      all 64 query rows; C^T operands come from transposing LDS reads.
// Steps 2 and 3 of consecutive chunks overlap (a score wave and a value wave
// share each SIMD), and the copies of step 1 are spread among the products of
// step 2.  Rows are split across workgroups when B * T * Hq is
// small; a combine kernel merges the splits by their log-sum-exp.
#include "common.hpp"

namespace lsa {

// Workgroups the split heuristic aims for (one per CU; a compile-time knob).
#ifndef LSA_ATT_WG_TARGET
#define LSA_ATT_WG_TARGET 256
#endif
constexpr int kAttWGTarget = LSA_ATT_WG_TARGET;
#ifndef LSA_ATT_TOP_ROWS
#define LSA_ATT_TOP_ROWS 0
#endif
constexpr int kAttTopRows = LSA_ATT_TOP_ROWS;   // rows per top-k split; 0 = as the HCA splits
// cache-policy operand of the row copies when every row is read by one workgroup
// only (one query group): nontemporal, as the rows are streamed once
constexpr int kAttNonTemporal = 2;
constexpr int kChunk = 32;          // attended rows per step
constexpr int kMaxSplitRows = 2048; // most rows one split may take (64 chunks: one per lane)
constexpr int64_t kMaxAttendRows = (int64_t)1 << 20;   // per sequence: at most 512 splits
constexpr int kMQ = 64;             // query rows per workgroup
constexpr int kAttRing = 4;         // ring slots of kChunk rows
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // keep the running max unless it grows by > 2^8

// Row pointer of attended row j of sequence b (nullptr past the end).
template <typename E>
__device__ __forceinline__ const E* att_row(int j, int nt, int n, const E* latent, int64_t lrs,
                                            const int32_t* idx, const E* hca, int64_t hrs,
                                            int Dl) {
    if (j < nt) return latent + (lrs + idx[j]) * Dl;
    if (j < n) return hca + (hrs + (j - nt)) * Dl;
    return nullptr;
}

// Work item = (b, t, head group, split).  Items of one (b, t) are laid out
// contiguously and dealt to XCDs in contiguous ranges: workgroup L runs on XCD
// L % 8 (round-robin dispatch), so the head groups that read the same rows and
// the splits whose partials are merged share one L2.
__device__ __forceinline__ int xcd_item(int n_items) {
    const int per_xcd = (n_items + 7) / 8;
    const int slot = blockIdx.x >> 3;
    const int item = (blockIdx.x & 7) * per_xcd + slot;
    return (slot < per_xcd && item < n_items) ? item : -1;
}

// 16-byte slot swizzle of a staged latent row (a multiple of 16 slots, so every
// row starts on the same bank): physical slot p of row r holds logical slot
// p ^ slot_swz(r), slot_swz(r) = 2 (r mod 4) + 8 ((r / 8) mod 2).  The LDS
// bank-conflict counters, measured over candidate lane patterns, fit this
// model of gfx950: 64 four-byte banks; a 16-byte read serves its lanes in four
// groups of 16, lane 16 g + n (n < 16) in group (g1, g0 ^ n2 ^ n3), where x_i
// is bit i of x; a transposing 8-byte read serves 32 consecutive lanes at a
// time.  Under it both reads of a staged chunk are conflict-free: the Q K^T
// operand (lane 16 g + n reads row n, logical slot 4 k + g: the slots a group
// touches are a bijection of n), and the transposing P C reads (lanes 4 j ..
// 4 j + 3 of each 16 read rows 8 g + j, + 4 for the upper half: the bank units
// of 32 consecutive lanes are a bijection of (n, g0)).  The swizzle depends on
// bits 0, 1 and 3 of r only, so rows r and r + 16 share it.
__device__ __forceinline__ int slot_swz(int r) {
    return 2 * (r & 3) + (r & 8);
}

// Reductions over RG adjacent lanes (RG in {4, 8, 16}) with DPP lane moves.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int RG>
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));                        // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));                        // quad_perm [2,3,0,1]
    if constexpr (RG >= 8) x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
    if constexpr (RG >= 16) x = fmaxf(x, dpp_mov<0x140>(x)); // row_mirror
    return x;
}
template <int RG>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    if constexpr (RG >= 8) x += dpp_mov<0x141>(x);
    if constexpr (RG >= 16) x += dpp_mov<0x140>(x);
    return x;
}

// Parameter order: what the first loads need comes first (14 dwords: the work
// item, the Q and index addresses, the count pointers), so a build that
// preloads kernel arguments into scalar registers issues them at launch.
//
// Eight waves.  Waves 0..3 ("score waves") stage the rows and compute
// S^T = K Q^T: score wave w owns query rows 16w .. 16w+15 against every row of
// a chunk, with its Q fragments in registers, so its rows' online softmax
// (running max, rescale decision, row sums) needs no other wave.  It publishes
// P (bf16) and, when its running max moved, the rescale factors.  Waves 4..7
// ("value waves") compute O += P C: value wave 4+u owns latent dims
// [u Dl/4, (u+1) Dl/4) of all 64 query rows.  Score wave w and value wave w+4
// share a SIMD, so one's matrix products overlap the other's LDS traffic.
template <int Dl, int NB, bool NT>
__global__ __launch_bounds__(512, 1) void k_attend_mfma(
    int n_items, int QG, int nsplit, int split0, int nloc, int nts, int rps_top,
    int rows_per_split, int M, int k, const int32_t* __restrict__ topk_idx,
    const bf16* __restrict__ qa,
    const int32_t* __restrict__ topk_count, const int32_t* __restrict__ hca_count,
    const int64_t* __restrict__ latent_row_start, const int64_t* __restrict__ hca_row_start,
    int64_t max_hca, const bf16* __restrict__ latent, const bf16* __restrict__ hca,
    float scale_log2, bf16* __restrict__ out, float* __restrict__ lse, bf16* __restrict__ part_o,
    float* __restrict__ part_lse) {
    constexpr int NS = 4;                       // score waves (0..3); value waves are 4..7
    constexpr int SL = Dl / 8;                  // 16-byte slots per latent row
    constexpr int RPI = 64 / SL;                // rows per direct-to-LDS instruction
    constexpr int IPW = kChunk / (RPI * NS);    // such row groups per score wave per chunk
    constexpr int CPW = kChunk / NS;            // buffer loads per score wave per chunk
    constexpr int KDT = Dl / 32;                // k-steps of one S^T tile
    constexpr int DPW = Dl / 4;                 // latent dims per value wave
    constexpr int NDT = DPW / 16;               // 16-wide dim tiles of P C
    constexpr int QT = kMQ / 16;                // 16-row query tiles
    constexpr int PROW = 40;                    // bf16 per query row of P (32 + padding)
    static_assert(SL >= 16 && IPW >= 1 && NB >= 3 && NB <= 4 && QT == NS, "tiling");
    static_assert(kMQ * Dl <= NB * kChunk * Dl, "output staging fits the ring");

    // One LDS object holds every buffer: the compiler then leaves the ordering of
    // the direct-to-LDS copies and the LDS reads to the explicit counted waits
    // and barriers below instead of draining all copies before each LDS read.
    constexpr int OFF_PBUF = NB * kChunk * Dl * 2;          // ring: NB slots of kChunk rows
    constexpr int OFF_ABUF = OFF_PBUF + 2 * kMQ * PROW * 2; // P (bf16), two buffers
    constexpr int OFF_FLAG = OFF_ABUF + 2 * kMQ * 4;        // rescale factors, two buffers
    constexpr int OFF_ML = OFF_FLAG + 2 * 4 * 4;            // per-query-tile rescale flags, two sets
    constexpr int LDS_BYTES = OFF_ML + 2 * kMQ * 4;         // final (m, l)
    static_assert(OFF_FLAG % 16 == 0, "flag sets are read as one 16-byte word");
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    bf16* const ring0 = reinterpret_cast<bf16*>(lds);
    bf16* const pbuf = reinterpret_cast<bf16*>(lds + OFF_PBUF);
    float* const abuf = reinterpret_cast<float*>(lds + OFF_ABUF);
    int* const flags = reinterpret_cast<int*>(lds + OFF_FLAG);
    float (*const mlbuf)[kMQ] = reinterpret_cast<float (*)[kMQ]>(lds + OFF_ML);

    // Work item and per-sequence values.  Every load here is unconditional (a
    // stand-in pointer replaces a missing HCA pool), so they issue together in
    // one round trip after the kernel arguments instead of one after another.
    // A workgroup past the last item (the grid is a multiple of 8) runs item 0
    // with no rows and stores nothing.
    const int item_raw = xcd_item(n_items);
    const bool active = item_raw >= 0;
    const int item = active ? item_raw : 0;
    const int tq = item / QG;
    const int qg = item - tq * QG;
    const int b = tq / nloc;                    // this launch covers splits split0 .. +nloc-1
    const int split = split0 + (tq - b * nloc);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    const int n16 = lane & 15;
    const int g = lane >> 4;
    const bool vwave = wave >= NS;
    const int u = wave - NS;                    // value wave: dims DPW*u ..

    const int32_t* idx = topk_idx + (int64_t)b * k;
    const int64_t qrow0 = (int64_t)b * M + (int64_t)qg * kMQ;   // first query row of the group
    const int mq = min(kMQ, M - qg * kMQ);                        // valid query rows

    // The per-sequence counts and row starts (scalar loads; they overlap the
    // score waves' first vector loads below).
    const int topk_cnt = topk_count[b];
    const int hca_cnt = hca_count[b];
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca_row_start[b];
    // Rows of the sequence: its top-k rows, then its HCA rows.  With nts = 0 the
    // splits take consecutive runs of rows_per_split of that list.  With nts > 0
    // splits 0 .. nts-1 take runs of rps_top top-k rows and the rest runs of
    // rows_per_split HCA rows, so a launch of HCA splits only never reads the
    // top-k list or its counts (it runs with ntop = 0: every row is an HCA row).
    const bool hsplit = nts > 0 && split >= nts;
    const int ntop = hsplit ? 0 : min(topk_cnt, k);
    const int nh = (int)min((int64_t)hca_cnt, max_hca);   // max_hca = 0 without a pool
    const int n = ntop + nh;
    const int rs = nts == 0 ? split * rows_per_split
                 : hsplit   ? (split - nts) * rows_per_split
                            : split * rps_top;
    const int re = nts > 0 && !hsplit ? min(ntop, rs + rps_top) : min(n, rs + rows_per_split);
    const int nchunks = (active && re > rs) ? (re - rs + kChunk - 1) / kChunk : 0;

    // Score wave w stages rows 8w .. 8w+7 of every chunk: lane c holds the 64-bit
    // addresses of those rows of chunk c (a split has at most 64 chunks), so a
    // copy costs two lane reads and no branches.
    uint32_t raddr_lo[8], raddr_hi[8];
    // score wave w's Q fragments and whether its query rows exist
    const bool q_ok = 16 * wave + n16 < mq;
    bf16x8 qf[KDT];

    // Chunk c -> ring slot c % NB.  Score wave w moves chunk rows 8w .. 8w+7, one
    // row per buffer load with the row's address as the (wave-uniform) buffer
    // base; when a row is shorter than the wave (Dl < 512), only the lanes that
    // cover it are active.  Lane L of an instruction fills LDS 16 bytes at
    // (instruction base) + 16 L, i.e. physical slot L % SL of row r, with logical
    // slot (L % SL) ^ swz(r).  Buffer (not flat) loads keep the LDS reads of
    // these waves on partial lgkmcnt waits: the compiler treats a flat load
    // into LDS as an unordered LDS access and would drain every LDS read.
    // Chunks past the split's last are issued too, with an empty buffer range
    // (the hardware's range check then reads no memory), so every step issues
    // the same number of copies and the waits are branch-free.
    // Copy m (0 <= m < CPW, a compile-time value) of chunk c.
    auto issue_copy = [&](int c, int m) {
        bf16* slot = ring0 + (c % NB) * (kChunk * Dl);
        const int range = c < nchunks ? Dl * 2 : 0;
        const int cl = c & 63;
        const int i = m / RPI, s2 = m % RPI;
        const int sub = lane / SL;                         // row of this lane in the instruction
        const int rbase = 8 * wave + RPI * i;
        const uint32_t lo = __builtin_amdgcn_readlane(raddr_lo[m], cl);
        const uint32_t hi = __builtin_amdgcn_readlane(raddr_hi[m], cl);
        void* row = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(row, (short)0, range, kBufferWord3);
        if (RPI == 1 || sub == s2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(slot + rbase * Dl), 16,
                (uint32_t)(16 * ((lane % SL) ^ slot_swz(rbase + s2))), 0, 0,
                NT ? kAttNonTemporal : 0);
    };
    auto issue_chunk = [&](int c) {
#pragma unroll
        for (int m = 0; m < CPW; ++m) issue_copy(c, m);
    };

    // Score wave state: running max (base 2) of query row 16w + n16 (the same in
    // the four lanes of that row), and this lane's share of its row sum.
    float m_ref = -INFINITY;
    float l_part = 0.0f;

    // Score wave w, chunk c: S^T tiles (chunk rows 16rt .., query rows 16w ..)
    // over the full latent depth, then P against the running max into
    // pbuf[c & 1], and this wave's rescale flag into flags[c & 1][w].  The copies
    // of chunk c + NB - 2 are issued among the products, one every NSTEP / CPW
    // steps: issued together after a barrier, the four score waves' copies
    // queue at the CU's address unit for about a fifth of a chunk's time.
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    auto score = [&](int c) {
        const int r0 = rs + c * kChunk;
        const bf16* sl = ring0 + (c % NB) * (kChunk * Dl);
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        {
            // A operand: chunk row 16rt + n16, dims 32kk + 8g .. +7.  Logical slot
            // 4kk + g sits at physical ((4(kk & 3) + g) ^ sw) + 16(kk >> 2); the
            // swizzle depends on bits 0, 1 and 3 of the row only, so rows r and r+16
            // share it, and four base addresses plus immediate offsets cover
            // every step.
            const int sw = slot_swz(n16);
            const bf16* kp[4];
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) kp[b4] = sl + n16 * Dl + 8 * ((4 * b4 + g) ^ sw);
            // Steps alternate between the two row tiles and between two partial
            // accumulators per tile, so four independent product chains are in
            // flight; reads run KW steps ahead of the products.
            constexpr int NSTEP = 2 * KDT;
            constexpr int KW = NSTEP < 16 ? NSTEP : 16;   // reads in flight
            auto kaddr = [&](int i) {
                const int rt = i & 1, kk = i >> 1;
                return reinterpret_cast<const bf16x8*>(kp[kk & 3] + rt * 16 * Dl + 128 * (kk >> 2));
            };
            f32x4 acc4[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                             f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            bf16x8 kb[KW];
#pragma unroll
            for (int i = 0; i < KW; ++i) kb[i] = *kaddr(i);
            constexpr int CSTEP = NSTEP / CPW;              // product steps per copy
            static_assert(CSTEP * CPW == NSTEP, "copies spread over the products");
#pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                acc4[i & 3] = mfma16(kb[i % KW], qf[i >> 1], acc4[i & 3]);
                if (i + KW < NSTEP) kb[i % KW] = *kaddr(i + KW);
                if (i % CSTEP == CSTEP - 1) issue_copy(c + NB - 2, i / CSTEP);
            }
            sacc[0] = acc4[0] + acc4[2];
            sacc[1] = acc4[1] + acc4[3];
        }
        // this lane holds query row 16w + n16 against chunk rows 16rt + 4g + v.
        // A full chunk (every chunk but a split's last) needs no row mask, and its
        // logits are finite, so neither the mask nor the -inf test below runs.
        const bool full = r0 + kChunk <= re;
        float x[2][4];
        bool over = false;
        float cmax;                                 // this lane's largest logit of the chunk
        if (full) {
            // Rounding is monotone, so the largest scaled logit is the scaled
            // largest product (smallest, for a negative scale): one product
            // instead of eight before the compare.
            float hi;
            if (scale_log2 >= 0.0f)
                hi = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                           fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
            else
                hi = fminf(fminf(fminf(sacc[0][0], sacc[0][1]), fminf(sacc[0][2], sacc[0][3])),
                           fminf(fminf(sacc[1][0], sacc[1][1]), fminf(sacc[1][2], sacc[1][3])));
            cmax = hi * scale_log2;
            over = cmax > m_ref + kRescaleSlack;
        } else {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool valid = r0 + 16 * rt + 4 * g + v < re;
                    x[rt][v] = valid ? sacc[rt][v] * scale_log2 : -INFINITY;
                    over = over || x[rt][v] > m_ref + kRescaleSlack;
                }
            cmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        }
        // Lazy rescale: the running max stands unless some logit of the chunk
        // exceeds it by more than kRescaleSlack (always on the first chunk, as
        // -inf + slack = -inf), so p <= 2^kRescaleSlack.  Rare: the row maxima are
        // met across the four lanes of each row, and the factors published.
        int grew = 0;
        if (__ballot(over) != 0) {
            float cm = cmax;
            cm = fmaxf(cm, __shfl_xor(cm, 16));
            cm = fmaxf(cm, __shfl_xor(cm, 32));
            const bool grow = cm > m_ref + kRescaleSlack;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - cm) : 1.0f;
            m_ref = grow ? cm : m_ref;
            l_part *= alpha;
            if (g == 0) abuf[(c & 1) * kMQ + 16 * wave + n16] = alpha;
            grew = __ballot(grow) != 0 ? 1 : 0;
        }
        bf16* pb = pbuf + (c & 1) * (kMQ * PROW) + (16 * wave + n16) * PROW + 4 * g;
        if (full) {
            // p = 2^(scale_log2 s - m_ref) with one rounding, converted two at a
            // time; the row sum adds the rounded pairs (bf16 times 1 is exact)
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x2 e01, e23;
                e01[0] = __builtin_amdgcn_exp2f(fmaf(sacc[rt][0], scale_log2, -m_ref));
                e01[1] = __builtin_amdgcn_exp2f(fmaf(sacc[rt][1], scale_log2, -m_ref));
                e23[0] = __builtin_amdgcn_exp2f(fmaf(sacc[rt][2], scale_log2, -m_ref));
                e23[1] = __builtin_amdgcn_exp2f(fmaf(sacc[rt][3], scale_log2, -m_ref));
                const bf16x2 p01 = __builtin_convertvector(e01, bf16x2);
                const bf16x2 p23 = __builtin_convertvector(e23, bf16x2);
                l_part = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, l_part, false);
                l_part = __builtin_amdgcn_fdot2_f32_bf16(p23, ones, l_part, false);
                const bf16x4 p4 = {p01[0], p01[1], p23[0], p23[1]};
                *reinterpret_cast<bf16x4*>(pb + 16 * rt) = p4;
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                bf16x4 p4;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    // after the rescale step m_ref is finite whenever the chunk has a row
                    const bf16 p = (bf16)(x[rt][v] != -INFINITY
                                              ? __builtin_amdgcn_exp2f(x[rt][v] - m_ref) : 0.0f);
                    p4[v] = p;
                    l_part += (float)p;             // the sums use the rounded P that P C uses
                }
                *reinterpret_cast<bf16x4*>(pb + 16 * rt) = p4;
            }
        }
        if (lane == 0) flags[4 * (c & 1) + wave] = grew;
    };

    // Value wave u, chunk c (after the barrier that published P(c)): rescale the
    // O rows whose running max moved, then O[:, dims_u] += P C[:, dims_u].
    f32x4 o[QT][NDT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) o[qt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto pv = [&](int c) {
        const bf16* sl = ring0 + (c % NB) * (kChunk * Dl);
        const bf16* pb = pbuf + (c & 1) * (kMQ * PROW);
        // A: query row 16qt + n16, chunk rows 8g .. 8g+7
        bf16x8 pa[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            pa[qt] = *reinterpret_cast<const bf16x8*>(&pb[(16 * qt + n16) * PROW + 8 * g]);
        // B from transposing reads: in each 16-lane group, lanes 4j..4j+3 point at
        // chunk row 8g + j (+4 for the upper half), 4 dims each, and lane i
        // receives dim i of those 4 rows.
        const int trow0 = 8 * g + (n16 >> 2);
        const int trow1 = trow0 + 4;
        const int sw0 = slot_swz(trow0), sw1 = slot_swz(trow1);
        const int q4 = n16 & 3;
        const int off = 4 * (q4 & 1);
        bf16x4 lo[NDT], hi[NDT];
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
            const int ls = (DPW / 8) * u + 2 * nt + (q4 >> 1);   // logical 16-byte slot
            lo[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(sl + trow0 * Dl + 8 * (ls ^ sw0) + off));
            hi[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(sl + trow1 * Dl + 8 * (ls ^ sw1) + off));
        }
        const int4 fl = *reinterpret_cast<const int4*>(flags + 4 * (c & 1));
        const int fl_any = __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w);
        if (fl_any) {
            const int fq[4] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                if (__builtin_amdgcn_readfirstlane(fq[qt])) {
                    const f32x4 al =
                        *reinterpret_cast<const f32x4*>(&abuf[(c & 1) * kMQ + 16 * qt + 4 * g]);
#pragma unroll
                    for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) o[qt][nt][v] *= al[v];
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
            bf16x8 cb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cb[j] = lo[nt][j];
                cb[4 + j] = hi[nt][j];
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][nt] = mfma16(pa[qt], cb, o[qt][nt]);
        }
    };

    // Pipeline, one barrier per chunk (X_c).  Between X_c and X_{c+1} the value
    // waves run P C of chunk c while the score waves refill chunk c-1's slot with
    // chunk c+NB-1 and run S^T and P of chunk c+1.  Before X_c every score wave
    // has waited for its own copies of chunk c+1, so the barrier certifies the
    // whole chunk staged; P, the factors and the flags alternate between two
    // buffers, so the writes for chunk c+1 never meet a late reader of chunk c-1.
    if (!vwave) {
        // Every vector load of the score waves sits in this one straight-line
        // region, so the compiler's own waits track them exactly.  Indices first:
        // the loads are speculative (clamped into the index row, used only for
        // rows below the top-k count), so they do not wait for the counts.
        int ridx[8];
#pragma unroll
        for (int j8 = 0; j8 < 8; ++j8)
            ridx[j8] = idx[min(rs + kChunk * lane + 8 * wave + j8, k - 1)];
        const int first_idx = idx[min(rs, k - 1)];
        __builtin_amdgcn_sched_barrier(0);      // the index loads stay ahead of Q's
        // Q fragments (B operand of S^T = K Q^T): query row 16w + n16, dims
        // 32kk + 8g .. +7, in flight while the row addresses are formed.  Rows
        // past the group's end read its first row and are zeroed before use.
        {
            const bf16* qp = qa + (qrow0 + (q_ok ? 16 * wave + n16 : 0)) * Dl + 8 * g;
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) qf[kk] = load8(qp + 32 * kk);
        }
        __builtin_amdgcn_sched_barrier(0);      // ... and Q's ahead of the first wait
        {
            // Rows past the split end re-read the split's first row (finite data,
            // probability zero).  Both candidate addresses, then a select.
            const uint64_t lat = (uint64_t)latent, hc = (uint64_t)hca;
#pragma unroll
            for (int j8 = 0; j8 < 8; ++j8) {
                const int j0 = rs + kChunk * lane + 8 * wave + j8;
                const bool past = j0 >= re;
                const int j = past ? rs : j0;
                const int e = past ? first_idx : ridx[j8];
                const uint64_t al = lat + (uint64_t)(lrs + e) * (uint64_t)(Dl * 2);
                const uint64_t ah = hc + (uint64_t)(hrs + (j - ntop)) * (uint64_t)(Dl * 2);
                const bool top = j < ntop;
                raddr_lo[j8] = top ? (uint32_t)al : (uint32_t)ah;
                raddr_hi[j8] = top ? (uint32_t)(al >> 32) : (uint32_t)(ah >> 32);
            }
        }
        // From here on the score waves issue no vector memory operation but the
        // copies, so the counted waits below are exact.  The value
        // waves never issue a copy, so their transposing LDS reads never wait for
        // one.
        // chunks 0 .. NB-3 now; score(c) issues chunk c + NB - 2 (and where no
        // score runs, the chunk is issued on its own: every step issues CPW copies)
#pragma unroll
        for (int c = 0; c < NB - 2; ++c) issue_chunk(c);
        wait_vmcnt<(NB - 3) * CPW>();       // chunk 0 staged (and Q, which is older)
        lds_barrier();                                          // X_{-1}: chunk 0 staged
        if (!q_ok) {
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) qf[kk] = zero8();
        }
        if (nchunks > 0) score(0); else issue_chunk(NB - 2);
        for (int c = 0; c < nchunks; ++c) {
            wait_vmcnt<(NB - 3) * CPW>();   // chunk c+1 staged (chunks up to c+NB-2 issued)
            lds_barrier();                                      // X_c
            if (c + 1 < nchunks) score(c + 1); else issue_chunk(c + NB - 1);
        }
        wait_vmcnt<0>();                    // no copy lands after the loop
        // the row sum of query row 16w + n16 and its running max, for the value waves
        float l = l_part + __shfl_xor(l_part, 16);
        l += __shfl_xor(l, 32);
        if (g == 0) {
            mlbuf[0][16 * wave + n16] = m_ref;
            mlbuf[1][16 * wave + n16] = l;
        }
    } else {
        lds_barrier();                                          // X_{-1}
        for (int c = 0; c < nchunks; ++c) {
            lds_barrier();                                      // X_c
            pv(c);
        }
    }
    lds_barrier();                                              // (m, l) published

    if (vwave) {
        // normalise this lane's O rows 16qt + 4g + v
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&mlbuf[1][16 * qt + 4 * g]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float inv = l4[v] > 0.0f ? 1.0f / l4[v] : 0.0f;
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt) o[qt][nt][v] *= inv;
            }
        }
        if (nsplit > 1) {
            // split partial in fragment order [u][qt][nt][lane][v] (bf16), read back
            // in the same order by the combine: 8 bytes per lane, 512 per store
            bf16* dst = part_o + ((int64_t)(b * nsplit + split) * QG + qg) * (int64_t)(kMQ * Dl) +
                        (int64_t)u * (QT * NDT * 256) + 4 * lane;
            if (active) {
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                    for (int nt = 0; nt < NDT; ++nt) {
                        bf16x4 h;
#pragma unroll
                        for (int v = 0; v < 4; ++v) h[v] = (bf16)o[qt][nt][v];
                        *reinterpret_cast<bf16x4*>(dst + (qt * NDT + nt) * 256) = h;
                    }
            }
        } else {
            // stage this wave's [kMQ x DPW] block in the (now idle) ring, then store
            // 16 bytes per lane along the output rows
            bf16* ost = ring0 + u * (kMQ * DPW);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int nt = 0; nt < NDT; ++nt)
                        ost[(16 * qt + 4 * g + v) * DPW + 16 * nt + n16] = (bf16)o[qt][nt][v];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): the wave's LDS writes land
            constexpr int LPR = DPW / 8;                // lanes per staged query row
            constexpr int RPS = 64 / LPR;               // query rows per store step
            bf16* dst_base = out + qrow0 * Dl;
#pragma unroll
            for (int i = 0; i < kMQ / RPS; ++i) {
                const int ql = RPS * i + lane / LPR;
                const int c8 = 8 * (lane % LPR);
                if (active && ql < mq)
                    *reinterpret_cast<bf16x8*>(dst_base + (int64_t)ql * Dl + DPW * u + c8) =
                        *reinterpret_cast<const bf16x8*>(ost + ql * DPW + c8);
            }
        }
    } else if (wave == 0 && active) {
        const float l = mlbuf[1][lane];
        const float v = l > 0.0f ? (mlbuf[0][lane] + log2f(l)) * kLn2 : -INFINITY;
        if (nsplit > 1) {
            part_lse[((int64_t)(b * nsplit + split) * QG + qg) * kMQ + lane] = v;
        } else if (lse && lane < mq) {
            lse[qrow0 + lane] = v;
        }
    }
}

// Merge the split partials of one (sequence, query group):
//   o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),  lse = M + ln(sum_s e^(lse_s - M))
// per query row (M = the row's largest lse_s).  The partials o_s are normalised
// per split, bf16, in the attention kernel's fragment order: element
// [u][qt][nt][lane][v] is query row 16qt + 4(lane/16) + v, latent dim
// (Dl/4)u + 16nt + lane%16.  A workgroup takes 512 fragments (4 values each) of
// one 16-row query tile qt, two adjacent ones per thread; its threads issue
// their loads of a batch of splits before the weights are formed, so the merge
// costs about one memory round trip plus the bytes.
template <int Dl, int SB, int CT>
__global__ __launch_bounds__(CT) void k_attend_combine(int n_blocks, int nsplit, int QG, int M,
                                                        const bf16* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        bf16* __restrict__ out,
                                                        float* __restrict__ lse) {
    constexpr int DPW = Dl / 4;
    constexpr int NDT = DPW / 16;
    constexpr int QT = kMQ / 16;
    constexpr int FPT = 4 * NDT * 64;           // fragments of one query tile (all u, nt, lanes)
    constexpr int WPT = FPT / (2 * CT);         // workgroups per query tile (2 fragments a thread)
    constexpr int NWV = CT / 64;                // waves
    constexpr int JS = CT / 16;                 // split stride of the weight threads
    static_assert(FPT % (2 * CT) == 0 && (CT == 128 || CT == 256), "fragment blocks");
    extern __shared__ float wsh[];              // [nsplit][16]: lse, then merge weights
    __shared__ float red[NWV][16];
    __shared__ float rinv[16];

    // Blocks are dealt to XCDs in contiguous ranges, as the attention kernel
    // deals its items, so a sequence's merge runs on the XCD whose L2 holds the
    // partials its splits just wrote.
    const int blk = xcd_item(n_blocks);
    if (blk < 0) return;
    const int part = blk % WPT;
    const int qt = (blk / WPT) % QT;
    const int bq = blk / (WPT * QT);            // b * QG + qg
    const int b = bq / QG;
    const int qg = bq - b * QG;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // this thread's fragments: f and f+1, f = 2(part*256 + tid), over (u, nt,
    // lane) of tile qt -- adjacent lanes of one tile, so the same four rows and
    // latent dims d, d+1, one 16-byte load per split
    const int f = 2 * (part * CT + tid);
    const int lanef = f & 63;
    const int nt = (f >> 6) % NDT;
    const int u = (f >> 6) / NDT;
    const int64_t blk_elems = (int64_t)kMQ * Dl;
    const int64_t frag_off = (int64_t)u * (QT * NDT * 256) + (qt * NDT + nt) * 256 + 4 * lanef;
    const int64_t split_stride = (int64_t)QG * blk_elems;
    const bf16* src = part_o + (int64_t)b * nsplit * split_stride + (int64_t)qg * blk_elems + frag_off;
    const int r4 = 4 * (lanef >> 4);            // the fragments' rows: r4 + j of the tile

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // Thread (r = tid % 16, j = tid / 16) forms the weights of row r for splits
    // j, j+JS, ...; the first LS of its lse values load before the partials, so
    // they do not queue behind them.
    constexpr int LS = SB / JS >= 2 ? SB / JS : 1;
    const float* pl = part_lse + ((int64_t)b * nsplit * QG + qg) * kMQ + 16 * qt;
    const int r = tid & 15, j = tid >> 4;
    float lsv[LS];
#pragma unroll
    for (int i = 0; i < LS; ++i) lsv[i] = pl[(int64_t)min(j + JS * i, nsplit - 1) * QG * kMQ + r];
    __builtin_amdgcn_sched_barrier(0);          // the lse loads stay ahead of the partials
    // SB loads in flight, unconditional: indices past the last split repeat it
    // and get no weight
    bf16x8 v[SB];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int s = 0; s < SB; ++s)
            v[s] = load8(src + (int64_t)min(s0 + s, nsplit - 1) * split_stride);
    };
    auto accumulate = [&](int s0) {
        const int ns = min(SB, nsplit - s0);
#pragma unroll
        for (int s = 0; s < SB; ++s) {
            const float4 w4 = *reinterpret_cast<const float4*>(&wsh[(s0 + min(s, ns - 1)) * 16 + r4]);
            const float wm = s < ns ? 1.0f : 0.0f;
            const float w[4] = {wm * w4.x, wm * w4.y, wm * w4.z, wm * w4.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                acc[jj] += w[jj] * (float)v[s][jj];
                acc[4 + jj] += w[jj] * (float)v[s][4 + jj];
            }
        }
    };
    load_batch(0);
    __builtin_amdgcn_sched_barrier(0);          // the first batch is in flight during the weights
    {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < LS; ++i) {
            const bool ok = j + JS * i < nsplit;
            mx = fmaxf(mx, ok ? lsv[i] : -INFINITY);
            if (ok) wsh[(j + JS * i) * 16 + r] = lsv[i];
        }
        for (int s = j + JS * LS; s < nsplit; s += JS) {
            const float ls = pl[(int64_t)s * QG * kMQ + r];
            wsh[s * 16 + r] = ls;
            mx = fmaxf(mx, ls);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (lane < 16) red[wave][r] = mx;
        lds_barrier();
        mx = red[0][r];
#pragma unroll
        for (int wv = 1; wv < NWV; ++wv) mx = fmaxf(mx, red[wv][r]);
        float tot = 0.0f;
        for (int s = j; s < nsplit; s += JS) {
            const float ls = wsh[s * 16 + r];
            const float w = ls == -INFINITY ? 0.0f : expf(ls - mx);
            wsh[s * 16 + r] = w;
            tot += w;
        }
        tot += __shfl_xor(tot, 16);
        tot += __shfl_xor(tot, 32);
        lds_barrier();                          // every wave has read red[] (maxima)
        if (lane < 16) red[wave][r] = tot;
        lds_barrier();
        if (tid < 16) {
            tot = NWV == 4 ? (red[0][r] + red[1][r]) + (red[2][r] + red[NWV - 1][r])
                           : red[0][r] + red[NWV - 1][r];
            rinv[r] = tot > 0.0f ? 1.0f / tot : 0.0f;
            const int ql = 16 * qt + r;
            if (lse && part == 0 && qg * kMQ + ql < M)
                lse[(int64_t)b * M + qg * kMQ + ql] = tot > 0.0f ? mx + logf(tot) : -INFINITY;
        }
        lds_barrier();                          // weights and 1/sum visible
    }
    accumulate(0);
    for (int s0 = SB; s0 < nsplit; s0 += SB) {
        load_batch(s0);
        accumulate(s0);
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const int d = DPW * u + 16 * nt + (lanef & 15);   // even: dims d, d+1
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int ql = 16 * qt + r4 + jj;
        if (qg * kMQ + ql < M) {
            bf16x2 h;
            h[0] = (bf16)(acc[jj] * rinv[r4 + jj]);
            h[1] = (bf16)(acc[4 + jj] * rinv[r4 + jj]);
            *reinterpret_cast<bf16x2*>(out + ((int64_t)b * M + qg * kMQ + ql) * Dl + d) = h;
        }
    }
}

// Vector path: one workgroup per (b, t, h); any Dl <= 1024, fp32 or bf16.
// Wave w takes rows w, w+4, w+8, ... with its own online softmax (each lane
// holds NPL = ceil(Dl/64) latent dims; the dot product is a wave reduction),
// four rows in flight at a time; the four waves' (max, sum, output) merge
// through LDS at the end.
template <typename E, int NPL>
__global__ __launch_bounds__(256) void k_attend_vector(
    const E* __restrict__ qa, int T, int Hq, int Dl, const E* __restrict__ latent,
    const int64_t* __restrict__ latent_row_start, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ topk_count, int k, const E* __restrict__ hca,
    const int64_t* __restrict__ hca_row_start, const int32_t* __restrict__ hca_count,
    int64_t max_hca, float scale, E* __restrict__ out, float* __restrict__ lse) {
    __shared__ float wml[2][4];
    __shared__ float wo[4][64 * NPL];
    const int h = blockIdx.x % Hq;
    const int64_t bt = blockIdx.x / Hq;
    const int b = (int)(bt / T);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ntop = min(topk_count[b], k);
    const int nh = hca ? (int)min((int64_t)hca_count[b], max_hca) : 0;
    const int n = ntop + nh;
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca ? hca_row_start[b] : 0;
    const int32_t* idx = topk_idx + (int64_t)b * k;
    const E* qrow = qa + (bt * Hq + h) * Dl;
    float qv[NPL], ov[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int d = lane + 64 * i;
        qv[i] = d < Dl ? (float)qrow[d] : 0.0f;
        ov[i] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    auto load_row = [&](int j, float (&rv)[NPL]) {
        const E* row = att_row<E>(j, ntop, n, latent, lrs, idx, hca, hrs, Dl);
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int d = lane + 64 * i;
            rv[i] = (row && d < Dl) ? (float)row[d] : 0.0f;
        }
    };
    auto consume = [&](const float (&rv)[NPL]) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) part += qv[i] * rv[i];
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        const float logit = part * scale;
        const float mn = fmaxf(m, logit);
        const float a = expf(m - mn);
        const float p = expf(logit - mn);
        l = l * a + p;
#pragma unroll
        for (int i = 0; i < NPL; ++i) ov[i] = ov[i] * a + p * rv[i];
        m = mn;
    };
    constexpr int RU = 4;                       // rows in flight per wave
    for (int j = wave; j < n; j += 4 * RU) {
        float rv[RU][NPL];
#pragma unroll
        for (int r = 0; r < RU; ++r) load_row(j + 4 * r, rv[r]);   // zeros past the end
#pragma unroll
        for (int r = 0; r < RU; ++r)
            if (j + 4 * r < n) consume(rv[r]);
    }
    if (lane == 0) {
        wml[0][wave] = m;
        wml[1][wave] = l;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) wo[wave][lane + 64 * i] = ov[i];
    __syncthreads();
    // merge: waves without rows (sum 0) get weight 0
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        if (wml[1][w] > 0.0f) M = fmaxf(M, wml[0][w]);
    float sc[4], L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        sc[w] = wml[1][w] > 0.0f ? expf(wml[0][w] - M) : 0.0f;
        L += sc[w] * wml[1][w];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int d = threadIdx.x; d < Dl; d += 256) {
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) o += sc[w] * wo[w][d];
        out[(bt * Hq + h) * Dl + d] = (E)(o * inv);
    }
    if (threadIdx.x == 0 && lse) lse[bt * Hq + h] = L > 0.0f ? M + logf(L) : -INFINITY;
}

// Split heuristic shared by the launches and the workspace query: groups of kMQ
// query rows, then enough row splits to give ~kAttWGTarget workgroups, keeping
// at least two row chunks per split.  When the rows are split and an HCA pool is
// given, no split mixes top-k rows and HCA rows: splits 0 .. nts-1 take the
// top-k list (rps_top rows each, at most k in all) and the rest the HCA rows,
// so the HCA splits can run before the top-k list exists.
struct AttendPlan {
    int QG;
    int nsplit;          // splits per (sequence, query group)
    int rows_per_split;  // rows per split (per HCA split when nts > 0)
    int nts;             // top-k splits; 0 = splits over the joined row list
    int rps_top;         // rows per top-k split (nts > 0)
    int n_items;         // B * QG * nsplit
};

static AttendPlan attend_plan(int B, int T, int Hq, int k, int64_t max_hca) {
    const int64_t rows = (int64_t)k + (max_hca > 0 ? max_hca : 0);
    const int64_t M = (int64_t)T * Hq;
    const int QG = (int)((M + kMQ - 1) / kMQ);
    const int64_t units = (int64_t)B * QG;
    int64_t ns = (kAttWGTarget + units - 1) / units;
    const int64_t max_ns = (rows + 2 * kChunk - 1) / (2 * kChunk);
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    int64_t rps = (rows + ns - 1) / ns;
    rps = (rps + kChunk - 1) / kChunk * kChunk;
    if (rps < kChunk) rps = kChunk;
    if (rps > kMaxSplitRows) rps = kMaxSplitRows;
    ns = (rows + rps - 1) / rps;
    if (ns < 1) ns = 1;
    if (ns == 1 || max_hca <= 0)
        return AttendPlan{QG, (int)ns, (int)rps, 0, 0, (int)(units * ns)};
    int64_t rtop = kAttTopRows > 0 ? kAttTopRows : rps;
    rtop = (rtop + kChunk - 1) / kChunk * kChunk;
    if (rtop > kMaxSplitRows) rtop = kMaxSplitRows;
    const int64_t nts = ((int64_t)k + rtop - 1) / rtop;
    const int64_t nhs = (max_hca + rps - 1) / rps;
    return AttendPlan{QG, (int)(nts + nhs), (int)rps, (int)nts, (int)rtop,
                      (int)(units * (nts + nhs))};
}

static bool attend_mfma_shape(int dtype, int Hq, int Dl) {
    (void)Hq;
    return dtype == LSA_DTYPE_BF16 && (Dl == 128 || Dl == 256 || Dl == 512);
}

}  // namespace lsa

using namespace lsa;

size_t lsa_attend_workspace(int dtype, int B, int T, int Hq, int Dl, int k, int64_t max_hca) {
    if (!attend_mfma_shape(dtype, Hq, Dl)) return 0;
    const AttendPlan p = attend_plan(B, T, Hq, k, max_hca);
    if (p.nsplit <= 1) return 0;
    const size_t n = (size_t)B * p.nsplit * p.QG * kMQ;   // partial query rows
    return n * Dl * sizeof(bf16) + n * sizeof(float);
}

// phase: kAttAll = every split and the merge; kAttHca = the HCA splits only
// (partials into the workspace; nothing when the plan has none);
// kAttSelected = the remaining splits and the merge.
enum { kAttAll = 0, kAttHca = 1, kAttSelected = 2 };

static int attend_impl(const char* name, int phase, const void* qa, int dtype, int B, int T,
                       int Hq, int Dl, const void* latent, const int64_t* latent_row_start,
                       const int32_t* topk_idx, const int32_t* topk_count, int k, const void* hca,
                       const int64_t* hca_row_start, const int32_t* hca_count, int64_t max_hca,
                       float scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
    clear_error();
    if (!qa || (phase != kAttHca && (!latent || !latent_row_start || !topk_idx || !topk_count ||
                                     !out)))
        return fail(LSA_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
    if (phase == kAttHca && !hca)
        return fail(LSA_ERR_INVALID_ARG, "%s: the HCA pool is NULL", name);
    if (hca && (!hca_row_start || !hca_count))
        return fail(LSA_ERR_INVALID_ARG, "%s: hca given without row starts/counts", name);
    if (B <= 0 || T <= 0 || Hq <= 0 || Dl <= 0 || k <= 0 || (hca && max_hca < 0))
        return fail(LSA_ERR_INVALID_ARG, "%s: B=%d T=%d Hq=%d Dl=%d k=%d", name, B, T, Hq, Dl, k);
    if (dtype != LSA_DTYPE_F32 && dtype != LSA_DTYPE_BF16)
        return fail(LSA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, dtype);
    if (!aligned16(qa) || (latent && !aligned16(latent)) || (hca && !aligned16(hca)))
        return fail(LSA_ERR_INVALID_ARG, "%s: qa/latent/hca must be 16-byte aligned", name);
    if (!(scale == scale)) return fail(LSA_ERR_INVALID_ARG, "%s: scale is NaN", name);
    if (Dl > 1024) return fail(LSA_ERR_UNSUPPORTED, "%s: Dl=%d > 1024", name, Dl);
    if (B > 65535 || T > 65535)
        return fail(LSA_ERR_UNSUPPORTED, "%s: B or T above 65535", name);
    if ((int64_t)k + (hca ? max_hca : 0) > kMaxAttendRows)
        return fail(LSA_ERR_UNSUPPORTED, "%s: k + max_hca above %lld rows", name,
                    (long long)kMaxAttendRows);
    const int64_t hmax = hca ? max_hca : 0;
    const size_t need = lsa_attend_workspace(dtype, B, T, Hq, Dl, k, hmax);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(LSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", name, workspace_bytes,
                    need);
    int cus = 0;
    int rc = check_device(&cus);
    if (rc != LSA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const bool mfma = attend_mfma_shape(dtype, Hq, Dl);
    if (phase == kAttHca) {
        // Only a split plan has HCA splits of their own; otherwise the selected
        // phase attends every row and this phase enqueues nothing.
        if (!mfma) return LSA_OK;
        const AttendPlan p = attend_plan(B, T, Hq, k, hmax);
        if (p.nts == 0) return LSA_OK;
        const size_t n = (size_t)B * p.nsplit * p.QG * kMQ;
        bf16* part_o = (bf16*)workspace;
        float* part_lse = (float*)(part_o + n * Dl);
        const int nloc = p.nsplit - p.nts;
        const int n_items = B * p.QG * nloc;
        const unsigned grid = (unsigned)(8 * ((n_items + 7) / 8));
        const float sl2 = scale * kLog2e;
        const int M = T * Hq;
        // Stand-ins for the top-k arguments: HCA splits read no top-k row, and
        // with k = 1 the kernel's speculative index loads stay inside hca_count.
#define LSA_ATT_H(dl, nt)                                                                      \
    hipLaunchKernelGGL((k_attend_mfma<dl, kAttRing, nt>), dim3(grid), dim3(512), 0, st,         \
                       n_items, p.QG, p.nsplit, p.nts, nloc, p.nts, p.rps_top, p.rows_per_split, \
                       M, 1, hca_count, (const bf16*)qa, hca_count, hca_count, hca_row_start,   \
                       hca_row_start, hmax, (const bf16*)hca, (const bf16*)hca, sl2,            \
                       (bf16*)nullptr, (float*)nullptr, part_o, part_lse)
        if (p.QG == 1) {
            if (Dl == 512) LSA_ATT_H(512, true); else if (Dl == 256) LSA_ATT_H(256, true); else LSA_ATT_H(128, true);
        } else {
            if (Dl == 512) LSA_ATT_H(512, false); else if (Dl == 256) LSA_ATT_H(256, false); else LSA_ATT_H(128, false);
        }
#undef LSA_ATT_H
        return launch_status("attend_mfma");
    }

    if (attend_mfma_shape(dtype, Hq, Dl)) {
        const AttendPlan p = attend_plan(B, T, Hq, k, hmax);
        const size_t n = (size_t)B * p.nsplit * p.QG * kMQ;
        bf16* part_o = (bf16*)workspace;
        float* part_lse = p.nsplit > 1 ? (float*)(part_o + n * Dl) : nullptr;
        // the selected phase runs the top-k splits only (the HCA splits ran before)
        const int nloc = (phase == kAttSelected && p.nts > 0) ? p.nts : p.nsplit;
        const int n_items = B * p.QG * nloc;
        const unsigned grid = (unsigned)(8 * ((n_items + 7) / 8));
        const float sl2 = scale * kLog2e;
        const int M = T * Hq;
        // Without an HCA pool the kernel reads valid stand-ins and attends zero
        // HCA rows (max_hca = 0), so it never branches on the pool.
        const void* hp = hca ? hca : latent;
        const int64_t* hrs_p = hca ? hca_row_start : latent_row_start;
        const int32_t* hcnt_p = hca ? hca_count : topk_count;
#define LSA_ATT(dl, nt)                                                                        \
    hipLaunchKernelGGL((k_attend_mfma<dl, kAttRing, nt>), dim3(grid), dim3(512), 0, st,         \
                       n_items, p.QG, p.nsplit, 0, nloc, p.nts, p.rps_top, p.rows_per_split,    \
                       M, k, topk_idx,                                                          \
                       (const bf16*)qa, topk_count, hcnt_p, latent_row_start, hrs_p, hmax,      \
                       (const bf16*)latent, (const bf16*)hp, sl2, (bf16*)out, lse, part_o,      \
                       part_lse)
        // With one query group every row is copied by one workgroup only: stream it
        // past the caches (6-7 % faster at decode_500k and ragged_mix); with more,
        // the groups of one split read the same rows and keep the default policy.
        if (p.QG == 1) {
            if (Dl == 512) LSA_ATT(512, true); else if (Dl == 256) LSA_ATT(256, true); else LSA_ATT(128, true);
        } else {
            if (Dl == 512) LSA_ATT(512, false); else if (Dl == 256) LSA_ATT(256, false); else LSA_ATT(128, false);
        }
#undef LSA_ATT
        rc = launch_status("attend_mfma");
        if (rc != LSA_OK || p.nsplit == 1) return rc;
        // partials: one [kMQ x Dl] block per (b, split, query group)
        // 256-thread blocks, or 128-thread ones (twice as many) when the 256-thread
        // grid would leave CUs idle: every thread keeps all SB loads in flight, so
        // the rate follows the number of CUs holding blocks
        const int blocks256 = B * p.QG * (kMQ / 16) * (Dl / 128);
        const bool small_blocks = blocks256 < cus;
        const int cblocks = small_blocks ? 2 * blocks256 : blocks256;
        const unsigned cgrid = (unsigned)(8 * ((cblocks + 7) / 8));
        const size_t cshm = sizeof(float) * 16 * (size_t)p.nsplit;
#define LSA_COMB_CT(dl, sb, ct)                                                                \
    hipLaunchKernelGGL((k_attend_combine<dl, sb, ct>), dim3(cgrid), dim3(ct), cshm, st, cblocks,  \
                       p.nsplit, p.QG, M, part_o, part_lse, (bf16*)out, lse)
#define LSA_COMB(dl, sb)                                                                       \
    if (small_blocks) LSA_COMB_CT(dl, sb, 128); else LSA_COMB_CT(dl, sb, 256)
#define LSA_COMB_DL(sb)                                                                        \
    if (Dl == 512) { LSA_COMB(512, sb); } else if (Dl == 256) { LSA_COMB(256, sb); }           \
    else { LSA_COMB(128, sb); }
        if (p.nsplit <= 8) { LSA_COMB_DL(8); }
        else if (p.nsplit <= 16) { LSA_COMB_DL(16); }
        else { LSA_COMB_DL(32); }
#undef LSA_COMB_DL
#undef LSA_COMB
#undef LSA_COMB_CT
        return launch_status("attend_combine");
    }
    const unsigned blocks = (unsigned)((int64_t)B * T * Hq);
#define LSA_ATTV(E, npl)                                                                       \
    hipLaunchKernelGGL((k_attend_vector<E, npl>), dim3(blocks), dim3(256), 0, st,              \
                       (const E*)qa, T, Hq, Dl, (const E*)latent, latent_row_start, topk_idx,  \
                       topk_count, k, (const E*)hca, hca_row_start, hca_count, hmax, scale,    \
                       (E*)out, lse)
#define LSA_ATTV_NPL(E)                                                                        \
    if (Dl <= 64) { LSA_ATTV(E, 1); }                                                          \
    else if (Dl <= 128) { LSA_ATTV(E, 2); }                                                    \
    else if (Dl <= 256) { LSA_ATTV(E, 4); }                                                    \
    else if (Dl <= 512) { LSA_ATTV(E, 8); }                                                    \
    else { LSA_ATTV(E, 16); }
    if (dtype == LSA_DTYPE_F32) {
        LSA_ATTV_NPL(float)
    } else {
        LSA_ATTV_NPL(bf16)
    }
#undef LSA_ATTV_NPL
#undef LSA_ATTV
    return launch_status("attend_vector");
}

extern "C" int lsa_sparse_attend(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                                 const void* latent, const int64_t* latent_row_start,
                                 const int32_t* topk_idx, const int32_t* topk_count, int k,
                                 const void* hca, const int64_t* hca_row_start,
                                 const int32_t* hca_count, int64_t max_hca, float scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return attend_impl("lsa_sparse_attend", kAttAll, qa, dtype, B, T, Hq, Dl, latent,
                       latent_row_start, topk_idx, topk_count, k, hca, hca_row_start, hca_count,
                       max_hca, scale, out, lse, workspace, workspace_bytes, stream);
}

extern "C" int lsa_sparse_attend_hca(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                                     int k, const void* hca, const int64_t* hca_row_start,
                                     const int32_t* hca_count, int64_t max_hca, float scale,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return attend_impl("lsa_sparse_attend_hca", kAttHca, qa, dtype, B, T, Hq, Dl, nullptr,
                       nullptr, nullptr, nullptr, k, hca, hca_row_start, hca_count, max_hca,
                       scale, nullptr, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int lsa_sparse_attend_selected(const void* qa, int dtype, int B, int T, int Hq,
                                          int Dl, const void* latent,
                                          const int64_t* latent_row_start,
                                          const int32_t* topk_idx, const int32_t* topk_count,
                                          int k, const void* hca, const int64_t* hca_row_start,
                                          const int32_t* hca_count, int64_t max_hca, float scale,
                                          void* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    return attend_impl("lsa_sparse_attend_selected", kAttSelected, qa, dtype, B, T, Hq, Dl,
                       latent, latent_row_start, topk_idx, topk_count, k, hca, hca_row_start,
                       hca_count, max_hca, scale, out, lse, workspace, workspace_bytes, stream);
}
