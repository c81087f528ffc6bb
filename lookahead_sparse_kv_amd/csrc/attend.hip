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
// pairs of b are flattened into M = T * Hq query rows.  A workgroup of four
// waves takes one (b, group of 32 query rows, row split) and walks its rows in
// chunks of 32:
//   1. the chunk's rows are copied from HBM straight into an LDS ring slot
//      (direct-to-LDS loads, each wave copying a quarter; NB-1 chunks ahead);
//   2. S = Q K^T: wave w owns the 16 x 16 tile (query rows 16(w&1).., chunk
//      rows 16(w>>1)..) over the full latent depth, Q held in registers, so
//      no partial logits cross waves;
//   3. online softmax in base 2: per-query-row maxima and sums of the two row
//      tiles meet in LDS, P (bf16) is published there;
//   4. O[:, dims_w] += P C[:, dims_w]: wave w owns Dl/4 latent dims of all 32
//      query rows; C^T operands come from transposing LDS reads of the slot.
// Rows are split across workgroups when B * T * Hq is small; a combine kernel
// merges the splits by their log-sum-exp.
#include "common.hpp"

namespace lsa {

constexpr int kAttWGTarget = 256;   // workgroups the split heuristic aims for
constexpr int kChunk = 32;          // attended rows per step
constexpr int kMaxSplitRows = 2048; // most rows one split may take (64 chunks: one per lane)
constexpr int kMQ = 32;             // query rows per workgroup
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
// p ^ slot_swz(r).  Conflict-free for 16 consecutive rows reading one logical
// slot (the Q K^T operand: the values over r mod 16 are a permutation of 0..15)
// and for the 8 rows {j, j+8 : j in 4h..4h+3} reading one even/odd slot pair
// (the transposing P C reads: those rows take 8 distinct values, all even or
// all odd).
__device__ __forceinline__ int slot_swz(int r) {
    return 2 * ((r & 3) + 4 * ((r >> 3) & 1)) + ((r >> 2) & 1);
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

// vmcnt(n) with the other counters left alone (n <= 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations retire
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, so the direct-to-LDS copies of later chunks stay in
// flight across it; each wave waits for its own copies with wait_vmcnt first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0), vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
}

// Parameter order: what the first loads need comes first (14 dwords: the work
// item, the Q and index addresses, the count pointers), so a build that
// preloads kernel arguments into scalar registers issues them at launch.
template <int Dl, int NB>
__global__ __launch_bounds__(512, 1) void k_attend_mfma(
    int n_items, int QG, int nsplit, int rows_per_split, int M, int k,
    const int32_t* __restrict__ topk_idx, const bf16* __restrict__ qa,
    const int32_t* __restrict__ topk_count, const int32_t* __restrict__ hca_count,
    const int64_t* __restrict__ latent_row_start, const int64_t* __restrict__ hca_row_start,
    int64_t max_hca, const bf16* __restrict__ latent, const bf16* __restrict__ hca,
    float scale_log2, bf16* __restrict__ out, float* __restrict__ lse, bf16* __restrict__ part_o,
    float* __restrict__ part_lse) {
    constexpr int NW = 4;                       // compute waves (waves 0..3)
    constexpr int NP = 4;                       // copy waves (waves 4..7)
    constexpr int SL = Dl / 8;                  // 16-byte slots per latent row
    constexpr int RPI = 64 / SL;                // rows per direct-to-LDS instruction
    constexpr int IPW = kChunk / (RPI * NP);    // such instructions per copy wave per chunk
    constexpr int KDT = Dl / 32;                // k-steps of Q K^T
    constexpr int DPW = Dl / NW;                // latent dims per wave in P C
    constexpr int NDT = DPW / 16;               // 16-wide dim tiles of P C
    constexpr int PROW = 40;                    // bf16 per query row of P (conflict-free reads)
    static_assert(SL >= 16 && IPW >= 1 && NB >= 2 && NB <= 4, "tiling");
    static_assert(kMQ * DPW * NW <= kChunk * Dl, "output staging fits one ring slot");

    // One LDS object holds every buffer: the compiler then leaves the ordering of
    // the direct-to-LDS copies and the LDS reads to the explicit counted waits
    // and barriers below instead of draining all copies before each LDS read.
    constexpr int OFF_PBUF = NB * kChunk * Dl * 2;          // ring: NB slots of kChunk rows
    constexpr int OFF_SMAX = OFF_PBUF + 2 * kMQ * PROW * 2; // P (bf16), two buffers
    constexpr int OFF_FLAG = OFF_SMAX + 2 * kMQ * 4;        // chunk maxima of the two row tiles
    constexpr int OFF_ABUF = OFF_FLAG + 32;                 // per-wave "running max moves" flags, two sets
    constexpr int OFF_ML = OFF_ABUF + kMQ * 4;              // rescale factors of O
    constexpr int LDS_BYTES = OFF_ML + 2 * kMQ * 4;         // final (m, l)
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    bf16* const ring0 = reinterpret_cast<bf16*>(lds);
    bf16* const pbuf = reinterpret_cast<bf16*>(lds + OFF_PBUF);
    float (*const smax)[kMQ] = reinterpret_cast<float (*)[kMQ]>(lds + OFF_SMAX);
    int* const flags = reinterpret_cast<int*>(lds + OFF_FLAG);
    float* const abuf = reinterpret_cast<float*>(lds + OFF_ABUF);
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
    const int b = tq / nsplit;
    const int split = tq - b * nsplit;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    const int n16 = lane & 15;
    const int g = lane >> 4;
    const bool copier = wave >= NW;
    const int rt = (wave >> 1) & 1;             // Q K^T: chunk rows 16rt .. 16rt+15
    const int ht = wave & 1;                    //        query rows 16ht .. 16ht+15

    const int rs = split * rows_per_split;
    const int32_t* idx = topk_idx + (int64_t)b * k;
    const int64_t qrow0 = (int64_t)b * M + (int64_t)qg * kMQ;   // first query row of the group
    const int mq = min(kMQ, M - qg * kMQ);                        // valid query rows

    // Q fragments (A operand): query row 16ht + n16, dims 32kk + 8g .. +7
    bf16x8 qf[KDT];
    if (!copier) {
        // rows past the group's end read its first row and are zeroed after
        const bool ok = 16 * ht + n16 < mq;
        const bf16* qp = qa + (qrow0 + (ok ? 16 * ht + n16 : 0)) * Dl + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KDT; ++kk) qf[kk] = load8(qp + 32 * kk);
        if (!ok) {
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) qf[kk] = zero8();
        }
    }
    // Copy wave p stages rows 8p .. 8p+7 of every chunk.  Lane c holds the
    // chosen-entry indices of those rows of chunk c (a split has at most 64
    // chunks); rows past the split end are clamped to its last row.
    // The loads are speculative (clamped into the index row, used only for rows
    // below the top-k count), so they do not wait for the counts; rows past the
    // split end re-read the split's first row.
    int ridx[8];
    int first_idx = 0;
    if (copier) {
#pragma unroll
        for (int j8 = 0; j8 < 8; ++j8)
            ridx[j8] = idx[min(rs + kChunk * lane + 8 * (wave - NW) + j8, k - 1)];
        first_idx = idx[min(rs, k - 1)];
    }
    // The per-sequence counts and row starts load while the vector loads above
    // are in flight.
    const int topk_cnt = topk_count[b];
    const int hca_cnt = hca_count[b];
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca_row_start[b];
    const int ntop = min(topk_cnt, k);
    const int nh = (int)min((int64_t)hca_cnt, max_hca);   // max_hca = 0 without a pool
    const int n = ntop + nh;
    const int re = min(n, rs + rows_per_split);
    const int nchunks = (active && re > rs) ? (re - rs + kChunk - 1) / kChunk : 0;
    // Q (compute waves) and the indices (copy waves) are complete before the
    // loop.  Only the copy waves issue copies, so their counted waits below are
    // exact, and the compute waves never have a copy outstanding when they read
    // LDS.
    wait_vmcnt<0>();
    // Copy waves: the 64-bit address of every row they stage, computed once
    // (lane c holds rows 8p .. 8p+7 of chunk c, p = wave - NW), so a copy costs
    // two lane reads and no branches.  Rows past the split end re-read the
    // split's first row (finite data, probability zero).
    uint32_t raddr_lo[8], raddr_hi[8];
    if (copier) {
        const uint64_t lat = (uint64_t)latent, hc = (uint64_t)hca;
#pragma unroll
        for (int j8 = 0; j8 < 8; ++j8) {
            const int j0 = rs + kChunk * lane + 8 * (wave - NW) + j8;
            const bool past = j0 >= re;
            const int j = past ? rs : j0;
            const int e = past ? first_idx : ridx[j8];
            const uint64_t a = j < ntop ? lat + (uint64_t)(lrs + e) * (uint64_t)(Dl * 2)
                                        : hc + (uint64_t)(hrs + (j - ntop)) * (uint64_t)(Dl * 2);
            raddr_lo[j8] = (uint32_t)a;
            raddr_hi[j8] = (uint32_t)(a >> 32);
        }
    }
    f32x4 o[2][NDT];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) o[h2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // wave 0 also accumulates P . 1: the row sums l of P, rescaled with O
    f32x4 ol[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // running max (base 2) and sum of query rows 16ht + 4g + v (sums kept by rt == 0)
    float m_ref[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        m_ref[v] = -INFINITY;
    }

    // Chunk c -> ring slot c % NB.  Instruction i of copy wave p moves chunk rows
    // 8p + RPI*i ..; lane L fills physical slot L % SL of its row r with logical
    // slot (L % SL) ^ swz(r).  Rows past the split end re-read its first row
    // (finite data, probability zero).
    auto issue_chunk = [&](int c) {
        bf16* slot = ring0 + (c % NB) * (kChunk * Dl);
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int sub = lane / SL;                     // row of this lane in the instruction
            const int rbase = 8 * (wave - NW) + RPI * i;
            const int rl = rbase + sub;
            uint32_t lo = __builtin_amdgcn_readlane(raddr_lo[RPI * i], c);
            uint32_t hi = __builtin_amdgcn_readlane(raddr_hi[RPI * i], c);
#pragma unroll
            for (int s2 = 1; s2 < RPI; ++s2)
                if (sub == s2) {
                    lo = __builtin_amdgcn_readlane(raddr_lo[RPI * i + s2], c);
                    hi = __builtin_amdgcn_readlane(raddr_hi[RPI * i + s2], c);
                }
            const bf16* row = reinterpret_cast<const bf16*>(((uint64_t)hi << 32) | lo);
            __builtin_amdgcn_global_load_lds(
                (const void*)(row + 8 * ((lane % SL) ^ slot_swz(rl))),
                (__attribute__((address_space(3))) void*)(slot + rbase * Dl), 16, 0, 0);
        }
    };

    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    // Q K^T of chunk c, then P against the running max into pbuf[c & 1] and this
    // wave's "running max must move" flag into flags[c & 1].  Returns the
    // base-2 logits (kept for the slow path).
    auto qk_p = [&](int c) -> f32x4 {
        const int r0 = rs + c * kChunk;
        const bf16* sl = ring0 + (c % NB) * (kChunk * Dl);
        // S tile: D[4g+v][n16] = query row 16ht + 4g + v against chunk row 16rt + n16
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const int r = 16 * rt + n16;
            const int sw = slot_swz(r);
            // logical slot 4kk + g sits at physical ((4(kk & 3) + g) ^ sw) + 16(kk >> 2):
            // the swizzle only touches the low four slot bits, so four base
            // addresses and immediate offsets cover every step
            const bf16* kp[4];
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) kp[b4] = sl + r * Dl + 8 * ((4 * b4 + g) ^ sw);
            // K operands through an 8-deep register window: 8 reads stay in flight
            constexpr int KW = KDT < 8 ? KDT : 8;
            bf16x8 kb[KW];
#pragma unroll
            for (int kk = 0; kk < KW; ++kk)
                kb[kk] = *reinterpret_cast<const bf16x8*>(kp[kk & 3] + 128 * (kk >> 2));
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) {
                sacc = mfma16(qf[kk], kb[kk % KW], sacc);
                if (kk + KW < KDT)
                    kb[kk % KW] = *reinterpret_cast<const bf16x8*>(kp[(kk + KW) & 3] + 128 * ((kk + KW) >> 2));
            }
            // schedule: the first KW reads, then one product per refill read
            __builtin_amdgcn_sched_group_barrier(0x100, KW, 0);
#pragma unroll
            for (int kk = 0; kk < KDT - KW; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KW, 0);
        }
        // this lane holds query rows q0 + v (v = 0..3) against chunk row 16rt + n16
        const int q0 = 16 * ht + 4 * g;
        const bool valid = r0 + 16 * rt + n16 < re;
        f32x4 x;
#pragma unroll
        for (int v = 0; v < 4; ++v) x[v] = valid ? sacc[v] * scale_log2 : -INFINITY;
        // Fast path: P against the running max, which stands unless some logit of
        // the chunk exceeds it by more than kRescaleSlack (lazy rescale; always on
        // the first chunk, as -inf + slack = -inf).  p <= 2^kRescaleSlack.
        bf16* pb = pbuf + (c & 1) * (kMQ * PROW);
        bool over = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            over = over || x[v] > m_ref[v] + kRescaleSlack;
            const float p = valid ? __builtin_amdgcn_exp2f(x[v] - m_ref[v]) : 0.0f;
            pb[(q0 + v) * PROW + 16 * rt + n16] = (bf16)p;
        }
        const bool wave_over = __ballot(over) != 0;
        if (lane == 0) flags[4 * (c & 1) + wave] = wave_over ? 1 : 0;
        return x;
    };
    // After the barrier that publishes chunk c's P and flags: the slow path if
    // any flag is set, then O[:, dims_w] += P C[:, dims_w].
    auto pv = [&](int c, f32x4 x) {
        const bf16* sl = ring0 + (c % NB) * (kChunk * Dl);
        bf16* pb = pbuf + (c & 1) * (kMQ * PROW);
        const int* fl = flags + 4 * (c & 1);
        // P C over this wave's dims.  A: query row 16h2 + n16, chunk rows 8g .. 8g+7.
        // B from transposing reads: in each 16-lane group, lanes 4j..4j+3 point at
        // chunk row 8g + j (+4 for the upper half), 4 dims each, and lane i receives
        // dim i of those 4 rows.
        bf16x8 pa[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            pa[h2] = *reinterpret_cast<const bf16x8*>(&pb[(16 * h2 + n16) * PROW + 8 * g]);
        const int trow0 = 8 * g + (n16 >> 2);
        const int trow1 = trow0 + 4;
        const int sw0 = slot_swz(trow0), sw1 = slot_swz(trow1);
        const int q4 = n16 & 3;
        const int off = 4 * (q4 & 1);
        // all of the chunk's C^T operands are read before the products, so the
        // transposing reads overlap each other rather than the matrix ops
        bf16x4 lo[NDT], hi[NDT];
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
            const int ls = (DPW / 8) * wave + 2 * nt + (q4 >> 1);   // logical 16-byte slot
            lo[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(sl + trow0 * Dl + 8 * (ls ^ sw0) + off));
            hi[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(sl + trow1 * Dl + 8 * (ls ^ sw1) + off));
        }
        // the flags are read with the operands, so their latency overlaps
        const bool slow = (fl[0] | fl[1] | fl[2] | fl[3]) != 0;   // uniform
        if (slow) {
            // Slow path: the chunk maxima of the two row tiles meet, the running
            // max moves where it grew by more than the slack (alpha = 2^(m_old -
            // m_new), 0 on the first chunk), and P is recomputed against it.
            const int q0 = 16 * ht + 4 * g;
            const bool valid = rs + c * kChunk + 16 * rt + n16 < re;
            f32x4 cm;
#pragma unroll
            for (int v = 0; v < 4; ++v) cm[v] = group_max<16>(x[v]);
            if (n16 == 0) *reinterpret_cast<f32x4*>(&smax[rt][q0]) = cm;
            lds_barrier();
            const f32x4 ma = *reinterpret_cast<const f32x4*>(&smax[0][q0]);
            const f32x4 mb = *reinterpret_cast<const f32x4*>(&smax[1][q0]);
            f32x4 alpha;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float cmax = fmaxf(ma[v], mb[v]);
                const bool grow = cmax > m_ref[v] + kRescaleSlack;
                alpha[v] = grow ? __builtin_amdgcn_exp2f(m_ref[v] - cmax) : 1.0f;
                m_ref[v] = grow ? cmax : m_ref[v];
                const float p = valid ? __builtin_amdgcn_exp2f(x[v] - m_ref[v]) : 0.0f;
                pb[(q0 + v) * PROW + 16 * rt + n16] = (bf16)p;
            }
            if (rt == 0 && n16 == 0) *reinterpret_cast<f32x4*>(&abuf[q0]) = alpha;
            lds_barrier();
            // rescale O (and wave 0's row sums) rows whose running max moved
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4 al = *reinterpret_cast<const f32x4*>(&abuf[16 * h2 + 4 * g]);
                if (al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f) {
#pragma unroll
                    for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) o[h2][nt][v] *= al[v];
#pragma unroll
                    for (int v = 0; v < 4; ++v) ol[h2][v] *= al[v];
                }
            }
            // P was rewritten: read the operands again
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                pa[h2] = *reinterpret_cast<const bf16x8*>(&pb[(16 * h2 + n16) * PROW + 8 * g]);
        }
        if (wave == 0) {
            bf16x8 ones;
#pragma unroll
            for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.0f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) ol[h2] = mfma16(pa[h2], ones, ol[h2]);
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
            for (int h2 = 0; h2 < 2; ++h2) o[h2][nt] = mfma16(pa[h2], cb, o[h2][nt]);
        }
    };

    // Pipeline, one barrier per chunk (X_c): before it, every compute wave has
    // published chunk c's P and flag and finished P C of chunk c-1, and the copy
    // waves have staged chunk c+1; after it, the copy waves refill chunk c-1's
    // slot with chunk c+NB-1 while the compute waves run P C of chunk c and
    // Q K^T of chunk c+1.  P and the flags alternate between two buffers, so the
    // writes for chunk c+1 never meet a late reader of chunk c.  The slow path
    // adds two barriers, taken by all eight waves (every wave reads the same
    // flags after X_c).
    if (copier) {
#pragma unroll
        for (int c = 0; c < NB - 1; ++c)
            if (c < nchunks) issue_chunk(c);
        static_assert(NB <= 4, "the waits below cover two later chunks");
        // X_{-1}: chunk 0 staged
        {
            const int after = min(nchunks - 1, NB - 2);   // chunks issued after chunk 0
            if (after >= 2) wait_vmcnt<2 * IPW>();
            else if (after == 1) wait_vmcnt<IPW>();
            else wait_vmcnt<0>();
        }
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            // chunk c+1 staged before X_c (chunks up to c+NB-2 are issued)
            const int after = min(nchunks - 1, c + NB - 2) - (c + 1);
            if (after >= 1) wait_vmcnt<IPW>();
            else wait_vmcnt<0>();
            lds_barrier();                                      // X_c
            if (c + NB - 1 < nchunks) issue_chunk(c + NB - 1);
            const int* fl = flags + 4 * (c & 1);
            if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
                lds_barrier();                                  // slow path: maxima met
                lds_barrier();                                  // slow path: P republished
            }
        }
        // the two barriers of the output stage below
        lds_barrier();
        lds_barrier();
        return;
    }
    lds_barrier();                                              // X_{-1}
    f32x4 xc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nchunks > 0) xc = qk_p(0);
    for (int c = 0; c < nchunks; ++c) {
        lds_barrier();                                          // X_c
        pv(c, xc);
        if (c + 1 < nchunks) xc = qk_p(c + 1);
    }

    // publish (m, l); every wave normalises its O columns and stages them in LDS
    // (ring slot 0, free now) so the stores to HBM are 16 bytes per lane
    if (rt == 0 && n16 == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) mlbuf[0][16 * ht + 4 * g + v] = m_ref[v];
    }
    if (wave == 0 && n16 == 0) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int v = 0; v < 4; ++v) mlbuf[1][16 * h2 + 4 * g + v] = ol[h2][v];
    }
    lds_barrier();
    bf16* ost = ring0 + wave * (kMQ * DPW);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int ql = 16 * h2 + 4 * g + v;
            const float l = mlbuf[1][ql];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int nt = 0; nt < NDT; ++nt) ost[ql * DPW + 16 * nt + n16] = (bf16)(o[h2][nt][v] * inv);
        }
    lds_barrier();
    {
        constexpr int LPR = DPW / 8;            // lanes per staged query row
        constexpr int RPS = 64 / LPR;           // query rows per store step
        bf16* dst_base = (nsplit == 1) ? out + qrow0 * Dl
                                       : part_o + ((int64_t)(b * nsplit + split) * M +
                                                   (int64_t)qg * kMQ) * Dl;
#pragma unroll
        for (int i = 0; i < kMQ / RPS; ++i) {
            const int ql = RPS * i + lane / LPR;
            const int c8 = 8 * (lane % LPR);
            if (active && ql < mq)
                *reinterpret_cast<bf16x8*>(dst_base + (int64_t)ql * Dl + DPW * wave + c8) =
                    *reinterpret_cast<const bf16x8*>(ost + ql * DPW + c8);
        }
    }
    if (active && tid < mq) {
        const float l = mlbuf[1][tid];
        const float v = l > 0.0f ? (mlbuf[0][tid] + log2f(l)) * kLn2 : -INFINITY;
        if (nsplit == 1) {
            if (lse) lse[qrow0 + tid] = v;
        } else {
            part_lse[(int64_t)(b * nsplit + split) * M + (int64_t)qg * kMQ + tid] = v;
        }
    }
}

// Merge the split partials: o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M) per
// query row; the partial o_s are normalised per split and stored in bf16.
// A workgroup of 256 threads merges 4 heads; each thread owns 8 dims (16-byte loads).
constexpr int kCombHeads = 4;

template <typename E>
__global__ __launch_bounds__(256) void k_attend_combine(int Hq, int Dl, int nsplit, int64_t nbh,
                                                        const bf16* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        E* __restrict__ out,
                                                        float* __restrict__ lse) {
    extern __shared__ float wsh[];          // [kCombHeads][nsplit] weights
    __shared__ float tot_sh[kCombHeads];
    const int wave = threadIdx.x >> 6;      // one head per wave
    const int lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * kCombHeads + wave;   // (b*T + t)*Hq + h
    if (bh >= nbh) return;
    const int h = (int)(bh % Hq);
    const int64_t bt = bh / Hq;
    float* w = wsh + wave * nsplit;
    float M = -INFINITY;
    for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, part_lse[(bt * nsplit + s) * Hq + h]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float tot = 0.0f;
    for (int s = lane; s < nsplit; s += 64) {
        const float ls = part_lse[(bt * nsplit + s) * Hq + h];
        const float wgt = (ls == -INFINITY) ? 0.0f : expf(ls - M);
        w[s] = wgt;
        tot += wgt;
    }
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane == 0 && lse) lse[bh] = tot > 0.0f ? M + logf(tot) : -INFINITY;
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    // every lane of the wave wrote its own weights; the wave reads them all
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): LDS writes visible to the wave
    const int64_t stride = (int64_t)Hq * Dl;
    for (int d = 8 * lane; d < Dl; d += 8 * 64) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        const bf16* po = part_o + (bt * nsplit * Hq + h) * (int64_t)Dl + d;
        int s = 0;
        for (; s + 4 <= nsplit; s += 4) {
            bf16x8 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load8(po + (s + u) * stride);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] += w[s + u] * (float)v[u][j];
        }
        for (; s < nsplit; ++s) {
            const bf16x8 v = load8(po + s * stride);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += w[s] * (float)v[j];
        }
        E* o = out + bh * Dl + d;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (E)(acc[j] * inv);
    }
}

// Vector path: one workgroup per (b, t, h); any Dl <= 1024, fp32 or bf16.
template <typename E>
__global__ __launch_bounds__(256) void k_attend_vector(
    const E* __restrict__ qa, int T, int Hq, int Dl, const E* __restrict__ latent,
    const int64_t* __restrict__ latent_row_start, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ topk_count, int k, const E* __restrict__ hca,
    const int64_t* __restrict__ hca_row_start, const int32_t* __restrict__ hca_count,
    int64_t max_hca, float scale, E* __restrict__ out, float* __restrict__ lse) {
    __shared__ float red[4];
    const int h = blockIdx.x % Hq;
    const int64_t bt = blockIdx.x / Hq;
    const int b = (int)(bt / T);
    const int ntop = min(topk_count[b], k);
    const int nh = hca ? (int)min((int64_t)hca_count[b], max_hca) : 0;
    const int n = ntop + nh;
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca ? hca_row_start[b] : 0;
    const int32_t* idx = topk_idx + (int64_t)b * k;
    const E* qrow = qa + (bt * Hq + h) * Dl;
    float qv[4], ov[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = threadIdx.x + 256 * i;
        qv[i] = d < Dl ? (float)qrow[d] : 0.0f;
        ov[i] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int j = 0; j < n; ++j) {
        const E* row = att_row<E>(j, ntop, n, latent, lrs, idx, hca, hrs, Dl);
        float rv[4];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = threadIdx.x + 256 * i;
            rv[i] = d < Dl ? (float)row[d] : 0.0f;
            part += qv[i] * rv[i];
        }
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
        __syncthreads();
        const float logit = (red[0] + red[1] + red[2] + red[3]) * scale;
        const float mn = fmaxf(m, logit);
        const float a = expf(m - mn);
        const float p = expf(logit - mn);
        l = l * a + p;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = ov[i] * a + p * rv[i];
        m = mn;
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = threadIdx.x + 256 * i;
        if (d < Dl) out[(bt * Hq + h) * Dl + d] = (E)(ov[i] * inv);
    }
    if (threadIdx.x == 0 && lse) lse[bt * Hq + h] = l > 0.0f ? m + logf(l) : -INFINITY;
}

// Split heuristic shared by the launch and the workspace query: groups of kMQ
// query rows, then enough row splits to give ~kAttWGTarget workgroups, keeping
// at least two row chunks per split.
struct AttendPlan {
    int QG;
    int nsplit;
    int rows_per_split;
    int n_items;
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
    return AttendPlan{QG, (int)ns, (int)rps, (int)(units * ns)};
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
    const size_t n = (size_t)B * T * p.nsplit * Hq;
    return n * Dl * sizeof(bf16) + n * sizeof(float);
}

extern "C" int lsa_sparse_attend(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                                 const void* latent, const int64_t* latent_row_start,
                                 const int32_t* topk_idx, const int32_t* topk_count, int k,
                                 const void* hca, const int64_t* hca_row_start,
                                 const int32_t* hca_count, int64_t max_hca, float scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    clear_error();
    if (!qa || !latent || !latent_row_start || !topk_idx || !topk_count || !out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: a required pointer is NULL");
    if (hca && (!hca_row_start || !hca_count))
        return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: hca given without row starts/counts");
    if (B <= 0 || T <= 0 || Hq <= 0 || Dl <= 0 || k <= 0 || (hca && max_hca < 0))
        return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: B=%d T=%d Hq=%d Dl=%d k=%d", B, T, Hq,
                    Dl, k);
    if (dtype != LSA_DTYPE_F32 && dtype != LSA_DTYPE_BF16)
        return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: unknown dtype %d", dtype);
    if (!aligned16(qa) || !aligned16(latent) || (hca && !aligned16(hca)))
        return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: qa/latent/hca must be 16-byte aligned");
    if (!(scale == scale)) return fail(LSA_ERR_INVALID_ARG, "lsa_sparse_attend: scale is NaN");
    if (Dl > 1024) return fail(LSA_ERR_UNSUPPORTED, "lsa_sparse_attend: Dl=%d > 1024", Dl);
    if (B > 65535 || T > 65535)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_sparse_attend: B or T above 65535");
    if ((int64_t)k + (hca ? max_hca : 0) > (int64_t)1 << 30)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_sparse_attend: too many attended rows");
    const int64_t hmax = hca ? max_hca : 0;
    const size_t need = lsa_attend_workspace(dtype, B, T, Hq, Dl, k, hmax);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(LSA_ERR_WORKSPACE, "lsa_sparse_attend: workspace %zu < %zu bytes",
                    workspace_bytes, need);
    int rc = check_device(nullptr);
    if (rc != LSA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;

    if (attend_mfma_shape(dtype, Hq, Dl)) {
        const AttendPlan p = attend_plan(B, T, Hq, k, hmax);
        const size_t n = (size_t)B * T * p.nsplit * Hq;
        bf16* part_o = (bf16*)workspace;
        float* part_lse = p.nsplit > 1 ? (float*)(part_o + n * Dl) : nullptr;
        const unsigned grid = (unsigned)(8 * ((p.n_items + 7) / 8));
        const float sl2 = scale * kLog2e;
        const int M = T * Hq;
        // Without an HCA pool the kernel reads valid stand-ins and attends zero
        // HCA rows (max_hca = 0), so it never branches on the pool.
        const void* hp = hca ? hca : latent;
        const int64_t* hrs_p = hca ? hca_row_start : latent_row_start;
        const int32_t* hcnt_p = hca ? hca_count : topk_count;
#define LSA_ATT(dl)                                                                            \
    hipLaunchKernelGGL((k_attend_mfma<dl, kAttRing>), dim3(grid), dim3(512), 0, st,             \
                       p.n_items, p.QG, p.nsplit, p.rows_per_split, M, k, topk_idx,             \
                       (const bf16*)qa, topk_count, hcnt_p, latent_row_start, hrs_p, hmax,      \
                       (const bf16*)latent, (const bf16*)hp, sl2, (bf16*)out, lse, part_o,      \
                       part_lse)
        if (Dl == 512) LSA_ATT(512); else if (Dl == 256) LSA_ATT(256); else LSA_ATT(128);
#undef LSA_ATT
        rc = launch_status("attend_mfma");
        if (rc != LSA_OK || p.nsplit == 1) return rc;
        // partials are laid out [b][split][query row]: merge with M = T * Hq rows per b
        const int64_t nbh = (int64_t)B * M;
        hipLaunchKernelGGL(k_attend_combine<bf16>,
                           dim3((unsigned)((nbh + kCombHeads - 1) / kCombHeads)), dim3(256),
                           sizeof(float) * kCombHeads * p.nsplit, st, M, Dl, p.nsplit, nbh,
                           part_o, part_lse, (bf16*)out, lse);
        return launch_status("attend_combine");
    }
    const unsigned blocks = (unsigned)((int64_t)B * T * Hq);
    if (dtype == LSA_DTYPE_F32)
        hipLaunchKernelGGL(k_attend_vector<float>, dim3(blocks), dim3(256), 0, st,
                           (const float*)qa, T, Hq, Dl, (const float*)latent, latent_row_start,
                           topk_idx, topk_count, k, (const float*)hca, hca_row_start, hca_count,
                           hmax, scale, (float*)out, lse);
    else
        hipLaunchKernelGGL(k_attend_vector<bf16>, dim3(blocks), dim3(256), 0, st, (const bf16*)qa,
                           T, Hq, Dl, (const bf16*)latent, latent_row_start, topk_idx, topk_count,
                           k, (const bf16*)hca, hca_row_start, hca_count, hmax, scale, (bf16*)out,
                           lse);
    return launch_status("attend_vector");
}
