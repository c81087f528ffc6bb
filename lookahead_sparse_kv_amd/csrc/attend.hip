// attend.hip -- lsa_sparse_attend: core attention over the chosen entries plus every HCA entry.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1: the heavily compressed
// (HCA, 128:1) entries are all retained, and the final core attention runs
// over the top-k entries chosen inside the fetched subset.  Each compressed
// entry carries one latent row that serves as key and value for all query
// heads (multi-query form over a shared latent).
//
// Matrix-core kernel (bf16, Hq <= 64, Dl = NW * DPW):
//   workgroup = one (b, t, group of 32 query heads, row split); its NW waves
//   split the latent dimension, wave w owning dims [w*DPW, (w+1)*DPW)
//   (8 waves x 64 dims for Dl = 512: two waves per SIMD hide each other's
//   latencies).  Per chunk of 32 attended rows:
//     1. each wave copies its DPW-wide slice of the 32 rows from HBM straight
//        into an LDS ring slot (direct-to-LDS loads, 2-3 chunks in flight);
//     2. partial logits S_w = Q[:, dims_w] . C[:, dims_w]^T (64 heads x 32);
//     3. the partial logits of the NW waves meet in LDS; each wave finishes
//        the softmax of 32/NW heads (online, base-2, lazily rescaled) and
//        publishes P (bf16) and the rescale factors;
//     4. O[:, dims_w] += P . C[:, dims_w] with C read transposed from the same
//        slot (transposing LDS reads).
//   The row slice each wave needs for P.V is exactly the slice it loaded, so
//   only the small logit tiles cross waves.  Rows are split across
//   workgroups when B*T is small; a combine kernel merges the splits by their
//   log-sum-exp.
#include "common.hpp"

namespace lsa {

constexpr int kAttWGTarget = 256;   // workgroups the split heuristic aims for
constexpr int kChunk = 32;          // attended rows per step
constexpr int kIdxWin = 128;        // row pointers staged in LDS at a time (multiple of kChunk)
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
    if (slot >= per_xcd) return -1;
    const int item = (blockIdx.x & 7) * per_xcd + slot;
    return item < n_items ? item : -1;
}

// 16-byte slot swizzle of a staged row slice (CH slots per row).  For 16- and
// 8-slot rows it makes two access patterns conflict-free: 16 consecutive rows
// reading one logical slot (the Q.K^T operand) and the 8 rows
// {j, j+8 : j in 4h..4h+3} reading one slot pair (the transposing P.V reads).
template <int CH>
__device__ __forceinline__ int slot_swz(int r) {
    if constexpr (CH == 16) {
        return 2 * ((r & 3) + 4 * ((r >> 3) & 1)) + ((r >> 2) & 1);
    } else if constexpr (CH == 8) {
        // two rows per 64 banks: the slot must differ among rows of equal parity
        return (((r >> 1) & 1) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 2);
    } else {
        return 0;
    }
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

template <int NW, int DPW, int HT>
__global__ __launch_bounds__(NW * 64, 2) void k_attend_mfma(
    const bf16* __restrict__ qa, int T, int Hq, const bf16* __restrict__ latent,
    const int64_t* __restrict__ latent_row_start, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ topk_count, int k, const bf16* __restrict__ hca,
    const int64_t* __restrict__ hca_row_start, const int32_t* __restrict__ hca_count,
    int64_t max_hca, float scale_log2, int HG, int nsplit, int rows_per_split, int n_items,
    bf16* __restrict__ out, float* __restrict__ lse, bf16* __restrict__ part_o,
    float* __restrict__ part_lse) {
    constexpr int Dl = NW * DPW;
    constexpr int KDT = DPW / 32;           // k-steps of Q.K^T over the wave's dims
    constexpr int NDT = DPW / 16;           // 16-wide dim tiles of P.V
    constexpr int CH = DPW / 8;             // 16-byte slots per row slice
    constexpr int SLICE = kChunk * DPW;     // bf16 per wave per ring slot
    constexpr int NBUF = NW >= 8 ? 3 : 4;   // ring depth (LDS: slots + partial logits <= 160 KiB)
    constexpr int RPI = 64 / CH;            // rows per DMA instruction
    constexpr int DMA = kChunk / RPI;       // DMA instructions per wave per chunk
    constexpr int SROW = 36;                // floats per head row of a partial-logit tile
    constexpr int PROW = 40;                // bf16 per head row of P
    constexpr int MH = 16 * HT;             // query heads per workgroup
    constexpr int HPW = MH / NW;            // heads whose softmax one wave finishes
    constexpr int RG = 64 / HPW;            // lanes sharing one head in that softmax
    constexpr int RPL = kChunk / RG;        // rows per lane in that softmax
    static_assert(KDT >= 1 && (RPL == 2 || RPL == 4) && (RG == 8 || RG == 16), "tiling");
    static_assert(DMA * NBUF < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) bf16 cring[NBUF][NW][SLICE];
    __shared__ __attribute__((aligned(16))) float sbuf[NW][MH * SROW];
    __shared__ __attribute__((aligned(16))) bf16 pbuf[MH * PROW];
    __shared__ __attribute__((aligned(16))) float abuf[MH];
    __shared__ float mlbuf[2][MH];
    __shared__ const bf16* sptr[kIdxWin];   // row pointers of a window of this split's rows

    const int item = xcd_item(n_items);
    if (item < 0) return;
    const int hg = item % HG;
    const int split = (item / HG) % nsplit;
    const int64_t bt = item / (HG * nsplit);
    const int b = (int)(bt / T);
    const int h0 = hg * MH;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;
    const int g = lane >> 4;
    const int si = lane / RG;               // softmax: local head HPW*wave + si
    const int sr = (lane % RG) * RPL;       // softmax: first row of this lane

    const int ntop = min(topk_count[b], k);
    const int nh = hca ? (int)min((int64_t)hca_count[b], max_hca) : 0;
    const int n = ntop + nh;
    const int rs = split * rows_per_split;
    const int re = min(n, rs + rows_per_split);
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca ? hca_row_start[b] : 0;
    const int32_t* idx = topk_idx + (int64_t)b * k;
    const int dim0 = wave * DPW;
    const int nchunks = re > rs ? (re - rs + kChunk - 1) / kChunk : 0;

    // Q fragments: A operand, heads h0 + 16ht + n16, dims dim0 + 32kk + 8g.
    bf16x8 qf[HT][KDT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
#pragma unroll
        for (int kk = 0; kk < KDT; ++kk)
            qf[ht][kk] = h < Hq ? load8(qa + (bt * Hq + h) * Dl + dim0 + 32 * kk + 8 * g) : zero8();
    }
    f32x4 o[HT][NDT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) o[ht][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;   // running max (base 2) of local head HPW*wave + si
    float l_run = 0.0f;

    // Row pointers of rows [win0, win0 + kIdxWin) staged in LDS; rows past the
    // split end point at its last row (finite data, probability zero).
    int win0 = -kIdxWin;
    auto stage_window = [&](int w0) {
        __syncthreads();
        for (int i = tid; i < kIdxWin; i += NW * 64) {
            const int j = min(w0 + i, re - 1);
            sptr[i] = j < ntop ? latent + (lrs + idx[j]) * Dl : hca + (hrs + (j - ntop)) * Dl;
        }
        __syncthreads();
        win0 = w0;
    };
    // DMA of this wave's slice of chunk c into ring slot c % NBUF: instruction i
    // moves rows RPI*i .. RPI*i+RPI-1, lane L filling physical slot L % CH of row
    // RPI*i + L / CH with logical slot (L % CH) ^ swz(row).
    auto issue_chunk = [&](int c) {
        const int r0 = rs + c * kChunk;
        if (min(r0 + kChunk, re) > win0 + kIdxWin) stage_window(r0);
        bf16* slot = &cring[c % NBUF][wave][0];
#pragma unroll
        for (int i = 0; i < DMA; ++i) {
            const int rl = RPI * i + lane / CH;
            const int ps = lane % CH;
            const bf16* src = sptr[min(r0 + rl, re - 1) - win0] + dim0 + 8 * (ps ^ slot_swz<CH>(rl));
            __builtin_amdgcn_global_load_lds(
                (const void*)src, (__attribute__((address_space(3))) void*)(slot + RPI * i * DPW),
                16, 0, 0);
        }
    };

    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    auto process = [&](int c) {
        const int r0 = rs + c * kChunk;
        const bf16* slot = &cring[c % NBUF][wave][0];
        // partial logits over this wave's dims; B operands from the staged slice
        f32x4 sp[HT][2];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) sp[ht][c2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            const int r = 16 * c2 + n16;
            const int sw = slot_swz<CH>(r);
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) {
                const bf16x8 kb = *reinterpret_cast<const bf16x8*>(slot + r * DPW + 8 * ((4 * kk + g) ^ sw));
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) sp[ht][c2] = mfma16(qf[ht][kk], kb, sp[ht][c2]);
            }
        }
        float* swb = sbuf[wave];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int v = 0; v < 4; ++v) swb[(16 * ht + 4 * g + v) * SROW + 16 * c2 + n16] = sp[ht][c2][v];
        __syncthreads();

        // softmax of local head HPW*wave + si over rows sr .. sr+3 of this chunk
        {
            const int h = HPW * wave + si;
            float x[RPL];
#pragma unroll
            for (int j = 0; j < RPL; ++j) x[j] = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                if constexpr (RPL == 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(&sbuf[w2][h * SROW + sr]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] += a[j];
                } else {
                    const float2 a = *reinterpret_cast<const float2*>(&sbuf[w2][h * SROW + sr]);
                    x[0] += a.x;
                    x[1] += a.y;
                }
            }
            float cmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                x[j] = (r0 + sr + j < re) ? x[j] * scale_log2 : -INFINITY;
                cmax = fmaxf(cmax, x[j]);
            }
            cmax = group_max<RG>(cmax);
            float alpha = 1.0f;
            if (cmax > m_ref + kRescaleSlack || (m_ref == -INFINITY && cmax != -INFINITY)) {
                alpha = (m_ref == -INFINITY) ? 0.0f : exp2f(m_ref - cmax);
                m_ref = cmax;
            }
            float psum = 0.0f;
            typedef __bf16 bf16xR __attribute__((ext_vector_type(RPL)));
            bf16xR pv;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const float p = (m_ref == -INFINITY) ? 0.0f : exp2f(x[j] - m_ref);
                pv[j] = (bf16)p;
                psum += (float)pv[j];
            }
            psum = group_sum<RG>(psum);
            l_run = alpha * l_run + psum;
            *reinterpret_cast<bf16xR*>(&pbuf[h * PROW + sr]) = pv;
            if (sr == 0) abuf[h] = alpha;
        }
        __syncthreads();

        // rescale O rows whose head max moved
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(&abuf[16 * ht + 4 * g]);
            if (al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f) {
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[ht][nt][v] *= al[v];
            }
        }
        // O[:, dims_w] += P . C[:, dims_w]; C^T operands come from transposing LDS reads:
        // in each 16-lane group, lanes 4j..4j+3 point at row (8g + j) (4 dims each) and
        // lane i receives dim i of those 4 rows.
        bf16x8 pa[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            pa[ht] = *reinterpret_cast<const bf16x8*>(&pbuf[(16 * ht + n16) * PROW + 8 * g]);
        const int trow0 = 8 * g + (n16 >> 2);
        const int trow1 = trow0 + 4;
        const int sw0 = slot_swz<CH>(trow0), sw1 = slot_swz<CH>(trow1);
        const int q4 = n16 & 3;
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
            const int ls = 2 * nt + (q4 >> 1);       // logical 16-byte slot
            const int off = 4 * (q4 & 1);            // bf16 offset inside the slot
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(slot + trow0 * DPW + 8 * (ls ^ sw0) + off));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(slot + trow1 * DPW + 8 * (ls ^ sw1) + off));
            bf16x8 cb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cb[j] = lo[j];
                cb[4 + j] = hi[j];
            }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) o[ht][nt] = mfma16(pa[ht], cb, o[ht][nt]);
        }
    };

    // Pipeline: chunks c+1 .. c+NBUF-1 are in flight while chunk c is processed.
#pragma unroll
    for (int c = 0; c < NBUF - 1; ++c)
        if (c < nchunks) issue_chunk(c);
    for (int c = 0; c < nchunks; ++c) {
        // refill the slot of chunk c-1 (its last reads were in the previous step)
        // before waiting, so the address work overlaps the wait and Q.K^T
        if (c + NBUF - 1 < nchunks) issue_chunk(c + NBUF - 1);
        const int after = min(nchunks - 1, c + NBUF - 1) - c;   // chunks issued after c
        if (after >= 3) wait_vmcnt<3 * DMA>();
        else if (after == 2) wait_vmcnt<2 * DMA>();
        else if (after == 1) wait_vmcnt<DMA>();
        else wait_vmcnt<0>();
        process(c);
    }

    // publish (m, l) of this wave's heads; every wave normalises its O rows
    if (sr == 0) {
        mlbuf[0][HPW * wave + si] = m_ref;
        mlbuf[1][HPW * wave + si] = l_run;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int hl = 16 * ht + 4 * g + v;
            const int h = h0 + hl;
            if (h >= Hq) continue;
            const float l = mlbuf[1][hl];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            bf16* orow = (nsplit == 1) ? out + (bt * Hq + h) * Dl + dim0
                                       : part_o + ((bt * nsplit + split) * Hq + h) * Dl + dim0;
#pragma unroll
            for (int nt = 0; nt < NDT; ++nt) orow[16 * nt + n16] = (bf16)(o[ht][nt][v] * inv);
        }
    if (tid < MH) {
        const int h = h0 + tid;
        if (h < Hq) {
            const float l = mlbuf[1][tid];
            const float v = l > 0.0f ? (mlbuf[0][tid] + log2f(l)) * kLn2 : -INFINITY;
            if (nsplit == 1) {
                if (lse) lse[bt * Hq + h] = v;
            } else {
                part_lse[(bt * nsplit + split) * Hq + h] = v;
            }
        }
    }
}

// Merge the split partials: o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M) per
// (b, t, h); the partial o_s are normalised per split and stored in bf16.
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

// Split heuristic shared by the launch and the workspace query: head groups of
// kMH heads, then enough row splits to give ~kAttWGTarget workgroups, keeping
// at least two row chunks per split.
constexpr int kMH = 32;

struct AttendPlan {
    int HG;
    int nsplit;
    int rows_per_split;
    int n_items;
};

static AttendPlan attend_plan(int B, int T, int Hq, int k, int64_t max_hca) {
    const int64_t rows = (int64_t)k + (max_hca > 0 ? max_hca : 0);
    const int HG = (Hq + kMH - 1) / kMH;
    const int64_t units = (int64_t)B * T * HG;
    int64_t ns = (kAttWGTarget + units - 1) / units;
    const int64_t max_ns = (rows + 2 * kChunk - 1) / (2 * kChunk);
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    int64_t rps = (rows + ns - 1) / ns;
    rps = (rps + kChunk - 1) / kChunk * kChunk;
    if (rps < kChunk) rps = kChunk;
    ns = (rows + rps - 1) / rps;
    if (ns < 1) ns = 1;
    return AttendPlan{HG, (int)ns, (int)rps, (int)(units * ns)};
}

static bool attend_mfma_shape(int dtype, int Hq, int Dl) {
    return dtype == LSA_DTYPE_BF16 && Hq <= 64 && (Dl == 128 || Dl == 256 || Dl == 512);
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
#define LSA_ATT(nw, dpw)                                                                        \
    hipLaunchKernelGGL((k_attend_mfma<nw, dpw, kMH / 16>), dim3(grid), dim3(nw * 64), 0, st,      \
                       (const bf16*)qa, T, Hq, (const bf16*)latent, latent_row_start, topk_idx,  \
                       topk_count, k, (const bf16*)hca, hca_row_start, hca_count, hmax, sl2,     \
                       p.HG, p.nsplit, p.rows_per_split, p.n_items, (bf16*)out, lse, part_o,     \
                       part_lse)
        if (Dl == 512) LSA_ATT(8, 64); else if (Dl == 256) LSA_ATT(4, 64); else LSA_ATT(4, 32);
#undef LSA_ATT
        rc = launch_status("attend_mfma");
        if (rc != LSA_OK || p.nsplit == 1) return rc;
        const int64_t nbh = (int64_t)B * T * Hq;
        hipLaunchKernelGGL(k_attend_combine<bf16>,
                           dim3((unsigned)((nbh + kCombHeads - 1) / kCombHeads)), dim3(256),
                           sizeof(float) * kCombHeads * p.nsplit, st, Hq, Dl, p.nsplit, nbh,
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
