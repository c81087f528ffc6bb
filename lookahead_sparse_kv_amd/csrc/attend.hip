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
//   workgroup = one (b, t, split); its NW waves split the latent dimension,
//   wave w owning dims [w*DPW, (w+1)*DPW) (8 waves x 64 dims for Dl = 512).  Per chunk of 32 attended rows:
//     1. each wave loads its DPW-wide slice of the 32 rows straight into
//        registers (B operand of Q.K^T, K = its dims), two chunks in flight;
//     2. partial logits S_w = Q[:, dims_w] . C[:, dims_w]^T (64 heads x 32);
//     3. the NW partial logits meet in LDS; wave w finishes the softmax of
//        64/NW heads (online, base-2, lazily rescaled) and publishes P (bf16)
//        and the rescale factors;
//     4. O[:, dims_w] += P . C[:, dims_w] with C re-read transposed from the
//        wave's private LDS copy of its slice.
//   The row slice each wave needs for P.V is exactly the slice it loaded, so
//   only the small logit tiles cross waves.  Rows are split across
//   workgroups when B*T is small; a combine kernel merges the splits by their
//   log-sum-exp.
#include "common.hpp"

namespace lsa {

constexpr int kAttWGTarget = 256;   // workgroups the split heuristic aims for
constexpr int kChunk = 32;          // attended rows per step
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

template <int NW, int DPW>
__global__ __launch_bounds__(NW * 64) void k_attend_mfma(
    const bf16* __restrict__ qa, int T, int Hq, const bf16* __restrict__ latent,
    const int64_t* __restrict__ latent_row_start, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ topk_count, int k, const bf16* __restrict__ hca,
    const int64_t* __restrict__ hca_row_start, const int32_t* __restrict__ hca_count,
    int64_t max_hca, float scale_log2, int rows_per_split, int nsplit, bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int Dl = NW * DPW;
    constexpr int KDT = DPW / 32;           // k-steps of Q.K^T over the wave's dims
    constexpr int NDT = DPW / 16;           // 16-wide dim tiles of P.V
    constexpr int CROW = DPW + 4;           // bf16 per staged row (8-byte pad)
    constexpr int SROW = 36;                // floats per head row of a partial-logit tile
    constexpr int PROW = 40;                // bf16 per head row of P
    constexpr int HPW = 64 / NW;            // heads whose softmax a wave finishes
    constexpr int RPL = kChunk * HPW / 64;  // rows per lane in that softmax
    static_assert(KDT >= 1 && NDT >= 1 && RPL >= 1 && RPL <= 8, "unsupported tiling");

    __shared__ __attribute__((aligned(16))) bf16 cbuf[NW][kChunk * CROW];
    __shared__ __attribute__((aligned(16))) float sbuf[NW][64 * SROW];
    __shared__ __attribute__((aligned(16))) bf16 pbuf[64 * PROW];
    __shared__ __attribute__((aligned(16))) float abuf[64];
    __shared__ float mlbuf[2][64];

    const int split = blockIdx.x;
    const int t = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;
    const int g = lane >> 4;
    const int si = lane % HPW;              // softmax: head 8*wave + si (NW = 8)
    const int sr = (lane / HPW) * RPL;      // softmax: first row of this lane

    const int ntop = min(topk_count[b], k);
    const int nh = hca ? (int)min((int64_t)hca_count[b], max_hca) : 0;
    const int n = ntop + nh;
    const int rs = split * rows_per_split;
    const int re = min(n, rs + rows_per_split);
    const int64_t lrs = latent_row_start[b];
    const int64_t hrs = hca ? hca_row_start[b] : 0;
    const int32_t* idx = topk_idx + (int64_t)b * k;
    const int64_t bt = (int64_t)b * T + t;
    const int dim0 = wave * DPW;

    // Q fragments: A operand, heads 16ht + n16, dims dim0 + 32kk + 8g.
    bf16x8 qf[4][KDT];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int h = 16 * ht + n16;
#pragma unroll
        for (int kk = 0; kk < KDT; ++kk)
            qf[ht][kk] = h < Hq ? load8(qa + (bt * Hq + h) * Dl + dim0 + 32 * kk + 8 * g) : zero8();
    }
    f32x4 o[4][NDT];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) o[ht][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;   // running max (base 2) of head HPW*wave + si
    float l_run = 0.0f;

    auto load_chunk = [&](int r0, bf16x8 (&kb)[2][KDT]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int j = r0 + 16 * c + n16;
            const bf16* p = (j < re) ? att_row<bf16>(j, ntop, n, latent, lrs, idx, hca, hrs, Dl)
                                     : nullptr;
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk)
                kb[c][kk] = p ? load8(p + dim0 + 32 * kk + 8 * g) : zero8();
        }
    };

    bf16* cw = cbuf[wave];
    auto process = [&](int r0, bf16x8 (&kb)[2][KDT]) {
        // partial logits over this wave's dims
        f32x4 sp[4][2];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int c = 0; c < 2; ++c) sp[ht][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KDT; ++kk)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int c = 0; c < 2; ++c) sp[ht][c] = mfma16(qf[ht][kk], kb[c][kk], sp[ht][c]);
        // stage the row slice (row-major) for the transposed reads of P.V
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < KDT; ++kk) {
                bf16* dst = cw + (16 * c + n16) * CROW + 32 * kk + 8 * g;
                const u32x4 v = __builtin_bit_cast(u32x4, kb[c][kk]);
                *reinterpret_cast<uint2*>(dst) = make_uint2(v[0], v[1]);
                *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v[2], v[3]);
            }
        float* sw = sbuf[wave];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int v = 0; v < 4; ++v) sw[(16 * ht + 4 * g + v) * SROW + 16 * c + n16] = sp[ht][c][v];
        __syncthreads();

        // softmax of heads HPW*wave .. +HPW-1: lane holds head HPW*wave + si, rows sr .. sr+RPL-1
        {
            const int h = HPW * wave + si;
            float x[RPL];
#pragma unroll
            for (int j = 0; j < RPL; ++j) x[j] = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
#pragma unroll
                for (int j4 = 0; j4 < RPL; j4 += 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(&sbuf[w2][h * SROW + sr + j4]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j4 + j] += a[j];
                }
            }
            float cmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                x[j] = (r0 + sr + j < re) ? x[j] * scale_log2 : -INFINITY;
                cmax = fmaxf(cmax, x[j]);
            }
#pragma unroll
            for (int off = HPW; off < 64; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
            float alpha = 1.0f;
            if (cmax > m_ref + kRescaleSlack || (m_ref == -INFINITY && cmax != -INFINITY)) {
                alpha = (m_ref == -INFINITY) ? 0.0f : exp2f(m_ref - cmax);
                m_ref = cmax;
            }
            float psum = 0.0f;
            bf16 pv[RPL];
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const float p = (m_ref == -INFINITY) ? 0.0f : exp2f(x[j] - m_ref);
                pv[j] = (bf16)p;
                psum += (float)pv[j];
            }
#pragma unroll
            for (int off = HPW; off < 64; off <<= 1) psum += __shfl_xor(psum, off);
            l_run = alpha * l_run + psum;
#pragma unroll
            for (int j = 0; j < RPL; ++j) pbuf[h * PROW + sr + j] = pv[j];
            if (sr == 0) abuf[h] = alpha;
        }
        __syncthreads();

        // rescale O rows whose head max moved
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(&abuf[16 * ht + 4 * g]);
            if (al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f) {
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[ht][nt][v] *= al[v];
            }
        }
        // O[:, dims_w] += P . C[:, dims_w]
        bf16x8 pa[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
            pa[ht] = *reinterpret_cast<const bf16x8*>(&pbuf[(16 * ht + n16) * PROW + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) {
            bf16x8 cb;
            const bf16* src = cw + (8 * g) * CROW + 16 * nt + n16;
#pragma unroll
            for (int j = 0; j < 8; ++j) cb[j] = src[j * CROW];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) o[ht][nt] = mfma16(pa[ht], cb, o[ht][nt]);
        }
    };

    const int nchunks = re > rs ? (re - rs + kChunk - 1) / kChunk : 0;
    bf16x8 kbA[2][KDT], kbB[2][KDT];
    if (nchunks > 0) load_chunk(rs, kbA);
    if (nchunks > 1) load_chunk(rs + kChunk, kbB);
    for (int c = 0; c < nchunks; c += 2) {
        process(rs + c * kChunk, kbA);
        if (c + 2 < nchunks) load_chunk(rs + (c + 2) * kChunk, kbA);
        if (c + 1 >= nchunks) break;
        process(rs + (c + 1) * kChunk, kbB);
        if (c + 3 < nchunks) load_chunk(rs + (c + 3) * kChunk, kbB);
    }

    // publish (m, l) of this wave's heads; every wave normalises its O rows
    if (sr == 0) {
        mlbuf[0][HPW * wave + si] = m_ref;
        mlbuf[1][HPW * wave + si] = l_run;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int h = 16 * ht + 4 * g + v;
            if (h >= Hq) continue;
            const float l = mlbuf[1][h];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            if (nsplit == 1) {
                bf16* orow = out + (bt * Hq + h) * Dl + dim0;
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt) orow[16 * nt + n16] = (bf16)(o[ht][nt][v] * inv);
            } else {
                float* prow = part_o + ((bt * nsplit + split) * Hq + h) * Dl + dim0;
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt) prow[16 * nt + n16] = o[ht][nt][v] * inv;
            }
        }
    if (wave == 0) {
        for (int h = lane; h < Hq; h += 64) {
            const float l = mlbuf[1][h];
            const float m = mlbuf[0][h];
            const float v = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
            if (nsplit == 1) {
                if (lse) lse[bt * Hq + h] = v;
            } else {
                part_lse[(bt * nsplit + split) * Hq + h] = v;
            }
        }
    }
}

// Merge split partials (o_s normalised, lse_s) of one (b, t, h).
template <typename E>
__global__ __launch_bounds__(256) void k_attend_combine(int Hq, int Dl, int nsplit,
                                                        const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        E* __restrict__ out,
                                                        float* __restrict__ lse) {
    const int64_t bt = blockIdx.x;
    const int h = blockIdx.y;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_lse[(bt * nsplit + s) * Hq + h]);
    float wsum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
        const float ls = part_lse[(bt * nsplit + s) * Hq + h];
        wsum += (M == -INFINITY) ? 0.0f : expf(ls - M);
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    for (int d = threadIdx.x; d < Dl; d += blockDim.x) {
        float acc = 0.0f;
        for (int s = 0; s < nsplit; ++s) {
            const float ls = part_lse[(bt * nsplit + s) * Hq + h];
            if (ls == -INFINITY) continue;
            acc += expf(ls - M) * part_o[((bt * nsplit + s) * Hq + h) * Dl + d];
        }
        out[(bt * Hq + h) * Dl + d] = (E)(acc * inv);
    }
    if (threadIdx.x == 0 && lse) lse[bt * Hq + h] = wsum > 0.0f ? M + logf(wsum) : -INFINITY;
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

// Split heuristic shared by the launch and the workspace query.
struct AttendPlan {
    int nsplit;
    int rows_per_split;
};

static AttendPlan attend_plan(int B, int T, int k, int64_t max_hca) {
    const int64_t rows = (int64_t)k + (max_hca > 0 ? max_hca : 0);
    const int64_t pairs = (int64_t)B * T;
    int64_t ns = (kAttWGTarget + pairs - 1) / pairs;
    const int64_t max_ns = (rows + 2 * kChunk - 1) / (2 * kChunk);  // >= 2 chunks per split
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    int64_t rps = (rows + ns - 1) / ns;
    rps = (rps + kChunk - 1) / kChunk * kChunk;
    if (rps < kChunk) rps = kChunk;
    ns = (rows + rps - 1) / rps;
    if (ns < 1) ns = 1;
    return AttendPlan{(int)ns, (int)rps};
}

static bool attend_mfma_shape(int dtype, int Hq, int Dl) {
    return dtype == LSA_DTYPE_BF16 && Hq <= 64 && (Dl == 128 || Dl == 256 || Dl == 512);
}

}  // namespace lsa

using namespace lsa;

size_t lsa_attend_workspace(int dtype, int B, int T, int Hq, int Dl, int k, int64_t max_hca) {
    if (!attend_mfma_shape(dtype, Hq, Dl)) return 0;
    const AttendPlan p = attend_plan(B, T, k, max_hca);
    if (p.nsplit <= 1) return 0;
    return sizeof(float) * (size_t)B * T * p.nsplit * Hq * (size_t)(Dl + 1);
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
        const AttendPlan p = attend_plan(B, T, k, hmax);
        float* part_o = (float*)workspace;
        float* part_lse = p.nsplit > 1 ? part_o + (size_t)B * T * p.nsplit * Hq * Dl : nullptr;
        dim3 grid((unsigned)p.nsplit, (unsigned)T, (unsigned)B);
        const float sl2 = scale * kLog2e;
#define LSA_ATT(nw, dpw)                                                                      \
    hipLaunchKernelGGL((k_attend_mfma<nw, dpw>), grid, dim3(nw * 64), 0, st, (const bf16*)qa, T, \
                       Hq, (const bf16*)latent, latent_row_start, topk_idx, topk_count, k,         \
                       (const bf16*)hca, hca_row_start, hca_count, hmax, sl2,                      \
                       p.rows_per_split, p.nsplit, (bf16*)out, lse, part_o, part_lse)
        if (Dl == 512) LSA_ATT(8, 64); else if (Dl == 256) LSA_ATT(8, 32); else LSA_ATT(4, 32);
#undef LSA_ATT
        rc = launch_status("attend_mfma");
        if (rc != LSA_OK || p.nsplit == 1) return rc;
        hipLaunchKernelGGL(k_attend_combine<bf16>, dim3((unsigned)(B * T), (unsigned)Hq),
                           dim3(256), 0, st, Hq, Dl, p.nsplit, part_o, part_lse, (bf16*)out, lse);
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
