// rescore.hip -- lsa_index_rescore: the native indexer's per-step score of the kept subset.
//
// Page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
// Lookahead Sparse Attention", Technical Summary 2.1 "Tiered Selection": inside
// the subset the Memory Indexer kept, the backbone's own (native) Lightning
// Indexer takes the fine-grained top-k; 2.3 "Decoupled Training": the
// compressed indexer keys are the backbone's frozen keys.  So the native
// indexer re-scores only the kept entries, against the same key rows, with its
// own per-step queries q' and weights w':
//     r[b,s] = sum_h w'[b,h] * max(0, <q'[b,h,:], k[b,s,:]>)
// a ranking logit (no bias, no sigmoid), written at r_out[entry_start[b] + s]
// for each candidate s, where lsa_topk reads its rank keys.
//
// Matrix-core kernel (bf16, H <= 64, D in {64, 128}): the decode score kernel
// in gather form.  A wave takes groups of 16 candidates; their indices are
// staged in LDS, and the 16 key rows of a group are copied from HBM into a
// wave-private LDS ring by buffer loads into LDS (base = the sequence's first
// key row, 32-bit byte offset per lane, range = its S_b rows, so an index
// outside the sequence reads no memory; its logit is not written), up to NB
// groups ahead.
// HBM-bound: 256 B of key row + 4 B of index + 4 B of logit per candidate.
#include "common.hpp"

namespace lsa {

constexpr int kRescoreRing = 3;          // LDS ring slots (groups of 16 rows) per wave
constexpr int kRescoreGroupsPerWave = 32;

// MFMA operands as in the decode score kernel: lane l, n = l%16 picks the
// candidate of the group, g = l/16 picks 8 of each 32 dims; A (queries) stays in
// registers; B (keys) for k-step kk is dims 32kk + 8g .. +7 of candidate n.
// Inside a staged row, 16-byte slot p holds logical slot p ^ (row & (SLOTS-1) & 15).
template <int MT, int KT>
__global__ __launch_bounds__(256) void k_rescore_mfma(
    const bf16* __restrict__ keys, const int64_t* __restrict__ key_row_start,
    const int32_t* __restrict__ seq_len, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ cand_idx, const int32_t* __restrict__ cand_count, int H,
    int64_t max_cand, const bf16* __restrict__ q, const float* __restrict__ w,
    float* __restrict__ r_out) {
    constexpr int D = 32 * KT;
    constexpr int SLOTS = D / 8;                 // 16-byte slots per key row
    constexpr int RPI = 64 / SLOTS;              // rows per copy instruction
    constexpr int DMAG = 16 / RPI;               // copy instructions per group of 16 rows
    constexpr int NB = kRescoreRing;
    constexpr int GPW = kRescoreGroupsPerWave;
    static_assert(SLOTS >= 8 && NB <= 4, "layout");
    // one LDS object: the rings, the staged candidate indices, the queries
    constexpr int OFF_IDX = 4 * NB * 16 * D * 2;
    constexpr int OFF_Q = OFF_IDX + 4 * GPW * 16 * 4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[OFF_Q + 64 * D * 2];
    bf16* const myring = reinterpret_cast<bf16*>(lds) + (threadIdx.x >> 6) * (NB * 16 * D);
    int* const myidx = reinterpret_cast<int*>(lds + OFF_IDX) + (threadIdx.x >> 6) * (GPW * 16);
    bf16* const sq = reinterpret_cast<bf16*>(lds + OFF_Q);    // [H][D] queries of the sequence

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n16 = lane & 15;
    const int g = lane >> 4;
    // Groups of 16 list positions are dealt to the sequence's waves round robin.
    // The list length is on the device, so the queries and this wave's candidate
    // indices are loaded speculatively, straight into LDS, together with the
    // counts: positions up to the most the grid can hold (from the host bound
    // max_cand), the index buffer ranged to the sequence's S_b slots, so no
    // load leaves the list's storage.  The key copies then follow one round
    // trip later.
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t G_grid = (max_cand + 15) / 16;
    const int ng_spec = (int)max((int64_t)0, min((G_grid - gw + nw - 1) / nw, (int64_t)GPW));
    const int64_t S = seq_len[b];
    const int64_t eo = entry_start[b];
    {
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(cand_idx + eo), (short)0, (int)min(S * 4, (int64_t)0x7fffffff), kBufferWord3);
        // lane L of copy k4 fills myidx[64 k4 + L]: group i = 4 k4 + L / 16, slot L % 16
#pragma unroll
        for (int k4 = 0; k4 < GPW / 4; ++k4) {
            if (4 * k4 < ng_spec) {
                const int i = 4 * k4 + g;
                const uint32_t pos = (uint32_t)(16 * (gw + nw * i) + n16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ir, (__attribute__((address_space(3))) void*)(myidx + 64 * k4), 4, 4u * pos,
                    0, 0, 0);
            }
        }
        // the sequence's [H][D] queries: 1 KiB per copy, copies dealt to the waves
        const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + (int64_t)b * H * D), (short)0, H * D * 2, kBufferWord3);
        for (int c = wave; c < (H * D * 2 + 1023) / 1024; c += 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                qr, (__attribute__((address_space(3))) void*)(reinterpret_cast<unsigned char*>(sq) + 1024 * c),
                16, (uint32_t)(1024 * c + 16 * lane), 0, 0, 0);
    }
    const int64_t C = min(min((int64_t)cand_count[b], max_cand), S);
    const int64_t G = (C + 15) / 16;
    wait_vmcnt<0>();                             // this wave's indices and query copies landed
    __syncthreads();                             // ... and every wave's queries
    if (gw >= G) return;
    const int ngroups = (int)min((G - gw + nw - 1) / nw, (int64_t)GPW);
    // key rows of the sequence; positions past the list hold no candidate: their
    // copies read whatever row their stale index names (or nothing, outside the
    // range) and their logits are never written
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(keys + key_row_start[b] * D), (short)0, (int)min(S * D * 2, (int64_t)0x7fffffff),
        kBufferWord3);

    // Group i goes to ring slot i % NB.  Copy j of a group moves rows RPI*j ..;
    // lane L fills physical slot L % SLOTS of row r = RPI*j + L/SLOTS.
    auto issue = [&](int i) {
        bf16* slot = myring + (i % NB) * 16 * D;
#pragma unroll
        for (int j = 0; j < DMAG; ++j) {
            const int r = RPI * j + lane / SLOTS;
            const int s = myidx[16 * i + r];
            const int ps = lane % SLOTS;
            const uint32_t off =
                (uint32_t)s * (uint32_t)(D * 2) + 16u * (uint32_t)(ps ^ (r & (SLOTS - 1) & 15));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                kr, (__attribute__((address_space(3))) void*)(slot + RPI * j * D), 16, off, 0, 0, 0);
        }
    };
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (i < ngroups) issue(i);

    bf16x8 qa[MT][KT];
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = min(16 * mt + n16, H - 1);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
            qa[mt][kk] = *reinterpret_cast<const bf16x8*>(sq + head * D + 32 * kk + 8 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int hv = 16 * mt + 4 * g + v;
            // padded heads carry zero weight, so their (duplicated) products drop out
            wv[mt][v] = hv < H ? w[(int64_t)b * H + hv] : 0.0f;
        }
    }
    const int rsw = n16 & (SLOTS - 1) & 15;

    for (int i = 0; i < ngroups; ++i) {
        // group i's copies landed; later groups' copies may stay in flight (the
        // first use of Q, loaded after the first NB groups, waits for those)
        const int after = min(ngroups - 1, i + NB - 1) - i;
        if (after >= 3) {
            wait_vmcnt<3 * DMAG>();
        } else if (after == 2) {
            wait_vmcnt<2 * DMAG>();
        } else if (after == 1) {
            wait_vmcnt<DMAG>();
        } else {
            wait_vmcnt<0>();
        }
        const bf16* slot = myring + (i % NB) * 16 * D + n16 * D;
        bf16x8 kb[KT];
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
            kb[kk] = *reinterpret_cast<const bf16x8*>(slot + 8 * ((4 * kk + g) ^ rsw));
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(qa[mt][kk], kb[kk], acc[mt]);
        const int s_out = myidx[16 * i + n16];
        // the operands are in registers: refill slot i % NB with group i + NB
        if (i + NB < ngroups) issue(i + NB);
        float sacc = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) sacc += wv[mt][v] * relu_bits(acc[mt][v]);
        sacc += __shfl_xor(sacc, 16);
        sacc += __shfl_xor(sacc, 32);
        const int64_t p = 16 * (gw + nw * (int64_t)i) + n16;
        if (g == 0 && p < C && s_out >= 0 && s_out < S) r_out[eo + s_out] = sacc;
    }
}

// Vector path: one thread per candidate; queries and weights in LDS as fp32.
template <typename E>
__global__ __launch_bounds__(256) void k_rescore_vector(
    const E* __restrict__ keys, const int64_t* __restrict__ key_row_start,
    const int32_t* __restrict__ seq_len, const int64_t* __restrict__ entry_start,
    const int32_t* __restrict__ cand_idx, const int32_t* __restrict__ cand_count, int H, int D,
    int64_t max_cand, const E* __restrict__ q, const float* __restrict__ w,
    float* __restrict__ r_out) {
    extern __shared__ float smem[];
    float* sq = smem;               // [H*D]
    float* sw = smem + H * D;       // [H]
    const int b = blockIdx.y;
    for (int i = threadIdx.x; i < H * D; i += blockDim.x) sq[i] = (float)q[(int64_t)b * H * D + i];
    for (int i = threadIdx.x; i < H; i += blockDim.x) sw[i] = w[(int64_t)b * H + i];
    __syncthreads();
    const int64_t S = seq_len[b];
    const int64_t C = min(min((int64_t)cand_count[b], max_cand), S);
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= C) return;
    const int64_t eo = entry_start[b];
    const int32_t s = cand_idx[eo + j];
    if (s < 0 || s >= S) return;                 // outside the sequence: nothing to score
    const E* row = keys + (key_row_start[b] + s) * D;
    float r = 0.0f;
    for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
        for (int d = 0; d < D; ++d) dot += sq[h * D + d] * (float)row[d];
        r += sw[h] * fmaxf(dot, 0.0f);
    }
    r_out[eo + s] = r;
}

}  // namespace lsa

using namespace lsa;

extern "C" int lsa_index_rescore(const void* keys, int dtype, const int64_t* key_row_start,
                                 const int32_t* seq_len, const int64_t* entry_start,
                                 const int32_t* cand_idx, const int32_t* cand_count, int B, int H,
                                 int D, int64_t max_cand, const void* q, const float* w,
                                 float* r_out, void* stream) {
    clear_error();
    if (!keys || !key_row_start || !seq_len || !entry_start || !cand_idx || !cand_count || !q ||
        !w || !r_out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_rescore: a required pointer is NULL");
    if (B <= 0 || H <= 0 || D <= 0 || max_cand < 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_rescore: B=%d H=%d D=%d max_cand=%lld", B, H,
                    D, (long long)max_cand);
    if (dtype != LSA_DTYPE_F32 && dtype != LSA_DTYPE_BF16)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_rescore: unknown dtype %d", dtype);
    if (!aligned16(keys) || !aligned16(q))
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_rescore: keys and q must be 16-byte aligned");
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "lsa_index_rescore: B=%d > 65535", B);
    const bool mfma_shape = dtype == LSA_DTYPE_BF16 && H <= 64 && (D == 64 || D == 128);
    // buffer byte offsets are 32-bit: a sequence's keys must span less than 2 GiB
    if (max_cand > (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_index_rescore: max_cand too large");
    if (!mfma_shape && (int64_t)H * (D + 1) > 16384)
        return fail(LSA_ERR_UNSUPPORTED,
                    "lsa_index_rescore: vector path needs H*(D+1) <= 16384 (H=%d D=%d)", H, D);
    int cus = 0;
    int rc = check_device(&cus);
    if (rc != LSA_OK) return rc;
    if (max_cand == 0) return LSA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (mfma_shape) {
        const int64_t groups = ceil_div(max_cand, 16);
        int64_t gpw = (groups * B) / ((int64_t)cus * 4);
        gpw = gpw < 1 ? 1 : (gpw > kRescoreGroupsPerWave ? kRescoreGroupsPerWave : gpw);
        dim3 grid((unsigned)ceil_div(groups, gpw * 4), (unsigned)B);
        const int MT = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
#define LSA_RS(mt, kt)                                                                          \
    hipLaunchKernelGGL((k_rescore_mfma<mt, kt>), grid, dim3(256), 0, st, (const bf16*)keys,       \
                       key_row_start, seq_len, entry_start, cand_idx, cand_count, H, max_cand,   \
                       (const bf16*)q, w, r_out)
        if (D == 128) {
            if (MT == 1) LSA_RS(1, 4); else if (MT == 2) LSA_RS(2, 4); else LSA_RS(4, 4);
        } else {
            if (MT == 1) LSA_RS(1, 2); else if (MT == 2) LSA_RS(2, 2); else LSA_RS(4, 2);
        }
#undef LSA_RS
        return launch_status("rescore_mfma");
    }
    dim3 grid((unsigned)ceil_div(max_cand, 256), (unsigned)B);
    const size_t shm = sizeof(float) * ((size_t)H * D + (size_t)H);
    if (dtype == LSA_DTYPE_F32)
        hipLaunchKernelGGL(k_rescore_vector<float>, grid, dim3(256), shm, st, (const float*)keys,
                           key_row_start, seq_len, entry_start, cand_idx, cand_count, H, D,
                           max_cand, (const float*)q, w, r_out);
    else
        hipLaunchKernelGGL(k_rescore_vector<bf16>, grid, dim3(256), shm, st, (const bf16*)keys,
                           key_row_start, seq_len, entry_start, cand_idx, cand_count, H, D,
                           max_cand, (const bf16*)q, w, r_out);
    return launch_status("rescore_vector");
}
