// score.hip -- lsa_index_score: the Memory Indexer's lookahead index score.
//
// Definition (page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context
// via Lookahead Sparse Attention", Technical Summary 2.1 "Scoring Mechanism";
// dot-product interaction per section 5): a head-fused, gated score
//     z[b,t,s] = sum_h w[b,t,h] * max(0, <q[b,t,h,:], k[b,s,:]>) + bias
// and I = sigmoid(z).  With T query positions per sequence the OR-union of
// per-position gates (section 2.4) is the gate on max_t z.
//
// Three kernels:
//  * score_decode (T = 1, bf16): streams each key row once from HBM.  All H
//    heads share the key, so one 256-byte key feeds 64 x 128 multiply-adds:
//    ~63 flop/byte, above the fp32 vector ridge (~20 flop/byte) and below the
//    bf16 matrix ridge, hence the matrix cores run over the head dimension
//    (M = heads, N = 16 entries, K = d) and HBM stays the bound.
//  * score_burst (T > 1, bf16): a dense contraction of T*H query rows against
//    the keys (matrix-core bound); the ReLU, the weighted head sum and the
//    max over positions are fused into the epilogue.
//  * score_vector: any shape, fp32 or bf16, plain vector arithmetic (small
//    shapes, tests).
#include "common.hpp"

namespace lsa {

constexpr int kScoreRing = 4;          // LDS ring slots per wave (decode kernel)
// cache-policy operand of the direct-to-LDS loads: keys are read once, so they are
// fetched as streaming (nontemporal) data
constexpr int kNonTemporal = 2;
constexpr int kScoreGroupsPerWave = 32;


// ----------------------------------------------------------------- decode
// One wave scores groups of 16 consecutive entries of one sequence.
//   Keys stream HBM -> a wave-private LDS ring with direct-to-LDS loads, each
//   instruction moving 1 KiB of consecutive rows (4 rows of 256 B), up to
//   NB groups ahead of use.  Inside a staged row, 16-byte slot p holds logical
//   slot p ^ (row & 15), so the operand reads below are bank-conflict-free.
//   MFMA operands: lane l, n = l%16 selects the entry, g = l/16 selects 8 of
//   each 32 dims; A (queries) stays in registers for the whole wave; B (keys)
//   for k-step kk is dims 32kk + 8g .. +7 of entry n.
//   D[4g+v][n] of head tile mt is head 16mt + 4g + v of entry n.
template <int MT, int KT, bool COMBINE>
__global__ __launch_bounds__(256) void k_score_decode(
    const bf16* __restrict__ keys, const int64_t* __restrict__ key_row_start,
    const int32_t* __restrict__ seq_len, const int64_t* __restrict__ entry_start, int H,
    int64_t max_len, const bf16* __restrict__ q, const float* __restrict__ w, float bias,
    float* __restrict__ z_out, float* __restrict__ prob_out, uint16_t* __restrict__ gate_bits,
    int64_t gstride, float gthr) {
    constexpr int D = 32 * KT;
    constexpr int SLOTS = D / 8;                 // 16-byte slots per key row
    constexpr int RPI = 64 / SLOTS;              // rows per direct-to-LDS instruction
    constexpr int DMAG = 16 / RPI;               // instructions per group of 16 rows
    constexpr int NB = kScoreRing;               // ring slots per wave
    static_assert(SLOTS >= 16 || SLOTS == 8, "row layout");
    __shared__ __attribute__((aligned(16))) bf16 ring[4][NB][16 * D];

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    // The waves of one sequence deal its groups round robin, so at any moment the
    // chip reads a compact window of the sequence rather than thousands of
    // separate streams.
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t G = (S + 15) / 16;
    if (gw >= G) return;
    const int ngroups = (int)((G - gw + nw - 1) / nw);
    const int64_t last = S;
    const int n16 = lane & 15;
    const int g = lane >> 4;

    const bf16* kbase = keys + key_row_start[b] * D;
    bf16* myring = &ring[wave][0][0];
    // Group i of this wave is group gw + nw*i of the sequence and goes to ring slot
    // i % NB; rows past the sequence re-read its last row.
    auto issue = [&](int i) {
        const int64_t e0 = 16 * (gw + nw * (int64_t)i);
        bf16* slot = myring + (i % NB) * 16 * D;
#pragma unroll
        for (int j = 0; j < DMAG; ++j) {
            const int r = RPI * j + lane / SLOTS;             // row inside the group
            const int64_t e = min(e0 + r, last - 1);
            const int ps = lane % SLOTS;
            const bf16* src = kbase + e * D + 8 * (ps ^ (r & (SLOTS - 1) & 15));
            __builtin_amdgcn_global_load_lds(
                (const void*)src, (__attribute__((address_space(3))) void*)(slot + RPI * j * D),
                16, 0, kNonTemporal);
        }
    };
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (i < ngroups) issue(i);

    bf16x8 qa[MT][KT];
    float wv[MT][4];
    const bf16* qb = q + (int64_t)b * H * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = min(16 * mt + n16, H - 1);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) qa[mt][kk] = load8(qb + (int64_t)head * D + 32 * kk + 8 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int hv = 16 * mt + 4 * g + v;
            // padded heads carry zero weight, so their (duplicated) products drop out
            wv[mt][v] = hv < H ? w[(int64_t)b * H + hv] : 0.0f;
        }
    }
    const int64_t eo = entry_start[b];
    const int rsw = n16 & (SLOTS - 1) & 15;

    for (int i = 0; i < ngroups; ++i) {
        // wait until group i's copies landed: later groups' copies may stay in flight
        // (vector memory operations complete in issue order)
        const int after = min(ngroups - 1, i + NB - 1) - i;
        static_assert(NB <= 4, "waits below cover up to three later groups");
        if (after >= 3) wait_vmcnt<3 * DMAG>();
        else if (after == 2) wait_vmcnt<2 * DMAG>();
        else if (after == 1) wait_vmcnt<DMAG>();
        else wait_vmcnt<0>();
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
        // the operands are in registers: refill slot i % NB with group i + NB
        if (i + NB < ngroups) issue(i + NB);
        float sacc = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) sacc += wv[mt][v] * relu_bits(acc[mt][v]);
        sacc += __shfl_xor(sacc, 16);
        sacc += __shfl_xor(sacc, 32);
        const int64_t grp = gw + nw * (int64_t)i;
        const int64_t n = 16 * grp + n16;
        const bool own = g == 0 && n < last;
        float z = sacc + bias;
        if (own) {
            if (COMBINE) z = fmaxf(z_out[eo + n], z);   // OR-union with earlier indexers
            z_out[eo + n] = z;
            if (prob_out) prob_out[eo + n] = sigmoidf(z);
        }
        // the gate of the group's 16 entries (lanes 0..15), one 16-bit word
        if (gate_bits) {
            const uint64_t m = __ballot(own && z >= gthr);
            if (lane == 0) gate_bits[(int64_t)b * gstride + grp] = (uint16_t)m;
        }
    }
}

// ------------------------------------------------------------ fused union
// OR-mode union of up to kUnionMax indexers in one pass (T = 1; the indexers of
// several layers united by OR, Technical Summary section 2.4): the decode
// kernel's streaming with (indexer, group) as the unit.  A wave takes its
// groups for indexer 0, then the same groups for indexer 1, ... ; the ring runs
// on across the switch (the copies of the next indexer's first groups are in
// flight while the last groups of the current one are scored), and the queries
// and weights of the next indexer load into registers at the switch.  The
// running maximum of the wave's <= kScoreGroupsPerWave groups stays in
// registers, spread over lanes (lane 16 j + n of zmax[s] holds entry n of group
// 4 s + j, which the head-sum shuffles leave in that lane), and is written
// once at the end.  Each entry's logit is computed as in the decode kernel, so
// the union is bit-identical to the one the combining launches produce.
constexpr int kUnionMax = 4;
struct UnionArgs {
    const bf16* keys[kUnionMax];
    const bf16* q[kUnionMax];
    const float* w[kUnionMax];
    float bias[kUnionMax];
    int n;
};

// u.x[l] for a wave-uniform l, kept in scalar registers: each argument passes
// through readfirstlane before the selection, so the choice cannot turn back
// into an indexed (vector) load of the argument block
__device__ __forceinline__ uint32_t sgpr32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ T* sgpr_ptr(T* p) {
    const uint64_t x = (uint64_t)p;
    return (T*)(((uint64_t)sgpr32((uint32_t)(x >> 32)) << 32) | sgpr32((uint32_t)x));
}
template <typename T>
__device__ __forceinline__ T* pick(T* const (&a)[kUnionMax], int l) {
    l = (int)sgpr32((uint32_t)l);
    T* r = sgpr_ptr(a[0]);
#pragma unroll
    for (int j = 1; j < kUnionMax; ++j)
        if (l == j) r = sgpr_ptr(a[j]);
    return r;
}
__device__ __forceinline__ float pick(const float (&a)[kUnionMax], int l) {
    l = (int)sgpr32((uint32_t)l);
    float r = __uint_as_float(sgpr32(__float_as_uint(a[0])));
#pragma unroll
    for (int j = 1; j < kUnionMax; ++j)
        if (l == j) r = __uint_as_float(sgpr32(__float_as_uint(a[j])));
    return r;
}

template <int MT, int KT>
__global__ __launch_bounds__(256) void k_score_union(
    UnionArgs u, const int64_t* __restrict__ key_row_start, const int32_t* __restrict__ seq_len,
    const int64_t* __restrict__ entry_start, int H, int64_t max_len, float* __restrict__ z_out,
    float* __restrict__ prob_out, uint16_t* __restrict__ gate_bits, int64_t gstride, float gthr) {
    constexpr int D = 32 * KT;
    constexpr int SLOTS = D / 8;
    constexpr int RPI = 64 / SLOTS;
    constexpr int DMAG = 16 / RPI;
    constexpr int NB = kScoreRing;
    constexpr int ZS = kScoreGroupsPerWave / 4;    // running-max registers per lane
    static_assert(SLOTS >= 16 || SLOTS == 8, "row layout");
    static_assert((NB & (NB - 1)) == 0, "ring slots: a power of two");
    __shared__ __attribute__((aligned(16))) bf16 ring[4][NB][16 * D];

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t G = (S + 15) / 16;
    if (gw >= G) return;
    // at most kScoreGroupsPerWave by the launch's grid
    const int ngroups = (int)min((G - gw + nw - 1) / nw, (int64_t)kScoreGroupsPerWave);
    const int nunits = ngroups * u.n;
    const int64_t last = S;
    const int n16 = lane & 15;
    const int g = lane >> 4;
    const int64_t krs = key_row_start[b];
    const int64_t eo = entry_start[b];
    bf16* myring = &ring[wave][0][0];

    // the next unit to copy: number vn, indexer il, group ii of this wave
    int vn = 0, il = 0, ii = 0;
    auto issue_next = [&]() {
        const bf16* kbase = pick(u.keys, il) + krs * D;
        const int64_t e0 = 16 * (gw + nw * (int64_t)ii);
        bf16* slot = myring + (vn & (NB - 1)) * 16 * D;
#pragma unroll
        for (int j = 0; j < DMAG; ++j) {
            const int r = RPI * j + lane / SLOTS;
            const int64_t e = min(e0 + r, last - 1);
            const int ps = lane % SLOTS;
            const bf16* src = kbase + e * D + 8 * (ps ^ (r & (SLOTS - 1) & 15));
            __builtin_amdgcn_global_load_lds(
                (const void*)src, (__attribute__((address_space(3))) void*)(slot + RPI * j * D),
                16, 0, kNonTemporal);
        }
        ++vn;
        if (++ii == ngroups) { ii = 0; ++il; }
    };
#pragma unroll
    for (int v = 0; v < NB; ++v)
        if (vn < nunits) issue_next();

    float zmax[ZS];
#pragma unroll
    for (int s8 = 0; s8 < ZS; ++s8) zmax[s8] = -INFINITY;
    const int rsw = n16 & (SLOTS - 1) & 15;
    int v = 0;                                     // unit being scored
    for (int l = 0; l < u.n; ++l) {
        bf16x8 qa[MT][KT];
        float wv[MT][4];
        const bf16* qb = pick(u.q, l) + (int64_t)b * H * D;
        const float* wb = pick(u.w, l) + (int64_t)b * H;
        const float bias = pick(u.bias, l);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int head = min(16 * mt + n16, H - 1);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk)
                qa[mt][kk] = load8(qb + (int64_t)head * D + 32 * kk + 8 * g);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int hv = 16 * mt + 4 * g + q4;
                wv[mt][q4] = hv < H ? wb[hv] : 0.0f;
            }
        }
        // queries and weights in registers (the ring's copies in flight retire too:
        // vector memory operations complete in issue order)
        wait_vmcnt<0>();
        for (int i = 0; i < ngroups; ++i, ++v) {
            // unit v's copies landed (later units' copies may stay in flight)
            const int after = min(nunits - 1, v + NB - 1) - v;
            static_assert(NB <= 4, "waits below cover up to three later units");
            if (after >= 3) wait_vmcnt<3 * DMAG>();
            else if (after == 2) wait_vmcnt<2 * DMAG>();
            else if (after == 1) wait_vmcnt<DMAG>();
            else wait_vmcnt<0>();
            const bf16* slot = myring + (v & (NB - 1)) * 16 * D + n16 * D;
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
            if (vn < nunits) issue_next();
            float sacc = 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) sacc += wv[mt][q4] * relu_bits(acc[mt][q4]);
            sacc += __shfl_xor(sacc, 16);
            sacc += __shfl_xor(sacc, 32);
            const float z = sacc + bias;
            // every lane holds entry n16's logit; lane 16 (i % 4) + n16 keeps it.
            // Indexer 0's logit is taken as it is and later ones are folded in with
            // fmaxf, exactly as the per-indexer calls combine them (so a NaN from
            // every indexer stays NaN, and a NaN from some yields the others' max).
#pragma unroll
            for (int s8 = 0; s8 < ZS; ++s8)
                if ((i >> 2) == s8 && (i & 3) == g) zmax[s8] = l == 0 ? z : fmaxf(zmax[s8], z);
        }
    }
#pragma unroll
    for (int s8 = 0; s8 < ZS; ++s8) {
        const int i = 4 * s8 + g;
        const int64_t grp = gw + nw * (int64_t)i;
        const int64_t n = 16 * grp + n16;
        const bool own = i < ngroups && n < last;
        if (own) {
            z_out[eo + n] = zmax[s8];
            if (prob_out) prob_out[eo + n] = sigmoidf(zmax[s8]);
        }
        // lanes 16 g .. 16 g + 15 hold group i's gate: one 16-bit word each
        if (gate_bits && 4 * s8 < ngroups) {
            const uint64_t m = __ballot(own && zmax[s8] >= gthr);
            if (n16 == 0 && i < ngroups)
                gate_bits[(int64_t)b * gstride + grp] = (uint16_t)(m >> (16 * g));
        }
    }
}

// ------------------------------------------------------------------ burst
// Workgroup = 4 waves x 64 entries of one sequence; it walks all T positions.
// Keys of the wave's 64 entries stay in registers as B operands (32x32x16,
// two entry tiles).  The queries and weights of each position (H <= 64 heads x
// D) are copied from HBM straight into an LDS ring of kBurstRing positions by
// buffer loads into LDS, kBurstRing-1 positions ahead of use, so their latency
// hides behind the matrix work of the positions before.  Query rows are
// XOR-swizzled by 16-byte chunk (applied on the source side of the copies) so
// the 32 heads read by one instruction hit distinct banks.  Head rows >= H are
// zero: their copies fall outside the buffer range and the ring starts zeroed.
// Compile-time knobs: ring depth (positions) and workgroups per CU.  With 3
// slots of 16 KiB the workgroup holds ~49 KiB of LDS and 142 VGPRs per lane, so
// three workgroups share a CU (three waves per SIMD).
#ifndef LSA_BURST_RING
#define LSA_BURST_RING 3
#endif
#ifndef LSA_BURST_MINB
#define LSA_BURST_MINB 3
#endif
constexpr int kBurstRing = LSA_BURST_RING;
constexpr int kBurstWaves = 4;                           // waves per workgroup
constexpr int kBurstTiles = 2;                           // 32-entry tiles per wave
constexpr int kBurstEntries = 32 * kBurstWaves * kBurstTiles;   // entries per workgroup (256)
constexpr int kBurstMinBlocks = LSA_BURST_MINB;          // workgroups per CU

template <int KS, int NW, int NT, int MINB>
__global__ __launch_bounds__(64 * NW, MINB) void k_score_burst(
    const bf16* __restrict__ keys, const int64_t* __restrict__ key_row_start,
    const int32_t* __restrict__ seq_len, const int64_t* __restrict__ entry_start, int T, int H,
    int64_t max_len, const bf16* __restrict__ q, const float* __restrict__ w, float bias,
    int reduce_max, float* __restrict__ z_out, float* __restrict__ prob_out,
    uint16_t* __restrict__ gate_bits, int64_t gstride, float gthr) {
    constexpr int D = 16 * KS;
    constexpr int CH = D / 8;                 // 16-byte chunks per query row
    constexpr int QCHUNKS = 64 * CH;          // per position (64 head slots)
    constexpr int NQ = kBurstRing;
    constexpr int IPQ = QCHUNKS / 64 / NW;    // query copies per wave per position
    constexpr int CPP = IPQ + 1;              // copies per wave per position (+ the weights)
    static_assert(IPQ >= 1 && NQ >= 2, "tiling");
    // one LDS object: NQ query slots, then NQ weight slots
    __shared__ __attribute__((aligned(16))) unsigned char lds[NQ * QCHUNKS * 16 + NQ * 64 * 4];
    bf16x8* const sq = reinterpret_cast<bf16x8*>(lds);
    float* const sw = reinterpret_cast<float*>(lds + NQ * QCHUNKS * 16);

    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t S = min((int64_t)seq_len[b], max_len);
    constexpr int EPW = 32 * NT;              // entries per wave
    const int64_t e_blk = (int64_t)blockIdx.x * (NW * EPW);
    if (e_blk >= S) return;
    const int n32 = lane & 31;
    const int g = lane >> 5;

    // B operands: this wave's NT tiles of 32 entries.
    bf16x8 kb[NT][KS];
    int64_t ent[NT];
    const bf16* kbase = keys + key_row_start[b] * D + 8 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        ent[nt] = e_blk + wave * EPW + nt * 32 + n32;
        const int64_t row = ent[nt] < S ? ent[nt] : e_blk;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[nt][ks] = load8(kbase + row * D + 16 * ks);
    }

    // Padded head rows (and weights) must read as zero: clear the ring once.
    if (H < 64) {
        for (int i = tid; i < NQ * QCHUNKS; i += 64 * NW) sq[i] = zero8();
        for (int i = tid; i < NQ * 64; i += 64 * NW) sw[i] = 0.0f;
    }
    lds_barrier();

    // Copies of position t into ring slot t % NQ.  Lane L of query copy i of wave
    // wv fills LDS chunk p = (IPQ wv + i) 64 + L: head h = p / CH, physical chunk
    // p % CH, which holds logical chunk (p % CH) ^ (h % CH).  The weights take one
    // 4-byte copy per lane (every wave issues it, so all waves count alike).
    // Positions past T are issued with an empty range: no memory is read.
    auto issue = [&](int t) {
        const int slot = t % NQ;
        const bool live = t < T;
        const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + ((int64_t)b * T + (live ? t : 0)) * H * D), (short)0,
            live ? H * D * 2 : 0, kBufferWord3);
#pragma unroll
        for (int i = 0; i < IPQ; ++i) {
            const int p0 = (IPQ * wave + i) * 64;
            const int p = p0 + lane;
            const int h = p / CH, pc = p % CH;
            const uint32_t off = (uint32_t)(h * D + 8 * (pc ^ (h & (CH - 1)))) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                qr, (__attribute__((address_space(3))) void*)(sq + slot * QCHUNKS + p0), 16, off, 0,
                0, 0);
        }
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(w + ((int64_t)b * T + (live ? t : 0)) * H), (short)0, live ? H * 4 : 0,
            kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(sw + slot * 64), 4, (uint32_t)(4 * lane), 0,
            0, 0);
    };

    float mx[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
    const int64_t eo = entry_start[b];
#pragma unroll
    for (int t = 0; t < NQ - 1; ++t) issue(t);
    for (int t = 0; t < T; ++t) {
        const int slot = t % NQ;
        wait_vmcnt<(NQ - 2) * CPP>();   // position t landed (later ones may be in flight)
        lds_barrier();                  // ... for every wave; all are done with t-1
        issue(t + NQ - 1);                    // into t-1's slot
        const bf16x8* qs = sq + slot * QCHUNKS;
        // The two 32-head halves one after the other: half the accumulators live
        // at a time, which leaves room for three waves per SIMD, so one wave's
        // epilogue arithmetic overlaps another's matrix products.
        float s[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = 0.0f;
#pragma unroll 1
        for (int mt = 0; mt < 2; ++mt) {
            f32x16 acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[nt][v] = 0.0f;
            const int h = 32 * mt + n32;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 2 * ks + g;
                const bf16x8 a = qs[h * CH + (ch ^ (h & (CH - 1)))];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32(a, kb[nt][ks], acc[nt]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 wq = *reinterpret_cast<const f32x4*>(&sw[slot * 64 + 32 * mt + 8 * j + 4 * g]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) s[nt] += wq[v] * relu_bits(acc[nt][4 * j + v]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            s[nt] += __shfl_xor(s[nt], 32);
            const float z = s[nt] + bias;
            if (reduce_max) {
                mx[nt] = fmaxf(mx[nt], z);
            } else if (g == 0 && ent[nt] < S) {
                const int64_t o = eo * T + (int64_t)t * S + ent[nt];
                z_out[o] = z;
                if (prob_out) prob_out[o] = sigmoidf(z);
            }
        }
    }
    wait_vmcnt<0>();                    // no copy lands after the workgroup ends
    if (reduce_max) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bool own = g == 0 && ent[nt] < S;
            float m = mx[nt];
            if (own) {
                // reduce_max == 2: OR-union with the indexers already in z_out
                if (reduce_max == 2) m = fmaxf(z_out[eo + ent[nt]], m);
                z_out[eo + ent[nt]] = m;
                if (prob_out) prob_out[eo + ent[nt]] = sigmoidf(m);
            }
            // lanes 0..31 hold two groups of 16 entries: two 16-bit words
            if (gate_bits) {
                const uint64_t bits = __ballot(own && m >= gthr);
                const int64_t grp = (e_blk + wave * EPW + nt * 32) / 16 + (lane >> 4);
                if ((lane == 0 || lane == 16) && 16 * grp < S)
                    gate_bits[(int64_t)b * gstride + grp] = (uint16_t)(bits >> lane);
            }
        }
    }
}

// ----------------------------------------------------------------- vector
// One thread per entry; queries and weights of the sequence sit in LDS as fp32.
template <typename E>
__global__ __launch_bounds__(256) void k_score_vector(
    const E* __restrict__ keys, const int64_t* __restrict__ key_row_start,
    const int32_t* __restrict__ seq_len, const int64_t* __restrict__ entry_start, int T, int H,
    int D, int64_t max_len, const E* __restrict__ q, const float* __restrict__ w, float bias,
    int reduce_max, float* __restrict__ z_out, float* __restrict__ prob_out,
    uint16_t* __restrict__ gate_bits, int64_t gstride, float gthr) {
    extern __shared__ float smem[];
    float* sq = smem;               // [T*H*D]
    float* sw = smem + T * H * D;   // [T*H]
    const int b = blockIdx.y;
    const int nq = T * H * D;
    for (int i = threadIdx.x; i < nq; i += blockDim.x) sq[i] = (float)q[(int64_t)b * nq + i];
    for (int i = threadIdx.x; i < T * H; i += blockDim.x) sw[i] = w[(int64_t)b * T * H + i];
    __syncthreads();
    const int64_t S = min((int64_t)seq_len[b], max_len);
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // a wave's 64 entries are four groups of 16; waves past the sequence end stop
    if (s - (threadIdx.x & 63) >= S) return;
    const bool live = s < S;
    const E* row = keys + (key_row_start[b] + (live ? s : 0)) * D;
    const int64_t eo = entry_start[b];
    float m = -INFINITY;
    float zlast = 0.0f;                 // the logit the gate reads
    if (live) for (int t = 0; t < T; ++t) {
        float u = 0.0f;
        // eight heads per pass over the row: each key element is loaded once per
        // pass, not once per head (head sums still added in head order)
        for (int h0 = 0; h0 < H; h0 += 8) {
            const int nh = min(8, H - h0);
            const float* q0 = sq + (t * H + h0) * D;
            float dot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int d = 0; d < D; ++d) {
                const float r = (float)row[d];
#pragma unroll
                for (int hh = 0; hh < 8; ++hh) dot[hh] += q0[min(hh, nh - 1) * D + d] * r;
            }
#pragma unroll
            for (int hh = 0; hh < 8; ++hh)
                if (hh < nh) u += sw[t * H + h0 + hh] * fmaxf(dot[hh], 0.0f);
        }
        const float z = u + bias;
        if (reduce_max) {
            m = fmaxf(m, z);
        } else {
            const int64_t o = eo * T + (int64_t)t * S + s;
            z_out[o] = z;
            if (prob_out) prob_out[o] = sigmoidf(z);
            zlast = z;
        }
    }
    if (reduce_max && live) {
        if (reduce_max == 2) m = fmaxf(z_out[eo + s], m);   // OR-union with earlier indexers
        z_out[eo + s] = m;
        if (prob_out) prob_out[eo + s] = sigmoidf(m);
        zlast = m;
    }
    // (gate bits are only asked for with one position or a reduction)
    if (gate_bits) {
        const int l = threadIdx.x & 63;
        const uint64_t bits = __ballot(live && zlast >= gthr);
        const int64_t grp = (s - l) / 16 + (l >> 4);
        if ((l & 15) == 0 && 16 * grp < S)
            gate_bits[(int64_t)b * gstride + grp] = (uint16_t)(bits >> l);
    }
}

template <int MT, int KT>
static void launch_decode(dim3 grid, hipStream_t st, const void* keys, const int64_t* krs,
                          const int32_t* lens, const int64_t* es, int H, int64_t max_len,
                          const void* q, const float* w, float bias, bool combine, float* z,
                          float* p, uint16_t* gb, int64_t gs, float gthr) {
    // the OR-union mode is its own instantiation: the plain kernel keeps its code
    if (combine)
        hipLaunchKernelGGL((k_score_decode<MT, KT, true>), grid, dim3(256), 0, st,
                           (const bf16*)keys, krs, lens, es, H, max_len, (const bf16*)q, w, bias, z,
                           p, gb, gs, gthr);
    else
        hipLaunchKernelGGL((k_score_decode<MT, KT, false>), grid, dim3(256), 0, st,
                           (const bf16*)keys, krs, lens, es, H, max_len, (const bf16*)q, w, bias, z,
                           p, gb, gs, gthr);
}

}  // namespace lsa

using namespace lsa;

extern "C" int lsa_index_score(const void* keys, int dtype, const int64_t* key_row_start,
                               const int32_t* seq_len, const int64_t* entry_start, int B, int T,
                               int H, int D, int64_t max_len, const void* q, const float* w,
                               float bias, int reduce_max, float* z_out, float* prob_out,
                               uint16_t* gate_bits, float gate_threshold, void* stream) {
    clear_error();
    if (!keys || !key_row_start || !seq_len || !entry_start || !q || !w || !z_out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: a required pointer is NULL");
    if (gate_bits && T > 1 && reduce_max == 0)
        return fail(LSA_ERR_INVALID_ARG,
                    "lsa_index_score: gate bits need one position or reduce_max (T=%d)", T);
    if (gate_bits && !aligned16(gate_bits))
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: gate_bits must be 16-byte aligned");
    if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || max_len < 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: B=%d T=%d H=%d D=%d max_len=%lld", B, T,
                    H, D, (long long)max_len);
    if (reduce_max < 0 || reduce_max > 2)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: reduce_max=%d not in {0, 1, 2}",
                    reduce_max);
    if (dtype != LSA_DTYPE_F32 && dtype != LSA_DTYPE_BF16)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: unknown dtype %d", dtype);
    if (!aligned16(keys) || !aligned16(q))
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score: keys and q must be 16-byte aligned");
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "lsa_index_score: B=%d > 65535", B);
    if (max_len > (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_index_score: max_len too large");
    const bool mfma_shape = dtype == LSA_DTYPE_BF16 && H <= 64 && (D == 64 || D == 128);
    if (!mfma_shape && (int64_t)T * H * (D + 1) > 16384)
        return fail(LSA_ERR_UNSUPPORTED,
                    "lsa_index_score: vector path needs T*H*(D+1) <= 16384 (T=%d H=%d D=%d)", T,
                    H, D);
    int cus = 0;
    int rc = check_device(&cus);
    if (rc != LSA_OK) return rc;
    if (max_len == 0) return LSA_OK;
    hipStream_t st = (hipStream_t)stream;
    const int64_t gs = lsa_gate_words(max_len);

    if (mfma_shape && T == 1) {
        const int64_t groups = ceil_div(max_len, 16);
        // Long-lived waves (each loads its query operands once): up to 32 groups of 16
        // entries per wave, fewer when the batch is too small to give every CU ~4 waves.
        int64_t gpw = (groups * B) / ((int64_t)cus * 4);
        gpw = gpw < 1 ? 1 : (gpw > kScoreGroupsPerWave ? kScoreGroupsPerWave : gpw);
        dim3 grid((unsigned)ceil_div(groups, gpw * 4), (unsigned)B);
        const int MT = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
#define LSA_DEC(mt, kt)                                                                      \
    launch_decode<mt, kt>(grid, st, keys, key_row_start, seq_len, entry_start, H, max_len, q, \
                          w, bias, reduce_max == 2, z_out, prob_out, gate_bits, gs, gate_threshold)
        // With one position the [T, S_b] layout and the reduced layout coincide.
        if (D == 128) {
            if (MT == 1) LSA_DEC(1, 4); else if (MT == 2) LSA_DEC(2, 4); else LSA_DEC(4, 4);
        } else {
            if (MT == 1) LSA_DEC(1, 2); else if (MT == 2) LSA_DEC(2, 2); else LSA_DEC(4, 2);
        }
#undef LSA_DEC
        return launch_status("score_decode");
    }
    if (mfma_shape) {
        // 4 waves x 64 entries per workgroup, three workgroups per CU: the waves
        // sharing a SIMD overlap one another's epilogues with the matrix work.
        dim3 grid((unsigned)ceil_div(max_len, kBurstEntries), (unsigned)B);
        if (D == 128)
            hipLaunchKernelGGL((k_score_burst<8, kBurstWaves, kBurstTiles, kBurstMinBlocks>), grid,
                               dim3(64 * kBurstWaves), 0, st, (const bf16*)keys, key_row_start,
                               seq_len, entry_start, T, H, max_len, (const bf16*)q, w, bias,
                               reduce_max, z_out, prob_out, gate_bits, gs, gate_threshold);
        else
            hipLaunchKernelGGL((k_score_burst<4, kBurstWaves, kBurstTiles, kBurstMinBlocks>), grid,
                               dim3(64 * kBurstWaves), 0, st, (const bf16*)keys, key_row_start,
                               seq_len, entry_start, T, H, max_len, (const bf16*)q, w, bias,
                               reduce_max, z_out, prob_out, gate_bits, gs, gate_threshold);
        return launch_status("score_burst");
    }
    dim3 grid((unsigned)ceil_div(max_len, 256), (unsigned)B);
    const size_t shm = sizeof(float) * ((size_t)T * H * D + (size_t)T * H);
    if (dtype == LSA_DTYPE_F32)
        hipLaunchKernelGGL(k_score_vector<float>, grid, dim3(256), shm, st, (const float*)keys,
                           key_row_start, seq_len, entry_start, T, H, D, max_len, (const float*)q,
                           w, bias, reduce_max, z_out, prob_out, gate_bits, gs, gate_threshold);
    else
        hipLaunchKernelGGL(k_score_vector<bf16>, grid, dim3(256), shm, st, (const bf16*)keys,
                           key_row_start, seq_len, entry_start, T, H, D, max_len, (const bf16*)q,
                           w, bias, reduce_max, z_out, prob_out, gate_bits, gs, gate_threshold);
    return launch_status("score_vector");
}

extern "C" int lsa_index_score_union(int n_idx, const void* const* keys, int dtype,
                                     const int64_t* key_row_start, const int32_t* seq_len,
                                     const int64_t* entry_start, int B, int T, int H, int D,
                                     int64_t max_len, const void* const* q,
                                     const float* const* w, const float* bias, float* z_out,
                                     float* prob_out, uint16_t* gate_bits, float gate_threshold,
                                     void* stream) {
    clear_error();
    if (!keys || !q || !w || !bias)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: a required array is NULL");
    if (n_idx < 1 || n_idx > kUnionMax)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: n_idx=%d not in 1..%d", n_idx,
                    kUnionMax);
    for (int l = 0; l < n_idx; ++l)
        if (!keys[l] || !q[l] || !w[l])
            return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: indexer %d has a NULL pointer",
                        l);
    // what differs between the indexers is checked for all of them before anything
    // is enqueued (the per-indexer calls below then fail on the first or not at all)
    for (int l = 0; l < n_idx; ++l) {
        if (!aligned16(keys[l]) || !aligned16(q[l]))
            return fail(LSA_ERR_INVALID_ARG,
                        "lsa_index_score_union: keys and q of indexer %d must be 16-byte aligned", l);
    }
    const bool fused = dtype == LSA_DTYPE_BF16 && T == 1 && H <= 64 && (D == 64 || D == 128);
    if (!fused) {
        // other shapes: one score launch per indexer, each combining with the last
        for (int l = 0; l < n_idx; ++l) {
            const int rc = lsa_index_score(keys[l], dtype, key_row_start, seq_len, entry_start, B,
                                           T, H, D, max_len, q[l], w[l], bias[l],
                                           l == 0 ? 1 : 2, z_out,
                                           l == n_idx - 1 ? prob_out : nullptr,
                                           l == n_idx - 1 ? gate_bits : nullptr, gate_threshold,
                                           stream);
            if (rc != LSA_OK) return rc;
        }
        return LSA_OK;
    }
    if (!key_row_start || !seq_len || !entry_start || !z_out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: a required pointer is NULL");
    if (B <= 0 || H <= 0 || max_len < 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: B=%d H=%d max_len=%lld", B, H,
                    (long long)max_len);
    if (gate_bits && !aligned16(gate_bits))
        return fail(LSA_ERR_INVALID_ARG, "lsa_index_score_union: gate_bits must be 16-byte aligned");
    if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "lsa_index_score_union: B=%d > 65535", B);
    if (max_len > (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "lsa_index_score_union: max_len too large");
    int cus = 0;
    int rc = check_device(&cus);
    if (rc != LSA_OK) return rc;
    if (max_len == 0) return LSA_OK;
    UnionArgs ua{};
    for (int l = 0; l < n_idx; ++l) {
        ua.keys[l] = (const bf16*)keys[l];
        ua.q[l] = (const bf16*)q[l];
        ua.w[l] = w[l];
        ua.bias[l] = bias[l];
    }
    ua.n = n_idx;
    const int64_t groups = ceil_div(max_len, 16);
    int64_t gpw = (groups * B) / ((int64_t)cus * 4);
    gpw = gpw < 1 ? 1 : (gpw > kScoreGroupsPerWave ? kScoreGroupsPerWave : gpw);
    dim3 grid((unsigned)ceil_div(groups, gpw * 4), (unsigned)B);
    const int MT = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
    hipStream_t st = (hipStream_t)stream;
#define LSA_UNI(mt, kt)                                                                       \
    hipLaunchKernelGGL((k_score_union<mt, kt>), grid, dim3(256), 0, st, ua, key_row_start,     \
                       seq_len, entry_start, H, max_len, z_out, prob_out, gate_bits,         \
                       lsa_gate_words(max_len), gate_threshold)
    if (D == 128) {
        if (MT == 1) LSA_UNI(1, 4); else if (MT == 2) LSA_UNI(2, 4); else LSA_UNI(4, 4);
    } else {
        if (MT == 1) LSA_UNI(1, 2); else if (MT == 2) LSA_UNI(2, 2); else LSA_UNI(4, 2);
    }
#undef LSA_UNI
    return launch_status("score_union");
}
