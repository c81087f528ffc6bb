/*
 * lsa_oracle.h -- plain CPU reference of the Lookahead Sparse Attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this library; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library under lookahead_sparse_kv_amd/csrc.
 *
 * Source of the method: the page "FlashMemory-DeepSeek-V4: Lightning Index
 * Ultra-Long Context via Lookahead Sparse Attention" (gist.science/paper/
 * 2606.09079), section "Technical Summary" 2.1 "Architectural Design"
 * (cited below as TS 2.1), and 2.4 "Optimal Configuration" (TS 2.4).
 *
 * Arithmetic: every floating-point step runs in IEEE double precision with
 * scalar loops.  bf16 and fp32 inputs are widened exactly.  Index arrays
 * (row starts, lengths, candidate lists) are host arrays here.
 *
 * Dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns, upper half of fp32).
 */
#ifndef LSA_ORACLE_H
#define LSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the oracle's loops may use: 1 in the single-threaded parity build,
 * the OpenMP thread count in the timing build (same source, -fopenmp). */
int lsa_ref_max_threads(void);

/* O1  Lookahead index score (TS 2.1 "Scoring Mechanism": a head-fused gated
 * matching score passed through a sigmoid; TS 5 "Architectural Constraints":
 * the query/key interaction is a dot product).  The instance computed here:
 *   u[b,t,s] = sum_h w[b,t,h] * max(0, sum_d q[b,t,h,d] * k[b,s,d])
 *   z = u + bias,   I = 1 / (1 + exp(-z)).
 * keys: pool of rows of D elements; sequence b's entry s is row
 *       key_row_start[b] + s.  seq_len[b] = S_b entries.
 * q: [B,T,H,D] (same dtype as keys); w: [B,T,H] fp32.
 * reduce_max = 0: z_out/prob_out hold [T,S_b] for sequence b starting at
 *                 element entry_start[b]*T.
 * reduce_max = 1: z_out holds m[b,s] = max_t z[b,t,s] at entry_start[b]+s
 *                 (TS 2.4: union of gates = gate on the maximum logit);
 *                 prob_out, if given, holds sigmoid(m).
 * reduce_max = 2: as 1, but z_out already holds the union of other indexers
 *                 (the several layers of TS 2.4, "OR-mode") and receives
 *                 max(z_out, m); prob_out, if given, holds sigmoid of that.
 * prob_out may be NULL.  Returns 0, or -1 on a bad argument. */
int lsa_ref_index_score(const void* keys, int dtype, const int64_t* key_row_start,
                        const int32_t* seq_len, const int64_t* entry_start,
                        int B, int T, int H, int D,
                        const void* q, const float* w, double bias, int reduce_max,
                        double* z_out, double* prob_out);

/* O1b Native re-score of the kept subset (TS 2.1 "Tiered Selection": inside
 * the fetched subset the backbone's native Lightning Indexer takes a
 * fine-grained top-k; TS 2.3: the compressed indexer keys are the frozen
 * keys K_IComp, shared with the Memory Indexer).  The reading taken here: the
 * native indexer scores a candidate with its own per-step queries q' and
 * weights w' against the same key rows, as a plain ranking logit (no bias,
 * no sigmoid):
 *   r[b,s] = sum_h w'[b,h] * max(0, sum_d q'[b,h,d] * k[b,s,d])
 * for every candidate s = cand_idx[entry_start[b]+j], j < cand_count[b],
 * written at r_out[entry_start[b]+s]; other elements of r_out are untouched.
 * q': [B,H,D] (same dtype as keys); w': [B,H] fp32.  Returns 0 or -1. */
int lsa_ref_index_rescore(const void* keys, int dtype, const int64_t* key_row_start,
                          const int64_t* entry_start, const int32_t* cand_idx,
                          const int32_t* cand_count, int B, int H, int D,
                          const void* q, const float* w, double* r_out);

/* O2  Dynamic fetching (TS 2.1 "Dynamic Fetching": every entry whose score
 * reaches 0.5 is kept, with no fixed count).  Since sigmoid(z) >= 0.5 exactly
 * when z >= 0, the gate is applied to the logit: cand = [s ascending :
 * z[entry_start[b]+s] >= threshold].  NaN is never kept.  cand_idx for
 * sequence b is written at cand_idx[entry_start[b] ...]; cand_count[b] is its
 * length. */
int lsa_ref_select(const double* z, const int64_t* entry_start, const int32_t* seq_len,
                   int B, double threshold, int32_t* cand_idx, int32_t* cand_count);

/* O3  Tiered selection (TS 2.1 "Tiered Selection": a fine-grained top-k
 * inside the kept subset).  Candidates of sequence b are ordered by rank key
 * r[entry_start[b]+s] descending, equal keys by smaller s first, NaN last;
 * the first min(k, count) are kept and written in ascending s to
 * topk_idx[b*k ...]; topk_count[b] = min(k, count).  With out_positions != 0
 * the row holds instead each kept entry's position j in the candidate list
 * (cand_idx[entry_start[b]+j] = s), ascending. */
int lsa_ref_topk(const double* r, const int64_t* entry_start, const int32_t* seq_len,
                 int B, const int32_t* cand_idx, const int32_t* cand_count, int k,
                 int out_positions, int32_t* topk_idx, int32_t* topk_count);

/* O0  Memory-Indexer query encoder (TS 2.1 "Memory Indexer": the query
 * token's hidden state h_t mapped into low-rank indexer queries; TS 2.3
 * "Query Optimization": low-rank projection matrices).  For token m:
 *   c[m]       = W_down h[m]              rank r
 *   q[m, h, :] = W_up[h*D .. h*D+D-1] c[m] D per indexer head
 *   w[m, h]    = W_gate[h] . h[m]         the head's gate weight
 * h [M, d_model], W_down [r, d_model], W_up [H*D, r], W_gate [H, d_model],
 * all of dtype (0 fp32, 1 bf16) and row-major; outputs fp64 c [M, r],
 * q [M, H, D], w [M, H]. */
int lsa_ref_query_encode(const void* h, int dtype, int M, int d_model, int r, int H, int D,
                         const void* w_down, const void* w_up, const void* w_gate,
                         double* c_out, double* q_out, double* w_out);

/* O5  Just-in-time fetch (TS 2.1 "Dynamic Fetching": the kept entries are
 * fetched from the CPU-side cold pool into GPU memory).  Row copy:
 *   dst row dst_row_start[b]+j = src row src_row_start[b] + idx[idx_start[b]+j]
 * for j < count[b]; rows are row_bytes long; other dst rows are untouched. */
int lsa_ref_fetch_rows(const void* src, int64_t row_bytes, const int64_t* src_row_start,
                       const int32_t* idx, const int64_t* idx_start, const int32_t* count,
                       int B, void* dst, const int64_t* dst_row_start);

/* O4  Core attention over the chosen entries (TS 2.1 "Tiered Selection",
 * final core attention) together with every heavily compressed (HCA) entry,
 * all of which are always retained (TS 2.1 opening paragraph, 128:1 HCA).
 * Latent rows serve as both key and value for every query head.
 * For each (b,t,h): rows A_b = latent rows latent_row_start[b]+topk_idx[b*k+j]
 * (j < topk_count[b]) followed by HCA rows hca_row_start[b]+i (i <
 * hca_count[b]); logit_j = scale * <qa[b,t,h,:], row_j>;
 * out = sum_j softmax(logit)_j * row_j, lse = logsumexp(logit).
 * An empty A_b gives out = 0 and lse = -inf.  hca may be NULL (no HCA rows).
 * qa: [B,T,Hq,Dl]; latent/hca rows of Dl elements; all of one dtype.
 * out: [B,T,Hq,Dl] double; lse: [B,T,Hq] double (may be NULL). */
int lsa_ref_sparse_attend(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                          const void* latent, const int64_t* latent_row_start,
                          const int32_t* topk_idx, const int32_t* topk_count, int k,
                          const void* hca, const int64_t* hca_row_start,
                          const int32_t* hca_count, double scale,
                          double* out, double* lse);

#ifdef __cplusplus
}
#endif

#endif
