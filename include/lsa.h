/*
 * lsa.h -- C ABI of the Lookahead Sparse Attention (LSA) hot path on MI355X (gfx950).
 *
 * The calls follow the decode path described on the page
 * "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via Lookahead
 * Sparse Attention" (gist.science/paper/2606.09079), Technical Summary
 * section 2.1 "Architectural Design":
 *   lsa_query_encode    -- the Memory Indexer's query encoder: hidden states
 *                          to the score's per-head queries and gate weights
 *                          ("Memory Indexer"; section 2.3);
 *   lsa_index_score     -- the Memory Indexer's lookahead index score I_{t,s}
 *                          against every preceding compressed entry ("Scoring
 *                          Mechanism"), with the OR-union over positions of
 *                          section 2.4 "Optimal Configuration";
 *   lsa_index_score_union -- the same score for the indexers of several
 *                          layers at once, united by OR (section 2.4
 *                          "Optimal Configuration");
 *   lsa_select_compact  -- keep every entry whose score reaches 0.5 ("Dynamic
 *                          Fetching"), as an ascending index list;
 *   lsa_index_rescore   -- the native indexer's per-step score of that
 *                          subset (rank keys for the next call);
 *   lsa_fetch_rows      -- copy the kept entries' rows from the cold pool
 *                          into a hot buffer ("Dynamic Fetching");
 *   lsa_topk            -- fine-grained top-k inside that subset ("Tiered
 *                          Selection");
 *   lsa_sparse_attend   -- the final core attention over the chosen entries
 *                          plus every heavily compressed (HCA, 128:1) entry,
 *                          which the design always keeps (opening paragraph of
 *                          section 2.1).  lsa_sparse_attend_hca and
 *                          lsa_sparse_attend_selected split it in two phases.
 * The output of each call is an input of the next.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless stated otherwise.  `stream` is a
 *   hipStream_t passed as void* (NULL = the null stream).  All work is
 *   enqueued asynchronously on `stream`; the library never synchronises.
 * - The caller owns every buffer, including the workspace (size it with
 *   lsa_workspace_bytes).  The library allocates and frees no device memory
 *   and keeps no pointer after a call returns.
 * - Ragged batches: sequence b (0 <= b < B) owns S_b = seq_len[b] compressed
 *   entries.  Its key rows are pool rows key_row_start[b] .. +S_b-1 (a start
 *   of 0 for every b shares one key set across the batch).  Per-entry outputs
 *   of sequence b (scores, candidate lists) live at element entry_start[b]
 *   of their arrays, so entry_start is normally the exclusive prefix sum of
 *   seq_len.  Entry indices s in index lists are relative to the sequence
 *   (0 <= s < S_b).
 * - max_len (host) must be >= every seq_len[b]; it sizes the grids without a
 *   device-to-host copy.  Device index arrays must satisfy the stated
 *   bounds; they are not checked on the host (that would need a sync).
 * - Row pools (keys, latent rows, HCA rows) are row-major with contiguous
 *   rows; base pointers and q/qa must be 16-byte aligned.
 * - Return value: LSA_OK, or a negative status.  Arguments are validated on
 *   the host before anything is enqueued; on error nothing is enqueued, no
 *   output is touched, and lsa_last_error() describes the problem.  Faults
 *   inside kernels surface at the caller's next synchronisation.
 * - Calls are reentrant and hold no global mutable state besides a
 *   thread-local error message, a per-device cache of the device's
 *   properties, and the built-in scratch array of lsa_select_compact_noalloc
 *   (one per GPU).
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_OK 0
#define LSA_ERR_INVALID_ARG (-1)  /* null pointer, bad size, misalignment, bad dtype  */
#define LSA_ERR_UNSUPPORTED (-2)  /* shape outside the kernels' envelope, not gfx950  */
#define LSA_ERR_WORKSPACE (-3)    /* workspace missing or smaller than required       */
#define LSA_ERR_HIP (-4)          /* the HIP runtime reported an error at launch      */

#define LSA_DTYPE_F32 0
#define LSA_DTYPE_BF16 1

#define LSA_OP_SELECT 1
#define LSA_OP_TOPK 2
#define LSA_OP_ATTEND 3

/* Gate bits: one uint16 word per group of 16 consecutive entries of a
 * sequence, bit i for entry 16 j + i of group j.  Sequence b's row starts at
 * word b * lsa_gate_words(max_len) = b * 8 * ceil(max_len / 128), so every
 * row is 16-byte aligned; words past ceil(S_b / 16) are not written. */
static inline int64_t lsa_gate_words(int64_t max_len) { return (max_len + 127) / 128 * 8; }

/* Lookahead index score (section 2.1 "Scoring Mechanism"; the query/key
 * interaction is a dot product per section 5 "Architectural Constraints").
 * This library's instance of the head-fused gated score:
 *     z[b,t,s] = sum_h w[b,t,h] * max(0, <q[b,t,h,:], k[b,s,:]>) + bias,
 *     I[b,t,s] = sigmoid(z[b,t,s]).
 *   keys   [rows, D] in `dtype` (LSA_DTYPE_BF16 or LSA_DTYPE_F32)
 *   q      [B, T, H, D], same dtype as keys
 *   w      [B, T, H] fp32 (any sign)
 *   bias   host fp32 scalar
 *   reduce_max = 0: z_out (and prob_out) hold, for sequence b, a [T, S_b]
 *                   block starting at element entry_start[b] * T.
 *   reduce_max = 1: z_out holds m[b,s] = max_t z[b,t,s] at element
 *                   entry_start[b] + s -- the OR-union of the per-position
 *                   gates of section 2.4 is exactly the gate on m;
 *                   prob_out, if given, holds sigmoid(m).
 *   reduce_max = 2: as 1, but z_out already holds the union of other
 *                   indexers (section 2.4's OR-mode across the indexers of
 *                   several layers: call once per indexer, the first with 1)
 *                   and receives max(z_out, m) (a NaN on either side yields
 *                   the other); prob_out, if given, holds its sigmoid.
 *   prob_out may be NULL.  Accumulation is fp32; bf16 products are exact.
 *   gate_bits, if not NULL (16-byte aligned, B rows of lsa_gate_words
 *              (max_len) words): the gate of section 2.1 "Dynamic Fetching"
 *              taken in the same launch on the value written to z_out --
 *              bit i of word j of row b is set iff entry 16 j + i < S_b and
 *              that logit >= gate_threshold (a NaN never passes).  It needs
 *              T = 1 or reduce_max != 0 (one logit per entry); with
 *              reduce_max = 2 the bits are those of the combined value.
 *              lsa_select_compact then compacts from the bits alone.
 * Envelope: B, T, H, D >= 1; the bf16 matrix-core path takes H <= 64 and
 * D in {64, 128}; other shapes (and fp32) use the vector path, which needs
 * T*H*(D+1) <= 16384.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_index_score(const void* keys, int dtype, const int64_t* key_row_start,
                    const int32_t* seq_len, const int64_t* entry_start, int B, int T, int H,
                    int D, int64_t max_len, const void* q, const float* w, float bias,
                    int reduce_max, float* z_out, float* prob_out, uint16_t* gate_bits,
                    float gate_threshold, void* stream);

/* OR-union of several indexers' scores in one call (section 2.4 "Optimal
 * Configuration": the indexers of three intermediate layers, united by OR; an
 * entry is kept when any indexer's gate keeps it, and as sigmoid is monotone
 * that is the gate on the largest logit).  For l = 0 .. n_idx-1, indexer l has its own keys[l],
 * q[l], w[l] and bias[l], laid out as for lsa_index_score; all share the
 * sequence layout (key_row_start, seq_len, entry_start), dtype, B, T, H, D.
 *   z_out[entry_start[b] + s] = max over l and t of z_l[b,t,s];
 *   prob_out, if not NULL, holds its sigmoid; gate_bits, if not NULL, the
 *   gate of that union against gate_threshold, laid out as for
 *   lsa_index_score.
 * keys, q, w and bias are HOST arrays of n_idx entries; the pointers in
 * keys, q and w are device pointers.  The bf16 matrix-core shapes with T = 1
 * (H <= 64, D in {64, 128}) stream every indexer's keys in one launch and
 * keep the running maximum in registers, so z_out is written once; the
 * result is bit-identical to calling lsa_index_score once per indexer
 * (reduce_max = 1, then 2), NaN logits included (an entry that every indexer
 * scores NaN stays NaN).  Other shapes make exactly those calls.
 * Envelope: 1 <= n_idx <= 4; otherwise as lsa_index_score.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_index_score_union(int n_idx, const void* const* keys, int dtype,
                          const int64_t* key_row_start, const int32_t* seq_len,
                          const int64_t* entry_start, int B, int T, int H, int D,
                          int64_t max_len, const void* const* q, const float* const* w,
                          const float* bias, float* z_out, float* prob_out,
                          uint16_t* gate_bits, float gate_threshold, void* stream);

/* Native re-score of the kept subset (section 2.1 "Tiered Selection": the
 * backbone's native Lightning Indexer takes the fine-grained top-k inside the
 * fetched subset; section 2.3 "Decoupled Training": the compressed indexer
 * keys are the backbone's frozen keys).  This library's reading: with its own
 * per-step queries q' and weights w' the native indexer scores only the
 * candidates, against the same key rows, as a ranking logit (no bias, no
 * sigmoid):
 *     r[b,s] = sum_h w'[b,h] * max(0, <q'[b,h,:], k[b,s,:]>)
 * for every candidate s = cand_idx[entry_start[b] + j], j < cand_count[b]
 * (lsa_select_compact's output layout), written at r_out[entry_start[b] + s]
 * -- where lsa_topk reads its rank keys.  Other elements of r_out are left
 * untouched.
 *   keys, key_row_start: as for lsa_index_score; seq_len[b] bounds the indices
 *              (an index outside [0, S_b) reads no key memory and writes
 *              nothing).
 *   q'  [B, H, D] in `dtype`; w' [B, H] fp32 (any sign).
 *   max_cand (host) >= every cand_count[b]; it sizes the grid.
 * Envelope: the bf16 matrix-core path takes H <= 64 and D in {64, 128} and a
 * sequence's keys spanning < 2 GiB; other shapes (and fp32) use the vector
 * path, which needs H*(D+1) <= 16384.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_index_rescore(const void* keys, int dtype, const int64_t* key_row_start,
                      const int32_t* seq_len, const int64_t* entry_start,
                      const int32_t* cand_idx, const int32_t* cand_count, int B, int H, int D,
                      int64_t max_cand, const void* q, const float* w, float* r_out,
                      void* stream);

/* Memory-Indexer query encoder (section 2.1 "Memory Indexer": the query
 * token's hidden state h_t is mapped into low-rank indexer queries; section
 * 2.3 "Query Optimization": the encoder's low-rank projection matrices).
 * For each of the M tokens (M = B*T, in the score's (b, t) order):
 *     c[m]       = W_down h[m]            rank r, rounded to bf16 in c_buf
 *     q[m, h, :] = W_up[h*D .. h*D+D-1] c[m]
 *     w[m, h]    = W_gate[h] . h[m]
 * fp32 accumulation; q is rounded to bf16, w stays fp32 -- exactly the q and
 * w that lsa_index_score takes.
 *   h       bf16 [M, d_model] row-major (device).
 *   w_down  bf16 [rank, d_model]; w_up bf16 [H*D, rank]; w_gate bf16 [H, d_model]:
 *           one weight row per output feature, row-major (device).
 *   c_buf   bf16 [M, rank], caller-owned; holds c on return.
 *   q_out   bf16 [M, H, D]; w_out fp32 [M, H].
 * Two launches on stream (the down and gate projections share the first).
 * Envelope: d_model and rank multiples of 64; h, the weights and c_buf
 * 16-byte aligned.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_query_encode(const void* h, int M, int d_model, int rank, int H, int D,
                     const void* w_down, const void* w_up, const void* w_gate, void* c_buf,
                     void* q_out, float* w_out, void* stream);

/* Dynamic fetching (section 2.1): keep every entry with I >= 0.5, with no
 * fixed count.  I >= 0.5 holds exactly when z >= 0, so the gate is taken on
 * the fp32 logit: candidate s of sequence b iff z[entry_start[b]+s] >=
 * threshold (pass 0.0f for the 0.5 gate; -0.0 passes, NaN never does).
 *   gate_bits  NULL: the gate is taken on z (two launches: per-tile counts,
 *              then the ordered scatter).  Otherwise the bits that
 *              lsa_index_score wrote in its launch for the same z, max_len
 *              and threshold (16-byte aligned): the kept set is the set bits,
 *              z is not read (it may be NULL), threshold and the workspace
 *              are not used (workspace may be NULL), and one launch compacts.
 *   cand_idx   int32, the ascending list of kept s for sequence b written at
 *              cand_idx[entry_start[b] ...]; capacity S_b per sequence.
 *   cand_count int32 [B].
 *   workspace  lsa_workspace_bytes(LSA_OP_SELECT, B, 0, 0, 0, max_len, 0, 0) bytes.
 * Deterministic: the list is in ascending s whatever the launch order; both
 * forms give the same list for bits made from the same logits.
 * Errors: INVALID_ARG, WORKSPACE, HIP. */
int lsa_select_compact(const float* z, const uint16_t* gate_bits, const int64_t* entry_start,
                       const int32_t* seq_len, int B, int64_t max_len, float threshold,
                       int32_t* cand_idx, int32_t* cand_count, void* workspace,
                       size_t workspace_bytes, void* stream);

/* lsa_select_compact without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as the z form
 * of lsa_select_compact (gate_bits NULL), minus the workspace (the bit form
 * needs none): the per-tile counts live in a
 * built-in device array of 2^18 int32 (1 MiB per GPU, held until the process
 * ends), so B * ceil(max_len / 2048) must not exceed 262144 (else
 * UNSUPPORTED).  The call allocates nothing.  Calls that overlap on one GPU
 * (other streams, other host threads) share that array and race; serialise
 * them.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_select_compact_noalloc(const float* z, const int64_t* entry_start,
                               const int32_t* seq_len, int B, int64_t max_len, float threshold,
                               int32_t* cand_idx, int32_t* cand_count, void* stream);

/* Tiered selection (section 2.1): the top-k candidates of each sequence by
 * rank key r[entry_start[b] + s] (fp32; the pipeline passes the indexer logit
 * or its max over positions).  Order: larger key first, equal keys by smaller
 * s, NaN after every number, -0.0 equal to +0.0.
 *   cand_idx/cand_count as written by lsa_select_compact (cand_count[b] <= S_b).
 *   topk_idx   int32 [B, k]: the kept s of sequence b in ascending order in
 *              row b; entries past topk_count[b] are left untouched.  With
 *              out_positions != 0 the row holds instead the kept entries'
 *              positions j in the candidate list (cand_idx[entry_start[b]+j]
 *              = s), also ascending: the rows of a hot buffer filled by
 *              lsa_fetch_rows from that list.
 *   topk_count int32 [B] = min(k, cand_count[b]).
 *   workspace  lsa_workspace_bytes(LSA_OP_TOPK, B, 0, 0, 0, max_len, k, 0) bytes.
 * Envelope: 1 <= k <= 65536.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int lsa_topk(const float* rank_key, const int64_t* entry_start, const int32_t* seq_len, int B,
             int64_t max_len, const int32_t* cand_idx, const int32_t* cand_count, int k,
             int32_t* topk_idx, int32_t* topk_count, int out_positions, void* workspace,
             size_t workspace_bytes, void* stream);

/* Just-in-time fetch of the kept entries (section 2.1 "Dynamic Fetching":
 * the entries whose score reaches 0.5 are fetched from the CPU-side cold pool
 * into GPU memory, which holds only this critical subset).  Row copy:
 *     dst row dst_row_start[b] + j  <-  src row src_row_start[b] + idx[idx_start[b] + j]
 * for j < count[b], each row row_bytes long.  With idx = cand_idx, idx_start =
 * entry_start and count = cand_count (lsa_select_compact's output), dst holds
 * sequence b's kept rows in list order; lsa_topk(..., out_positions = 1)
 * then names rows of dst, and lsa_sparse_attend can attend over dst with
 * latent_row_start = dst_row_start.
 *   src        host memory that is pinned and mapped into the device's
 *              address space (hipHostMalloc / a pinned torch tensor), or
 *              device memory; read by the GPU directly (zero copy).
 *              Pageable host memory is refused (INVALID_ARG).
 *   dst        device memory, rows of row_bytes; the caller sizes each
 *              sequence's rows for its largest count.
 *   row_bytes  a positive multiple of 16; src and dst 16-byte aligned.
 *   max_count (host) >= every count[b]; it sizes the grid.  idx values must
 *              be valid rows of sequence b's source range (not checked).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int lsa_fetch_rows(const void* src, int64_t row_bytes, const int64_t* src_row_start,
                   const int32_t* idx, const int64_t* idx_start, const int32_t* count, int B,
                   int64_t max_count, void* dst, const int64_t* dst_row_start, void* stream);

/* Core attention over the chosen entries plus all HCA entries (section 2.1).
 * One latent row per compressed entry serves as both key and value for all
 * Hq query heads.  For each (b, t, h) the attended rows are
 *     latent rows latent_row_start[b] + topk_idx[b*k + j], j < topk_count[b],
 *     then HCA rows hca_row_start[b] + i, i < hca_count[b];
 * logit_j = scale * <qa[b,t,h,:], row_j>,
 * out[b,t,h,:] = sum_j softmax(logit)_j * row_j,  lse[b,t,h] = logsumexp(logit).
 * Rows with no attended entry give out = 0 and lse = -inf.
 *   qa  [B, T, Hq, Dl] in `dtype`; latent and hca rows of Dl elements, same dtype.
 *   hca may be NULL (then hca_row_start/hca_count are ignored); otherwise
 *   hca_count[b] <= max_hca (host).
 *   out [B, T, Hq, Dl] in `dtype`; lse [B, T, Hq] fp32 or NULL.
 *   workspace  lsa_workspace_bytes(LSA_OP_ATTEND, B, T, Hq, Dl, 0, k, max_hca)
 *              bytes (split partial results); may be 0 for some shapes.
 * Envelope: the bf16 matrix-core path takes Dl in {128, 256, 512} and any Hq
 * (a sequence's T*Hq query rows are taken 64 at a time); other shapes (and
 * fp32) use the vector path (Dl <= 1024).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int lsa_sparse_attend(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                      const void* latent, const int64_t* latent_row_start,
                      const int32_t* topk_idx, const int32_t* topk_count, int k,
                      const void* hca, const int64_t* hca_row_start, const int32_t* hca_count,
                      int64_t max_hca, float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The same attention in two phases (section 2.1: the HCA entries are kept for
 * every query, whatever the selection, so their part of the softmax needs no
 * top-k list).  Softmax over a union of row sets is the log-sum-exp merge of
 * per-set partials, so the phases give the output of lsa_sparse_attend, bit
 * for bit, on the same arguments:
 *   lsa_sparse_attend_hca       partials over the HCA rows into `workspace`.
 *                               It reads neither the top-k list nor its
 *                               counts, so it may run while they are produced
 *                               (e.g. on a second stream beside lsa_topk).
 *   lsa_sparse_attend_selected  the top-k rows and the merge of all partials
 *                               into out/lse.  It takes every argument of
 *                               lsa_sparse_attend.
 * The selected phase must run after the HCA phase has completed, on the same
 * workspace and the same qa, dtype, B, T, Hq, Dl, k, hca, hca_row_start,
 * hca_count, max_hca and scale; the caller orders the two (one stream, or an
 * event between two streams).  The workspace is sized as for lsa_sparse_attend.
 * When that size is 0 or the shape takes the vector path, the HCA phase
 * enqueues nothing and the selected phase computes everything.
 * hca must not be NULL in lsa_sparse_attend_hca (INVALID_ARG).
 * Errors: as lsa_sparse_attend. */
int lsa_sparse_attend_hca(const void* qa, int dtype, int B, int T, int Hq, int Dl, int k,
                          const void* hca, const int64_t* hca_row_start,
                          const int32_t* hca_count, int64_t max_hca, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);
int lsa_sparse_attend_selected(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                               const void* latent, const int64_t* latent_row_start,
                               const int32_t* topk_idx, const int32_t* topk_count, int k,
                               const void* hca, const int64_t* hca_row_start,
                               const int32_t* hca_count, int64_t max_hca, float scale, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes needed by op (LSA_OP_*) for the given host-side sizes;
 * arguments an op does not use are ignored.  Returns 0 for an unknown op. */
size_t lsa_workspace_bytes(int op, int B, int T, int Hq, int Dl, int64_t max_len, int k,
                           int64_t max_hca);

/* Static description of a status code. */
const char* lsa_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* lsa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int lsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
