/*
 * lsa_oracle.c -- plain CPU reference of the Lookahead Sparse Attention hot
 * path.  TEST INFRASTRUCTURE ONLY (see lsa_oracle.h): slow, scalar, IEEE
 * double precision, written to be checked by eye against the definitions on
 * the page "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
 * Lookahead Sparse Attention" (gist.science), Technical Summary 2.1 and 2.4.
 *
 * Built with plain gcc, no -ffast-math, no intrinsics.  The same source is
 * built twice: once single-threaded (the parity build; the OpenMP pragmas
 * below are then ignored) and once with -fopenmp (the timing build, and the
 * build the full-size tests use).  The pragmas only share out iterations of
 * loops whose iterations are independent -- queries, entries, sequences,
 * (position, head) rows -- so every output element is computed by the same
 * scalar operations in the same order in both builds.
 */
#include "lsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below may use (1 in the single-threaded build). */
int lsa_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exact widening of one stored element to double. */
static double load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == 0) {
        return (double)((const float*)base)[i];
    }
    /* bf16: the 16 stored bits are the upper half of an fp32 pattern. */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int dtype_ok(int dtype) { return dtype == 0 || dtype == 1; }

/* O0 -- TS 2.1 "Memory Indexer" and TS 2.3 "Query Optimization": two low-rank
 * projections for the queries, one linear projection for the gate weights. */
int lsa_ref_query_encode(const void* h, int dtype, int M, int d_model, int r, int H, int D,
                         const void* w_down, const void* w_up, const void* w_gate,
                         double* c_out, double* q_out, double* w_out) {
    if (!h || !w_down || !w_up || !w_gate || !c_out || !q_out || !w_out) return -1;
    if (M <= 0 || d_model <= 0 || r <= 0 || H <= 0 || D <= 0 || !dtype_ok(dtype)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        const int64_t hrow = (int64_t)m * d_model;
        /* the low-rank latent of this token */
        for (int i = 0; i < r; ++i) {
            double acc = 0.0;
            for (int k = 0; k < d_model; ++k)
                acc += load_elem(w_down, dtype, (int64_t)i * d_model + k) *
                       load_elem(h, dtype, hrow + k);
            c_out[(int64_t)m * r + i] = acc;
        }
        /* each head's query from the latent */
        for (int hd = 0; hd < H; ++hd) {
            for (int d = 0; d < D; ++d) {
                const int64_t urow = ((int64_t)hd * D + d) * r;
                double acc = 0.0;
                for (int i = 0; i < r; ++i)
                    acc += load_elem(w_up, dtype, urow + i) * c_out[(int64_t)m * r + i];
                q_out[((int64_t)m * H + hd) * D + d] = acc;
            }
        }
        /* each head's gate weight from the hidden state */
        for (int hd = 0; hd < H; ++hd) {
            double acc = 0.0;
            for (int k = 0; k < d_model; ++k)
                acc += load_elem(w_gate, dtype, (int64_t)hd * d_model + k) *
                       load_elem(h, dtype, hrow + k);
            w_out[(int64_t)m * H + hd] = acc;
        }
    }
    return 0;
}

/* O1 -- TS 2.1 "Scoring Mechanism"; dot-product interaction per TS 5. */
int lsa_ref_index_score(const void* keys, int dtype, const int64_t* key_row_start,
                        const int32_t* seq_len, const int64_t* entry_start,
                        int B, int T, int H, int D,
                        const void* q, const float* w, double bias, int reduce_max,
                        double* z_out, double* prob_out) {
    if (!keys || !key_row_start || !seq_len || !entry_start || !q || !w || !z_out) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || !dtype_ok(dtype)) return -1;
    if (reduce_max < 0 || reduce_max > 2) return -1;

    for (int b = 0; b < B; ++b) {
        const int64_t S = seq_len[b];
#pragma omp parallel for schedule(dynamic, 256)
        for (int64_t s = 0; s < S; ++s) {
            const int64_t krow = (key_row_start[b] + s) * (int64_t)D;
            double m = -INFINITY;
            for (int t = 0; t < T; ++t) {
                double u = 0.0;
                for (int h = 0; h < H; ++h) {
                    const int64_t qrow = (((int64_t)b * T + t) * H + h) * (int64_t)D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) {
                        dot += load_elem(q, dtype, qrow + d) * load_elem(keys, dtype, krow + d);
                    }
                    const double gated = dot > 0.0 ? dot : 0.0;   /* ReLU gate */
                    u += (double)w[((int64_t)b * T + t) * H + h] * gated;
                }
                const double z = u + bias;
                if (!reduce_max) {
                    const int64_t o = entry_start[b] * T + (int64_t)t * S + s;
                    z_out[o] = z;
                    if (prob_out) prob_out[o] = 1.0 / (1.0 + exp(-z));
                } else if (t == 0 || z > m) {
                    m = z;
                }
            }
            if (reduce_max) {
                /* TS 2.4 OR-mode over indexers: keep the larger of the union so far
                 * and this indexer's maximum (a NaN on either side yields the other) */
                const double prev = z_out[entry_start[b] + s];
                if (reduce_max == 2 && (isnan(m) || prev > m)) m = prev;
                z_out[entry_start[b] + s] = m;
                if (prob_out) prob_out[entry_start[b] + s] = 1.0 / (1.0 + exp(-m));
            }
        }
    }
    return 0;
}

/* O1b -- TS 2.1 "Tiered Selection" (native indexer inside the fetched subset),
 * TS 2.3 (frozen compressed keys); no bias and no sigmoid in this reading. */
int lsa_ref_index_rescore(const void* keys, int dtype, const int64_t* key_row_start,
                          const int64_t* entry_start, const int32_t* cand_idx,
                          const int32_t* cand_count, int B, int H, int D,
                          const void* q, const float* w, double* r_out) {
    if (!keys || !key_row_start || !entry_start || !cand_idx || !cand_count || !q || !w || !r_out)
        return -1;
    if (B <= 0 || H <= 0 || D <= 0 || !dtype_ok(dtype)) return -1;
    for (int b = 0; b < B; ++b) {
#pragma omp parallel for schedule(dynamic, 64)
        for (int32_t j = 0; j < cand_count[b]; ++j) {
            const int32_t s = cand_idx[entry_start[b] + j];
            const int64_t krow = (key_row_start[b] + s) * (int64_t)D;
            double r = 0.0;
            for (int h = 0; h < H; ++h) {
                const int64_t qrow = ((int64_t)b * H + h) * (int64_t)D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += load_elem(q, dtype, qrow + d) * load_elem(keys, dtype, krow + d);
                r += (double)w[(int64_t)b * H + h] * (dot < 0.0 ? 0.0 : dot);   /* ReLU gate */
            }
            r_out[entry_start[b] + s] = r;
        }
    }
    return 0;
}

/* O2 -- TS 2.1 "Dynamic Fetching" (keep every entry with I >= 0.5, i.e. z >= 0),
 * TS 2.4 (OR-union, applied by the caller through the maximum logit). */
int lsa_ref_select(const double* z, const int64_t* entry_start, const int32_t* seq_len,
                   int B, double threshold, int32_t* cand_idx, int32_t* cand_count) {
    if (!z || !entry_start || !seq_len || !cand_idx || !cand_count || B <= 0) return -1;
    for (int b = 0; b < B; ++b) {
        int32_t n = 0;
        for (int64_t s = 0; s < seq_len[b]; ++s) {
            const double v = z[entry_start[b] + s];
            if (v >= threshold) {          /* false for NaN */
                cand_idx[entry_start[b] + n] = (int32_t)s;
                ++n;
            }
        }
        cand_count[b] = n;
    }
    return 0;
}

typedef struct {
    double r;
    int32_t s;
    int32_t j;    /* position in the candidate list */
} ranked_t;

/* Order: larger r first; NaN after every number; equal r -> smaller s first. */
static int by_rank(const void* pa, const void* pb) {
    const ranked_t* a = (const ranked_t*)pa;
    const ranked_t* b = (const ranked_t*)pb;
    const int an = isnan(a->r), bn = isnan(b->r);
    if (an != bn) return an ? 1 : -1;
    if (!an && a->r != b->r) return a->r > b->r ? -1 : 1;
    return (a->s > b->s) - (a->s < b->s);
}

static int by_index(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* O3 -- TS 2.1 "Tiered Selection". */
int lsa_ref_topk(const double* r, const int64_t* entry_start, const int32_t* seq_len,
                 int B, const int32_t* cand_idx, const int32_t* cand_count, int k,
                 int out_positions, int32_t* topk_idx, int32_t* topk_count) {
    if (!r || !entry_start || !seq_len || !cand_idx || !cand_count || !topk_idx || !topk_count)
        return -1;
    if (B <= 0 || k <= 0) return -1;
    for (int b = 0; b < B; ++b)
        if (cand_count[b] < 0 || cand_count[b] > seq_len[b]) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int32_t n = cand_count[b];
        ranked_t* items = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(n > 0 ? n : 1));
        if (!items) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int32_t j = 0; j < n; ++j) {
            const int32_t s = cand_idx[entry_start[b] + j];
            items[j].s = s;
            items[j].j = j;
            items[j].r = r[entry_start[b] + s];
        }
        qsort(items, (size_t)n, sizeof(ranked_t), by_rank);
        const int32_t keep = n < k ? n : k;
        int32_t* out = topk_idx + (int64_t)b * k;
        for (int32_t j = 0; j < keep; ++j) out[j] = out_positions ? items[j].j : items[j].s;
        qsort(out, (size_t)keep, sizeof(int32_t), by_index);
        topk_count[b] = keep;
        free(items);
    }
    return failed ? -1 : 0;
}

/* O4 -- TS 2.1 final core attention over the top-k entries plus all HCA rows. */
int lsa_ref_sparse_attend(const void* qa, int dtype, int B, int T, int Hq, int Dl,
                          const void* latent, const int64_t* latent_row_start,
                          const int32_t* topk_idx, const int32_t* topk_count, int k,
                          const void* hca, const int64_t* hca_row_start,
                          const int32_t* hca_count, double scale,
                          double* out, double* lse) {
    if (!qa || !latent || !latent_row_start || !topk_idx || !topk_count || !out) return -1;
    if (B <= 0 || T <= 0 || Hq <= 0 || Dl <= 0 || k <= 0 || !dtype_ok(dtype)) return -1;
    if (hca && (!hca_row_start || !hca_count)) return -1;

    int failed = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t nt = topk_count[b];
        const int32_t nh = hca ? hca_count[b] : 0;
        const int32_t n = nt + nh;
        /* element offset of attended row j */
        int64_t* row_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
        const void** row_src = (const void**)malloc(sizeof(void*) * (size_t)(n > 0 ? n : 1));
        if (!row_off || !row_src) {
            free(row_off);
            free((void*)row_src);
            return -1;
        }
        for (int32_t j = 0; j < nt; ++j) {
            row_src[j] = latent;
            row_off[j] = (latent_row_start[b] + topk_idx[(int64_t)b * k + j]) * (int64_t)Dl;
        }
        for (int32_t i = 0; i < nh; ++i) {
            row_src[nt + i] = hca;
            row_off[nt + i] = (hca_row_start[b] + i) * (int64_t)Dl;
        }
        /* every (position, head) row of sequence b is independent of the others */
#pragma omp parallel
        {
            double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            if (!logit) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int th = 0; th < T * Hq; ++th) {
                if (!logit) continue;
                const int t = th / Hq, h = th % Hq;
                const int64_t qoff = (((int64_t)b * T + t) * Hq + h) * (int64_t)Dl;
                double* o = out + qoff;
                for (int d = 0; d < Dl; ++d) o[d] = 0.0;
                const int64_t lidx = ((int64_t)b * T + t) * Hq + h;
                if (n == 0) {
                    if (lse) lse[lidx] = -INFINITY;
                    continue;
                }
                double mu = -INFINITY;
                for (int32_t j = 0; j < n; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < Dl; ++d)
                        dot += load_elem(qa, dtype, qoff + d) * load_elem(row_src[j], dtype, row_off[j] + d);
                    logit[j] = scale * dot;
                    if (logit[j] > mu) mu = logit[j];
                }
                double Z = 0.0;
                for (int32_t j = 0; j < n; ++j) {
                    const double p = exp(logit[j] - mu);
                    Z += p;
                    for (int d = 0; d < Dl; ++d) o[d] += p * load_elem(row_src[j], dtype, row_off[j] + d);
                }
                for (int d = 0; d < Dl; ++d) o[d] /= Z;
                if (lse) lse[lidx] = mu + log(Z);
            }
            free(logit);
        }
        free(row_off);
        free((void*)row_src);
    }
    return failed ? -1 : 0;
}

/* O5 -- TS 2.1 "Dynamic Fetching": the kept rows, copied in list order. */
int lsa_ref_fetch_rows(const void* src, int64_t row_bytes, const int64_t* src_row_start,
                       const int32_t* idx, const int64_t* idx_start, const int32_t* count,
                       int B, void* dst, const int64_t* dst_row_start) {
    if (!src || !src_row_start || !idx || !idx_start || !count || !dst || !dst_row_start) return -1;
    if (B <= 0 || row_bytes <= 0) return -1;
    for (int b = 0; b < B; ++b) {
        for (int32_t j = 0; j < count[b]; ++j) {
            const int64_t from = src_row_start[b] + idx[idx_start[b] + j];
            const int64_t to = dst_row_start[b] + j;
            memcpy((char*)dst + to * row_bytes, (const char*)src + from * row_bytes,
                   (size_t)row_bytes);
        }
    }
    return 0;
}
