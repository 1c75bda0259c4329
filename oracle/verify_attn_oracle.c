/*
 * CPU oracle for MLA tree-verify attention (test infrastructure only).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library. The HIP product path never links, calls or falls back
 * to it, and it shares no code, header or table with that path.
 *
 * What it computes (plain definition, fp64 arithmetic throughout):
 * speculative-decoding verify attention for Multi-head Latent Attention.
 * Draft tokens are verified by attending to the whole KV cache ("The
 * Milestone Commit", Input Knowledge), in the extend layout where a sequence's prefix
 * KV slots come first and the draft tokens' slots follow them, with a custom
 * mask of stride prefix + q_len ("The Checkpoint Report", Mistakes and
 * Incorrect Assumptions). The draft tokens form a DDTree draft tree, so the
 * mask lets each draft node see the whole prefix plus itself and its
 * ancestors in the tree.
 *
 * For sequence b, draft node t < T and head h:
 *   seg_b  = seq_lens[0] + ... + seq_lens[b-1]
 *   P_b    = seq_lens[b] - T                       (prefix length)
 *   K_j    = kv_pool[slot_idx[seg_b + j]]          (576 values, j < P_b + T)
 *   V_j    = first 512 values of K_j
 *   vis(t) = {0 .. P_b-1}  U  {P_b + u : u == t or u an ancestor of t}
 *            (ancestors: follow tree_parent from t until -1)
 *   s_j    = sm_scale * sum_{d<576} q[b,t,h,d] * K_j[d]      for j in vis(t)
 *   w_j    = exp(s_j - max s) / sum_{i in vis(t)} exp(s_i - max s)
 *   out[b,t,h,d] = sum_{j in vis(t)} w_j * V_j[d]          d < 512
 *
 * Layouts: q [B, T, H, 576] bf16 bits; kv_pool [pool_slots, 576] bf16 bits;
 * slot_idx int32 [sum seq_lens]; seq_lens int32 [B]; tree_parent int32 [B, T];
 * out fp64 [B, T, H, 512]. The *_f32 entry points take q and kv_pool as IEEE
 * binary32 values instead (the data type of the first, fp32 kernel of "The
 * Checkpoint Report", Architecture of the Report); everything else is the same.
 *
 * The exponent is taken relative to the exact maximum (two passes), and the
 * sums run over j in increasing order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KV_DIM 576
#define V_DIM 512

enum {
    ORACLE_OK = 0,
    ORACLE_BAD_ARG = -1,
    ORACLE_BAD_TREE = -2,
    ORACLE_BAD_SLOT = -3,
    ORACLE_NO_MEMORY = -4,
};

/* A bfloat16 value is the upper half of an IEEE binary32 value. */
static double bf16_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element idx of a q or kv_pool array: bf16 bits, or binary32 when f32 != 0. */
static double elem(const void* base, int64_t idx, int f32) {
    if (f32) return (double)((const float*)base)[idx];
    return bf16_to_double(((const uint16_t*)base)[idx]);
}

/* Check the host-side inputs the definition relies on. */
static int check_inputs(int B, int H, int T, int64_t pool_slots, const int32_t* slot_idx,
                        const int32_t* seq_lens, const int32_t* tree_parent) {
    if (B < 1 || H < 1 || T < 1 || pool_slots < 1) return ORACLE_BAD_ARG;
    int64_t seg = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < T) return ORACLE_BAD_ARG;
        for (int t = 0; t < T; ++t) {
            int p = tree_parent[(int64_t)b * T + t];
            if (p < -1 || p >= t) return ORACLE_BAD_TREE;
        }
        for (int64_t j = 0; j < seq_lens[b]; ++j) {
            int32_t s = slot_idx[seg + j];
            if (s < 0 || s >= pool_slots) return ORACLE_BAD_SLOT;
        }
        seg += seq_lens[b];
    }
    return ORACLE_OK;
}

/* visible[j] for j < P + T, for draft node t of sequence b. */
static void visible_set(int P, int T, int t, const int32_t* parent_b, unsigned char* visible) {
    for (int j = 0; j < P; ++j) visible[j] = 1;
    for (int u = 0; u < T; ++u) visible[P + u] = 0;
    for (int u = t; u != -1; u = parent_b[u]) visible[P + u] = 1;
}

/*
 * One output row (b, t, h). scores/visible are caller scratch of length
 * seq_lens[b]. If weights != NULL it receives w_j for every j < seq_lens[b]
 * (0 for keys outside vis(t)).
 */
static void attend_row(int B, int H, int T, const void* q, const void* kv_pool, int f32,
                       const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                       double sm_scale, int b, int t, int h, double* scores, unsigned char* visible,
                       double* out_row, double* weights) {
    (void)B;
    int64_t seg = 0;
    for (int i = 0; i < b; ++i) seg += seq_lens[i];
    const int N = seq_lens[b];
    const int P = N - T;
    visible_set(P, T, t, tree_parent + (int64_t)b * T, visible);

    const int64_t qrow = (((int64_t)b * T + t) * H + h) * KV_DIM;
    double qd[KV_DIM];
    for (int d = 0; d < KV_DIM; ++d) qd[d] = elem(q, qrow + d, f32);

    /* pass 1: scores and their maximum */
    double smax = -INFINITY;
    for (int j = 0; j < N; ++j) {
        if (!visible[j]) continue;
        const int64_t krow = (int64_t)slot_idx[seg + j] * KV_DIM;
        double dot = 0.0;
        for (int d = 0; d < KV_DIM; ++d) dot += qd[d] * elem(kv_pool, krow + d, f32);
        scores[j] = sm_scale * dot;
        if (scores[j] > smax) smax = scores[j];
    }
    /* pass 2: normaliser */
    double denom = 0.0;
    for (int j = 0; j < N; ++j)
        if (visible[j]) denom += exp(scores[j] - smax);
    /* pass 3: weighted sum of the value rows */
    for (int d = 0; d < V_DIM; ++d) out_row[d] = 0.0;
    for (int j = 0; j < N; ++j) {
        double w = visible[j] ? exp(scores[j] - smax) / denom : 0.0;
        if (weights) weights[j] = w;
        if (w == 0.0) continue;
        const int64_t vrow = (int64_t)slot_idx[seg + j] * KV_DIM;
        for (int d = 0; d < V_DIM; ++d) out_row[d] += w * elem(kv_pool, vrow + d, f32);
    }
}

static int max_len(int B, const int32_t* seq_lens) {
    int m = 0;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > m) m = seq_lens[b];
    return m;
}

/* Selected rows: rows_bth holds nrows triples (b, t, h); out is [nrows, 512]. */
static int verify_rows(int B, int H, int T, const void* q, const void* kv_pool, int f32,
                       int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                       const int32_t* tree_parent, double sm_scale, int64_t nrows,
                       const int32_t* rows_bth, double* out, int nthreads) {
    int rc = check_inputs(B, H, T, pool_slots, slot_idx, seq_lens, tree_parent);
    if (rc) return rc;
    for (int64_t r = 0; r < nrows; ++r) {
        int b = rows_bth[3 * r], t = rows_bth[3 * r + 1], h = rows_bth[3 * r + 2];
        if (b < 0 || b >= B || t < 0 || t >= T || h < 0 || h >= H) return ORACLE_BAD_ARG;
    }
    const int N = max_len(B, seq_lens);
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)N);
        unsigned char* visible = (unsigned char*)malloc((size_t)N);
        if (!scores || !visible) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t r = 0; r < nrows; ++r)
                attend_row(B, H, T, q, kv_pool, f32, slot_idx, seq_lens, tree_parent, sm_scale,
                           rows_bth[3 * r], rows_bth[3 * r + 1], rows_bth[3 * r + 2], scores,
                           visible, out + r * V_DIM, NULL);
        }
        free(scores);
        free(visible);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_verify_attn_rows(int B, int H, int T, const uint16_t* q, const uint16_t* kv_pool,
                            int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                            const int32_t* tree_parent, double sm_scale, int64_t nrows,
                            const int32_t* rows_bth, double* out, int nthreads) {
    return verify_rows(B, H, T, q, kv_pool, 0, pool_slots, slot_idx, seq_lens, tree_parent,
                       sm_scale, nrows, rows_bth, out, nthreads);
}

int oracle_verify_attn_rows_f32(int B, int H, int T, const float* q, const float* kv_pool,
                                int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                                const int32_t* tree_parent, double sm_scale, int64_t nrows,
                                const int32_t* rows_bth, double* out, int nthreads) {
    return verify_rows(B, H, T, q, kv_pool, 1, pool_slots, slot_idx, seq_lens, tree_parent,
                       sm_scale, nrows, rows_bth, out, nthreads);
}

/* Every row: out is [B, T, H, 512]. */
static int verify_all(int B, int H, int T, const void* q, const void* kv_pool, int f32,
                      int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                      const int32_t* tree_parent, double sm_scale, double* out, int nthreads) {
    const int64_t nrows = (int64_t)B * T * H;
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)nrows);
    if (!rows) return ORACLE_NO_MEMORY;
    int64_t r = 0;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h, ++r) {
                rows[3 * r] = b;
                rows[3 * r + 1] = t;
                rows[3 * r + 2] = h;
            }
    int rc = verify_rows(B, H, T, q, kv_pool, f32, pool_slots, slot_idx, seq_lens, tree_parent,
                         sm_scale, nrows, rows, out, nthreads);
    free(rows);
    return rc;
}

int oracle_verify_attn(int B, int H, int T, const uint16_t* q, const uint16_t* kv_pool,
                       int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                       const int32_t* tree_parent, double sm_scale, double* out, int nthreads) {
    return verify_all(B, H, T, q, kv_pool, 0, pool_slots, slot_idx, seq_lens, tree_parent,
                      sm_scale, out, nthreads);
}

int oracle_verify_attn_f32(int B, int H, int T, const float* q, const float* kv_pool,
                           int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                           const int32_t* tree_parent, double sm_scale, double* out, int nthreads) {
    return verify_all(B, H, T, q, kv_pool, 1, pool_slots, slot_idx, seq_lens, tree_parent,
                      sm_scale, out, nthreads);
}

/* Softmax weights of one row: weights has seq_lens[b] entries; out_row 512. */
int oracle_row_weights(int B, int H, int T, const uint16_t* q, const uint16_t* kv_pool,
                       int64_t pool_slots, const int32_t* slot_idx, const int32_t* seq_lens,
                       const int32_t* tree_parent, double sm_scale, int b, int t, int h,
                       double* weights, double* out_row) {
    int rc = check_inputs(B, H, T, pool_slots, slot_idx, seq_lens, tree_parent);
    if (rc) return rc;
    if (b < 0 || b >= B || t < 0 || t >= T || h < 0 || h >= H) return ORACLE_BAD_ARG;
    const int N = seq_lens[b];
    double* scores = (double*)malloc(sizeof(double) * (size_t)N);
    unsigned char* visible = (unsigned char*)malloc((size_t)N);
    if (!scores || !visible) {
        free(scores);
        free(visible);
        return ORACLE_NO_MEMORY;
    }
    attend_row(B, H, T, q, kv_pool, 0, slot_idx, seq_lens, tree_parent, sm_scale, b, t, h, scores,
               visible, out_row, weights);
    free(scores);
    free(visible);
    return ORACLE_OK;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
