/*
 * vegas_oracle.c -- plain, slow, obviously correct CPU reference of the Vegas
 * attention hot path (verification attention with logit collection, exact
 * top-k selection, index-gathered decode attention).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.
 *
 * All arithmetic is IEEE double.  The loops follow the definitions in the
 * order the pages state them; the only parallelism is an OpenMP loop over
 * independent (sequence, KV head) or (sequence, query head) tasks, which
 * does not change any summation order.
 */
#include "vegas_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Widen one stored element to double.  bf16 is the upper half of an IEEE
 * binary32 pattern, so shifting it into place is exact. */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == VO_DTYPE_F32) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* <q_row, k_row> over head_dim elements, in double. */
static double dot_rows(const void* q, int64_t q_off, const void* k, int64_t k_off,
                       int dtype, int head_dim) {
    double acc = 0.0;
    for (int d = 0; d < head_dim; ++d)
        acc += load_elem(q, dtype, q_off + d) * load_elem(k, dtype, k_off + d);
    return acc;
}

/* Softmax over z[0..n) followed by the weighted sum of the listed value rows:
 * out[d] = sum_j exp(z_j - max z) * v[row_j, d] / sum_j exp(z_j - max z).
 * rows[j] is the absolute value-row offset (in elements) of key j. */
static void softmax_weighted_sum(const double* z, const int64_t* rows, int64_t n,
                                 const void* v, int dtype, int head_dim,
                                 double* out) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (z[j] > m) m = z[j];
    double den = 0.0;
    for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(z[j] - m);
        den += w;
        for (int d = 0; d < head_dim; ++d) out[d] += w * load_elem(v, dtype, rows[j] + d);
    }
    for (int d = 0; d < head_dim; ++d) out[d] /= den;
}

static int shape_ok(int dtype, int batch, int hq, int hkv, int d) {
    if (dtype != VO_DTYPE_F32 && dtype != VO_DTYPE_BF16) return 0;
    if (batch < 0 || hq <= 0 || hkv <= 0 || d <= 0) return 0;
    if (hq % hkv != 0) return 0;
    return 1;
}

/*
 * Verification attention (page "Vegas ...", sec. 4 "Attention kernel
 * implementation": the logits are read after the causal mask and before
 * softmax normalisation) with Collect-2-Query style collection (sec. 3.3;
 * gist.science summary sec. 2B): the collected rows are the set given by
 * collect_mask, and the collected quantity is summed over the query heads of
 * each KV head here and over KV heads in vo_select_topk, which together form
 * the sum over t and h in the summary's selection formula (sec. 2A).
 */
int vo_verify_attn(int dtype, int batch, int num_q_heads, int num_kv_heads,
                   int head_dim, int gamma, double scale,
                   const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens_k, int64_t total_kv,
                   uint32_t collect_mask, double* out, double* scores) {
    return vo_verify_attn_local(dtype, batch, num_q_heads, num_kv_heads, head_dim, gamma, scale, q, k, v,
                                cu_seqlens_k, total_kv, 0, collect_mask, out, scores);
}

/*
 * The same with an optional local (banded) mask, the "local masking" the
 * page's sec. 4 names beside the causal one (gpt-oss alternates banded and
 * dense layers, sec. 5.1): with window > 0, row r sees only the `window`
 * newest keys up to its own position, L_b + r - window < j <= L_b + r.
 * Collection under a local mask is not defined here (the pages select only
 * in dense layers): scores must be NULL or collect_mask 0 when window > 0.
 */
int vo_verify_attn_local(int dtype, int batch, int num_q_heads, int num_kv_heads,
                         int head_dim, int gamma, double scale,
                         const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_k, int64_t total_kv, int window,
                         uint32_t collect_mask, double* out, double* scores) {
    if (!shape_ok(dtype, batch, num_q_heads, num_kv_heads, head_dim)) return -1;
    if (gamma < 0 || gamma > 31 || !cu_seqlens_k || !out) return -1;
    if (window < 0 || (window > 0 && scores && collect_mask)) return -1;
    const int W = gamma + 1;
    const int G = num_q_heads / num_kv_heads;
    if (cu_seqlens_k[0] != 0 || cu_seqlens_k[batch] != total_kv) return -1;
    for (int b = 0; b < batch; ++b)
        if (cu_seqlens_k[b + 1] - cu_seqlens_k[b] < W) return -1;

    const int64_t kv_row = (int64_t)num_kv_heads * head_dim;   /* elements per token */
    const int64_t q_row = (int64_t)num_q_heads * head_dim;     /* elements per query row */
    const int ntask = batch * num_kv_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (int task = 0; task < ntask; ++task) {
        const int b = task / num_kv_heads;
        const int g = task % num_kv_heads;
        const int64_t start = cu_seqlens_k[b];
        const int64_t len = cu_seqlens_k[b + 1] - start;
        const int64_t L = len - W;                  /* committed prefix length */
        double* z = (double*)malloc(sizeof(double) * (size_t)len);
        int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)len);

        if (scores && collect_mask)
            for (int64_t i = 0; i < L; ++i) scores[(int64_t)g * total_kv + start + i] = 0.0;

        for (int hl = 0; hl < G; ++hl) {
            const int h = g * G + hl;
            for (int r = 0; r < W; ++r) {
                const int64_t q_off = ((int64_t)b * W + r) * q_row + (int64_t)h * head_dim;
                /* keys first .. L+r: all of them, or the last `window` under a local mask */
                const int64_t first = (window > 0 && L + r + 1 > window) ? L + r + 1 - window : 0;
                const int64_t visible = L + r + 1 - first;
                for (int64_t j = 0; j < visible; ++j) {
                    rows[j] = (start + first + j) * kv_row + (int64_t)g * head_dim;
                    z[j] = scale * dot_rows(q, q_off, k, rows[j], dtype, head_dim);
                }
                softmax_weighted_sum(z, rows, visible, v, dtype, head_dim,
                                     out + ((int64_t)b * W + r) * q_row + (int64_t)h * head_dim);
                if (scores && ((collect_mask >> r) & 1u))
                    for (int64_t i = 0; i < L; ++i)
                        scores[(int64_t)g * total_kv + start + i] += z[i];
            }
        }
        free(z);
        free(rows);
    }
    return 0;
}

typedef struct { double s; int32_t pos; } scored_pos;

/* Larger score first; equal scores: lower position first. */
static int by_score_desc_pos_asc(const void* a, const void* b) {
    const scored_pos* x = (const scored_pos*)a;
    const scored_pos* y = (const scored_pos*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int int_asc(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * Selection (gist.science summary sec. 2A "Formulation"): T is the size-k
 * subset of the prefix that maximises the summed logits.  For a sum of
 * per-position terms that set is exactly the k positions with the largest
 * per-position sums, which is what the sort below takes.  The pages fix
 * neither tie order nor output order: lower position wins a tie and the
 * result is ascending.
 */
int vo_select_topk(int batch, int num_kv_heads, int gamma,
                   const double* scores, const int32_t* cu_seqlens_k,
                   int64_t total_kv, const int32_t* cu_k, int32_t* indices,
                   double* theta, double* S_out) {
    if (batch < 0 || num_kv_heads <= 0 || gamma < 0 || gamma > 31) return -1;
    if (!scores || !cu_seqlens_k || !cu_k) return -1;
    const int W = gamma + 1;
    if (cu_seqlens_k[0] != 0 || cu_seqlens_k[batch] != total_kv || cu_k[0] != 0) return -1;
    for (int b = 0; b < batch; ++b) {
        int64_t L = (int64_t)cu_seqlens_k[b + 1] - cu_seqlens_k[b] - W;
        int64_t kb = (int64_t)cu_k[b + 1] - cu_k[b];
        if (L < 0 || kb < 0 || kb > L) return -1;
    }
    if (cu_k[batch] > 0 && !indices) return -1;

#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int64_t start = cu_seqlens_k[b];
        const int64_t L = (int64_t)cu_seqlens_k[b + 1] - start - W;
        const int64_t kb = (int64_t)cu_k[b + 1] - cu_k[b];
        scored_pos* sp = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(L > 0 ? L : 1));
        for (int64_t i = 0; i < L; ++i) {
            double s = 0.0;
            for (int g = 0; g < num_kv_heads; ++g) s += scores[(int64_t)g * total_kv + start + i];
            sp[i].s = s;
            sp[i].pos = (int32_t)i;
            if (S_out) S_out[start + i] = s;
        }
        qsort(sp, (size_t)L, sizeof(scored_pos), by_score_desc_pos_asc);
        int32_t* dst = indices + cu_k[b];
        for (int64_t j = 0; j < kb; ++j) dst[j] = sp[j].pos;
        qsort(dst, (size_t)kb, sizeof(int32_t), int_asc);
        if (theta) theta[b] = kb > 0 ? sp[kb - 1].s : NAN;
        free(sp);
    }
    return 0;
}

/*
 * Sparse drafting attention (page "Vegas ...", sec. 4 "Serving framework
 * integration": paged attention with one-token pages whose page indices are
 * the selected positions, so only those keys take part; sec. 2.2: the output
 * is the softmax-weighted average of the selected values).
 */
int vo_sparse_decode_attn(int dtype, int batch, int num_q_heads,
                          int num_kv_heads, int head_dim, double scale,
                          const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_k, const int32_t* indices,
                          const int32_t* cu_idx, double* out) {
    if (!shape_ok(dtype, batch, num_q_heads, num_kv_heads, head_dim)) return -1;
    if (!cu_seqlens_k || !cu_idx || !out) return -1;
    if (cu_idx[0] != 0) return -1;
    for (int b = 0; b < batch; ++b) {
        int64_t len = (int64_t)cu_seqlens_k[b + 1] - cu_seqlens_k[b];
        if (cu_idx[b + 1] < cu_idx[b]) return -1;
        for (int64_t j = cu_idx[b]; j < cu_idx[b + 1]; ++j)
            if (indices[j] < 0 || indices[j] >= len) return -1;
    }
    const int G = num_q_heads / num_kv_heads;
    const int64_t kv_row = (int64_t)num_kv_heads * head_dim;
    const int64_t q_row = (int64_t)num_q_heads * head_dim;
    const int ntask = batch * num_q_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (int task = 0; task < ntask; ++task) {
        const int b = task / num_q_heads;
        const int h = task % num_q_heads;
        const int g = h / G;
        const int64_t start = cu_seqlens_k[b];
        const int64_t n = (int64_t)cu_idx[b + 1] - cu_idx[b];
        double* o = out + (int64_t)b * q_row + (int64_t)h * head_dim;
        if (n == 0) {
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n);
        int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        const int64_t q_off = (int64_t)b * q_row + (int64_t)h * head_dim;
        for (int64_t j = 0; j < n; ++j) {
            rows[j] = (start + indices[cu_idx[b] + j]) * kv_row + (int64_t)g * head_dim;
            z[j] = scale * dot_rows(q, q_off, k, rows[j], dtype, head_dim);
        }
        softmax_weighted_sum(z, rows, n, v, dtype, head_dim, o);
        free(z);
        free(rows);
    }
    return 0;
}

/*
 * StreamingLLM-style query-agnostic lists (the "MagicDec-Stream" baseline the
 * page's sec. 5.1 compares against; sec. 2.2 describes the sink-plus-recent
 * pattern): with a budget of k_b positions, sequence b's list is the first
 * min(sinks, k_b) prefix positions followed by the most recent remaining
 * ones, ascending, no duplicates, all inside the prefix [0, L_b).
 */
int vo_streaming_indices(int batch, int gamma, int sinks, const int32_t* cu_seqlens_k,
                         const int32_t* cu_idx, int32_t* indices) {
    if (batch < 0 || gamma < 0 || gamma > 31 || sinks < 0 || !cu_seqlens_k || !cu_idx) return -1;
    const int W = gamma + 1;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = (int64_t)cu_seqlens_k[b + 1] - cu_seqlens_k[b] - W;
        const int64_t kb = (int64_t)cu_idx[b + 1] - cu_idx[b];
        if (L < 0 || kb < 0 || kb > L) return -1;
        int32_t* dst = indices + cu_idx[b];
        const int64_t ns = sinks < kb ? sinks : kb;
        for (int64_t j = 0; j < ns; ++j) dst[j] = (int32_t)j;
        for (int64_t j = ns; j < kb; ++j) dst[j] = (int32_t)(L - (kb - j));
    }
    return 0;
}

/*
 * Speculative-sampling acceptance (the blog "You Could Have Come Up with
 * Speculative Decoding", section "Preservation of Target Distribution"): draft
 * token y_j, proposed from q_j, is kept when u_j <= min(1, p_j(y_j) / q_j(y_j)),
 * i.e. u_j * q_j(y_j) <= p_j(y_j); at the first rejection a replacement is drawn
 * from the residual max(0, p_j - q_j) normalised; when all gamma drafts are
 * kept, the bonus token is drawn from p_{gamma+1} (section "Guessing is
 * Enough?").  Arithmetic fixed here so that the chosen token does not depend on
 * summation order:
 *   - the acceptance test is evaluated exactly: the product of two binary32
 *     values is exact in binary64;
 *   - masses are taken in fixed point, m_y = floor(x_y * 2^40) of the binary32
 *     value x_y (residual or target probability), summed as integers;
 *   - with u_int = floor(u * 2^24) and M = sum m_y, the drawn token is the
 *     smallest y with m_0 + ... + m_y > floor(u_int * M / 2^24);
 *   - if the residual mass is zero (only possible through rounding or
 *     unnormalised inputs) the replacement is drawn from p_j itself; if that is
 *     zero too, token 0.
 */
static uint64_t fixed_mass(double x) {
    if (!(x > 0.0)) return 0;
    double f = floor(x * 1099511627776.0);        /* 2^40 */
    if (f > 1099511627776.0) f = 1099511627776.0;  /* masses above 1 are capped at 1 */
    return (uint64_t)f;
}

static int32_t draw_fixed(const float* p, const float* q, int64_t vocab, float u) {
    /* q == NULL: masses of p; else residual masses max(0, p - q) */
    uint64_t total = 0;
    for (int64_t y = 0; y < vocab; ++y) {
        double x = q ? (double)p[y] - (double)q[y] : (double)p[y];
        total += fixed_mass(x);
    }
    if (total == 0) return q ? draw_fixed(p, NULL, vocab, u) : 0;
    double uf = floor((double)u * 16777216.0);    /* 2^24 */
    uint64_t ui = uf < 0.0 ? 0 : (uf > 16777215.0 ? 16777215u : (uint64_t)uf);
    const uint64_t thr = (total >> 24) * ui + (((total & 16777215u) * ui) >> 24);
    uint64_t run = 0;
    for (int64_t y = 0; y < vocab; ++y) {
        double x = q ? (double)p[y] - (double)q[y] : (double)p[y];
        run += fixed_mass(x);
        if (run > thr) return (int32_t)y;
    }
    return (int32_t)(vocab - 1);
}

int vo_spec_accept(int batch, int gamma, int64_t vocab, const float* p, const float* q,
                   const int32_t* draft, const float* u_accept, const float* u_sample,
                   int32_t* n_accepted, int32_t* next_token) {
    if (batch < 0 || gamma < 0 || vocab < 1 || !p || (gamma > 0 && (!q || !draft || !u_accept)) ||
        !u_sample || !n_accepted || !next_token)
        return -1;
    for (int b = 0; b < batch; ++b) {
        const float* pb = p + (int64_t)b * (gamma + 1) * vocab;
        const float* qb = gamma > 0 ? q + (int64_t)b * gamma * vocab : NULL;
        int j = 0;
        for (; j < gamma; ++j) {
            int32_t y = draft[(int64_t)b * gamma + j];
            if (y < 0 || y >= vocab) return -1;
            double lhs = (double)u_accept[(int64_t)b * gamma + j] * (double)qb[(int64_t)j * vocab + y];
            if (!(lhs <= (double)pb[(int64_t)j * vocab + y])) break;   /* rejected */
        }
        n_accepted[b] = j;
        next_token[b] = j < gamma ? draw_fixed(pb + (int64_t)j * vocab, qb + (int64_t)j * vocab, vocab, u_sample[b])
                                  : draw_fixed(pb + (int64_t)gamma * vocab, NULL, vocab, u_sample[b]);
    }
    return 0;
}
