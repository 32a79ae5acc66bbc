/*
 * vegas_oracle.h -- plain CPU reference of the Vegas attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, includes or calls it, and it shares no code with it.
 *
 * Every quantity is accumulated in IEEE double.  Inputs are the exact bits the
 * GPU consumes (fp32, or bf16 given as raw uint16 bit patterns), widened to
 * double without rounding.
 *
 * Source of the method: "Vegas: Self-Speculative Decoding with
 * Verification-Guided Sparse Attention" (paperpeel page) -- sec. 3.2
 * (verification-guided KV selection), sec. 3.3 (Collect-2-Query), sec. 4
 * (logits taken after causal masking and before softmax; sparse drafting
 * with one-token pages indexed by the selected positions) -- and the
 * gist.science "Technical Summary" of the same paper, sec. 2 "A. Aggregated
 * Attention Logit Selection" (the argmax-over-sets formulation) and
 * "B. Collect-2-Query Mechanism".
 *
 * Layouts (shared convention with the public C ABI, restated here so that
 * this file stands alone):
 *   q_verify  [batch*(gamma+1), Hq, D]   row r of sequence b at b*(gamma+1)+r
 *   k, v      [total_kv, Hkv, D]         sequence b owns rows
 *                                        [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *   scores    [Hkv, total_kv]            per-KV-head collected logit sum
 *   q_decode  [batch, Hq, D]
 *   KV head of query head h is h / (Hq/Hkv).
 *
 * Return value: 0 on success, -1 on an argument error.
 */
#ifndef VEGAS_ORACLE_H
#define VEGAS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { VO_DTYPE_F32 = 0, VO_DTYPE_BF16 = 1 };

/* Full verification attention for the gamma+1 new rows of every sequence.
 * Row r of sequence b (prefix length L_b = len_b - (gamma+1)) attends to keys
 * j = 0 .. L_b + r (bottom-right causal mask).  out receives the attention
 * output in double.  If scores is non-NULL it receives, for every prefix
 * position i < L_b and KV head g, the sum over the rows r whose bit is set in
 * collect_mask and over the query heads of group g of the pre-softmax logit
 * scale * <q, k_i>.  Entries at i >= L_b are left untouched. */
int vo_verify_attn(int dtype, int batch, int num_q_heads, int num_kv_heads,
                   int head_dim, int gamma, double scale,
                   const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens_k, int64_t total_kv,
                   uint32_t collect_mask, double* out, double* scores);

/* As vo_verify_attn, with an optional local mask: window > 0 limits row r
 * to the keys L_b + r - window < j <= L_b + r.  Collection must be off
 * (scores NULL or collect_mask 0) when window > 0. */
int vo_verify_attn_local(int dtype, int batch, int num_q_heads, int num_kv_heads,
                         int head_dim, int gamma, double scale,
                         const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_k, int64_t total_kv, int window,
                         uint32_t collect_mask, double* out, double* scores);

/* Query-agnostic sink-plus-recent lists with a budget of
 * k_b = cu_idx[b+1] - cu_idx[b] <= L_b positions: the first min(sinks, k_b)
 * prefix positions, then the k_b - min(sinks, k_b) most recent ones
 * (ending at L_b - 1), ascending. */
int vo_streaming_indices(int batch, int gamma, int sinks, const int32_t* cu_seqlens_k,
                         const int32_t* cu_idx, int32_t* indices);

/* Speculative-sampling acceptance per sequence: p [batch, gamma+1, vocab]
 * target probabilities, q [batch, gamma, vocab] draft probabilities, draft
 * [batch, gamma] tokens, u_accept [batch, gamma] and u_sample [batch] uniforms
 * in [0, 1).  n_accepted[b] = drafts kept before the first rejection;
 * next_token[b] = the replacement drawn from the residual at that rejection,
 * or the bonus token drawn from p_{gamma+1} when all are kept.  The
 * acceptance test is exact and the draw uses 2^-40 fixed-point masses (see
 * the source). */
int vo_spec_accept(int batch, int gamma, int64_t vocab, const float* p, const float* q,
                   const int32_t* draft, const float* u_accept, const float* u_sample,
                   int32_t* n_accepted, int32_t* next_token);

/* Exact top-k of the score summed over KV heads, per sequence.
 * S_b[i] = sum_g scores[g, cu_seqlens_k[b] + i] for i < L_b.  The k_b
 * (= cu_k[b+1] - cu_k[b]) positions with the largest S_b are written to
 * indices[cu_k[b] ...] in ascending order; among equal scores the lower
 * position wins.  theta (optional, [batch]) receives the k_b-th largest S_b
 * (NaN when k_b == 0); S_out (optional, [total_kv]) receives S_b[i] at
 * cu_seqlens_k[b] + i. */
int vo_select_topk(int batch, int num_kv_heads, int gamma,
                   const double* scores, const int32_t* cu_seqlens_k,
                   int64_t total_kv, const int32_t* cu_k, int32_t* indices,
                   double* theta, double* S_out);

/* Single-query attention of every head over a per-sequence list of key
 * positions (relative to the sequence start), no mask.  An empty list gives
 * an all-zero output row. */
int vo_sparse_decode_attn(int dtype, int batch, int num_q_heads,
                          int num_kv_heads, int head_dim, double scale,
                          const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_k, const int32_t* indices,
                          const int32_t* cu_idx, double* out);

#ifdef __cplusplus
}
#endif
#endif
