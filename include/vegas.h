/*
 * vegas.h -- C ABI of the MI355X (gfx950) Vegas attention hot path.
 *
 * One decoder layer, one GPU, three steps per speculative iteration:
 *   1. vegas_verify_attn        full attention of the gamma+1 verification rows
 *                               over the whole KV cache, also emitting the
 *                               collected pre-softmax logits (Collect-2-Query);
 *   2. vegas_select_topk        the per-sequence top-k prefix positions of the
 *                               collected logits summed over rows and heads;
 *   3. vegas_sparse_decode_attn single-query drafting attention restricted to
 *                               the selected token positions (run gamma times).
 *
 * The method is the one of "Vegas: Self-Speculative Decoding with
 * Verification-Guided Sparse Attention" (paperpeel page: sec. 3.2 selection
 * guided by verification, sec. 3.3 Collect-2-Query, sec. 4 implementation)
 * and of its gist.science "Technical Summary" (sec. 2A selection formula,
 * sec. 2B Collect-2-Query).
 *
 * Common conventions
 * ------------------
 *  - Every tensor argument is a caller-owned DEVICE pointer.  The library
 *    never allocates or frees device memory; scratch space is the caller's
 *    `workspace`, sized by the matching *_workspace_size query.  Its contents
 *    are undefined before and after a call.
 *  - All calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream) and never synchronise the host.  Calls that share a
 *    workspace must be ordered (same stream, or synchronised).
 *  - Layouts are dense, row-major, element-contiguous:
 *      KV cache   k, v  [total_kv, Hkv, D]; sequence b owns token rows
 *                       [cu_seqlens_k[b], cu_seqlens_k[b+1]) (varlen packing
 *                       as in flash_attn_varlen_func, which the pages hook).
 *      query head h reads KV head h / (Hq / Hkv).
 *  - dtype of q, k, v and out: VEGAS_DTYPE_BF16 (bf16 storage, fp32
 *    accumulation and softmax) or VEGAS_DTYPE_F32.  D (head_dim) is 64 or
 *    128.  q, k, v, out must be 16-byte aligned.
 *  - Placement (performance only): the passes read the K and V rows of the
 *    same positions together, so their speed depends on where v sits
 *    relative to k.  On MI355X, 128K Qwen3-8B-shaped layer: with v's
 *    address equal to k's modulo 2 MB, as two large allocations' addresses
 *    usually are, some KV heads read slower (v 256-768 bytes off made the
 *    layer-step ~1.3% faster); beyond 2 MB, v 1 GiB + 10 MiB + 512 B past k
 *    in one allocation read 320-323 us per verification against 339-340 at
 *    1 GiB + 2 MiB + 512 B, and two separate allocations read anywhere in
 *    between from layer to layer.  The library takes the caller's pointers
 *    as given.
 *  - Errors: arguments are validated on the host before any launch; a
 *    non-OK status launches nothing (VEGAS_ERR_HIP: a launch failed after
 *    validation).  vegas_last_error_message() returns a per-thread detail
 *    string for the last non-OK status.  Device-side faults surface at the
 *    caller's next synchronisation, as with any HIP kernel.  Position and
 *    index values read from device memory are clamped to the owning
 *    sequence, so malformed device data gives unspecified results, never an
 *    out-of-bounds access.
 */
#ifndef VEGAS_H
#define VEGAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEGAS_ABI_VERSION 1

typedef enum {
    VEGAS_OK = 0,
    VEGAS_ERR_INVALID_ARGUMENT = 1,
    VEGAS_ERR_UNSUPPORTED = 2,
    VEGAS_ERR_WORKSPACE_TOO_SMALL = 3,
    VEGAS_ERR_HIP = 4
} vegas_status_t;

typedef enum { VEGAS_DTYPE_F32 = 0, VEGAS_DTYPE_BF16 = 1 } vegas_dtype_t;

/* Attention geometry shared by the two attention entry points. */
typedef struct {
    int32_t dtype;          /* vegas_dtype_t */
    int32_t batch;          /* number of sequences, 1 .. 1024 */
    int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads */
    int32_t num_kv_heads;   /* Hkv >= 1 */
    int32_t head_dim;       /* D: 64 or 128 */
    float softmax_scale;    /* s > 0; logits are s * <q, k> */
} vegas_attn_shape_t;

int32_t vegas_abi_version(void);
const char* vegas_status_string(vegas_status_t status);
const char* vegas_last_error_message(void);

/*
 * Verification attention with logit collection.
 * Defined by "Vegas ..." sec. 4 "Attention kernel implementation" (full
 * attention over the KV cache; logits are read after the causal mask and
 * before softmax normalisation; with collection switched off the kernel
 * behaves as plain attention) and sec. 3.3 / the summary's sec. 2B (collect
 * only the first draft token and the bonus token).
 *
 *  gamma          number of draft tokens, 0..31; each sequence has W =
 *                 gamma+1 verification rows.  W * (Hq/Hkv) must be <= 64.
 *  q              [batch*W, Hq, D]; row r of sequence b at b*W + r.
 *  k, v           [total_kv, Hkv, D]; len_b = cu_seqlens_k[b+1]-cu_seqlens_k[b]
 *                 >= W.  The last W rows of each sequence are the K/V of the
 *                 verification rows themselves; the first L_b = len_b - W
 *                 rows are the committed prefix.
 *  cu_seqlens_k   device int32 [batch+1], cu_seqlens_k[0] = 0, non-decreasing.
 *  max_seqlen_k   host scalar >= every len_b (sizes the split grid).
 *  total_kv       host scalar = cu_seqlens_k[batch].
 *  collect_mask   bit r set: row r enters the collected score.  Vegas'
 *                 Collect-2-Query is (1u | 1u << gamma); 0 disables
 *                 collection.  Bits >= W must be clear.
 *  scores         fp32 [Hkv, total_kv].  For every prefix position i < L_b
 *                 and KV head g, scores[g, cu_seqlens_k[b] + i] receives
 *                 s * sum over collected rows r and over the query heads h of
 *                 group g of <q[b,r,h], k[i,g]>.  Entries at verification
 *                 positions (i >= L_b) are not written.  May be NULL iff
 *                 collect_mask == 0.
 *  out            [batch*W, Hq, D] in dtype: row r of sequence b attends to
 *                 keys 0 .. L_b + r (bottom-right causal alignment).
 */
vegas_status_t vegas_verify_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                           int32_t max_seqlen_k, size_t* bytes);
vegas_status_t vegas_verify_attn(const vegas_attn_shape_t* shape, int32_t gamma,
                                 const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                 int32_t total_kv, uint32_t collect_mask, float* scores,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Verification-guided KV selection.
 * Defined by the summary's sec. 2A formulation: T is the size-k subset of the
 * prefix that maximises the collected logits summed over rows and query
 * heads; for a sum of per-position terms that is the k positions with the
 * largest summed score S_b[i] = sum_g scores[g, cu_seqlens_k[b] + i].
 * One T per sequence (and layer), shared by all heads.
 *
 *  scores         fp32 [num_kv_heads, total_kv] as written by vegas_verify_attn.
 *  cu_seqlens_k   as above; L_b = len_b - (gamma+1) candidate positions.
 *  cu_k           device int32 [batch+1]; k_b = cu_k[b+1]-cu_k[b] with
 *                 0 <= k_b <= L_b (larger k_b is clamped to L_b).
 *  indices        device int32 [cu_k[batch]]; receives T_b at
 *                 indices[cu_k[b] ...], positions relative to the sequence
 *                 start, strictly ascending.  Among equal scores the lower
 *                 position is taken.  The summed score is accumulated in
 *                 fp32 over KV heads 0..Hkv-1 in order.
 */
vegas_status_t vegas_select_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t gamma,
                                           int32_t max_seqlen_k, int32_t total_kv,
                                           size_t* bytes);
vegas_status_t vegas_select_topk(int32_t batch, int32_t num_kv_heads, int32_t gamma,
                                 const float* scores, const int32_t* cu_seqlens_k,
                                 int32_t max_seqlen_k, int32_t total_kv,
                                 const int32_t* cu_k, int32_t* indices,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verification followed by selection, in one call.
 * The two steps of "Vegas ..." sec. 3 (verification with Collect-2-Query,
 * then the top-k of the summed logits, summary sec. 2A) as they follow each
 * other in a decoding iteration.  Results are those of vegas_verify_attn and
 * then vegas_select_topk with the same arguments, bit for bit: out, scores
 * and indices are written as described there.  The difference is the launch
 * sequence: the selection's histogram clearing rides on the verification's
 * split kernel and its score summation on the verification's combine
 * kernel, which saves two kernel launches per call.
 *
 *  collect_mask   must be non-zero (VEGAS_ERR_INVALID_ARGUMENT otherwise).
 *  cu_k, indices  as for vegas_select_topk.
 *  workspace      at least vegas_verify_select_workspace_size bytes (the
 *                 verification workspace, rounded up to 256 bytes, then the
 *                 selection workspace); contents undefined between calls.
 * Errors: those of both calls; nothing is launched unless every argument of
 * both steps is valid.
 */
vegas_status_t vegas_verify_select_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                  int32_t max_seqlen_k, int32_t total_kv,
                                                  size_t* bytes);
vegas_status_t vegas_verify_select(const vegas_attn_shape_t* shape, int32_t gamma,
                                   const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                   int32_t total_kv, uint32_t collect_mask,
                                   const int32_t* cu_k, float* scores, int32_t* indices,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Host copies of the offset arrays, for the *_hostplan entry points.
 * A serving loop (the pages hook vLLM, "Vegas ..." sec. 4) keeps every
 * sequence's length on the host.  Given host copies, the library computes
 * the split plan on the host and passes it in the kernel arguments, so the
 * kernels start without reading the offsets or planning on the device.  The
 * plan is the one the device computes from the same values, so the
 * *_hostplan calls give exactly the results of the calls without the suffix,
 * with one exception: when the sequence lengths are unequal enough that the
 * per-sequence splits leave some workgroups with clearly more than an equal
 * share, verification splits the batch's positions, laid end to end, into
 * equal slices instead (the scores, the selection and the drafting outputs
 * stay bit-identical; the verification output then differs only in the
 * rounding of the split merge, and is deterministic).  Batches above 16
 * sequences are planned on the device as before.
 *
 *  cu_seqlens_k   host int32 [batch+1]: the values of the device array.
 *  cu_idx         host int32 [batch+1]: the values of the device cu_k (for
 *                 vegas_verify_select_hostplan) or cu_idx (for
 *                 vegas_sparse_decode_attn_hostplan); unused (may be NULL)
 *                 by vegas_verify_attn_hostplan.
 * Both are read during the call only (not kept).  They are checked on the
 * host: non-decreasing, starting at >= 0, cu_seqlens_k within total_kv with
 * every length in [gamma+1, max_seqlen_k] (verification), every list at most
 * max_idx long (drafting); a violation returns VEGAS_ERR_INVALID_ARGUMENT and
 * launches nothing.  The device arrays must hold the same values; they are
 * still passed (and still read where the plan does not cover them).
 */
typedef struct {
    const int32_t* cu_seqlens_k;
    const int32_t* cu_idx;
} vegas_host_offsets_t;

/* vegas_verify_attn with host offsets (cu_idx unused); workspace as for
 * vegas_verify_attn. */
vegas_status_t vegas_verify_attn_hostplan(const vegas_attn_shape_t* shape, int32_t gamma,
                                          const void* q, const void* k, const void* v,
                                          const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                          int32_t total_kv, uint32_t collect_mask, float* scores,
                                          void* out, void* workspace, size_t workspace_bytes,
                                          void* stream, const vegas_host_offsets_t* host);
/*
 * Which split plan a host-planned verification call takes for these offsets
 * (the plan is a design choice of this library, not a step of the method):
 * *balanced = 1 when the batch's positions are cut into equal slices (the
 * case above whose verification output differs from the device-planned
 * call's in the merge's rounding), 0 for the per-sequence plan or a batch
 * planned on the device; *workgroups = workgroups per KV head of the
 * verification launch.  Host arguments only; validated as by
 * vegas_verify_attn_hostplan (VEGAS_ERR_INVALID_ARGUMENT on bad offsets).
 * Nothing is launched.
 */
vegas_status_t vegas_verify_hostplan_info(const vegas_attn_shape_t* shape, int32_t gamma,
                                          int32_t max_seqlen_k, int32_t total_kv,
                                          const vegas_host_offsets_t* host, int32_t* balanced,
                                          int32_t* workgroups);
/* vegas_verify_select with host offsets; workspace as for vegas_verify_select. */
vegas_status_t vegas_verify_select_hostplan(const vegas_attn_shape_t* shape, int32_t gamma,
                                            const void* q, const void* k, const void* v,
                                            const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                            int32_t total_kv, uint32_t collect_mask,
                                            const int32_t* cu_k, float* scores, int32_t* indices,
                                            void* out, void* workspace, size_t workspace_bytes,
                                            void* stream, const vegas_host_offsets_t* host);

/*
 * vegas_verify_select_hostplan in two halves, for callers that run the
 * selection's last steps on another stream beside later work.  The selected
 * positions are used only by the next drafting pass ("Vegas ...", sec. 3:
 * selection follows verification, drafting uses its result), while the next
 * layer's verification needs only this layer's output; the second half can
 * then overlap the next layer's verification.
 *   _begin: the verification kernels, with the selection's histogram
 *           clearing (out and scores are complete when it finishes);
 *   _end:   the selection's remaining steps, from the summed scores and
 *           their keys to the lists (indices complete when it finishes), on
 *           any stream ordered after _begin's completion (for example by an
 *           event the caller records on _begin's stream).
 * Both take the same arguments as vegas_verify_select_hostplan, with the same
 * workspace, which must not be reused until _end has finished; both validate
 * them, and _end launches nothing else.  Together they give the results of
 * vegas_verify_select_hostplan bit for bit.
 */
vegas_status_t vegas_verify_select_begin_hostplan(const vegas_attn_shape_t* shape, int32_t gamma,
                                                  const void* q, const void* k, const void* v,
                                                  const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                                  int32_t total_kv, uint32_t collect_mask,
                                                  const int32_t* cu_k, float* scores, int32_t* indices,
                                                  void* out, void* workspace, size_t workspace_bytes,
                                                  void* stream, const vegas_host_offsets_t* host);
vegas_status_t vegas_verify_select_end_hostplan(const vegas_attn_shape_t* shape, int32_t gamma,
                                                const void* q, const void* k, const void* v,
                                                const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                                int32_t total_kv, uint32_t collect_mask,
                                                const int32_t* cu_k, float* scores, int32_t* indices,
                                                void* out, void* workspace, size_t workspace_bytes,
                                                void* stream, const vegas_host_offsets_t* host);

/*
 * Sparse drafting attention over selected tokens.
 * Defined by "Vegas ..." sec. 4 "Serving framework integration" (paged
 * attention with a page size of one token whose page indices are the
 * selected positions, so only those keys are read) and sec. 2.2 (the output
 * is the softmax-weighted average of the selected values).  No mask: every
 * listed position takes part, duplicates count as listed.
 *
 *  q              [batch, Hq, D], one query row per sequence.
 *  k, v,
 *  cu_seqlens_k   the KV cache, as for vegas_verify_attn.
 *  indices        device int32; sequence b's list is
 *                 indices[cu_idx[b] .. cu_idx[b+1]), positions in [0, len_b).
 *  cu_idx         device int32 [batch+1], cu_idx[0] = 0, non-decreasing.
 *  max_idx        host scalar >= every list length (sizes the split grid).
 *  out            [batch, Hq, D] in dtype; an empty list gives a zero row.
 */
vegas_status_t vegas_sparse_decode_workspace_size(const vegas_attn_shape_t* shape,
                                                  int32_t max_idx, size_t* bytes);
vegas_status_t vegas_sparse_decode_attn(const vegas_attn_shape_t* shape, const void* q,
                                        const void* k, const void* v,
                                        const int32_t* cu_seqlens_k, int32_t total_kv,
                                        const int32_t* indices, const int32_t* cu_idx,
                                        int32_t max_idx, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);
/* vegas_sparse_decode_attn with host offsets (vegas_host_offsets_t above);
 * workspace: vegas_sparse_decode_workspace_size. */
vegas_status_t vegas_sparse_decode_attn_hostplan(const vegas_attn_shape_t* shape, const void* q,
                                                 const void* k, const void* v,
                                                 const int32_t* cu_seqlens_k, int32_t total_kv,
                                                 const int32_t* indices, const int32_t* cu_idx,
                                                 int32_t max_idx, void* out, void* workspace,
                                                 size_t workspace_bytes, void* stream,
                                                 const vegas_host_offsets_t* host);

/*
 * vegas_sparse_decode_attn without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation).  Same kernels and results as
 * vegas_sparse_decode_attn (host != NULL: as vegas_sparse_decode_attn_hostplan
 * with those host offsets); allocates nothing.
 * Scratch: a static device array of vegas_noalloc_scratch_bytes() bytes (16 MiB)
 * inside the library, one copy per GPU, held until the process ends.  A call
 * whose vegas_sparse_decode_workspace_size exceeds it returns
 * VEGAS_ERR_UNSUPPORTED and launches nothing.  All calls on one GPU share the
 * array: calls that may overlap on one GPU (different streams, or threads)
 * race and must be ordered by the caller.
 */
vegas_status_t vegas_sparse_decode_attn_noalloc(const vegas_attn_shape_t* shape, const void* q,
                                                const void* k, const void* v,
                                                const int32_t* cu_seqlens_k, int32_t total_kv,
                                                const int32_t* indices, const int32_t* cu_idx,
                                                int32_t max_idx, void* out, void* stream,
                                                const vegas_host_offsets_t* host);
size_t vegas_noalloc_scratch_bytes(void);

/*
 * Paged KV cache, beside the contiguous layout above.
 * The pages hook vLLM's attention, whose KV cache is paged, and run drafting
 * as paged attention with a page size of one token ("Vegas ...", sec. 4
 * "Serving framework integration"; its Appendix D reports the same latency
 * for page sizes 1 to 16).  These variants read K and V from a page pool:
 *
 *  k, v           [num_pages, page_size, Hkv, D]: pool page p holds page_size
 *                 consecutive token rows.
 *  block_table    device int32 [batch, max_pages_per_seq]: position t of
 *                 sequence b is row t % page_size of pool page
 *                 block_table[b * max_pages_per_seq + t / page_size].
 *  page_size      a power of two, 1 .. 256.
 *  num_pages      pages in the pool; num_pages * page_size < 2^31.  Page
 *                 numbers read from the table are clamped into the pool.
 *  max_pages_per_seq * page_size must be >= max_seqlen_k.
 *
 * Sequence lengths still come from cu_seqlens_k (length of sequence b =
 * cu_seqlens_k[b+1] - cu_seqlens_k[b]), which also packs `scores` exactly as
 * in vegas_verify_attn; q, out, indices and the workspace are as in the
 * contiguous entry points, and the results are the same.
 */
typedef struct {
    const int32_t* block_table;
    int32_t max_pages_per_seq;
    int32_t page_size;
    int32_t num_pages;
} vegas_paged_kv_t;

/* Workspace of vegas_verify_attn_paged for a cache of `page_size` (0: the
 * contiguous cache, same as vegas_verify_workspace_size).  A split stages its
 * page list in LDS beside its collected scores, so small pages cap the
 * positions one split covers (1-token pages: 11200 at D = 128, bf16) and can
 * need more splits, hence more workspace. */
vegas_status_t vegas_verify_paged_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                 int32_t max_seqlen_k, int32_t page_size, size_t* bytes);
vegas_status_t vegas_verify_attn_paged(const vegas_attn_shape_t* shape, int32_t gamma,
                                       const void* q, const void* k, const void* v,
                                       const vegas_paged_kv_t* pages, const int32_t* cu_seqlens_k,
                                       int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                       float* scores, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream);
/* Workspace: vegas_sparse_decode_workspace_size. */
vegas_status_t vegas_sparse_decode_attn_paged(const vegas_attn_shape_t* shape, const void* q,
                                              const void* k, const void* v,
                                              const vegas_paged_kv_t* pages,
                                              const int32_t* cu_seqlens_k, int32_t total_kv,
                                              const int32_t* indices, const int32_t* cu_idx,
                                              int32_t max_idx, void* out, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * Local (banded) verification attention.
 * The page's sec. 4 takes logits "after causal or local masking"; gpt-oss
 * alternates banded and dense attention layers and Vegas drafts sparsely only
 * in the dense ones (sec. 5.1).  This entry point computes the banded layers'
 * verification: row r of sequence b attends to keys j with
 * L_b + r - window < j <= L_b + r, and only those keys are read.  Arguments as
 * for vegas_verify_attn; there is no collection (nothing is selected in a
 * banded layer).  window >= 1.
 */
vegas_status_t vegas_verify_local_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                 int32_t max_seqlen_k, int32_t window, size_t* bytes);
vegas_status_t vegas_verify_attn_local(const vegas_attn_shape_t* shape, int32_t gamma,
                                       const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                       int32_t total_kv, int32_t window, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Query-agnostic index lists: attention sinks plus the most recent tokens
 * (the StreamingLLM selection behind the MagicDec-Stream baseline of the
 * page's sec. 5.1, described in sec. 2.2).  With the same budget k_b as Vegas'
 * selection they feed vegas_sparse_decode_attn unchanged.
 *
 *  cu_idx       device int32 [batch+1]: budget k_b = cu_idx[b+1] - cu_idx[b]
 *               <= L_b (larger budgets are clamped to L_b and the extra slots
 *               repeat the last position).
 *  total_idx    host scalar = cu_idx[batch].
 *  indices      device int32 [total_idx]: sequence b gets the positions
 *               0 .. min(sinks, k_b)-1, then L_b - (k_b - min(sinks, k_b)) ..
 *               L_b - 1, ascending.
 */
vegas_status_t vegas_streaming_indices(int32_t batch, int32_t gamma, int32_t sinks,
                                       const int32_t* cu_seqlens_k, int32_t total_kv,
                                       const int32_t* cu_idx, int32_t total_idx, int32_t* indices,
                                       void* stream);

/*
 * Speculative-sampling acceptance: the step after verification that decides
 * how many drafts are kept (blog "You Could Have Come Up with Speculative
 * Decoding", section "Preservation of Target Distribution").  Draft y_j,
 * proposed from q_j, is kept when u_j * q_j(y_j) <= p_j(y_j); at the first
 * rejection the replacement is drawn from max(0, p_j - q_j) normalised; if all
 * gamma drafts are kept, the bonus token is drawn from p_{gamma+1}.  The
 * emitted tokens then follow p exactly.  The caller supplies the uniforms.
 *
 *  p             device fp32 [batch, gamma+1, vocab]: target probabilities of
 *                the verification rows (after temperature / top-k / top-p).
 *  q             device fp32 [batch, gamma, vocab]: draft probabilities.
 *  draft_tokens  device int32 [batch, gamma], in [0, vocab) (out-of-range
 *                tokens are clamped).
 *  u_accept      device fp32 [batch, gamma], u_sample device fp32 [batch]:
 *                uniforms in [0, 1).
 *  n_accepted    device int32 [batch]: drafts kept before the first rejection.
 *  next_token    device int32 [batch]: the replacement, or the bonus token.
 *  workspace     caller-owned device scratch of vegas_spec_accept_workspace_size
 *                bytes (contents undefined between calls).
 * Decisions are exact and independent of summation order: the test is
 * evaluated in binary64 (exact for a product of two binary32 values); draws
 * use masses floor(x * 2^40) summed as integers and pick the smallest y whose
 * running mass exceeds floor(floor(u * 2^24) * M / 2^24), M the total mass; an
 * empty residual falls back to p_j, an empty p to token 0.
 */
vegas_status_t vegas_spec_accept_workspace_size(int32_t batch, int32_t vocab, size_t* bytes);
vegas_status_t vegas_spec_accept(int32_t batch, int32_t gamma, int32_t vocab, const float* p,
                                 const float* q, const int32_t* draft_tokens, const float* u_accept,
                                 const float* u_sample, int32_t* n_accepted, int32_t* next_token,
                                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VEGAS_H */
