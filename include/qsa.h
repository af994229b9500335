/*
 * qsa.h - C ABI of the Qwen Sparse Attention (QSA) hot path for AMD MI355X
 * (gfx950).  Library: libqsa.so.
 *
 * The method (page "Qwen's million-token window has a 2,048-token keyhole",
 * opening section and section "A million-token window with a selective
 * view"): a light indexer with four query heads and one shared key head
 * compresses keys four at a time into micro-blocks, ranks the micro-blocks
 * for every query, keeps at most 512 of them (2,048 tokens) plus the
 * query's own unfinished tail block, expands the winners back to token
 * positions, and runs core grouped-query attention only over those tokens.
 *
 * Fixed method constants (validated, not configurable):
 *   indexer query heads 4, indexer key heads 1, indexer dim 64,
 *   block 4 tokens, top-k 512 blocks, core head dim 128.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - bf16 tensors travel as uint16_t bit patterns.
 *  - Every data pointer is a DEVICE pointer, owned by the caller, contiguous
 *    in the layout given below and 16-byte aligned (QSA_ERR_ALIGN otherwise).
 *    `lens` and `first_block` are device int32 arrays too.
 *  - Nothing is allocated, freed or synchronised inside a call: all work is
 *    enqueued on `stream` (a hipStream_t, NULL = the default stream) and the
 *    call returns before it finishes.  Scratch memory comes from the caller's
 *    workspace `ws` of `ws_bytes` bytes (see qsa_workspace_bytes).
 *  - Host-visible arguments are checked before anything is launched; on an
 *    error nothing is launched and no output is touched.  No C++ exception
 *    crosses the ABI.
 *  - Sequence b holds lens[b] tokens (query tokens included); its queries are
 *    the LAST n_query positions t = lens[b] - n_query + i, i < n_query.  The
 *    caller guarantees n_query <= lens[b] <= max_len.  Kernels clamp lens to
 *    [0, max_len] and skip positions t < 0 (such rows get n_sel = n_tok = 0,
 *    zero output and lse = -inf), so a broken `lens` cannot make them read
 *    or write out of bounds; with QSA_CHECK=1 in the environment the library
 *    copies `lens` to the host (a synchronising copy) and returns
 *    QSA_ERR_SHAPE when the contract is broken.
 *  - Calls that share a workspace must not overlap in time; calls on
 *    different streams need different workspaces.
 *
 * Layouts (row-major):
 *   q_idx [B][Nq][4][64]       k_idx [B][Lmax][64]      k_cmp [B][Lmax/4][64]
 *   q     [B][Nq][Hq][128]     k, v  [B][Lmax][Hkv][128]
 *   sel   [B][Nq][512] int32   n_sel [B][Nq] int32
 *   tok   [B][Nq][2052] int32  n_tok [B][Nq] int32
 *   out   [B][Nq][Hq][128] bf16          lse [B][Nq][Hq] float (natural log)
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qsa_status;

enum {
  QSA_OK = 0,
  QSA_ERR_NULL = 1,       /* a required pointer is NULL */
  QSA_ERR_ALIGN = 2,      /* a pointer is not 16-byte aligned */
  QSA_ERR_SHAPE = 3,      /* unsupported or inconsistent shape */
  QSA_ERR_WORKSPACE = 4,  /* workspace missing or smaller than qsa_workspace_bytes */
  QSA_ERR_DEVICE = 5,     /* current device is not gfx950 / no device */
  QSA_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
  QSA_ERR_SCRATCH = 7     /* the shape needs more scratch than qsa_forward_noalloc holds */
};

#define QSA_IDX_HEADS 4
#define QSA_IDX_DIM 64
#define QSA_BLOCK 4
#define QSA_TOPK 512
#define QSA_HEAD_DIM 128
#define QSA_MAX_TOK (QSA_TOPK * QSA_BLOCK + QSA_BLOCK) /* 2052 */

/* qsa_shape.flags: choice of the top-k engine.  Both give bit-identical
 * results; they differ in speed and workspace.  0 = automatic. */
#define QSA_FLAG_TOPK_TABLE 1u  /* score table + global histogram threshold */
#define QSA_FLAG_TOPK_STREAM 2u /* streaming per-query threshold, no score table */
#define QSA_FLAG_TOPK_SCAN 4u   /* sampled per-row bound, candidate segments per slice
                                   (shapes it cannot take fall back to STREAM) */

typedef struct {
  int32_t batch;     /* B >= 0 */
  int32_t max_len;   /* Lmax: cache capacity in tokens, > 0, multiple of 4, <= 2^30 */
  int32_t n_query;   /* Nq >= 0 query positions per sequence, <= max_len */
  int32_t q_heads;   /* Hq: core query heads, >= 1 */
  int32_t kv_heads;  /* Hkv: core KV heads, >= 1, divides Hq, Hq/Hkv <= 64 */
  float scale;       /* softmax scale; <= 0 selects 1/sqrt(128) */
  uint32_t flags;    /* at most one QSA_FLAG_TOPK_* ; 0 = automatic */
} qsa_shape;

/* Workspace query.  op is one of QSA_OP_*.  Returns the number of bytes the
 * call needs for this shape (0 when it needs none); ws may be NULL only when
 * the answer is 0. */
enum {
  QSA_OP_COMPRESS = 0,
  QSA_OP_INDEX_TOPK = 1,
  QSA_OP_EXPAND = 2,
  QSA_OP_SPARSE_ATTEND = 3,
  QSA_OP_FORWARD = 4,
  QSA_OP_DENSE_DECODE = 5,
  QSA_OP_BLOCK_TEACHER = 6
};
size_t qsa_workspace_bytes(const qsa_shape* shape, int32_t op);

/* Human-readable text of a status code (static storage, never NULL). */
const char* qsa_status_string(qsa_status status);

/* Step 1, key compression: the indexer folds every four consecutive keys
 * into one micro-block key (page section "A million-token window with a
 * selective view").  For every sequence b writes
 *   k_cmp[b][j][:] = bf16( sum_{r<4} k_idx[b][4j+r][:] )
 * for j in [first_block[b], floor(lens[b]/4)): the sum is formed exactly (in
 * float64) and rounded once to nearest-even bf16.  Blocks outside that range
 * are not touched, so a decode loop compresses only newly completed blocks.
 * first_block may be NULL (= 0 for every sequence). */
qsa_status qsa_compress_keys(const qsa_shape* shape, const uint16_t* k_idx,
                             const int32_t* lens, const int32_t* first_block,
                             uint16_t* k_cmp, void* stream);

/* Steps 2 and 3, indexer scoring and top-k: every query scores the
 * compressed blocks and keeps the best-ranked ones (section "A million-token
 * window with a selective view"), at most 512 of them (opening section).
 * For the query at position t with
 * bt = floor(t/4) the candidates are the completed blocks j < bt, scored
 *   s_j = sum_{h<4} max(0, q_idx[h] . k_cmp[j])
 * (fp32 accumulation: exact for integer-valued inputs whose products and
 * sums stay below 2^24).  If bt <= 512 all candidates are kept, otherwise
 * the 512 largest under (score descending, index ascending).  sel holds the
 * kept block ids in ascending order, padded with -1; n_sel = min(bt, 512).
 * k_cmp must hold blocks [0, floor(max over queries of t / 4)) of each
 * sequence. */
qsa_status qsa_index_topk(const qsa_shape* shape, const uint16_t* q_idx,
                          const uint16_t* k_cmp, const int32_t* lens,
                          int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes,
                          void* stream);

/* Step 4, expansion: the kept blocks become the token positions they cover
 * (section "A million-token window with a selective view"), and the
 * unfinished tail block is added (opening section).  tok = ascending( {4j..4j+3 : j in sel} U {4bt..t} ),
 * padded with -1 to 2052; n_tok = 4*n_sel + (t mod 4) + 1.  sel must be
 * ascending with every id < bt (as qsa_index_topk writes it). */
qsa_status qsa_expand_blocks(const qsa_shape* shape, const int32_t* lens,
                             const int32_t* sel, const int32_t* n_sel, int32_t* tok,
                             int32_t* n_tok, void* stream);

/* Step 5, sparse core attention: core attention reads only the expanded
 * positions (section "A million-token window with a selective view").  The
 * token list of every query is rebuilt from (sel, n_sel) as in
 * qsa_expand_blocks; query head h reads KV head floor(h / (Hq/Hkv)):
 *   out[h] = softmax_s(scale * q[h] . k[s]) V[s],  lse[h] = ln sum_s exp(.)
 * bf16 inputs, fp32 accumulation and softmax, bf16 out.  lse may be NULL. */
qsa_status qsa_sparse_attend(const qsa_shape* shape, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, const int32_t* lens,
                             const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/* The whole sparse-attention module in one call: the measured module is the
 * indexer together with the sparse core attention (section "Three speed
 * claims, three different experiments"), whose steps are compression, block
 * ranking, expansion of the winners and attention over them (section "A
 * million-token window with a selective view").  Compresses blocks
 * [first_block[b], lens[b]/4) of k_idx into the caller-owned cache k_cmp
 * (first_block NULL = every block), then runs qsa_index_topk,
 * qsa_expand_blocks and qsa_sparse_attend on it, all enqueued on one stream;
 * outputs as those calls define them.  sel_out / n_sel_out may be NULL (then
 * the selection stays in the workspace); when given, both must be.  lse may
 * be NULL.  Blocks of k_cmp before first_block[b] must already hold the
 * compressed keys, as an earlier call wrote them. */
qsa_status qsa_forward(const qsa_shape* shape, const uint16_t* q_idx,
                       const uint16_t* k_idx, uint16_t* k_cmp, const int32_t* first_block,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* lens, uint16_t* out, float* lse, int32_t* sel_out,
                       int32_t* n_sel_out, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * serving loops or harnesses that forbid allocation): qsa_forward with the
 * same arguments except the workspace.  Its scratch memory is a device array
 * of QSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; shapes whose qsa_workspace_bytes(shape, QSA_OP_FORWARD)
 * exceeds it are rejected with QSA_ERR_SCRATCH before anything is launched
 * (the 1M-context batch-4 x 4 decode needs well under it; a 16K-query
 * prefill chunk does not fit and needs qsa_forward).  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.  Every
 * call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (different streams or threads) race; serialise them.  Results are
 * those of qsa_forward. */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qsa_status qsa_forward_noalloc(const qsa_shape* shape, const uint16_t* q_idx,
                               const uint16_t* k_idx, uint16_t* k_cmp,
                               const int32_t* first_block, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* lens, uint16_t* out, float* lse,
                               int32_t* sel_out, int32_t* n_sel_out, void* stream);

/* Comparator: dense causal GQA over every position 0..t of each query (the
 * pages' speed baseline is grouped-query attention over the full context,
 * section "Three speed claims, three different experiments").  Same math and
 * layouts as qsa_sparse_attend with tok = {0..t}.  lse may be NULL. */
qsa_status qsa_dense_gqa_decode(const qsa_shape* shape, const uint16_t* q,
                                const uint16_t* k, const uint16_t* v,
                                const int32_t* lens, uint16_t* out, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

/* Paged K/V (the pages' speed baseline attends over a paged cache, section
 * "Three speed claims, three different experiments").  The core K and V of
 * all sequences live in pools of fixed-size pages, [n_pages][page_size][Hkv]
 * [128] bf16 each; token tok of sequence b is row tok mod page_size of page
 * page_table[b * max_pages + tok / page_size].  page_size is a power of two
 * in [1, 2^20]; max_pages * page_size >= Lmax; n_pages * page_size
 * < 2^31 (pool rows are 32-bit indices); page ids must lie in
 * [0, n_pages) (an id outside it is clamped: the read stays inside the pool
 * but returns another page).  Only pages holding tokens < lens[b] are read.
 * page_table is device memory owned by the caller.  The indexer caches
 * (k_idx, k_cmp) stay per sequence, as in qsa_forward. */
typedef struct {
  const int32_t* page_table; /* [B][max_pages] int32, device */
  int32_t page_size;         /* tokens per page */
  int32_t max_pages;         /* page-table entries per sequence */
  int32_t n_pages;           /* pages in each pool */
} qsa_paged_kv;

/* qsa_sparse_attend over paged K/V: same selection, math and outputs; k and
 * v are the page pools.  Workspace: QSA_OP_SPARSE_ATTEND. */
qsa_status qsa_sparse_attend_paged(const qsa_shape* shape, const uint16_t* q,
                                   const uint16_t* k_pool, const uint16_t* v_pool,
                                   const qsa_paged_kv* kv, const int32_t* lens,
                                   const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream);

/* qsa_forward over paged K/V: same arguments and results, K and V read
 * through the page table.  Workspace: QSA_OP_FORWARD. */
qsa_status qsa_forward_paged(const qsa_shape* shape, const uint16_t* q_idx,
                             const uint16_t* k_idx, uint16_t* k_cmp, const int32_t* first_block,
                             const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const qsa_paged_kv* kv, const int32_t* lens, uint16_t* out,
                             float* lse, int32_t* sel_out, int32_t* n_sel_out, void* ws,
                             size_t ws_bytes, void* stream);

/* qsa_dense_gqa_decode over paged K/V (the comparator as the pages run it).
 * Workspace: QSA_OP_DENSE_DECODE. */
qsa_status qsa_dense_gqa_decode_paged(const qsa_shape* shape, const uint16_t* q,
                                      const uint16_t* k_pool, const uint16_t* v_pool,
                                      const qsa_paged_kv* kv, const int32_t* lens,
                                      uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                      void* stream);

/* Comparator for a prefill chunk: dense causal GQA over positions 0..t of
 * each of the Nq queries (the pages compare a prefill chunk of the attention
 * module against paged GQA, section "Three speed claims, three different
 * experiments").  Same math and layouts as qsa_dense_gqa_decode, organised
 * for many queries: each workgroup stages K/V tiles once for up to 256
 * (query, head) columns of one KV head.  kv NULL: k and v are the contiguous
 * caches [B][Lmax][Hkv][128]; otherwise the page pools of *kv.  No
 * workspace; lse may be NULL. */
qsa_status qsa_dense_gqa_prefill(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const qsa_paged_kv* kv,
                                 const int32_t* lens, uint16_t* out, float* lse, void* stream);

/* The indexer's training target: the indexer is trained together with the
 * model and learns from the full-attention distribution (page "Qwen's
 * million-token window has a 2,048-token keyhole", section "The indexer is
 * trained, not bolted on").  Reading: that distribution pooled per
 * micro-block and averaged over the core query heads.  For every query row
 * writes teacher[b][i][j] (float, layout [B][Nq][Lmax/4]) =
 *   (1/Hq) sum_h sum_{s in block j, s <= t} exp(scale q_h . k_s - lse_h),
 * lse_h the dense causal log-sum-exp of head h over 0..t (so each row sums
 * to 1 over blocks 0..floor(t/4), the last one partial); entries past the
 * query's own block are 0.  A dense pass over K and V (for lse) and one over
 * K; float accumulation, the per-block sums added atomically (the last bits
 * of an entry may differ from run to run).  Workspace: QSA_OP_BLOCK_TEACHER. */
qsa_status qsa_block_teacher(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* lens, float* teacher,
                             void* ws, size_t ws_bytes, void* stream);

/* Selection recall: the share of a row's teacher mass on the positions QSA
 * attends to, its kept micro-blocks and its own block (whether the selection
 * keeps what the dense attention looks at, section "What a serious
 * evaluation should preserve").  recall[b][i] = sum_{j in sel} teacher[j] +
 * teacher[floor(t/4)], with (sel, n_sel) as qsa_index_topk writes them and
 * teacher as qsa_block_teacher writes it.  Equals the mean over heads of
 * exp(lse_sparse - lse_dense) up to rounding. */
qsa_status qsa_teacher_recall(const qsa_shape* shape, const int32_t* lens, const float* teacher,
                              const int32_t* sel, const int32_t* n_sel, float* recall,
                              void* stream);

/* Backward passes: the indexer and the model are trained together (section
 * "The indexer is trained, not bolted on"), so the sparse attention and the
 * indexer's scoring have gradients.  Float32 arithmetic; gradients of K, V,
 * k_cmp and k_idx are ADDED into caller-zeroed float32 buffers (atomically:
 * the last bits may vary from run to run), so chunks of a sequence can
 * accumulate into one buffer.
 *
 * qsa_sparse_attend_backward: given the forward's selection (sel, n_sel), its
 * output `out` (bf16) and log-sum-exp `lse`, and d_out = dL/dout (bf16, the
 * layout of out), over each query's token list (as qsa_sparse_attend):
 *   dq[h]  = scale sum_s ds_s k_s            (written, float [B][Nq][Hq][128])
 *   dk[s] += scale sum_h ds_s q_h, dv[s] += sum_h p_s d_out_h
 *                                             (added, float [B][Lmax][Hkv][128])
 * with p the attention weights, ds_s = p_s (d_out_h . v_s - d_out_h . out_h). */
qsa_status qsa_sparse_attend_backward(const qsa_shape* shape, const uint16_t* q,
                                      const uint16_t* k, const uint16_t* v, const int32_t* lens,
                                      const int32_t* sel, const int32_t* n_sel,
                                      const uint16_t* out, const float* lse,
                                      const uint16_t* d_out, float* dq, float* dk, float* dv,
                                      void* stream);

/* qsa_index_scores_backward: given d_scores = dL/ds (float [B][Nq][Lmax/4],
 * entries of each query's candidate blocks j < floor(t/4) read, others
 * ignored) of the indexer scores s_j = sum_h max(0, q_idx[h] . k_cmp[j]):
 *   dq_idx[h] += sum_j d_scores_j [q_idx[h] . k_cmp[j] > 0] k_cmp[j]
 *                                            (added, float [B][Nq][4][64])
 *   dk_cmp[j] += sum_i sum_h d_scores_ij [q_ih . k_cmp[j] > 0] q_ih
 *                                            (added, float [B][Lmax/4][64]). */
qsa_status qsa_index_scores_backward(const qsa_shape* shape, const uint16_t* q_idx,
                                     const uint16_t* k_cmp, const int32_t* lens,
                                     const float* d_scores, float* dq_idx, float* dk_cmp,
                                     void* stream);

/* qsa_compress_keys_backward: the compressed key is the sum of its block's
 * four token keys (section "A million-token window with a selective view"),
 * so dk_idx[b][4j + r] += dk_cmp[b][j] for r < 4 and every completed block
 * j < lens[b]/4 (float [B][Lmax][64] and [B][Lmax/4][64]). */
qsa_status qsa_compress_keys_backward(const qsa_shape* shape, const int32_t* lens,
                                      const float* dk_cmp, float* dk_idx, void* stream);

/* Debug builds (the library compiled with QSA_DEBUG, lib/libqsa_debug.so),
 * for finding caller bugs (not part of the method).  Every kernel clamps
 * caller-supplied values that index memory or bound a loop (lens outside
 * [Nq, Lmax], a selected block outside [0, bt), n_sel outside
 * [0, min(bt, 512)], a page id outside the pool, first_block past the
 * completed blocks) so that no access leaves its buffer; a debug build also
 * counts each value a guard caught.  qsa_debug_build returns 1 in such a
 * build, 0 otherwise.  qsa_debug_guard_hits waits for the current device to
 * finish its work, then stores the count since the previous call (clearing
 * it); in other builds it stores 0.  Not for use while kernels run on other
 * streams of the device. */
int32_t qsa_debug_build(void);
qsa_status qsa_debug_guard_hits(uint64_t* hits);

/* Kernel timing hook, for benchmarks and profilers (not part of the method).
 * qsa_profile_attach hands the library n_events caller-created hipEvent_t
 * handles (created with timing enabled, owned by the caller).  From then on,
 * on the calling thread, the i-th kernel the library enqueues carries
 * events[2i] and events[2i+1] in its own dispatch (hipExtLaunchKernel's start
 * and stop events), so their interval is that kernel's execution, until
 * n_events/2 launches have been recorded.
 * qsa_profile_detach stops recording and returns the number of bracketed
 * launches; qsa_profile_kernel_name(i) names the i-th one ("" when out of
 * range; valid until the next attach on this thread).  Recording adds no
 * packets to the stream. */
qsa_status qsa_profile_attach(void** events, int32_t n_events);
int32_t qsa_profile_detach(void);
const char* qsa_profile_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
