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
  QSA_ERR_HIP = 6         /* a HIP runtime call or kernel launch failed */
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

typedef struct {
  int32_t batch;     /* B >= 0 */
  int32_t max_len;   /* Lmax: cache capacity in tokens, > 0, multiple of 4, <= 2^30 */
  int32_t n_query;   /* Nq >= 0 query positions per sequence, <= max_len */
  int32_t q_heads;   /* Hq: core query heads, >= 1 */
  int32_t kv_heads;  /* Hkv: core KV heads, >= 1, divides Hq, Hq/Hkv <= 64 */
  float scale;       /* softmax scale; <= 0 selects 1/sqrt(128) */
  uint32_t flags;    /* QSA_FLAG_* ; 0 = automatic */
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
  QSA_OP_DENSE_DECODE = 5
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

/* The whole layer step: compression of blocks [first_block[b], lens[b]/4)
 * into the caller-owned cache k_cmp, scoring and top-k, expansion and sparse
 * attention, all enqueued on one stream.  sel_out / n_sel_out may be NULL;
 * when given they receive the selection.  lse may be NULL. */
qsa_status qsa_forward(const qsa_shape* shape, const uint16_t* q_idx,
                       const uint16_t* k_idx, uint16_t* k_cmp, const int32_t* first_block,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* lens, uint16_t* out, float* lse, int32_t* sel_out,
                       int32_t* n_sel_out, void* ws, size_t ws_bytes, void* stream);

/* Comparator: dense causal GQA over every position 0..t of each query (the
 * pages' speed baseline is grouped-query attention over the full context,
 * section "Three speed claims, three different experiments").  Same math and
 * layouts as qsa_sparse_attend with tok = {0..t}.  lse may be NULL. */
qsa_status qsa_dense_gqa_decode(const qsa_shape* shape, const uint16_t* q,
                                const uint16_t* k, const uint16_t* v,
                                const int32_t* lens, uint16_t* out, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

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
