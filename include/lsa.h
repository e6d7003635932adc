/*
 * lsa.h -- C ABI of the Latent Sparse Attention (LSA) hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow the pages about the preprint "Latent Sparse
 * Attention: Towards Subquadratic Ultra-Long Context Attention" (arXiv
 * 2610.42147):
 *   - index build: "Latent Sparse Attention: un indice gerarchico per
 *     contesti lunghi" (mauroscia.it), paragraph on the index -- consecutive
 *     keys are pooled in small groups, the pooled sequence is split into
 *     blocks, the vectors of each block are grouped by similarity into
 *     buckets that keep a centroid and the indices of their original keys;
 *   - search: same page, next paragraph -- the query is compared with the
 *     centroids to pick the buckets whose keys are fetched, then attention
 *     runs on the selected keys and values;
 *   - budget: same page, D-LSA configuration paragraph -- 64-d index
 *     representations, a fixed number of long-range keys (outside the recent
 *     window), plus the most recent keys and a few sink keys at the start;
 *   - hierarchy: "Prefrontal's Latent Sparse Attention speeds up one
 *     attention layer 72x at 10M tokens" (sysnote.net), section "What it
 *     changes" -- clusters grouped into a hierarchy that a query walks down,
 *     with the attention kernel itself unchanged.
 *
 * Conventions
 *   - Every device buffer is owned by the caller; the library never
 *     allocates device memory.  Pointers prefixed d_ are device pointers.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream); none synchronises it.
 *   - Arguments are validated before anything is enqueued; on an error
 *     nothing is enqueued and the index descriptor is unchanged.  A runtime
 *     or launch failure returns LSA_E_HIP.  lsa_last_error() gives a
 *     thread-local message for the last failing call.  No C++ exception
 *     crosses the ABI.
 *   - Calls on one index must be ordered on one stream; the API is not
 *     thread-safe per index.
 *   - Latents are int8, 64 per token, row-major [token][64].
 *   - Q / K / V / O are bf16 bit patterns (uint16), token-major:
 *     Q and O [nq][Hq][D], K and V [rows][Hkv][D].  Head h reads KV head
 *     floor(h * Hkv / Hq).
 *   - Selected key lists are int32 rows of `max_sel` = budget + window + sinks
 *     entries: `cnt[i]` distinct key positions followed by -1 padding.  The
 *     row is a set written in a fixed order: the taken buckets, each with
 *     its eligible keys in ascending position, then the sinks not in the
 *     window, then the window.  lsa_select and lsa_prefill_chunk write the
 *     best-scoring taken bucket first and the others in ascending id (the
 *     grouped attention puts queries with equal first keys together); the
 *     decode step writes them in ascending id, and lsa_dense_select (one key
 *     a "bucket") its keys in an order of its own.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_API __attribute__((visibility("default")))

enum {
  LSA_OK = 0,
  LSA_E_ARG = 1,          /* null pointer, bad size or parameter */
  LSA_E_UNSUPPORTED = 2,  /* latent dim != 64, D not in {64,128}, Hq/Hkv not in 1..16, ... */
  LSA_E_CAPACITY = 3,     /* T beyond the index capacity, workspace too small */
  LSA_E_STATE = 4,        /* descriptor not initialised / corrupt */
  LSA_E_HIP = 5           /* HIP runtime or launch failure */
};

/* workspace query ops */
enum {
  LSA_OP_BUILD = 0,    /* n = T */
  LSA_OP_APPEND = 1,   /* n = new keys */
  LSA_OP_SELECT = 2,   /* n = queries */
  LSA_OP_ATTN = 3,     /* n = queries */
  LSA_OP_PREFILL = 4,  /* n = chunk length */
  LSA_OP_DECODE = 5,   /* n = sequences */
  LSA_OP_DENSE = 6,    /* n = queries */
  LSA_OP_ATTN_BWD = 7, /* n = queries; index, select and attention params */
  LSA_OP_ATTN_GROUPED = 8  /* n = queries; select and attention params */
};

/* Index shape.  dim must be 64.  pool >= 1.  block (pooled vectors per
 * block) is a multiple of 64 in [64, 16384]; buckets (clusters per block)
 * is a multiple of 16 in [16, 256] and <= block; iters >= 1.  Tree:
 * tree_group blocks per super group (0 = Flat), tree_super clusters per
 * group (multiple of 16, <= 256, tree_group*buckets <= 16384 and a multiple
 * of 64), tree_iters >= 1.  max_tokens = capacity in keys.  Third Tree
 * level (the hierarchy of the sysnote.net page, "What it changes", one
 * level deeper): the super clusters of each complete run of tree2_group
 * groups are clustered into tree2_super top nodes (tree2_group = 0: two
 * levels; else tree_group > 0, tree2_super a multiple of 16 in [16, 256],
 * tree2_group*tree_super <= 16384 and a multiple of 64, tree2_iters >= 1). */
typedef struct lsa_index_params {
  int32_t dim, pool, block, buckets, iters;
  int32_t tree_group, tree_super, tree_iters;
  int64_t max_tokens;
  int32_t tree2_group, tree2_super, tree2_iters;
} lsa_index_params;

/* Per-query selection: budget long-range keys (sinks <= j <= t - window),
 * the window [t-window+1, t] and the sinks [0, sinks).  window >= pool.
 * tree_top = super clusters a query walks into (Tree indexes only).
 * Position-dependent budget (mauroscia.it, D-LSA paragraph: on GLM, Flat
 * takes 2048 long-range keys for queries before position 1M): a query at
 * t < early_until takes early_budget long-range keys instead of budget;
 * 0 <= early_budget <= budget.  early_until = 0 turns it off.  Rows keep the
 * stride budget + window + sinks.  tree2_top = top nodes a query walks into
 * on an index with a third level (>= 1 there); the tree_top super clusters
 * are then the best among those under the chosen top nodes and those not
 * under any top node yet. */
typedef struct lsa_select_params {
  int32_t budget, window, sinks, tree_top;
  int32_t early_budget, early_until;
  int32_t tree2_top;
} lsa_select_params;

/* Attention shape.  D in {64, 128}; 1 <= Hq/Hkv <= 16, Hq % Hkv == 0.
 * scale = softmax scale (0 => 1/sqrt(D)).  out_f32 = 0: bf16 output;
 * 1: float32 output (same arithmetic, no final rounding). */
typedef struct lsa_attn_params {
  int32_t Hq, Hkv, D, out_f32;
  float scale;
} lsa_attn_params;

/* Opaque host descriptor; the caller provides lsa_index_sizeof() bytes. */
typedef struct lsa_index lsa_index;

/* Counts and arena byte offsets of the arrays of a built index.
 *   pooled   int8  [n_pool][64]     pooled latent vectors
 *   cent     int8  [n_bkt][64]      bucket centroids: block b owns ids b*C..b*C+C-1,
 *                                   then one singleton bucket per tail pooled vector
 *   bcnt     int32 [n_bkt]          members per bucket
 *   boff     int32 [n_bkt]          first member's slot in bmem
 *   bmem     int32 [n_pool]         pooled ids, grouped by bucket, ascending in each
 *   bfirst   int32 [n_bkt]          smallest member pooled id (INT32_MAX if empty)
 *   blast    int32 [n_bkt]          largest member pooled id (-1 if empty)
 *   scent    int8  [n_sup][64]      super centroids (Tree)
 *   scnt     int32 [n_sup]          leaves per super cluster
 *   soff     int32 [n_sup]          first leaf's slot in smem
 *   smem     int32 [n_grp*G*C]      leaf ids grouped by super cluster, ascending
 *   tcent    int8  [n_top][64]      top-node centroids (third level)
 *   tcnt     int32 [n_top]          super clusters per top node
 *   toff     int32 [n_top]          first super's slot in tmem
 *   tmem     int32 [n_grp2*G2*S]    super ids grouped by top node, ascending
 * Key ids of pooled id g are g*pool .. g*pool+pool-1. */
typedef struct lsa_index_info {
  int64_t T, n_pool, n_full, n_bkt, n_grp, n_sup;
  int64_t off_pooled, off_cent, off_bcnt, off_boff, off_bmem, off_bfirst, off_blast;
  int64_t off_scent, off_scnt, off_soff, off_smem;
  int64_t arena_bytes;
  int64_t n_grp2, n_top, off_tcent, off_tcnt, off_toff, off_tmem;
} lsa_index_info;

LSA_API const char* lsa_status_str(int status);
LSA_API const char* lsa_last_error(void);
/* Waits for the work enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and reports whether it ran: LSA_OK, or LSA_E_HIP with the HIP
 * error in lsa_last_error() when an earlier call's kernels failed on the
 * device (the calls themselves return once their work is enqueued). */
LSA_API int lsa_check(void* stream);

LSA_API size_t lsa_index_sizeof(void);
/* Device arena bytes needed for an index with these params (LSA_E_ARG /
 * LSA_E_UNSUPPORTED on invalid params). */
LSA_API int lsa_index_bytes(const lsa_index_params* prm, size_t* bytes);
/* Initialise the host descriptor `h` (lsa_index_sizeof() bytes) over the
 * caller's device arena (256-byte aligned).  The index starts empty (T=0). */
LSA_API int lsa_index_init(lsa_index* h, const lsa_index_params* prm, void* d_arena,
                           size_t arena_bytes);
LSA_API int lsa_index_get_info(const lsa_index* h, lsa_index_info* out);

/* Workspace bytes for `op` with `n` as documented in the LSA_OP_* enum.
 * Index params are needed for BUILD/APPEND/PREFILL/DECODE/SELECT, select
 * params for SELECT/PREFILL/DECODE/DENSE/ATTN_GROUPED, attention params for
 * ATTN/DECODE/ATTN_GROUPED; unused ones may be NULL.  For PREFILL the
 * attention params are optional: given, the size also covers the grouped
 * attention the chunk then runs. */
LSA_API int lsa_workspace_bytes(int op, const lsa_index_params* iprm,
                                const lsa_select_params* sprm, const lsa_attn_params* aprm,
                                int64_t n, size_t* bytes);

/* Build the index over keys [0, T) from scratch (pool, block k-means, tail
 * singletons, Tree super level).  d_latk: int8 [T][64], 16-byte aligned
 * (LSA_E_ARG otherwise; the same holds for the latent keys of
 * lsa_append_keys, lsa_prefill_chunk and lsa_decode_step). */
LSA_API int lsa_build_index(lsa_index* h, const int8_t* d_latk, int64_t T, void* d_ws,
                            size_t ws_bytes, void* stream);

/* Append n keys (positions T .. T+n-1).  Complete pooled groups become tail
 * singleton buckets; a tail block that fills is clustered; a Tree group that
 * completes gets its super level.  The result equals lsa_build_index over
 * all T+n keys. */
LSA_API int lsa_append_keys(lsa_index* h, const int8_t* d_latk_new, int64_t n, void* d_ws,
                            size_t ws_bytes, void* stream);

/* Select keys for nq queries: d_latq int8 [nq][64], d_qpos int32 [nq] with
 * 0 <= qpos < T (not checked on the device; a negative position is read as
 * 0).  Writes d_idx int32 [nq][max_sel] and d_cnt int32 [nq].  With a
 * workspace of lsa_workspace_bytes(LSA_OP_SELECT, .., nq) bytes, Flat
 * batches of 64 or more queries take the single-scan list path; without one
 * every query takes the exact refinement path (same rows, slower). */
LSA_API int lsa_select(const lsa_index* h, const int8_t* d_latq, const int32_t* d_qpos,
                       int32_t nq, const lsa_select_params* sp, int32_t* d_idx, int32_t* d_cnt,
                       void* d_ws, size_t ws_bytes, void* stream);

/* Attention of nq query tokens over their selected rows.  d_q [nq][Hq][D],
 * d_k / d_v [kv_rows][Hkv][D] bf16; d_idx / d_cnt as written by lsa_select
 * (row stride max_sel; key ids are clamped to [0, kv_rows)).  d_out
 * [nq][Hq][D] bf16 (or float32 when out_f32). */
LSA_API int lsa_sparse_attn(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                            int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                            int32_t max_sel, int32_t nq, const lsa_attn_params* ap, void* d_out,
                            void* d_ws, size_t ws_bytes, void* stream);

/* Attention of nq consecutive query tokens at positions qpos0 .. qpos0+nq-1
 * over rows in the layout lsa_select writes with select params *sp: each row
 * holds the long-range keys, then the sinks not in the window, then the
 * window (the order documented above).  The sinks and the window are not
 * read from the rows: they are the positions the select rule gives each
 * query, and each group of 16/G consecutive queries (G = Hq/Hkv) reads the
 * union of its sinks and windows once.  Requires max_sel >= budget + window +
 * sinks and qpos0 + nq <= kv_rows.  Same attention over the same key set as
 * lsa_sparse_attn on those rows; only the summation order differs.  (The
 * selection paragraphs of the mauroscia.it page fix the sinks and window;
 * sharing them between queries is this library's design.) */
LSA_API int lsa_sparse_attn_window(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                                   int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                                   int32_t max_sel, int32_t nq, int64_t qpos0,
                                   const lsa_select_params* sp, const lsa_attn_params* ap,
                                   void* d_out, void* stream);

/* lsa_sparse_attn_window with the long-range keys read once per group of
 * queries that share them.  Queries are put in an order where neighbours
 * select alike and taken 16/G at a time.  With d_latq (nullable; the int8
 * [nq][64] latent queries the rows were selected with) the order follows the
 * components of the queries' nearest-neighbour graph by latent distance, a
 * component's queries together and components ordered by the first entry of
 * their root query's row; with d_latq NULL it is by the first entry of each
 * row (on rows from lsa_select, the first key of the best-scoring bucket),
 * then by a MinHash of the row.  Either order is a pure function of the
 * inputs.  On the Flat 10M chunk the latent order leaves 0.69 of the
 * long-range entries to read against 0.77; on a three-level Tree index the
 * row order does better (0.60 against 0.63).  Each group's long-range entries are
 * merged into one list of distinct keys (the first query's row, then each
 * next query's keys not yet in it) with a mask of the queries that hold each
 * key, and the group walks that list once with each query's softmax masked
 * to its own keys, on top of its sinks and window (attended first, as in
 * lsa_sparse_attn_window).  Same attention over the same key set per query;
 * only the summation order differs, and it is the same on every call.  Needs D in {64, 128}, G = Hq/Hkv in {4,
 * 8, 16}, (16/G) * budget <= 16384, kv_rows < 2^28 and nq <= 2^26 (else
 * LSA_E_UNSUPPORTED), and a workspace of lsa_workspace_bytes(
 * LSA_OP_ATTN_GROUPED, .., nq) bytes (else LSA_E_CAPACITY).  A group holding
 * a row with more than `budget` long-range entries is walked row by row.
 * d_lse (nullable): as in lsa_sparse_attn_fwd, float32 [nq][Hq], for the
 * training forward.  (Grouping queries is this library's design; the pages
 * fix only what each query attends to.) */
LSA_API int lsa_sparse_attn_grouped(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                                    int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                                    int32_t max_sel, int32_t nq, int64_t qpos0,
                                    const int8_t* d_latq, const lsa_select_params* sp,
                                    const lsa_attn_params* ap, void* d_out, float* d_lse,
                                    void* d_ws, size_t ws_bytes, void* stream);

/* The two halves of lsa_sparse_attn_grouped, same arguments (prepare takes
 * no outputs, walk no latents), enqueued one after the other on one stream with the same
 * workspace: prepare attends every query's sinks and window into partial
 * results and builds the query order and the groups' unions in the
 * workspace; walk reads them, attends the unions and writes d_out (and
 * d_lse when not NULL).  The
 * split lets a caller time or schedule the long-range walk on its own. */
LSA_API int lsa_attn_grouped_prepare(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                                     int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                                     int32_t max_sel, int32_t nq, int64_t qpos0,
                                     const int8_t* d_latq, const lsa_select_params* sp,
                                     const lsa_attn_params* ap, void* d_ws, size_t ws_bytes,
                                     void* stream);
LSA_API int lsa_attn_grouped_walk(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                                  int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                                  int32_t max_sel, int32_t nq, int64_t qpos0,
                                  const lsa_select_params* sp, const lsa_attn_params* ap,
                                  void* d_out, float* d_lse, void* d_ws, size_t ws_bytes,
                                  void* stream);

/* Training forward: lsa_sparse_attn_window that also stores, per (query,
 * head), the natural log of the softmax denominator over the query's
 * selected keys, lse = log sum_j exp(scale * q . k_j): d_lse float32
 * [nq][Hq].  The backward takes it to rebuild the probabilities. */
LSA_API int lsa_sparse_attn_fwd(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                                int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                                int32_t max_sel, int32_t nq, int64_t qpos0,
                                const lsa_select_params* sp, const lsa_attn_params* ap,
                                void* d_out, float* d_lse, void* stream);

/* Backward of the sparse attention over stored selections (the N-LSA
 * paragraph of the mauroscia.it page: training keeps the selected key
 * indices for the backward pass).  The selection is fixed; gradients flow
 * through the softmax attention only.  Inputs are those of
 * lsa_sparse_attn_fwd plus its outputs d_out (bf16, or float32 when
 * ap->out_f32) and d_lse, and the upstream gradient d_dout bf16
 * [nq][Hq][D].  The rows must be the ones lsa_select / lsa_prefill_chunk
 * wrote for queries at positions qpos0 .. qpos0+nq-1 with index `h` in its
 * current state and select params *sp (the backward finds each taken bucket
 * in them: a run of long-range entries in one bucket, ending at the largest
 * key taken).  Requires qpos0 + nq <= T of the index <= kv_rows and sinks <=
 * 64.  Writes float32 d_dq [nq][Hq][D] and d_dk, d_dv [kv_rows][Hkv][D]
 * (every row; zero for keys no query selected).  Workspace:
 * lsa_workspace_bytes(LSA_OP_ATTN_BWD, .., nq).  Deterministic: every
 * gradient is summed in a fixed order.  d_latq (nullable, int8 [nq][64]):
 * dQ's long-range part walks groups of queries ordered as
 * lsa_sparse_attn_grouped orders them with these latents (else by their
 * rows). */
LSA_API int lsa_sparse_attn_bwd(const lsa_index* h, const uint16_t* d_q, const uint16_t* d_k,
                                const uint16_t* d_v, int64_t kv_rows, const int32_t* d_idx,
                                const int32_t* d_cnt, int32_t max_sel, int32_t nq, int64_t qpos0,
                                const int8_t* d_latq, const lsa_select_params* sp,
                                const lsa_attn_params* ap,
                                const void* d_out, const float* d_lse, const uint16_t* d_dout,
                                float* d_dq, float* d_dk, float* d_dv, void* d_ws,
                                size_t ws_bytes, void* stream);

/* One prefill chunk: append the chunk's n_chunk latent keys, select for its
 * n_chunk queries (positions T_old .. T_old+n_chunk-1, scored against the
 * index that already holds the chunk's keys), attend.  The caller has
 * written K/V rows up to T_old+n_chunk.  d_idx_opt / d_cnt_opt (nullable)
 * receive the selection; otherwise it lives in the workspace.  Attention
 * runs as lsa_sparse_attn_grouped when the shape allows it and the
 * workspace holds lsa_workspace_bytes(LSA_OP_PREFILL, .., ap, n_chunk) (the
 * attention params make that size cover the grouped attention; it passes
 * d_latq on a Flat or two-level Tree index and NULL on a three-level Tree
 * index, whose queries it then groups by their rows), else as
 * lsa_sparse_attn_window. */
LSA_API int lsa_prefill_chunk(lsa_index* h, const int8_t* d_latk_chunk, int64_t n_chunk,
                              const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                              const uint16_t* d_v, int64_t kv_rows, const lsa_select_params* sp,
                              const lsa_attn_params* ap, void* d_out, int32_t* d_idx_opt,
                              int32_t* d_cnt_opt, void* d_ws, size_t ws_bytes, void* stream);

/* One decode step for nseq (<= 16) independent sequences: append one key
 * per sequence (d_latk_new int8 [nseq][64]), select for each sequence's
 * new position with d_latq [nseq][64], attend with d_q [nseq][Hq][D].
 * Sequence i's K/V rows start at d_k + i*seq_stride_rows*Hkv*D (the caller
 * has written the new rows).  d_out [nseq][Hq][D].  All sequences' indexes
 * must share one lsa_index_params.  After the step the workspace begins
 * with the step's selection: int32 idx [nseq][max_sel], then, at the next
 * 256-byte boundary, int32 cnt [nseq]. */
LSA_API int lsa_decode_step(lsa_index* const* hs, int32_t nseq, const int8_t* d_latk_new,
                            const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                            const uint16_t* d_v, int64_t seq_stride_rows,
                            const lsa_select_params* sp, const lsa_attn_params* ap, void* d_out,
                            void* d_ws, size_t ws_bytes, void* stream);

/* lsa_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as lsa_decode_step, without the
 * workspace: the step runs in a device array inside the library, one per
 * GPU, of lsa_decode_step_noalloc_max_bytes() bytes (128 MiB), held until the
 * process ends.  A step that needs more workspace than that (see
 * lsa_workspace_bytes with LSA_OP_DECODE) returns LSA_E_CAPACITY and
 * enqueues nothing.  The call allocates nothing: no hipMalloc, no
 * allocating library routine.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller. */
LSA_API size_t lsa_decode_step_noalloc_max_bytes(void);
LSA_API int lsa_decode_step_noalloc(lsa_index* const* hs, int32_t nseq, const int8_t* d_latk_new,
                                    const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                                    const uint16_t* d_v, int64_t seq_stride_rows,
                                    const lsa_select_params* sp, const lsa_attn_params* ap,
                                    void* d_out, void* stream);

/* Quadratic comparator: every long-range key scored on its own latent
 * (q . latk[j]), best `budget` by (score desc, position asc), plus window
 * and sinks.  Same output format as lsa_select.  With a workspace of
 * lsa_workspace_bytes(LSA_OP_DENSE, .., nq) bytes and nq >= 64 it runs as
 * a sampled score threshold per query, one thresholded int8-MFMA scan of all
 * latents (split over key ranges) and an exact top-budget per query; without,
 * every query takes the exact refinement kernel. */
LSA_API int lsa_dense_select(const int8_t* d_latk, int64_t T, const int8_t* d_latq,
                             const int32_t* d_qpos, int32_t nq, const lsa_select_params* sp,
                             int32_t* d_idx, int32_t* d_cnt, void* d_ws, size_t ws_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
