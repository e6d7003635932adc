// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

constexpr int kDim = 64;          // latent dimension (bytes per latent row)
constexpr int kSupMaskWords = 64; // Tree decode: one bit per super (at most 2048 supers)
constexpr uint64_t kMagic = 0x4c53414d49333535ull;

// Host descriptor behind the opaque lsa_index.
struct Index {
  uint64_t magic;
  lsa_index_params prm;
  char* arena;
  size_t arena_bytes;
  int64_t T;        // keys covered
  int64_t n_pool;   // complete pooled groups = T / pool
  int64_t n_full;   // complete blocks
  int64_t n_grp;    // complete Tree groups
  int64_t n_grp2;   // complete runs of tree2_group groups (third level)
  int32_t pend_slot;  // which of the two pending-latent slots is live
  // capacities
  int64_t max_pool, max_full, max_bkt, max_grp, max_sup, max_smem, max_grp2, max_top;
  // arena byte offsets
  int64_t off_pooled, off_cent, off_bcnt, off_boff, off_bmem, off_bfirst, off_blast;
  int64_t off_scent, off_scnt, off_soff, off_smem, off_leafsup, off_pend;
  int64_t off_tcent, off_tcnt, off_toff, off_tmem, off_suptop;
  int64_t off_sblk, off_skey;     // per super, per block of its group (Tree walk fill)
  int64_t off_bdesc;              // per bucket {first, last, count, offset}, packed
  int64_t off_kmws, kmws_bytes;   // k-means scratch (few-block clustering)
  int64_t used_bytes;

  template <class T> T* at(int64_t off) const { return reinterpret_cast<T*>(arena + off); }
  int64_t n_bkt() const { return n_full * prm.buckets + (n_pool - n_full * prm.block); }
};
static_assert(sizeof(Index) <= 512, "descriptor size");
constexpr size_t kIndexSizeof = 512;

// Device view of an index for the selection kernels.
struct IdxView {
  const int8_t* cent;     // [n_bkt][64]
  const int32_t* bcnt;    // members per bucket
  const int32_t* boff;    // first member slot
  const int32_t* bmem;    // member pooled ids
  const int32_t* bfirst;  // first member pooled id
  const int32_t* blast;   // last member pooled id
  const int4* bdesc;      // the four above, packed per bucket: {first, last, count, offset}
  const int32_t* leafsup; // leaf -> super id (Tree) or nullptr
  int32_t n_bkt;
  int32_t pool;
  int32_t dense;          // 1: cent = raw latents, bucket j = key j (pool 1)
  int32_t n_sup;
  const int8_t* scent;    // [n_sup][64]
  const int32_t* scnt;    // leaves per super cluster (Tree)
  const int32_t* soff;    // first leaf slot in smem
  const int32_t* smem;    // leaf ids grouped by super cluster
  int32_t covered;        // leaves inside complete groups (n_grp * group * buckets)
  // third level (n_top = 0: none)
  int32_t n_top;
  int32_t covered_sup;    // supers inside complete top groups (n_grp2 * group2 * tree_super)
  const int8_t* tcent;    // [n_top][64]
  const int32_t* tcnt;    // supers per top node
  const int32_t* toff;    // first super slot in tmem
  const int32_t* tmem;    // super ids grouped by top node
  const int32_t* suptop;  // super -> top node id, or -1
  int32_t n_pool;         // pooled vectors (keys [0, n_pool * pool) are in buckets)
  // Tree walk fill: per super s, G + 1 entries each (G = tgroup): sblk[s][k] is
  // the first slot of s's member list (relative to soff[s]) whose leaf lies in
  // block k of s's group or later, skey[s][k] the keys of s's leaves in blocks
  // before k of the group
  const int32_t* sblk;
  const int32_t* skey;
  int32_t tgroup;         // blocks per group (G)
  int32_t tsuper;         // supers per group (S)
  int32_t bpb;            // buckets per full block (C)
  int32_t tgroup2;        // groups per top group (third level)
  int64_t blk_keys;       // keys per block (block * pool)
};

struct SelArgs {
  const int8_t* latq;     // [nq][64]
  const int32_t* qpos;    // [nq], or nullptr: position = qpos_base + query index
  int32_t qpos_base;
  int32_t nq;
  int32_t budget, window, sinks, tree_top;
  int32_t early_budget, early_until;   // queries at t < early_until take early_budget
  int32_t tree2_top;                   // top nodes walked into (third Tree level)
  int32_t max_sel;
  int32_t* idx;           // [nq][max_sel]
  int32_t* cnt;           // [nq]
  const int32_t* only;    // nullable: serve only queries with only[q] != 0
};

// Long-range key budget of the query at position t.
__host__ __device__ inline int budget_at(const SelArgs& a, int t) {
  return t < a.early_until ? a.early_budget : a.budget;
}

// Batched one-key append for decode (all indexes share one layout).
struct DecodeAppendArgs {
  char* arena[16];
  int64_t n_pool[16];
  int64_t n_full[16];
  int32_t n_pend[16];
  int32_t pend_slot[16];
  int32_t batched[16];
  int64_t off_pooled, off_cent, off_bcnt, off_boff, off_bmem, off_bfirst, off_blast, off_pend;
  int64_t off_bdesc;
  int32_t p, N, C;
};

// Set the text lsa_last_error() reports and return `code` (LSA_E_HIP with
// the runtime's error string for fail_hip).
int fail_status(int code, const char* fmt, ...);
int fail_hip(hipError_t e, const char* where);

// Runs set() once per device (the current one), whatever the number of host
// threads calling; `done` is the caller's per-device bit set (devices 0..63;
// on a higher device id set() runs on every call).  For kernel attributes,
// which are set per device.
hipError_t once_per_device(std::atomic<unsigned long long>& done, hipError_t (*set)());

// ---- launchers (return hipError_t) ----
hipError_t launch_decode_append(const DecodeAppendArgs& a, const int8_t* src, int nseq,
                                hipStream_t s);
hipError_t launch_select_multi(const IdxView* views, const int32_t* qpos, int32_t nseq,
                               const SelArgs& a, hipStream_t s);
hipError_t launch_pool(const int8_t* pend, int32_t n_pend, const int8_t* src, int64_t n_src,
                       int32_t p, int8_t* pooled_out, int64_t n_groups, hipStream_t s);
hipError_t launch_save_pending(const int8_t* pend, int32_t n_pend, const int8_t* src,
                               int64_t n_src, int32_t keep, int8_t* dst, hipStream_t s);
// Scratch for clustering up to kKmMaxBlk blocks of N points into C clusters
// with several workgroups per block (0: that path is not used).
constexpr int kKmMaxBlk = 8;
size_t kmeans_scratch_bytes(int32_t N, int32_t C);
hipError_t launch_kmeans(const int8_t* X, int32_t N, int32_t C, int32_t iters, int32_t nblk,
                         int64_t row0, int8_t* cent_out, int32_t* cnt_out, int32_t* off_out,
                         int32_t* mem_out, int32_t* first_out, int32_t* last_out,
                         int32_t* map_out, int32_t map_base, void* scratch,
                         size_t scratch_bytes, hipStream_t s);
// Per-super tables of the Tree walk for supers [s0, s0 + nsup) (see IdxView).
hipError_t launch_sup_tables(const int32_t* soff, const int32_t* scnt, const int32_t* smem,
                             const int32_t* bcnt, int32_t s0, int32_t nsup, int32_t S, int32_t G,
                             int32_t C, int32_t p, int32_t* sblk, int32_t* skey, hipStream_t s);
// Packed descriptors bdesc[b] = {bfirst, blast, bcnt, boff}[b] for buckets [b0, b1).
hipError_t launch_pack_desc(const int32_t* bfirst, const int32_t* blast, const int32_t* bcnt,
                            const int32_t* boff, int64_t b0, int64_t b1, int4* bdesc, hipStream_t s);
hipError_t launch_tail(const int8_t* pooled, int64_t g0, int64_t g1, int64_t n_full, int32_t N,
                       int32_t C, int8_t* cent, int32_t* bcnt, int32_t* boff, int32_t* bmem,
                       int32_t* bfirst, int32_t* blast, hipStream_t s);

size_t select_ws_bytes(int32_t nq);
hipError_t launch_select(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s);
// large Flat batches: list-based single full pass (+ exact kernel for flagged queries)
size_t select_fast_ws_bytes(int32_t nq);
hipError_t launch_select_fast(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s);
size_t dense_ws_bytes(int32_t nq);
hipError_t launch_dense_select(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s);
// Tree selection, one workgroup per query; workspace: select_tree_ws_bytes(nq)
size_t select_tree_ws_bytes(int32_t nq);
hipError_t launch_select_tree(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s);
// Tree decode: query i is sequence i's new position on its own index (<= 16);
// flags: nseq ints of workspace (0 served, 1 for the exact kernel, 2 for the streaming
// decode kernels with the chosen supers in supmask, kSupMaskWords per
// sequence; supmask nullptr: no flag 2)
hipError_t launch_select_tree_multi(const IdxView* views, const int32_t* qpos, int32_t nseq,
                                   const SelArgs& a, int32_t* flags, uint32_t* supmask, hipStream_t s);
// decode: one query per sequence, each on its own index (max_bkt = bucket
// capacity).  app (nullable): the one-key append of the batched sequences,
// enqueued before the selection (fused into its first kernel where it can);
// views describe the indexes after that append.
size_t select_dec_ws_bytes(int32_t nseq, int64_t max_bkt);
hipError_t launch_select_dec(const IdxView* views, const int32_t* qpos, int32_t nseq,
                             int64_t max_bkt, const SelArgs& a, void* ws, hipStream_t s,
                             const DecodeAppendArgs* app, const int8_t* app_src);

size_t attn_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t splits);
hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t kv_rows,
                       int64_t seq_stride_rows, int32_t seq_of_query_div,
                       const int32_t* idx, const int32_t* cnt, int32_t max_sel, int32_t nq,
                       const lsa_attn_params& ap, void* out, void* ws, int32_t splits,
                       hipStream_t s);
// consecutive query positions qpos0.., rows ending with the select rule's sinks and window
hipError_t launch_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              int64_t kv_rows, const int32_t* idx, const int32_t* cnt,
                              int32_t max_sel, int32_t nq, int64_t qpos0, int32_t window,
                              int32_t sinks, const lsa_attn_params& ap, void* out, float* lse,
                              hipStream_t s);

// Grouped variant of launch_attn_window: queries sorted by their rows' first
// long-range key and taken 16 / G at a time; each group's long-range rows
// are read once as a union.  Needs D in {64, 128}, G in {4, 8, 16} and
// grouped_attn_ok(); the workspace holds the sort, the sinks-and-window
// partials and the unions.  lcap: per-query long-range rows held in a union
// (a group with a longer row is walked row by row).  lse (nullable): per
// (query, head) natural log-sum-exp of the scaled logits, as the window path.
bool grouped_attn_ok(const lsa_attn_params& ap, int32_t lcap, int64_t kv_rows);
// queries one grouped call takes (the sort's padded size stays in int32)
constexpr int64_t kGroupedMaxQueries = (int64_t)1 << 26;
bool grouped_nq_ok(int64_t nq);
size_t attn_grouped_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t lcap);
// parts: kGroupedPrepare (sinks-and-window partials, query order, unions into
// the workspace) and / or kGroupedWalk (the long-range walk from them).
// latq (nullable, int8 [nq][64]): order the queries by the components of
// their latent nearest-neighbour graph; else by (first long-range key,
// MinHash of the row).
constexpr int kGroupedPrepare = 1, kGroupedWalk = 2;
hipError_t launch_attn_grouped(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int64_t kv_rows, const int32_t* idx, const int32_t* cnt,
                               int32_t max_sel, int32_t nq, int64_t qpos0, int32_t window,
                               int32_t sinks, int32_t lcap, const lsa_attn_params& ap,
                               const int8_t* latq, void* out, float* lse, void* ws, int parts,
                               hipStream_t s);

// The grouped attention's plan alone: query order (perm: slot -> query) and
// the unions of each group of qpw consecutive slots (urow / umask, ucap apart;
// ucnt -1 for a group over the cap), in the workspace's first
// grouped_plan_ws_bytes bytes.
struct GroupPlanView {
  const int32_t* perm;
  const int32_t* urow;
  const uint8_t* umask;
  const int32_t* ucnt;
  int32_t ucap, qpw, ngrp;
};
size_t grouped_plan_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t lcap);
hipError_t launch_grouped_plan(const int32_t* idx, const int32_t* cnt, int32_t max_sel, int32_t nq,
                               int64_t qpos0, int32_t window, int32_t sinks, int64_t kv_rows,
                               int32_t lcap, const lsa_attn_params& ap, const int8_t* latq, void* ws,
                               GroupPlanView* view, hipStream_t s);

// Backward of the sparse attention (dQ, dK, dV) over rows the select wrote
// for consecutive query positions qpos0.., with the index they came from.
struct BwdInputs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;            // forward output, bf16 or float32 (attention params out_f32)
  const uint16_t* dout;
  const float* lse;         // [nq][Hq] natural log-sum-exp from the forward
  int64_t kv_rows;
  const int32_t* idx;
  const int32_t* cnt;
  const int8_t* latq;       // nullable [nq][64]: the grouped dQ's order by latent neighbours
  int32_t max_sel, nq;
  int64_t qpos0;
  int32_t window, sinks, budget;
  float* dq;                // [nq][Hq][D]
  float* dk;                // [kv_rows][Hkv][D]
  float* dv;
  const int32_t* bcnt;
  const int32_t* boff;
  const int32_t* bmem;
  int32_t n_bkt, pool, n_pool;
  int64_t max_pool, max_bkt;  // index capacities (workspace layout)
  void* ws;
};
size_t attn_bwd_ws_bytes(int32_t nq, const lsa_attn_params& ap, int64_t max_pool, int64_t max_bkt,
                         int32_t budget);
hipError_t launch_attn_bwd(const BwdInputs& in, const lsa_attn_params& ap, hipStream_t s);

}  // namespace lsa
