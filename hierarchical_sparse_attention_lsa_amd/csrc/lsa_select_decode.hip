// Selection for decode steps: one query per sequence, each on its own index.
//
// The rule is the pages' ("Latent Sparse Attention: un indice gerarchico per
// contesti lunghi", search and D-LSA configuration paragraphs): buckets in
// (score desc, bucket asc) order, their eligible keys in ascending position
// until the long-range budget is met, then the window and the sinks.
//
// A decode step has few queries and a small index per sequence, so the work
// is spread differently from prefill:
//   k_dec_score   one thread per (sequence, bucket), 1024-bucket workgroups:
//                 the int8 dot product (v_dot4), the bucket's eligible keys
//                 for the new position and its first key slot go to the
//                 workspace, and each workgroup writes its histogram of
//                 eligible keys over score bins (a log scale of the score);
//   k_dec_select  one 1024-thread workgroup per slice of 1024 buckets of a
//                 sequence sums the partial histograms; the bin where the
//                 eligible keys reach the budget is the cutoff bin.  Buckets
//                 above it are taken whole: each slice writes its own, in
//                 ascending id order, after the earlier slices' (whose key
//                 counts the histograms give).  One more workgroup per
//                 sequence, alongside the slices, finds the same cutoff bin,
//                 gathers its (few) buckets, ranks them by order
//                 key, takes them in turn and writes their keys in id order
//                 after all the keys above the bin, then the sinks and the
//                 window.  A cutoff bin with more than BCAP buckets (many
//                 equal scores) takes the general path for those keys:
//                 histogram refinement of the order-key range until the
//                 bracket holding the cutoff has at most 256 entries, which
//                 are sorted.
//   k_dec_select_big  the same rule for indexes beyond the registers (more
//                 than 24576 buckets): the histogram summed from the partials,
//                 the scores streamed once from the workspace to classify.
#include <climits>
#include <cstring>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {
using namespace sel;

constexpr int DT = 1024;            // threads of the select workgroup
constexpr int DW = DT / 64;
constexpr int PERT_MAX = 24;        // buckets per thread (indexes of up to 24576 buckets)
constexpr int RB = 256;
constexpr int RCAP = 256;
// Score bins of the decode histogram, monotone in the score: magnitudes below
// 64 get a bin each, larger ones 64 bins per power of two (relative width
// 1/64), negative scores mirrored below zero.  |q . mu| <= 64 * 128 * 128 =
// 2^20, so a magnitude code stays below 1024 and a bin below NBIN.
constexpr int NBIN = 2048;
__device__ __forceinline__ int mag_code(int u) {
  if (u < 64) return u;
  const int e = 31 - __clz(u);
  return 64 + ((e - 6) << 6) + ((u >> (e - 6)) & 63);
}
__device__ __forceinline__ int score_bin(int s) { return s >= 0 ? 1024 + mag_code(s) : 1023 - mag_code(-s); }
// the magnitudes [lo, hi] with code c
__device__ __forceinline__ void code_range(int c, int* lo, int* hi) {
  if (c < 64) { *lo = *hi = c; return; }
  const int e = 6 + ((c - 64) >> 6), m = (c - 64) & 63;
  *lo = (64 + m) << (e - 6);
  *hi = ((65 + m) << (e - 6)) - 1;
}
// the scores [lo, hi] of bin b
__device__ __forceinline__ void bin_range(int b, int* lo, int* hi) {
  int a, z;
  if (b >= 1024) { code_range(b - 1024, &a, &z); *lo = a; *hi = z; }
  else { code_range(1023 - b, &a, &z); *lo = -z; *hi = -a; }
}
// Every taken bucket gives at least one key and the budget is at most 4096
// keys, so at most 4096 buckets are taken.
constexpr int TCAP = 4096;
constexpr int BCAP = 256;           // buckets of the cutoff bin the fast path ranks
static_assert(BCAP <= RCAP && BCAP <= DT, "the cutoff bin uses the bracket arrays, one thread per entry");
static_assert(TCAP % DT == 0 && DT * PERT_MAX / 32 <= DT, "list and bitmap shapes");

// dynamic LDS: the general path's per-bucket array, or the fast path's lists
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int dec_lds(int pert) { return cmax(pert * DT, 4 * TCAP + 2 * (DT * pert / 32)) * 4; }
constexpr int list_cap(int pert) { return pert * DT / 2; }   // taken buckets the emission list holds

struct DecViews {                   // first kernel argument (read through the kernarg pointer)
  IdxView v[16];
  int32_t qpos[16];
  int32_t nseq;
  int32_t cap;                      // workspace entries per sequence
};

struct DecWs {
  int32_t* score;                   // [nseq][cap] int8 dot products
  int32_t* elig;                    // [nseq][cap] eligible keys
  int32_t* kstart;                  // [nseq][cap] first eligible key slot
  int32_t* hpart;                   // [nseq][cap / DT rounded up][NBIN] eligible keys per score bin,
                                    // one histogram per score workgroup
  int32_t n_part;                   // histograms per sequence
  uint32_t* supmask;                // [nseq][kSupMaskWords] Tree: supers chosen
};



// crow: the bucket's centroid (global memory, or LDS for a bucket appended by
// this workgroup); bi: its descriptor
__device__ __forceinline__ void score_one(const IdxView& V, const SelArgs& A, const DecWs& W, int t,
                                          int seq, int cap, int beta, const int8_t* crow,
                                          const BucketInfo& bi, int* hist, bool cand) {
  const int* q4 = reinterpret_cast<const int*>(A.latq + (int64_t)seq * kDim);
  const int4* c4 = reinterpret_cast<const int4*>(crow);
  int acc = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int4 c = c4[k];
    acc = __builtin_amdgcn_sdot4(q4[4 * k + 0], c.x, acc, false);
    acc = __builtin_amdgcn_sdot4(q4[4 * k + 1], c.y, acc, false);
    acc = __builtin_amdgcn_sdot4(q4[4 * k + 2], c.z, acc, false);
    acc = __builtin_amdgcn_sdot4(q4[4 * k + 3], c.w, acc, false);
  }
  int klo = 0;
  const int e = cand ? eligible<false>(V, beta, bi, t, A.window, A.sinks, &klo) : 0;
  const int64_t at = (int64_t)seq * cap + beta;
  W.score[at] = acc;
  W.elig[at] = e;
  W.kstart[at] = bi.off * V.pool + klo;
  if (e > 0) atomicAdd(&hist[score_bin(acc)], e);
}

// The one-key append of each batched sequence is done here too (one launch
// less per step): the key goes to the pending buffer, or, when it completes
// a pooled group, the workgroup holding the new singleton bucket pools it,
// writes the bucket and scores it from LDS.  No other workgroup reads the new
// bucket, and the selection kernel runs after this one.
// TREE: only sequences with tsel[seq] == 2 are scored, and only their
// candidate leaves count as eligible: the leaves of the supers in W.supmask
// and the leaves outside complete groups.  No append then.
template <bool TREE>
__global__ void __launch_bounds__(DT) k_dec_score(DecViews VS, SelArgs A, DecWs W, DecodeAppendArgs D,
                                                  const int8_t* __restrict__ src,
                                                  const int32_t* __restrict__ tsel) {
  __shared__ int hist[NBIN];
  __shared__ __attribute__((aligned(16))) int8_t s_pv[kDim];
  __shared__ unsigned s_mask[kSupMaskWords];
  const DecViews* vsp = (const DecViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int seq = blockIdx.y;
  const IdxView V = vsp->v[seq];
  if (TREE) {
    if (tsel[seq] != 2) return;
    if (threadIdx.x < kSupMaskWords) s_mask[threadIdx.x] = W.supmask[(int64_t)seq * kSupMaskWords + threadIdx.x];
  }
  int beta_new = -1;
  int64_t g_new = 0;
  if (!TREE && D.batched[seq]) {                        // uniform
    char* abase = D.arena[seq];
    int8_t* pend = reinterpret_cast<int8_t*>(abase + D.off_pend) + (int64_t)D.pend_slot[seq] * D.p * kDim;
    const int np = D.n_pend[seq];
    if (np + 1 < D.p) {
      if (blockIdx.x == 0 && threadIdx.x < kDim)
        pend[np * kDim + threadIdx.x] = src[(int64_t)seq * kDim + threadIdx.x];
    } else {
      g_new = D.n_pool[seq];
      const int64_t nf = D.n_full[seq];
      const int64_t bn = nf * D.C + (g_new - nf * D.N);
      if ((int64_t)blockIdx.x == bn / DT) {             // uniform
        beta_new = (int)bn;
        if (threadIdx.x < kDim) {
          const int d = threadIdx.x;
          int sum = src[(int64_t)seq * kDim + d];
          for (int r = 0; r < np; ++r) sum += pend[r * kDim + d];
          const int8_t pv = (int8_t)rhe_div(sum, D.p);
          s_pv[d] = pv;
          reinterpret_cast<int8_t*>(abase + D.off_pooled)[g_new * kDim + d] = pv;
          reinterpret_cast<int8_t*>(abase + D.off_cent)[bn * kDim + d] = pv;
          if (d == 0) {
            reinterpret_cast<int32_t*>(abase + D.off_bcnt)[bn] = 1;
            reinterpret_cast<int32_t*>(abase + D.off_boff)[bn] = (int32_t)g_new;
            reinterpret_cast<int32_t*>(abase + D.off_bmem)[g_new] = (int32_t)g_new;
            reinterpret_cast<int32_t*>(abase + D.off_bfirst)[bn] = (int32_t)g_new;
            reinterpret_cast<int32_t*>(abase + D.off_blast)[bn] = (int32_t)g_new;
            reinterpret_cast<int4*>(abase + D.off_bdesc)[bn] = make_int4((int)g_new, (int)g_new, 1, (int)g_new);
          }
        }
      }
    }
  }
  if ((int)blockIdx.x * DT >= V.n_bkt) return;          // uniform: past this sequence's index
  for (int b = threadIdx.x; b < NBIN; b += DT) hist[b] = 0;
  __syncthreads();                                      // (also publishes the appended bucket here)
  const int beta = blockIdx.x * DT + threadIdx.x;
  if (beta < V.n_bkt) {
    bool cand = true;
    if (TREE && beta < V.covered) {
      const unsigned ls = (unsigned)V.leafsup[beta];
      cand = ls < 32u * kSupMaskWords && ((s_mask[ls >> 5] >> (ls & 31)) & 1u);
    }
    if (beta == beta_new) {
      BucketInfo bi;
      bi.first = bi.last = bi.off = (int)g_new;
      bi.cnt = 1;
      score_one(V, A, W, vsp->qpos[seq], seq, VS.cap, beta, s_pv, bi, hist, cand);
    } else {
      score_one(V, A, W, vsp->qpos[seq], seq, VS.cap, beta, V.cent + (int64_t)beta * kDim,
                load_bucket<false>(V, beta), hist, cand);
    }
  }
  __syncthreads();
  // the whole histogram, zeros included: nothing has to be cleared beforehand
  int2* out = reinterpret_cast<int2*>(W.hpart + ((int64_t)seq * W.n_part + blockIdx.x) * NBIN);
  for (int b = threadIdx.x; b < NBIN / 2; b += DT) out[b] = make_int2(hist[2 * b], hist[2 * b + 1]);
}


// ---- pieces shared by the decode select kernels (one workgroup per sequence) ----

// The window and the sinks after `out` taken keys, -1 padding, the count (wave 0).
__device__ __forceinline__ void dec_finish_row(const SelArgs& A, int seq, int t, int out) {
  const int lane = lane_id();
  if ((threadIdx.x >> 6) != 0) return;
  int32_t* row = A.idx + (int64_t)seq * A.max_sel;
  const int wstart = max(0, t - A.window + 1);
  const int ns = max(0, min(A.sinks, wstart));
  const int nw = t - wstart + 1;
  for (int k = lane; k < ns; k += 64) row[out + k] = k;
  for (int k = lane; k < nw; k += 64) row[out + ns + k] = wstart + k;
  const int totalk = out + ns + nw;
  for (int k = totalk + lane; k < A.max_sel; k += 64) row[k] = -1;
  if (lane == 0) A.cnt[seq] = totalk;
}

// Output slots [o_begin, out_total) from the nt taken buckets listed in
// ascending output offset: bucket r starts at output offset l_off[r] (the
// first at o_begin) and first key slot l_ks[r]; one output key per thread
// and round, four rounds in flight.
__device__ __forceinline__ void dec_emit_keys(const IdxView& V, const SelArgs& A, int seq, const int* l_off,
                                              const int* l_ks, int nt, int out_total, int o_begin = 0) {
  const int tid = threadIdx.x, p = V.pool;
  int32_t* row = A.idx + (int64_t)seq * A.max_sel;
  for (int o0 = o_begin + tid; o0 < out_total; o0 += 4 * DT) {
    int sl[4], g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = o0 + j * DT;
      sl[j] = 0;
      if (o < out_total) {
        int a = 0, b = nt - 1;         // last entry with l_off <= o
        while (a < b) {
          const int m = (a + b + 1) >> 1;
          if (l_off[m] <= o) a = m; else b = m - 1;
        }
        sl[j] = l_ks[a] + (o - l_off[a]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = o0 + j * DT < out_total ? V.bmem[sl[j] / p] : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (o0 + j * DT < out_total) row[o0 + j * DT] = g[j] * p + sl[j] % p;
  }
}

// LDS of the histogram path's tail.
struct DecTail {
  long long* cq;                    // [BCAP] order keys of the cutoff bin's buckets
  int* ci;                          // [BCAP] their ids
  int* ce;                          // [BCAP] their eligible keys
  int* re;                          // [BCAP] eligible keys by rank
  int* rs;                          // [BCAP] cutoff-bin slot by rank
  int* ired;                        // [DW] block scan scratch
  int* nt;                          // taken buckets so far
  int* ids;                         // [TCAP] taken bucket ids, any order; later output offsets
  int* tks;                         // [TCAP] keys taken from them; later first key slots
  int* sid;                         // [TCAP] taken bucket ids, ascending
  int* stk;                         // [TCAP] keys taken, ascending bucket id
  unsigned* bm;                     // [nw] taken-id bitmap (cleared by the caller)
  int* wp;                          // [nw] taken ids before each word
};

// On entry ids/tks hold the buckets taken whole (*nt of them, any order) and
// cq/ci/ce the nb (<= BCAP) buckets of the cutoff bin.  Ranks the cutoff bin
// by order key, takes its buckets in turn until the budget is met (the last
// one cut at its lowest positions), orders every taken bucket by id through a
// bitmap of nw words, gives them output offsets and writes the row.
__device__ void dec_tail(const IdxView& V, const SelArgs& A, const int32_t* kstart, int seq, int t, int B,
                         int above, int nb, int nw, const DecTail& L) {
  const int tid = threadIdx.x;
  if (nb > 0) {                        // uniform
    // rank in the cut bin (order keys are distinct): larger keys first
    if (tid < nb) {
      const long long k = L.cq[tid];
      int r = 0;
      for (int i = 0; i < nb; ++i) r += L.cq[i] > k ? 1 : 0;
      L.re[r] = L.ce[tid];
      L.rs[r] = tid;
    }
    __syncthreads();
    int tot;
    const int x = tid < nb ? L.re[tid] : 0;
    const int before = block_excl_scan<DT>(x, L.ired, &tot);
    const int tk = max(0, min(x, B - above - before));
    if (tk > 0) {
      const int sl = L.rs[tid];
      const int q = atomicAdd(L.nt, 1);
      if (q < TCAP) { L.ids[q] = L.ci[sl]; L.tks[q] = tk; }
    }
    __syncthreads();
  }
  const int nt = min(*L.nt, TCAP);
  // ascending ids: an entry's rank is the number of taken ids below it
  for (int i = tid; i < nt; i += DT) atomicOr(&L.bm[L.ids[i] >> 5], 1u << (L.ids[i] & 31));
  __syncthreads();
  {                                    // word prefixes: thread tid takes words [tid*WPT, +WPT)
    const int wpt = (nw + DT - 1) / DT;
    int loc = 0;
    for (int k = 0; k < wpt; ++k) {
      const int w = tid * wpt + k;
      loc += w < nw ? __popc(L.bm[w]) : 0;
    }
    int totw;
    int pre = block_excl_scan<DT>(loc, L.ired, &totw);
    for (int k = 0; k < wpt; ++k) {
      const int w = tid * wpt + k;
      if (w < nw) { L.wp[w] = pre; pre += __popc(L.bm[w]); }
    }
  }
  __syncthreads();
  for (int i = tid; i < nt; i += DT) {
    const int id = L.ids[i], w = id >> 5;
    const int r = L.wp[w] + __popc(L.bm[w] & ((1u << (id & 31)) - 1u));
    L.sid[r] = id;
    L.stk[r] = L.tks[i];
  }
  __syncthreads();
  // output offsets: thread tid sums entries [tid*ENT, tid*ENT + ENT)
  constexpr int ENT = TCAP / DT;
  int loc = 0;
#pragma unroll
  for (int k = 0; k < ENT; ++k) {
    const int r = tid * ENT + k;
    loc += r < nt ? L.stk[r] : 0;
  }
  int out_total;
  int off = block_excl_scan<DT>(loc, L.ired, &out_total);   // its barriers end the reads of ids, tks
  int* soff = L.ids;
  int* sks = L.tks;
#pragma unroll
  for (int k = 0; k < ENT; ++k) {
    const int r = tid * ENT + k;
    if (r < nt) { soff[r] = off; off += L.stk[r]; }
  }
  for (int r = tid; r < nt; r += DT) sks[r] = kstart[L.sid[r]];
  __syncthreads();
  dec_emit_keys(V, A, seq, soff, sks, nt, out_total);
  dec_finish_row(A, seq, t, out_total);
}

// Order key from a score and a bucket id, recomputed where it is used: the
// empty asm keeps the compiler from hoisting all of a thread's keys out of the
// refinement loop as 64-bit loop invariants (which would not fit in registers).
__device__ __forceinline__ long long rebuilt_key(int s, int beta) {
  asm volatile("" : "+v"(beta));
  return order_key(s, beta);
}

// PERT buckets per thread: the smallest instance that holds the index is
// launched, since every pass costs VALU time per slot, used or not.  One
// workgroup per slice of DT buckets (grid: slices + 1 x sequences); the last
// workgroup of each sequence's row of the grid finishes the row, alongside
// the slices.
template <int PERT>
__global__ void __launch_bounds__(DT) k_dec_select(DecViews VS, SelArgs A, DecWs W,
                                                   int32_t* __restrict__ flags) {
  constexpr int kListCap = list_cap(PERT);
  __shared__ int s_hk[RB], s_hb[RB];
  __shared__ long long s_red[DW];
  __shared__ int s_ired[DW];
  __shared__ long long s_cq[RCAP];
  __shared__ int s_ci[RCAP];
  __shared__ int s_nc;
  __shared__ int s_cut[2];
  __shared__ long long s_r3[DW][3];
  extern __shared__ int s_e[];         // [bucket id]: eligible keys, later the keys taken
  const DecViews* vsp = (const DecViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int seq = blockIdx.y;
  const bool fin = blockIdx.x == gridDim.x - 1;     // the finishing workgroup
  const int slice = fin ? -1 : (int)blockIdx.x;    // buckets slice*DT .. slice*DT + DT - 1
  const IdxView V = vsp->v[seq];
  const int t = vsp->qpos[seq];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int B = budget_at(A, t);
  const int n = V.n_bkt;
  const int p = V.pool;
  const int64_t base = (int64_t)seq * VS.cap;
  const int nsl = max(1, (n + DT - 1) / DT);
  if (slice >= nsl) return;            // uniform: past this sequence's index
  if (n > DT * PERT) {                 // too large for registers: the exact kernel serves it
    if (fin && tid == 0) flags[seq] = 1;
    return;
  }
  // ---- fast path: the cutoff located in the score histogram ----
  // Buckets whose score bin lies above the bin where the eligible keys reach
  // the budget are taken whole; the buckets of that bin are ranked by order
  // key and taken in turn, the last one cut.  Every slice's workgroup finds
  // the cut bin from the summed partial histograms, writes the keys of its
  // own buckets above it (slices in order, ids ascending within a slice: the
  // earlier slices' keys above the cut give its output offset).  The
  // finishing workgroup finds the same cut bin, collects its buckets over the
  // whole sequence, ranks them, writes their keys after all the keys above the
  // bin, then the sinks and the window.  A cutoff bin of more than BCAP buckets (many equal
  // or near-equal scores) takes the general path below for those keys.
  int* l_off = s_e;                    // taken buckets: output offset, first key slot
  int* l_ks = s_e + DT;
  __shared__ int s_nt, s_nb;
  __shared__ int s_ce[BCAP], s_re[BCAP], s_rs[BCAP];
  __shared__ int s_fc[4];              // cut bin, keys above it, its scores [lo, hi]
  // bins from the top score down: thread tid takes bins NBIN-1-2tid (he[0])
  // and NBIN-2-2tid (he[1]), summed over the score workgroups (the slices),
  // and the same over the slices before this one (hb) and this one (hm)
  int he[2] = {0, 0}, hb[2] = {0, 0}, hm[2] = {0, 0};
  {
    {
      const int2* hp = reinterpret_cast<const int2*>(W.hpart + (int64_t)seq * W.n_part * NBIN) + (NBIN / 2 - 1 - tid);
      const int nh = (n + DT - 1) / DT;    // score workgroups that wrote a histogram (0 for an empty index)
      int w = 0;
      for (; w + 4 <= nh; w += 4) {
        int2 x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = hp[(int64_t)(w + k) * (NBIN / 2)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          he[0] += x[k].y; he[1] += x[k].x;
          if (w + k < slice) { hb[0] += x[k].y; hb[1] += x[k].x; }
          if (w + k == slice) { hm[0] = x[k].y; hm[1] = x[k].x; }
        }
      }
      for (; w < nh; ++w) {
        const int2 x = hp[(int64_t)w * (NBIN / 2)];
        he[0] += x.y; he[1] += x.x;
        if (w < slice) { hb[0] += x.y; hb[1] += x.x; }
        if (w == slice) { hm[0] = x.y; hm[1] = x.x; }
      }
    }
    if (tid == 0) { s_fc[0] = NBIN; s_fc[1] = 0; s_fc[2] = INT_MAX; s_fc[3] = INT_MAX; s_nt = 0; s_nb = 0; }
    // a thread's sum saturates at B + 1: every prefix below the budget stays exact
    int te;
    const int pe = block_excl_scan<DT>(min(he[0] + he[1], B + 1), s_ired, &te);
    if (B > 0 && te <= B) {            // every eligible bucket is taken whole
      if (tid == 0) { s_fc[0] = -1; s_fc[1] = te; s_fc[2] = INT_MIN; s_fc[3] = INT_MIN; }
    } else if (B > 0) {                // the bin where the keys above reach the budget
      int ce = pe;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (ce < B && he[j] >= B - ce) {
          const int bin = NBIN - 1 - (2 * tid + j);
          int lo, hi;
          bin_range(bin, &lo, &hi);
          s_fc[0] = bin; s_fc[1] = ce; s_fc[2] = lo; s_fc[3] = hi;
        }
        ce = he[j] >= B - ce ? B : ce + he[j];
      }
    }
    __syncthreads();
  }
  if (!fin) {                          // uniform: a slice's workgroup
    const int cut = s_fc[0], hi_s = s_fc[3];
    // keys above the cut bin in the earlier slices (this slice's output
    // offset) and in this one; both at most the budget
    long long pk = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (NBIN - 1 - (2 * tid + j) > cut) pk += ((long long)hb[j] << 32) | (long long)hm[j];
    pk = block_sum_ll<DT>(pk, s_red);
    const int before = (int)(pk >> 32), mine = (int)(pk & 0xffffffffll);
    // this slice's bucket of the thread, above the cut bin or in it
    const int j = slice * DT + tid;
    const int scv = j < n ? W.score[base + j] : 0;
    const int ev = j < n ? W.elig[base + j] : 0;
    const bool is_above = ev > 0 && scv > hi_s;
    // taken buckets in id order: output offset and first key slot (LDS)
    {
      int tot;
      const int pre = block_excl_scan<DT>(is_above ? (ev << 16) | 1 : 0, s_ired, &tot);
      if (is_above) {
        l_off[pre & 0xffff] = before + (pre >> 16);
        l_ks[pre & 0xffff] = W.kstart[base + j];
      }
      __syncthreads();
      dec_emit_keys(V, A, seq, l_off, l_ks, tot & 0xffff, before + mine, before);
    }
    return;
  }
  // ---- the finishing workgroup: the cutoff bin and the rest of the row ----
  const int above = s_fc[1], lo_s = s_fc[2], hi_s = s_fc[3];
  {
    // the sequence's buckets in the cutoff bin: thread tid reads buckets
    // u*DT + tid (all loads in flight before the first use)
    int sc[PERT], ev[PERT];
#pragma unroll
    for (int u = 0; u < PERT; ++u) {
      const int j = u * DT + tid;
      sc[u] = j < n ? W.score[base + j] : 0;
      ev[u] = j < n ? W.elig[base + j] : 0;
    }
    if (tid == 0) s_nb = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PERT; ++u) {
      if (ev[u] > 0 && sc[u] >= lo_s && sc[u] <= hi_s) {
        const int q = atomicAdd(&s_nb, 1);
        if (q < BCAP) { s_cq[q] = order_key(sc[u], u * DT + tid); s_ci[q] = u * DT + tid; s_ce[q] = ev[u]; }
      }
    }
    __syncthreads();
  }
  {
    const int nb = s_nb;
    if (nb <= BCAP) {                  // uniform; else the general path below
      // rank in the cut bin (order keys are distinct): larger keys first
      if (tid < nb) {
        const long long k = s_cq[tid];
        int r = 0;
        for (int i = 0; i < nb; ++i) r += s_cq[i] > k ? 1 : 0;
        s_re[r] = s_ce[tid];
        s_rs[r] = tid;
      }
      __syncthreads();
      int tot;
      const int x = tid < nb ? s_re[tid] : 0;
      const int bef = block_excl_scan<DT>(x, s_ired, &tot);
      const int tk = max(0, min(x, B - above - bef));
      // the taken ones (a prefix of the ranks), ordered by id: rank by id among them
      int* t_id = s_e + 2 * DT;
      int* t_tk = s_e + 3 * DT;
      if (tid < nb) { t_id[tid] = tk > 0 ? s_ci[s_rs[tid]] : INT_MAX; t_tk[tid] = tk; }
      __syncthreads();
      int my_id = INT_MAX, my_tk = 0, r = 0;
      if (tid < nb && t_tk[tid] > 0) {
        my_id = t_id[tid];
        my_tk = t_tk[tid];
        for (int i = 0; i < nb; ++i) r += t_id[i] < my_id ? 1 : 0;
      }
      __syncthreads();
      if (my_tk > 0) { t_id[r] = my_id; t_tk[r] = my_tk; }
      int nt_cut;
      const int ncut = __syncthreads_count(my_tk > 0);
      nt_cut = ncut;
      // output offsets after the keys above the cut bin, in id order
      const int xo = tid < nt_cut ? t_tk[tid] : 0;
      int cut_total;
      const int ob = block_excl_scan<DT>(xo, s_ired, &cut_total);
      if (tid < nt_cut) {
        l_off[tid] = above + ob;
        l_ks[tid] = W.kstart[base + t_id[tid]];
      }
      __syncthreads();
      dec_emit_keys(V, A, seq, l_off, l_ks, nt_cut, above + cut_total, above);
      dec_finish_row(A, seq, t, above + cut_total);
      if (tid == 0) flags[seq] = 0;
      return;
    }
  }
  // General path: the exact cutoff by histogram refinement of the order keys
  // over every bucket (thread tid holds the scores of buckets u*DT + tid, the
  // order key rebuilt from the score and the implicit bucket id; the eligible
  // counts sit in LDS indexed by bucket id); only the cutoff bin's buckets are
  // written here, after the `above` keys the slices wrote.
  int sc[PERT];
#define KEY(u) rebuilt_key(sc[u], (u) * DT + tid)
#define E(u) s_e[(u) * DT + tid]
  // f(u, E(u)) for every bucket of the thread; the LDS reads of each batch of
  // four are issued together instead of one round trip per bucket
  auto each = [&](auto&& f) {
#pragma unroll
    for (int u0 = 0; u0 < PERT; u0 += 4) {
      int eb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) eb[j] = E(u0 + j);
#pragma unroll
      for (int j = 0; j < 4; ++j) f(u0 + j, eb[j]);
    }
  };
  long long lo = LLONG_MAX, hi = LLONG_MIN, tot = 0;
  {
    int ev[PERT];                      // all loads in flight before the first use
#pragma unroll
    for (int u = 0; u < PERT; ++u) {
      const int j = u * DT + tid;
      sc[u] = j < n ? W.score[base + j] : 0;
      ev[u] = j < n ? W.elig[base + j] : 0;
    }
    __syncthreads();                   // the fast path's reads of s_e are over
#pragma unroll
    for (int u = 0; u < PERT; ++u) {   // branch-free: selects, no divergent blocks
      E(u) = ev[u];
      const long long ku = KEY(u);
      const bool ok = ev[u] > 0;
      lo = min(lo, ok ? ku : LLONG_MAX);
      hi = max(hi, ok ? ku : LLONG_MIN);
      tot += ok ? ev[u] : 0;
    }
  }
  // one block reduction for (sum, min, max)
  tot = lane63(wave_incl_scan(tot, 0ll, [](long long a, long long b) { return a + b; }));
  lo = lane63(wave_incl_scan(lo, LLONG_MAX, [](long long a, long long b) { return min(a, b); }));
  hi = lane63(wave_incl_scan(hi, LLONG_MIN, [](long long a, long long b) { return max(a, b); }));
  if (lane == 0) { s_r3[wave][0] = tot; s_r3[wave][1] = lo; s_r3[wave][2] = hi; }
  __syncthreads();
  tot = 0; lo = LLONG_MAX; hi = LLONG_MIN;
#pragma unroll
  for (int w = 0; w < DW; ++w) {
    tot += s_r3[w][0];
    lo = min(lo, s_r3[w][1]);
    hi = max(hi, s_r3[w][2]);
  }
  // keys above `hi` are taken whole; the bracket [lo, hi] holds the cutoff
  if (B <= 0) {
    hi = LLONG_MAX;                  // nothing is taken
    lo = LLONG_MAX;
  } else if (tot <= B) {
    hi = LLONG_MIN;                  // every eligible bucket is taken whole
    lo = LLONG_MIN + 1;
  } else {
    for (int pass = 0; pass < 8; ++pass) {
      const long long range = hi - lo + 1;
      int sh = 0;
      while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
      for (int i = tid; i < RB; i += DT) { s_hk[i] = 0; s_hb[i] = 0; }
      __syncthreads();
      long long ab = 0;
      each([&](int u, int eu) {
        const long long ku = KEY(u);
        ab += (eu > 0 && ku > hi) ? eu : 0;
        if (eu <= 0 || ku > hi || ku < lo) return;
        const int bin = (int)((hi - ku) >> sh);
        atomicAdd(&s_hk[bin], eu);
        atomicAdd(&s_hb[bin], 1);
      });
      ab = block_sum_ll<DT>(ab, s_red);
      if (wave == 0) {
        int h[RB / 64], c[RB / 64], loc = 0;
#pragma unroll
        for (int k = 0; k < RB / 64; ++k) { h[k] = s_hk[(RB / 64) * lane + k]; c[k] = s_hb[(RB / 64) * lane + k]; loc += h[k]; }
        int wt;
        const int ex = wave_excl_scan(loc, &wt);
        long long cum = ab + ex;
        int found = -1, fb = 0;
#pragma unroll
        for (int k = 0; k < RB / 64; ++k) {
          if (found < 0 && cum + h[k] >= B) { found = (RB / 64) * lane + k; fb = c[k]; }
          cum += h[k];
        }
        const unsigned long long mk = __ballot(found >= 0);
        const int src = mk ? __ffsll((long long)mk) - 1 : 0;
        const int bsel = __shfl(found, src), nbsel = __shfl(fb, src);
        if (lane == 0) {
          s_cut[0] = mk ? bsel : -1;
          s_cut[1] = mk ? nbsel : 0;
        }
      }
      __syncthreads();
      const int bin = s_cut[0], nb = s_cut[1];
      if (bin < 0) break;              // cannot happen: the bracket holds the cutoff
      const long long nhi = hi - ((long long)bin << sh);
      long long nlo = hi - ((long long)(bin + 1) << sh) + 1;
      if (nlo < lo) nlo = lo;
      lo = nlo; hi = nhi;
      __syncthreads();
      if (nb <= RCAP) break;
    }
  }
  // bracket entries: sorted by (score desc, id asc), taken in order, last one cut
  if (tid == 0) s_nc = 0;
  __syncthreads();
  long long full = 0;
  each([&](int u, int eu) {
    const long long ku = KEY(u);
    full += (eu > 0 && ku > hi) ? eu : 0;
    if (eu <= 0 || ku > hi || ku < lo) return;
    const int c = atomicAdd(&s_nc, 1);
    if (c < RCAP) { s_cq[c] = -ku; s_ci[c] = u * DT + tid; }
  });
  full = block_sum_ll<DT>(full, s_red);
  const int nc = min(s_nc, RCAP);
  const bool overflow = s_nc > RCAP;
  if (wave == 0 && nc > 0 && !overflow) {
    int np = 1;
    while (np < nc) np <<= 1;
    for (int i = nc + lane; i < np; i += 64) { s_cq[i] = LLONG_MAX; s_ci[i] = -1; }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int k = 2; k <= np; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = lane; i < np; i += 64) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const long long x = s_cq[i], y = s_cq[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { s_cq[i] = y; s_cq[ixj] = x; const int tmp = s_ci[i]; s_ci[i] = s_ci[ixj]; s_ci[ixj] = tmp; }
          }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
    }
    long long need = B - full;
    for (int b0 = 0; b0 < nc; b0 += 64) {
      const int i = b0 + lane;
      int ee = 0, li = -1;
      if (i < nc) { li = s_ci[i]; ee = s_e[li]; }
      int tot2;
      const int before = wave_excl_scan(ee, &tot2);
      const long long tk = max(0ll, min((long long)ee, need - before));
      if (li >= 0) s_e[li] = (int)tk;
      need -= tot2;
    }
  }
  __syncthreads();
  // keys taken per bucket: whole above the bracket, as the walk set them inside
  // it; the buckets above the cutoff bin are the slices' (written already).
  // (The bin's bounds are read back from LDS here: registers are short.)
  {
    // score <= the bin's top score exactly when the order key is <= that of
    // (top score, bucket 0), the largest key with that score
    const long long khs = order_key(s_fc[3], 0);
    each([&](int u, int eu) {
      const long long ku = KEY(u);
      E(u) = (eu > 0 && ku >= lo && ku <= khs) ? eu : 0;
    });
  }
  __syncthreads();
  // output offsets in ascending bucket id: thread tid sums ids
  // [tid*PERT, tid*PERT + PERT), block scans join the chunks
  int tk[PERT];
  int mine = 0, mcnt = 0;
#pragma unroll
  for (int u = 0; u < PERT; ++u) {
    tk[u] = s_e[tid * PERT + u];
    mine += tk[u];
    mcnt += tk[u] > 0 ? 1 : 0;
  }
  // one scan of (keys << 16 | buckets): key totals stay <= budget <= 4096 and
  // bucket totals <= 24576, so neither half carries into the other
  int packed_total;
  // (an overflowed bracket leaves more keys here; that result is discarded)
  const int packed = block_excl_scan<DT>((min(mine, 4096) << 16) | mcnt, s_ired, &packed_total);
  const int gab = s_fc[1];             // keys above the cutoff bin
  int off = gab + (packed >> 16), rank = packed & 0xffff;   // the scan's barriers end all reads of s_e
  const int out_total = gab + (packed_total >> 16), nt = packed_total & 0xffff;
  const bool ok = !overflow && nt <= kListCap;
  // list of taken buckets (output offset, first key slot), ascending ids, over s_e
  l_off = s_e;
  l_ks = s_e + kListCap;
  if (ok) {
#pragma unroll
    for (int u = 0; u < PERT; ++u) {
      if (tk[u] <= 0) continue;
      l_off[rank] = off;
      l_ks[rank] = W.kstart[base + tid * PERT + u];
      ++rank;
      off += tk[u];
    }
  }
  __syncthreads();
  if (ok) {
    dec_emit_keys(V, A, seq, l_off, l_ks, nt, out_total, gab);
    dec_finish_row(A, seq, t, out_total);
  }
  if (tid == 0) flags[seq] = ok ? 0 : 1;
#undef KEY
#undef E
}

// Indexes beyond the register-resident instance (more than DT * PERT_MAX
// buckets, up to BIG_NW * 32): the same rule, with the histogram summed from
// the score kernel's partials and the scores streamed from the workspace once
// to classify against the cutoff bin's score range; then the shared tail.  A
// cutoff bin of more than BCAP buckets flags the sequence for the exact kernel.
constexpr int BIG_NW = 10240;       // bitmap words: bucket ids below 327680
constexpr int BIG_LDS = (4 * TCAP + 2 * BIG_NW) * 4;
constexpr int BIG_U = 16;           // buckets per thread and batch (loads in flight)

// tree != 0: serve exactly the sequences flagged 2 by the Tree kernel (any
// size; the score kernel filtered their candidates), leaving the others.
__global__ void __launch_bounds__(DT) k_dec_select_big(DecViews VS, SelArgs A, DecWs W,
                                                       int32_t* __restrict__ flags, int tree) {
  __shared__ int s_ired[DW];
  __shared__ long long s_cq[BCAP];
  __shared__ int s_ci[BCAP], s_ce[BCAP], s_re[BCAP], s_rs[BCAP];
  __shared__ int s_fc[4];              // cut bin, keys above it, its scores [lo, hi]
  __shared__ int s_nt, s_nb;
  extern __shared__ int s_e[];         // ids, tks, sid, stk [TCAP], bm, wp [BIG_NW]
  const DecViews* vsp = (const DecViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int seq = blockIdx.x;
  const IdxView V = vsp->v[seq];
  const int t = vsp->qpos[seq];
  const int tid = threadIdx.x, lane = lane_id();
  const int B = budget_at(A, t);
  const int n = V.n_bkt;
  const int64_t base = (int64_t)seq * VS.cap;
  if (tree) {                          // uniform
    if (flags[seq] != 2) return;
  } else if (n <= DT * PERT_MAX) {     // k_dec_select serves it
    return;
  }
  if (n > BIG_NW * 32) {               // beyond the bitmap: the exact kernel serves it
    if (tid == 0) flags[seq] = 1;
    return;
  }
  const int32_t* sc = W.score + base;
  const int32_t* el = W.elig + base;
  if (tid == 0) { s_fc[0] = NBIN; s_fc[1] = 0; s_fc[2] = INT_MAX; s_fc[3] = INT_MAX; s_nt = 0; s_nb = 0; }
  // bins from the top score down: thread tid takes bins NBIN-1-2tid (he[0])
  // and NBIN-2-2tid (he[1]), summed over the score workgroups' partials
  int he[2] = {0, 0};
  {
    const int nwg = (n + DT - 1) / DT;
    const int2* hp = reinterpret_cast<const int2*>(W.hpart + (int64_t)seq * W.n_part * NBIN) + (NBIN / 2 - 1 - tid);
    int w = 0;
    for (; w + 8 <= nwg; w += 8) {
      int2 x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = hp[(int64_t)(w + k) * (NBIN / 2)];
#pragma unroll
      for (int k = 0; k < 8; ++k) { he[0] += x[k].y; he[1] += x[k].x; }
    }
    for (; w < nwg; ++w) {
      const int2 x = hp[(int64_t)w * (NBIN / 2)];
      he[0] += x.y;
      he[1] += x.x;
    }
  }
  int te;
  const int pe = block_excl_scan<DT>(min(he[0] + he[1], B + 1), s_ired, &te);
  if (B > 0 && te <= B) {
    if (tid == 0) { s_fc[0] = -1; s_fc[1] = te; s_fc[2] = INT_MIN; s_fc[3] = INT_MIN; }
  } else if (B > 0) {
    int ce = pe;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (ce < B && he[j] >= B - ce) {
        const int bin = NBIN - 1 - (2 * tid + j);
        int lo, hi;
        bin_range(bin, &lo, &hi);
        s_fc[0] = bin; s_fc[1] = ce; s_fc[2] = lo; s_fc[3] = hi;
      }
      ce = he[j] >= B - ce ? B : ce + he[j];
    }
  }
  __syncthreads();
  const int above = s_fc[1], lo_s = s_fc[2], hi_s = s_fc[3];
  const int nw = (n + 31) / 32;
  int* ids = s_e;
  int* tks = s_e + TCAP;
  int* sid = s_e + 2 * TCAP;
  int* stk = s_e + 3 * TCAP;
  unsigned* bm = reinterpret_cast<unsigned*>(s_e + 4 * TCAP);
  int* wp = s_e + 4 * TCAP + BIG_NW;
  for (int w = tid; w < nw; w += DT) bm[w] = 0u;
  // buckets above the cut bin are taken whole (slots reserved once per wave
  // and batch); the cut bin's buckets are collected
  // (every lane runs the same number of batches: the wave scan needs them all)
  for (int j0 = 0; j0 < n; j0 += BIG_U * DT) {
    int sv[BIG_U], ev[BIG_U];
#pragma unroll
    for (int u = 0; u < BIG_U; ++u) {
      const int j = j0 + u * DT + tid;
      sv[u] = j < n ? sc[j] : 0;
      ev[u] = j < n ? el[j] : 0;
    }
    unsigned m_above = 0, m_cut = 0;
#pragma unroll
    for (int u = 0; u < BIG_U; ++u) {
      const bool e = ev[u] > 0;
      m_above |= (e && sv[u] > hi_s ? 1u : 0u) << u;
      m_cut |= (e && sv[u] >= lo_s && sv[u] <= hi_s ? 1u : 0u) << u;
    }
    int wt;
    const int wpre = wave_excl_scan(__popc(m_above), &wt);
    int wb = 0;
    if (lane == 0 && wt > 0) wb = atomicAdd(&s_nt, wt);
    int pos = __shfl(wb, 0) + wpre;
#pragma unroll
    for (int u = 0; u < BIG_U; ++u) {
      if ((m_above & (1u << u)) && pos < TCAP) { ids[pos] = j0 + u * DT + tid; tks[pos] = ev[u]; }
      pos += (m_above >> u) & 1u;
    }
    if (m_cut) {
#pragma unroll
      for (int u = 0; u < BIG_U; ++u) {
        if (!(m_cut & (1u << u))) continue;
        const int q = atomicAdd(&s_nb, 1);
        if (q < BCAP) {
          s_cq[q] = order_key(sv[u], j0 + u * DT + tid);
          s_ci[q] = j0 + u * DT + tid;
          s_ce[q] = ev[u];
        }
      }
    }
  }
  __syncthreads();
  const int nb = s_nb;
  if (nb > BCAP) {                     // many equal scores: the exact kernel serves it
    if (tid == 0) flags[seq] = 1;
    return;
  }
  DecTail L{s_cq, s_ci, s_ce, s_re, s_rs, s_ired, &s_nt, ids, tks, sid, stk, bm, wp};
  dec_tail(V, A, W.kstart + base, seq, t, B, above, nb, nw, L);
  if (tid == 0) flags[seq] = 0;
}

size_t dec_layout(int32_t nseq, int32_t cap, DecWs* W, int32_t** flags, void* ws) {
  char* p = static_cast<char*>(ws);
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += (bytes + 255) / 256 * 256; return r; };
  DecWs w;
  const size_t n = (size_t)nseq * cap;
  w.score = reinterpret_cast<int32_t*>(take(n * sizeof(int32_t)));
  w.elig = reinterpret_cast<int32_t*>(take(n * sizeof(int32_t)));
  w.kstart = reinterpret_cast<int32_t*>(take(n * sizeof(int32_t)));
  w.n_part = (cap + DT - 1) / DT;
  w.hpart = reinterpret_cast<int32_t*>(take((size_t)nseq * w.n_part * NBIN * sizeof(int32_t)));
  w.supmask = reinterpret_cast<uint32_t*>(take((size_t)nseq * kSupMaskWords * sizeof(uint32_t)));
  int32_t* f = reinterpret_cast<int32_t*>(take((size_t)nseq * sizeof(int32_t)));
  if (W) *W = w;
  if (flags) *flags = f;
  return o;
}

}  // namespace

size_t select_dec_ws_bytes(int32_t nseq, int64_t max_bkt) {
  return dec_layout(nseq, (int32_t)max_bkt, nullptr, nullptr, nullptr);
}

hipError_t launch_select_dec(const IdxView* views, const int32_t* qpos, int32_t nseq,
                             int64_t max_bkt, const SelArgs& a, void* ws, hipStream_t s,
                             const DecodeAppendArgs* app, const int8_t* app_src) {
  if (nseq <= 0) return hipSuccess;
  DecViews vs;
  memset(&vs, 0, sizeof vs);
  bool tree = false;
  int nmax = 0, nmin = INT_MAX;
  for (int i = 0; i < nseq; ++i) {
    vs.v[i] = views[i];
    vs.qpos[i] = qpos[i];
    tree |= views[i].leafsup != nullptr;
    nmax = nmax > views[i].n_bkt ? nmax : views[i].n_bkt;
    nmin = nmin < views[i].n_bkt ? nmin : views[i].n_bkt;
  }
  vs.nseq = nseq;
  vs.cap = (int32_t)max_bkt;
  SelArgs b = a;
  b.nq = nseq;
  DecWs W;
  int32_t* flags;
  dec_layout(nseq, vs.cap, &W, &flags, ws);
  // the append rides on the score kernel; the other paths launch it first
  const bool fused = !tree && nmax > 0 && nmax <= BIG_NW * 32;
  if (app && !fused) {
    hipError_t e = launch_decode_append(*app, app_src, nseq, s);
    if (e != hipSuccess) return e;
  }
  static std::atomic<unsigned long long> big_done{0};
  auto big_attr = []() {
    return hipFuncSetAttribute((const void*)k_dec_select_big, hipFuncAttributeMaxDynamicSharedMemorySize,
                               BIG_LDS);
  };
  DecodeAppendArgs none;
  memset(&none, 0, sizeof none);
  if (tree) {
    // the Tree kernel; sequences whose candidates overflow it (flag 2) go
    // through the streaming pair on their candidate leaves; what is still
    // flagged goes to the exact kernel
    hipError_t e = launch_select_tree_multi(views, qpos, nseq, b, flags, W.supmask, s);
    if (e != hipSuccess) return e;
    if (nmax > 0 && nmax <= BIG_NW * 32) {
      e = once_per_device(big_done, big_attr);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_dec_score<true>, dim3((unsigned)((nmax + DT - 1) / DT), (unsigned)nseq), dim3(DT), 0,
                         s, vs, b, W, none, (const int8_t*)nullptr, (const int32_t*)flags);
      hipLaunchKernelGGL(k_dec_select_big, dim3((unsigned)nseq), dim3(DT), BIG_LDS, s, vs, b, W, flags, 1);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    b.only = flags;
    return launch_select_multi(views, qpos, nseq, b, s);
  }
  if (nmax > BIG_NW * 32) return launch_select_multi(views, qpos, nseq, b, s);
  const bool big = nmax > DT * PERT_MAX;
  const bool small = nmax <= DT * 20;
  if (nmax > 0) {
    hipLaunchKernelGGL(k_dec_score<false>, dim3((unsigned)((nmax + DT - 1) / DT), (unsigned)nseq), dim3(DT), 0,
                       s, vs, b, W, app ? *app : none, app_src, (const int32_t*)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t ae = once_per_device(attr_done, []() {
    hipError_t e = hipFuncSetAttribute((const void*)k_dec_select<20>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, dec_lds(20));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)k_dec_select<PERT_MAX>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, dec_lds(PERT_MAX));
  });
  if (ae != hipSuccess) return ae;
  // one workgroup per slice of DT buckets of each sequence, and one more
  // (the last) that finishes the row
  const unsigned nslx = (unsigned)max(1, min((nmax + DT - 1) / DT, PERT_MAX)) + 1;
  if (big) {
    // sequences above DT * PERT_MAX buckets: the streaming kernel (the other
    // kernels flag them and return; this one overwrites their flags); any
    // sequence flagged then goes to the exact kernel
    ae = once_per_device(big_done, big_attr);
    if (ae != hipSuccess) return ae;
    if (nmin <= DT * PERT_MAX)
      hipLaunchKernelGGL((k_dec_select<PERT_MAX>), dim3(nslx, (unsigned)nseq), dim3(DT), dec_lds(PERT_MAX), s,
                         vs, b, W, flags);
    hipLaunchKernelGGL(k_dec_select_big, dim3((unsigned)nseq), dim3(DT), BIG_LDS, s, vs, b, W, flags, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b.only = flags;
    return launch_select_multi(views, qpos, nseq, b, s);
  }
  if (small)
    hipLaunchKernelGGL((k_dec_select<20>), dim3(nslx, (unsigned)nseq), dim3(DT), dec_lds(20), s, vs, b, W, flags);
  else
    hipLaunchKernelGGL((k_dec_select<PERT_MAX>), dim3(nslx, (unsigned)nseq), dim3(DT), dec_lds(PERT_MAX), s, vs,
                       b, W, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The bracket always fits: every refinement pass narrows the key range by
  // more than 128x and keys span < 2^54, so at most 32 keys remain after 7
  // passes. The emission list can only overflow when more than kListCap
  // buckets are taken, which needs a budget above kListCap; only then can a
  // sequence be flagged, and the exact kernel serves the flagged ones.
  if (a.budget <= list_cap(small ? 20 : PERT_MAX)) return hipSuccess;
  b.only = flags;
  return launch_select_multi(views, qpos, nseq, b, s);
}

}  // namespace lsa
