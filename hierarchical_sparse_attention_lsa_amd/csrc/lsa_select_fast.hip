// Flat selection for prefill batches in one full scan of the centroids, as
// two kernels: a scan that collects candidate buckets and a per-query
// resolve.
//
// Same result as the exact refinement kernel (lsa_select.hip) -- the pages'
// rule: buckets in (score desc, bucket asc) order, their eligible keys in
// ascending position until the long-range budget is met ("Latent Sparse
// Attention: un indice gerarchico per contesti lunghi", search and D-LSA
// configuration paragraphs).
//
// k_scan (a workgroup per 64 queries):
//   1. sampled pass: score max / mean of each query over the non-empty
//      buckets of a strided subset of the centroids;
//   2. sampled pass: histogram of the sampled buckets' key counts between
//      mean and max; the threshold slo is set where the sample predicts
//      about twice the budget above it;
//   3. full pass: every (query, bucket) with score >= slo is appended to the
//      query's list, one contiguous array per query with its length in LDS
//      (a workgroup keeps one partly written line per query open, so the L2
//      merges the rare 8-byte appends into whole lines).
//   The centroids and bucket sizes stream through LDS in double-buffered
//   chunks (each centroid byte is read once per workgroup, all lanes keep
//   loads in flight) and the full pass is MFMA + compare + rare store.
// k_resolve (one 256-thread workgroup per query; the list's entries sit in
// registers, 16 per thread):
//   eligible key counts of the entries; if they reach the budget the cutoff
//   is in the list: histogram refinement finds a bracket of <= 256 entries,
//   entries above it are taken whole, the bracket is sorted and taken in
//   order with the last bucket cut; the taken buckets are sorted, the
//   best-scoring one first and the rest by id (bitonic, in registers), and
//   their keys written, every thread on its own output slots (ascending
//   bucket ids keep each query's gather walking the KV cache once from start
//   to end; the first key of a row names the query's best bucket, which the
//   grouped attention uses to put queries with similar selections together).
//   A query whose list overflowed or
//   falls short of the budget is flagged and the exact refinement kernel
//   recomputes it.
// The dense per-key comparator reuses k_scan with every latent key its own
// bucket: a sample launch sets each query's threshold, the full pass runs
// over key ranges x query tiles with a sub-list per (query, range), and
// k_dense_resolve keeps the budget's largest keys of each query.
#include <climits>
#include <cstring>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {
using namespace sel;

constexpr int CHT = 16;             // centroid tiles (16 buckets each) per staged chunk
constexpr int NB2 = 32;             // sample histogram bins
constexpr int LC = 8192;            // list entries per query slot
constexpr int RB = 256;             // list histogram bins
constexpr int RCAP = 256;           // bracket entries resolved by sorting
constexpr int ECAP = 1024;          // taken buckets per query (else the exact kernel)
constexpr int SAMPLE_CHUNKS = 64;

struct FastViews {                  // first kernel argument (read through the kernarg pointer)
  IdxView v[16];
  int32_t qpos[16];
  int32_t nviews;
  int32_t view_per_query;           // Tree: query q uses view q at position qpos[q]
};

struct ListWs {
  long long* key;     // [slots][LC] order keys
  int32_t* elig;      // [slots][LC] eligible keys, then the taken keys
  int32_t* kstart;    // [slots][LC] member slot * p + offset of the first eligible key
  int32_t* nlist;     // [slots] list lengths (may exceed LC: overflow)
  int32_t* meta;      // [slots][3]  query index (-1: empty slot), position, 1: the list holds
                      //             every bucket with an eligible key
  int32_t* flags;     // [nq] 1: recompute with the exact kernel
  int32_t* slo;       // dense: [slots] score threshold of each query (sample kernel -> scan)
};

// Dense comparator lists: the scan is split over kDenseSplit ranges of the
// keys, and each (query, range) appends to its own sub-list of kDenseSub
// entries, so no counter is shared between workgroups.  A query holds up to
// 4x the largest budget; its threshold aims at 2x.
constexpr int kDenseSplit = 8;
constexpr int kDenseList = 16384;
constexpr int kDenseSub = kDenseList / kDenseSplit;

template <int FW, int QS>
struct Cfg {
  static constexpr int FT = FW * 64;
  static constexpr int NQW = QS / 16;        // query groups (16 MFMA rows each)
  static constexpr int PH = FW / NQW;        // waves sharing a query group (tile phases)
  static_assert(FW % NQW == 0 && (PH == 1 || PH == 2 || PH == 4), "unsupported scan shape");
};

template <int FW, int QS>
struct __attribute__((aligned(16))) ScanLds {
  int q[QS];
  int t[QS];
  int smax[QS];
  int sn[QS];
  int slo[QS];
  int rhi[QS], rsh[QS], rabove[QS], rtarget[QS];   // second-level bins of the crossing bin
  long long ssum[QS];
  int hist[QS][NB2];
  int nl[QS];                       // list lengths
  v4i cent[2][CHT * 64];
  int cnt[2][CHT * 16];
  int2 fl[2][CHT * 16];             // first and last key position of each bucket (causal only)
};

// Runs f(c, buf) for chunks c = c0, c0 + step, ... < nchunks with chunk c
// staged in LDS buffer buf.  NSTG later chunks are in flight in registers
// while f runs (the stages take turns, so no register copy waits on a
// load), and each goes to the other LDS buffer after f.
// DENSE: the "centroids" are the latent keys themselves, each its own bucket
// of one key (pool 1): no bucket records are read.
template <bool DENSE, int NSTG, int FW, int QS, class F>
__device__ __forceinline__ void stream_chunks(const IdxView& V, ScanLds<FW, QS>& S, int c0,
                                              int step, int nchunks, bool causal, F&& f) {
  using C = Cfg<FW, QS>;
  const int tid = threadIdx.x;
  constexpr int PER = (CHT * 64 + C::FT - 1) / C::FT;
  struct Stage {
    v4i r[PER];
    int rc;
    int2 rfl;
  };
  auto gload = [&](Stage& st, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = k * C::FT + tid;
      const int tile = c * CHT + e / 64, slot = e & 63;
      const int beta = tile * 16 + (slot & 15);
      st.r[k] = (e < CHT * 64 && beta < V.n_bkt)
                    ? *reinterpret_cast<const v4i*>(V.cent + (int64_t)beta * kDim + 16 * (slot >> 4))
                    : v4i{0, 0, 0, 0};
    }
    const int bb = c * CHT * 16 + tid;
    const bool in = tid < CHT * 16 && bb < V.n_bkt;
    st.rc = in ? (DENSE ? 1 : V.bcnt[bb]) : 0;
    // without causal staging every bucket reads as eligible from key 0 (the
    // rule the threshold used before a query could precede most of the index)
    if (DENSE) st.rfl = (in && causal) ? make_int2(bb, bb) : make_int2(0, 0);
    else st.rfl = (in && causal) ? make_int2(V.bfirst[bb] * V.pool, V.blast[bb] * V.pool + V.pool - 1)
                                 : make_int2(0, 0);
  };
  auto swrite = [&](const Stage& st, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (k * C::FT + tid < CHT * 64) S.cent[buf][k * C::FT + tid] = st.r[k];
    if (tid < CHT * 16) { S.cnt[buf][tid] = st.rc; S.fl[buf][tid] = st.rfl; }
  };
  Stage st[NSTG];
  if (c0 < nchunks) { gload(st[0], c0); swrite(st[0], 0); }
#pragma unroll
  for (int k = 0; k < NSTG; ++k)
    if (c0 + (k + 1) * step < nchunks) gload(st[k], c0 + (k + 1) * step);
  __syncthreads();
  int buf = 0;
  int c = c0;
  // invariant at the top of step k: chunk c in LDS[buf], stage (k + j) % NSTG
  // holds chunk c + (j + 1) step for j < NSTG
  while (c < nchunks) {
#pragma unroll
    for (int k = 0; k < NSTG; ++k) {
      f(c, buf);
      if (c + step < nchunks) swrite(st[k], buf ^ 1);
      __syncthreads();
      buf ^= 1;
      if (c + (NSTG + 1) * step < nchunks) gload(st[k], c + (NSTG + 1) * step);
      c += step;
      if (c >= nchunks) break;
    }
  }
}

// Prefill over one index: slot s of workgroup b is query b*QS + s.  DENSE:
// the quadratic comparator (every long-range key scored on its own latent);
// only eligible keys join the lists, and the sample is denser (the cut is a
// few thousand keys out of millions).
// MODE 0: all phases in one workgroup per query tile (Flat).  The dense
// comparator splits them: MODE 1 runs the sampled passes and stores each
// query's threshold; MODE 2 runs the full pass over one of kDenseSplit key
// ranges per workgroup (grid: ranges x query tiles, range-major, so the
// workgroups resident together stream the same latents and share them in L2).
template <int FW, int QS, bool DENSE, int MODE = 0>
__global__ void __launch_bounds__(FW * 64) k_scan(FastViews VS, SelArgs A, ListWs W) {
  using C = Cfg<FW, QS>;
  // chunks in flight in registers: three where registers allow it without
  // costing occupancy, two for the dense full pass (three workgroups per CU)
  constexpr int kStages = 4;
  static_assert(MODE == 0 || DENSE, "only the dense scan is split");
  __shared__ ScanLds<FW, QS> S;
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const IdxView V = vsp->v[0];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int nqt = MODE == 2 ? (int)gridDim.x / kDenseSplit : (int)gridDim.x;
  const int krange = MODE == 2 ? (int)blockIdx.x / nqt : 0;
  const int64_t lbase = (int64_t)(MODE == 2 ? (int)blockIdx.x % nqt : (int)blockIdx.x) * QS;
  const int qgrp = wave % C::NQW;
  const int phase = wave / C::NQW;
  const int qrow = qgrp * 16 + 4 * (lane >> 4);    // slot of score row v = 0
  const int col = lane & 15;
  const int p = V.pool;

  for (int i = tid; i < QS; i += C::FT) {
    int q = (int)(lbase + i);
    if (q >= A.nq) q = -1;
    const int t = q < 0 ? -1 : max(0, A.qpos ? A.qpos[q] : A.qpos_base + q);
    S.q[i] = q; S.t[i] = t;
    S.smax[i] = INT_MIN; S.ssum[i] = 0; S.sn[i] = 0;
    if (MODE != 2) {
      W.meta[3 * (lbase + i)] = q;
      W.meta[3 * (lbase + i) + 1] = t;
    }
  }
  for (int e = tid; e < QS * NB2; e += C::FT) (&S.hist[0][0])[e] = 0;
  for (int e = tid; e < QS; e += C::FT) S.nl[e] = 0;
  __syncthreads();

  // Causal staging (each bucket's key range, so the threshold counts only the
  // keys a query may take and the lists skip buckets wholly past it) when more
  // than 1/8 of the index's keys lie past the earliest query's long-range
  // keys: a training-like batch.  Every wave finds the same answer.
  bool causal;
  {
    int tm = INT_MAX;
    for (int i = lane; i < QS; i += 64) tm = S.t[i] >= 0 ? min(tm, S.t[i]) : tm;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) tm = min(tm, __shfl_xor(tm, m));
    const long long keys = (long long)V.n_pool * V.pool;
    causal = tm != INT_MAX && keys - ((long long)tm - A.window) > keys / 8;
  }

  v4i qa = {0, 0, 0, 0};
  {
    const int q = S.q[qgrp * 16 + col];
    if (q >= 0) qa = *reinterpret_cast<const v4i*>(A.latq + (int64_t)q * kDim + 16 * (lane >> 4));
  }
  const int ntiles = (V.n_bkt + 15) >> 4;
  const int nchunks = (ntiles + CHT - 1) / CHT;
  const int sstep = max(1, nchunks / (DENSE ? 10 * SAMPLE_CHUNKS : SAMPLE_CHUNKS));
  bool act[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) act[v] = S.t[qrow + v] >= 0;
  // last long-range key position of each row's query (scalars: an array here
  // would be placed in LDS by the compiler)
  const int tl0 = S.t[qrow] - A.window, tl1 = S.t[qrow + 1] - A.window;
  const int tl2 = S.t[qrow + 2] - A.window, tl3 = S.t[qrow + 3] - A.window;

  if constexpr (MODE != 2) {
  // ---- 1. sampled max / mean over non-empty buckets ----
  {
    int smax[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN}, sn[4] = {0, 0, 0, 0};
    long long ssum[4] = {0, 0, 0, 0};
    stream_chunks<DENSE, kStages>(V, S, 0, sstep, nchunks, causal, [&](int c, int buf) __attribute__((always_inline)) {
      for (int tl = phase; tl < CHT; tl += C::PH) {
        const v4i z = {0, 0, 0, 0};
        const v4i sc = mfma_i8_16x16x64(qa, S.cent[buf][tl * 64 + lane], z);
        if (S.cnt[buf][tl * 16 + col] <= 0) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) { smax[v] = max(smax[v], sc[v]); ssum[v] += sc[v]; sn[v] += 1; }
      }
    });
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        smax[v] = max(smax[v], __shfl_xor(smax[v], m));
        sn[v] += __shfl_xor(sn[v], m);
        ssum[v] += shfl_xor_i64(ssum[v], m);
      }
      if (col == 0 && act[v]) {
        atomicMax(&S.smax[qrow + v], smax[v]);
        atomicAdd(&S.sn[qrow + v], sn[v]);
        atomicAdd((unsigned long long*)&S.ssum[qrow + v], (unsigned long long)ssum[v]);
      }
    }
    __syncthreads();
  }

  // ---- 2. sampled key-count histograms -> threshold ----
  // The sampled buckets' keys are binned by score (NB2 bins), first over
  // [mean, max]; the bin where the count from the top reaches the target is
  // then binned again, NB2 times finer, in a second sampled pass, so the
  // threshold sits within 1/NB2^2 of that range of the predicted cut.  A
  // bucket counts with all its keys when they are all long-range for the
  // query (the index may hold keys past it), else not at all.
  auto sample_hist = [&](const int (&lo)[4], const int (&hi)[4], const int (&sh)[4]) __attribute__((always_inline)) {
    stream_chunks<DENSE, kStages>(V, S, 0, sstep, nchunks, causal, [&](int c, int buf) __attribute__((always_inline)) {
      for (int tl = phase; tl < CHT; tl += C::PH) {
        const v4i z = {0, 0, 0, 0};
        const v4i sc = mfma_i8_16x16x64(qa, S.cent[buf][tl * 64 + lane], z);
        const int w = S.cnt[buf][tl * 16 + col] * p;
        const int kl = S.fl[buf][tl * 16 + col].y;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tv = v == 0 ? tl0 : v == 1 ? tl1 : v == 2 ? tl2 : tl3;
          if (sc[v] >= lo[v] && sc[v] <= hi[v] && w > 0 && kl <= tv)
            atomicAdd(&S.hist[qrow + v][(hi[v] - sc[v]) >> sh[v]], w);
        }
      }
    });
  };
  constexpr int TAKE_ALL = -(1 << 30);
  {
    int lo[4], hi[4], sh[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int qs = qrow + v;
      const int n = S.sn[qs];
      hi[v] = S.smax[qs];
      lo[v] = (act[v] && n > 0) ? (int)(S.ssum[qs] / n) : INT_MAX;
      int s = 0;
      if (lo[v] != INT_MAX)
        while (s < 30 && (((hi[v] - lo[v] + 1) + (1 << s) - 1) >> s) > NB2) ++s;
      sh[v] = s;
    }
    sample_hist(lo, hi, sh);
    // A query whose sample does not reach the target within [mean, max] takes
    // every bucket with an eligible key into its list (TAKE_ALL: any score
    // passes), and its list is then complete.
    for (int qs = tid; qs < QS; qs += C::FT) {
      int slo = INT_MAX, all = 0;
      S.rsh[qs] = -1;                  // no second-level pass
      if (S.t[qs] >= 0) {
        slo = TAKE_ALL;
        all = 1;
        const int n = S.sn[qs];
        if (n > 0) {
          const int mx = S.smax[qs], mn = (int)(S.ssum[qs] / n);
          int s = 0;
          while (s < 30 && (((mx - mn + 1) + (1 << s) - 1) >> s) > NB2) ++s;
          const int sampled = (nchunks + sstep - 1) / sstep;
          // twice the budget (Flat: buckets hold tens of keys, so the list is a
          // few hundred entries; dense: single keys, a list holds 4x the budget)
          const long long want = 2ll * budget_at(A, S.t[qs]);
          const long long target = (want * sampled + nchunks - 1) / nchunks;
          long long cum = 0;
          for (int b = 0; b < NB2; ++b) {
            const int hb = S.hist[qs][b];
            cum += hb;
            if (cum >= target) {
              slo = max(mn, mx - ((b + 1) << s) + 1);
              all = 0;
              if (s > 0) {             // the crossing bin [slo, mx - (b << s)], binned finer
                const int bhi = mx - (b << s);
                int s2 = 0;
                while (s2 < 30 && (((bhi - slo + 1) + (1 << s2) - 1) >> s2) > NB2) ++s2;
                S.rhi[qs] = bhi; S.rsh[qs] = s2;
                S.rabove[qs] = (int)min(cum - hb, (long long)INT_MAX);
                S.rtarget[qs] = (int)min(target, (long long)INT_MAX);
              }
              break;
            }
          }
        }
      }
      S.slo[qs] = slo;
      W.meta[3 * (lbase + qs) + 2] = all;
    }
    __syncthreads();
  }
  {
    // second-level bins of each query's crossing bin (queries without one
    // take part with an empty range)
    for (int e = tid; e < QS * NB2; e += C::FT) (&S.hist[0][0])[e] = 0;
    __syncthreads();
    int lo[4], hi[4], sh[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int qs = qrow + v;
      const bool two = act[v] && S.rsh[qs] >= 0;
      lo[v] = two ? S.slo[qs] : INT_MAX;
      hi[v] = two ? S.rhi[qs] : INT_MIN;
      sh[v] = two ? S.rsh[qs] : 0;
    }
    sample_hist(lo, hi, sh);
    __syncthreads();
    for (int qs = tid; qs < QS; qs += C::FT) {
      if (S.t[qs] < 0 || S.rsh[qs] < 0) continue;
      long long cum = S.rabove[qs];
      const int bhi = S.rhi[qs], s2 = S.rsh[qs];
      for (int b = 0; b < NB2; ++b) {
        cum += S.hist[qs][b];
        if (cum >= S.rtarget[qs]) { S.slo[qs] = max(S.slo[qs], bhi - ((b + 1) << s2) + 1); break; }
      }
    }
    __syncthreads();
  }
  if (MODE == 1) {
    for (int qs = tid; qs < QS; qs += C::FT) W.slo[lbase + qs] = S.slo[qs];
    return;
  }
  } else {
    for (int qs = tid; qs < QS; qs += C::FT) S.slo[qs] = W.slo[lbase + qs];
    __syncthreads();
  }

  // ---- 3. full pass: buckets at or above the threshold join the lists ----
  // The MFMA starts from -threshold, so a (query, bucket) pair is a hit when
  // its result is >= 0.  Per group of four tiles a lane folds the sign bits
  // of its 16 results into a mask (one alignbit each); only lanes with hits
  // loop over them (about one pair in a hundred), picking the result with a
  // select tree and taking the query's next list slot from an LDS counter.
  {
    constexpr int TPW = CHT / C::PH;    // this wave's tiles per chunk: phase, phase + PH, ...
    static_assert(TPW % 4 == 0, "the full pass takes groups of four of a wave's tiles");
    v4i bias;
#pragma unroll
    for (int v = 0; v < 4; ++v) bias[v] = act[v] ? -S.slo[qrow + v] : -(1 << 30);   // 1<<30: no score reaches it
    // each row's threshold as a scalar (selected by a run-time row below; an
    // array would be placed in scratch memory)
    const int sl0 = S.slo[qrow], sl1 = S.slo[qrow + 1], sl2 = S.slo[qrow + 2], sl3 = S.slo[qrow + 3];
    // Without causal staging every bucket's first key reads as 0, so a hit is
    // kept exactly when its row has long-range keys: one mask per group.
    unsigned rows_ok = 0;
    if (!DENSE && !causal)
      rows_ok = (tl0 >= 0 ? 0x1111u : 0u) | (tl1 >= 0 ? 0x2222u : 0u) | (tl2 >= 0 ? 0x4444u : 0u) |
                (tl3 >= 0 ? 0x8888u : 0u);
    // MODE 2: chunks [cb, ce) of this workgroup's key range, and the
    // (query, range) sub-list
    const int cb = MODE == 2 ? (int)((int64_t)krange * nchunks / kDenseSplit) : 0;
    const int ce = MODE == 2 ? (int)((int64_t)(krange + 1) * nchunks / kDenseSplit) : nchunks;
    constexpr int lcap = MODE == 2 ? kDenseSub : LC;
    const int64_t lstride = MODE == 2 ? kDenseList : LC;
    const int64_t loff = MODE == 2 ? (int64_t)krange * kDenseSub : 0;
    stream_chunks<DENSE, kStages>(V, S, cb, 1, ce, causal, [&](int c, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < TPW; g += 4) {
        int d[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const v4i r = mfma_i8_16x16x64(qa, S.cent[buf][(phase + C::PH * (g + u)) * 64 + lane], bias);
#pragma unroll
          for (int v = 0; v < 4; ++v) d[4 * u + v] = r[v];
        }
        unsigned miss = 0;                // bit k: pair k = 4u + v below the threshold
#pragma unroll
        for (int k = 15; k >= 0; --k) miss = __builtin_amdgcn_alignbit(miss, (unsigned)d[k], 31);
        unsigned hits = ~miss & 0xffffu;
        if (!DENSE && !causal) hits &= rows_ok;
        const int tb = c * CHT + phase + C::PH * g;   // tile of u: tb + PH * u
        if ((c + 1) * CHT * 16 > V.n_bkt) {           // last chunk: no buckets past the end
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if ((tb + C::PH * u) * 16 + col >= V.n_bkt) hits &= ~(0xfu << (4 * u));
        }
        while (hits) {
          const int k = __builtin_ctz(hits);
          hits &= hits - 1;
          // d[k] as a tree of bit selects (a plain d[k] would put d in memory)
          const unsigned m0 = 0u - (k & 1), m1 = 0u - ((k >> 1) & 1);
          const unsigned m2 = 0u - ((k >> 2) & 1), m3 = 0u - ((k >> 3) & 1);
          unsigned x[8], y[4], z[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = ((unsigned)d[2 * i + 1] & m0) | ((unsigned)d[2 * i] & ~m0);
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = (x[2 * i + 1] & m1) | (x[2 * i] & ~m1);
#pragma unroll
          for (int i = 0; i < 2; ++i) z[i] = (y[2 * i + 1] & m2) | (y[2 * i] & ~m2);
          const int dk = (int)((z[1] & m3) | (z[0] & ~m3));
          const int v = k & 3, u = k >> 2;
          // row v's threshold and last long-range position, as bit selects (a
          // select chain or an array indexed by v is turned into a table in
          // scratch memory)
          const int r0 = -(v & 1), r1 = -((v >> 1) & 1);
          const int s01 = sl0 ^ ((sl0 ^ sl1) & r0), s23 = sl2 ^ ((sl2 ^ sl3) & r0);
          const int t01 = tl0 ^ ((tl0 ^ tl1) & r0), t23 = tl2 ^ ((tl2 ^ tl3) & r0);
          const int sv = s01 ^ ((s01 ^ s23) & r1);
          const int tv = t01 ^ ((t01 ^ t23) & r1);
          const int beta = (tb + C::PH * u) * 16 + col;
          // a bucket whose first key is past the query's long-range range has no
          // eligible key (first pooled id of bucket beta: chunk-local slot beta - c*CHT*16;
          // without causal staging rows_ok has filtered the hits already);
          // a dense key joins only when it is eligible itself
          if (DENSE ? (beta >= A.sinks && beta <= tv)
                    : (!causal || S.fl[buf][beta - c * CHT * 16].x <= tv)) {
            const int qs = qrow + v;
            const int pos = atomicAdd(&S.nl[qs], 1);
            if (pos < lcap) W.key[(lbase + qs) * lstride + loff + pos] = order_key(dk + sv, beta);
          }
        }
      }
    });
    for (int e = tid; e < QS; e += C::FT)
      W.nlist[MODE == 2 ? (lbase + e) * kDenseSplit + krange : lbase + e] = S.nl[e];
  }
}

// One 256-thread workgroup per query slot.  The list's entries are dealt to
// the threads: thread tid holds entries tid + RT*u (u < TPQ) in registers.
constexpr int RT = 256;
constexpr int TPQ = 16;             // entries per thread
constexpr int KCAP = TPQ * RT;      // entries per query (else the exact kernel)
constexpr int ECAP2 = 1024;         // taken buckets per query (else the exact kernel)
constexpr int EPT = ECAP2 / RT;     // sorted taken buckets per thread

// Shared tail of the list resolve and the Tree select: exact selection over
// the entries a workgroup of RT threads holds in registers (order keys K,
// eligible key counts e; entries with e <= 0 take no part), then the row.
// Keys above `hi` are taken whole and the cutoff lies in [lo, hi] (the
// block-wide min / max of the keys with e > 0); `tot` is this thread's sum of
// e.  ksof(u) gives the first key slot of the thread's entry u.  `complete`:
// the entries are all of the query's candidates, so fewer eligible keys than
// the budget means every one is taken; otherwise the list must reach the
// budget.  Returns false (nothing written) when the query must go to the
// exact kernel.
struct ResolveLds {
  int hk[RB], hb[RB];
  long long red[RT / 64];
  int ired[RT / 64];
  long long cq[RCAP];   // bracket: -order key, then sorted
  int ci[RCAP];         // bracket: collection index (payload of the sort)
  int ce[RCAP], cks[RCAP];
  long long key[ECAP2]; // taken: (bucket id << 32 | entry); sort scratch; (offset << 32 | first key slot)
  int tk[ECAP2], ks[ECAP2];
  int nc, nt, cut[2];
};

template <int TPQ, class KsOf>
__device__ __forceinline__ bool select_and_emit(ResolveLds& L, const IdxView& V, const SelArgs& A,
                                                int q, int t, bool ok, const long long (&K)[TPQ],
                                                const int (&e)[TPQ], long long lo, long long hi,
                                                long long tot, bool complete, KsOf ksof) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int B = budget_at(A, t);
  const int p = V.pool;
  tot = block_sum_ll<RT>(tot, L.red);
  lo = block_min_ll<RT>(lo, L.red);
  hi = block_max_ll<RT>(hi, L.red);
  // the best-scoring eligible bucket (always taken when anything is): its
  // keys go first in the row, so a row's first long-range key names it
  const int top_id = hi == LLONG_MIN ? -1 : (int)(0xffffffffu - (unsigned)(hi & 0xffffffffll));
  bool all = false;
  if (complete && tot <= B) {         // every eligible candidate is taken whole
    all = true;
    hi = LLONG_MIN;
    lo = LLONG_MIN + 1;
  }
  ok = ok && (all || tot >= B);       // a list must hold the cutoff

  // histogram refinement: keys above `hi` are taken whole, the cutoff is in [lo, hi]
  if (ok && !all) {
    for (int pass = 0; pass < 8; ++pass) {
      const long long range = hi - lo + 1;
      int sh = 0;
      while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
      for (int i = tid; i < RB; i += RT) { L.hk[i] = 0; L.hb[i] = 0; }
      __syncthreads();
      long long ab = 0;
#pragma unroll
      for (int u = 0; u < TPQ; ++u) {
        ab += (e[u] > 0 && K[u] > hi) ? e[u] : 0;
        if (e[u] <= 0 || K[u] > hi || K[u] < lo) continue;
        const int bin = (int)((hi - K[u]) >> sh);
        atomicAdd(&L.hk[bin], e[u]);
        atomicAdd(&L.hb[bin], 1);
      }
      ab = block_sum_ll<RT>(ab, L.red);
      if (wave == 0) {
        int h[RB / 64], c[RB / 64], loc = 0;
#pragma unroll
        for (int k = 0; k < RB / 64; ++k) { h[k] = L.hk[(RB / 64) * lane + k]; c[k] = L.hb[(RB / 64) * lane + k]; loc += h[k]; }
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
        if (lane == 0) { L.cut[0] = mk ? bsel : -1; L.cut[1] = mk ? nbsel : 0; }
      }
      __syncthreads();
      const int bin = L.cut[0], nb = L.cut[1];
      if (bin < 0) { ok = false; break; }   // not reached: the bracket holds the cutoff
      const long long nhi = hi - ((long long)bin << sh);
      long long nlo = hi - ((long long)(bin + 1) << sh) + 1;
      if (nlo < lo) nlo = lo;
      lo = nlo; hi = nhi;
      __syncthreads();
      if (nb <= RCAP) break;
    }
  }

  // taken entries: above the bracket whole (straight into the taken list);
  // bracket entries collected for the ordered walk
    if (ok) {
#pragma unroll
    for (int u = 0; u < TPQ; ++u) {
      if (e[u] <= 0 || K[u] < lo) continue;
      const int beta = (int)(0xffffffffu - (unsigned)(K[u] & 0xffffffffll));
      if (K[u] > hi) {
        const int r = atomicAdd(&L.nt, 1);
        if (r < ECAP2) {
          L.key[r] = ((long long)beta << 32) | (unsigned)r;
          L.tk[r] = e[u];
          L.ks[r] = ksof(u);
        }
      } else {
        const int c = atomicAdd(&L.nc, 1);
        if (c < RCAP) { L.cq[c] = -K[u]; L.ci[c] = c; L.ce[c] = e[u]; L.cks[c] = ksof(u); }
      }
    }
  }
  long long full = 0;
#pragma unroll
  for (int u = 0; u < TPQ; ++u) full += (ok && e[u] > 0 && K[u] > hi) ? e[u] : 0;
  full = block_sum_ll<RT>(full, L.red);
  const int nc = L.nc;
  ok = ok && nc <= RCAP;
  if (ok && wave == 0 && nc > 0) {
    int np = 1;
    while (np < nc) np <<= 1;
    for (int i = nc + lane; i < np; i += 64) { L.cq[i] = LLONG_MAX; L.ci[i] = -1; }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int k = 2; k <= np; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = lane; i < np; i += 64) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const long long x = L.cq[i], y = L.cq[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { L.cq[i] = y; L.cq[ixj] = x; const int tmp = L.ci[i]; L.ci[i] = L.ci[ixj]; L.ci[ixj] = tmp; }
          }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
    }
    // walk in (score desc, id asc) order; the last bucket taken is cut
    long long need = B - full;
    for (int b0 = 0; b0 < nc; b0 += 64) {
      const int i = b0 + lane;
      int ee = 0, c = -1;
      if (i < nc) { c = L.ci[i]; ee = L.ce[c]; }
      int tot2;
      const int before = wave_excl_scan(ee, &tot2);
      const int tk = (int)max(0ll, min((long long)ee, need - before));
      if (tk > 0) {
        const int r = atomicAdd(&L.nt, 1);
        if (r < ECAP2) {
          const long long Kc = -L.cq[i];
          const int beta = (int)(0xffffffffu - (unsigned)(Kc & 0xffffffffll));
          L.key[r] = ((long long)beta << 32) | (unsigned)r;
          L.tk[r] = tk;
          L.ks[r] = L.cks[c];
        }
      }
      need -= tot2;
    }
  }
  __syncthreads();
  const int nt = L.nt;
  ok = ok && nt <= ECAP2;

  int32_t* row = A.idx + (int64_t)q * A.max_sel;
  if (ok) {
    // taken buckets: the best-scoring one first, then ascending id order
    // (padding sorts last); entry r of L.key is (id << 32 | r).  The sort key
    // is (id + 1, r), and (0, r) for the best bucket; ids below 2^21 - 1 sort
    // as 32-bit ((id + 1) << 10 | r).
    int src[EPT];
    if (V.n_bkt < (1 << 21) - 1) {
      int v[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        const int id = e < nt ? (int)(L.key[e] >> 32) : 0;
        v[i] = e < nt ? (int)(((id == top_id ? 0 : id + 1) << 10) | (L.key[e] & (ECAP2 - 1))) : INT_MAX;
      }
      block_bitonic<ECAP2, RT>(v, reinterpret_cast<int*>(L.key));
#pragma unroll
      for (int i = 0; i < EPT; ++i) src[i] = v[i] & (ECAP2 - 1);
    } else {
      long long v[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        const long long id = e < nt ? (L.key[e] >> 32) : 0;
        v[i] = e < nt ? (((id == top_id ? 0ll : id + 1) << 32) | (L.key[e] & 0xffffffffll)) : LLONG_MAX;
      }
      block_bitonic<ECAP2, RT>(v, L.key);
#pragma unroll
      for (int i = 0; i < EPT; ++i) src[i] = (int)(v[i] & 0xffffffffll);
    }
    // output offsets: a block scan over the sorted order
    int tk[EPT], ks[EPT], mine = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const bool in = tid * EPT + i < nt;
      tk[i] = in ? L.tk[src[i]] : 0;
      ks[i] = in ? L.ks[src[i]] : 0;
      mine += tk[i];
    }
    int out_total;
    int off = block_excl_scan<RT>(mine, L.ired, &out_total);   // barriers: the sort's reads of L.key are done
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (tid * EPT + i < nt) L.key[tid * EPT + i] = ((long long)off << 32) | (unsigned)ks[i];
      off += tk[i];
    }
    __syncthreads();
    // keys: thread tid writes output slots [tid*PO, tid*PO + PO), walking the
    // taken buckets from one binary search; all its member loads in flight
    constexpr int MAXPO = 16;          // budget <= 4096 = MAXPO * RT
    const int PO = (((out_total + RT - 1) / RT) + 3) & ~3;
    const int o0 = tid * PO;
    if (o0 < out_total) {
      int a = 0, b = nt - 1;           // last taken bucket with offset <= o0
      while (a < b) {
        const int m = (a + b + 1) >> 1;
        if ((int)(L.key[m] >> 32) <= o0) a = m; else b = m - 1;
      }
      long long ev = L.key[a];
      int nextoff = a + 1 < nt ? (int)(L.key[a + 1] >> 32) : INT_MAX;
      int sl[MAXPO], g[MAXPO];
#pragma unroll
      for (int jv = 0; jv < MAXPO; ++jv) {
        const int o = o0 + jv;
        sl[jv] = -1;
        if (jv < PO && o < out_total) {
          while (o >= nextoff) {
            ++a;
            ev = L.key[a];
            nextoff = a + 1 < nt ? (int)(L.key[a + 1] >> 32) : INT_MAX;
          }
          sl[jv] = (int)(ev & 0xffffffffll) + (o - (int)(ev >> 32));
        }
      }
#pragma unroll
      for (int jv = 0; jv < MAXPO; ++jv) g[jv] = sl[jv] >= 0 ? V.bmem[sl[jv] / p] : 0;
#pragma unroll
      for (int jv = 0; jv < MAXPO; jv += 4) {
        if (sl[jv] < 0) continue;
        int4 w;
        w.x = g[jv] * p + sl[jv] % p;
        w.y = g[jv + 1] * p + sl[jv + 1] % p;
        w.z = g[jv + 2] * p + sl[jv + 2] % p;
        w.w = g[jv + 3] * p + sl[jv + 3] % p;
        int32_t* dst = row + o0 + jv;
        if (sl[jv + 3] >= 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          *reinterpret_cast<int4*>(dst) = w;
        } else {
          dst[0] = w.x;
          if (sl[jv + 1] >= 0) dst[1] = w.y;
          if (sl[jv + 2] >= 0) dst[2] = w.z;
          if (sl[jv + 3] >= 0) dst[3] = w.w;
        }
      }
    }
    if (wave == 0) {
      const int out = out_total;
      const int wstart = max(0, t - A.window + 1);
      const int ns = max(0, min(A.sinks, wstart));
      const int nw = t - wstart + 1;
      for (int k = lane; k < ns; k += 64) row[out + k] = k;
      for (int k = lane; k < nw; k += 64) row[out + ns + k] = wstart + k;
      const int totalk = out + ns + nw;
      for (int k = totalk + lane; k < A.max_sel; k += 64) row[k] = -1;
      if (lane == 0) A.cnt[q] = totalk;
    }
  }
  return ok;
}

__global__ void __launch_bounds__(RT, 4) k_resolve(FastViews VS, SelArgs A, ListWs W) {
  __shared__ ResolveLds L;
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t slot = blockIdx.x;
  const int q = W.meta[3 * slot];
  if (q < 0) return;                 // uniform over the workgroup
  const int t = W.meta[3 * slot + 1];
  const bool complete = W.meta[3 * slot + 2] != 0;
  const IdxView V = vsp->v[0];
  const int B = budget_at(A, t);
  const int p = V.pool;
  const long long* lk = W.key + slot * LC;
  const int ntot = W.nlist[slot];
  if (tid == 0) { L.nc = 0; L.nt = 0; }
  // more entries than the registers hold (or than the list kept): exact kernel
  bool ok = B > 0 && ntot <= KCAP;

  // entries, their eligible keys and first key slots (all loads of a thread in flight together)
  // (the first key slot of entry f goes to kstart[f])
  long long K[TPQ];
  int e[TPQ];
  long long lo = LLONG_MAX, hi = LLONG_MIN, tot = 0;
  if (ok) {
#pragma unroll
    for (int u = 0; u < TPQ; ++u) {
      const int f = tid + RT * u;
      K[u] = f < ntot ? lk[f] : LLONG_MIN;
    }
    BucketInfo bi[TPQ];
#pragma unroll
    for (int u = 0; u < TPQ; ++u) {
      const int beta = (int)(0xffffffffu - (unsigned)(K[u] & 0xffffffffll));
      bi[u] = K[u] != LLONG_MIN ? load_bucket<false>(V, beta) : BucketInfo{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < TPQ; ++u) {
      e[u] = 0;
      if (K[u] == LLONG_MIN) continue;
      int klo;
      e[u] = eligible<false>(V, 0, bi[u], t, A.window, A.sinks, &klo);
      W.kstart[slot * LC + tid + RT * u] = bi[u].off * p + klo;
    }
#pragma unroll
    for (int u = 0; u < TPQ; ++u) {
      const bool in = e[u] > 0;
      lo = min(lo, in ? K[u] : LLONG_MAX);
      hi = max(hi, in ? K[u] : LLONG_MIN);
      tot += in ? e[u] : 0;
    }
  }
  ok = select_and_emit<TPQ>(L, V, A, q, t, ok, K, e, lo, hi, tot, complete,
                           [&](int u) { return W.kstart[slot * LC + tid + RT * u]; });
  if (tid == 0) W.flags[q] = ok ? 0 : 1;
}

// Dense comparator resolve: one RTD-thread workgroup per query slot.  Each
// list entry is one eligible key with its order key (score desc, position
// asc), in the query's kDenseSplit sub-lists; the query keeps its budget's
// largest keys (the result does not depend on the entries' order).  A
// histogram bracket narrows to at most RCAP entries around the cutoff, which
// one wave sorts; the kept keys are sorted by position and written, then the
// sinks and the window.  A sub-list that overflowed, or lists holding fewer
// than the budget without being complete, flag the query for the exact kernel.
constexpr int RTD = 512;
constexpr int DPT = kDenseList / RTD;   // list entries per thread
constexpr int DSUB = kDenseSub / RTD;   // of them per sub-list
constexpr int DKEEP = 4096;             // budget <= 4096
static_assert(DKEEP % RTD == 0 && kDenseSub % RTD == 0, "list and kept-key shapes");

__global__ void __launch_bounds__(RTD) k_dense_resolve(SelArgs A, ListWs W) {
  __shared__ int s_h[RB];
  __shared__ long long s_red[RTD / 64];
  __shared__ int s_ired[RTD / 64];
  __shared__ long long s_cq[RCAP];
  __shared__ int s_nc, s_cut;
  __shared__ int s_keys[DKEEP];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t slot = blockIdx.x;
  const int q = W.meta[3 * slot];
  if (q < 0) return;                 // uniform over the workgroup
  const int t = W.meta[3 * slot + 1];
  const bool complete = W.meta[3 * slot + 2] != 0;
  const int B = budget_at(A, t);
  int nsub[kDenseSplit], ntot = 0;
  bool over = false;
#pragma unroll
  for (int k = 0; k < kDenseSplit; ++k) {
    nsub[k] = W.nlist[slot * kDenseSplit + k];
    ntot += min(nsub[k], kDenseSub);
    over |= nsub[k] > kDenseSub;
  }
  if (over || (ntot < B && !complete)) {
    if (tid == 0) W.flags[q] = 1;
    return;
  }
  // entry u of this thread: sub-list u / DSUB, offset tid + RTD * (u % DSUB)
  const long long* lk = W.key + slot * kDenseList;
  long long K[DPT];
#pragma unroll
  for (int u = 0; u < DPT; ++u) {
    const int k = u / DSUB, f = tid + RTD * (u % DSUB);
    K[u] = f < nsub[k] ? lk[k * kDenseSub + f] : LLONG_MIN;
  }
  const int take = min(B, ntot);
  long long cut = LLONG_MIN + 1;     // keys >= cut are kept; padding (LLONG_MIN) never is
  if (take < ntot) {
    long long lo = LLONG_MAX, hi = LLONG_MIN;
#pragma unroll
    for (int u = 0; u < DPT; ++u) {
      if (K[u] == LLONG_MIN) continue;
      lo = min(lo, K[u]);
      hi = max(hi, K[u]);
    }
    lo = block_min_ll<RTD>(lo, s_red);
    hi = block_max_ll<RTD>(hi, s_red);
    for (int pass = 0; pass < 8; ++pass) {
      const long long range = hi - lo + 1;
      int sh = 0;
      while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
      for (int i = tid; i < RB; i += RTD) s_h[i] = 0;
      __syncthreads();
      long long ab = 0;
#pragma unroll
      for (int u = 0; u < DPT; ++u) {
        if (K[u] == LLONG_MIN) continue;
        if (K[u] > hi) { ++ab; continue; }
        if (K[u] >= lo) atomicAdd(&s_h[(int)((hi - K[u]) >> sh)], 1);
      }
      ab = block_sum_ll<RTD>(ab, s_red);
      if (wave == 0) {
        int h[RB / 64], loc = 0;
#pragma unroll
        for (int k = 0; k < RB / 64; ++k) { h[k] = s_h[(RB / 64) * lane + k]; loc += h[k]; }
        int wt;
        const int ex = wave_excl_scan(loc, &wt);
        long long cum = ab + ex;
        int found = -1, fb = 0;
#pragma unroll
        for (int k = 0; k < RB / 64; ++k) {
          if (found < 0 && cum + h[k] >= take) { found = (RB / 64) * lane + k; fb = h[k]; }
          cum += h[k];
        }
        const unsigned long long mk = __ballot(found >= 0);
        const int src = mk ? __ffsll((long long)mk) - 1 : 0;
        const int bsel = __shfl(found, src), nbsel = __shfl(fb, src);
        if (lane == 0) { s_cut = bsel; s_nc = nbsel; }
      }
      __syncthreads();
      const int bin = s_cut, nb = s_nc;
      __syncthreads();
      // (the bracket always holds the cutoff: bin >= 0)
      const long long nhi = hi - ((long long)bin << sh);
      long long nlo = hi - ((long long)(bin + 1) << sh) + 1;
      if (nlo < lo) nlo = lo;
      lo = nlo;
      hi = nhi;
      if (nb <= RCAP) break;
    }
    // the bracket's entries, sorted descending; the cutoff is the one that
    // completes `take` with the entries above the bracket
    if (tid == 0) s_nc = 0;
    __syncthreads();
    long long ab = 0;
#pragma unroll
    for (int u = 0; u < DPT; ++u) {
      if (K[u] == LLONG_MIN) continue;
      if (K[u] > hi) { ++ab; continue; }
      if (K[u] >= lo) {
        const int c = atomicAdd(&s_nc, 1);
        if (c < RCAP) s_cq[c] = -K[u];
      }
    }
    ab = block_sum_ll<RTD>(ab, s_red);
    const int nc = min(s_nc, RCAP);
    if (wave == 0) {
      int np = 1;
      while (np < nc) np <<= 1;
      for (int i = nc + lane; i < np; i += 64) s_cq[i] = LLONG_MAX;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      wave_bitonic(s_cq, np);
    }
    __syncthreads();
    cut = -s_cq[take - (int)ab - 1];
  }
  // kept keys, compacted in thread order, then sorted by position
  int mine = 0;
#pragma unroll
  for (int u = 0; u < DPT; ++u) mine += K[u] >= cut ? 1 : 0;
  int total;
  int at = block_excl_scan<RTD>(mine, s_ired, &total);
#pragma unroll
  for (int u = 0; u < DPT; ++u)
    if (K[u] >= cut) s_keys[at++] = (int)(0xffffffffu - (unsigned)(K[u] & 0xffffffffll));
  __syncthreads();
  constexpr int KPT = DKEEP / RTD;
  int v[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) v[i] = tid * KPT + i < total ? s_keys[tid * KPT + i] : INT_MAX;
  block_bitonic<DKEEP, RTD>(v, s_keys);
  int32_t* row = A.idx + (int64_t)q * A.max_sel;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (tid * KPT + i < total) row[tid * KPT + i] = v[i];
  if (wave == 0) {
    const int wstart = max(0, t - A.window + 1);
    const int ns = max(0, min(A.sinks, wstart));
    const int nw = t - wstart + 1;
    for (int k = lane; k < ns; k += 64) row[total + k] = k;
    for (int k = lane; k < nw; k += 64) row[total + ns + k] = wstart + k;
    const int totalk = total + ns + nw;
    for (int k = totalk + lane; k < A.max_sel; k += 64) row[k] = -1;
    if (lane == 0) A.cnt[q] = totalk;
  }
  if (tid == 0) W.flags[q] = 0;
}

// Tree selection ("Prefrontal's Latent Sparse Attention speeds up one
// attention layer 72x at 10M tokens", section "What it changes": clusters
// grouped into a hierarchy that a query walks down).  One 256-thread
// workgroup per query: score every super cluster (v_dot4), keep the
// tree_top best by (score desc, id asc) with a bitonic sort, enumerate their
// leaves plus the leaves outside complete groups, score those, and finish
// with the same exact selection and row emission as the list resolve.  A
// query with more supers or candidates than the registers hold is flagged
// for the exact kernel.
constexpr int SUPN = 2048;          // supers sorted per query (n_sup <= SUPN)
constexpr int CPT = 16;             // candidate leaves per thread
constexpr int TOPCAP = 256;         // tree_top served here
constexpr int kTreeStreamMin = 1024; // decode: more candidates may go to the streaming pair

__device__ __forceinline__ int dot64(const int (&qv)[16], const int8_t* c) {
  const int4* c4 = reinterpret_cast<const int4*>(c);
  int acc = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int4 x = c4[k];
    acc = __builtin_amdgcn_sdot4(qv[4 * k + 0], x.x, acc, false);
    acc = __builtin_amdgcn_sdot4(qv[4 * k + 1], x.y, acc, false);
    acc = __builtin_amdgcn_sdot4(qv[4 * k + 2], x.z, acc, false);
    acc = __builtin_amdgcn_sdot4(qv[4 * k + 3], x.w, acc, false);
  }
  return acc;
}

// Order of node `id` (< SUPN) with score s as 32 bits: (score desc, id asc)
// is the descending order of this key.  A 64-dim int8 dot product lies in
// [-1040384, 1048576], so s + 2^20 - 1 takes 21 bits and the id 11.
static_assert(SUPN <= 2048, "node ids take 11 bits of the node key");
__device__ __forceinline__ unsigned node_key(int s, int id) {
  return ((unsigned)(s + (1 << 20) - 1) << 11) | (unsigned)(2047 - id);
}

// The R best of n nodes by (score desc, id asc): candidate c is node id_of(c)
// with centroid cent[id]; out[r] = id of rank r (R <= n <= NS).  Every
// thread reads its candidates before the sort's first barrier and writes
// after it.
template <int NS, class IdOf>
__device__ __forceinline__ void top_nodes(const int8_t* cent, int n, IdOf id_of,
                                          const int (&qv)[16], int R, long long* tmp, int* out) {
  constexpr int PT = NS / RT;
  const int tid = threadIdx.x;
  // ascending sort of the complemented keys; padding (all ones) sorts last,
  // above every real key's complement (real keys are at least 8191 << 11)
  unsigned v[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int c = tid * PT + i;
    unsigned key = 0xffffffffu;
    if (c < n) {
      const int id = id_of(c);
      key = ~node_key(dot64(qv, cent + (int64_t)id * kDim), id);
    }
    v[i] = key;
  }
  block_bitonic<NS, RT>(v, reinterpret_cast<unsigned*>(tmp));
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int r = tid * PT + i;
    if (r < R) out[r] = 2047 - (int)(~v[i] & 2047u);
  }
}

// the smallest sort that holds the n nodes (n <= SUPN)
template <class IdOf>
__device__ __forceinline__ void top_nodes_any(const int8_t* cent, int n, IdOf id_of,
                                              const int (&qv)[16], int R, long long* tmp, int* out) {
  if (n <= 256) top_nodes<256>(cent, n, id_of, qv, R, tmp, out);
  else if (n <= 512) top_nodes<512>(cent, n, id_of, qv, R, tmp, out);
  else if (n <= 1024) top_nodes<1024>(cent, n, id_of, qv, R, tmp, out);
  else top_nodes<SUPN>(cent, n, id_of, qv, R, tmp, out);
}

// Prefix sums over the counts of the R nodes out[0..R) (wave 0): pre[j] =
// members of nodes before j, pre[TOPCAP] = all.
__device__ __forceinline__ void node_prefix(const int32_t* cnt, const int* nodes, int R, int* pre) {
  const int lane = lane_id();
  int c[TOPCAP / 64], loc = 0;
#pragma unroll
  for (int k = 0; k < TOPCAP / 64; ++k) {
    const int j = (TOPCAP / 64) * lane + k;
    c[k] = j < R ? cnt[nodes[j]] : 0;
    loc += c[k];
  }
  int all;
  int ex = wave_excl_scan(loc, &all);
#pragma unroll
  for (int k = 0; k < TOPCAP / 64; ++k) {
    pre[(TOPCAP / 64) * lane + k] = ex;
    ex += c[k];
  }
  if (lane == 0) pre[TOPCAP] = all;
}

// member f of the nodes listed in `nodes` (prefix `pre`): last node starting
// at or before f, then its slot in the member array
__device__ __forceinline__ int nth_member(const int32_t* off, const int32_t* mem, const int* nodes,
                                          const int* pre, int R, int f) {
  int a = 0, b = R - 1;
  while (a < b) {
    const int m = (a + b + 1) >> 1;
    if (pre[m] <= f) a = m; else b = m - 1;
  }
  return mem[off[nodes[a]] + (f - pre[a])];
}

// The walk over ranked nodes (ids[0..n) best first, n <= RT, out of `total`
// nodes): the first min(quota, total), then more in order while the keys held
// (`held`, plus w(id) of every node taken) stay below `need`.  Returns the
// number taken, or -1 when the n ranked nodes do not reach `need` and more
// nodes exist.  Every thread of the block must call it.
template <class W>
__device__ __forceinline__ int block_walk(const int* ids, int n, int total, int quota, long long held,
                                          int need, W w, int* ired, long long* lred) {
  const int tid = threadIdx.x;
  const int x = tid < n ? w(ids[tid]) : 0;
  int all;
  const int ex = block_excl_scan<RT>(x, ired, &all);
  const bool hit = tid < n && held + ex + x >= need;
  const long long first = block_min_ll<RT>(hit ? tid : LLONG_MAX, lred);
  const int base = min(quota, total);
  if (held >= need) return base;
  if (first != LLONG_MAX) return max(base, (int)first + 1);
  return n == total ? total : -1;
}

static_assert(SUPN / 32 == kSupMaskWords, "Tree decode super mask size");

// supmask (nullable, decode): a query whose supers were chosen but whose
// candidates overflow the registers (or whose cut does not resolve here) gets
// the chosen supers as a bit mask (kSupMaskWords words per query) and flag 2,
// for the streaming decode kernels; other flagged queries get flag 1.
__global__ void __launch_bounds__(RT, 4) k_tree_select(FastViews VS, SelArgs A, int32_t* flags,
                                                       uint32_t* supmask) {
  __shared__ ResolveLds L;
  __shared__ long long s_tmp[SUPN];
  __shared__ int s_sup[TOPCAP];       // selected supers
  __shared__ int s_pre[TOPCAP + 1];   // candidates before selected super j
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int q = blockIdx.x;
  // one index for every query (prefill), or one per query (decode: each
  // sequence's index and new position)
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const bool per_q = VS.view_per_query != 0;
  const IdxView V = vsp->v[per_q ? q : 0];
  const int t = max(0, per_q ? vsp->qpos[q] : (A.qpos ? A.qpos[q] : A.qpos_base + q));
  const int R = min(A.tree_top, V.n_sup);
  const int n_unc = V.n_bkt - V.covered;
  // no super level yet (no complete group): every leaf is a candidate
  const bool sup = V.n_sup > 0;
  bool ok = budget_at(A, t) > 0 && (!sup || (R >= 1 && R <= TOPCAP)) && V.n_sup <= SUPN;
  if (tid == 0) { L.nc = 0; L.nt = 0; }
  int qv[16];
  {
    const int4* q4 = reinterpret_cast<const int4*>(A.latq + (int64_t)q * kDim);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int4 x = q4[k];
      qv[4 * k] = x.x; qv[4 * k + 1] = x.y; qv[4 * k + 2] = x.z; qv[4 * k + 3] = x.w;
    }
  }
  // The walk: a level takes its quota of best nodes, then the next best while
  // the candidates hold fewer eligible keys than the budget.  The nodes are
  // ranked up to TOPCAP deep; a walk that needs more goes to the exact kernel.
  const int need = budget_at(A, t);
  const long long held_leaf = sup ? loose_leaf_eligible(V, t, A.window, A.sinks) : 0;
  int Rs = 0;                          // supers taken
  if (ok && sup && V.n_top > 0) {
    // third level: top nodes first; the supers ranked are the members of the
    // top nodes taken and the supers under no top node
    const int R2 = min(A.tree2_top, V.n_top);
    ok = R2 >= 1 && R2 <= TOPCAP;
    if (ok) {
      const int nr2 = min(V.n_top, TOPCAP);
      top_nodes_any(V.tcent, V.n_top, [](int c) { return c; }, qv, nr2, s_tmp, s_sup);
      __syncthreads();
      const long long held_top = held_leaf + loose_sup_eligible(V, t, A.window, A.sinks);
      const int R2w = block_walk(s_sup, nr2, V.n_top, R2, held_top, need,
                                 [&](int n) { return top_eligible(V, n, t, A.window, A.sinks, need); },
                                 L.ired, L.red);
      ok = R2w >= 0;
      if (ok) {
        if (wave == 0) node_prefix(V.tcnt, s_sup, R2w, s_pre);
        __syncthreads();
        const int nsel2 = s_pre[TOPCAP];
        const int ncs = nsel2 + (V.n_sup - V.covered_sup);
        ok = ncs <= SUPN;
        if (ok) {
          const int nrs = min(ncs, TOPCAP);
          top_nodes_any(V.scent, ncs, [&](int c) {
            return c < nsel2 ? nth_member(V.toff, V.tmem, s_sup, s_pre, R2w, c)
                             : V.covered_sup + (c - nsel2);
          }, qv, nrs, s_tmp, s_sup);
          __syncthreads();
          Rs = block_walk(s_sup, nrs, ncs, R, held_leaf, need,
                          [&](int sp) { return sup_eligible(V, sp, t, A.window, A.sinks); }, L.ired,
                          L.red);
          ok = Rs >= 0;
        }
      }
    }
  } else if (ok && sup) {
    const int nrs = min(V.n_sup, TOPCAP);
    top_nodes_any(V.scent, V.n_sup, [](int c) { return c; }, qv, nrs, s_tmp, s_sup);
    __syncthreads();
    Rs = block_walk(s_sup, nrs, V.n_sup, R, held_leaf, need,
                    [&](int sp) { return sup_eligible(V, sp, t, A.window, A.sinks); }, L.ired, L.red);
    ok = Rs >= 0;
  }
  if (ok && sup) {
    __syncthreads();
    if (wave == 0) node_prefix(V.scnt, s_sup, Rs, s_pre);   // leaves of the taken supers
    __syncthreads();
  }
  const bool supok = ok;               // uniform: the chosen supers are final
  const int nsel = ok && sup ? s_pre[TOPCAP] : 0;
  const int ncand = nsel + n_unc;
  // decode: one workgroup scores about 256 candidates per round of dependent
  // loads, the streaming pair every leaf at once over many workgroups; many
  // candidates that are also a large share of the leaves go to the latter
  const bool to_stream = supmask != nullptr && ncand > kTreeStreamMin && 8ll * ncand > V.n_bkt;
  ok = ok && ncand <= CPT * RT && !to_stream;

  long long K[CPT];
  int e[CPT], ks[CPT];
  long long lo = LLONG_MAX, hi = LLONG_MIN, tot = 0;
#pragma unroll
  for (int u = 0; u < CPT; ++u) { K[u] = LLONG_MIN; e[u] = 0; ks[u] = 0; }
  if (ok) {
    int leaf[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int f = tid + RT * u;
      leaf[u] = -1;
      if (f < nsel) {
        leaf[u] = nth_member(V.soff, V.smem, s_sup, s_pre, Rs, f);
      } else if (f < ncand) {
        leaf[u] = V.covered + (f - nsel);
      }
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      if (leaf[u] >= 0) K[u] = order_key(dot64(qv, V.cent + (int64_t)leaf[u] * kDim), leaf[u]);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      if (leaf[u] < 0) continue;
      const BucketInfo bi = load_bucket<false>(V, leaf[u]);
      int klo;
      e[u] = eligible<false>(V, leaf[u], bi, t, A.window, A.sinks, &klo);
      ks[u] = bi.off * V.pool + klo;
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const bool in = e[u] > 0;
      lo = min(lo, in ? K[u] : LLONG_MAX);
      hi = max(hi, in ? K[u] : LLONG_MIN);
      tot += in ? e[u] : 0;
    }
  }
  ok = select_and_emit<CPT>(L, V, A, q, t, ok, K, e, lo, hi, tot, true,
                            [&](int u) { return ks[u]; });
  const bool stream = supmask != nullptr && supok;   // uniform
  if (stream) {
    __shared__ unsigned s_mask[kSupMaskWords];
    __syncthreads();
    if (tid < kSupMaskWords) s_mask[tid] = 0u;
    __syncthreads();
    if (sup)
      for (int j = tid; j < Rs; j += RT) atomicOr(&s_mask[s_sup[j] >> 5], 1u << (s_sup[j] & 31));
    __syncthreads();
    if (tid < kSupMaskWords) supmask[(int64_t)q * kSupMaskWords + tid] = s_mask[tid];
  }
  if (tid == 0) flags[q] = ok ? 0 : (stream ? 2 : 1);
}

constexpr int kPrefW = 8, kPrefQ = 64;     // prefill scan: 8 waves (two per query group), 64 query slots
// dense comparator: 8 waves, one per 16-query group, each over every tile of a
// chunk (128 query slots; 58 against 64 ms for 64 slots at 10M, where the
// Flat scan is faster with 64)
constexpr int kDenseW = 8, kDenseQ = 128;

size_t ws_layout(size_t slots, size_t nq, ListWs* W, void* base) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += (bytes + 255) / 256 * 256; return r; };
  ListWs w;
  w.key = reinterpret_cast<long long*>(take(slots * LC * sizeof(long long)));
  w.elig = reinterpret_cast<int32_t*>(take(slots * LC * sizeof(int32_t)));
  w.kstart = reinterpret_cast<int32_t*>(take(slots * LC * sizeof(int32_t)));
  w.nlist = reinterpret_cast<int32_t*>(take(slots * sizeof(int32_t)));
  w.meta = reinterpret_cast<int32_t*>(take(slots * 3 * sizeof(int32_t)));
  w.flags = reinterpret_cast<int32_t*>(take(nq * sizeof(int32_t)));
  w.slo = nullptr;
  if (W) *W = w;
  return o;
}

// Dense comparator: [slots][kDenseList] order keys in kDenseSplit sub-lists,
// [slots][kDenseSplit] sub-list lengths, meta, thresholds, flags.
size_t dense_layout(size_t slots, size_t nq, ListWs* W, void* base) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += (bytes + 255) / 256 * 256; return r; };
  ListWs w;
  w.key = reinterpret_cast<long long*>(take(slots * kDenseList * sizeof(long long)));
  w.elig = nullptr;
  w.kstart = nullptr;
  w.nlist = reinterpret_cast<int32_t*>(take(slots * kDenseSplit * sizeof(int32_t)));
  w.meta = reinterpret_cast<int32_t*>(take(slots * 3 * sizeof(int32_t)));
  w.slo = reinterpret_cast<int32_t*>(take(slots * sizeof(int32_t)));
  w.flags = reinterpret_cast<int32_t*>(take(nq * sizeof(int32_t)));
  if (W) *W = w;
  return o;
}

}  // namespace

size_t select_fast_ws_bytes(int32_t nq) {
  const size_t slots = ((size_t)nq + kPrefQ - 1) / kPrefQ * kPrefQ;
  return ws_layout(slots, nq, nullptr, nullptr);
}

hipError_t launch_select_fast(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const size_t slots = ((size_t)a.nq + kPrefQ - 1) / kPrefQ * kPrefQ;
  ListWs W;
  ws_layout(slots, a.nq, &W, ws);
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  vs.v[0] = v;
  vs.nviews = 1;
  hipLaunchKernelGGL((k_scan<kPrefW, kPrefQ, false>), dim3((unsigned)(slots / kPrefQ)), dim3(kPrefW * 64),
                     0, s, vs, a, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_resolve, dim3((unsigned)slots), dim3(RT), 0, s, vs, a, W);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exact refinement for the (rare) flagged queries; other workgroups exit at once
  SelArgs b = a;
  b.only = W.flags;
  return launch_select(v, b, nullptr, s);
}

size_t dense_ws_bytes(int32_t nq) {
  const size_t slots = ((size_t)nq + kDenseQ - 1) / kDenseQ * kDenseQ;
  return dense_layout(slots, nq, nullptr, nullptr);
}

// The dense comparator: per query tile the sampled threshold, then the full
// pass split over key ranges, the exact top-budget per query, and the exact
// kernel for the (rare) flagged queries.
hipError_t launch_dense_select(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const size_t slots = ((size_t)a.nq + kDenseQ - 1) / kDenseQ * kDenseQ;
  const unsigned nqt = (unsigned)(slots / kDenseQ);
  ListWs W;
  dense_layout(slots, a.nq, &W, ws);
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  vs.v[0] = v;
  vs.nviews = 1;
  hipLaunchKernelGGL((k_scan<kDenseW, kDenseQ, true, 1>), dim3(nqt), dim3(kDenseW * 64), 0, s, vs, a, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_scan<kDenseW, kDenseQ, true, 2>), dim3(nqt * kDenseSplit), dim3(kDenseW * 64), 0, s, vs,
                     a, W);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dense_resolve, dim3((unsigned)slots), dim3(RTD), 0, s, a, W);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelArgs b = a;
  b.only = W.flags;
  return launch_select(v, b, nullptr, s);
}

size_t select_tree_ws_bytes(int32_t nq) { return ((size_t)nq * sizeof(int32_t) + 255) / 256 * 256; }

hipError_t launch_select_tree_multi(const IdxView* views, const int32_t* qpos, int32_t nseq,
                                   const SelArgs& a, int32_t* flags, uint32_t* supmask, hipStream_t s) {
  if (nseq <= 0) return hipSuccess;
  if (nseq > 16) return hipErrorInvalidValue;
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  for (int i = 0; i < nseq; ++i) {
    vs.v[i] = views[i];
    vs.qpos[i] = qpos[i];
  }
  vs.nviews = nseq;
  vs.view_per_query = 1;
  SelArgs b = a;
  b.nq = nseq;
  hipLaunchKernelGGL(k_tree_select, dim3((unsigned)nseq), dim3(RT), 0, s, vs, b, flags, supmask);
  return hipGetLastError();
}

hipError_t launch_select_tree(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  int32_t* flags = static_cast<int32_t*>(ws);
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  vs.v[0] = v;
  vs.nviews = 1;
  hipLaunchKernelGGL(k_tree_select, dim3((unsigned)a.nq), dim3(RT), 0, s, vs, a, flags,
                     (uint32_t*)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exact refinement for the flagged queries; other workgroups exit at once
  SelArgs b = a;
  b.only = flags;
  return launch_select(v, b, nullptr, s);
}

}  // namespace lsa
