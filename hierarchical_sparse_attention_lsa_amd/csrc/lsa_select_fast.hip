// Flat selection in one full scan of the centroids (prefill batches and
// decode steps).
//
// Same result as the exact refinement kernel (lsa_select.hip) -- the pages'
// rule: buckets in (score desc, bucket asc) order, their eligible keys in
// ascending position until the long-range budget is met ("Latent Sparse
// Attention: un indice gerarchico per contesti lunghi", search and D-LSA
// configuration paragraphs) -- computed with fewer passes:
//   1. sampled pass: score max / mean of each query over a strided subset of
//      the buckets;
//   2. sampled pass: histogram of the sampled buckets' key counts between
//      mean and max; the threshold slo is set where the sample predicts
//      about twice the budget above it;
//   3. full pass: every (query, bucket) with score >= slo is appended to the
//      query's list (global workspace, one sub-list per lane: no atomics);
//   4. per query: the list entries' eligible key counts are computed; if
//      they reach the budget (and nothing overflowed) the cutoff is in the
//      list and is found by histogram refinement over the list, the bracket
//      sorted, the buckets taken in order, the last one cut; otherwise the
//      query is flagged and the exact refinement kernel recomputes it.
// The workgroup streams the centroids (and bucket sizes) through LDS in
// double-buffered chunks, so every centroid byte is fetched once per
// workgroup while all lanes keep loads in flight, and the scans are pure
// MFMA + compare.  Prefill: 64 queries per workgroup (4 waves x 16 MFMA
// rows).  Decode: one sequence per workgroup (its own index), 8 waves
// splitting each chunk's tiles.
#include <climits>
#include <cstring>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {
using namespace sel;

constexpr int CHT = 16;             // centroid tiles (16 buckets each) per staged chunk
constexpr int NB2 = 64;             // sample histogram bins
constexpr int LCAP = 4096;          // candidate list capacity per query slot (global)
constexpr int RB = 256;             // list histogram bins
constexpr int RCAP = 256;           // bracket entries resolved by sorting
constexpr int ECAP = 1024;          // taken buckets per query (else fallback)
constexpr int SAMPLE_CHUNKS = 64;

struct FastViews {                  // first kernel argument (read through the kernarg pointer)
  IdxView v[16];
  int32_t qpos[16];
  int32_t nviews;
};

template <int FW, int QS>
struct Cfg {
  static constexpr int FT = FW * 64;
  static constexpr int NQW = QS / 16;        // query groups (16 MFMA rows each)
  static constexpr int PH = FW / NQW;        // waves sharing a query group (tile phases)
  static constexpr int NSUB = PH * 16;       // sub-lists per query
  static constexpr int SUBCAP = LCAP / NSUB;
  static_assert(FW % NQW == 0, "waves must cover the query groups");
};

template <int FW, int QS>
struct __attribute__((aligned(16))) FastLds {
  using C = Cfg<FW, QS>;
  int q[QS];                  // query index of each slot (-1: empty)
  int t[QS];
  int smax[QS];
  long long ssum[QS];
  int sn[QS];
  int slo[QS];
  int lsub[QS][C::NSUB];
  int hist[QS][NB2];
  union {
    struct { v4i cent[2][CHT * 64]; int cnt[2][CHT * 16]; } st;          // 32 + 2 KB
    struct { int hk[FW][RB]; int hb[FW][RB]; long long cand[FW][RCAP]; int em[FW][ECAP]; } r;
  } u;
};

// All threads: stream chunks c0, c0+step, ... (16 tiles of centroids and
// bucket sizes) into LDS, double-buffered; each wave then calls
// f(tile, scores, LDS bucket sizes of the tile) on its phase's tiles.
template <int FW, int QS, class F>
__device__ __forceinline__ void scan_chunks(const IdxView& V, FastLds<FW, QS>& S, int c0, int step,
                                            int nchunks, int phase, const v4i& qa, F&& f) {
  using C = Cfg<FW, QS>;
  const int tid = threadIdx.x, lane = lane_id();
  constexpr int PER = (CHT * 64 + C::FT - 1) / C::FT;
  v4i r[PER];
  int rc = 0;
  auto gload = [&](int c) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = k * C::FT + tid;
      const int tile = c * CHT + e / 64, slot = e & 63;
      const int beta = tile * 16 + (slot & 15);
      r[k] = (e < CHT * 64 && beta < V.n_bkt)
                 ? *reinterpret_cast<const v4i*>(V.cent + (int64_t)beta * kDim + 16 * (slot >> 4))
                 : v4i{0, 0, 0, 0};
    }
    const int bb = c * CHT * 16 + tid;
    rc = (tid < CHT * 16 && bb < V.n_bkt) ? V.bcnt[bb] : 0;
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (k * C::FT + tid < CHT * 64) S.u.st.cent[buf][k * C::FT + tid] = r[k];
    if (tid < CHT * 16) S.u.st.cnt[buf][tid] = rc;
  };
  if (c0 < nchunks) { gload(c0); swrite(0); }
  __syncthreads();
  int buf = 0;
  for (int c = c0; c < nchunks; c += step) {
    const int cn = c + step;
    if (cn < nchunks) gload(cn);
#pragma unroll 4
    for (int tl = phase; tl < CHT; tl += C::PH) {
      const v4i b = S.u.st.cent[buf][tl * 64 + lane];
      const v4i z = {0, 0, 0, 0};
      f(c * CHT + tl, mfma_i8_16x16x64(qa, b, z), &S.u.st.cnt[buf][tl * 16]);
    }
    if (cn < nchunks) swrite(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

// Prefill (nviews == 1): slot s of workgroup b is query b*QS + s.
// Decode (nviews > 1): workgroup b serves query b alone, on index b.
template <int FW, int QS>
__global__ void __launch_bounds__(FW * 64)
k_select_fast(FastViews VS, SelArgs A, long long* __restrict__ lists, int32_t* __restrict__ lelig,
              int32_t* __restrict__ flags) {
  using C = Cfg<FW, QS>;
  __shared__ FastLds<FW, QS> S;
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const bool multi = VS.nviews > 1;
  const IdxView V = vsp->v[multi ? blockIdx.x : 0];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t lbase = (int64_t)blockIdx.x * QS;  // list slots of this workgroup
  const int qgrp = wave % C::NQW;                  // this wave's 16-slot group
  const int phase = wave / C::NQW;                 // this wave's tile phase
  const int wq0 = qgrp * 16;
  const int qrow = wq0 + 4 * (lane >> 4);          // slot of score row v = 0
  const int sub = phase * 16 + (lane & 15);        // this lane's sub-list
  const int B = A.budget;
  const int p = V.pool;

  for (int i = tid; i < QS; i += C::FT) {
    int q = multi ? (i == 0 ? (int)blockIdx.x : -1) : (int)(lbase + i);
    if (q >= A.nq) q = -1;
    S.q[i] = q;
    S.t[i] = q < 0 ? -1 : max(0, multi ? vsp->qpos[blockIdx.x] : (A.qpos ? A.qpos[q] : A.qpos_base + q));
    S.smax[i] = INT_MIN; S.ssum[i] = 0; S.sn[i] = 0;
  }
  for (int e = tid; e < QS * NB2; e += C::FT) (&S.hist[0][0])[e] = 0;
  __syncthreads();

  v4i qa = {0, 0, 0, 0};
  {
    const int q = S.q[wq0 + (lane & 15)];
    if (q >= 0) qa = *reinterpret_cast<const v4i*>(A.latq + (int64_t)q * kDim + 16 * (lane >> 4));
  }
  const int ntiles = (V.n_bkt + 15) >> 4;
  const int nchunks = (ntiles + CHT - 1) / CHT;
  const int sstep = max(1, nchunks / SAMPLE_CHUNKS);
  bool act[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) act[v] = S.t[qrow + v] >= 0;

  // ---- 1. sampled max / mean (non-empty buckets; eligibility comes later) ----
  {
    int smax[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN}, sn[4] = {0, 0, 0, 0};
    long long ssum[4] = {0, 0, 0, 0};
    scan_chunks(V, S, 0, sstep, nchunks, phase, qa, [&](int tile, const v4i& sc, const int* cnt) {
      const int beta = tile * 16 + (lane & 15);
      if (beta >= V.n_bkt || cnt[lane & 15] <= 0) return;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        smax[v] = max(smax[v], sc[v]);
        ssum[v] += sc[v];
        sn[v] += 1;
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
      if ((lane & 15) == 0 && act[v]) {
        atomicMax(&S.smax[qrow + v], smax[v]);
        atomicAdd(&S.sn[qrow + v], sn[v]);
        atomicAdd((unsigned long long*)&S.ssum[qrow + v], (unsigned long long)ssum[v]);
      }
    }
    __syncthreads();
  }

  // ---- 2. sampled histogram of key counts in [mean, max] -> threshold ----
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
    scan_chunks(V, S, 0, sstep, nchunks, phase, qa, [&](int tile, const v4i& sc, const int* cnt) {
      const int beta = tile * 16 + (lane & 15);
      if (beta >= V.n_bkt) return;
      const int w = cnt[lane & 15] * p;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (sc[v] >= lo[v] && w > 0) atomicAdd(&S.hist[qrow + v][(hi[v] - sc[v]) >> sh[v]], w);
    });
    for (int qs = tid; qs < QS; qs += C::FT) {
      int slo = INT_MAX;
      if (S.t[qs] >= 0) {
        slo = INT_MIN;
        const int n = S.sn[qs];
        if (n > 0) {
          const int mx = S.smax[qs], mn = (int)(S.ssum[qs] / n);
          int s = 0;
          while (s < 30 && (((mx - mn + 1) + (1 << s) - 1) >> s) > NB2) ++s;
          const int sampled = (nchunks + sstep - 1) / sstep;
          const long long target = (2ll * B * sampled + nchunks - 1) / nchunks;
          long long cum = 0;
          slo = mn;
          for (int b = 0; b < NB2; ++b) {
            cum += S.hist[qs][b];
            if (cum >= target) { slo = max(mn, mx - ((b + 1) << s) + 1); break; }
          }
        }
      }
      S.slo[qs] = slo;
    }
    __syncthreads();
  }

  // ---- 3. full pass: every bucket at or above the threshold joins the list ----
  {
    int slo[4], nl[4] = {0, 0, 0, 0};
    long long* lp[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      slo[v] = act[v] ? S.slo[qrow + v] : INT_MAX;
      lp[v] = lists + (lbase + qrow + v) * LCAP + sub;
    }
    scan_chunks(V, S, 0, 1, nchunks, phase, qa, [&](int tile, const v4i& sc, const int* cnt) {
      const int beta = tile * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (sc[v] >= slo[v] && beta < V.n_bkt) {
          if (nl[v] < C::SUBCAP) lp[v][(int64_t)nl[v] * C::NSUB] = order_key(sc[v], beta);
          ++nl[v];
        }
      }
    });
#pragma unroll
    for (int v = 0; v < 4; ++v) S.lsub[qrow + v][sub] = act[v] ? nl[v] : 0;
    __syncthreads();
  }

  // ---- 4. per query (one wave each): eligibility, refinement, emit ----
  int* hk = S.u.r.hk[wave];
  int* hb = S.u.r.hb[wave];
  long long* cq = S.u.r.cand[wave];
  int* em = S.u.r.em[wave];
  for (int qs = wave; qs < QS; qs += FW) {
    const int q = S.q[qs];
    if (q < 0) continue;
    const int t = S.t[qs];
    long long* lk = lists + (lbase + qs) * LCAP;
    int32_t* le = lelig + (lbase + qs) * LCAP;
    const int* ls = S.lsub[qs];
    // sub-list sizes: entries are (k, sub) with k < size of sub, at k*NSUB + sub
    int kmax = 0, over = 0;
    for (int j = lane; j < C::NSUB; j += 64) {
      kmax = max(kmax, ls[j]);
      over |= ls[j] > C::SUBCAP;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      kmax = max(kmax, __shfl_xor(kmax, m));
      over |= __shfl_xor(over, m);
    }
    bool ok = B > 0 && !over;
    const int ngrid = kmax * C::NSUB;
    // eligible keys of every entry (stored next to it), list total and bracket
    long long lo = LLONG_MAX, hi = LLONG_MIN;
    if (ok) {
      int total = 0;
      for (int i = lane; i < ngrid; i += 64) {
        if (i / C::NSUB >= ls[i % C::NSUB]) continue;
        const long long K = lk[i];
        const int beta = (int)(0xffffffffu - (unsigned)(K & 0xffffffffll));
        const BucketInfo bi = load_bucket<false>(V, beta);
        int klo;
        const int e = eligible<false>(V, beta, bi, t, A.window, A.sinks, &klo);
        le[i] = e;
        total += e;
        if (e > 0) { lo = min(lo, K); hi = max(hi, K); }
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        lo = min(lo, shfl_xor_i64(lo, m));
        hi = max(hi, shfl_xor_i64(hi, m));
        total += __shfl_xor(total, m);
      }
      ok = total >= B;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    bool done = false;
    for (int pass = 0; ok && pass < 8 && !done; ++pass) {
      const long long range = hi - lo + 1;
      int sh = 0;
      while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
      for (int i = lane; i < RB; i += 64) { hk[i] = 0; hb[i] = 0; }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      int ab = 0;
      for (int i = lane; i < ngrid; i += 64) {
        if (i / C::NSUB >= ls[i % C::NSUB]) continue;
        const int e = le[i];
        if (e <= 0) continue;
        const long long K = lk[i];
        if (K > hi) { ab += e; continue; }
        if (K < lo) continue;
        const int bin = (int)((hi - K) >> sh);
        atomicAdd(&hk[bin], e);
        atomicAdd(&hb[bin], 1);
      }
      int abt;
      wave_excl_scan(ab, &abt);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      int h[RB / 64], c[RB / 64], loc = 0;
#pragma unroll
      for (int k = 0; k < RB / 64; ++k) { h[k] = hk[(RB / 64) * lane + k]; c[k] = hb[(RB / 64) * lane + k]; loc += h[k]; }
      int tot;
      const int ex = wave_excl_scan(loc, &tot);
      int cum = abt + ex, found = -1, fb = 0;
#pragma unroll
      for (int k = 0; k < RB / 64; ++k) {
        if (found < 0 && cum + h[k] >= B) { found = (RB / 64) * lane + k; fb = c[k]; }
        cum += h[k];
      }
      const unsigned long long mk = __ballot(found >= 0);
      if (!mk) { ok = false; break; }
      const int src = __ffsll((long long)mk) - 1;
      const int bin = __shfl(found, src);
      const int nb = __shfl(fb, src);
      const long long nhi = hi - ((long long)bin << sh);
      long long nlo = hi - ((long long)(bin + 1) << sh) + 1;
      if (nlo < lo) nlo = lo;
      lo = nlo; hi = nhi;
      done = nb <= RCAP;
    }
    ok = ok && done;
    if (ok) {
      // entries above the bracket are taken whole; the bracket is sorted
      int ntake = 0, nc = 0, full = 0, pb = -1, ptake = 0;
      for (int base = 0; base < ngrid; base += 64) {
        const int i = base + lane;
        const bool in = i < ngrid && i / C::NSUB < ls[i % C::NSUB];
        const long long K = in ? lk[i] : LLONG_MIN;
        const int e = in ? le[i] : 0;
        const bool tk = in && e > 0 && K > hi;
        const bool cd = in && e > 0 && K >= lo && K <= hi;
        const unsigned long long mt = __ballot(tk), mc = __ballot(cd);
        const unsigned long long below = (1ull << lane) - 1ull;
        if (tk) {
          const int slot = ntake + __popcll(mt & below);
          if (slot < ECAP) em[slot] = (int)(0xffffffffu - (unsigned)(K & 0xffffffffll));
        }
        if (cd) cq[nc + __popcll(mc & below)] = -K;
        ntake += __popcll(mt);
        nc += __popcll(mc);
        int et;
        wave_excl_scan(tk ? e : 0, &et);
        full += et;
      }
      ok = ntake <= ECAP;
      if (ok && nc > 0) {
        int np = 1;
        while (np < nc) np <<= 1;
        for (int i = nc + lane; i < np; i += 64) cq[i] = LLONG_MAX;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        wave_bitonic(cq, np);
        int need = B - full;
        for (int base = 0; base < nc && need > 0; base += 64) {
          const int i = base + lane;
          int e = 0, beta = -1, klo;
          if (i < nc) {
            beta = (int)(0xffffffffu - (unsigned)((-cq[i]) & 0xffffffffll));
            const BucketInfo bi = load_bucket<false>(V, beta);
            e = eligible<false>(V, beta, bi, t, A.window, A.sinks, &klo);
          }
          int tot;
          const int before = wave_excl_scan(e, &tot);
          const int take = min(e, max(0, need - before));
          const unsigned long long m2 = __ballot(take > 0);
          const int slot = ntake + __popcll(m2 & ((1ull << lane) - 1ull));
          if (take > 0 && slot < ECAP) em[slot] = beta;
          if (take > 0 && take < e) { pb = beta; ptake = take; }
          ntake += __popcll(m2);
          need -= tot;
        }
        const unsigned long long mp = __ballot(pb >= 0);
        if (mp) {
          const int src = __ffsll((long long)mp) - 1;
          pb = __shfl(pb, src);
          ptake = __shfl(ptake, src);
        }
        ok = ntake <= ECAP;
      }
      if (ok) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        emit_row<false>(V, em, ntake, pb, ptake, t, A.window, A.sinks, A.max_sel,
                        A.idx + (int64_t)q * A.max_sel, A.cnt + q);
      }
    }
    if (lane == 0) flags[q] = ok ? 0 : 1;
  }
}

constexpr int kPrefW = 4, kPrefQ = 64;     // prefill: 4 waves, 64 query slots
constexpr int kDecW = 8, kDecQ = 16;       // decode: 8 waves on one 16-slot group

size_t lists_bytes(size_t slots) { return slots * LCAP * (sizeof(long long) + sizeof(int32_t)); }

}  // namespace

size_t select_fast_ws_bytes(int32_t nq) {
  const size_t slots = ((size_t)nq + kPrefQ - 1) / kPrefQ * kPrefQ;
  return lists_bytes(slots) + ((size_t)nq * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_select_fast(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const size_t slots = ((size_t)a.nq + kPrefQ - 1) / kPrefQ * kPrefQ;
  long long* lists = static_cast<long long*>(ws);
  int32_t* lelig = reinterpret_cast<int32_t*>(lists + slots * LCAP);
  int32_t* flags = lelig + slots * LCAP;
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  vs.v[0] = v;
  vs.nviews = 1;
  hipLaunchKernelGGL((k_select_fast<kPrefW, kPrefQ>), dim3((unsigned)(slots / kPrefQ)),
                     dim3(kPrefW * 64), 0, s, vs, a, lists, lelig, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exact refinement for the (rare) flagged queries; other workgroups exit at once
  SelArgs b = a;
  b.only = flags;
  return launch_select(v, b, nullptr, s);
}

size_t select_decode_ws_bytes(int32_t nseq) {
  return lists_bytes((size_t)nseq * kDecQ) + ((size_t)nseq * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_select_decode(const IdxView* views, const int32_t* qpos, int32_t nseq,
                                const SelArgs& a, void* ws, hipStream_t s) {
  if (nseq <= 0) return hipSuccess;
  FastViews vs;
  memset(&vs, 0, sizeof vs);
  bool tree = false;
  for (int i = 0; i < nseq; ++i) {
    vs.v[i] = views[i];
    vs.qpos[i] = qpos[i];
    tree |= views[i].leafsup != nullptr;
  }
  vs.nviews = nseq;
  SelArgs b = a;
  b.nq = nseq;
  if (tree || nseq < 2) {
    // Tree indexes (candidate masks) and single sequences take the exact kernel
    return launch_select_multi(views, qpos, nseq, b, s);
  }
  const size_t slots = (size_t)nseq * kDecQ;
  long long* lists = static_cast<long long*>(ws);
  int32_t* lelig = reinterpret_cast<int32_t*>(lists + slots * LCAP);
  int32_t* flags = lelig + slots * LCAP;
  hipLaunchKernelGGL((k_select_fast<kDecW, kDecQ>), dim3((unsigned)nseq), dim3(kDecW * 64), 0, s,
                     vs, b, lists, lelig, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  b.only = flags;
  return launch_select_multi(views, qpos, nseq, b, s);
}

}  // namespace lsa
