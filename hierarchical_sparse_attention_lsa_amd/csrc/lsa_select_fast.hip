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
//      query's list -- 64 sub-lists per query, one per bucket id residue
//      mod 64, each filled in ascending id order by a single lane (no
//      atomics).
//   The centroids and bucket sizes stream through LDS in double-buffered
//   chunks (each centroid byte is read once per workgroup, all lanes keep
//   loads in flight) and the full pass is MFMA + compare + rare store.
// k_resolve (one wave per query; lane j owns sub-list j):
//   eligible key counts of the entries; if they reach the budget the cutoff
//   is in the list: histogram refinement finds a bracket of <= 256 entries,
//   entries above it are taken whole, the bracket is sorted and taken in
//   order with the last bucket cut; the taken buckets are sorted by id and
//   their keys written (ascending bucket ids keep each query's gather
//   walking the KV cache once from start to end).  A query whose list
//   overflowed or falls short of the budget is flagged and the exact
//   refinement kernel recomputes it.
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
constexpr int NSUB = 64;            // sub-lists per query (bucket id mod 64)
constexpr int LC = 8192;            // list entries per query slot (128 per sub-list)
constexpr int SUBCAP = LC / NSUB;
constexpr int RB = 256;             // list histogram bins
constexpr int RCAP = 256;           // bracket entries resolved by sorting
constexpr int ECAP = 1024;          // taken buckets per query (else the exact kernel)
constexpr int SAMPLE_CHUNKS = 64;

struct FastViews {                  // first kernel argument (read through the kernarg pointer)
  IdxView v[16];
  int32_t qpos[16];
  int32_t nviews;
  int32_t slots_per_view;           // decode: query slots per sequence
};

struct ListWs {
  long long* key;     // [slots][LC] order keys, sub-list j entry k at k*64 + j
  int32_t* elig;      // [slots][LC] eligible keys, then the taken keys
  int32_t* kstart;    // [slots][LC] member slot * p + offset of the first eligible key
  int32_t* nsub;      // [slots][64] sub-list sizes
  int32_t* meta;      // [slots][2]  query index (-1: empty slot), position
  int32_t* flags;     // [nq] 1: recompute with the exact kernel
};

template <int FW, int QS>
struct Cfg {
  static constexpr int FT = FW * 64;
  static constexpr int NQW = QS / 16;        // query groups (16 MFMA rows each)
  static constexpr int PH = FW / NQW;        // waves sharing a query group (tile phases)
  static_assert(FW % NQW == 0 && (PH == 1 || PH == 4), "unsupported scan shape");
};

template <int FW, int QS>
struct __attribute__((aligned(16))) ScanLds {
  int q[QS];
  int t[QS];
  int smax[QS];
  int sn[QS];
  int slo[QS];
  long long ssum[QS];
  int hist[QS][NB2];
  v4i cent[2][CHT * 64];
  int cnt[2][CHT * 16];
};

template <int FW, int QS, class F>
__device__ __forceinline__ void stream_chunks(const IdxView& V, ScanLds<FW, QS>& S, int c0,
                                              int step, int nchunks, F&& f) {
  using C = Cfg<FW, QS>;
  const int tid = threadIdx.x;
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
      if (k * C::FT + tid < CHT * 64) S.cent[buf][k * C::FT + tid] = r[k];
    if (tid < CHT * 16) S.cnt[buf][tid] = rc;
  };
  if (c0 < nchunks) { gload(c0); swrite(0); }
  __syncthreads();
  int buf = 0;
  for (int c = c0; c < nchunks; c += step) {
    const int cn = c + step;
    if (cn < nchunks) gload(cn);
    f(c, buf);
    if (cn < nchunks) swrite(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

// Prefill (nviews == 1): slot s of workgroup b is query b*QS + s.
// Decode (nviews > 1): workgroup b serves query b alone (slot 0), on index b.
template <int FW, int QS>
__global__ void __launch_bounds__(FW * 64) k_scan(FastViews VS, SelArgs A, ListWs W) {
  using C = Cfg<FW, QS>;
  __shared__ ScanLds<FW, QS> S;
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const bool multi = VS.nviews > 1;
  const IdxView V = vsp->v[multi ? blockIdx.x : 0];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t lbase = (int64_t)blockIdx.x * QS;
  const int qgrp = wave % C::NQW;
  const int phase = wave / C::NQW;
  const int qrow = qgrp * 16 + 4 * (lane >> 4);    // slot of score row v = 0
  const int col = lane & 15;
  const int B = A.budget;
  const int p = V.pool;

  for (int i = tid; i < QS; i += C::FT) {
    int q = multi ? (i == 0 ? (int)blockIdx.x : -1) : (int)(lbase + i);
    if (q >= A.nq) q = -1;
    const int t = q < 0 ? -1 : max(0, multi ? vsp->qpos[blockIdx.x] : (A.qpos ? A.qpos[q] : A.qpos_base + q));
    S.q[i] = q; S.t[i] = t;
    S.smax[i] = INT_MIN; S.ssum[i] = 0; S.sn[i] = 0;
    W.meta[2 * (lbase + i)] = q;
    W.meta[2 * (lbase + i) + 1] = t;
  }
  for (int e = tid; e < QS * NB2; e += C::FT) (&S.hist[0][0])[e] = 0;
  __syncthreads();

  v4i qa = {0, 0, 0, 0};
  {
    const int q = S.q[qgrp * 16 + col];
    if (q >= 0) qa = *reinterpret_cast<const v4i*>(A.latq + (int64_t)q * kDim + 16 * (lane >> 4));
  }
  const int ntiles = (V.n_bkt + 15) >> 4;
  const int nchunks = (ntiles + CHT - 1) / CHT;
  const int sstep = max(1, nchunks / SAMPLE_CHUNKS);
  bool act[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) act[v] = S.t[qrow + v] >= 0;

  // ---- 1. sampled max / mean over non-empty buckets ----
  {
    int smax[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN}, sn[4] = {0, 0, 0, 0};
    long long ssum[4] = {0, 0, 0, 0};
    stream_chunks(V, S, 0, sstep, nchunks, [&](int c, int buf) {
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

  // ---- 2. sampled key-count histogram in [mean, max] -> threshold ----
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
    stream_chunks(V, S, 0, sstep, nchunks, [&](int c, int buf) {
      for (int tl = phase; tl < CHT; tl += C::PH) {
        const v4i z = {0, 0, 0, 0};
        const v4i sc = mfma_i8_16x16x64(qa, S.cent[buf][tl * 64 + lane], z);
        const int w = S.cnt[buf][tl * 16 + col] * p;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (sc[v] >= lo[v] && w > 0) atomicAdd(&S.hist[qrow + v][(hi[v] - sc[v]) >> sh[v]], w);
      }
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

  // ---- 3. full pass: buckets at or above the threshold join the lists ----
  {
    // prefill: a lane sees tiles of every residue mod 4 (4 sub-lists per
    // query); decode: each wave's tiles share one residue (1 sub-list)
    constexpr int NSL = C::PH == 1 ? 4 : 1;
    int slo[4], nl[NSL][4];
    long long* lp[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      slo[v] = act[v] ? S.slo[qrow + v] : INT_MAX;
      lp[v] = W.key + (lbase + qrow + v) * LC + col;
#pragma unroll
      for (int u = 0; u < NSL; ++u) nl[u][v] = 0;
    }
    stream_chunks(V, S, 0, 1, nchunks, [&](int c, int buf) {
      constexpr int TPW = CHT / C::PH;              // tiles of this wave per chunk
#pragma unroll
      for (int g = 0; g < TPW; g += 4) {
        v4i sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const v4i z = {0, 0, 0, 0};
          sc[u] = mfma_i8_16x16x64(qa, S.cent[buf][(phase + (g + u) * C::PH) * 64 + lane], z);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int tile = c * CHT + phase + (g + u) * C::PH;
          const int beta = tile * 16 + col;
          const int su = NSL == 4 ? u : 0;
          const int sub = (tile & 3) * 16 + col;      // = beta mod 64
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (sc[u][v] >= slo[v] && beta < V.n_bkt) {
              if (nl[su][v] < SUBCAP)
                lp[v][(int64_t)nl[su][v] * NSUB + (sub - col)] = order_key(sc[u][v], beta);
              ++nl[su][v];
            }
          }
        }
      }
    });
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (!act[v]) continue;
#pragma unroll
      for (int u = 0; u < NSL; ++u) {
        const int sub = (NSL == 4 ? u : phase) * 16 + col;
        W.nsub[(lbase + qrow + v) * NSUB + sub] = nl[u][v];
      }
    }
  }
}

// One wave per query slot.
constexpr int RW = 4;               // waves per resolve workgroup

__global__ void __launch_bounds__(RW * 64) k_resolve(FastViews VS, SelArgs A, ListWs W,
                                                     int32_t nslots) {
  __shared__ int s_hk[RW][RB];
  __shared__ int s_hb[RW][RB];
  __shared__ long long s_cq[RW][RCAP];
  __shared__ int s_ci[RW][RCAP];
  __shared__ long long s_em[RW][ECAP];
  const FastViews* vsp = (const FastViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t slot = (int64_t)blockIdx.x * RW + wave;
  if (slot >= nslots) return;
  const int q = W.meta[2 * slot];
  if (q < 0) return;
  const int t = W.meta[2 * slot + 1];
  const IdxView V = vsp->v[VS.nviews > 1 ? (int)(slot / VS.slots_per_view) : 0];
  const int B = A.budget;
  const int p = V.pool;
  int* hk = s_hk[wave];
  int* hb = s_hb[wave];
  long long* cq = s_cq[wave];
  int* ci = s_ci[wave];
  long long* em = s_em[wave];
  long long* lk = W.key + slot * LC;
  int32_t* le = W.elig + slot * LC;
  int32_t* ls = W.kstart + slot * LC;

  // lane j owns sub-list j: entries k*64 + j, k < len
  const int len = W.nsub[slot * NSUB + lane];
  bool ok = B > 0 && __ballot(len > SUBCAP) == 0ull;
  int kmax = min(len, SUBCAP);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) kmax = max(kmax, __shfl_xor(kmax, m));
  const int mylen = min(len, SUBCAP);

  // eligible keys of each entry and where its first key sits
  long long lo = LLONG_MAX, hi = LLONG_MIN;
  int total = 0;
  if (ok) {
    for (int k0 = 0; k0 < kmax; k0 += 8) {
      long long K[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) K[u] = k0 + u < mylen ? lk[(k0 + u) * NSUB + lane] : LLONG_MIN;
      BucketInfo bi[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int beta = (int)(0xffffffffu - (unsigned)(K[u] & 0xffffffffll));
        bi[u] = K[u] != LLONG_MIN ? load_bucket<false>(V, beta) : BucketInfo{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (K[u] == LLONG_MIN) continue;
        int klo;
        const int e = eligible<false>(V, 0, bi[u], t, A.window, A.sinks, &klo);
        le[(k0 + u) * NSUB + lane] = e;
        ls[(k0 + u) * NSUB + lane] = bi[u].off * p + klo;
        total += e;
        if (e > 0) { lo = min(lo, K[u]); hi = max(hi, K[u]); }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      lo = min(lo, shfl_xor_i64(lo, m));
      hi = max(hi, shfl_xor_i64(hi, m));
      total += __shfl_xor(total, m);
    }
    ok = total >= B;
  }
  __threadfence_block();

  // histogram refinement over the list until the cutoff bracket is small
  bool done = false;
  for (int pass = 0; ok && pass < 8 && !done; ++pass) {
    const long long range = hi - lo + 1;
    int sh = 0;
    while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
    for (int i = lane; i < RB; i += 64) { hk[i] = 0; hb[i] = 0; }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int ab = 0;
    for (int k0 = 0; k0 < kmax; k0 += 4) {
      long long K[4];
      int e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = k0 + u < mylen;
        K[u] = in ? lk[(k0 + u) * NSUB + lane] : 0;
        e[u] = in ? le[(k0 + u) * NSUB + lane] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (e[u] <= 0) continue;
        if (K[u] > hi) { ab += e[u]; continue; }
        if (K[u] < lo) continue;
        const int bin = (int)((hi - K[u]) >> sh);
        atomicAdd(&hk[bin], e[u]);
        atomicAdd(&hb[bin], 1);
      }
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
    // takes: entries above the bracket whole, below nothing; the bracket's
    // entries collected for the ordered walk
    int nc = 0, full = 0;
    for (int k0 = 0; k0 < kmax; ++k0) {
      const bool in = k0 < mylen;
      const int i = k0 * NSUB + lane;
      const long long K = in ? lk[i] : 0;
      const int e = in ? le[i] : 0;
      const bool tk = e > 0 && K > hi;
      const bool cd = e > 0 && K >= lo && K <= hi;
      const unsigned long long mc = __ballot(cd);
      const int r = nc + __popcll(mc & ((1ull << lane) - 1ull));
      if (cd) { cq[r] = -K; ci[r] = i; }
      nc += __popcll(mc);
      if (in) le[i] = tk ? e : 0;
      full += tk ? e : 0;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) full += __shfl_xor(full, m);
    // bracket in (score desc, id asc) order; payload = list index
    int np = 1;
    while (np < nc) np <<= 1;
    for (int i = nc + lane; i < np; i += 64) { cq[i] = LLONG_MAX; ci[i] = -1; }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int k = 2; k <= np; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = lane; i < np; i += 64) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const long long x = cq[i], y = cq[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { cq[i] = y; cq[ixj] = x; const int tmp = ci[i]; ci[i] = ci[ixj]; ci[ixj] = tmp; }
          }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
    }
    __threadfence_block();
    int need = B - full;
    for (int base = 0; base < nc; base += 64) {
      const int i = base + lane;
      int e = 0, li = -1;
      if (i < nc) {
        li = ci[i];
        const long long K = -cq[i];
        const int beta = (int)(0xffffffffu - (unsigned)(K & 0xffffffffll));
        const BucketInfo bi = load_bucket<false>(V, beta);
        int klo;
        e = eligible<false>(V, 0, bi, t, A.window, A.sinks, &klo);
      }
      int tot;
      const int before = wave_excl_scan(e, &tot);
      const int take = min(e, max(0, need - before));
      if (li >= 0) le[li] = take;
      need -= tot;
    }
    __threadfence_block();

    // taken buckets sorted by id (key: id << 32 | list index), keys written in order
    int ntake = 0;
    for (int k0 = 0; k0 < kmax; ++k0) {
      const int i = k0 * NSUB + lane;
      const int take = k0 < mylen ? le[i] : 0;
      const unsigned long long mt = __ballot(take > 0);
      if (take > 0) {
        const int r = ntake + __popcll(mt & ((1ull << lane) - 1ull));
        if (r < ECAP) {
          const long long K = lk[i];
          em[r] = ((long long)(0xffffffffu - (unsigned)(K & 0xffffffffll)) << 32) | (long long)i;
        }
      }
      ntake += __popcll(mt);
    }
    ok = ntake <= ECAP;
  }
  if (ok) {
    int ntake = 0;
    for (int k0 = 0; k0 < kmax; ++k0) ntake += __popcll(__ballot(k0 < mylen && le[k0 * NSUB + lane] > 0));
    int np = 1;
    while (np < ntake) np <<= 1;
    for (int i = ntake + lane; i < np; i += 64) em[i] = LLONG_MAX;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (ntake > 1) wave_bitonic(em, np);
    int32_t* row = A.idx + (int64_t)q * A.max_sel;
    int out_total = 0;
    for (int base = 0; base < ntake; base += 64) {
      const int j = base + lane;
      int take = 0, ks = 0;
      if (j < ntake) {
        const int i = (int)(em[j] & 0xffffffffll);
        take = le[i];
        ks = ls[i];
      }
      int tot;
      const int off = out_total + wave_excl_scan(take, &tot);
      const int nround = min(64, ntake - base);
      if (tot >= 16 * nround) {
        for (int jj = 0; jj < nround; ++jj) {
          const int tj = __shfl(take, jj), kj = __shfl(ks, jj), oj = __shfl(off, jj);
          for (int k = lane; k < tj; k += 64) {
            const int sl = kj + k;
            row[oj + k] = V.bmem[sl / p] * p + sl % p;
          }
        }
      } else {
        for (int k = 0; k < take;) {
          const int sl = ks + k;
          const int r0 = sl % p;
          const int g = V.bmem[sl / p];
          const int nh = min(p - r0, take - k);
          for (int r = 0; r < nh; ++r) row[off + k + r] = g * p + r0 + r;
          k += nh;
        }
      }
      out_total += tot;
    }
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
  if (lane == 0) W.flags[q] = ok ? 0 : 1;
}

constexpr int kPrefW = 4, kPrefQ = 64;     // prefill scan: 4 waves, 64 query slots

size_t ws_layout(size_t slots, size_t nq, ListWs* W, void* base) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += (bytes + 255) / 256 * 256; return r; };
  ListWs w;
  w.key = reinterpret_cast<long long*>(take(slots * LC * sizeof(long long)));
  w.elig = reinterpret_cast<int32_t*>(take(slots * LC * sizeof(int32_t)));
  w.kstart = reinterpret_cast<int32_t*>(take(slots * LC * sizeof(int32_t)));
  w.nsub = reinterpret_cast<int32_t*>(take(slots * NSUB * sizeof(int32_t)));
  w.meta = reinterpret_cast<int32_t*>(take(slots * 2 * sizeof(int32_t)));
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
  vs.slots_per_view = (int32_t)slots;
  hipLaunchKernelGGL((k_scan<kPrefW, kPrefQ>), dim3((unsigned)(slots / kPrefQ)), dim3(kPrefW * 64),
                     0, s, vs, a, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_resolve, dim3((unsigned)((slots + RW - 1) / RW)), dim3(RW * 64), 0, s, vs, a,
                     W, (int32_t)slots);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exact refinement for the (rare) flagged queries; other workgroups exit at once
  SelArgs b = a;
  b.only = W.flags;
  return launch_select(v, b, nullptr, s);
}

}  // namespace lsa
