// Flat selection for large query batches (prefill): one full scan of the
// centroids per query group.
//
// Same result as the exact refinement kernel (lsa_select.hip) -- the pages'
// rule: buckets in (score desc, bucket asc) order, their eligible keys in
// ascending position until the long-range budget is met ("Latent Sparse
// Attention: un indice gerarchico per contesti lunghi", search and D-LSA
// configuration paragraphs) -- computed with fewer passes:
//   1. sampled pass: score max / mean of each query over a strided subset of
//      the buckets;
//   2. sampled pass: histogram of the sampled eligible key counts between
//      mean and max; the threshold slo is set where the sample predicts about
//      twice the budget above it;
//   3. full pass: every (query, bucket) with score >= slo and eligible keys is
//      appended to the query's list (global workspace);
//   4. per query: if the list holds at least `budget` eligible keys and fits
//      its capacity, it contains the cutoff: sort it by (score desc, bucket
//      asc), take buckets until the budget is met, emit.  Otherwise the query
//      is flagged and the exact refinement kernel recomputes it.
// A workgroup owns 64 queries (4 waves x 16 MFMA rows) and streams the
// centroids through LDS in 16 KB chunks, double-buffered, so each centroid
// byte is fetched once per 64 queries and all 256 lanes keep loads in flight.
#include <climits>
#include <cstring>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {
using namespace sel;

constexpr int FW = 4;               // waves
constexpr int FT = FW * 64;
constexpr int QW = 16;              // queries per wave (MFMA rows)
constexpr int QG = FW * QW;         // queries per workgroup
constexpr int CHT = 16;             // centroid tiles (16 buckets each) per staged chunk
constexpr int NB2 = 64;             // sample histogram bins
constexpr int LCAP = 4096;          // candidate list capacity per query (global)
constexpr int RB = 256;             // list histogram bins
constexpr int RCAP = 256;           // bracket entries resolved by sorting
constexpr int ECAP = 1024;          // taken buckets per query (else fallback)
constexpr int SAMPLE_CHUNKS = 64;

struct __attribute__((aligned(16))) FastLds {
  int t[QG];
  int smax[QG];
  int smean[QG];
  int slo[QG];
  int lcount[QG];
  int lkeys[QG];
  int hist[QG][NB2];
  union {
    v4i stage[2][CHT * 64];                                    // 32 KB
    struct {                                                   // per wave: 2 + 2 + 2 + 4 KB
      int hk[FW][RB];
      int hb[FW][RB];
      long long cand[FW][RCAP];
      int em[FW][ECAP];
    } r;
  } u;
};

// All threads of the workgroup: stream centroid chunks c0, c0+step, ... into
// LDS (double-buffered) and call f(tile, scores) for every tile of every
// chunk with this wave's 16 queries as the A operand.
template <class F>
__device__ __forceinline__ void scan_chunks(const IdxView& V, v4i (*stage)[CHT * 64], int c0,
                                            int step, int nchunks, const v4i& qa, F&& f) {
  const int tid = threadIdx.x, lane = lane_id();
  constexpr int PER = CHT * 64 / FT;          // 16-byte loads per thread per chunk
  v4i r[PER];
  auto gload = [&](int c) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = k * FT + tid;
      const int tile = c * CHT + e / 64, slot = e & 63;
      const int beta = tile * 16 + (slot & 15);
      r[k] = beta < V.n_bkt
                 ? *reinterpret_cast<const v4i*>(V.cent + (int64_t)beta * kDim + 16 * (slot >> 4))
                 : v4i{0, 0, 0, 0};
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER; ++k) stage[buf][k * FT + tid] = r[k];
  };
  if (c0 < nchunks) { gload(c0); swrite(0); }
  __syncthreads();
  int buf = 0;
  for (int c = c0; c < nchunks; c += step) {
    const int cn = c + step;
    if (cn < nchunks) gload(cn);
#pragma unroll 4
    for (int tl = 0; tl < CHT; ++tl) {
      const v4i b = stage[buf][tl * 64 + lane];
      const v4i z = {0, 0, 0, 0};
      f(c * CHT + tl, mfma_i8_16x16x64(qa, b, z));
    }
    if (cn < nchunks) swrite(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

__global__ void __launch_bounds__(FT) k_select_fast(IdxView V, SelArgs A, long long* __restrict__ lists,
                                                    int32_t* __restrict__ lelig,
                                                    int32_t* __restrict__ flags) {
  __shared__ FastLds S;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int g0 = blockIdx.x * QG;                  // first query of the workgroup
  const int wq0 = wave * QW;                       // this wave's first query slot
  const int qrow = wq0 + 4 * (lane >> 4);          // slot of score row v = 0
  const int B = A.budget;

  v4i qa = {0, 0, 0, 0};
  {
    const int q = g0 + wq0 + (lane & 15);
    if (q < A.nq) qa = *reinterpret_cast<const v4i*>(A.latq + (int64_t)q * kDim + 16 * (lane >> 4));
  }
  if (tid < QG) {
    const int q = g0 + tid;
    S.t[tid] = q < A.nq ? max(0, A.qpos ? A.qpos[q] : A.qpos_base + q) : -1;
    S.lcount[tid] = 0;
    S.lkeys[tid] = 0;
  }
  for (int e = tid; e < QG * NB2; e += FT) (&S.hist[0][0])[e] = 0;
  __syncthreads();

  const int ntiles = (V.n_bkt + 15) >> 4;
  const int nchunks = (ntiles + CHT - 1) / CHT;
  const int sstep = max(1, nchunks / SAMPLE_CHUNKS);
  int tq[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) tq[v] = S.t[qrow + v];

  // ---- 1. sampled max / mean ----
  {
    int smax[4], sn[4];
    long long ssum[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) { smax[v] = INT_MIN; sn[v] = 0; ssum[v] = 0; }
    scan_chunks(V, S.u.stage, 0, sstep, nchunks, qa, [&](int tile, const v4i& sc) {
      const int beta = tile * 16 + (lane & 15);
      if (beta >= V.n_bkt) return;
      const BucketInfo bi = load_bucket<false>(V, beta);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int klo;
        if (tq[v] < 0 || eligible<false>(V, beta, bi, tq[v], A.window, A.sinks, &klo) <= 0) continue;
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
      if ((lane & 15) == 0) {
        S.smax[qrow + v] = smax[v];
        S.smean[qrow + v] = sn[v] > 0 ? (int)(ssum[v] / sn[v]) : INT_MIN;
      }
    }
    __syncthreads();
  }

  // ---- 2. sampled histogram of eligible keys in [mean, max] ----
  {
    int lo[4], sh[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mx = S.smax[qrow + v], mn = S.smean[qrow + v];
      lo[v] = (mn == INT_MIN) ? INT_MAX : mn;
      const int range = mx - lo[v] + 1;
      int s = 0;
      while (s < 30 && ((range + (1 << s) - 1) >> s) > NB2) ++s;
      sh[v] = s;
    }
    int hi[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) hi[v] = S.smax[qrow + v];
    scan_chunks(V, S.u.stage, 0, sstep, nchunks, qa, [&](int tile, const v4i& sc) {
      const int beta = tile * 16 + (lane & 15);
      if (beta >= V.n_bkt) return;
      bool any = false;
#pragma unroll
      for (int v = 0; v < 4; ++v) any |= sc[v] >= lo[v];
      if (!any) return;
      const BucketInfo bi = load_bucket<false>(V, beta);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (sc[v] < lo[v] || sc[v] > hi[v]) continue;
        int klo;
        const int e = eligible<false>(V, beta, bi, tq[v], A.window, A.sinks, &klo);
        if (e > 0) atomicAdd(&S.hist[qrow + v][(hi[v] - sc[v]) >> sh[v]], e);
      }
    });
    // threshold: where the sample predicts ~2x the budget above it
    if (tid < QG && S.t[tid] >= 0) {
      const int mx = S.smax[tid], mn = S.smean[tid];
      int slo = INT_MIN;
      if (mn != INT_MIN) {
        int s = 0;
        const int range = mx - mn + 1;
        while (s < 30 && ((range + (1 << s) - 1) >> s) > NB2) ++s;
        const int sampled = (nchunks + sstep - 1) / sstep;
        const long long target = (2ll * B * sampled + nchunks - 1) / nchunks;
        long long cum = 0;
        slo = mn;
        for (int b = 0; b < NB2; ++b) {
          cum += S.hist[tid][b];
          if (cum >= target) { slo = max(mn, mx - ((b + 1) << s) + 1); break; }
        }
      }
      S.slo[tid] = slo;
    }
    __syncthreads();
  }

  // ---- 3. full pass: collect every bucket at or above the threshold ----
  {
    int slo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) slo[v] = tq[v] >= 0 ? S.slo[qrow + v] : INT_MAX;
    scan_chunks(V, S.u.stage, 0, 1, nchunks, qa, [&](int tile, const v4i& sc) {
      const int beta = tile * 16 + (lane & 15);
      if (beta >= V.n_bkt) return;
      bool any = false;
#pragma unroll
      for (int v = 0; v < 4; ++v) any |= sc[v] >= slo[v];
      if (!any) return;
      const BucketInfo bi = load_bucket<false>(V, beta);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (sc[v] < slo[v]) continue;
        int klo;
        const int e = eligible<false>(V, beta, bi, tq[v], A.window, A.sinks, &klo);
        if (e <= 0) continue;
        const int qs = qrow + v;
        const int pos = atomicAdd(&S.lcount[qs], 1);
        if (pos < LCAP) {
          lists[(int64_t)(g0 + qs) * LCAP + pos] = order_key(sc[v], beta);
          lelig[(int64_t)(g0 + qs) * LCAP + pos] = e;
        }
        atomicAdd(&S.lkeys[qs], e);
      }
    });
  }
  // (scan_chunks ends with a barrier; the staging buffers are free now)

  // ---- 4. resolve and emit, one wave per query ----
  // The list holds every bucket at or above the threshold with its eligible
  // key count; if those counts reach the budget the cutoff is in the list.
  // It is found by histogram refinement over the list's order keys (keys
  // above the bracket are taken whole), then the bracket (<= RCAP entries)
  // is sorted and taken in order, the last bucket cut.
  int* hk = S.u.r.hk[wave];
  int* hb = S.u.r.hb[wave];
  long long* cq = S.u.r.cand[wave];
  int* em = S.u.r.em[wave];
  for (int qs = wq0; qs < wq0 + QW; ++qs) {
    const int q = g0 + qs;
    if (q >= A.nq) break;
    const int t = S.t[qs];
    const int n = S.lcount[qs];
    const long long* lk = lists + (int64_t)q * LCAP;
    const int32_t* le = lelig + (int64_t)q * LCAP;
    bool ok = n <= LCAP && S.lkeys[qs] >= B && B > 0;
    if (ok) {
      // bracket = [min, max] of the list
      long long lo = LLONG_MAX, hi = LLONG_MIN;
      for (int i = lane; i < n; i += 64) { const long long K = lk[i]; lo = min(lo, K); hi = max(hi, K); }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        lo = min(lo, shfl_xor_i64(lo, m));
        hi = max(hi, shfl_xor_i64(hi, m));
      }
      int above = 0;            // keys taken whole (above the bracket)
      bool done = false;
      for (int pass = 0; pass < 8 && !done; ++pass) {
        const long long range = hi - lo + 1;
        int sh = 0;
        while (sh < 62 && ((range + (1ll << sh) - 1) >> sh) > RB) ++sh;
        for (int i = lane; i < RB; i += 64) { hk[i] = 0; hb[i] = 0; }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        int ab = 0;
        for (int i = lane; i < n; i += 64) {
          const long long K = lk[i];
          if (K > hi) { ab += le[i]; continue; }
          if (K < lo) continue;
          const int bin = (int)((hi - K) >> sh);
          atomicAdd(&hk[bin], le[i]);
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
        above = abt;
        // the list reaches the budget, so the cutoff bin exists
        int cum = above + ex, found = -1, fb = 0;
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
      int ntake = 0, pb = -1, ptake = 0, full = 0;
      if (ok) {
        // entries above the bracket are taken whole; the bracket is sorted
        int nc = 0;
        for (int base = 0; base < n; base += 64) {
          const int i = base + lane;
          const long long K = i < n ? lk[i] : LLONG_MIN;
          const bool tk = i < n && K > hi;
          const bool cd = i < n && K >= lo && K <= hi;
          const unsigned long long mt = __ballot(tk), mc = __ballot(cd);
          const unsigned long long below = (1ull << lane) - 1ull;
          if (tk) {
            const int slot = ntake + __popcll(mt & below);
            if (slot < ECAP) em[slot] = (int)(0xffffffffu - (unsigned)(K & 0xffffffffll));
          }
          if (cd) cq[nc + __popcll(mc & below)] = -K;
          ntake += __popcll(mt);
          nc += __popcll(mc);
          int e = tk ? le[i] : 0, et;
          wave_excl_scan(e, &et);
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
    }
    if (lane == 0) flags[q] = ok ? 0 : 1;
  }
}

}  // namespace

size_t select_fast_ws_bytes(int32_t nq) {
  const size_t nqp = ((size_t)nq + QG - 1) / QG * QG;
  return nqp * LCAP * (sizeof(long long) + sizeof(int32_t)) + (nqp * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_select_fast(const IdxView& v, const SelArgs& a, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const size_t nqp = ((size_t)a.nq + QG - 1) / QG * QG;
  long long* lists = static_cast<long long*>(ws);
  int32_t* lelig = reinterpret_cast<int32_t*>(lists + nqp * LCAP);
  int32_t* flags = lelig + nqp * LCAP;
  hipLaunchKernelGGL(k_select_fast, dim3((unsigned)(nqp / QG)), dim3(FT), 0, s, v, a, lists, lelig,
                     flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exact refinement for the (rare) flagged queries; other workgroups exit at once
  SelArgs b = a;
  b.only = flags;
  return launch_select(v, b, nullptr, s);
}

}  // namespace lsa
