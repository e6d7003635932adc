// Helpers shared by the selection kernels: order keys, bucket eligibility,
// key enumeration and a wave-level bitonic sort.
#pragma once

#include <climits>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {
namespace sel {

constexpr long long KOFF = 1ll << 21;
constexpr long long KMINP = (-(1ll << 20) + KOFF) << 32;
constexpr long long KMAXP = (((1ll << 20) + KOFF) << 32) | 0xffffffffll;

enum { ST_REFINE = 1, ST_DONE = 2 };


__device__ __forceinline__ long long order_key(int s, int beta) {
  return ((long long)(s + KOFF) << 32) | (long long)(0xffffffffu - (unsigned)beta);
}

// Number of keys of a bucket that are < x (members ascending, p keys each).
__device__ __forceinline__ int keys_below(const int32_t* __restrict__ mem, int cnt, int p, int x) {
  int lo = 0, hi = cnt;  // first member with m*p + p > x
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((long long)mem[mid] * p + p <= x) lo = mid + 1; else hi = mid;
  }
  int r = lo * p;
  if (lo < cnt) r += min(p, max(0, x - mem[lo] * p));
  return r;
}

struct BucketInfo {
  int first, last, cnt, off;
};

// Eligible long-range keys of a bucket for the query at t: keys j with
// sinks <= j <= t - window.  They form one run [klo, klo + e) of the
// bucket's ascending key list.
template <bool DENSE>
__device__ __forceinline__ int eligible(const IdxView& V, int beta, const BucketInfo& b, int t,
                                        int window, int sinks, int* klo) {
  const int hiK = t - window;
  *klo = 0;
  if (DENSE) return (beta >= sinks && beta <= hiK) ? 1 : 0;
  if (b.cnt <= 0) return 0;
  const int p = V.pool;
  const long long kf = (long long)b.first * p;
  const long long kl = (long long)b.last * p + p - 1;
  if (kf >= sinks && kl <= hiK) return b.cnt * p;
  if (kl < sinks || kf > hiK || hiK < sinks) return 0;
  const int32_t* m = V.bmem + b.off;
  const int a = keys_below(m, b.cnt, p, sinks);
  const int z = keys_below(m, b.cnt, p, hiK + 1);
  *klo = a;
  return z - a;
}

template <bool DENSE>
__device__ __forceinline__ BucketInfo load_bucket(const IdxView& V, int beta) {
  BucketInfo b;
  if (DENSE || beta >= V.n_bkt) { b.first = beta; b.last = beta; b.cnt = beta < V.n_bkt; b.off = beta; return b; }
  const int4 d = V.bdesc[beta];        // one 16-byte load: {first, last, count, offset}
  b.first = d.x;
  b.last = d.y;
  b.cnt = d.z;
  b.off = d.w;
  return b;
}

// Key at position k of a bucket's ascending key list.
template <bool DENSE>
__device__ __forceinline__ int bucket_key(const IdxView& V, int beta, const BucketInfo& b, int k) {
  if (DENSE) return beta;
  const int p = V.pool;
  return V.bmem[b.off + k / p] * p + k % p;
}

// ---- Tree walk ("Prefrontal's Latent Sparse Attention speeds up one
// attention layer 72x at 10M tokens", section "What it changes": a query
// walks the cluster hierarchy down; the walk keeps taking the next best node
// while the candidates hold fewer eligible keys than the query's budget,
// since a query reads a fixed number of keys, mauroscia.it D-LSA paragraph).

// Keys j in [a, b) with sinks <= j <= t - window.
__device__ __forceinline__ long long span_eligible(long long a, long long b, int t, int window,
                                                   int sinks) {
  const long long lo = a > sinks ? a : (long long)sinks;
  const long long hi = b - 1 < (long long)t - window ? b - 1 : (long long)t - window;
  return hi >= lo ? hi - lo + 1 : 0;
}

// Eligible keys at t under super cluster s: the blocks of its group that lie
// wholly inside [sinks, t - window] come from the key table, the (at most
// two) blocks that hold an end of that range are counted leaf by leaf.
__device__ __forceinline__ int sup_eligible(const IdxView& V, int s, int t, int window, int sinks) {
  const long long lo = sinks, hi = (long long)t - window;
  if (hi < lo) return 0;
  const int G = V.tgroup;
  const long long KB = V.blk_keys;
  const long long b0 = (long long)(s / V.tsuper) * G;
  const int32_t* sk = V.skey + (int64_t)s * (G + 1);
  const long long g_lo = b0 * KB, g_hi = (b0 + G) * KB - 1;
  if (g_hi < lo || g_lo > hi) return 0;
  if (g_lo >= lo && g_hi <= hi) return sk[G];
  long long f0 = (lo + KB - 1) / KB - b0, f1 = (hi + 1) / KB - b0;   // whole blocks [f0, f1)
  f0 = f0 < 0 ? 0 : f0;
  f1 = f1 > G ? G : f1;
  int e = f1 > f0 ? sk[f1] - sk[f0] : 0;
  const int32_t* sb = V.sblk + (int64_t)s * (G + 1);
  const int32_t* mem = V.smem + V.soff[s];
  const long long kl = lo / KB - b0, kh = hi / KB - b0;
  for (int i = 0; i < 2; ++i) {
    const long long k = i == 0 ? kl : kh;
    if ((i == 1 && kh == kl) || k < 0 || k >= G || (k >= f0 && k < f1)) continue;
    for (int j = sb[k]; j < sb[k + 1]; ++j) {
      const int leaf = mem[j];
      const BucketInfo bi = load_bucket<false>(V, leaf);
      int klo;
      e += eligible<false>(V, leaf, bi, t, window, sinks, &klo);
    }
  }
  return e;
}

// Eligible keys at t under top node n (third level): the sum over its
// supers, stopped once it reaches `cap`.  The walks only ask whether a prefix
// of these weights reaches the budget, so with cap = the budget a weight that
// is exact below it and at least the budget otherwise gives the same answers;
// a top node typically holds far more keys than the budget, and one or two of
// its supers settle it.
__device__ __forceinline__ int top_eligible(const IdxView& V, int n, int t, int window, int sinks, int cap) {
  const int32_t* m = V.tmem + V.toff[n];
  const int c = V.tcnt[n];
  int e = 0;
  for (int j = 0; j < c && e < cap; ++j) e += sup_eligible(V, m[j], t, window, sinks);
  return e;
}

// Eligible keys at t of the leaves outside the complete groups (always
// candidates): they cover keys [first key of the first uncovered block, n_pool * pool).
__device__ __forceinline__ long long loose_leaf_eligible(const IdxView& V, int t, int window,
                                                         int sinks) {
  return span_eligible((long long)(V.covered / V.bpb) * V.blk_keys, (long long)V.n_pool * V.pool, t,
                       window, sinks);
}

// Eligible keys at t under the supers outside the complete top groups (third
// level): the keys of groups covered_sup / S .. n_sup / S - 1.
__device__ __forceinline__ long long loose_sup_eligible(const IdxView& V, int t, int window,
                                                        int sinks) {
  const long long gk = (long long)V.tgroup * V.blk_keys;
  return span_eligible((long long)(V.covered_sup / V.tsuper) * gk, (long long)(V.n_sup / V.tsuper) * gk,
                       t, window, sinks);
}

// Bitonic sort (ascending) of n_pow2 int32 / int64 in LDS by one wave.
template <class T>
__device__ void wave_bitonic(T* a, int n) {
  const int lane = lane_id();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < n; i += 64) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const T x = a[i], y = a[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) { a[i] = y; a[ixj] = x; }
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  }
}


// Block-wide reductions and an exclusive scan over NT threads; `red` is LDS
// scratch of NT/64 entries.  Every thread of the block must call them.
template <int NT>
__device__ __forceinline__ long long block_sum_ll(long long x, long long* red) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  x = lane63(wave_incl_scan(x, 0ll, [](long long a, long long b) { return a + b; }));
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  long long s = 0;
  for (int w = 0; w < NT / 64; ++w) s += red[w];
  return s;
}

template <int NT>
__device__ __forceinline__ long long block_min_ll(long long x, long long* red) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  x = lane63(wave_incl_scan(x, LLONG_MAX, [](long long a, long long b) { return min(a, b); }));
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  long long s = LLONG_MAX;
  for (int w = 0; w < NT / 64; ++w) s = min(s, red[w]);
  return s;
}

template <int NT>
__device__ __forceinline__ long long block_max_ll(long long x, long long* red) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  x = lane63(wave_incl_scan(x, LLONG_MIN, [](long long a, long long b) { return max(a, b); }));
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  long long s = LLONG_MIN;
  for (int w = 0; w < NT / 64; ++w) s = max(s, red[w]);
  return s;
}

// Ascending bitonic sort of a block's N values, N / NT consecutive ones per
// thread (element tid*(N/NT) + i in v[i]): partners in the same thread swap
// in registers, in the same wave through shuffles, across waves through
// `tmp` (N values of LDS).
__device__ __forceinline__ int shfl_xor_t(int v, int m) { return __shfl_xor(v, m); }
__device__ __forceinline__ long long shfl_xor_t(long long v, int m) { return shfl_xor_i64(v, m); }
__device__ __forceinline__ unsigned shfl_xor_t(unsigned v, int m) { return (unsigned)__shfl_xor((int)v, m); }

template <int N, int NT, class T>
__device__ __forceinline__ void block_bitonic(T (&v)[N / NT], T* tmp) {
  constexpr int PT = N / NT;
  const int tid = threadIdx.x;
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      T pv[PT];
      if (j < PT) {
#pragma unroll
        for (int i = 0; i < PT; ++i) pv[i] = v[i ^ j];
      } else if (j < PT * 64) {
#pragma unroll
        for (int i = 0; i < PT; ++i) pv[i] = shfl_xor_t(v[i], j / PT);
      } else {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PT; ++i) tmp[tid * PT + i] = v[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PT; ++i) pv[i] = tmp[(tid * PT + i) ^ j];
      }
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int e = tid * PT + i;
        const bool up = (e & k) == 0, lower = (e & j) == 0;
        const T mn = min(v[i], pv[i]), mx = max(v[i], pv[i]);
        v[i] = (up == lower) ? mn : mx;
      }
    }
  }
}

// Exclusive prefix sum over the block in thread order; *total = block sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* red, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int wt;
  const int ex = wave_excl_scan(x, &wt);
  __syncthreads();
  if (lane == 0) red[wave] = wt;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < NT / 64; ++w) {
    const int v = red[w];
    before += w < wave ? v : 0;
    all += v;
  }
  *total = all;
  return before + ex;
}

// Writes one query's selection row: the taken buckets em[0..n) (bucket ids,
// any order; `pb` is the one cut bucket, taking `ptake` keys, or -1), bucket
// `top` first (the best-scoring taken one; -1: none) and the others in
// ascending id order, each with its eligible keys in ascending position,
// then the sinks not covered by the window, then the window, then -1
// padding.  The bucket-list paths write rows in this order.  `em` must have
// room for the next power of two >= n.  One wave.
template <bool DENSE>
__device__ void emit_row(const IdxView& V, int* em, int n, int pb, int ptake, int t, int window,
                         int sinks, int max_sel, int32_t* __restrict__ row, int32_t* cnt_out,
                         int top) {
  const int lane = lane_id();
  int np = 1;
  while (np < n) np <<= 1;
  for (int i = n + lane; i < np; i += 64) em[i] = INT_MAX;
  for (int i = lane; i < n; i += 64) em[i] = em[i] == top ? -1 : em[i];   // sorts first
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (n > 1) wave_bitonic(em, np);
  int out = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    int beta = -1, take = 0, klo = 0;
    BucketInfo bi = {0, 0, 0, 0};
    if (i < n) {
      beta = em[i] < 0 ? top : em[i];
      bi = load_bucket<DENSE>(V, beta);
      const int e = eligible<DENSE>(V, beta, bi, t, window, sinks, &klo);
      take = beta == pb ? ptake : e;
    }
    int tot;
    const int off = out + wave_excl_scan(take, &tot);
    const int nround = min(64, n - base);
    if (tot >= 16 * nround) {
      // large buckets: one bucket at a time, lanes over its keys
      for (int j = 0; j < nround; ++j) {
        const int bj = __shfl(beta, j), tj = __shfl(take, j), kj = __shfl(klo, j), oj = __shfl(off, j);
        BucketInfo b;
        b.first = __shfl(bi.first, j); b.last = __shfl(bi.last, j);
        b.cnt = __shfl(bi.cnt, j); b.off = __shfl(bi.off, j);
        for (int k = lane; k < tj; k += 64) row[oj + k] = bucket_key<DENSE>(V, bj, b, kj + k);
      }
    } else {
      // small buckets: each lane writes its own bucket, one member (p keys) per load
      const int p = DENSE ? 1 : V.pool;
      for (int k = 0; k < take;) {
        const int kk = klo + k;
        const int r0 = kk % p;
        const int g = DENSE ? beta : V.bmem[bi.off + kk / p];
        const int nh = min(p - r0, take - k);
        for (int r = 0; r < nh; ++r) row[off + k + r] = g * p + r0 + r;
        k += nh;
      }
    }
    out += tot;
  }
  const int wstart = max(0, t - window + 1);
  const int ns = max(0, min(sinks, wstart));
  const int nw = t - wstart + 1;
  for (int k = lane; k < ns; k += 64) row[out + k] = k;
  for (int k = lane; k < nw; k += 64) row[out + ns + k] = wstart + k;
  const int total = out + ns + nw;
  for (int k = total + lane; k < max_sel; k += 64) row[k] = -1;
  if (lane == 0) *cnt_out = total;
}

}  // namespace sel
}  // namespace lsa
