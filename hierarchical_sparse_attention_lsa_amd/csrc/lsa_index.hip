// Index build kernels: pooling, per-block integer k-means with member lists,
// tail singleton buckets.
//
// Follows "Latent Sparse Attention: un indice gerarchico per contesti lunghi"
// (mauroscia.it), paragraph on the index: small groups of consecutive keys
// are pooled, the pooled sequence is cut into blocks, the vectors of a block
// are grouped by similarity into buckets, and each bucket keeps a centroid
// and the indices of its original keys.  The same k-means kernel builds the
// upper level of the hierarchy ("Prefrontal's Latent Sparse Attention speeds
// up one attention layer 72x at 10M tokens", section "What it changes") by
// clustering the leaf centroids of a group of blocks.
#include <climits>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

// ---------------------------------------------------------------- pooling
// Pooled vector g = round-half-even mean of rows g*p .. g*p+p-1 of the
// virtual sequence (pend[0..n_pend) ++ src[0..n_src)).  One thread per
// (pooled vector, 16 dims): 16-byte loads, four threads per 64-byte row.
__device__ __forceinline__ int sbyte(int w, int j) { return (w << (24 - 8 * j)) >> 24; }

__global__ void __launch_bounds__(256) k_pool(const int8_t* __restrict__ pend, int n_pend,
                                              const int8_t* __restrict__ src, int p,
                                              int8_t* __restrict__ out, int64_t n_groups) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t g = t >> 2;
  const int c = (int)(t & 3) * 16;
  if (g >= n_groups) return;
  int acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0;
  for (int r = 0; r < p; ++r) {
    const int64_t row = g * p + r;
    const int8_t* rp = row < n_pend ? pend + row * kDim : src + (row - n_pend) * kDim;
    const int4 v = *reinterpret_cast<const int4*>(rp + c);
    const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[4 * k + j] += sbyte(w[k], j);
  }
  int o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unsigned x = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) x |= ((unsigned)rhe_div(acc[4 * k + j], p) & 0xffu) << (8 * j);
    o[k] = (int)x;
  }
  *reinterpret_cast<int4*>(out + g * kDim + c) = make_int4(o[0], o[1], o[2], o[3]);
}

// Copy the last `keep` rows of (pend ++ src) into dst.
__global__ void k_save_pending(const int8_t* __restrict__ pend, int n_pend,
                               const int8_t* __restrict__ src, int64_t n_src, int keep,
                               int8_t* __restrict__ dst) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= keep * kDim) return;
  const int r = t / kDim, c = t % kDim;
  const int64_t row = (int64_t)n_pend + n_src - keep + r;
  dst[t] = row < n_pend ? pend[row * kDim + c] : src[(row - n_pend) * kDim + c];
}

// ---------------------------------------------------------------- tail
// Pooled vectors g0 .. g1-1 of the partial tail block become singleton
// buckets with id n_full*C + (g - n_full*N).
__global__ void k_tail(const int8_t* __restrict__ pooled, int64_t g0, int64_t g1, int64_t n_full,
                       int N, int C, int8_t* __restrict__ cent, int32_t* __restrict__ bcnt,
                       int32_t* __restrict__ boff, int32_t* __restrict__ bmem,
                       int32_t* __restrict__ bfirst, int32_t* __restrict__ blast) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t g = g0 + (t >> 2);
  if (g >= g1) return;
  const int part = (int)(t & 3);
  const int64_t beta = n_full * C + (g - n_full * N);
  reinterpret_cast<int4*>(cent + beta * kDim)[part] =
      reinterpret_cast<const int4*>(pooled + g * kDim)[part];
  if (part == 0) {
    bcnt[beta] = 1;
    boff[beta] = (int32_t)g;
    bmem[g] = (int32_t)g;
    bfirst[beta] = (int32_t)g;
    blast[beta] = (int32_t)g;
  }
}

// ---------------------------------------------------------------- k-means
// One workgroup clusters one block of N vectors (int8 [N][64]) into C
// centroids with `iters` Lloyd iterations:
//   init     mu_c = X[c * (N / C)]
//   assign   a_i = argmin_c |X_i - mu_c|^2 (lowest c on ties), evaluated as
//            |mu_c|^2 - 2 X_i . mu_c with int8 MFMA (exact int32)
//   update   mu_c = round-half-even(sum of members / count) when non-empty
// then writes a stable member list (members of each cluster in ascending
// row order), counts, offsets, first/last member and the centroids.
constexpr int kKmWaves = 16;
constexpr int kKmThreads = kKmWaves * 64;

__host__ __device__ inline size_t kmeans_lds_bytes(int N, int C) {
  size_t b = 0;
  b += (size_t)C * kDim;                 // mu int8
  b += (size_t)C * 4;                    // argmin key bias per centroid
  b += (size_t)C * kDim * 4;             // sums (reused for first/last rows)
  b += (size_t)C * 4;                    // counts
  b += (size_t)C * 4;                    // exclusive offsets
  b += (size_t)kKmWaves * C * 4;         // per-wave counts / cursors
  b += ((size_t)N * 2 + 15) / 16 * 16;   // assignments (uint16)
  return b;
}

// Argmin key of a (row x, centroid c) pair, larger = nearer:
//   256 * (2 x.mu_c - |mu_c|^2) + (255 - c)
// orders by |x - mu_c|^2 - |x|^2 = |mu_c|^2 - 2 x.mu_c ascending, then by c
// ascending (C <= 256).  |x.mu_c| <= 64 * 128 * 128 = 2^20 and |mu_c|^2 <=
// 2^20, so the key lies in (-2^30, 2^30).  km_bias(c) = 255 - c - 256 |mu_c|^2
// is kept per centroid, and a key is one shift-add of the MFMA dot product.
__device__ __forceinline__ int km_bias(const int8_t* m, int c) {
  const int4* m4 = reinterpret_cast<const int4*>(m);
  int sq = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int4 v = m4[k];
    sq = __builtin_amdgcn_sdot4(v.x, v.x, sq, false);
    sq = __builtin_amdgcn_sdot4(v.y, v.y, sq, false);
    sq = __builtin_amdgcn_sdot4(v.z, v.z, sq, false);
    sq = __builtin_amdgcn_sdot4(v.w, v.w, sq, false);
  }
  return 255 - c - 256 * sq;
}
__device__ __forceinline__ int km_key(int dot, int bias) { return (int)((unsigned)dot << 9) + bias; }

// Nearest centroid (lowest index on ties) of the 16 rows of one tile: lane l
// supplies the MFMA operand of row l % 16, bytes 16 * (l / 16) ..; every
// lane of the 16-lane group g receives the clusters of rows 4g .. 4g + 3.
__device__ __forceinline__ void km_nearest(v4i a, const int8_t* mu, const int* bias, int C, int cl[4]) {
  const int lane = lane_id();
  const int8_t* mp = mu + (lane & 15) * kDim + 16 * (lane >> 4);
  const int* bp = bias + (lane & 15);
  const v4i z = {0, 0, 0, 0};
  int best[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  const int nct = C >> 4;
  int ct = 0;
  for (; ct + 3 < nct; ct += 4) {
    v4i bq[4], d[4];
    int k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bq[u] = *reinterpret_cast<const v4i*>(mp + (ct + u) * 16 * kDim);
      k[u] = bp[(ct + u) * 16];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] = mfma_i8_16x16x64(a, bq[u], z);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      best[v] = max(best[v], max(km_key(d[0][v], k[0]), km_key(d[1][v], k[1])));
      best[v] = max(best[v], max(km_key(d[2][v], k[2]), km_key(d[3][v], k[3])));
    }
  }
  for (; ct < nct; ++ct) {
    const v4i b0 = *reinterpret_cast<const v4i*>(mp + ct * 16 * kDim);
    const int k0 = bp[ct * 16];
    const v4i d0 = mfma_i8_16x16x64(a, b0, z);
#pragma unroll
    for (int v = 0; v < 4; ++v) best[v] = max(best[v], km_key(d0[v], k0));
  }
  // lane l holds centroid l % 16 of its group's rows: maximum over the 16
  // lanes (quad swaps, then half-row and row mirrors)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    int x = best[v];
    x = max(x, dpp_move<0xB1, 0xf>(INT_MIN, x));
    x = max(x, dpp_move<0x4E, 0xf>(INT_MIN, x));
    x = max(x, dpp_move<0x141, 0xf>(INT_MIN, x));
    x = max(x, dpp_move<0x140, 0xf>(INT_MIN, x));
    cl[v] = 255 - (x & 255);
  }
}

// Cluster of the row whose operand this lane holds (row l % 16), from the
// km_nearest results: that row's cluster sits in lanes 16 * (row / 4) ..,
// value row % 4.
__device__ __forceinline__ int km_row_cluster(const int cl[4]) {
  const int lane = lane_id(), r = lane & 15;
  // cl[lane % 4] as bit selects (a select over the array by a run-time index
  // would be placed in scratch memory)
  const int m0 = -(lane & 1), m1 = -((lane >> 1) & 1);
  const int c0 = cl[0], c1 = cl[1], c2 = cl[2], c3 = cl[3];
  const int x01 = c0 ^ ((c0 ^ c1) & m0), x23 = c2 ^ ((c2 ^ c3) & m0);
  const int sel = x01 ^ ((x01 ^ x23) & m1);
  return __shfl(sel, 16 * (r >> 2) + (r & 3));
}

// Cluster sums laid out [dim][cluster], the cluster index of dims 16g ..
// 16g + 15 XOR-ed with 8g (within what C allows): the lanes of one LDS
// atomic add to one dim of each group's rows, so the four groups adding to
// the same cluster land on different banks.
__device__ __forceinline__ int km_sum_at(int d, int c, int C) {
  const int xm = (C & 31) ? 8 : 24;
  return d * C + (c ^ (((d >> 4) << 3) & xm));
}

// The tile's 16 rows join their clusters' sums and counts, from the operand
// bytes this lane holds (row l % 16, dims 16 * (l / 16) ..).
__device__ __forceinline__ void km_accumulate(v4i a, int cr, int C, int* sums, int* counts) {
  const int lane = lane_id(), g = lane >> 4;
  if (lane < 16) atomicAdd(&counts[cr], 1);
  int* sd = sums + km_sum_at(16 * g, cr, C);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int w4 = a[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) atomicAdd(&sd[(4 * k + j) * C], (w4 << (24 - 8 * j)) >> 24);
  }
}

// Round-half-even of s / n for |s| <= 128 n (a mean of int8 values), n > 0,
// with rn ~ 1/n: |s/n| <= 128, so the float quotient is within 2^-14 of the
// exact one and its floor within one of the exact floor; the remainder
// corrects it.
__device__ __forceinline__ int rhe_div_small(int s, int n, float rn) {
  int q = (int)floorf((float)s * rn);
  int r = s - q * n;
  if (r < 0) { q -= 1; r += n; } else if (r >= n) { q += 1; r -= n; }
  const int twice = 2 * r;
  return q + ((twice > n) | ((twice == n) & (q & 1)));
}

// mu_in / asg_in (members mode, iters = 0): the final centroids and
// assignments come from the multi-workgroup iterations; only the member lists
// and bucket records are built here.
__global__ void __launch_bounds__(kKmThreads)
k_kmeans(const int8_t* __restrict__ X_all, int N, int C, int iters, int64_t row0,
         int8_t* __restrict__ cent_all, int32_t* __restrict__ cnt_all,
         int32_t* __restrict__ off_all, int32_t* __restrict__ mem_all,
         int32_t* __restrict__ first_all, int32_t* __restrict__ last_all,
         int32_t* __restrict__ map_all, int32_t map_base, const int8_t* __restrict__ mu_in,
         const uint16_t* __restrict__ asg_in) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int8_t* mu = reinterpret_cast<int8_t*>(smem);
  int32_t* bias = reinterpret_cast<int32_t*>(mu + (size_t)C * kDim);
  int32_t* sums = bias + C;
  int32_t* counts = sums + C * kDim;
  int32_t* offs = counts + C;
  int32_t* cw = offs + C;
  uint16_t* assign = reinterpret_cast<uint16_t*>(cw + kKmWaves * C);

  const int blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int8_t* X = X_all + (int64_t)blk * N * kDim;
  const int stride = N / C;

  // init at strided members (members mode: the final centroids and assignments)
  for (int e = tid; e < C * 4; e += kKmThreads) {
    const int c = e >> 2, part = e & 3;
    const int8_t* src = mu_in ? mu_in + ((int64_t)blk * C + c) * kDim : X + (int64_t)c * stride * kDim;
    reinterpret_cast<int4*>(mu + c * kDim)[part] = reinterpret_cast<const int4*>(src)[part];
  }
  for (int e = tid; e < C; e += kKmThreads) counts[e] = 0;
  if (iters > 0)
    for (int e = tid; e < C * kDim; e += kKmThreads) sums[e] = 0;
  __syncthreads();
  if (asg_in) {
    for (int i = tid; i < N; i += kKmThreads) {
      const uint16_t c = asg_in[(int64_t)blk * N + i];
      assign[i] = c;
      atomicAdd(&counts[c], 1);
    }
  }
  for (int c = tid; c < C; c += kKmThreads) bias[c] = km_bias(mu + c * kDim, c);
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    // ---- assign (16-row tiles, all C centroids per tile), each row added to
    // its cluster's sums from the MFMA operand the lane already holds ----
    const int ntile = N >> 4;
    const int8_t* xl = X + (int64_t)(lane & 15) * kDim + 16 * (lane >> 4);
    v4i a_next = wave < ntile ? *reinterpret_cast<const v4i*>(xl + (int64_t)wave * 16 * kDim) : v4i{0, 0, 0, 0};
    for (int rt = wave; rt < ntile; rt += kKmWaves) {
      const v4i a = a_next;
      if (rt + kKmWaves < ntile) a_next = *reinterpret_cast<const v4i*>(xl + (int64_t)(rt + kKmWaves) * 16 * kDim);
      int cl[4];
      km_nearest(a, mu, bias, C, cl);
      const int cr = km_row_cluster(cl);
      if (lane < 16) assign[rt * 16 + lane] = (uint16_t)cr;
      km_accumulate(a, cr, C, sums, counts);
    }
    __syncthreads();
    // ---- update: one task per (cluster, 16 dims); the four tasks of a
    // cluster are the lanes of one quad.  Sums are cleared as they are read;
    // the last iteration's counts stay for the member lists. ----
    for (int task = tid; task < C * 4; task += kKmThreads) {
      const int c = task >> 2, ch = task & 3;
      const int n = counts[c];
      int4* mp = reinterpret_cast<int4*>(mu + c * kDim + 16 * ch);
      int4 m = *mp;
      if (n > 0) {
        const float rn = __builtin_amdgcn_rcpf((float)n);
        int w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          unsigned x = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            int* sp = sums + km_sum_at(16 * ch + 4 * k + j, c, C);
            x |= ((unsigned)rhe_div_small(*sp, n, rn) & 0xffu) << (8 * j);
            *sp = 0;
          }
          w[k] = (int)x;
        }
        m = make_int4(w[0], w[1], w[2], w[3]);
        *mp = m;
      }
      int sq = 0;
      sq = __builtin_amdgcn_sdot4(m.x, m.x, sq, false);
      sq = __builtin_amdgcn_sdot4(m.y, m.y, sq, false);
      sq = __builtin_amdgcn_sdot4(m.z, m.z, sq, false);
      sq = __builtin_amdgcn_sdot4(m.w, m.w, sq, false);
      sq += dpp_move<0xB1, 0xf>(0, sq);
      sq += dpp_move<0x4E, 0xf>(0, sq);
      if (ch == 0) {
        bias[c] = 255 - c - 256 * sq;
        if (it + 1 < iters) counts[c] = 0;
      }
    }
    __syncthreads();
  }

  // ---- stable member lists (counting sort by cluster, rows ascending) ----
  // rows per wave: contiguous ranges so that wave order = row order
  const int per_wave = (N + kKmWaves - 1) / kKmWaves;
  const int r_begin = wave * per_wave;
  const int r_end = min(N, r_begin + per_wave);
  int32_t* firstrow = sums;
  int32_t* lastrow = sums + C;
  for (int e = tid; e < kKmWaves * C; e += kKmThreads) cw[e] = 0;
  for (int e = tid; e < C; e += kKmThreads) { firstrow[e] = INT_MAX; lastrow[e] = -1; }
  __syncthreads();
  for (int r = r_begin + lane; r < r_end; r += 64) atomicAdd(&cw[wave * C + assign[r]], 1);
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const int x = c < C ? counts[c] : 0;
      int tot;
      const int ex = wave_excl_scan(x, &tot);
      if (c < C) offs[c] = carry + ex;
      carry += tot;
    }
  }
  __syncthreads();
  for (int c = tid; c < C; c += kKmThreads) {
    int run = offs[c];
    for (int w = 0; w < kKmWaves; ++w) {
      const int x = cw[w * C + c];
      cw[w * C + c] = run;
      run += x;
    }
  }
  __syncthreads();
  const int64_t gbase = row0 + (int64_t)blk * N;
  for (int r0 = r_begin; r0 < r_end; r0 += 64) {
    const int r = r0 + lane;
    const bool valid = r < r_end;
    const int c = valid ? (int)assign[r] : 0;
    unsigned long long mask = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (c >> bit) & 1;
      const unsigned long long bb = __ballot(on);
      mask &= on ? bb : ~bb;
    }
    if (valid) {
      const unsigned long long below = mask & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      const int pos = cw[wave * C + c] + rank;
      mem_all[(int64_t)blk * N + pos] = (int32_t)(gbase + r);
      if (map_all) map_all[gbase + r] = map_base + blk * C + c;
      atomicMin(&firstrow[c], r);
      atomicMax(&lastrow[c], r);
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (mask & ((1ull << lane) - 1ull)) == 0ull) cw[wave * C + c] += __popcll(mask);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int c = tid; c < C; c += kKmThreads) {
    const int64_t b = (int64_t)blk * C + c;
    cnt_all[b] = counts[c];
    off_all[b] = (int32_t)(gbase + offs[c]);   // slot in the member array
    if (first_all) {
      first_all[b] = counts[c] > 0 ? (int32_t)(gbase + firstrow[c]) : INT_MAX;
      last_all[b] = counts[c] > 0 ? (int32_t)(gbase + lastrow[c]) : -1;
    }
  }
  for (int e = tid; e < C * 4; e += kKmThreads) {
    const int c = e >> 2, part = e & 3;
    reinterpret_cast<int4*>(cent_all + ((int64_t)blk * C + c) * kDim)[part] =
        reinterpret_cast<const int4*>(mu + c * kDim)[part];
  }
}

// ---------------------------------------------------------------- few-block k-means
// When only a few blocks complete (a prefill chunk, a decode step, a Tree
// group), one workgroup per block would leave the GPU idle, so each block's
// points are split over W workgroups.  Per iteration: k_km_assign (centroids
// of the iteration, MFMA distances, argmin with lowest-index ties, per-
// workgroup integer sums and counts of its points) then k_km_reduce (sums
// over the W parts, round-half-even means, empty clusters keep their
// centroid); the member lists come from k_kmeans in members mode.  Integer
// sums are order-free, so the result equals the one-workgroup kernel's.
constexpr int kKmW = 16;            // most workgroups per block
constexpr int kKmAT = 256;          // threads of k_km_assign

struct KmScratch {
  int32_t* part;                    // [nblk][W][C][65]: 64 dim sums + count
  int8_t* cent;                     // [nblk][C][64]: centroids of the last reduce
  uint16_t* asg;                    // [nblk][N]: last assignment
};

size_t km_layout(int N, int C, int nblk, KmScratch* S, void* base) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += (bytes + 255) / 256 * 256; return r; };
  KmScratch k;
  k.part = reinterpret_cast<int32_t*>(take((size_t)nblk * kKmW * C * 65 * 4));
  k.cent = reinterpret_cast<int8_t*>(take((size_t)nblk * C * kDim));
  k.asg = reinterpret_cast<uint16_t*>(take((size_t)nblk * N * 2));
  if (S) *S = k;
  return o;
}

int km_parts(int N) {               // W: N must split into 16-row tiles
  int w = kKmW;
  while (w > 1 && N % (16 * w)) w >>= 1;
  return w;
}

__global__ void __launch_bounds__(kKmAT) k_km_assign(const int8_t* __restrict__ X_all, int N, int C,
                                                     int W, int it, KmScratch S) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int8_t* mu = reinterpret_cast<int8_t*>(smem);
  int32_t* bias = reinterpret_cast<int32_t*>(mu + (size_t)C * kDim);
  int32_t* sums = bias + C;
  int32_t* cnts = sums + C * kDim;
  const int b = blockIdx.x / W, w = blockIdx.x % W;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int8_t* X = X_all + (int64_t)b * N * kDim;
  const int stride = N / C;
  for (int e = tid; e < C * 4; e += kKmAT) {
    const int c = e >> 2, part = e & 3;
    const int8_t* src = it == 0 ? X + (int64_t)c * stride * kDim : S.cent + ((int64_t)b * C + c) * kDim;
    reinterpret_cast<int4*>(mu + c * kDim)[part] = reinterpret_cast<const int4*>(src)[part];
  }
  for (int e = tid; e < C * kDim; e += kKmAT) sums[e] = 0;
  for (int e = tid; e < C; e += kKmAT) cnts[e] = 0;
  __syncthreads();
  for (int c = tid; c < C; c += kKmAT) bias[c] = km_bias(mu + c * kDim, c);
  __syncthreads();
  const int rows = N / W;
  const int r0 = w * rows;
  for (int rt = wave; rt < rows / 16; rt += kKmAT / 64) {
    const int row = r0 + rt * 16;
    const v4i a = *reinterpret_cast<const v4i*>(X + (int64_t)(row + (lane & 15)) * kDim + 16 * (lane >> 4));
    int cl[4];
    km_nearest(a, mu, bias, C, cl);
    const int cr = km_row_cluster(cl);
    if (lane < 16) S.asg[(int64_t)b * N + row + lane] = (uint16_t)cr;
    km_accumulate(a, cr, C, sums, cnts);
  }
  __syncthreads();
  int32_t* part = S.part + ((int64_t)b * W + w) * C * 65;
  for (int e = tid; e < C * 65; e += kKmAT) {
    const int c = e / 65, d = e % 65;
    part[e] = d < kDim ? sums[km_sum_at(d, c, C)] : cnts[c];
  }
}

// One thread per (block, cluster, dimension).
__global__ void __launch_bounds__(256) k_km_reduce(const int8_t* __restrict__ X_all, int N, int C,
                                                   int W, int it, int nblk, KmScratch S) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)nblk * C * kDim) return;
  const int b = (int)(e / (C * kDim));
  const int c = (int)((e / kDim) % C);
  const int d = (int)(e % kDim);
  const int32_t* part = S.part + (int64_t)b * W * C * 65 + c * 65;
  int sum = 0, n = 0;
  for (int w = 0; w < W; ++w) {
    sum += part[(int64_t)w * C * 65 + d];
    n += part[(int64_t)w * C * 65 + kDim];
  }
  int8_t* dst = S.cent + ((int64_t)b * C + c) * kDim + d;
  const int8_t prev = it == 0 ? X_all[((int64_t)b * N + (int64_t)c * (N / C)) * kDim + d] : *dst;
  *dst = n > 0 ? (int8_t)rhe_div(sum, n) : prev;
}

size_t kmeans_mw_lds(int C) { return (size_t)C * kDim + (size_t)C * 4 + (size_t)C * kDim * 4 + (size_t)C * 4; }

// ---------------------------------------------------------------- decode append
// One new key per sequence (workgroup i = sequence i, thread = dimension).
// The key joins its sequence's pending partial group; when the group
// completes it is pooled into a new tail singleton bucket.  Sequences whose
// append completes a block are handled by the general path instead.
__global__ void __launch_bounds__(64) k_decode_append(DecodeAppendArgs a, const int8_t* __restrict__ src) {
  const int i = blockIdx.x, d = threadIdx.x;
  if (!a.batched[i]) return;
  char* base = a.arena[i];
  int8_t* pend = reinterpret_cast<int8_t*>(base + a.off_pend) + (int64_t)a.pend_slot[i] * a.p * kDim;
  const int8_t val = src[(int64_t)i * kDim + d];
  const int np = a.n_pend[i];
  if (np + 1 < a.p) {
    pend[np * kDim + d] = val;
    return;
  }
  int sum = val;
  for (int r = 0; r < np; ++r) sum += pend[r * kDim + d];
  const int64_t g = a.n_pool[i];
  const int8_t pv = (int8_t)rhe_div(sum, a.p);
  reinterpret_cast<int8_t*>(base + a.off_pooled)[g * kDim + d] = pv;
  const int64_t nf = a.n_full[i];
  const int64_t beta = nf * a.C + (g - nf * a.N);
  reinterpret_cast<int8_t*>(base + a.off_cent)[beta * kDim + d] = pv;
  if (d == 0) {
    reinterpret_cast<int32_t*>(base + a.off_bcnt)[beta] = 1;
    reinterpret_cast<int32_t*>(base + a.off_boff)[beta] = (int32_t)g;
    reinterpret_cast<int32_t*>(base + a.off_bmem)[g] = (int32_t)g;
    reinterpret_cast<int32_t*>(base + a.off_bfirst)[beta] = (int32_t)g;
    reinterpret_cast<int32_t*>(base + a.off_blast)[beta] = (int32_t)g;
    reinterpret_cast<int4*>(base + a.off_bdesc)[beta] = make_int4((int)g, (int)g, 1, (int)g);
  }
}

// ---------------------------------------------------------------- packed descriptors
__global__ void k_pack_desc(const int32_t* __restrict__ bfirst, const int32_t* __restrict__ blast,
                            const int32_t* __restrict__ bcnt, const int32_t* __restrict__ boff,
                            int64_t b0, int64_t b1, int4* __restrict__ bdesc) {
  const int64_t b = b0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b < b1) bdesc[b] = make_int4(bfirst[b], blast[b], bcnt[b], boff[b]);
}

hipError_t launch_pack_desc(const int32_t* bfirst, const int32_t* blast, const int32_t* bcnt,
                            const int32_t* boff, int64_t b0, int64_t b1, int4* bdesc, hipStream_t s) {
  if (b1 <= b0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_desc, dim3((unsigned)((b1 - b0 + 255) / 256)), dim3(256), 0, s, bfirst, blast,
                     bcnt, boff, b0, b1, bdesc);
  return hipGetLastError();
}

// ---------------------------------------------------------------- Tree walk tables
// For super s (group g = s / S, leaves of blocks g*G .. g*G + G - 1, leaf id
// b*C + c for block b): sblk[s][k] = first slot of s's ascending member list
// whose leaf lies in block g*G + k or later (sblk[s][G] = member count), and
// skey[s][k] = keys of s's leaves in the group's blocks before k.  One wave
// per super, lanes over k.
__global__ void __launch_bounds__(64) k_sup_tables(const int32_t* __restrict__ soff,
                                                   const int32_t* __restrict__ scnt,
                                                   const int32_t* __restrict__ smem,
                                                   const int32_t* __restrict__ bcnt, int s0, int S,
                                                   int G, int C, int p, int32_t* __restrict__ sblk,
                                                   int32_t* __restrict__ skey) {
  const int s = s0 + blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* mem = smem + soff[s];
  const int n = scnt[s];
  const int leaf0 = (s / S) * G * C;
  int32_t* sb = sblk + (int64_t)s * (G + 1);
  int32_t* sk = skey + (int64_t)s * (G + 1);
  auto first_slot = [&](int k) {       // first member with leaf id >= leaf0 + k*C
    int lo = 0, hi = n;
    const int x = leaf0 + k * C;
    while (lo < hi) {
      const int m = (lo + hi) >> 1;
      if (mem[m] < x) lo = m + 1; else hi = m;
    }
    return lo;
  };
  int carry = 0;
  for (int k0 = 0; k0 <= G; k0 += 64) {
    const int k = k0 + lane;
    int a = 0, keys = 0;
    if (k <= G) {
      a = first_slot(k);
      if (k < G) {
        const int z = first_slot(k + 1);
        for (int j = a; j < z; ++j) keys += bcnt[mem[j]] * p;
      }
    }
    int tot;
    const int ex = wave_excl_scan(keys, &tot);
    if (k <= G) {
      sb[k] = a;
      sk[k] = carry + ex;
    }
    carry += tot;
  }
}

hipError_t launch_sup_tables(const int32_t* soff, const int32_t* scnt, const int32_t* smem,
                             const int32_t* bcnt, int32_t s0, int32_t nsup, int32_t S, int32_t G,
                             int32_t C, int32_t p, int32_t* sblk, int32_t* skey, hipStream_t s) {
  if (nsup <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sup_tables, dim3((unsigned)nsup), dim3(64), 0, s, soff, scnt, smem, bcnt, s0,
                     S, G, C, p, sblk, skey);
  return hipGetLastError();
}

hipError_t launch_decode_append(const DecodeAppendArgs& a, const int8_t* src, int nseq,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_decode_append, dim3(nseq), dim3(64), 0, s, a, src);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
hipError_t launch_pool(const int8_t* pend, int32_t n_pend, const int8_t* src, int64_t n_src,
                       int32_t p, int8_t* pooled_out, int64_t n_groups, hipStream_t s) {
  (void)n_src;
  if (n_groups <= 0) return hipSuccess;
  const int64_t threads = n_groups * 4;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(k_pool, dim3(grid), dim3(256), 0, s, pend, n_pend, src, p, pooled_out,
                     n_groups);
  return hipGetLastError();
}

hipError_t launch_save_pending(const int8_t* pend, int32_t n_pend, const int8_t* src,
                               int64_t n_src, int32_t keep, int8_t* dst, hipStream_t s) {
  if (keep <= 0) return hipSuccess;
  const int threads = keep * kDim;
  hipLaunchKernelGGL(k_save_pending, dim3((threads + 255) / 256), dim3(256), 0, s, pend, n_pend,
                     src, n_src, keep, dst);
  return hipGetLastError();
}

hipError_t launch_tail(const int8_t* pooled, int64_t g0, int64_t g1, int64_t n_full, int32_t N,
                       int32_t C, int8_t* cent, int32_t* bcnt, int32_t* boff, int32_t* bmem,
                       int32_t* bfirst, int32_t* blast, hipStream_t s) {
  if (g1 <= g0) return hipSuccess;
  const int64_t threads = (g1 - g0) * 4;
  hipLaunchKernelGGL(k_tail, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, pooled,
                     g0, g1, n_full, N, C, cent, bcnt, boff, bmem, bfirst, blast);
  return hipGetLastError();
}

size_t kmeans_scratch_bytes(int32_t N, int32_t C) {
  return km_layout(N, C, kKmMaxBlk, nullptr, nullptr);
}

hipError_t launch_kmeans(const int8_t* X, int32_t N, int32_t C, int32_t iters, int32_t nblk,
                         int64_t row0, int8_t* cent_out, int32_t* cnt_out, int32_t* off_out,
                         int32_t* mem_out, int32_t* first_out, int32_t* last_out,
                         int32_t* map_out, int32_t map_base, void* scratch,
                         size_t scratch_bytes, hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t ae = once_per_device(attr_done, []() {
    hipError_t e = hipFuncSetAttribute((const void*)k_kmeans,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)k_km_assign, hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024);
  });
  if (ae != hipSuccess) return ae;
  const size_t lds = kmeans_lds_bytes(N, C);
  const int W = km_parts(N);
  // few blocks: W workgroups per block, one launch pair per iteration
  if (scratch && nblk <= kKmMaxBlk && W > 1 && nblk * W <= 256 && iters > 0 &&
      scratch_bytes >= km_layout(N, C, nblk, nullptr, nullptr)) {
    KmScratch S;
    km_layout(N, C, nblk, &S, scratch);
    const size_t alds = kmeans_mw_lds(C);
    const unsigned rgrid = (unsigned)(((int64_t)nblk * C * kDim + 255) / 256);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(k_km_assign, dim3((unsigned)(nblk * W)), dim3(kKmAT), alds, s, X, N, C, W,
                         it, S);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_km_reduce, dim3(rgrid), dim3(256), 0, s, X, N, C, W, it, nblk, S);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_kmeans, dim3(nblk), dim3(kKmThreads), lds, s, X, N, C, 0, row0, cent_out,
                       cnt_out, off_out, mem_out, first_out, last_out, map_out, map_base,
                       (const int8_t*)S.cent, (const uint16_t*)S.asg);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_kmeans, dim3(nblk), dim3(kKmThreads), lds, s, X, N, C, iters, row0,
                     cent_out, cnt_out, off_out, mem_out, first_out, last_out, map_out, map_base,
                     (const int8_t*)nullptr, (const uint16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace lsa
