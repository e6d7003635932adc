// Backward of the sparse attention over stored selections.
//
// "Latent Sparse Attention: un indice gerarchico per contesti lunghi"
// (mauroscia.it), N-LSA paragraph: native training keeps the indices of the
// selected keys for the backward pass.  The selection itself is discrete;
// gradients reach Q, K and V through the softmax attention over each query's
// selected rows.  With s = scale * k . q, P = exp(s - lse), the forward's
// output O and the upstream gradient dO, per (query, head):
//   dsum = sum_d dO[d] O[d]          dS = P (dO . v - dsum)
//   dQ   = scale * sum_j dS_j k_j    dK_j += scale * dS_j q    dV_j += P_j dO
//
// Design (gfx950).
// * dQ is query-centric, like the forward: a wave owns 16/G consecutive
//   queries of one KV head (16 MFMA columns = (query, head) pairs), walks each
//   query's long-range rows, then the union of the group's sinks and windows
//   once.  K and V rows go straight from HBM into the A operands of
//   S^T = K q and dP^T = V dO; K is also staged key-major through LDS for
//   dQ += dS K.  The forward's log-sum-exp makes P direct (no online max).
// * dK / dV are key-centric, so every key's gradient is summed by one
//   workgroup in a fixed order (deterministic, no atomics on the outputs).
//   A workgroup owns 64 keys of one KV head and walks the queries that
//   selected them in groups of 16/G, with Q and dO staged in LDS:
//     - band: 64 consecutive keys and the queries whose windows reach them;
//       it stores every key row, so it runs first;
//     - long range: the keys of one bucket (a taken bucket brings all its
//       eligible keys, the last one a prefix of them), and the queries that
//       took the bucket, each with the largest key it took;
//     - sinks: the sink keys outside the window, for a chunk of queries,
//       into partial sums that a last pass adds in chunk order.
//   The (bucket -> queries) lists come from the rows: a run of consecutive
//   long-range entries in one bucket is one taken bucket, and its last entry
//   is the largest key taken.  A counting sort over (bucket, query tile)
//   orders every list by query.
#include <algorithm>
#include <climits>
#include <cstring>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {

constexpr int BW = 8;            // waves per dQ workgroup
constexpr int BT = BW * 64;
constexpr int KT = 16;           // keys per dQ tile
constexpr int KW = 4;            // waves per key-tile workgroup
constexpr int KTT = KW * 16;     // keys per key tile
constexpr int QT = 64;           // queries per inversion tile
constexpr int SINK_QC = 2048;    // queries per sink partial sum
constexpr float kLog2e = 1.4426950408889634f;

enum { M_BAND = 0, M_LR = 1, M_SINK = 2 };

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;
  int32_t o_f32;
  const uint16_t* dout;
  const float* lse;
  int64_t kv_rows;
  const int32_t* idx;
  const int32_t* cnt;
  int32_t max_sel, nq;
  int32_t qpos0;
  int32_t window, sinks;
  int32_t Hq, Hkv, G, qpw;
  float scale, scale_log2;
  float* dq;
  float* dk;
  float* dv;
  float* dsum;              // [nq][Hq]
  // long-range inversion
  const int32_t* bcnt;
  const int32_t* boff;
  const int32_t* bmem;
  int32_t n_bkt, pool, n_pool;
  int32_t* map;             // [n_pool] pooled id -> bucket
  int32_t* tcnt;            // [n_bkt][n_tiles] runs per (bucket, query tile), then offsets
  int32_t* btot;            // [n_bkt] queries per bucket
  int32_t* ntl;             // [n_bkt] key tiles per bucket (0 if nobody took it)
  int32_t* bstart;          // [n_bkt + 1] first list entry of bucket b
  int32_t* ktile0;          // [n_bkt + 1] first key tile of bucket b
  int2* list;               // (query, largest key taken)
  int64_t list_cap;
  int32_t n_tiles;
  float* sink_part;         // [n_sink_chunks][Hkv][KTT][D] dK, then the same for dV
  int32_t n_sink_chunks;
  // grouped dQ: query order and unions of each group of gqpw slots
  const int32_t* perm;
  const int32_t* urow;
  const uint8_t* umask;
  const int32_t* ucnt;
  int32_t ucap, gqpw;
};

__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  const int per = nwg >> 3, rem = nwg & 7, x = b & 7, k = b >> 3;
  return x * per + min(x, rem) + k;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bf16 hi + lo split of x (the pair carries x to about 2^-16 relative)
__device__ __forceinline__ void split_bf16(float x, short& hi, short& lo) {
  const uint32_t hb = f32_to_bf16_bits(x);
  hi = (short)hb;
  lo = (short)f32_to_bf16_bits(x - bf16_bits_to_f32(hb));
}

// sum over 8 bf16 (packed in v4i) times 8 floats
__device__ __forceinline__ float dot8_bf16(v4i a, const float (&b)[8]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += bf16_bits_to_f32((uint32_t)a[i] & 0xffffu) * b[2 * i];
    s += bf16_bits_to_f32((uint32_t)a[i] >> 16) * b[2 * i + 1];
  }
  return s;
}

// eight consecutive elements of the forward output as float
__device__ __forceinline__ void load_o8(const BwdArgs& a, int64_t e, float (&o)[8]) {
  if (a.o_f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.o) + e);
    const float4 x = p[0], y = p[1];
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
  } else {
    const v4i r = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(a.o) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16_bits_to_f32((uint32_t)r[i] & 0xffffu);
      o[2 * i + 1] = bf16_bits_to_f32((uint32_t)r[i] >> 16);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one 16-key tile.  Lane l loads K and V row `r` (key slot l % 16) into
// the A operands; bit v of vmask says whether key 4*(l/16)+v of the tile
// counts for column l % 16, whose lse (log2 domain) and dsum the lane holds.
template <int D>
__device__ __forceinline__ void dq_tile(const v8bf (&qb)[D / 32], const v8bf (&db)[D / 32],
                                        const uint16_t* kbase, const uint16_t* vbase,
                                        int64_t rowstride, int r, unsigned vmask, float sl2,
                                        float lse2, float dsum, char* kl, v4f (&acc)[D / 16]) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int KROW = D * 2 + 16;
  const int lane = lane_id();
  const int hl = lane & 15, grp = lane >> 4;
  v8bf ka[NKK], va[NKK];
  const uint16_t* kp = kbase + (int64_t)r * rowstride + 8 * grp;
  const uint16_t* vp = vbase + (int64_t)r * rowstride + 8 * grp;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    ka[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kp + 32 * kk));
    va[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(vp + 32 * kk));
  }
  v4f s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    s = mfma_bf16_16x16x32(ka[kk], qb[kk], s);
    dp = mfma_bf16_16x16x32(va[kk], db[kk], dp);
  }
  // K rows, key-major, for the B operand of dS K
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    *reinterpret_cast<v4i*>(kl + hl * KROW + (32 * kk + 8 * grp) * 2) = __builtin_bit_cast(v4i, ka[kk]);
  v4s dhi, dlo;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float p = (vmask >> v) & 1u ? exp2f(s[v] * sl2 - lse2) : 0.f;
    const float ds = p * (dp[v] - dsum);
    short h, l;
    split_bf16(ds, h, l);
    dhi[v] = h;
    dlo[v] = l;
  }
  wave_sync_lds();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const char* p2 = kl + (4 * grp) * KROW + (16 * nb + hl) * 2;
    v4s kb;
#pragma unroll
    for (int e = 0; e < 4; ++e) kb[e] = *reinterpret_cast<const short*>(p2 + e * KROW);
    acc[nb] = mfma_bf16_16x16x16(dhi, kb, acc[nb]);
    acc[nb] = mfma_bf16_16x16x16(dlo, kb, acc[nb]);
  }
  wave_sync_lds();
}

// MODE 0: a query's long-range rows and the group's sinks and windows; MODE
// 1: the sinks and windows alone (the grouped pass adds the long range).
template <int D, int MODE>
__global__ void __launch_bounds__(BT, 2) k_bwd_dq(BwdArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int KROW = D * 2 + 16;
  __shared__ __attribute__((aligned(16))) char klds[BW][KT * KROW];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int item = xcd_remap(blockIdx.x, gridDim.x) * BW + wave;
  const int QPW = a.qpw;
  const int ngrp = (a.nq + QPW - 1) / QPW;
  if (item >= ngrp * a.Hkv) return;
  const int g = item % a.Hkv;
  const int q0 = (item / a.Hkv) * QPW;
  const int nqw = min(QPW, a.nq - q0);
  const int G = a.G;
  const int hl = lane & 15, grp = lane >> 4;
  const int jc = hl / G, hc = hl % G;
  const bool cval = jc < nqw;
  const int64_t qh = (int64_t)(q0 + (cval ? jc : 0)) * a.Hq + (int64_t)g * G + hc;

  // q and dO of column hl as B operands; dsum of the column
  v8bf qb[NKK], db[NKK];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int64_t e = qh * D + 32 * kk + 8 * grp;
    v4i rq = {0, 0, 0, 0}, rd = {0, 0, 0, 0};
    if (cval) {
      rq = *reinterpret_cast<const v4i*>(a.q + e);
      rd = *reinterpret_cast<const v4i*>(a.dout + e);
      float o8[8];
      load_o8(a, e, o8);
      dpart += dot8_bf16(rd, o8);
    }
    qb[kk] = __builtin_bit_cast(v8bf, rq);
    db[kk] = __builtin_bit_cast(v8bf, rd);
  }
  dpart += __shfl_xor(dpart, 16);
  dpart += __shfl_xor(dpart, 32);
  const float dsum = dpart;
  const float lse2 = cval ? a.lse[qh] * kLog2e : 0.f;
  if (cval && grp == 0) a.dsum[qh] = dsum;

  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};

  char* kl = klds[wave];
  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int64_t rmax = a.kv_rows - 1;
  const uint16_t* kbase = a.k + (int64_t)g * D;
  const uint16_t* vbase = a.v + (int64_t)g * D;
  const int tq0 = a.qpos0 + q0;
  auto wstart_of = [&](int t) { return max(0, t - a.window + 1); };
  auto nsink_of = [&](int ws) { return max(0, min(a.sinks, ws)); };

  // 1. long-range rows of each query (its own columns unmasked)
  for (int j = 0; j < (MODE == 0 ? nqw : 0); ++j) {
    const int q = q0 + j;
    const int t = tq0 + j;
    const int ws = wstart_of(t);
    const int nfix = nsink_of(ws) + (t - ws + 1);
    const int nlr = max(0, min(a.cnt[q], a.max_sel) - nfix);
    const int32_t* idxrow = a.idx + (int64_t)q * a.max_sel;
    const bool mine = cval && jc == j;
    for (int kb = 0; kb < nlr; kb += KT) {
      const int slot = kb + hl;
      int r = slot < nlr ? idxrow[slot] : 0;
      r = (int)min((int64_t)max(r, 0), rmax);
      unsigned vmask = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) vmask |= (mine && kb + 4 * grp + v < nlr ? 1u : 0u) << v;
      dq_tile<D>(qb, db, kbase, vbase, rowstride, r, vmask, a.scale_log2, lse2, dsum, kl, acc);
    }
  }
  // 2. the union of the group's sinks and windows, once
  {
    const int tl = tq0 + nqw - 1;
    const int nsl = nsink_of(wstart_of(tl));
    const int w0 = max(wstart_of(tq0), nsl);
    const int nu = nsl + (tl - w0 + 1);
    const int ct = tq0 + jc;
    const int cws = wstart_of(ct);
    const int cns = nsink_of(cws);
    const int shift = w0 - nsl;
    for (int kb = 0; kb < nu; kb += KT) {
      const int u = kb + hl;
      const int pos = u < nsl ? u : u + shift;
      const int r = (int)min((int64_t)pos, rmax);
      unsigned vmask = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int uv = kb + 4 * grp + v;
        const int pv = uv < nsl ? uv : uv + shift;
        const bool in = cval && uv < nu && (pv < cns || (pv >= cws && pv <= ct));
        vmask |= (in ? 1u : 0u) << v;
      }
      dq_tile<D>(qb, db, kbase, vbase, rowstride, r, vmask, a.scale_log2, lse2, dsum, kl, acc);
    }
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const int j = col / G, h = col % G;
    if (j >= nqw) continue;
    const int64_t ob = ((int64_t)(q0 + j) * a.Hq + (int64_t)g * G + h) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a.dq[ob + 16 * nb + hl] = acc[nb][v] * a.scale;
  }
}

// long-range entries of query qi: the row's entries before its sinks and window
__device__ __forceinline__ int lr_count(const BwdArgs& a, int qi) {
  const int t = a.qpos0 + qi;
  const int ws = max(0, t - a.window + 1);
  const int nfix = max(0, min(a.sinks, ws)) + (t - ws + 1);
  return max(0, min(a.cnt[qi], a.max_sel) - nfix);
}

// Grouped dQ: the long-range part of dQ over the grouped attention's plan.
// One wave per (group, KV head); the columns are (query slot, head) of the
// group's queries (perm), the union's rows are walked once, each column
// masked to its query's rows (a group over the cap walks each query's rows
// in turn).  dsum comes from the window pass (k_bwd_dq<D, 1>), which also
// wrote the window part of dQ; this pass adds to it (each (query, head) row
// of dQ is one wave's in each pass).
template <int D>
__global__ void __launch_bounds__(BT, 2) k_bwd_dq_grp(BwdArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int KROW = D * 2 + 16;
  __shared__ __attribute__((aligned(16))) char klds[BW][KT * KROW];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int item = xcd_remap(blockIdx.x, gridDim.x) * BW + wave;
  const int QPW = a.gqpw;
  const int ngrp = (a.nq + QPW - 1) / QPW;
  if (item >= ngrp * a.Hkv) return;
  const int g = item % a.Hkv;
  const int gi = item / a.Hkv;
  const int G = a.G;
  const int hl = lane & 15, grp = lane >> 4;
  const int jc = hl / G, hc = hl % G;
  const int slot = gi * QPW + jc;
  const bool cval = jc < QPW && slot < a.nq;
  const int qc = cval ? a.perm[slot] : 0;
  const int64_t qh = (int64_t)qc * a.Hq + (int64_t)g * G + hc;

  v8bf qb[NKK], db[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int64_t e = qh * D + 32 * kk + 8 * grp;
    v4i rq = {0, 0, 0, 0}, rd = {0, 0, 0, 0};
    if (cval) {
      rq = *reinterpret_cast<const v4i*>(a.q + e);
      rd = *reinterpret_cast<const v4i*>(a.dout + e);
    }
    qb[kk] = __builtin_bit_cast(v8bf, rq);
    db[kk] = __builtin_bit_cast(v8bf, rd);
  }
  const float dsum = cval ? a.dsum[qh] : 0.f;
  const float lse2 = cval ? a.lse[qh] * kLog2e : 0.f;

  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};

  char* kl = klds[wave];
  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int64_t rmax = a.kv_rows - 1;
  const uint16_t* kbase = a.k + (int64_t)g * D;
  const uint16_t* vbase = a.v + (int64_t)g * D;
  const int nu = a.ucnt[gi];
  if (nu >= 0) {
    const int32_t* ur = a.urow + (int64_t)gi * a.ucap;
    const uint8_t* um = a.umask + (int64_t)gi * a.ucap;
    for (int kb = 0; kb < nu; kb += KT) {
      const int sl = kb + hl;
      int r = sl < nu ? ur[sl] : 0;
      r = (int)min((int64_t)max(r, 0), rmax);
      // masks of union rows kb + 4 grp .. +3 (ucap is a multiple of 4)
      const int k4 = kb + 4 * grp;
      const unsigned m4 = k4 < nu ? *reinterpret_cast<const unsigned*>(um + k4) : 0u;
      unsigned vmask = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool in = cval && k4 + v < nu && ((m4 >> (8 * v + jc)) & 1u);
        vmask |= (in ? 1u : 0u) << v;
      }
      dq_tile<D>(qb, db, kbase, vbase, rowstride, r, vmask, a.scale_log2, lse2, dsum, kl, acc);
    }
  } else {
    for (int j = 0; j < QPW; ++j) {
      const int sl = gi * QPW + j;
      if (sl >= a.nq) break;
      const int q = a.perm[sl];
      const int nlr = lr_count(a, q);
      const int32_t* idxrow = a.idx + (int64_t)q * a.max_sel;
      const bool mine = cval && jc == j;
      for (int kb = 0; kb < nlr; kb += KT) {
        const int s2 = kb + hl;
        int r = s2 < nlr ? idxrow[s2] : 0;
        r = (int)min((int64_t)max(r, 0), rmax);
        unsigned vmask = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) vmask |= (mine && kb + 4 * grp + v < nlr ? 1u : 0u) << v;
        dq_tile<D>(qb, db, kbase, vbase, rowstride, r, vmask, a.scale_log2, lse2, dsum, kl, acc);
      }
    }
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const int qv = __shfl(qc, col);
    const bool vv = __shfl((int)cval, col) != 0;
    if (!vv) continue;
    const int64_t ob = ((int64_t)qv * a.Hq + (int64_t)g * G + col % G) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a.dq[ob + 16 * nb + hl] += acc[nb][v] * a.scale;
  }
}

// ---------------------------------------------------------------------------
// (bucket -> queries) lists

__global__ void k_bwd_map(BwdArgs a) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.n_bkt) return;
  const int c = a.bcnt[b], o = a.boff[b];
  for (int e = lane_id(); e < c; e += 64) a.map[a.bmem[o + e]] = b;
}

__device__ __forceinline__ int bucket_of_key(const BwdArgs& a, int j) {
  if (j < 0) return -1;
  const int m = j / a.pool;
  return m < a.n_pool ? a.map[m] : -1;
}


// MODE 0: count the runs per (bucket, tile); MODE 1: place them.  A run ends
// at entry e when the next entry lies in another bucket.
template <int PLACE>
__global__ void __launch_bounds__(256) k_bwd_runs(BwdArgs a) {
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int qbeg = tile * QT, qend = min(a.nq, qbeg + QT);
  // counting may take the tile's queries in any order: one wave per query;
  // placing takes them one after another so each list is ordered by query
  const int step = PLACE ? 256 : 64;
  const int first = PLACE ? tid : (tid & 63);
  for (int qi0 = qbeg; qi0 < qend; qi0 += PLACE ? 1 : 4) {
    const int qi = PLACE ? qi0 : qi0 + (tid >> 6);
    if (qi < qend) {
      const int nlr = lr_count(a, qi);
      const int32_t* row = a.idx + (int64_t)qi * a.max_sel;
      for (int e = first; e < nlr; e += step) {
        const int j = row[e];
        const int b = bucket_of_key(a, j);
        const int bn = e + 1 < nlr ? bucket_of_key(a, row[e + 1]) : -2;
        if (b >= 0 && bn != b) {
          int32_t* c = a.tcnt + (int64_t)b * a.n_tiles + tile;
          if (PLACE) {
            const int64_t pos = (int64_t)a.bstart[b] + atomicAdd(c, 1);
            if (pos < a.list_cap) a.list[pos] = make_int2(qi, j);
          } else {
            atomicAdd(c, 1);
          }
        }
      }
    }
    if (PLACE) __syncthreads();
  }
}

// per bucket: exclusive offsets over its query tiles, total, key tiles
__global__ void __launch_bounds__(256) k_bwd_scan_tiles(BwdArgs a) {
  __shared__ int red[4];
  const int b = blockIdx.x;
  int carry = 0;
  for (int i0 = 0; i0 < a.n_tiles; i0 += 256) {
    const int i = i0 + threadIdx.x;
    int32_t* c = a.tcnt + (int64_t)b * a.n_tiles + i;
    const int x = i < a.n_tiles ? *c : 0;
    int tot;
    const int ex = sel::block_excl_scan<256>(x, red, &tot);
    if (i < a.n_tiles) *c = carry + ex;
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.btot[b] = carry;
    const int nk = a.bcnt[b] * a.pool;
    a.ntl[b] = carry > 0 ? (nk + KTT - 1) / KTT : 0;
  }
}

// one workgroup: bucket starts and key-tile starts
__global__ void __launch_bounds__(1024) k_bwd_scan_buckets(BwdArgs a) {
  __shared__ int red[16];
  int c1 = 0, c2 = 0;
  for (int b0 = 0; b0 < a.n_bkt; b0 += 1024) {
    const int b = b0 + threadIdx.x;
    const int x1 = b < a.n_bkt ? a.btot[b] : 0;
    const int x2 = b < a.n_bkt ? a.ntl[b] : 0;
    int t1, t2;
    const int e1 = sel::block_excl_scan<1024>(x1, red, &t1);
    __syncthreads();
    const int e2 = sel::block_excl_scan<1024>(x2, red, &t2);
    if (b < a.n_bkt) {
      a.bstart[b] = c1 + e1;
      a.ktile0[b] = c2 + e2;
    }
    c1 += t1;
    c2 += t2;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.bstart[a.n_bkt] = c1;
    a.ktile0[a.n_bkt] = c2;
  }
}

// ---------------------------------------------------------------------------
// dK / dV over one key tile (64 keys of one KV head, 16 per wave) and a list
// of queries, 16/G at a time.  Column c of a group = (query c / G, head c % G).
// S[col][key] = q . k with Q rows as the A operand (from LDS) and the wave's
// keys as the B operand (registers), so each lane holds P and dS as the A
// operand (rows = keys, k = columns) of dV += P^T dO and dK += dS^T Q.
template <int D, int MODE>
__global__ void __launch_bounds__(KW * 64, 2) k_bwd_dkv(BwdArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int KROW = D * 2 + 16;
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int NLD = (2 * 16 * CH + KW * 64 - 1) / (KW * 64);
  __shared__ __attribute__((aligned(16))) char s_q[16 * KROW];
  __shared__ __attribute__((aligned(16))) char s_d[16 * KROW];
  __shared__ float s_lse[16], s_dsum[16];
  __shared__ int s_lo[16], s_hi[16];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int hl = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x % a.Hkv;
  const int unit = blockIdx.x / a.Hkv;
  const int G = a.G, QPW = a.qpw;

  // keys of this workgroup (lane: key slot hl of the wave) and its query list
  int key = -1;               // key id of slot hl (-1: none)
  int c0 = 0, c1 = 0;         // range of queries (band, sinks) or list entries (long range)
  int64_t lbase = 0;
  if (MODE == M_BAND) {
    const int j = unit * KTT + wave * 16 + hl;
    key = j < a.kv_rows ? j : -1;
    const int j0 = unit * KTT;
    c0 = max(0, j0 - a.qpos0);
    c1 = min(a.nq, j0 + KTT - 1 + a.window - 1 - a.qpos0 + 1);
  } else if (MODE == M_SINK) {
    const int j = wave * 16 + hl;
    key = j < a.sinks ? j : -1;
    c0 = unit * SINK_QC;
    c1 = min(a.nq, c0 + SINK_QC);
  } else {
    if (unit >= a.ktile0[a.n_bkt]) return;     // uniform
    int lo = 0, hi = a.n_bkt;                  // last b with ktile0[b] <= unit
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.ktile0[mid] <= unit) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int kt = unit - a.ktile0[b];
    const int kidx = kt * KTT + wave * 16 + hl;     // key number inside the bucket
    if (kidx < a.bcnt[b] * a.pool)
      key = a.bmem[a.boff[b] + kidx / a.pool] * a.pool + kidx % a.pool;
    lbase = a.bstart[b];
    c0 = 0;
    c1 = a.btot[b];
  }
  const bool kval = key >= 0;

  // the wave's keys as B operands
  v8bf kb[NKK], vb[NKK];
  {
    const int64_t rb = ((int64_t)(kval ? key : 0) * a.Hkv + g) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i rk = {0, 0, 0, 0}, rv = {0, 0, 0, 0};
      if (kval) {
        rk = *reinterpret_cast<const v4i*>(a.k + rb + 32 * kk);
        rv = *reinterpret_cast<const v4i*>(a.v + rb + 32 * kk);
      }
      kb[kk] = __builtin_bit_cast(v8bf, rk);
      vb[kk] = __builtin_bit_cast(v8bf, rv);
    }
  }

  v4f ak[NB], av[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ak[nb] = v4f{0.f, 0.f, 0.f, 0.f};
    av[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // query of list position c (band / sinks: query index; long range: entry)
  auto query_of = [&](int c, int& jmax) -> int {
    if (MODE == M_LR) {
      const int2 e = a.list[lbase + c];
      jmax = e.y;
      return min(max(e.x, 0), a.nq - 1);   // entries are query indices; clamp against misuse
    }
    jmax = 0;
    return c;
  };

  // one group's loads, held in registers until the group is staged in LDS:
  // Q and dO chunks, and (threads 0..15) the column's lse, dsum and key range
  struct Grp {
    v4i ld[NLD];
    float l2, ds;
    int lo, hi;
  };
  auto fetch = [&](Grp& R, int cg) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + i * KW * 64;
      R.ld[i] = v4i{0, 0, 0, 0};
      if (c < 2 * 16 * CH) {
        const int tsel = c / (16 * CH);
        const int rem = c % (16 * CH);
        const int col = rem / CH, ch = rem % CH;
        const int cpos = cg + col / G;
        if (col / G < QPW && cpos < c1) {
          int jm;
          const int qi = query_of(cpos, jm);
          const int64_t e = ((int64_t)qi * a.Hq + (int64_t)g * G + col % G) * D + ch * 8;
          R.ld[i] = *reinterpret_cast<const v4i*>((tsel ? a.dout : a.q) + e);
        }
      }
    }
    R.l2 = 0.f; R.ds = 0.f; R.lo = 1; R.hi = 0;      // empty key range
    if (tid < 16) {
      const int col = tid;
      const int cpos = cg + col / G;
      if (col / G < QPW && cpos < c1) {
        int jm;
        const int qi = query_of(cpos, jm);
        const int64_t qh = (int64_t)qi * a.Hq + (int64_t)g * G + col % G;
        R.l2 = a.lse[qh] * kLog2e;
        R.ds = a.dsum[qh];
        const int t = a.qpos0 + qi;
        if (MODE == M_BAND) { R.lo = t - a.window + 1; R.hi = t; }
        else if (MODE == M_SINK) { R.lo = 0; R.hi = min(a.sinks - 1, t - a.window); }
        else { R.lo = a.sinks; R.hi = jm; }
      }
    }
  };
  auto stash = [&](const Grp& R) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + i * KW * 64;
      if (c < 2 * 16 * CH) {
        const int tsel = c / (16 * CH);
        const int rem = c % (16 * CH);
        const int col = rem / CH, ch = rem % CH;
        *reinterpret_cast<v4i*>((tsel ? s_d : s_q) + col * KROW + ch * 16) = R.ld[i];
      }
    }
    if (tid < 16) {
      s_lse[tid] = R.l2;
      s_dsum[tid] = R.ds;
      s_lo[tid] = R.lo;
      s_hi[tid] = R.hi;
    }
  };

  // a wave none of whose key slots holds a key (the tail of a bucket's last
  // 64-key tile; most tiles of the small buckets queries take) still loads
  // and stages its share of each group, but computes nothing
  const bool wave_live = __builtin_amdgcn_ballot_w64(kval) != 0;

  // two groups in flight ahead of the one being computed
  Grp ra, rb;
  if (c0 < c1) fetch(ra, c0);
  if (c0 + QPW < c1) fetch(rb, c0 + QPW);
  for (int cg = c0; cg < c1; cg += QPW) {
    __syncthreads();                 // previous group's LDS reads are done
    stash(ra);
    __syncthreads();
    ra = rb;
    if (cg + 2 * QPW < c1) fetch(rb, cg + 2 * QPW);
    if (!wave_live) continue;        // wave-uniform; the barriers above stay matched

    v8bf qa[NKK], da[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qa[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(s_q + hl * KROW + (32 * kk + 8 * grp) * 2));
      da[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(s_d + hl * KROW + (32 * kk + 8 * grp) * 2));
    }
    v4f s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s = mfma_bf16_16x16x32(qa[kk], kb[kk], s);
      dp = mfma_bf16_16x16x32(da[kk], vb[kk], dp);
    }
    // lane: key slot hl, columns 4*grp + v
    v4s phi, plo, dhi, dlo;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = 4 * grp + v;
      const bool in = kval && key >= s_lo[col] && key <= s_hi[col];
      const float p = in ? exp2f(s[v] * a.scale_log2 - s_lse[col]) : 0.f;
      const float ds = p * (dp[v] - s_dsum[col]);
      short h, l;
      split_bf16(p, h, l);
      phi[v] = h; plo[v] = l;
      split_bf16(ds, h, l);
      dhi[v] = h; dlo[v] = l;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      v4s bo, bq;
      const int off = (4 * grp) * KROW + (16 * nb + hl) * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bo[e] = *reinterpret_cast<const short*>(s_d + off + e * KROW);
        bq[e] = *reinterpret_cast<const short*>(s_q + off + e * KROW);
      }
      av[nb] = mfma_bf16_16x16x16(phi, bo, av[nb]);
      av[nb] = mfma_bf16_16x16x16(plo, bo, av[nb]);
      ak[nb] = mfma_bf16_16x16x16(dhi, bq, ak[nb]);
      ak[nb] = mfma_bf16_16x16x16(dlo, bq, ak[nb]);
    }
  }

  // lane holds rows (key slots) 4*grp + v, column d = 16*nb + hl
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rkey = __shfl(key, 4 * grp + v);
    if (MODE == M_SINK) {
      const int slot = wave * 16 + 4 * grp + v;
      float* pk = a.sink_part + (((int64_t)unit * a.Hkv + g) * KTT + slot) * D;
      float* pv = pk + (int64_t)a.n_sink_chunks * a.Hkv * KTT * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        pk[16 * nb + hl] = ak[nb][v] * a.scale;
        pv[16 * nb + hl] = av[nb][v];
      }
      continue;
    }
    if (rkey < 0) continue;
    const int64_t ob = ((int64_t)rkey * a.Hkv + g) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t e = ob + 16 * nb + hl;
      if (MODE == M_BAND) {
        a.dk[e] = ak[nb][v] * a.scale;
        a.dv[e] = av[nb][v];
      } else {
        a.dk[e] += ak[nb][v] * a.scale;
        a.dv[e] += av[nb][v];
      }
    }
  }
}

// sink keys: add the chunk partial sums, in chunk order
template <int D>
__global__ void k_bwd_sink_reduce(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (g, key, d)
  const int64_t n = (int64_t)a.Hkv * a.sinks * D;
  if (i >= n) return;
  const int d = (int)(i % D);
  const int j = (int)((i / D) % a.sinks);
  const int g = (int)(i / ((int64_t)D * a.sinks));
  const int64_t half = (int64_t)a.n_sink_chunks * a.Hkv * KTT * D;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < a.n_sink_chunks; ++c) {
    const int64_t e = (((int64_t)c * a.Hkv + g) * KTT + j) * D + d;
    sk += a.sink_part[e];
    sv += a.sink_part[half + e];
  }
  const int64_t o = ((int64_t)j * a.Hkv + g) * D + d;
  a.dk[o] += sk;
  a.dv[o] += sv;
}

__global__ void k_zero_i32(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

struct BwdLayout {
  int64_t dsum, map, tcnt, btot, ntl, bstart, ktile0, list, sink, total;
  int64_t list_cap;
  int32_t n_tiles, n_sink_chunks;
};

// plan_bytes: the grouped dQ's plan, which shares the list's bytes (the plan
// is used up before the lists are written)
BwdLayout bwd_layout(int32_t nq, int32_t Hq, int32_t Hkv, int32_t D, int64_t max_pool,
                     int64_t max_bkt, int32_t budget, int64_t plan_bytes) {
  BwdLayout L;
  L.n_tiles = (nq + QT - 1) / QT;
  L.n_sink_chunks = (nq + SINK_QC - 1) / SINK_QC;
  L.list_cap = (int64_t)nq * (budget < max_bkt ? (int64_t)budget : max_bkt);
  int64_t o = 0;
  L.dsum = o;   o = align256(o + (int64_t)nq * Hq * 4);
  L.map = o;    o = align256(o + max_pool * 4);
  L.tcnt = o;   o = align256(o + max_bkt * L.n_tiles * 4);
  L.btot = o;   o = align256(o + max_bkt * 4);
  L.ntl = o;    o = align256(o + max_bkt * 4);
  L.bstart = o; o = align256(o + (max_bkt + 1) * 4);
  L.ktile0 = o; o = align256(o + (max_bkt + 1) * 4);
  L.list = o;   o = align256(o + std::max(L.list_cap * 8, plan_bytes));
  L.sink = o;   o = align256(o + (int64_t)L.n_sink_chunks * Hkv * KTT * D * 2 * 4);
  L.total = o;
  return L;
}

}  // namespace

namespace {
// bytes of the grouped dQ's plan (0 when the shape takes the ungrouped dQ)
int64_t bwd_plan_bytes(int32_t nq, const lsa_attn_params& ap, int32_t budget) {
  return grouped_attn_ok(ap, budget, 1) && grouped_nq_ok(nq) ? (int64_t)grouped_plan_ws_bytes(nq, ap, budget)
                                                              : 0;
}
}  // namespace

size_t attn_bwd_ws_bytes(int32_t nq, const lsa_attn_params& ap, int64_t max_pool, int64_t max_bkt,
                         int32_t budget) {
  return (size_t)bwd_layout(nq, ap.Hq, ap.Hkv, ap.D, max_pool, max_bkt, budget,
                            bwd_plan_bytes(nq, ap, budget)).total;
}

hipError_t launch_attn_bwd(const BwdInputs& in, const lsa_attn_params& ap, hipStream_t s) {
  if (in.nq <= 0) return hipSuccess;
  const int64_t plan_bytes = bwd_plan_bytes(in.nq, ap, in.budget);
  const BwdLayout L = bwd_layout(in.nq, ap.Hq, ap.Hkv, ap.D, in.max_pool, in.max_bkt, in.budget,
                                 plan_bytes);
  char* ws = static_cast<char*>(in.ws);
  BwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = in.q; a.k = in.k; a.v = in.v; a.o = in.o; a.o_f32 = ap.out_f32 != 0; a.dout = in.dout;
  a.lse = in.lse; a.kv_rows = in.kv_rows; a.idx = in.idx; a.cnt = in.cnt;
  a.max_sel = in.max_sel; a.nq = in.nq; a.qpos0 = (int32_t)in.qpos0;
  a.window = in.window; a.sinks = in.sinks;
  a.Hq = ap.Hq; a.Hkv = ap.Hkv; a.G = ap.Hq / ap.Hkv; a.qpw = 16 / a.G;
  a.scale = ap.scale > 0.f ? ap.scale : 1.0f / sqrtf((float)ap.D);
  a.scale_log2 = a.scale * kLog2e;
  a.dq = in.dq; a.dk = in.dk; a.dv = in.dv;
  a.dsum = reinterpret_cast<float*>(ws + L.dsum);
  a.bcnt = in.bcnt; a.boff = in.boff; a.bmem = in.bmem;
  a.n_bkt = in.n_bkt; a.pool = in.pool; a.n_pool = in.n_pool;
  a.map = reinterpret_cast<int32_t*>(ws + L.map);
  a.tcnt = reinterpret_cast<int32_t*>(ws + L.tcnt);
  a.btot = reinterpret_cast<int32_t*>(ws + L.btot);
  a.ntl = reinterpret_cast<int32_t*>(ws + L.ntl);
  a.bstart = reinterpret_cast<int32_t*>(ws + L.bstart);
  a.ktile0 = reinterpret_cast<int32_t*>(ws + L.ktile0);
  a.list = reinterpret_cast<int2*>(ws + L.list);
  a.list_cap = L.list_cap;
  a.n_tiles = L.n_tiles;
  a.sink_part = reinterpret_cast<float*>(ws + L.sink);
  a.n_sink_chunks = L.n_sink_chunks;
  const bool d128 = ap.D == 128;

  // dQ (and dsum): grouped (window pass, then the long range over the plan's
  // unions) when the shape allows, else one pass
  {
    const int64_t items = (int64_t)((in.nq + a.qpw - 1) / a.qpw) * ap.Hkv;
    const unsigned grid = (unsigned)((items + BW - 1) / BW);
    if (plan_bytes > 0 && grouped_attn_ok(ap, in.budget, in.kv_rows)) {
      GroupPlanView pv;
      if (hipError_t e = launch_grouped_plan(in.idx, in.cnt, in.max_sel, in.nq, in.qpos0, in.window,
                                             in.sinks, in.kv_rows, in.budget, ap, in.latq, ws + L.list,
                                             &pv, s))
        return e;
      a.perm = pv.perm; a.urow = pv.urow; a.umask = pv.umask; a.ucnt = pv.ucnt;
      a.ucap = pv.ucap; a.gqpw = pv.qpw;
      if (d128) hipLaunchKernelGGL((k_bwd_dq<128, 1>), dim3(grid), dim3(BT), 0, s, a);
      else hipLaunchKernelGGL((k_bwd_dq<64, 1>), dim3(grid), dim3(BT), 0, s, a);
      if (hipError_t e = hipGetLastError()) return e;
      const int64_t gitems = (int64_t)pv.ngrp * ap.Hkv;
      const unsigned ggrid = (unsigned)((gitems + BW - 1) / BW);
      if (d128) hipLaunchKernelGGL(k_bwd_dq_grp<128>, dim3(ggrid), dim3(BT), 0, s, a);
      else hipLaunchKernelGGL(k_bwd_dq_grp<64>, dim3(ggrid), dim3(BT), 0, s, a);
    } else {
      if (d128) hipLaunchKernelGGL((k_bwd_dq<128, 0>), dim3(grid), dim3(BT), 0, s, a);
      else hipLaunchKernelGGL((k_bwd_dq<64, 0>), dim3(grid), dim3(BT), 0, s, a);
    }
    if (hipError_t e = hipGetLastError()) return e;
  }
  // band: stores every key row of dK / dV
  {
    const unsigned grid = (unsigned)(((in.kv_rows + KTT - 1) / KTT) * ap.Hkv);
    if (d128) hipLaunchKernelGGL((k_bwd_dkv<128, M_BAND>), dim3(grid), dim3(KW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dkv<64, M_BAND>), dim3(grid), dim3(KW * 64), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  // long range
  if (a.n_bkt > 0) {
    const int64_t nt = (int64_t)a.n_bkt * a.n_tiles;
    hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, a.tcnt, nt);
    hipLaunchKernelGGL(k_bwd_map, dim3((unsigned)((a.n_bkt + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_runs<0>, dim3((unsigned)a.n_tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_scan_tiles, dim3((unsigned)a.n_bkt), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_bwd_scan_buckets, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_bwd_runs<1>, dim3((unsigned)a.n_tiles), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
    // at most one partial tile per bucket beyond the full ones
    const int64_t tiles = (int64_t)a.n_bkt + ((int64_t)a.n_pool * a.pool + KTT - 1) / KTT;
    const unsigned grid = (unsigned)(tiles * ap.Hkv);
    if (d128) hipLaunchKernelGGL((k_bwd_dkv<128, M_LR>), dim3(grid), dim3(KW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dkv<64, M_LR>), dim3(grid), dim3(KW * 64), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  // sinks outside the window
  if (a.sinks > 0) {
    const unsigned grid = (unsigned)(a.n_sink_chunks * ap.Hkv);
    if (d128) hipLaunchKernelGGL((k_bwd_dkv<128, M_SINK>), dim3(grid), dim3(KW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dkv<64, M_SINK>), dim3(grid), dim3(KW * 64), 0, s, a);
    const int64_t n = (int64_t)ap.Hkv * a.sinks * ap.D;
    if (d128) hipLaunchKernelGGL(k_bwd_sink_reduce<128>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_bwd_sink_reduce<64>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace lsa
