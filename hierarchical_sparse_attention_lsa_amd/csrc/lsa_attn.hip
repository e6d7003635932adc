// Sparse GQA attention over the selected K/V rows.
//
// "Prefrontal's Latent Sparse Attention speeds up one attention layer 72x at
// 10M tokens" (sysnote.net), section "What it changes": the attention itself
// is unchanged and runs over a fixed number of keys whatever the context
// length; LSA only decides which keys are read.  "Latent Sparse Attention:
// un indice gerarchico per contesti lunghi" (mauroscia.it), search
// paragraph: attention is computed on the selected keys and values; the KV
// cache keeps the original representations.
//
// Design (gfx950): one wave owns one (query token, KV head) pair and walks
// its selected rows 16 at a time.  K rows go straight from HBM into the A
// operand of v_mfma_f32_16x16x32_bf16 (keys on M, head dim on K), with the
// group's query heads as the B operand (N = 16 padded heads), so the output
// tile is S^T [16 keys][16 heads] and each lane already holds the four
// probabilities it must feed, as the A operand, to the 16x16x16 PV product.
// V rows are staged through LDS (per-wave region, no workgroup barrier) and
// read back key-major for the B operand.  Softmax runs online in fp32 with
// exp2; P enters the PV product as bf16 hi + bf16 lo so that the probability
// rounding stays far below the output tolerance.  The eight waves of a
// workgroup take the eight KV heads of one query, so each 2 KiB K/V row is
// fetched by one workgroup at once.  Workgroups are remapped so that each
// XCD (own L2) walks a contiguous range of queries, whose recent windows
// overlap.
#include <climits>
#include <cstring>
#include <utility>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select_common.h"

namespace lsa {

namespace {

constexpr int AW = 8;            // waves per workgroup
constexpr int AT = AW * 64;
constexpr int KT = 16;           // keys per tile

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_rows;           // rows per sequence (clamp bound of key ids)
  int64_t seq_stride_rows;   // rows between sequences (decode)
  int32_t qdiv;              // query -> sequence divisor
  const int32_t* idx;
  const int32_t* cnt;
  int32_t max_sel;
  int32_t nq;
  int32_t Hq, Hkv, G;
  int32_t splits;
  float scale_log2;          // softmax scale * log2(e)
  void* out;
  float* part_o;             // [items][G][D] unnormalised partial outputs (split mode)
  float* part_ml;            // [items][16][2] running max (log2 domain) and sum
  // window-sharing mode: queries are positions qpos0 .. qpos0+nq-1 and their
  // rows end with the sinks and window of the select rule
  int64_t qpos0;
  int32_t window, sinks;
  int32_t qpw;               // queries per wave (16 / G)
  float* lse;                // nullable [nq][Hq]: natural log-sum-exp of the scaled logits
  // grouped mode: a wave's queries are perm[gi*qpw ..]; their long-range rows
  // are the union urow[gi][0 .. ucnt[gi]) with umask bit j set for the
  // group's query j; the sinks and window come from the window partials
  // (part_o [nq][Hq][D], part_ml [nq][Hq][2])
  const int32_t* perm;
  const int32_t* urow;
  const uint8_t* umask;
  const int32_t* ucnt;
  int32_t ucap;
};

__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  const int per = nwg >> 3, rem = nwg & 7, x = b & 7, k = b >> 3;
  return x * per + min(x, rem) + k;
}

// One 16-key tile of the online-softmax attention of a wave, in two halves so
// that a caller can keep the next tile's loads in flight: tile_load fetches
// K rows into the A operand and V rows into registers; tile_compute does the
// QK^T MFMAs, the online softmax and the PV MFMAs.  Lane l loads K row `r`
// for key slot l % 16 (every lane of that slot passes the same r); bit v of
// `vmask` says whether S^T[4*(l/16)+v][l%16] (key 4*(l/16)+v of the tile,
// column l%16) takes part.  o / m_run / l_run: the column's state.
constexpr float kLazy = 8.f;     // log2 headroom before the reference max moves

// Sum of a column's partial softmax denominators over the four lanes that
// hold it (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float finish_l(float l) {
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  return l;
}

template <int D>
struct TileRegs {
  v8bf ka[D / 32];
  v4i vr[KT * (D / 8) / 64];
};

template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& T, const uint16_t* kbase, const uint16_t* vbase,
                                          int64_t rowstride, int r) {
  constexpr int NKK = D / 32;
  constexpr int VCH = D / 8;
  constexpr int VLD = KT * VCH / 64;
  const int lane = lane_id();
  const int grp = lane >> 4;
  const uint16_t* kp = kbase + (int64_t)r * rowstride + 8 * grp;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    T.ka[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kp + 32 * kk));
#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    const int c = i * 64 + lane;
    const int key = c / VCH, ch = c % VCH;
    const int rv = __shfl(r, key);
    T.vr[i] = *reinterpret_cast<const v4i*>(vbase + (int64_t)rv * rowstride + ch * 8);
  }
}

// The query operand of the QK^T MFMAs (B: lane l supplies column l % 16,
// head-dim elements 32 kk + 8 (l / 16) ..), from registers or from LDS.
template <int D>
struct QRegs {
  v8bf b[D / 32];
  __device__ __forceinline__ v8bf operator()(int kk) const { return b[kk]; }
};
constexpr int qrow_bytes(int D) { return D * 2 + 16; }       // padded LDS row of one column
template <int D>
struct QLds {
  const char* p;                    // this lane's column row + its 16-byte group
  __device__ __forceinline__ v8bf operator()(int kk) const {
    return *reinterpret_cast<const v8bf*>(p + 64 * kk);
  }
};

template <int D, class QOp>
__device__ __forceinline__ void tile_compute(const QOp& qb, const TileRegs<D>& T,
                                             unsigned vmask, float scale_log2, char* vl,
                                             v4f (&o)[D / 16], float& m_run, float& l_run) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int VROW = D * 2 + 16;
  constexpr int VCH = D / 8;
  constexpr int VLD = KT * VCH / 64;
  const int lane = lane_id();
  const int hl = lane & 15;
  const int grp = lane >> 4;

  // S^T[key][column]
  v4f s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) s = mfma_bf16_16x16x32(T.ka[kk], qb(kk), s);

#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    const int c = i * 64 + lane;
    const int key = c / VCH, ch = c % VCH;
    *reinterpret_cast<v4i*>(vl + key * VROW + ch * 16) = T.vr[i];
  }

  // online softmax for column hl over keys 4*grp + v.  The reference max
  // m_run moves only when a logit exceeds it by more than kLazy (log2
  // units), so most tiles skip the cross-lane max and the rescale of the
  // accumulators; probabilities stay below 2^kLazy.  l_run is this lane's
  // partial sum (keys 4*grp + v); finish_l adds the four partials.
  float sv[4];
  float tmax = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sv[v] = (vmask >> v) & 1u ? s[v] * scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, sv[v]);
  }
  if (__builtin_amdgcn_ballot_w64(tmax > m_run + kLazy) != 0) {      // wave-uniform
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
    // rescale the accumulators: o rows are columns 4*grp + v
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, 4 * grp + v);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb][v] *= av;
    }
  }
  float p[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    p[v] = exp2f(sv[v] - m_run);
    l_run += p[v];
  }

  // P (A operand, rows = columns, k = keys 4*grp..+3) as bf16 hi + lo
  v4s phi, plo;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t hb = f32_to_bf16_bits(p[v]);
    const float rem = p[v] - bf16_bits_to_f32(hb);
    phi[v] = (short)hb;
    plo[v] = (short)f32_to_bf16_bits(rem);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // O += P V, V^T operand read key-major from LDS
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const char* vp = vl + (4 * grp) * VROW + (16 * nb + hl) * 2;
    v4s vb;
#pragma unroll
    for (int e = 0; e < 4; ++e) vb[e] = *reinterpret_cast<const short*>(vp + e * VROW);
    o[nb] = mfma_bf16_16x16x16(phi, vb, o[nb]);
    o[nb] = mfma_bf16_16x16x16(plo, vb, o[nb]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, class QOp>
__device__ __forceinline__ void attn_tile(const QOp& qb, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t rowstride, int r,
                                          unsigned vmask, float scale_log2, char* vl,
                                          v4f (&o)[D / 16], float& m_run, float& l_run) {
  TileRegs<D> T;
  tile_load<D>(T, kbase, vbase, rowstride, r);
  tile_compute<D>(qb, T, vmask, scale_log2, vl, o, m_run, l_run);
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(AT) k_attn(AttnArgs a) {
  constexpr int NKK = D / 32;         // 32-deep slices of the head dim
  constexpr int NB = D / 16;          // 16-wide output column blocks
  constexpr int VROW = D * 2 + 16;    // padded LDS row (bytes)
  __shared__ __attribute__((aligned(16))) char vlds[AW][KT * VROW];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nwg = gridDim.x;
  const int item = xcd_remap(blockIdx.x, nwg) * AW + wave;
  if (item >= a.nq * a.Hkv) return;
  const int q = item / a.Hkv;
  const int g = item % a.Hkv;
  const int G = a.G;
  const int hl = lane & 15;           // head (S^T column) / key row for K loads
  const int grp = lane >> 4;

  const int cnt = min(a.cnt[q], a.max_sel);
  const int kbeg = 0, kend = cnt;
  const int64_t rowbase = (int64_t)(q / a.qdiv) * a.seq_stride_rows;
  const int64_t rowstride = (int64_t)a.Hkv * D;        // elements per K/V row
  const int32_t* idxrow = a.idx + (int64_t)q * a.max_sel;

  // query heads of this group as the B operand (zero for padded heads)
  QRegs<D> qb;
  {
    const bool hv = hl < G;
    const uint16_t* qp = a.q + ((int64_t)q * a.Hq + (int64_t)g * G + (hv ? hl : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = hv ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      qb.b[kk] = __builtin_bit_cast(v8bf, raw);
    }
  }

  v4f o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;    // stats of head hl (replicated over grp)

  char* vl = vlds[wave];
  const uint16_t* kbase = a.k + (rowbase * a.Hkv + g) * D;
  const uint16_t* vbase = a.v + (rowbase * a.Hkv + g) * D;
  const int64_t rmax = a.kv_rows - 1;                 // rows of one sequence

  for (int kb = kbeg; kb < kend; kb += KT) {
    // selected rows of this tile: lane l holds key slot kb + (l % 16)
    const int slot = kb + hl;
    int r = slot < kend ? idxrow[slot] : 0;
    r = (int)min((int64_t)max(r, 0), rmax);
    unsigned vmask = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) vmask |= (kb + 4 * grp + v < kend ? 1u : 0u) << v;
    attn_tile<D>(qb, kbase, vbase, rowstride, r, vmask, a.scale_log2, vl, o, m_run, l_run);
  }

  l_run = finish_l(l_run);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * grp + v;
    const float lh = __shfl(l_run, h);
    if (h >= G) continue;
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    const int64_t ob = ((int64_t)q * a.Hq + (int64_t)g * G + h) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float val = o[nb][v] * inv;
      if (OUT_F32) reinterpret_cast<float*>(a.out)[ob + 16 * nb + hl] = val;
      else reinterpret_cast<uint16_t*>(a.out)[ob + 16 * nb + hl] = (uint16_t)f32_to_bf16_bits(val);
    }
  }
}

// Window-sharing variant for consecutive query positions (prefill chunks).
// The rows the select writes end with the sinks and the recent window, and
// consecutive queries share almost all of their windows.  A wave here owns
// QPW = 16 / G consecutive queries of one KV head: the 16 columns of S^T are
// (query, head) pairs, so the MFMA tiles are full.  The wave first walks each
// query's long-range keys (its own columns unmasked), then the union of the
// group's sinks and windows once, as contiguous K/V rows, each column masked
// to its own query's sinks and window.  Per query the result is the same
// attention over the same key set; only the summation order differs.
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(AT, 4) k_attn_win(AttnArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int VROW = D * 2 + 16;
  __shared__ __attribute__((aligned(16))) char vlds[AW][KT * VROW];
  __shared__ __attribute__((aligned(16))) char qlds[AW][16 * qrow_bytes(D)];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nwg = gridDim.x;
  const int item = xcd_remap(blockIdx.x, nwg) * AW + wave;
  const int QPW = a.qpw;
  const int ngrp = (a.nq + QPW - 1) / QPW;
  if (item >= ngrp * a.Hkv) return;
  const int g = item % a.Hkv;
  const int q0 = (item / a.Hkv) * QPW;
  const int nqw = min(QPW, a.nq - q0);     // queries of this wave
  const int G = a.G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  // this lane's column: query jc of the group, head hc of the KV group
  const int jc = hl / G, hc = hl % G;
  const bool cval = jc < nqw;

  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int64_t rmax = a.kv_rows - 1;

  // query operand: column hl = (query q0 + jc, head g*G + hc), staged in
  // this wave's LDS rows (registers held across the whole walk would leave
  // too few for the K/V loads in flight)
  char* ql = qlds[wave];
  {
    const uint16_t* qp = a.q + ((int64_t)(q0 + (cval ? jc : 0)) * a.Hq + (int64_t)g * G + hc) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = cval ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(ql + hl * qrow_bytes(D) + (32 * kk + 8 * grp) * 2) = raw;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const QLds<D> qb{ql + hl * qrow_bytes(D) + 16 * grp};

  v4f o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;

  char* vl = vlds[wave];
  const uint16_t* kbase = a.k + (int64_t)g * D;
  const uint16_t* vbase = a.v + (int64_t)g * D;

  // the select rule's sinks and window for query position t (positions fit
  // in int32: an index holds fewer than 2^31 keys)
  const int tq0 = (int)a.qpos0 + q0;
  auto wstart_of = [&](int t) { return max(0, t - a.window + 1); };
  auto nsink_of = [&](int ws) { return max(0, min(a.sinks, ws)); };

  // 1. long-range keys of each query: the row's entries before its sinks and window
  for (int j = 0; j < nqw; ++j) {
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
      attn_tile<D>(qb, kbase, vbase, rowstride, r, vmask, a.scale_log2, vl, o, m_run, l_run);
    }
  }

  // 2. the union of the group's sinks and windows, once: positions
  //    [0, ns_last) then [max(ws_first, ns_last), t_last]
  {
    const int tl = tq0 + nqw - 1;
    const int nsl = nsink_of(wstart_of(tl));
    const int w0 = max(wstart_of(tq0), nsl);
    const int nu = nsl + (tl - w0 + 1);
    // this lane's column: its query's sinks [0, cns) and window [cws, ct]
    const int ct = tq0 + jc;
    const int cws = wstart_of(ct);
    const int cns = nsink_of(cws);
    const int shift = w0 - nsl;       // position of union slot u >= nsl is u + shift
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
      attn_tile<D>(qb, kbase, vbase, rowstride, r, vmask, a.scale_log2, vl, o, m_run, l_run);
    }
  }

  l_run = finish_l(l_run);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const float lh = __shfl(l_run, col);
    const float mh = __shfl(m_run, col);
    const int j = col / G, h = col % G;
    if (j >= nqw) continue;
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    const int64_t ob = ((int64_t)(q0 + j) * a.Hq + (int64_t)g * G + h) * D;
    // log-sum-exp: m_run and l_run are in the log2 domain of the scaled logits
    if (a.lse && hl == 0) a.lse[(int64_t)(q0 + j) * a.Hq + (int64_t)g * G + h] =
        (mh + __log2f(lh)) * 0.6931471805599453f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float val = o[nb][v] * inv;
      if (OUT_F32) reinterpret_cast<float*>(a.out)[ob + 16 * nb + hl] = val;
      else reinterpret_cast<uint16_t*>(a.out)[ob + 16 * nb + hl] = (uint16_t)f32_to_bf16_bits(val);
    }
  }
}

// Sinks-and-window partials for the grouped attention, the K/V tiles shared
// by a workgroup.  Consecutive queries' windows are nearly the same rows, so
// a workgroup takes SW * qpw consecutive queries of one KV head: each 16-row
// tile of the union of their sinks and windows is loaded once into LDS (K and
// V, double-buffered, one 16-byte load per thread) and each wave multiplies it
// against its own qpw queries' columns, each column masked to its query's
// sinks and window (a tile with none of a wave's keys is skipped by that
// wave).  Per query the key set is the rule's; the unnormalised output and
// (max, sum) per (query, head) go to part_o / part_ml, where the grouped
// long-range kernel starts from them.  Each wave reads every tile from LDS instead of from L2, which
// bounded a per-wave walk of the same windows.
constexpr int SW = 8;                  // waves (query groups) per workgroup

template <int D>
__global__ void __launch_bounds__(SW * 64) k_attn_swin(AttnArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int VROW = D * 2 + 16;
  constexpr int VCH = D / 8;           // 16-byte chunks of one head's row
  constexpr int NCH = KT * VCH;        // chunks of a tile's K (or V) rows: 256 or 128
  static_assert(NCH <= SW * 32, "K loads by the first half of the threads, V by the second");
  __shared__ __attribute__((aligned(16))) char klds[2][KT * VROW];
  __shared__ __attribute__((aligned(16))) char vlds[2][KT * VROW];
  __shared__ __attribute__((aligned(16))) char qlds[SW][16 * qrow_bytes(D)];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int QPW = a.qpw;
  const int span = SW * QPW;
  const int nspan = (a.nq + span - 1) / span;
  const int item = xcd_remap(blockIdx.x, gridDim.x);     // (query span, KV head)
  if (item >= nspan * a.Hkv) return;                     // the whole workgroup
  const int g = item % a.Hkv;
  const int qs0 = (item / a.Hkv) * span;                 // the workgroup's first query
  const int nqs = min(span, a.nq - qs0);
  const int q0 = qs0 + wave * QPW;                       // this wave's first query
  const int nqw = max(0, min(QPW, a.nq - q0));
  const int G = a.G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int jc = hl / G, hc = hl % G;
  const bool cval = jc < nqw;
  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int64_t rmax = a.kv_rows - 1;

  // query operand: column hl = (query q0 + jc, head g*G + hc), in this wave's LDS rows
  char* ql = qlds[wave];
  {
    const int qq = min(q0 + (cval ? jc : 0), a.nq - 1);
    const uint16_t* qp = a.q + ((int64_t)qq * a.Hq + (int64_t)g * G + hc) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = cval ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(ql + hl * qrow_bytes(D) + (32 * kk + 8 * grp) * 2) = raw;
    }
  }
  const QLds<D> qb{ql + hl * qrow_bytes(D) + 16 * grp};

  // the union of the workgroup's sinks and windows: positions [0, nsl), then
  // [w0, tl] (sink counts grow with the position, so the last query's hold
  // every query's; w0 >= nsl keeps the two parts apart)
  auto wstart_of = [&](int t) { return max(0, t - a.window + 1); };
  auto nsink_of = [&](int ws) { return max(0, min(a.sinks, ws)); };
  const int tq0 = (int)a.qpos0 + qs0;
  const int tl = tq0 + nqs - 1;
  const int nsl = nsink_of(wstart_of(tl));
  const int w0 = max(wstart_of(tq0), nsl);
  const int nu = nsl + (tl - w0 + 1);
  const int shift = w0 - nsl;          // position of union slot u >= nsl is u + shift
  // this lane's column: its query's sinks [0, cns) and window [cws, ct]
  const int ct = (int)a.qpos0 + q0 + jc;
  const int cws = wstart_of(ct);
  const int cns = nsink_of(cws);

  // tile loads: threads [0, NCH) take K chunks, [SW * 32, SW * 32 + NCH) V chunks
  const bool ldk = tid < NCH;
  const bool ldv = tid >= SW * 32 && tid < SW * 32 + NCH;
  const bool ld = ldk || ldv;
  const int ci = ldk ? tid : tid - SW * 32;
  const int ckey = ci / VCH, cch = ci % VCH;
  const uint16_t* src = (ldk ? a.k : a.v) + (int64_t)g * D + cch * 8;
  auto gload = [&](int kb) -> v4i {
    const int u = min(kb + ckey, nu - 1);
    const int pos = u < nsl ? u : u + shift;
    return *reinterpret_cast<const v4i*>(src + min((int64_t)pos, rmax) * rowstride);
  };
  auto swrite = [&](int buf, v4i x) {
    *reinterpret_cast<v4i*>((ldk ? klds[buf] : vlds[buf]) + ckey * VROW + cch * 16) = x;
  };

  v4f o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;

  // Tile i is computed from LDS buffer i & 1 while tiles i + 1 .. i + NST wait
  // in registers: st[i % NST] holds tile i + 1 at step i and is refilled with
  // tile i + 1 + NST once it has gone to LDS.
  constexpr int NST = 4;
  const int ntile = (nu + KT - 1) / KT;
  v4i st[NST];
  if (ld && ntile > 0) swrite(0, gload(0));
#pragma unroll
  for (int k = 0; k < NST; ++k) st[k] = ld && k + 1 < ntile ? gload((k + 1) * KT) : v4i{0, 0, 0, 0};
  __syncthreads();
  for (int i0 = 0; i0 < ntile; i0 += NST) {
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const int i = i0 + k;
    if (i >= ntile) break;
    const int buf = i & 1;
    const int kb = i * KT;
    unsigned vmask = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int uv = kb + 4 * grp + v;
      const int pv = uv < nsl ? uv : uv + shift;
      const bool in = cval && uv < nu && (pv < cns || (pv >= cws && pv <= ct));
      vmask |= (in ? 1u : 0u) << v;
    }
    if (__builtin_amdgcn_ballot_w64(vmask != 0) != 0) {   // wave-uniform
      // S^T[key][column]: lane l holds K row l % 16, elements 32 kk + 8 (l / 16) ..
      const char* kr = klds[buf] + hl * VROW + 16 * grp;
      v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sc = mfma_bf16_16x16x32(*reinterpret_cast<const v8bf*>(kr + 64 * kk), qb(kk), sc);
      // online softmax of column hl over keys 4*grp + v, the reference max
      // moving only past kLazy of headroom (as in tile_compute)
      float sv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[v] = (vmask >> v) & 1u ? sc[v] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[v]);
      }
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + kLazy) != 0) {
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float av = __shfl(alpha, 4 * grp + v);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][v] *= av;
        }
      }
      v4s phi, plo;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pr = exp2f(sv[v] - m_run);
        l_run += pr;
        const uint32_t hb = f32_to_bf16_bits(pr);
        phi[v] = (short)hb;
        plo[v] = (short)f32_to_bf16_bits(pr - bf16_bits_to_f32(hb));
      }
      // O += P V, V^T operand read key-major from the shared tile
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const char* vp = vlds[buf] + (4 * grp) * VROW + (16 * nb + hl) * 2;
        v4s vb;
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[e] = *reinterpret_cast<const short*>(vp + e * VROW);
        o[nb] = mfma_bf16_16x16x16(phi, vb, o[nb]);
        o[nb] = mfma_bf16_16x16x16(plo, vb, o[nb]);
      }
    }
    // buffer buf ^ 1 was last read in the previous step, before its barrier
    if (ld && i + 1 < ntile) swrite(buf ^ 1, st[k]);
    if (ld && i + 1 + NST < ntile) st[k] = gload((i + 1 + NST) * KT);
    __syncthreads();
  }
  }

  l_run = finish_l(l_run);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const float lh = __shfl(l_run, col);
    const float mh = __shfl(m_run, col);
    const int j = col / G, h = col % G;
    if (j >= nqw) continue;
    const int64_t pr = (int64_t)(q0 + j) * a.Hq + (int64_t)g * G + h;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a.part_o[pr * D + 16 * nb + hl] = o[nb][v];
    if (hl == 0) { a.part_ml[2 * pr] = mh; a.part_ml[2 * pr + 1] = lh; }
  }
}

// ---- grouped long-range attention ----
// Queries with similar selections share most of their long-range keys (the
// select writes a row's best bucket first, so equal first keys mean the same
// best bucket).  The queries are sorted by (first long-range key, MinHash of
// the row, index) and taken qpw at a time; each group's long-range rows are merged into one list
// with a mask of the queries that selected each row, so a shared K/V row is
// read once per group instead of once per query.  The sinks and window are
// attended separately, in position order (k_attn_swin), and the grouped
// kernel starts each query's softmax state from that partial result.

// Long-range entries of a row: the select's rows end with the sinks and window.
__device__ __forceinline__ int long_range_count(const AttnArgs& a, int q) {
  const int t = (int)a.qpos0 + q;
  const int ws = max(0, t - a.window + 1);
  const int nfix = max(0, min(a.sinks, ws)) + (t - ws + 1);
  return max(0, min(a.cnt[q], a.max_sel) - nfix);
}

// Sort key of query q, one wave per query: (first long-range key, MinHash of
// the row, q) packed as 28 + 16 + 20 bits when the chunk has fewer than 2^20
// queries (the MinHash - the smallest of a fixed 32-bit mix over the row's
// pooled-group ids - puts rows with the same best bucket and more keys in
// common next to each other), else (first key, q) as 32 + 32 bits.  Rows
// without long-range keys take first key 2^28 - 1; padding sorts last.
constexpr int kGrpMhBits = 20;         // query bits of the MinHash key
__device__ __forceinline__ unsigned grp_mix(unsigned x) {
  x *= 0x9E3779B1u;
  x ^= x >> 15;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  return x;
}
__global__ void __launch_bounds__(256) k_grp_key(AttnArgs a, unsigned long long* keys, int n_pad,
                                                 int use_mh) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (q >= n_pad) return;
  unsigned long long k = ~0ull;
  if (q < a.nq) {
    const int nlr = long_range_count(a, q);
    const int32_t* row = a.idx + (int64_t)q * a.max_sel;
    const int kmax = (int)(a.kv_rows - 1);
    const unsigned first = nlr > 0 ? (unsigned)min(max(row[0], 0), kmax) : (1u << 28) - 1;
    if (use_mh) {
      unsigned m = 0xffffffffu;
      for (int e = lane; e < nlr; e += 64) m = min(m, grp_mix((unsigned)min(max(row[e], 0), kmax) >> 2));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) m = min(m, (unsigned)__shfl_xor((int)m, o));
      k = ((unsigned long long)first << 36) | ((unsigned long long)(m >> 16) << kGrpMhBits) | (unsigned)q;
    } else {
      k = ((unsigned long long)first << 32) | (unsigned)q;
    }
  }
  if (lane == 0) keys[q] = k;
}

// Ascending bitonic sort of each run of GS_TILE keys (GS_T threads, two each).
constexpr int GS_T = 1024, GS_TILE = 2 * GS_T;
__global__ void __launch_bounds__(GS_T) k_grp_sort_tile(unsigned long long* keys) {
  __shared__ unsigned long long s[GS_TILE];
  unsigned long long* base = keys + (int64_t)blockIdx.x * GS_TILE;
  const int tid = threadIdx.x;
  s[tid] = base[tid];
  s[tid + GS_T] = base[tid + GS_T];
  __syncthreads();
  for (int k = 2; k <= GS_TILE; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < GS_TILE; i += GS_T) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = s[i], y = s[ixj];
          if ((x > y) == ((i & k) == 0)) { s[i] = y; s[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
  base[tid] = s[tid];
  base[tid + GS_T] = s[tid + GS_T];
}

// Merge sorted runs of w keys pairwise into runs of 2w: a key's output slot
// is its index in its run plus the number of keys of the partner run that go
// before it (smaller ones; for the right run also equal ones, so equal keys
// such as the padding keep distinct slots).
__global__ void k_grp_merge(const unsigned long long* in, unsigned long long* out, int n, int w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int r = i / w, o = i % w;
  const bool right = r & 1;
  const unsigned long long x = in[i];
  const unsigned long long* other = in + (int64_t)(r ^ 1) * w;
  int lo = 0, hi = w;
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    if (other[m] < x || (right && other[m] == x)) lo = m + 1; else hi = m;
  }
  out[(int64_t)(r & ~1) * w + o + lo] = x;
}

__global__ void k_grp_perm(const unsigned long long* keys, int32_t* perm, int nq, int use_mh) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const unsigned long long qmask = use_mh ? (1ull << kGrpMhBits) - 1 : 0xffffffffull;
  if (i < nq) perm[i] = (int32_t)(keys[i] & qmask);
}

// ---- grouping by latent neighbours ----
// Queries whose latent vectors lie close together score the index alike and
// take much the same buckets.  Given the chunk's query latents (int8 [nq][64]),
// each query's nearest other query by squared distance within its block of
// kNnBlock consecutive queries is found -- the j != i maximising
// 2 x_i.x_j - |x_j|^2, exact in int32, ties to the lowest j -- and the
// components of that nearest-neighbour graph become the sort's classes.
// Distances are symmetric and ties go to the lowest index, so the graph has no
// cycle longer than two: each component is a tree hanging off one mutual pair,
// found by pointer jumping (p <- p[p], ceil(log2 nq) + 1 rounds reach the pair
// from any depth) and named by the pair's lower index.  The sort key is then
// (first long-range key of that root >> 4, root, q) in 24 + 20 + 20 bits: a
// component's queries sit together, components with the same best bucket next
// to each other.

// -|x_i|^2 for i < nq, 0 up to the next multiple of 16
__global__ void k_grp_nrm(const int8_t* lq, int nq, int n16, int32_t* nnrm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n16) return;
  int acc = 0;
  if (i < nq) {
    const int* r = reinterpret_cast<const int*>(lq + (int64_t)i * 64);
#pragma unroll
    for (int d = 0; d < 16; ++d) acc = __builtin_amdgcn_sdot4(r[d], r[d], acc, false);
  }
  nnrm[i] = -acc;
}

// One wave per (64 queries, candidate range): int8 MFMAs 16x16x64 with 16
// candidates as A (lane l: candidate l % 16, bytes 16 (l / 16) ..) and 16
// queries as B, so lane l holds the dot products of candidates 4 (l / 16) + v
// with query l % 16 of each block.  A score s = 2 x_i.x_j - |x_j|^2 lies in
// (-2^22, 2^20), so (s << 9 | 511 - loc) fits an int32, where loc = 4 tile + v
// numbers the lane's candidates within a chunk of up to 128 tiles: a plain
// max then keeps the best score and, of equal ones, the lowest candidate.
// The next tile's loads are issued before the current tile's MFMAs; the
// range's best goes to part[range][i], packed so that the larger word is
// better (score, then lower j); 0 when the range holds no other query.
constexpr int NN_QW = 64;
constexpr int NN_CHUNK = 128;
constexpr int kNnBlock = 32768;       // a multiple of NN_QW; its pointers fill 128 KiB of LDS
__global__ void __launch_bounds__(256) k_grp_nn(const int8_t* lq, const int32_t* nnrm, int nq, int nrange,
                                                int csz, unsigned long long* part) {
  const int lane = lane_id();
  const int hl = lane & 15, grp = lane >> 4;
  const int nqb = (nq + NN_QW - 1) / NN_QW;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= nqb * nrange) return;
  const int qb = item % nqb, rg = item / nqb;     // a workgroup's waves share the range
  const int i0 = qb * NN_QW;
  const int base = i0 / kNnBlock * kNnBlock;      // the wave's queries' block
  v4i bq[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int i = i0 + 16 * b + hl;
    bq[b] = i < nq ? *reinterpret_cast<const v4i*>(lq + (int64_t)i * 64 + 16 * grp) : v4i{0, 0, 0, 0};
  }
  auto load_a = [&](int j0) -> v4i {
    const int jr = j0 + hl;
    return jr < nq ? *reinterpret_cast<const v4i*>(lq + (int64_t)jr * 64 + 16 * grp) : v4i{0, 0, 0, 0};
  };
  auto load_n = [&](int j0) -> v4i {     // nnrm holds a multiple of 16 entries
    return *reinterpret_cast<const v4i*>(nnrm + j0 + 4 * grp);
  };
  int bs[4], bj[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) { bs[b] = INT_MIN; bj[b] = -1; }
  const int jb = base + rg * csz, je = min(min(nq, base + kNnBlock), jb + csz);
  for (int c0 = jb; c0 < je; c0 += 16 * NN_CHUNK) {
    const int ce = min(je, c0 + 16 * NN_CHUNK);
    int pk[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
    v4i ca = load_a(c0), nv = load_n(c0);
    for (int j0 = c0; j0 < ce; j0 += 16) {
      const int jn = j0 + 16 < ce ? j0 + 16 : j0;
      const v4i ca_n = load_a(jn), nv_n = load_n(jn);
      const int low0 = 511 - 4 * ((j0 - c0) >> 4);
      // the tile crosses the range's end or holds one of the wave's queries
      const bool edge = j0 + 16 > je || (j0 < i0 + NN_QW && j0 + 16 > i0);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v4i c = mfma_i8_16x16x64(ca, bq[b], v4i{0, 0, 0, 0});
        const int i = i0 + 16 * b + hl;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int sc = 2 * c[v] + nv[v];
          int pv = (int)(((unsigned)sc << 9) | (unsigned)(low0 - v));
          if (edge) {
            const int j = j0 + 4 * grp + v;
            pv = j < je && j != i ? pv : INT_MIN;
          }
          pk[b] = max(pk[b], pv);
        }
      }
      ca = ca_n;
      nv = nv_n;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {          // chunks ascend: a strictly better score wins
      if (pk[b] == INT_MIN) continue;
      const int sc = pk[b] >> 9, loc = 511 - (pk[b] & 511);
      if (bj[b] < 0 || sc > bs[b]) { bs[b] = sc; bj[b] = c0 + (loc >> 2) * 16 + 4 * grp + (loc & 3); }
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const int os = __shfl_xor(bs[b], o), oj = __shfl_xor(bj[b], o);
      if (oj >= 0 && (bj[b] < 0 || os > bs[b] || (os == bs[b] && oj < bj[b]))) { bs[b] = os; bj[b] = oj; }
    }
    const int i = i0 + 16 * b + hl;
    if (grp == 0 && i < nq)
      part[(int64_t)rg * nq + i] =
          bj[b] < 0 ? 0ull
                    : ((unsigned long long)((unsigned)bs[b] ^ 0x80000000u) << 32) | (0xffffffffu - (unsigned)bj[b]);
  }
}

// nearest neighbour over the ranges (itself when there is no other query),
// and the first pointer of the jumps
__global__ void k_grp_nn_fin(const unsigned long long* part, int nq, int nrange, int32_t* nn, int32_t* p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nq) return;
  unsigned long long best = 0;
  for (int r = 0; r < nrange; ++r) best = max(best, part[(int64_t)r * nq + i]);
  const int j = best ? (int)(0xffffffffu - (unsigned)(best & 0xffffffffull)) : i;
  nn[i] = j;
  p[i] = j;
}

// pointer jumping, one workgroup per block of kNnBlock queries (the graph's
// edges stay inside a block), the block's pointers in LDS: a pointer updated
// in place only ever moves further along its chain, so each round still at
// least doubles the reach, and 2^rounds >= 2 n reaches the pair from any depth
__global__ void __launch_bounds__(1024) k_grp_jump(int32_t* p, int nq) {
  __shared__ int32_t s[kNnBlock];
  const int base = blockIdx.x * kNnBlock;
  const int n = min(kNnBlock, nq - base);
  for (int i = threadIdx.x; i < n; i += 1024) s[i] = min(max(p[base + i] - base, 0), n - 1);
  __syncthreads();
  for (int reach = 1; reach < 2 * n; reach *= 2) {
    for (int i = threadIdx.x; i < n; i += 1024) s[i] = s[s[i]];
    __syncthreads();
  }
  for (int i = threadIdx.x; i < n; i += 1024) p[base + i] = base + s[i];
}

// sort key (first long-range key of the root >> 4, root, q); padding last
__global__ void k_grp_key_nn(AttnArgs a, const int32_t* nn, const int32_t* p, unsigned long long* keys,
                             int n_pad) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_pad) return;
  unsigned long long k = ~0ull;
  if (q < a.nq) {
    const int pq = min(max(p[q], 0), a.nq - 1);
    const int root = min(pq, min(max(nn[pq], 0), a.nq - 1));
    const int nlr = long_range_count(a, root);
    const int kmax = (int)(a.kv_rows - 1);
    const unsigned first = nlr > 0 ? (unsigned)min(max(a.idx[(int64_t)root * a.max_sel], 0), kmax) : (1u << 28) - 1;
    k = ((unsigned long long)(first >> 4) << 40) | ((unsigned long long)root << kGrpMhBits) | (unsigned)q;
  }
  keys[q] = k;
}

// Union of a group's long-range rows, one workgroup of GU_T threads per
// group.  An LDS hash set (linear probing) holds word (key << 4 | mask), one
// mask bit per query slot of the group.  The group's QP queries are taken
// one after another: a key already in the set gets the query's bit, a new
// key is inserted with it and appended to the union at the next free
// position (a block scan keeps row order), so the union is the first query's
// row, then the second's new keys, ... - the same order on every call.  A
// row holds a key at most once, so all of one query's entries are probed at
// once without two of them racing for the same key; the slots that colliding
// keys land in may vary, the set's contents and the union's order do not.
// TS: table slots, >= 2 x QP x lcap; thread t holds entries t*EPT .. +EPT-1
// of each row (EPT x GU_T >= lcap).  A group with a row over the cap gets
// ucnt = -1 and is walked row by row instead.
constexpr int GU_T = 1024;
template <int TS, int QP>
__global__ void __launch_bounds__(GU_T) k_grp_union(AttnArgs a, int lcap, int32_t* urow,
                                                    uint8_t* umask, int32_t* ucnt) {
  constexpr unsigned EMPTY = 0xffffffffu;
  constexpr int LOG_TS = __builtin_ctz(TS);
  constexpr int EPT = TS / (2 * GU_T * QP) > 0 ? TS / (2 * GU_T * QP) : 1;
  __shared__ unsigned tab[TS];
  __shared__ int red[GU_T / 64];
  const int tid = threadIdx.x;
  const int gi = blockIdx.x;
  int qs[QP], nl[QP];
  bool over = false;
#pragma unroll
  for (int j = 0; j < QP; ++j) {
    const int slot = gi * QP + j;
    const bool in = slot < a.nq;
    qs[j] = in ? a.perm[slot] : 0;
    nl[j] = in ? long_range_count(a, qs[j]) : 0;
    over |= nl[j] > lcap;
  }
  if (over) {                          // block-uniform
    if (tid == 0) ucnt[gi] = -1;
    return;
  }
  // every entry first, all loads in flight at once
  int ent[QP][EPT];
#pragma unroll
  for (int j = 0; j < QP; ++j) {
    const int32_t* row = a.idx + (int64_t)qs[j] * a.max_sel;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      ent[j][i] = e < nl[j] ? min(max(row[e], 0), (int)(a.kv_rows - 1)) : -1;
    }
  }
  {
    const uint4 e4 = {EMPTY, EMPTY, EMPTY, EMPTY};
    for (int i = tid; i < TS / 4; i += GU_T) reinterpret_cast<uint4*>(tab)[i] = e4;
  }
  __syncthreads();

  int32_t* ur = urow + (int64_t)gi * a.ucap;
  uint8_t* um = umask + (int64_t)gi * a.ucap;
  int own_slot[QP][EPT], own_pos[QP][EPT];    // this thread's appended keys
  int nu = 0;                                   // union length so far (block-uniform)
#pragma unroll
  for (int j = 0; j < QP; ++j) {
    const unsigned bit = 1u << j;
    int fresh = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      own_slot[j][i] = -1;
      if (ent[j][i] < 0) continue;
      const unsigned key = (unsigned)ent[j][i];
      unsigned h = (key * 0x9E3779B1u) >> (32 - LOG_TS);
      for (;;) {                       // ends: the table is at most half full
        const unsigned w = tab[h];
        if (w != EMPTY && (w >> 4) == key) { atomicOr(&tab[h], bit); break; }
        if (w == EMPTY) {
          if (atomicCAS(&tab[h], EMPTY, (key << 4) | bit) == EMPTY) {
            own_slot[j][i] = (int)h;
            ++fresh;
            break;
          }
          continue;                    // another key took the slot: look at it again
        }
        h = (h + 1) & (TS - 1);
      }
    }
    int tot;
    int pos = nu + sel::block_excl_scan<GU_T>(fresh, red, &tot);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      own_pos[j][i] = pos;
      if (own_slot[j][i] >= 0) ur[pos++] = ent[j][i];
    }
    nu += tot;
  }
  __syncthreads();                     // every bit is in the table
#pragma unroll
  for (int j = 0; j < QP; ++j)
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (own_slot[j][i] >= 0) um[own_pos[j][i]] = (uint8_t)(tab[own_slot[j][i]] & 15u);
  if (tid == 0) ucnt[gi] = nu;
}

// One wave per (group, KV head): the group's qpw queries x G heads are the
// 16 columns; the state starts from the sinks-and-window partial, then the
// union rows are walked once, each column masked to the rows its query took.
// GW waves per workgroup (4: a group's KV heads in two workgroups, which
// measured 1.4% faster than all 8 in one); with kGrpPipe the next tile's
// loads are in flight during the current tile's MFMAs (168 VGPRs, 3 waves per
// SIMD: no faster, so off).
constexpr int GW = 4;
constexpr bool kGrpPipe = false;
constexpr int GWAVES = kGrpPipe ? 3 : 4;   // waves per SIMD the registers allow
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(GW * 64, GWAVES) k_attn_grp(AttnArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int VROW = D * 2 + 16;
  __shared__ __attribute__((aligned(16))) char vlds[GW][KT * VROW];
  __shared__ __attribute__((aligned(16))) char qlds[GW][16 * qrow_bytes(D)];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nwg = gridDim.x;
  const int item = xcd_remap(blockIdx.x, nwg) * GW + wave;
  const int QPW = a.qpw;
  const int ngrp = (a.nq + QPW - 1) / QPW;
  if (item >= ngrp * a.Hkv) return;
  const int g = item % a.Hkv;
  const int gi = item / a.Hkv;
  const int G = a.G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  // this lane's column: query slot jc of the group, head hc of the KV group
  const int jc = hl / G, hc = hl % G;
  const int slot = gi * QPW + jc;
  const bool cval = jc < QPW && slot < a.nq;
  // the plan comes from the workspace: its order and counts are clamped, so a
  // walk on a workspace no prepare wrote reads nothing out of bounds
  const int qc = cval ? min(max(a.perm[slot], 0), a.nq - 1) : 0;

  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int64_t rmax = a.kv_rows - 1;

  char* ql = qlds[wave];
  {
    const uint16_t* qp = a.q + ((int64_t)qc * a.Hq + (int64_t)g * G + hc) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = cval ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(ql + hl * qrow_bytes(D) + (32 * kk + 8 * grp) * 2) = raw;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const QLds<D> qb{ql + hl * qrow_bytes(D) + 16 * grp};

  // state of the sinks and window: o for columns 4*grp + v, (m, l) for column hl
  v4f o[NB];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const int qv = __shfl(qc, col);
    const bool vv = __shfl((int)cval, col) != 0;
    const int64_t pr = (int64_t)qv * a.Hq + (int64_t)g * G + col % G;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb][v] = vv ? a.part_o[pr * D + 16 * nb + hl] : 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  if (cval) {
    const int64_t pr = (int64_t)qc * a.Hq + (int64_t)g * G + hc;
    m_run = a.part_ml[2 * pr];
    l_run = grp == 0 ? a.part_ml[2 * pr + 1] : 0.f;   // the lanes' partial sums are added at the end
  }

  char* vl = vlds[wave];
  const uint16_t* kbase = a.k + (int64_t)g * D;
  const uint16_t* vbase = a.v + (int64_t)g * D;
  const int nu = min(a.ucnt[gi], a.ucap);
  if (nu >= 0) {
    const int32_t* ur = a.urow + (int64_t)gi * a.ucap;
    const uint8_t* um = a.umask + (int64_t)gi * a.ucap;
    auto row_of = [&](int kb) -> int {
      const int sl = kb + hl;
      const int r = sl < nu ? ur[sl] : 0;
      return (int)min((int64_t)max(r, 0), rmax);
    };
    auto mask_of = [&](int kb) -> unsigned {
      // masks of union rows kb + 4 grp .. +3 (ucap is a multiple of 4)
      const int k4 = kb + 4 * grp;
      const unsigned m4 = k4 < nu ? *reinterpret_cast<const unsigned*>(um + k4) : 0u;
      unsigned vmask = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool in = cval && k4 + v < nu && ((m4 >> (8 * v + jc)) & 1u);
        vmask |= (in ? 1u : 0u) << v;
      }
      return vmask;
    };
    if (kGrpPipe) {
      TileRegs<D> T0, T1;
      if (nu > 0) tile_load<D>(T0, kbase, vbase, rowstride, row_of(0));
      int kb = 0;
      for (; kb + KT < nu; kb += 2 * KT) {
        tile_load<D>(T1, kbase, vbase, rowstride, row_of(kb + KT));
        tile_compute<D>(qb, T0, mask_of(kb), a.scale_log2, vl, o, m_run, l_run);
        if (kb + 2 * KT < nu) tile_load<D>(T0, kbase, vbase, rowstride, row_of(kb + 2 * KT));
        tile_compute<D>(qb, T1, mask_of(kb + KT), a.scale_log2, vl, o, m_run, l_run);
      }
      if (kb < nu) tile_compute<D>(qb, T0, mask_of(kb), a.scale_log2, vl, o, m_run, l_run);
    } else {
      for (int kb = 0; kb < nu; kb += KT)
        attn_tile<D>(qb, kbase, vbase, rowstride, row_of(kb), mask_of(kb), a.scale_log2, vl, o, m_run,
                     l_run);
    }
  } else {
    // a row over the union cap: each query's long-range keys in turn
    for (int j = 0; j < QPW; ++j) {
      const int sl = gi * QPW + j;
      if (sl >= a.nq) break;
      const int q = min(max(a.perm[sl], 0), a.nq - 1);
      const int nlr = long_range_count(a, q);
      const int32_t* idxrow = a.idx + (int64_t)q * a.max_sel;
      const bool mine = cval && jc == j;
      for (int kb = 0; kb < nlr; kb += KT) {
        const int slot = kb + hl;
        int r = slot < nlr ? idxrow[slot] : 0;
        r = (int)min((int64_t)max(r, 0), rmax);
        unsigned vmask = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) vmask |= (mine && kb + 4 * grp + v < nlr ? 1u : 0u) << v;
        attn_tile<D>(qb, kbase, vbase, rowstride, r, vmask, a.scale_log2, vl, o, m_run, l_run);
      }
    }
  }

  l_run = finish_l(l_run);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int col = 4 * grp + v;
    const float lh = __shfl(l_run, col);
    const float mh = __shfl(m_run, col);
    const int qv = __shfl(qc, col);
    const bool vv = __shfl((int)cval, col) != 0;
    if (!vv) continue;
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    const int64_t ob = ((int64_t)qv * a.Hq + (int64_t)g * G + col % G) * D;
    // log-sum-exp: m_run and l_run are in the log2 domain of the scaled logits
    if (a.lse && hl == 0) a.lse[(int64_t)qv * a.Hq + (int64_t)g * G + col % G] =
        (mh + __log2f(lh)) * 0.6931471805599453f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float val = o[nb][v] * inv;
      if (OUT_F32) reinterpret_cast<float*>(a.out)[ob + 16 * nb + hl] = val;
      else reinterpret_cast<uint16_t*>(a.out)[ob + 16 * nb + hl] = (uint16_t)f32_to_bf16_bits(val);
    }
  }
}

// Decode: split-K attention.  A wave owns one split of one (sequence, KV
// head), the workgroup's waves the KV heads of one (sequence, split); its row ids for up to MAXT tiles are fetched at once (entry e in
// lane e % 64 of register e / 64) and the next tile's K/V loads are issued
// before the current tile's MFMAs, so a split costs about one memory round
// trip plus its tiles' compute.  The split's unnormalised result and its
// (max, sum) per head go to the workspace for k_attn_merge.
constexpr int MAXT = 16;
constexpr bool kDecPipe = true;     // next tile's loads in flight during the current tile

template <int D, bool PIPE>
__global__ void __launch_bounds__(AT) k_attn_dec(AttnArgs a) {
  constexpr int NKK = D / 32;
  constexpr int NB = D / 16;
  constexpr int VROW = D * 2 + 16;
  constexpr int NRID = MAXT * KT / 64;
  __shared__ __attribute__((aligned(16))) char vlds[AW][KT * VROW];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int item = xcd_remap(blockIdx.x, gridDim.x) * AW + wave;
  if (item >= a.nq * a.Hkv * a.splits) return;
  // the 8 waves of a workgroup take the KV heads of one (query, split), so
  // every 2 KiB K/V row is fetched by one workgroup at once
  const int g = item % a.Hkv;
  const int split = (item / a.Hkv) % a.splits;
  const int q = item / (a.Hkv * a.splits);
  const int64_t pitem = ((int64_t)q * a.Hkv + g) * a.splits + split;   // partial-result slot
  const int G = a.G;
  const int hl = lane & 15;
  const int grp = lane >> 4;

  const int cnt = min(a.cnt[q], a.max_sel);
  const int ch = ((cnt + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kbeg = min(cnt, split * ch);
  const int kend = min(cnt, kbeg + ch);
  const int64_t rowbase = (int64_t)(q / a.qdiv) * a.seq_stride_rows;
  const int64_t rowstride = (int64_t)a.Hkv * D;
  const int32_t* idxrow = a.idx + (int64_t)q * a.max_sel;
  const int64_t rmax = a.kv_rows - 1;

  int rid[NRID];
#pragma unroll
  for (int j = 0; j < NRID; ++j) {
    const int slot = kbeg + lane + 64 * j;
    const int r = slot < kend ? idxrow[slot] : 0;
    rid[j] = (int)min((int64_t)max(r, 0), rmax);
  }
  auto row_of = [&](int i) -> int {   // this lane's key row of tile i
    if (i < MAXT) {
      const int j = i >> 2;
      const int v = j == 0 ? rid[0] : j == 1 ? rid[1] : j == 2 ? rid[2] : rid[3];
      return __shfl(v, (i & 3) * 16 + hl);
    }
    const int slot = kbeg + i * KT + hl;
    const int r = slot < kend ? idxrow[slot] : 0;
    return (int)min((int64_t)max(r, 0), rmax);
  };
  auto mask_of = [&](int i) -> unsigned {
    unsigned m = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) m |= (kbeg + i * KT + 4 * grp + v < kend ? 1u : 0u) << v;
    return m;
  };

  QRegs<D> qb;
  {
    const bool hv = hl < G;
    const uint16_t* qp = a.q + ((int64_t)q * a.Hq + (int64_t)g * G + (hv ? hl : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = hv ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      qb.b[kk] = __builtin_bit_cast(v8bf, raw);
    }
  }
  v4f o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  char* vl = vlds[wave];
  const uint16_t* kbase = a.k + (rowbase * a.Hkv + g) * D;
  const uint16_t* vbase = a.v + (rowbase * a.Hkv + g) * D;

  const int ntl = (kend - kbeg + KT - 1) / KT;
  if (PIPE) {
    TileRegs<D> T0, T1;
    if (ntl > 0) tile_load<D>(T0, kbase, vbase, rowstride, row_of(0));
    int i = 0;
    for (; i + 1 < ntl; i += 2) {
      tile_load<D>(T1, kbase, vbase, rowstride, row_of(i + 1));
      tile_compute<D>(qb, T0, mask_of(i), a.scale_log2, vl, o, m_run, l_run);
      if (i + 2 < ntl) tile_load<D>(T0, kbase, vbase, rowstride, row_of(i + 2));
      tile_compute<D>(qb, T1, mask_of(i + 1), a.scale_log2, vl, o, m_run, l_run);
    }
    if (i < ntl) tile_compute<D>(qb, T0, mask_of(i), a.scale_log2, vl, o, m_run, l_run);
  } else {
    for (int i = 0; i < ntl; ++i) {
      TileRegs<D> T0;
      tile_load<D>(T0, kbase, vbase, rowstride, row_of(i));
      tile_compute<D>(qb, T0, mask_of(i), a.scale_log2, vl, o, m_run, l_run);
    }
  }

  // this split's partial result: [slot][G][D] and (max, sum) per head
  float* po = a.part_o + pitem * G * D;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * grp + v;
    if (h >= G) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) po[h * D + 16 * nb + hl] = o[nb][v];
  }
  l_run = finish_l(l_run);
  if (grp == 0) {
    a.part_ml[pitem * 32 + 2 * hl] = m_run;
    a.part_ml[pitem * 32 + 2 * hl + 1] = l_run;
  }
}

// Combine the splits of each (query, head): one wave per head row.  Lane s
// holds split s's (max, sum), the wave reduces the common max and the
// denominator, then every lane sums its D/64 output dims over the splits
// with the weights broadcast from their lanes (loads in flight together).
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(256) k_attn_merge(AttnArgs a) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // q * Hq + head
  if (row >= a.nq * a.Hq) return;
  const int q = row / a.Hq, head = row % a.Hq;
  const int g = head / a.G, h = head % a.G;
  const int64_t it0 = ((int64_t)q * a.Hkv + g) * a.splits;
  const int S = a.splits;                                  // <= 64
  float ms = -INFINITY, ls = 0.f;
  if (lane < S) {
    ms = a.part_ml[(it0 + lane) * 32 + 2 * h];
    ls = a.part_ml[(it0 + lane) * 32 + 2 * h + 1];
  }
  float M = ls > 0.f ? ms : -INFINITY;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
  const float w = (ls > 0.f) ? exp2f(ms - M) : 0.f;
  float den = ls * w;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m);
  const float* po = a.part_o + (it0 * a.G + h) * D + lane;
  float num[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) num[c] = 0.f;
  // 16 splits' partial rows in flight at once, then their weighted sum
  for (int s0 = 0; s0 < S; s0 += 16) {
    float pv[16][D / 64];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
        pv[j][c] = s0 + j < S ? po[(int64_t)(s0 + j) * a.G * D + 64 * c] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float ws = __shfl(w, s0 + j);
#pragma unroll
      for (int c = 0; c < D / 64; ++c) num[c] += pv[j][c] * ws;
    }
  }
  const int64_t ob = (int64_t)row * D + lane;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    const float val = den > 0.f ? num[c] / den : 0.f;
    if (OUT_F32) reinterpret_cast<float*>(a.out)[ob + 64 * c] = val;
    else reinterpret_cast<uint16_t*>(a.out)[ob + 64 * c] = (uint16_t)f32_to_bf16_bits(val);
  }
}

}  // namespace

size_t attn_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t items = (size_t)nq * ap.Hkv * splits;
  return items * 16 * ap.D * sizeof(float) + items * 32 * sizeof(float);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t kv_rows,
                       int64_t seq_stride_rows, int32_t qdiv, const int32_t* idx,
                       const int32_t* cnt, int32_t max_sel, int32_t nq, const lsa_attn_params& ap,
                       void* out, void* ws, int32_t splits, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.kv_rows = kv_rows; a.seq_stride_rows = seq_stride_rows;
  a.qdiv = qdiv > 0 ? qdiv : 1;
  a.idx = idx; a.cnt = cnt; a.max_sel = max_sel; a.nq = nq;
  a.Hq = ap.Hq; a.Hkv = ap.Hkv; a.G = ap.Hq / ap.Hkv;
  a.splits = splits > 1 ? splits : 1;
  const float scale = ap.scale > 0.f ? ap.scale : 1.0f / sqrtf((float)ap.D);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  const size_t items = (size_t)nq * ap.Hkv * a.splits;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = a.part_o ? a.part_o + items * 16 * ap.D : nullptr;
  const unsigned grid = (unsigned)((items + AW - 1) / AW);
  const bool f32 = ap.out_f32 != 0;
  if (a.splits > 1) {
    if (a.splits > 64) return hipErrorInvalidValue;
    if (ap.D == 128) hipLaunchKernelGGL((k_attn_dec<128, kDecPipe>), dim3(grid), dim3(AT), 0, s, a);
    else hipLaunchKernelGGL((k_attn_dec<64, kDecPipe>), dim3(grid), dim3(AT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned mg = (unsigned)((nq * ap.Hq + 3) / 4);
    if (ap.D == 128) {
      if (f32) hipLaunchKernelGGL((k_attn_merge<128, true>), dim3(mg), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_attn_merge<128, false>), dim3(mg), dim3(256), 0, s, a);
    } else {
      if (f32) hipLaunchKernelGGL((k_attn_merge<64, true>), dim3(mg), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_attn_merge<64, false>), dim3(mg), dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  if (ap.D == 128) {
    if (f32) hipLaunchKernelGGL((k_attn<128, true>), dim3(grid), dim3(AT), 0, s, a);
    else hipLaunchKernelGGL((k_attn<128, false>), dim3(grid), dim3(AT), 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((k_attn<64, true>), dim3(grid), dim3(AT), 0, s, a);
    else hipLaunchKernelGGL((k_attn<64, false>), dim3(grid), dim3(AT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              int64_t kv_rows, const int32_t* idx, const int32_t* cnt,
                              int32_t max_sel, int32_t nq, int64_t qpos0, int32_t window,
                              int32_t sinks, const lsa_attn_params& ap, void* out, float* lse,
                              hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.kv_rows = kv_rows; a.seq_stride_rows = 0; a.qdiv = 1;
  a.idx = idx; a.cnt = cnt; a.max_sel = max_sel; a.nq = nq;
  a.Hq = ap.Hq; a.Hkv = ap.Hkv; a.G = ap.Hq / ap.Hkv;
  a.splits = 1;
  const float scale = ap.scale > 0.f ? ap.scale : 1.0f / sqrtf((float)ap.D);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.qpos0 = qpos0; a.window = window; a.sinks = sinks;
  a.qpw = 16 / a.G;
  a.lse = lse;
  const size_t items = (size_t)((nq + a.qpw - 1) / a.qpw) * ap.Hkv;
  const unsigned grid = (unsigned)((items + AW - 1) / AW);
  const bool f32 = ap.out_f32 != 0;
  if (ap.D == 128) {
    if (f32) hipLaunchKernelGGL((k_attn_win<128, true>), dim3(grid), dim3(AT), 0, s, a);
    else hipLaunchKernelGGL((k_attn_win<128, false>), dim3(grid), dim3(AT), 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((k_attn_win<64, true>), dim3(grid), dim3(AT), 0, s, a);
    else hipLaunchKernelGGL((k_attn_win<64, false>), dim3(grid), dim3(AT), 0, s, a);
  }
  return hipGetLastError();
}

namespace {
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr int kGrpMinSort = GS_TILE;
int grp_sort_n(int32_t nq) {
  int n = kGrpMinSort;
  while (n < nq) n <<= 1;
  return n;
}
int grp_table_n(int qpw, int32_t lcap) {    // hash slots: at least twice the entries
  int n = 2048;
  while (n < 2 * qpw * lcap) n <<= 1;
  return n;
}
// The plan (query order and unions) first, then the sinks-and-window partials:
// the backward's dQ uses the plan alone.
struct GrpLayout {
  size_t keys_a, keys_b, perm, urow, umask, ucnt, nrm, nnpart, nn, pa, plan_total, part_o, part_ml,
      total;
  int n_pad, qpw, ngrp, ucap, nrange, csz;
};
GrpLayout grp_layout(int32_t nq, const lsa_attn_params& ap, int32_t lcap) {
  GrpLayout L;
  const int G = ap.Hq / ap.Hkv;
  L.qpw = 16 / G;
  L.n_pad = grp_sort_n(nq);
  L.ngrp = (nq + L.qpw - 1) / L.qpw;
  L.ucap = (L.qpw * lcap + 3) & ~3;
  size_t o = 0;
  L.keys_a = o; o += al256((size_t)L.n_pad * 8);
  L.keys_b = o; o += al256((size_t)L.n_pad * 8);
  L.perm = o; o += al256((size_t)nq * 4);
  L.urow = o; o += al256((size_t)L.ngrp * L.ucap * 4);
  L.umask = o; o += al256((size_t)L.ngrp * L.ucap);
  L.ucnt = o; o += al256((size_t)L.ngrp * 4);
  // the latent nearest-neighbour search: enough candidate ranges per block
  // for about 8192 waves, each range a multiple of 16 candidates
  const int nqb = (nq + NN_QW - 1) / NN_QW;
  L.nrange = std::max(1, std::min(64, (8192 + nqb - 1) / nqb));
  const int nbs = std::min(nq, kNnBlock);
  L.csz = ((nbs + L.nrange - 1) / L.nrange + 15) / 16 * 16;
  L.nrm = o; o += al256((size_t)(nq + 15) / 16 * 16 * 4);
  L.nnpart = o; o += al256((size_t)L.nrange * nq * 8);
  L.nn = o; o += al256((size_t)nq * 4);
  L.pa = o; o += al256((size_t)nq * 4);
  L.plan_total = o;
  L.part_o = o; o += al256((size_t)nq * ap.Hq * ap.D * 4);
  L.part_ml = o; o += al256((size_t)nq * ap.Hq * 2 * 4);
  L.total = o;
  return L;
}

// The query order and the groups' unions (a.idx, a.cnt, a.max_sel, a.nq,
// a.qpos0, a.window, a.sinks, a.kv_rows and a.qpw set; a.perm, a.urow,
// a.umask, a.ucnt and a.ucap are set here).
hipError_t grouped_plan(AttnArgs& a, const GrpLayout& L, char* w, int32_t lcap, const int8_t* latq,
                        hipStream_t s) {
  int32_t* perm = reinterpret_cast<int32_t*>(w + L.perm);
  int32_t* urow = reinterpret_cast<int32_t*>(w + L.urow);
  uint8_t* umask = reinterpret_cast<uint8_t*>(w + L.umask);
  int32_t* ucnt = reinterpret_cast<int32_t*>(w + L.ucnt);
  a.perm = perm;
  a.urow = urow; a.umask = umask; a.ucnt = ucnt; a.ucap = L.ucap;   // the union kernel's stride
  const int nq = a.nq;
  // the order of the queries: sort (first long-range key, MinHash, query)
  unsigned long long* ka = reinterpret_cast<unsigned long long*>(w + L.keys_a);
  unsigned long long* kb = reinterpret_cast<unsigned long long*>(w + L.keys_b);
  const int use_mh = nq < (1 << kGrpMhBits) - 1 ? 1 : 0;
  if (latq && use_mh) {
    // components of the latent nearest-neighbour graph
    const int n16 = (nq + 15) / 16 * 16;
    int32_t* nrm = reinterpret_cast<int32_t*>(w + L.nrm);
    unsigned long long* part = reinterpret_cast<unsigned long long*>(w + L.nnpart);
    int32_t* nn = reinterpret_cast<int32_t*>(w + L.nn);
    int32_t* pa = reinterpret_cast<int32_t*>(w + L.pa);
    hipLaunchKernelGGL(k_grp_nrm, dim3((n16 + 255) / 256), dim3(256), 0, s, latq, nq, n16, nrm);
    const int nqb = (nq + NN_QW - 1) / NN_QW;
    hipLaunchKernelGGL(k_grp_nn, dim3((nqb * L.nrange + 3) / 4), dim3(256), 0, s, latq, nrm, nq, L.nrange,
                       L.csz, part);
    hipLaunchKernelGGL(k_grp_nn_fin, dim3((nq + 255) / 256), dim3(256), 0, s, part, nq, L.nrange, nn, pa);
    hipLaunchKernelGGL(k_grp_jump, dim3((nq + kNnBlock - 1) / kNnBlock), dim3(1024), 0, s, pa, nq);
    hipLaunchKernelGGL(k_grp_key_nn, dim3((L.n_pad + 255) / 256), dim3(256), 0, s, a, nn, pa, ka, L.n_pad);
  } else {
    hipLaunchKernelGGL(k_grp_key, dim3((L.n_pad + 3) / 4), dim3(256), 0, s, a, ka, L.n_pad, use_mh);
  }
  hipLaunchKernelGGL(k_grp_sort_tile, dim3(L.n_pad / GS_TILE), dim3(GS_T), 0, s, ka);
  for (int wd = GS_TILE; wd < L.n_pad; wd <<= 1) {
    hipLaunchKernelGGL(k_grp_merge, dim3((L.n_pad + 255) / 256), dim3(256), 0, s, ka, kb, L.n_pad, wd);
    std::swap(ka, kb);
  }
  hipLaunchKernelGGL(k_grp_perm, dim3((nq + 255) / 256), dim3(256), 0, s, ka, perm, nq, use_mh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the groups' unions of long-range rows
  const int ts = grp_table_n(L.qpw, lcap);
#define LSA_UNION(TS_, QP_) \
  hipLaunchKernelGGL((k_grp_union<TS_, QP_>), dim3(L.ngrp), dim3(GU_T), 0, s, a, lcap, urow, umask, ucnt)
#define LSA_UNION_QP(TS_)                 \
  switch (L.qpw) {                        \
    case 4: LSA_UNION(TS_, 4); break;     \
    case 2: LSA_UNION(TS_, 2); break;     \
    default: LSA_UNION(TS_, 1); break;    \
  }
  switch (ts) {
    case 2048: LSA_UNION_QP(2048); break;
    case 4096: LSA_UNION_QP(4096); break;
    case 8192: LSA_UNION_QP(8192); break;
    case 16384: LSA_UNION_QP(16384); break;
    case 32768: LSA_UNION_QP(32768); break;
    default: return hipErrorInvalidValue;
  }
#undef LSA_UNION_QP
#undef LSA_UNION
  return hipGetLastError();
}
}  // namespace

bool grouped_nq_ok(int64_t nq) { return nq >= 0 && nq <= kGroupedMaxQueries; }

bool grouped_attn_ok(const lsa_attn_params& ap, int32_t lcap, int64_t kv_rows) {
  if (ap.D != 64 && ap.D != 128) return false;
  if (ap.Hkv <= 0 || ap.Hq % ap.Hkv != 0) return false;
  const int G = ap.Hq / ap.Hkv;
  if (G != 4 && G != 8 && G != 16) return false;
  if (lcap < 1 || (16 / G) * (int64_t)lcap > 16384) return false;
  return kv_rows >= 1 && kv_rows < (int64_t)1 << 28;     // key << 4 | mask fits 32 bits
}

size_t attn_grouped_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t lcap) {
  if (nq <= 0 || !grouped_nq_ok(nq)) return 0;
  return grp_layout(nq, ap, lcap).total;
}

size_t grouped_plan_ws_bytes(int32_t nq, const lsa_attn_params& ap, int32_t lcap) {
  if (nq <= 0 || !grouped_nq_ok(nq)) return 0;
  return grp_layout(nq, ap, lcap).plan_total;
}

hipError_t launch_grouped_plan(const int32_t* idx, const int32_t* cnt, int32_t max_sel, int32_t nq,
                               int64_t qpos0, int32_t window, int32_t sinks, int64_t kv_rows,
                               int32_t lcap, const lsa_attn_params& ap, const int8_t* latq, void* ws,
                               GroupPlanView* view, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  if (!grouped_attn_ok(ap, lcap, kv_rows) || !grouped_nq_ok(nq)) return hipErrorInvalidValue;
  const GrpLayout L = grp_layout(nq, ap, lcap);
  char* w = static_cast<char*>(ws);
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.kv_rows = kv_rows; a.idx = idx; a.cnt = cnt; a.max_sel = max_sel; a.nq = nq;
  a.Hq = ap.Hq; a.Hkv = ap.Hkv; a.G = ap.Hq / ap.Hkv;
  a.qpos0 = qpos0; a.window = window; a.sinks = sinks; a.qpw = L.qpw;
  hipError_t e = grouped_plan(a, L, w, lcap, latq, s);
  if (e != hipSuccess) return e;
  view->perm = reinterpret_cast<const int32_t*>(w + L.perm);
  view->urow = reinterpret_cast<const int32_t*>(w + L.urow);
  view->umask = reinterpret_cast<const uint8_t*>(w + L.umask);
  view->ucnt = reinterpret_cast<const int32_t*>(w + L.ucnt);
  view->ucap = L.ucap;
  view->qpw = L.qpw;
  view->ngrp = L.ngrp;
  return hipSuccess;
}

hipError_t launch_attn_grouped(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int64_t kv_rows, const int32_t* idx, const int32_t* cnt,
                               int32_t max_sel, int32_t nq, int64_t qpos0, int32_t window,
                               int32_t sinks, int32_t lcap, const lsa_attn_params& ap,
                               const int8_t* latq, void* out, float* lse, void* ws, int parts,
                               hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  if (!grouped_attn_ok(ap, lcap, kv_rows) || !grouped_nq_ok(nq)) return hipErrorInvalidValue;
  const GrpLayout L = grp_layout(nq, ap, lcap);
  char* w = static_cast<char*>(ws);
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.kv_rows = kv_rows; a.seq_stride_rows = 0; a.qdiv = 1;
  a.idx = idx; a.cnt = cnt; a.max_sel = max_sel; a.nq = nq;
  a.Hq = ap.Hq; a.Hkv = ap.Hkv; a.G = ap.Hq / ap.Hkv;
  a.splits = 1;
  const float scale = ap.scale > 0.f ? ap.scale : 1.0f / sqrtf((float)ap.D);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.qpos0 = qpos0; a.window = window; a.sinks = sinks;
  a.qpw = L.qpw;
  a.lse = nullptr;                     // the partials carry no log-sum-exp; the walk writes it
  a.part_o = reinterpret_cast<float*>(w + L.part_o);
  a.part_ml = reinterpret_cast<float*>(w + L.part_ml);
  int32_t* perm = reinterpret_cast<int32_t*>(w + L.perm);
  int32_t* urow = reinterpret_cast<int32_t*>(w + L.urow);
  uint8_t* umask = reinterpret_cast<uint8_t*>(w + L.umask);
  int32_t* ucnt = reinterpret_cast<int32_t*>(w + L.ucnt);
  a.perm = perm; a.urow = urow; a.umask = umask; a.ucnt = ucnt; a.ucap = L.ucap;
  const unsigned grid = (unsigned)(((size_t)L.ngrp * ap.Hkv + AW - 1) / AW);
  const bool f32 = ap.out_f32 != 0;

  hipError_t e = hipSuccess;
  if (parts & kGroupedPrepare) {
    // 1. sinks and window of every query, in position order, as partials
    const size_t span = (size_t)SW * L.qpw;
    const unsigned sgrid = (unsigned)((nq + span - 1) / span * ap.Hkv);
    if (ap.D == 128) hipLaunchKernelGGL((k_attn_swin<128>), dim3(sgrid), dim3(SW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_attn_swin<64>), dim3(sgrid), dim3(SW * 64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. the query order and the groups' unions
    e = grouped_plan(a, L, w, lcap, latq, s);
    if (e != hipSuccess) return e;
  }
  if (!(parts & kGroupedWalk)) return hipSuccess;
  a.lse = lse;

  // 3. the unions, each column masked to its query's rows, on top of the partials
  const unsigned ggrid = (unsigned)(((size_t)L.ngrp * ap.Hkv + GW - 1) / GW);
  if (ap.D == 128) {
    if (f32) hipLaunchKernelGGL((k_attn_grp<128, true>), dim3(ggrid), dim3(GW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_attn_grp<128, false>), dim3(ggrid), dim3(GW * 64), 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((k_attn_grp<64, true>), dim3(ggrid), dim3(GW * 64), 0, s, a);
    else hipLaunchKernelGGL((k_attn_grp<64, false>), dim3(ggrid), dim3(GW * 64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lsa
