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

#include "lsa_device.h"
#include "lsa_internal.h"

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

template <int D>
__device__ __forceinline__ void tile_compute(const v8bf (&qb)[D / 32], const TileRegs<D>& T,
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
  for (int kk = 0; kk < NKK; ++kk) s = mfma_bf16_16x16x32(T.ka[kk], qb[kk], s);

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

template <int D>
__device__ __forceinline__ void attn_tile(const v8bf (&qb)[D / 32], const uint16_t* kbase,
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
  v8bf qb[NKK];
  {
    const bool hv = hl < G;
    const uint16_t* qp = a.q + ((int64_t)q * a.Hq + (int64_t)g * G + (hv ? hl : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = hv ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      qb[kk] = __builtin_bit_cast(v8bf, raw);
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

  // query operand: column hl = (query q0 + jc, head g*G + hc)
  v8bf qb[NKK];
  {
    const uint16_t* qp = a.q + ((int64_t)(q0 + (cval ? jc : 0)) * a.Hq + (int64_t)g * G + hc) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = cval ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      qb[kk] = __builtin_bit_cast(v8bf, raw);
    }
  }

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

  v8bf qb[NKK];
  {
    const bool hv = hl < G;
    const uint16_t* qp = a.q + ((int64_t)q * a.Hq + (int64_t)g * G + (hv ? hl : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      v4i raw = hv ? *reinterpret_cast<const v4i*>(qp + 32 * kk + 8 * grp) : v4i{0, 0, 0, 0};
      qb[kk] = __builtin_bit_cast(v8bf, raw);
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

}  // namespace lsa
