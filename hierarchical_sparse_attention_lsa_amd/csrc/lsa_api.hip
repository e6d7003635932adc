// Host side of the C ABI declared in include/lsa.h: argument validation,
// arena layout, index bookkeeping (all shape decisions are made on the host
// from T, so no call ever waits on the device) and kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "lsa_internal.h"

using namespace lsa;

namespace lsa {

hipError_t once_per_device(std::atomic<unsigned long long>& done, hipError_t (*set)()) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 64) return set();
  const unsigned long long bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  static std::mutex m;
  std::lock_guard<std::mutex> lock(m);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = set();
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace lsa

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(LSA_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

}  // namespace

namespace lsa {
int fail_status(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int fail_hip(hipError_t e, const char* where) { return hip_fail(e, where); }
}  // namespace lsa

namespace {

#define LSA_HIP(call, where)                         \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

constexpr int64_t kAlign = 256;
constexpr int kFastSelectMinQ = 64;
int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_index_params(const lsa_index_params* p) {
  if (!p) return fail(LSA_E_ARG, "index params are NULL");
  if (p->dim != kDim) return fail(LSA_E_UNSUPPORTED, "latent dim %d (only 64 is supported)", p->dim);
  if (p->pool < 1 || p->pool > 64) return fail(LSA_E_ARG, "pool %d not in [1, 64]", p->pool);
  if (p->block < 64 || p->block > 16384 || p->block % 64)
    return fail(LSA_E_UNSUPPORTED, "block %d: need a multiple of 64 in [64, 16384]", p->block);
  if (p->buckets < 16 || p->buckets > 256 || p->buckets % 16 || p->buckets > p->block)
    return fail(LSA_E_UNSUPPORTED, "buckets %d: need a multiple of 16 in [16, min(256, block)]",
                p->buckets);
  if (p->iters < 1) return fail(LSA_E_ARG, "iters %d < 1", p->iters);
  if (p->tree_group < 0) return fail(LSA_E_ARG, "tree_group %d < 0", p->tree_group);
  if (p->tree_group > 0) {
    const int64_t n = (int64_t)p->tree_group * p->buckets;
    if (n > 16384 || n % 64)
      return fail(LSA_E_UNSUPPORTED, "tree_group*buckets = %lld: need a multiple of 64 <= 16384",
                  (long long)n);
    if (p->tree_super < 16 || p->tree_super > 256 || p->tree_super % 16 || p->tree_super > n)
      return fail(LSA_E_UNSUPPORTED, "tree_super %d: need a multiple of 16 in [16, 256]",
                  p->tree_super);
    if (p->tree_iters < 1) return fail(LSA_E_ARG, "tree_iters %d < 1", p->tree_iters);
  }
  if (p->tree2_group < 0) return fail(LSA_E_ARG, "tree2_group %d < 0", p->tree2_group);
  if (p->tree2_group > 0) {
    if (p->tree_group <= 0) return fail(LSA_E_ARG, "a third Tree level needs tree_group > 0");
    const int64_t n = (int64_t)p->tree2_group * p->tree_super;
    if (n > 16384 || n % 64)
      return fail(LSA_E_UNSUPPORTED, "tree2_group*tree_super = %lld: need a multiple of 64 <= 16384",
                  (long long)n);
    if (p->tree2_super < 16 || p->tree2_super > 256 || p->tree2_super % 16 || p->tree2_super > n)
      return fail(LSA_E_UNSUPPORTED, "tree2_super %d: need a multiple of 16 in [16, 256]",
                  p->tree2_super);
    if (p->tree2_iters < 1) return fail(LSA_E_ARG, "tree2_iters %d < 1", p->tree2_iters);
  }
  if (p->max_tokens < 0 || p->max_tokens > INT32_MAX - 64)
    return fail(LSA_E_ARG, "max_tokens %lld out of range", (long long)p->max_tokens);
  return LSA_OK;
}

// Capacities and arena offsets.
void layout(const lsa_index_params& p, Index* h) {
  h->max_pool = p.max_tokens / p.pool;
  h->max_full = h->max_pool / p.block;
  h->max_bkt = h->max_full * p.buckets + p.block;
  h->max_grp = p.tree_group > 0 ? h->max_full / p.tree_group : 0;
  h->max_sup = h->max_grp * p.tree_super;
  h->max_smem = h->max_grp * p.tree_group * p.buckets;
  h->max_grp2 = p.tree2_group > 0 ? h->max_grp / p.tree2_group : 0;
  h->max_top = h->max_grp2 * p.tree2_super;
  int64_t o = 0;
  h->off_pooled = o; o = align_up(o + h->max_pool * kDim);
  h->off_cent = o;   o = align_up(o + h->max_bkt * kDim);
  h->off_bcnt = o;   o = align_up(o + h->max_bkt * 4);
  h->off_boff = o;   o = align_up(o + h->max_bkt * 4);
  h->off_bmem = o;   o = align_up(o + h->max_pool * 4);
  h->off_bfirst = o; o = align_up(o + h->max_bkt * 4);
  h->off_blast = o;  o = align_up(o + h->max_bkt * 4);
  h->off_scent = o;  o = align_up(o + h->max_sup * kDim);
  h->off_scnt = o;   o = align_up(o + h->max_sup * 4);
  h->off_soff = o;   o = align_up(o + h->max_sup * 4);
  h->off_smem = o;   o = align_up(o + h->max_smem * 4);
  h->off_leafsup = o; o = align_up(o + (p.tree_group > 0 ? h->max_bkt * 4 : 0));
  h->off_pend = o;   o = align_up(o + 2 * (int64_t)p.pool * kDim);
  h->off_tcent = o;  o = align_up(o + h->max_top * kDim);
  h->off_tcnt = o;   o = align_up(o + h->max_top * 4);
  h->off_toff = o;   o = align_up(o + h->max_top * 4);
  h->off_tmem = o;   o = align_up(o + h->max_grp2 * p.tree2_group * p.tree_super * 4);
  h->off_suptop = o; o = align_up(o + (p.tree2_group > 0 ? h->max_sup * 4 : 0));
  h->off_sblk = o;   o = align_up(o + h->max_sup * (p.tree_group + 1) * 4);
  h->off_skey = o;   o = align_up(o + h->max_sup * (p.tree_group + 1) * 4);
  h->off_bdesc = o;  o = align_up(o + h->max_bkt * 16);
  {
    size_t km = kmeans_scratch_bytes(p.block, p.buckets);
    if (p.tree_group > 0) {
      const size_t kt = kmeans_scratch_bytes(p.tree_group * p.buckets, p.tree_super);
      km = km > kt ? km : kt;
    }
    if (p.tree2_group > 0) {
      const size_t k2 = kmeans_scratch_bytes(p.tree2_group * p.tree_super, p.tree2_super);
      km = km > k2 ? km : k2;
    }
    h->kmws_bytes = (int64_t)km;
  }
  h->off_kmws = o;   o = align_up(o + h->kmws_bytes);
  h->used_bytes = o;
}

Index* as_index(lsa_index* h) { return reinterpret_cast<Index*>(h); }
const Index* as_index(const lsa_index* h) { return reinterpret_cast<const Index*>(h); }

int check_index(const Index* h) {
  if (!h) return fail(LSA_E_ARG, "index is NULL");
  if (h->magic != kMagic) return fail(LSA_E_STATE, "index descriptor not initialised");
  return LSA_OK;
}

int check_select_params(const lsa_select_params* sp, bool tree, bool tree3 = false) {
  if (!sp) return fail(LSA_E_ARG, "select params are NULL");
  if (tree3 && sp->tree2_top < 1) return fail(LSA_E_ARG, "tree2_top %d < 1", sp->tree2_top);
  if (sp->budget < 0 || sp->budget > 4096)
    return fail(LSA_E_UNSUPPORTED, "budget %d not in [0, 4096]", sp->budget);
  if (sp->window < 1 || sp->window > (1 << 20)) return fail(LSA_E_ARG, "window %d not in [1, 2^20]", sp->window);
  if (sp->sinks < 0 || sp->sinks > (1 << 20)) return fail(LSA_E_ARG, "sinks %d not in [0, 2^20]", sp->sinks);
  if (tree && sp->tree_top < 1) return fail(LSA_E_ARG, "tree_top %d < 1", sp->tree_top);
  if (sp->early_until < 0) return fail(LSA_E_ARG, "early_until %d < 0", sp->early_until);
  if (sp->early_until > 0 && (sp->early_budget < 0 || sp->early_budget > sp->budget))
    return fail(LSA_E_ARG, "early_budget %d not in [0, budget]", sp->early_budget);
  return LSA_OK;
}

int check_attn_params(const lsa_attn_params* ap) {
  if (!ap) return fail(LSA_E_ARG, "attention params are NULL");
  if (ap->D != 64 && ap->D != 128) return fail(LSA_E_UNSUPPORTED, "head dim %d (64 or 128)", ap->D);
  if (ap->Hkv < 1 || ap->Hq < 1 || ap->Hq % ap->Hkv)
    return fail(LSA_E_UNSUPPORTED, "Hq %d must be a positive multiple of Hkv %d", ap->Hq, ap->Hkv);
  if (ap->Hq / ap->Hkv > 16) return fail(LSA_E_UNSUPPORTED, "Hq/Hkv %d > 16", ap->Hq / ap->Hkv);
  if (!(ap->scale >= 0.f) || isinf(ap->scale)) return fail(LSA_E_ARG, "bad scale");
  return LSA_OK;
}

int32_t max_sel_of(const lsa_select_params* sp) { return sp->budget + sp->window + sp->sinks; }

IdxView view_of(const Index* h) {
  IdxView v;
  memset(&v, 0, sizeof v);
  v.cent = h->at<int8_t>(h->off_cent);
  v.bcnt = h->at<int32_t>(h->off_bcnt);
  v.boff = h->at<int32_t>(h->off_boff);
  v.bmem = h->at<int32_t>(h->off_bmem);
  v.bfirst = h->at<int32_t>(h->off_bfirst);
  v.blast = h->at<int32_t>(h->off_blast);
  v.bdesc = h->at<int4>(h->off_bdesc);
  v.n_bkt = (int32_t)h->n_bkt();
  v.pool = h->prm.pool;
  v.n_pool = (int32_t)h->n_pool;
  v.dense = 0;
  if (h->prm.tree_group > 0 && h->n_grp > 0) {
    v.leafsup = h->at<int32_t>(h->off_leafsup);
    v.n_sup = (int32_t)(h->n_grp * h->prm.tree_super);
    v.scent = h->at<int8_t>(h->off_scent);
    v.scnt = h->at<int32_t>(h->off_scnt);
    v.soff = h->at<int32_t>(h->off_soff);
    v.smem = h->at<int32_t>(h->off_smem);
    v.covered = (int32_t)(h->n_grp * h->prm.tree_group * h->prm.buckets);
    v.sblk = h->at<int32_t>(h->off_sblk);
    v.skey = h->at<int32_t>(h->off_skey);
    v.tgroup = h->prm.tree_group;
    v.tsuper = h->prm.tree_super;
    v.bpb = h->prm.buckets;
    v.tgroup2 = h->prm.tree2_group;
    v.blk_keys = (int64_t)h->prm.block * h->prm.pool;
    if (h->prm.tree2_group > 0 && h->n_grp2 > 0) {
      v.n_top = (int32_t)(h->n_grp2 * h->prm.tree2_super);
      v.covered_sup = (int32_t)(h->n_grp2 * h->prm.tree2_group * h->prm.tree_super);
      v.tcent = h->at<int8_t>(h->off_tcent);
      v.tcnt = h->at<int32_t>(h->off_tcnt);
      v.toff = h->at<int32_t>(h->off_toff);
      v.tmem = h->at<int32_t>(h->off_tmem);
      v.suptop = h->at<int32_t>(h->off_suptop);
    }
  }
  return v;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Leaf -> super and super -> top-node maps start at -1 ("not covered"):
// entries are written when their group (top group) is clustered.
hipError_t reset_tree_maps(Index* h, hipStream_t s) {
  hipError_t e = fill_i32(h->at<int32_t>(h->off_leafsup), h->max_bkt, -1, s);
  if (e == hipSuccess && h->prm.tree2_group > 0)
    e = fill_i32(h->at<int32_t>(h->off_suptop), h->max_sup, -1, s);
  return e;
}

// Append n latent rows (device) to the index.  Shapes come from host counters.
int append_impl(Index* h, const int8_t* src, int64_t n, hipStream_t s) {
  const lsa_index_params& P = h->prm;
  const int p = P.pool, N = P.block, C = P.buckets;
  if (n > 0 && reinterpret_cast<uintptr_t>(src) % 16)
    return fail(LSA_E_ARG, "latent keys must be 16-byte aligned (pooling reads 16-byte words)");
  if (h->T + n > P.max_tokens)
    return fail(LSA_E_CAPACITY, "T %lld + %lld exceeds capacity %lld", (long long)h->T,
                (long long)n, (long long)P.max_tokens);
  if (n == 0) return LSA_OK;
  const int n_pend = (int)(h->T - h->n_pool * p);
  int8_t* pend = h->at<int8_t>(h->off_pend) + (int64_t)h->pend_slot * p * kDim;
  int8_t* pend2 = h->at<int8_t>(h->off_pend) + (int64_t)(h->pend_slot ^ 1) * p * kDim;
  const int64_t total = n_pend + n;
  const int64_t newg = total / p;
  const int keep = (int)(total % p);
  const int64_t g0 = h->n_pool;
  int8_t* pooled = h->at<int8_t>(h->off_pooled);
  LSA_HIP(launch_pool(pend, n_pend, src, n, p, pooled + g0 * kDim, newg, s), "pool");
  LSA_HIP(launch_save_pending(pend, n_pend, src, n, keep, pend2, s), "pending");

  const int64_t n_pool = g0 + newg;
  const int64_t nf_old = h->n_full, nf_new = n_pool / N;
  int8_t* cent = h->at<int8_t>(h->off_cent);
  int32_t* bcnt = h->at<int32_t>(h->off_bcnt);
  int32_t* boff = h->at<int32_t>(h->off_boff);
  int32_t* bmem = h->at<int32_t>(h->off_bmem);
  int32_t* bfirst = h->at<int32_t>(h->off_bfirst);
  int32_t* blast = h->at<int32_t>(h->off_blast);
  if (nf_new > nf_old) {
    LSA_HIP(launch_kmeans(pooled + nf_old * N * kDim, N, C, P.iters, (int32_t)(nf_new - nf_old),
                          nf_old * N, cent + nf_old * C * kDim, bcnt + nf_old * C,
                          boff + nf_old * C, bmem + nf_old * N, bfirst + nf_old * C,
                          blast + nf_old * C, nullptr, 0, h->at<char>(h->off_kmws),
                          (size_t)h->kmws_bytes, s),
            "kmeans");
  }
  const int64_t t0 = nf_new == nf_old ? g0 : nf_new * N;
  LSA_HIP(launch_tail(pooled, t0, n_pool, nf_new, N, C, cent, bcnt, boff, bmem, bfirst, blast, s),
          "tail");
  // packed descriptors of every bucket this append wrote: the blocks it
  // completed and the tail singletons
  LSA_HIP(launch_pack_desc(bfirst, blast, bcnt, boff, nf_old * C,
                           nf_new * C + (n_pool - nf_new * N), h->at<int4>(h->off_bdesc), s),
          "descriptors");
  int64_t ng_new = h->n_grp;
  if (P.tree_group > 0) {
    const int G = P.tree_group, S = P.tree_super;
    ng_new = nf_new / G;
    if (ng_new > h->n_grp) {
      const int64_t g = h->n_grp;
      const int64_t NL = (int64_t)G * C;
      LSA_HIP(launch_kmeans(cent + g * NL * kDim, (int32_t)NL, S, P.tree_iters,
                            (int32_t)(ng_new - g), g * NL, h->at<int8_t>(h->off_scent) + g * S * kDim,
                            h->at<int32_t>(h->off_scnt) + g * S, h->at<int32_t>(h->off_soff) + g * S,
                            h->at<int32_t>(h->off_smem) + g * NL, nullptr, nullptr,
                            h->at<int32_t>(h->off_leafsup), (int32_t)(g * S),
                            h->at<char>(h->off_kmws), (size_t)h->kmws_bytes, s),
              "tree kmeans");
      LSA_HIP(launch_sup_tables(h->at<int32_t>(h->off_soff), h->at<int32_t>(h->off_scnt),
                                h->at<int32_t>(h->off_smem), bcnt, (int32_t)(g * S),
                                (int32_t)((ng_new - g) * S), S, G, C, p, h->at<int32_t>(h->off_sblk),
                                h->at<int32_t>(h->off_skey), s),
              "tree walk tables");
    }
  }
  int64_t ng2_new = h->n_grp2;
  if (P.tree2_group > 0) {
    const int G2 = P.tree2_group, S = P.tree_super, S2 = P.tree2_super;
    ng2_new = ng_new / G2;
    if (ng2_new > h->n_grp2) {
      const int64_t g2 = h->n_grp2;
      const int64_t NS = (int64_t)G2 * S;
      LSA_HIP(launch_kmeans(h->at<int8_t>(h->off_scent) + g2 * NS * kDim, (int32_t)NS, S2,
                            P.tree2_iters, (int32_t)(ng2_new - g2), g2 * NS,
                            h->at<int8_t>(h->off_tcent) + g2 * S2 * kDim,
                            h->at<int32_t>(h->off_tcnt) + g2 * S2, h->at<int32_t>(h->off_toff) + g2 * S2,
                            h->at<int32_t>(h->off_tmem) + g2 * NS, nullptr, nullptr,
                            h->at<int32_t>(h->off_suptop), (int32_t)(g2 * S2),
                            h->at<char>(h->off_kmws), (size_t)h->kmws_bytes, s),
              "top-level kmeans");
    }
  }
  h->T += n;
  h->n_pool = n_pool;
  h->n_full = nf_new;
  h->n_grp = ng_new;
  h->n_grp2 = ng2_new;
  h->pend_slot ^= 1;
  return LSA_OK;
}

int select_impl(const Index* h, const int8_t* latq, const int32_t* qpos, int32_t qpos_base,
                int32_t nq, const lsa_select_params* sp, int32_t* idx, int32_t* cnt,
                void* ws, size_t ws_bytes, hipStream_t s) {
  IdxView v = view_of(h);
  if (v.leafsup && v.n_sup > 2048)
    return fail(LSA_E_UNSUPPORTED, "%d super clusters (at most 2048)", v.n_sup);
  SelArgs a;
  a.latq = latq; a.qpos = qpos; a.qpos_base = qpos_base; a.nq = nq;
  a.budget = sp->budget; a.window = sp->window; a.sinks = sp->sinks; a.tree_top = sp->tree_top;
  a.early_budget = sp->early_budget; a.early_until = sp->early_until; a.tree2_top = sp->tree2_top;
  a.max_sel = max_sel_of(sp);
  a.idx = idx; a.cnt = cnt; a.only = nullptr;
  if (!v.leafsup && nq >= kFastSelectMinQ && ws && ws_bytes >= select_fast_ws_bytes(nq)) {
    LSA_HIP(launch_select_fast(v, a, ws, s), "select");
  } else if (v.leafsup && ws && ws_bytes >= select_tree_ws_bytes(nq)) {
    LSA_HIP(launch_select_tree(v, a, ws, s), "select");
  } else {
    LSA_HIP(launch_select(v, a, nullptr, s), "select");
  }
  return LSA_OK;
}

constexpr int kDecodeSplits = 32;

}  // namespace

// Arguments shared by the window-sharing attention entry points.
static int check_window_attn(int64_t kv_rows, int32_t max_sel, int32_t nq, int64_t qpos0,
                      const lsa_select_params* sp, const lsa_attn_params* ap) {
  if (int e = check_attn_params(ap)) return e;
  if (!sp) return fail(LSA_E_ARG, "select params are NULL");
  if (sp->window < 1 || sp->sinks < 0 || sp->budget < 0)
    return fail(LSA_E_ARG, "bad select params (window %d, sinks %d, budget %d)", sp->window, sp->sinks,
                sp->budget);
  if (nq < 0 || kv_rows < 1 || qpos0 < 0) return fail(LSA_E_ARG, "bad nq / kv_rows / qpos0");
  if (max_sel < max_sel_of(sp)) return fail(LSA_E_ARG, "max_sel %d < budget + window + sinks", max_sel);
  if (qpos0 + nq > kv_rows) return fail(LSA_E_ARG, "query positions reach beyond kv_rows");
  if (kv_rows > INT32_MAX - 64) return fail(LSA_E_ARG, "kv_rows beyond int32");
  return LSA_OK;
}

extern "C" {

const char* lsa_status_str(int status) {
  switch (status) {
    case LSA_OK: return "ok";
    case LSA_E_ARG: return "invalid argument";
    case LSA_E_UNSUPPORTED: return "unsupported shape or parameter";
    case LSA_E_CAPACITY: return "capacity exceeded";
    case LSA_E_STATE: return "bad index state";
    case LSA_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lsa_last_error(void) { return g_err.c_str(); }

int lsa_check(void* stream) {
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(LSA_E_HIP, "%s", hipGetErrorString(e));
  return LSA_OK;
}

size_t lsa_index_sizeof(void) { return kIndexSizeof; }

int lsa_index_bytes(const lsa_index_params* prm, size_t* bytes) {
  if (int e = check_index_params(prm)) return e;
  if (!bytes) return fail(LSA_E_ARG, "bytes is NULL");
  Index tmp;
  memset(&tmp, 0, sizeof tmp);
  layout(*prm, &tmp);
  *bytes = (size_t)tmp.used_bytes;
  return LSA_OK;
}

int lsa_index_init(lsa_index* hh, const lsa_index_params* prm, void* d_arena, size_t arena_bytes) {
  if (!hh) return fail(LSA_E_ARG, "index is NULL");
  if (int e = check_index_params(prm)) return e;
  if (!d_arena) return fail(LSA_E_ARG, "arena is NULL");
  if (reinterpret_cast<uintptr_t>(d_arena) % kAlign) return fail(LSA_E_ARG, "arena not 256-byte aligned");
  Index tmp;
  memset(&tmp, 0, sizeof tmp);
  layout(*prm, &tmp);
  if ((int64_t)arena_bytes < tmp.used_bytes)
    return fail(LSA_E_CAPACITY, "arena %zu bytes < %lld needed", arena_bytes, (long long)tmp.used_bytes);
  tmp.magic = kMagic;
  tmp.prm = *prm;
  tmp.arena = static_cast<char*>(d_arena);
  tmp.arena_bytes = arena_bytes;
  memset(hh, 0, kIndexSizeof);
  memcpy(hh, &tmp, sizeof tmp);
  return LSA_OK;
}

int lsa_index_get_info(const lsa_index* hh, lsa_index_info* out) {
  const Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (!out) return fail(LSA_E_ARG, "info is NULL");
  out->T = h->T; out->n_pool = h->n_pool; out->n_full = h->n_full; out->n_bkt = h->n_bkt();
  out->n_grp = h->n_grp; out->n_sup = h->n_grp * h->prm.tree_super;
  out->off_pooled = h->off_pooled; out->off_cent = h->off_cent; out->off_bcnt = h->off_bcnt;
  out->off_boff = h->off_boff; out->off_bmem = h->off_bmem; out->off_bfirst = h->off_bfirst;
  out->off_blast = h->off_blast; out->off_scent = h->off_scent; out->off_scnt = h->off_scnt;
  out->off_soff = h->off_soff; out->off_smem = h->off_smem;
  out->arena_bytes = h->used_bytes;
  out->n_grp2 = h->n_grp2; out->n_top = h->n_grp2 * h->prm.tree2_super;
  out->off_tcent = h->off_tcent; out->off_tcnt = h->off_tcnt; out->off_toff = h->off_toff;
  out->off_tmem = h->off_tmem;
  return LSA_OK;
}

int lsa_workspace_bytes(int op, const lsa_index_params* iprm, const lsa_select_params* sprm,
                        const lsa_attn_params* aprm, int64_t n, size_t* bytes) {
  if (!bytes) return fail(LSA_E_ARG, "bytes is NULL");
  if (n < 0) return fail(LSA_E_ARG, "n < 0");
  (void)iprm;
  switch (op) {
    case LSA_OP_BUILD: case LSA_OP_APPEND: case LSA_OP_ATTN:
      *bytes = 0;
      return LSA_OK;
    case LSA_OP_SELECT:
      *bytes = select_fast_ws_bytes((int32_t)n);
      return LSA_OK;
    case LSA_OP_DENSE:
      *bytes = dense_ws_bytes((int32_t)n);
      return LSA_OK;
    case LSA_OP_PREFILL: {
      if (int e = check_select_params(sprm, false)) return e;
      size_t phase = select_fast_ws_bytes((int32_t)n);
      if (aprm) {
        if (int e = check_attn_params(aprm)) return e;
        if (grouped_attn_ok(*aprm, sprm->budget, 1) && grouped_nq_ok(n))
          phase = std::max(phase, attn_grouped_ws_bytes((int32_t)n, *aprm, sprm->budget));
      }
      *bytes = (size_t)align_up(n * max_sel_of(sprm) * 4) + (size_t)align_up(n * 4) + phase;
      return LSA_OK;
    }
    case LSA_OP_ATTN_GROUPED: {
      if (int e = check_select_params(sprm, false)) return e;
      if (int e = check_attn_params(aprm)) return e;
      if (!grouped_nq_ok(n)) return fail(LSA_E_UNSUPPORTED, "grouped attention takes at most %lld queries",
                                         (long long)kGroupedMaxQueries);
      *bytes = attn_grouped_ws_bytes((int32_t)n, *aprm, sprm->budget);
      return LSA_OK;
    }
    case LSA_OP_DECODE: {
      if (int e = check_index_params(iprm)) return e;
      if (int e = check_select_params(sprm, false)) return e;
      if (int e = check_attn_params(aprm)) return e;
      Index tmp;
      memset(&tmp, 0, sizeof tmp);
      layout(*iprm, &tmp);
      *bytes = (size_t)align_up(n * max_sel_of(sprm) * 4) + (size_t)align_up(n * 4) +
               (size_t)align_up((int64_t)attn_ws_bytes((int32_t)n, *aprm, kDecodeSplits)) +
               select_dec_ws_bytes((int32_t)n, tmp.max_bkt);
      return LSA_OK;
    }
    case LSA_OP_ATTN_BWD: {
      if (int e = check_index_params(iprm)) return e;
      if (int e = check_select_params(sprm, false)) return e;
      if (int e = check_attn_params(aprm)) return e;
      if (n > INT32_MAX) return fail(LSA_E_ARG, "n > INT32_MAX");
      Index tmp;
      memset(&tmp, 0, sizeof tmp);
      layout(*iprm, &tmp);
      *bytes = attn_bwd_ws_bytes((int32_t)n, *aprm, tmp.max_pool, tmp.max_bkt, sprm->budget);
      return LSA_OK;
    }
    default:
      return fail(LSA_E_ARG, "unknown op %d", op);
  }
}

int lsa_build_index(lsa_index* hh, const int8_t* d_latk, int64_t T, void* d_ws, size_t ws_bytes,
                    void* stream) {
  (void)d_ws; (void)ws_bytes;
  Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (T < 0) return fail(LSA_E_ARG, "T < 0");
  if (T > 0 && !d_latk) return fail(LSA_E_ARG, "latents are NULL");
  if (T > h->prm.max_tokens)
    return fail(LSA_E_CAPACITY, "T %lld exceeds capacity %lld", (long long)T,
                (long long)h->prm.max_tokens);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Index saved = *h;
  h->T = 0; h->n_pool = 0; h->n_full = 0; h->n_grp = 0; h->n_grp2 = 0; h->pend_slot = 0;
  if (h->prm.tree_group > 0) {
    hipError_t e = reset_tree_maps(h, s);
    if (e != hipSuccess) { *h = saved; return hip_fail(e, "fill"); }
  }
  int rc = append_impl(h, d_latk, T, s);
  if (rc != LSA_OK) *h = saved;
  return rc;
}

int lsa_append_keys(lsa_index* hh, const int8_t* d_latk_new, int64_t n, void* d_ws, size_t ws_bytes,
                    void* stream) {
  (void)d_ws; (void)ws_bytes;
  Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (n < 0) return fail(LSA_E_ARG, "n < 0");
  if (n > 0 && !d_latk_new) return fail(LSA_E_ARG, "latents are NULL");
  if (h->T == 0 && h->prm.tree_group > 0) {
    hipError_t e = reset_tree_maps(h, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fill");
  }
  Index saved = *h;
  int rc = append_impl(h, d_latk_new, n, static_cast<hipStream_t>(stream));
  if (rc != LSA_OK) *h = saved;
  return rc;
}

int lsa_select(const lsa_index* hh, const int8_t* d_latq, const int32_t* d_qpos, int32_t nq,
               const lsa_select_params* sp, int32_t* d_idx, int32_t* d_cnt, void* d_ws,
               size_t ws_bytes, void* stream) {
  const Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (int e = check_select_params(sp, h->prm.tree_group > 0, h->prm.tree2_group > 0)) return e;
  if (nq < 0) return fail(LSA_E_ARG, "nq < 0");
  if (nq > 0 && (!d_latq || !d_qpos || !d_idx || !d_cnt)) return fail(LSA_E_ARG, "NULL buffer");
  return select_impl(h, d_latq, d_qpos, 0, nq, sp, d_idx, d_cnt, d_ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

int lsa_sparse_attn(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v, int64_t kv_rows,
                    const int32_t* d_idx, const int32_t* d_cnt, int32_t max_sel, int32_t nq,
                    const lsa_attn_params* ap, void* d_out, void* d_ws, size_t ws_bytes,
                    void* stream) {
  (void)d_ws; (void)ws_bytes;
  if (int e = check_attn_params(ap)) return e;
  if (nq < 0 || max_sel < 1 || kv_rows < 1) return fail(LSA_E_ARG, "bad nq / max_sel / kv_rows");
  if (nq > 0 && (!d_q || !d_k || !d_v || !d_idx || !d_cnt || !d_out)) return fail(LSA_E_ARG, "NULL buffer");
  LSA_HIP(launch_attn(d_q, d_k, d_v, kv_rows, 0, nq > 0 ? nq : 1, d_idx, d_cnt, max_sel, nq, *ap,
                      d_out, nullptr, 1, static_cast<hipStream_t>(stream)),
          "attention");
  return LSA_OK;
}

int lsa_sparse_attn_window(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                           int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                           int32_t max_sel, int32_t nq, int64_t qpos0, const lsa_select_params* sp,
                           const lsa_attn_params* ap, void* d_out, void* stream) {
  if (int e = check_window_attn(kv_rows, max_sel, nq, qpos0, sp, ap)) return e;
  if (nq > 0 && (!d_q || !d_k || !d_v || !d_idx || !d_cnt || !d_out)) return fail(LSA_E_ARG, "NULL buffer");
  LSA_HIP(launch_attn_window(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, sp->window,
                             sp->sinks, *ap, d_out, nullptr, static_cast<hipStream_t>(stream)),
          "attention");
  return LSA_OK;
}

static int grouped_parts(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                         int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                         int32_t max_sel, int32_t nq, int64_t qpos0, const int8_t* d_latq,
                         const lsa_select_params* sp, const lsa_attn_params* ap, void* d_out,
                         float* d_lse, void* d_ws, size_t ws_bytes, void* stream, int parts) {
  if (int e = check_window_attn(kv_rows, max_sel, nq, qpos0, sp, ap)) return e;
  if (!grouped_attn_ok(*ap, sp->budget, kv_rows) || !grouped_nq_ok(nq))
    return fail(LSA_E_UNSUPPORTED, "grouped attention needs D in {64, 128}, Hq/Hkv in {4, 8, 16}, "
                "(16 / (Hq/Hkv)) * budget <= 16384, kv_rows < 2^28 and nq <= 2^26");
  if (nq == 0) return LSA_OK;
  if (!d_q || !d_k || !d_v || !d_idx || !d_cnt || ((parts & kGroupedWalk) && !d_out))
    return fail(LSA_E_ARG, "NULL buffer");
  const size_t need = attn_grouped_ws_bytes(nq, *ap, sp->budget);
  if (!d_ws || ws_bytes < need) return fail(LSA_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  LSA_HIP(launch_attn_grouped(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, sp->window,
                              sp->sinks, sp->budget, *ap, d_latq, d_out, d_lse, d_ws, parts,
                              static_cast<hipStream_t>(stream)),
          "grouped attention");
  return LSA_OK;
}

int lsa_sparse_attn_grouped(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                            int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                            int32_t max_sel, int32_t nq, int64_t qpos0, const int8_t* d_latq,
                            const lsa_select_params* sp, const lsa_attn_params* ap, void* d_out,
                            float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
  return grouped_parts(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, d_latq, sp, ap,
                       d_out, d_lse, d_ws, ws_bytes, stream, kGroupedPrepare | kGroupedWalk);
}

int lsa_attn_grouped_prepare(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                             int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                             int32_t max_sel, int32_t nq, int64_t qpos0, const int8_t* d_latq,
                             const lsa_select_params* sp, const lsa_attn_params* ap, void* d_ws,
                             size_t ws_bytes, void* stream) {
  return grouped_parts(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, d_latq, sp, ap,
                       nullptr, nullptr, d_ws, ws_bytes, stream, kGroupedPrepare);
}

int lsa_attn_grouped_walk(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                          int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                          int32_t max_sel, int32_t nq, int64_t qpos0, const lsa_select_params* sp,
                          const lsa_attn_params* ap, void* d_out, float* d_lse, void* d_ws,
                          size_t ws_bytes, void* stream) {
  return grouped_parts(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, nullptr, sp, ap,
                       d_out, d_lse, d_ws, ws_bytes, stream, kGroupedWalk);
}

int lsa_sparse_attn_fwd(const uint16_t* d_q, const uint16_t* d_k, const uint16_t* d_v,
                        int64_t kv_rows, const int32_t* d_idx, const int32_t* d_cnt,
                        int32_t max_sel, int32_t nq, int64_t qpos0, const lsa_select_params* sp,
                        const lsa_attn_params* ap, void* d_out, float* d_lse, void* stream) {
  if (int e = check_window_attn(kv_rows, max_sel, nq, qpos0, sp, ap)) return e;
  if (nq > 0 && (!d_q || !d_k || !d_v || !d_idx || !d_cnt || !d_out || !d_lse))
    return fail(LSA_E_ARG, "NULL buffer");
  LSA_HIP(launch_attn_window(d_q, d_k, d_v, kv_rows, d_idx, d_cnt, max_sel, nq, qpos0, sp->window,
                             sp->sinks, *ap, d_out, d_lse, static_cast<hipStream_t>(stream)),
          "attention");
  return LSA_OK;
}

int lsa_sparse_attn_bwd(const lsa_index* hh, const uint16_t* d_q, const uint16_t* d_k,
                        const uint16_t* d_v, int64_t kv_rows, const int32_t* d_idx,
                        const int32_t* d_cnt, int32_t max_sel, int32_t nq, int64_t qpos0,
                        const int8_t* d_latq, const lsa_select_params* sp,
                        const lsa_attn_params* ap, const void* d_out,
                        const float* d_lse, const uint16_t* d_dout, float* d_dq, float* d_dk,
                        float* d_dv, void* d_ws, size_t ws_bytes, void* stream) {
  const Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (int e = check_select_params(sp, false)) return e;
  if (int e = check_window_attn(kv_rows, max_sel, nq, qpos0, sp, ap)) return e;
  if (sp->sinks > 64) return fail(LSA_E_UNSUPPORTED, "sinks %d > 64 in the backward", sp->sinks);
  if (qpos0 + nq > h->T) return fail(LSA_E_ARG, "query positions reach beyond the index (T %lld)",
                                     (long long)h->T);
  if (nq == 0) return LSA_OK;
  if (!d_q || !d_k || !d_v || !d_idx || !d_cnt || !d_out || !d_lse || !d_dout || !d_dq || !d_dk ||
      !d_dv)
    return fail(LSA_E_ARG, "NULL buffer");
  const size_t need = attn_bwd_ws_bytes(nq, *ap, h->max_pool, h->max_bkt, sp->budget);
  if (!d_ws || ws_bytes < need) return fail(LSA_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  const IdxView v = view_of(h);
  BwdInputs in;
  memset(&in, 0, sizeof in);
  in.q = d_q; in.k = d_k; in.v = d_v; in.o = d_out; in.dout = d_dout; in.lse = d_lse;
  in.kv_rows = kv_rows; in.idx = d_idx; in.cnt = d_cnt; in.latq = d_latq; in.max_sel = max_sel; in.nq = nq;
  in.qpos0 = qpos0; in.window = sp->window; in.sinks = sp->sinks; in.budget = sp->budget;
  in.dq = d_dq; in.dk = d_dk; in.dv = d_dv;
  in.bcnt = v.bcnt; in.boff = v.boff; in.bmem = v.bmem;
  in.n_bkt = v.n_bkt; in.pool = v.pool; in.n_pool = (int32_t)h->n_pool;
  in.max_pool = h->max_pool; in.max_bkt = h->max_bkt;
  in.ws = d_ws;
  LSA_HIP(launch_attn_bwd(in, *ap, static_cast<hipStream_t>(stream)), "attention backward");
  return LSA_OK;
}

int lsa_prefill_chunk(lsa_index* hh, const int8_t* d_latk_chunk, int64_t n_chunk,
                      const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                      const uint16_t* d_v, int64_t kv_rows, const lsa_select_params* sp,
                      const lsa_attn_params* ap, void* d_out, int32_t* d_idx_opt,
                      int32_t* d_cnt_opt, void* d_ws, size_t ws_bytes, void* stream) {
  Index* h = as_index(hh);
  if (int e = check_index(h)) return e;
  if (int e = check_select_params(sp, h->prm.tree_group > 0, h->prm.tree2_group > 0)) return e;
  if (int e = check_attn_params(ap)) return e;
  if (n_chunk < 0 || n_chunk > INT32_MAX / 2) return fail(LSA_E_ARG, "bad n_chunk");
  if (n_chunk == 0) return LSA_OK;
  if (!d_latk_chunk || !d_latq || !d_q || !d_k || !d_v || !d_out) return fail(LSA_E_ARG, "NULL buffer");
  if (kv_rows < h->T + n_chunk) return fail(LSA_E_ARG, "kv_rows %lld < T + n_chunk", (long long)kv_rows);
  if (h->T + n_chunk > h->prm.max_tokens) return fail(LSA_E_CAPACITY, "chunk exceeds capacity");
  const int32_t max_sel = max_sel_of(sp);
  int32_t* idx = d_idx_opt;
  int32_t* cnt = d_cnt_opt;
  const size_t a_idx = (size_t)align_up(n_chunk * max_sel * 4) + (size_t)align_up(n_chunk * 4);
  const size_t need = a_idx + select_fast_ws_bytes((int32_t)n_chunk);
  if (!d_ws || ws_bytes < need) return fail(LSA_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!idx || !cnt) {
    idx = static_cast<int32_t*>(d_ws);
    cnt = reinterpret_cast<int32_t*>(static_cast<char*>(d_ws) + align_up(n_chunk * max_sel * 4));
  }
  void* sel_ws = static_cast<char*>(d_ws) + a_idx;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t t0 = h->T;
  if (h->T == 0 && h->prm.tree_group > 0) {
    LSA_HIP(reset_tree_maps(h, s), "fill");
  }
  Index saved = *h;
  int rc = append_impl(h, d_latk_chunk, n_chunk, s);
  if (rc != LSA_OK) { *h = saved; return rc; }
  rc = select_impl(h, d_latq, nullptr, (int32_t)t0, (int32_t)n_chunk, sp, idx, cnt, sel_ws,
                   select_fast_ws_bytes((int32_t)n_chunk), s);
  if (rc != LSA_OK) return rc;
  if (grouped_attn_ok(*ap, sp->budget, kv_rows) && grouped_nq_ok(n_chunk) &&
      ws_bytes - a_idx >= attn_grouped_ws_bytes((int32_t)n_chunk, *ap, sp->budget)) {
    // Flat and two-level Tree: queries grouped by their latent neighbours;
    // three-level Tree: by their rows.  Measured on 10M-key chunks of 32768
    // queries: latent order leaves unions of 0.693 (Flat) and 0.708 (two
    // levels) of the long-range entries against 0.765 and 0.772 by rows, but
    // 0.632 against 0.602 by rows with a third level, whose walk makes
    // neighbouring queries' rows alike beyond what their latents show.
    const int8_t* glat = h->prm.tree2_group > 0 ? nullptr : d_latq;
    LSA_HIP(launch_attn_grouped(d_q, d_k, d_v, kv_rows, idx, cnt, max_sel, (int32_t)n_chunk, t0,
                                sp->window, sp->sinks, sp->budget, *ap, glat, d_out, nullptr, sel_ws,
                                kGroupedPrepare | kGroupedWalk, s),
            "grouped attention");
    return LSA_OK;
  }
  LSA_HIP(launch_attn_window(d_q, d_k, d_v, kv_rows, idx, cnt, max_sel, (int32_t)n_chunk, t0,
                             sp->window, sp->sinks, *ap, d_out, nullptr, s),
          "attention");
  return LSA_OK;
}

int lsa_decode_step(lsa_index* const* hs, int32_t nseq, const int8_t* d_latk_new,
                    const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                    const uint16_t* d_v, int64_t seq_stride_rows, const lsa_select_params* sp,
                    const lsa_attn_params* ap, void* d_out, void* d_ws, size_t ws_bytes,
                    void* stream) {
  if (!hs || nseq < 1 || nseq > 16) return fail(LSA_E_ARG, "nseq %d not in [1, 16]", nseq);
  if (int e = check_attn_params(ap)) return e;
  if (!d_latk_new || !d_latq || !d_q || !d_k || !d_v || !d_out) return fail(LSA_E_ARG, "NULL buffer");
  const Index* h0 = as_index(hs[0]);
  if (int e = check_index(h0)) return e;
  for (int i = 0; i < nseq; ++i) {
    const Index* h = as_index(hs[i]);
    if (int e = check_index(h)) return e;
    if (int e = check_select_params(sp, h->prm.tree_group > 0, h->prm.tree2_group > 0)) return e;
    if (memcmp(&h->prm, &h0->prm, sizeof h->prm) != 0)
      return fail(LSA_E_ARG, "sequence %d has different index params", i);
    if (h->T + 1 > h->prm.max_tokens) return fail(LSA_E_CAPACITY, "sequence %d is full", i);
    if (seq_stride_rows < h->T + 1) return fail(LSA_E_ARG, "seq_stride_rows < T + 1 for sequence %d", i);
    if (h->prm.tree_group > 0) {
      // super clusters after this key's append (it may complete a block, and
      // with it a Tree group): the decode walk holds at most 2048
      const int64_t np1 = h->T + 1 - h->n_pool * h->prm.pool;
      const int64_t pool_after = h->n_pool + (np1 == h->prm.pool ? 1 : 0);
      const int64_t grp_after = pool_after / h->prm.block / h->prm.tree_group;
      if (grp_after * h->prm.tree_super > 2048)
        return fail(LSA_E_UNSUPPORTED, "sequence %d: %lld super clusters (at most 2048 in decode)", i,
                    (long long)(grp_after * h->prm.tree_super));
    }
    for (int j = 0; j < i; ++j)
      if (hs[j] == hs[i]) return fail(LSA_E_ARG, "sequence %d repeats an index", i);
  }
  const int32_t max_sel = max_sel_of(sp);
  const size_t a_idx = (size_t)align_up((int64_t)nseq * max_sel * 4);
  const size_t a_cnt = (size_t)align_up((int64_t)nseq * 4);
  const size_t a_att = (size_t)align_up((int64_t)attn_ws_bytes(nseq, *ap, kDecodeSplits));
  const size_t a_sel = select_dec_ws_bytes(nseq, h0->max_bkt);
  if (!d_ws || ws_bytes < a_idx + a_cnt + a_att + a_sel)
    return fail(LSA_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, a_idx + a_cnt + a_att + a_sel);
  char* ws = static_cast<char*>(d_ws);
  int32_t* idx = reinterpret_cast<int32_t*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + a_idx);
  void* att = ws + a_idx + a_cnt;
  void* selws = ws + a_idx + a_cnt + a_att;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int p = h0->prm.pool, N = h0->prm.block;

  // Every descriptor as it was: if any launch below fails, all of them are
  // put back, so no sequence counts a key the device did not get.  (Arrays
  // past the restored counters may hold partial writes; the next append
  // rewrites them, and no kernel reads past the counters.)
  Index saved[16];
  for (int i = 0; i < nseq; ++i) saved[i] = *as_index(hs[i]);
  auto restore_all = [&](int rc) {
    for (int i = 0; i < nseq; ++i) *as_index(hs[i]) = saved[i];
    return rc;
  };

  // 1. append one key per sequence: one batched launch; a sequence whose key
  //    completes a block (a k-means is due) takes the general path
  DecodeAppendArgs da;
  memset(&da, 0, sizeof da);
  da.off_pooled = h0->off_pooled; da.off_cent = h0->off_cent; da.off_bcnt = h0->off_bcnt;
  da.off_boff = h0->off_boff; da.off_bmem = h0->off_bmem; da.off_bfirst = h0->off_bfirst;
  da.off_blast = h0->off_blast; da.off_pend = h0->off_pend; da.off_bdesc = h0->off_bdesc;
  da.p = p; da.N = N; da.C = h0->prm.buckets;
  int32_t qpos[16];
  bool any_batched = false;
  for (int i = 0; i < nseq; ++i) {
    Index* h = as_index(hs[i]);
    qpos[i] = (int32_t)h->T;
    const int np = (int)(h->T - h->n_pool * p);
    const bool completes_group = np + 1 == p;
    const bool completes_block = completes_group && (h->n_pool + 1) % N == 0;
    if (h->T == 0 && h->prm.tree_group > 0) {
      hipError_t e = reset_tree_maps(h, s);
      if (e != hipSuccess) return restore_all(hip_fail(e, "fill"));
    }
    if (completes_block) {
      int rc = append_impl(h, d_latk_new + (int64_t)i * kDim, 1, s);
      if (rc != LSA_OK) return restore_all(rc);
      continue;
    }
    da.arena[i] = h->arena;
    da.n_pool[i] = h->n_pool; da.n_full[i] = h->n_full;
    da.n_pend[i] = np; da.pend_slot[i] = h->pend_slot;
    da.batched[i] = 1;
    any_batched = true;
  }
  // (the batched append itself is enqueued by the selection below, first)
  for (int i = 0; i < nseq; ++i) {
    if (!da.batched[i]) continue;
    Index* h = as_index(hs[i]);
    const int np = (int)(h->T - h->n_pool * p);
    h->T += 1;
    if (np + 1 == p) h->n_pool += 1;
  }

  // 2. select: one workgroup per sequence, each on its own index
  IdxView views[16];
  for (int i = 0; i < nseq; ++i) {
    views[i] = view_of(as_index(hs[i]));
    if (views[i].leafsup && views[i].n_sup > 2048)   // unreachable: rejected above
      return restore_all(fail(LSA_E_UNSUPPORTED, "%d super clusters (at most 2048)", views[i].n_sup));
  }
  SelArgs a;
  memset(&a, 0, sizeof a);
  a.latq = d_latq; a.qpos = nullptr; a.qpos_base = 0; a.nq = nseq;
  a.budget = sp->budget; a.window = sp->window; a.sinks = sp->sinks; a.tree_top = sp->tree_top;
  a.early_budget = sp->early_budget; a.early_until = sp->early_until; a.tree2_top = sp->tree2_top;
  a.max_sel = max_sel; a.idx = idx; a.cnt = cnt; a.only = nullptr;
  hipError_t e = launch_select_dec(views, qpos, nseq, h0->max_bkt, a, selws, s,
                                  any_batched ? &da : nullptr, d_latk_new);
  if (e != hipSuccess) return restore_all(hip_fail(e, "decode append + select"));

  // 3. split-K attention over each sequence's own rows, then the merge
  e = launch_attn(d_q, d_k, d_v, seq_stride_rows, seq_stride_rows, 1, idx, cnt, max_sel, nseq, *ap,
                  d_out, att, kDecodeSplits, s);
  if (e != hipSuccess) return restore_all(hip_fail(e, "decode attention"));
  return LSA_OK;
}

int lsa_dense_select(const int8_t* d_latk, int64_t T, const int8_t* d_latq, const int32_t* d_qpos,
                     int32_t nq, const lsa_select_params* sp, int32_t* d_idx, int32_t* d_cnt,
                     void* d_ws, size_t ws_bytes, void* stream) {
  if (int e = check_select_params(sp, false)) return e;
  if (T < 0 || T > INT32_MAX - 64 || nq < 0) return fail(LSA_E_ARG, "bad T / nq");
  if (nq > 0 && (!d_latk || !d_latq || !d_qpos || !d_idx || !d_cnt)) return fail(LSA_E_ARG, "NULL buffer");
  IdxView v;
  memset(&v, 0, sizeof v);
  v.cent = d_latk;
  v.n_bkt = (int32_t)T;
  v.pool = 1;
  v.n_pool = (int32_t)T;
  v.dense = 1;
  SelArgs a;
  a.latq = d_latq; a.qpos = d_qpos; a.qpos_base = 0; a.nq = nq;
  a.budget = sp->budget; a.window = sp->window; a.sinks = sp->sinks; a.tree_top = 0;
  a.early_budget = sp->early_budget; a.early_until = sp->early_until; a.tree2_top = sp->tree2_top;
  a.max_sel = max_sel_of(sp);
  a.idx = d_idx; a.cnt = d_cnt; a.only = nullptr;
  // large batches with a workspace: a sampled threshold per query, one
  // thresholded int8-MFMA pass over all latents, then an exact top-budget per
  // query (the exact kernel serves the few queries whose lists cannot hold the
  // cutoff); otherwise the exact kernel
  if (nq >= kFastSelectMinQ && d_ws && ws_bytes >= dense_ws_bytes(nq))
    LSA_HIP(launch_dense_select(v, a, d_ws, static_cast<hipStream_t>(stream)), "dense select");
  else
    LSA_HIP(launch_select(v, a, nullptr, static_cast<hipStream_t>(stream)), "dense select");
  return LSA_OK;
}

}  // extern "C"
