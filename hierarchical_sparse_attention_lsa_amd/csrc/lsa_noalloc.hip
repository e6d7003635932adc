// Decode step for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the step's workspace is a file-scope device array instead of a caller
// buffer.  The kernels are those of lsa_decode_step; only the workspace
// pointer differs.
#include <mutex>

#include "lsa_internal.h"

namespace {

// Workspace of the no-allocation decode step: each GPU the library runs on
// holds one copy of it until the process ends.  128 MiB covers 16 sequences
// of 10 * 2^20 keys at a 4096 + 512 + 4 key budget with GQA 32/8, D = 128
// (that step needs 84 MiB).
constexpr size_t kScratchBytes = 128ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current.  (In host code the array's name is a host-side
// stand-in, not a device address.)
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return lsa::fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return lsa::fail_status(LSA_E_UNSUPPORTED, "device %d: the no-allocation step serves devices 0..63", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return lsa::fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return lsa::fail_status(LSA_E_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return LSA_OK;
}

}  // namespace

extern "C" {

size_t lsa_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

int lsa_decode_step_noalloc(lsa_index* const* hs, int32_t nseq, const int8_t* d_latk_new,
                            const int8_t* d_latq, const uint16_t* d_q, const uint16_t* d_k,
                            const uint16_t* d_v, int64_t seq_stride_rows,
                            const lsa_select_params* sp, const lsa_attn_params* ap, void* d_out,
                            void* stream) {
  if (!hs || nseq < 1 || nseq > 16) return lsa::fail_status(LSA_E_ARG, "nseq %d not in [1, 16]", nseq);
  const lsa::Index* h0 = reinterpret_cast<const lsa::Index*>(hs[0]);
  if (!h0 || h0->magic != lsa::kMagic) return lsa::fail_status(LSA_E_STATE, "index 0 not initialised");
  size_t need = 0;
  if (int e = lsa_workspace_bytes(LSA_OP_DECODE, &h0->prm, sp, ap, nseq, &need)) return e;
  if (need > kScratchBytes)
    return lsa::fail_status(LSA_E_CAPACITY,
                            "decode step needs %zu bytes of workspace; the no-allocation entry point "
                            "holds %zu (use lsa_decode_step with a caller workspace)",
                            need, kScratchBytes);
  void* ws = nullptr;
  if (int e = scratch_ptr(&ws)) return e;
  return lsa_decode_step(hs, nseq, d_latk_new, d_latq, d_q, d_k, d_v, seq_stride_rows, sp, ap, d_out,
                         ws, kScratchBytes, stream);
}

}  // extern "C"
