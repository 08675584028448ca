// csa_index_topk without a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// indexer's score scratch lives in a file-scope device array of fixed size instead.
//
// The array is a device symbol: in host code its name is only a stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and
// that address, never the name, is what the kernels receive.  Every call on one GPU shares
// that GPU's copy; it keeps whatever the last call left there.  The indexer reads only the
// scores it has written in the same call (the visible entries of each query), so nothing is
// cleared between calls.  Calls that overlap in time on one GPU (different streams or host
// threads without ordering) race on the array.
#include <mutex>

#include "../../include/dsv4attn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(32) << 20;  // DSV4_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == DSV4_NOALLOC_SCRATCH_BYTES, "header and library agree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first call per device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess)
    return dsv4::report_error(DSV4_ERR_LAUNCH, "csa_index_topk_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return dsv4::report_error(DSV4_ERR_UNSUPPORTED, "csa_index_topk_noalloc: device index above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return dsv4::report_error(DSV4_ERR_LAUNCH, "csa_index_topk_noalloc: hipGetSymbolAddress failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSV4_OK;
}

}  // namespace

extern "C" int csa_index_topk_noalloc(const void* q_idx, const float* w_idx, const void* k_pool,
                                      const int* q_pos0, const int* n_pool, int* topk_idx,
                                      float* topk_score, int B, int T, int nI, int cI, int N_cap,
                                      int m, int k, int dtype, void* stream) {
  const size_t need = csa_index_topk_workspace_size(B, T, N_cap, k);
  if (need > kScratchBytes)
    return dsv4::report_error(DSV4_ERR_UNSUPPORTED,
                              "csa_index_topk_noalloc: B*T*N_cap*4 bytes of scores exceed the "
                              "32 MiB static scratch; call csa_index_topk with a workspace");
  void* ptr = nullptr;
  if (B > 0 && T > 0) {
    const int rc = scratch_address(&ptr);
    if (rc != DSV4_OK) return rc;
  }
  return csa_index_topk(q_idx, w_idx, k_pool, q_pos0, n_pool, topk_idx, topk_score, B, T, nI, cI,
                        N_cap, m, k, ptr, kScratchBytes, dtype, stream);
}
