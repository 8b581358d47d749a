// Hash-sparse forward that allocates nothing and takes no workspace: its
// scratch (block statistics, bucket segments, live-tile lists) lives in a
// file-scope device array of fixed size, one copy per GPU, held until the
// process ends.  For callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array's name is only a host-side stand-in for the device symbol; its
// device address is looked up once per device with hipGetSymbolAddress and
// cached, and only that address is handed to the kernels (as the workspace of
// scfa_hash_sparse_fwd).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/scfa.h"
#include "scfa_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch` (looked up on first use).
hipError_t scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t scfa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int scfa_hash_sparse_fwd_noalloc(const void *q, const void *k, const void *v, const int32_t *q_idx,
                                 const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash, void *o,
                                 float *lse, int B, int H, int Tq, int Tk, int d, int block, float scale, int dtype,
                                 unsigned flags, void *stream) {
  const size_t need = scfa_workspace_size(SCFA_OP_HASH_FWD, B, H, Tq, Tk, d, block, 0);
  char msg[256];
  if (need > kScratchBytes) {  // checked on the host, before any device call
    snprintf(msg, sizeof(msg), "scratch needed (%zu bytes) exceeds the static scratch of %zu bytes", need,
             kScratchBytes);
    return scfa::report_error(SCFA_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  void *ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "static scratch lookup: HIP error %d (%s)", (int)e, hipGetErrorString(e));
    return scfa::report_error(SCFA_ERR_HIP, msg);
  }
  return scfa_hash_sparse_fwd(q, k, v, q_idx, k_idx, q_hash, k_hash, o, lse, B, H, Tq, Tk, d, block, scale, dtype,
                              flags, ws, kScratchBytes, stream);
}

}  // extern "C"
