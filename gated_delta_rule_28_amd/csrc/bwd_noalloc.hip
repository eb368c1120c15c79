// gdr_chunk_bwd_noalloc: gdr_chunk_bwd with its workspace in a static device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving or training loops, harnesses that forbid hipMalloc).
//
// The array lives in this library's device code object: every GPU the
// library runs on holds one copy of kScratchBytes until the process ends.
// Its device address is looked up once per device (hipGetSymbolAddress with
// that device current) and kept; host code passes that address, never the
// array's name, which in host code is only a host-side stand-in.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdr.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // GDR_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GDR_NOALLOC_SCRATCH_BYTES, "header and library agree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_ptr[kMaxDevices];        // device address of `scratch`, per device (null: not yet)

// the current device's address of `scratch`, looked up on first use
int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDR_EHIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDR_EHIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" int gdr_chunk_bwd_noalloc(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int in_dtype, int gate, const void *q, const void *k,
                                     const void *v, const float *beta, const float *log_alpha,
                                     const float *initial_state, const void *d_o,
                                     const float *d_final_state, float *dq, float *dk,
                                     float *dv, float *dbeta, float *dlog_alpha,
                                     float *d_initial_state, hipStream_t stream) {
  // sizes beyond the array are refused before anything is looked up or launched
  const size_t need =
      gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, gate);
  if (need > kScratchBytes) return GDR_EWORKSPACE;
  void *ws = nullptr;
  if (need > 0) {
    const int st = scratch_ptr(&ws);
    if (st != GDR_OK) return st;
  }
  // the workspace's contents on entry are ignored: nothing needs clearing
  return gdr_chunk_bwd(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
                       initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                       d_initial_state, ws, need > 0 ? kScratchBytes : 0, stream);
}
