// Allocation-free decode: ss_attn_decode with the split workspace taken from
// a fixed device array of this library instead of caller memory, for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops, hosts that forbid allocation).
//
// The array lives for the whole process on every GPU the library runs on.
// Host code never uses its name as an address: at the first call on a device
// (with that device current) its device address is looked up once with
// hipGetSymbolAddress and kept per device; kernels receive that pointer as
// they receive a caller's workspace.  Nothing in it must start at zero:
// published running maxima carry a launch tag, and every other region is
// written before it is read within one call.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "launch.h"
#include "ss_attn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)SS_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
    return ssattn::report_error(SS_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return ssattn::report_error(SS_ERR_UNSUPPORTED, "device index outside the scratch table");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s",
               e != hipSuccess ? hipGetErrorString(e) : "null address");
      return ssattn::report_error(SS_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SS_OK;
}

}  // namespace

extern "C" int ss_attn_decode_noalloc(const void* q, const void* k, const void* v, void* out,
                                      int B, int Hq, int Hkv, int Lk, int D, int Dv, float scale,
                                      float threshold, int num_splits, uint8_t* skip_mask_out,
                                      hipStream_t stream) {
  if (!out) return ssattn::report_error(SS_ERR_INVALID_ARG, "out must be non-null");
  ss_decode_params p{q, k, v, out, B, Hq, Hkv, Lk, D, Dv, scale, threshold, num_splits,
                     SS_SPLIT_CHAINED, skip_mask_out, nullptr, 0};
  if (num_splits == 0) {
    const size_t need = ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, 0);
    if (need > kScratchBytes) {
      // Chained decisions do not depend on the split count: take the largest
      // count below the automatic one whose workspace fits.
      for (int s = ss_decode_num_splits(B, Hq, Hkv, Lk, D, Dv) - 1; s >= 1; --s) {
        if (ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, s) <= kScratchBytes) {
          p.num_splits = s;
          break;
        }
      }
    }
  }
  // Every host-side check first, against the array's size, with a stand-in
  // address that is only compared with null (nothing is launched here).
  p.workspace = &g_mutex;
  p.workspace_bytes = kScratchBytes;
  if (int rc = ssattn::validate_decode(&p)) {
    if (rc != SS_ERR_WORKSPACE) return rc;
    char msg[320];
    snprintf(msg, sizeof(msg),
             "this decode needs %zu bytes of split workspace; the allocation-free entry point "
             "holds %zu (use ss_attn_decode with a caller workspace, or fewer splits)",
             ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, p.num_splits), kScratchBytes);
    return ssattn::report_error(SS_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (int rc = scratch_of_current_device(&ws)) return rc;
  p.workspace = ws;
  return ss_attn_decode_ex(&p, stream);
}
