// The allocation-free forward: pack3d_forward with its workspace in a static
// device array instead of a caller buffer, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The launches and kernels are the forward's own.
#include <mutex>

#include "pack3d_internal.h"

namespace {

// The forward's workspace (rotated Q/K, summaries, the fp32 local branch,
// summary norms) for problems that need at most PACK3D_NOALLOC_SCRATCH_BYTES.
// Every device the library runs on holds its own copy until the process ends.
// In host code this name is a host-side stand-in, never a device address:
// host code uses only the per-device address looked up below.
static __device__ __align__(256) char scratch[PACK3D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pack3d::api_fail(PACK3D_ERR_HIP, "pack3d_forward_noalloc: hipGetDevice: %s",
                            hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pack3d::api_fail(PACK3D_ERR_UNSUPPORTED,
                            "pack3d_forward_noalloc: device %d beyond the %d supported", dev,
                            kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pack3d::api_fail(PACK3D_ERR_HIP,
                              "pack3d_forward_noalloc: hipGetSymbolAddress(scratch) on device "
                              "%d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return PACK3D_OK;
}

}  // namespace

extern "C" int pack3d_forward_noalloc(const pack3d_problem* prob, const void* q,
                                      const void* k_loc, const void* v_loc, const void* k_cmp,
                                      const void* v_cmp, const float* a, const int32_t* coords,
                                      const int32_t* cell_to_pos, const float* gate_logits,
                                      void* out, void* stream) {
  static const char* fn = "pack3d_forward_noalloc";
  const pack3d::FwdArgs x{q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate_logits, out};
  pack3d::Geom g;
  int rc = pack3d::forward_check(fn, prob, x, &g);
  if (rc) return rc;
  const size_t need = pack3d::forward_workspace_bytes(g);
  if (need > (size_t)PACK3D_NOALLOC_SCRATCH_BYTES)
    return pack3d::api_fail(PACK3D_ERR_WORKSPACE,
                            "%s: the problem needs %zu bytes of workspace, more than the %zu of "
                            "the static scratch array (use pack3d_forward with a workspace)",
                            fn, need, (size_t)PACK3D_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return pack3d::forward_launch(g, x, ws, (hipStream_t)stream, nullptr);
}
