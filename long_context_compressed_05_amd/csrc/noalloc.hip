// csa_hca_decode_noalloc: the one-launch decode step on a scratch buffer the
// library holds, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The fused decode's workspace (candidate keys, lists, partials, control
// words) lives in the file-scope array `scratch` below: one copy per GPU,
// kScratchBytes long, held until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is only a stand-in): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
//
// The fused kernel needs its workspace zero-filled whenever the layout
// changes (its words carry a launch-epoch tag, and a word of one layout read
// under another could match a tag by chance).  The entry point records, per
// device, the layout of the last launch it made; before the first launch on a
// device and before any launch whose layout differs from the last one's it
// clears the bytes the new layout uses with a fill kernel on the caller's
// stream (no memset node, so the step stays capturable).  Launches of the
// same layout reuse the words as the caller-owned workspace does.  Every call
// on a device shares its array: calls that overlap on one GPU (other streams,
// other host threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/csa.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// the arguments the fused plan (the workspace layout) is made from
struct Layout {
  int R, H, k, W, W_hca;
  int64_t max_pool, max_hpool;
  bool operator==(const Layout& o) const {
    return R == o.R && H == o.H && k == o.k && W == o.W && W_hca == o.W_hca && max_pool == o.max_pool &&
           max_hpool == o.max_hpool;
  }
};

struct DeviceScratch {
  void* ptr = nullptr;  // device address of `scratch` on this device
  bool launched = false;
  Layout last{};        // layout of the last launch made on this device
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ __launch_bounds__(256) void k_zero16(uint4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

namespace csa {

int noalloc_prepare(int R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca, hipStream_t stream,
                    void** ws, size_t* ws_bytes, const char** err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *err = "no usable HIP device (or a device index beyond 63)";
    return CSA_ERR_DEVICE;
  }
  const FusedPlan pl = plan_fused(R, max_pool, max_hpool, H, k, W, W_hca);
  if (pl.grid <= 0) {
    *err = "could not size the fused decode launch on this device";
    return CSA_ERR_DEVICE;
  }
  if (pl.ws_bytes > kScratchBytes) {
    *err = "the step needs more scratch than the library's static 64 MiB (use csa_hca_decode with a workspace)";
    return CSA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& ds = g_dev[dev];
  if (!ds.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *err = "hipGetSymbolAddress of the static scratch failed";
      return CSA_ERR_DEVICE;
    }
    ds.ptr = p;
  }
  const Layout lay{R, H, k, W, W_hca, max_pool, max_hpool};
  if (!ds.launched || !(ds.last == lay)) {
    // a new layout: clear the bytes it uses (and any longer tail of the last one
    // stays as it is: the new layout never reads it)
    const size_t n16 = (pl.ws_bytes + 15) / 16;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 2048 ? (n16 + 255) / 256 : 2048);
    if (launch(-1, kProfNone, k_zero16, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, (uint4*)ds.ptr, n16) !=
        hipSuccess) {
      (void)hipGetLastError();
      *err = "launch of the scratch clearing kernel failed";
      return CSA_ERR_DEVICE;
    }
    ds.launched = true;
    ds.last = lay;
  }
  *ws = ds.ptr;
  *ws_bytes = kScratchBytes;
  return CSA_OK;
}

}  // namespace csa
