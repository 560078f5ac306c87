// scratch.hip -- the library's static device scratch: the workspace of the
// handles that ep_handle_create_static makes, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy at its own address until the process ends.  In host code its
// name is only a host-side stand-in, so the device address is taken once per
// device with hipGetSymbolAddress (that device current) and used everywhere
// host code needs the memory (kernel arguments, the clearing kernel).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ep_internal.h"

namespace epk {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_base[kMaxDevices];  // device address of `scratch` on each device, once known
}  // namespace

// Device address of the scratch array on the current device (*dev receives
// the device ordinal).
hipError_t scratch_base(int *dev, void **base) {
  int d = 0;
  hipError_t err = hipGetDevice(&d);
  if (err != hipSuccess) return err;
  if (d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_base[d]) {
    void *ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_base[d] = ptr;
  }
  *dev = d;
  *base = g_base[d];
  return hipSuccess;
}

// Zero `words` 16-byte words at p (a kernel, not a memset, so the call can be
// captured into a graph and replayed).
__global__ __launch_bounds__(256) void k_zero(uint4 *__restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)((bytes + 15) / 16);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint4 *>(p), words);
  return hipGetLastError();
}

}  // namespace epk
