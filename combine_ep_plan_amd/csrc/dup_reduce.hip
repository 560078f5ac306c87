// dup_reduce.hip -- fold duplicated-expert gradients into the owner's
// gradients (MoonEP article, paragraph 5: a dedicated reduce buffer carries
// replica gradients back to the owner's local parameter gradients).
//
// Grid: y = replica i, x = 8-element vectors of the parameter slice.  Only
// the first replica of each owner does work: it loads the owner's fp32
// values once, adds every replica of that owner in replica order in fp64,
// rounds once to fp32 and stores.  Owners are therefore read and written
// once, replicas read once, and the result does not depend on scheduling.
#include "device.h"
#include "ep_internal.h"

namespace epk {

__global__ __launch_bounds__(256) void k_dup_reduce(const uint16_t *__restrict__ rep,
                                                    const int32_t *__restrict__ rep_e,
                                                    int32_t n, int64_t P, int32_t E_owner,
                                                    float *__restrict__ owner,
                                                    uint32_t *__restrict__ status) {
  const int32_t i = blockIdx.y;
  const int32_t e = rep_e[i];
  if (e < 0 || e >= E_owner) {
    if (e != -1 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, kFlagIndexRange);
    return;
  }
  for (int32_t i2 = 0; i2 < i; ++i2)
    if (rep_e[i2] == e) return;  // an earlier replica of this owner does the work
  const int64_t p0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (p0 >= P) return;
  float *o = owner + (int64_t)e * P + p0;
  if ((P & 7) == 0) {
    const f32x4 a = reinterpret_cast<const f32x4 *>(o)[0];
    const f32x4 b = reinterpret_cast<const f32x4 *>(o)[1];
    double acc[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    for (int32_t i2 = i; i2 < n; ++i2) {
      if (rep_e[i2] != e) continue;
      float f[8];
      unpack8(*reinterpret_cast<const u32x4 *>(rep + (int64_t)i2 * P + p0), f);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += (double)f[c];
    }
    reinterpret_cast<f32x4 *>(o)[0] = f32x4{(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
    reinterpret_cast<f32x4 *>(o)[1] = f32x4{(float)acc[4], (float)acc[5], (float)acc[6], (float)acc[7]};
  } else {
    const int cnt = (int)((P - p0) < 8 ? (P - p0) : 8);
    for (int c = 0; c < cnt; ++c) {
      double acc = o[c];
      for (int32_t i2 = i; i2 < n; ++i2)
        if (rep_e[i2] == e) acc += (double)__uint_as_float((uint32_t)rep[(int64_t)i2 * P + p0 + c] << 16);
      o[c] = (float)acc;
    }
  }
}

hipError_t launch_dup_reduce(const uint16_t *rep, const int32_t *rep_e, int32_t n, int64_t P,
                             int32_t E_owner, float *owner, uint32_t *status, hipStream_t s) {
  if (n == 0 || P == 0) return hipSuccess;
  const int64_t blocks = (P + 8 * 256 - 1) / (8 * 256);
  hipLaunchKernelGGL(k_dup_reduce, dim3((unsigned)blocks, (unsigned)n), dim3(256), 0, s, rep,
                     rep_e, n, P, E_owner, owner, status);
  return hipGetLastError();
}

}  // namespace epk
