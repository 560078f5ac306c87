// device.h -- small gfx950 device helpers: native vector types, bf16 unpack
// and pack, exact bf16 rounding of a product, cache-policy stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 values of a 16-byte vector -> fp32 (exact).
__device__ __forceinline__ void unpack8(const u32x4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  u32x4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

// bf16 nearest (ties to even) to the exact product a*b.  The fp32 product p
// can only differ from the exact value on the bf16 side of a rounding
// boundary when p lands exactly on a bf16 midpoint (midpoints are fp32
// values); there the sign of the exact error fma(a, b, -p) decides.
__device__ __forceinline__ uint32_t bf16_of_product(float a, float b) {
  float p = a * b;
  float e = __builtin_fmaf(a, b, -p);
  uint32_t u = __float_as_uint(p);
  if ((u & 0xFFFFu) == 0x8000u && e != 0.0f) {
    bool away = (e > 0.0f) == (p > 0.0f);
    return (u >> 16) + (away ? 1u : 0u);
  }
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Streaming store: the line is not kept in the caches (written once, read by
// a later kernel long after it would have been evicted).
template <typename V>
__device__ __forceinline__ void store_stream(V *p, const V &v) {
  __builtin_nontemporal_store(v, p);
}

template <typename V>
__device__ __forceinline__ V load_stream(const V *p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Instantiate a kernel for the common top-k values; 0 = any k <= 16.
#define EP_K_SWITCH(k, F) \
  switch (k) {            \
    case 1: F(1); break;  \
    case 2: F(2); break;  \
    case 4: F(4); break;  \
    case 8: F(8); break;  \
    default: F(0); break; \
  }

}  // namespace epk
