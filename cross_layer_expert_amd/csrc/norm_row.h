// One row of the RMS normalisation y = x / sqrt(mean(x^2) + eps), by one
// wavefront: each lane sums the squares of its 16-byte column groups in
// float32 in column order, the lanes are combined by a fixed butterfly, and
// the row is scaled and rounded once to the storage type (bitwise
// reproducible).  Shared by the normalisation kernel and the launch that
// normalises rows next to the router's top-k.
#pragma once
#include "cle_internal.h"

namespace cle {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* f) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* f);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

template <typename T>
__device__ __forceinline__ void rmsnorm_row(const T* x, T* y, int H, float eps, int lane) {
  float ss = 0.f;
  for (int c = lane * 8; c < H; c += kWave * 8) {
    float f[8];
    load8<T>(x + c, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  for (int c = lane * 8; c < H; c += kWave * 8) {
    float f[8];
    load8<T>(x + c, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] *= r;
    store8<T>(y + c, f);
  }
}

}  // namespace cle
