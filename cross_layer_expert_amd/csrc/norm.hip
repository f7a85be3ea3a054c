// RMS normalisation of the MoE block's input rows: y = x / sqrt(mean(x^2) + eps).
// "EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.1: the MoE of layer l takes the post-attention state h'_l and its output
// is added to it.  The expert input is normalised first (a unit-weight RMS
// norm) while the residual keeps the raw state, so the residual stream stays
// bounded over many layers.
//
// One wavefront per row: each lane sums the squares of its 16-byte column
// groups in float32 in column order, the lanes are combined by a fixed
// butterfly, and the row is scaled and rounded once to the storage type.
// The result is bitwise reproducible.
#include "cle_internal.h"

namespace cle {
namespace {

struct NormArgs {
  const void* x[CLE_MAX_MICROBATCHES];
  void* y[CLE_MAX_MICROBATCHES];
  const cle_loop_state* st;  // non-NULL: only micro-batches in st->todo
};

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
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a, int T_, int H, float eps) {
  const int j = blockIdx.y;
  if (a.st && !(a.st->todo >> j & 1)) return;  // uniform over the block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T_) return;
  const T* x = static_cast<const T*>(a.x[j]) + static_cast<int64_t>(t) * H;
  T* y = static_cast<T*>(a.y[j]) + static_cast<int64_t>(t) * H;
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

}  // namespace

cle_status launch_rmsnorm(int n, const void* const* x, void* const* y, int T, int H, float eps,
                          cle_dtype dt, const cle_loop_state* st, hipStream_t s) {
  if (T == 0) return CLE_OK;
  NormArgs a;
  for (int j = 0; j < n; ++j) {
    a.x[j] = x[j];
    a.y[j] = y[j];
  }
  a.st = st;
  const dim3 grid((T + 3) / 4, n);
  if (dt == CLE_BF16)
    rmsnorm_kernel<uint16_t><<<grid, dim3(256), 0, s>>>(a, T, H, eps);
  else
    rmsnorm_kernel<float><<<grid, dim3(256), 0, s>>>(a, T, H, eps);
  return launch_status();
}

}  // namespace cle

extern "C" cle_status cle_rmsnorm_many(int32_t n, const void* const* x, void* const* y, int32_t T,
                                       int32_t H, float eps, cle_dtype dt, void* stream) {
  using namespace cle;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || !x || !y) return CLE_EINVAL;
  if (T < 0 || H < 8 || H % 8 || !(eps >= 0.0f)) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  for (int j = 0; j < n; ++j) {
    if (!x[j] || !y[j] || !aligned(x[j], 16) || !aligned(y[j], 16)) return CLE_EINVAL;
  }
  return launch_rmsnorm(n, x, y, T, H, eps, dt, nullptr, as_stream(stream));
}
