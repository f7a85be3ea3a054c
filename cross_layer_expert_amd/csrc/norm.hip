// RMS normalisation of the MoE block's input rows: y = x / sqrt(mean(x^2) + eps).
// "EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.1: the MoE of layer l takes the post-attention state h'_l and its output
// is added to it.  The expert input is normalised first (a unit-weight RMS
// norm) while the residual keeps the raw state, so the residual stream stays
// bounded over many layers.
//
// One wavefront per row (the row code is in norm_row.h).
#include "norm_row.h"

namespace cle {
namespace {

struct NormArgs {
  const void* x[CLE_MAX_MICROBATCHES];
  void* y[CLE_MAX_MICROBATCHES];
  const cle_loop_state* st;  // non-NULL: only micro-batches in st->todo
};

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a, int T_, int H, float eps) {
  const int j = blockIdx.y;
  if (a.st && !(a.st->todo >> j & 1)) return;  // uniform over the block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T_) return;
  rmsnorm_row<T>(static_cast<const T*>(a.x[j]) + static_cast<int64_t>(t) * H,
                 static_cast<T*>(a.y[j]) + static_cast<int64_t>(t) * H, H, eps, lane);
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
