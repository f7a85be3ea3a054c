// Per-group workloads and step statistics.
// "EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.3: w^(l) = (w_1, ..., w_D) across D devices, Eq. (2) effective workload
// max_d w_d, Eq. (3) utilisation; Figure 1's even expert-device mapping puts
// experts [d*E/D, (d+1)*E/D) on group d.  One block; integer only.
#include "cle_internal.h"

namespace cle {
namespace {

constexpr int kMaxCells = 8192;  // n * D

__global__ __launch_bounds__(1024) void workload_stats_kernel(const int* __restrict__ counts,
                                                              int n, int E, int D, uint64_t mask,
                                                              int* __restrict__ w,
                                                              long long* __restrict__ acc) {
  __shared__ int sw[kMaxCells];
  __shared__ long long s_sum, s_max, s_sep;
  const int g = E / D;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_sum = 0;
    s_max = 0;
    s_sep = 0;
  }
  for (int p = tid; p < n * D; p += blockDim.x) {
    const int j = p / D, d = p % D;
    const int* c = counts + static_cast<int64_t>(j) * E + static_cast<int64_t>(d) * g;
    int s = 0;
    for (int e = 0; e < g; ++e) s += c[e];
    sw[p] = s;
    w[p] = s;
  }
  __syncthreads();
  if (mask == 0) return;  // uniform across the block
  // W_d of the step and its sum / max
  for (int d = tid; d < D; d += blockDim.x) {
    long long Wd = 0;
    for (int j = 0; j < n; ++j)
      if ((mask >> j) & 1ull) Wd += sw[j * D + d];
    atomicAdd(reinterpret_cast<unsigned long long*>(&s_sum), static_cast<unsigned long long>(Wd));
    atomicMax(reinterpret_cast<unsigned long long*>(&s_max), static_cast<unsigned long long>(Wd));
  }
  // each member's own peak (the same work run alone)
  for (int j = tid; j < n; j += blockDim.x) {
    if (!((mask >> j) & 1ull)) continue;
    int mx = 0;
    for (int d = 0; d < D; ++d) mx = sw[j * D + d] > mx ? sw[j * D + d] : mx;
    atomicAdd(reinterpret_cast<unsigned long long*>(&s_sep), static_cast<unsigned long long>(mx));
  }
  __syncthreads();
  if (tid == 0) {
    acc[0] += s_sum;
    acc[1] += s_max;
    acc[2] += s_sep;
    acc[3] += 1;
  }
}

}  // namespace
}  // namespace cle

extern "C" cle_status cle_workload_stats(const int32_t* counts, int32_t n, int32_t E, int32_t D,
                                         uint64_t runset_mask, int32_t* w, int64_t* acc,
                                         void* stream) {
  using namespace cle;
  if (!counts || !w) return CLE_EINVAL;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || E < 1 || D < 1 || E % D) return CLE_EINVAL;
  if (static_cast<int64_t>(n) * D > kMaxCells) return CLE_EUNSUPPORTED;
  if (n < 64 && (runset_mask >> n) != 0) return CLE_EINVAL;
  if (runset_mask != 0 && !acc) return CLE_EINVAL;
  workload_stats_kernel<<<dim3(1), dim3(1024), 0, as_stream(stream)>>>(
      counts, n, E, D, runset_mask, w, reinterpret_cast<long long*>(acc));
  return launch_status();
}
