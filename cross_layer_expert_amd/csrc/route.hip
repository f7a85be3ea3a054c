// Router top-k with renormalised softmax gates.
// "EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.1: W_l, I_l = topk(G(h'_l)); here the router scores are given.
//
// One wavefront per token.  Each lane holds up to VPL logits as 64-bit keys
//   key = (order-preserving bits of the logit) << 32 | (0xffffffff - expert)
// so that an unsigned max picks the largest logit and, among equal logits,
// the smallest expert id.  Each of the k rounds is one wave-wide max; the
// winner's key is cleared.  Key 0 never belongs to a finite logit.
//
// A launch can also carry the RMS normalisation of the micro-batches' rows
// (norm_row.h) in blocks of its own after the routing blocks: the two jobs
// are independent when the scores are given, and one launch does both.
#include <type_traits>

#include "norm_row.h"

namespace cle {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

// Buffers of the micro-batches of one launch (blockIdx.y picks one).  With a
// loop state, only the micro-batches in its `todo` mask are routed, each at
// its layer l_j: logits[j] is then the base of [L, T, E].
struct RouteArgs {
  const float* logits[CLE_MAX_MICROBATCHES];
  int* idx[CLE_MAX_MICROBATCHES];
  float* gate[CLE_MAX_MICROBATCHES];
  const cle_loop_state* st;
  int64_t layer_stride;
  // normalisation blocks (blockIdx.x >= route_blocks): rows of nx[j] into ny[j]
  const void* nx[CLE_MAX_MICROBATCHES];
  void* ny[CLE_MAX_MICROBATCHES];
  int route_blocks;
  int H;
  float eps;
};
static_assert(sizeof(RouteArgs) <= 4096, "kernel argument size");

__device__ __forceinline__ uint32_t ord_bits(float z) {
  if (z == 0.0f) z = 0.0f;  // -0.0 and +0.0 are the same logit
  uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_ord_bits(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}

// One DPP step of the wave-wide unsigned 64-bit max: each lane takes the max
// of its key and the key DPP control CTRL moves to it (rows of ROW_MASK only;
// a lane whose source is outside its row reads 0, the neutral key).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xf, true));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, ROW_MASK, 0xf, true));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > v ? o : v;
}

// Max of the 64 lanes' keys, in every lane: shifts by 1, 2, 4 and 8 lanes
// leave each 16-lane row's max in its last lane, the broadcasts of lanes 15
// and 31 carry it into the following rows, and lane 63 ends with the max of
// all (register-to-register moves instead of LDS permutes).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// NT: element type of the rows to normalise in the same launch, or void.
// KSEL: slots the selected scores are kept for (k <= KSEL); the LDS a block
// holds, and so the blocks a CU runs at once, scale with it.
template <int VPL, typename NT, int KSEL = CLE_MAX_E>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs args, int T, int E, int k) {
  const int j = blockIdx.y;
  if constexpr (!std::is_void<NT>::value) {
    if (static_cast<int>(blockIdx.x) >= args.route_blocks) {  // uniform over the block
      if (args.st && !(args.st->todo >> j & 1)) return;
      const int nwave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
      const int t = (blockIdx.x - args.route_blocks) * kRouteWaves + nwave;
      if (t >= T) return;
      const int64_t off = static_cast<int64_t>(t) * args.H;
      rmsnorm_row<NT>(static_cast<const NT*>(args.nx[j]) + off, static_cast<NT*>(args.ny[j]) + off,
                      args.H, args.eps, threadIdx.x % kWave);
      return;
    }
  }
  const float* __restrict__ logits = args.logits[j];
  if (args.st) {  // uniform over the block
    if (!(args.st->todo >> j & 1)) return;
    logits += static_cast<int64_t>(args.st->layer[j]) * args.layer_stride;
  }
  int* __restrict__ idx = args.idx[j];
  float* __restrict__ gate = args.gate[j];
  __shared__ float zsel[kRouteWaves][KSEL];
  __shared__ int esel[kRouteWaves][KSEL];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kRouteWaves + wave;
  if (t >= T) return;  // whole wavefront leaves; no block barrier follows

  const float* row = logits + static_cast<int64_t>(t) * E;
  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane * VPL + v;
    key[v] = 0;
    if (e < E)
      key[v] = (static_cast<uint64_t>(ord_bits(row[e])) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
  }

  double z0 = 0.0;
  for (int s = 0; s < k; ++s) {
    uint64_t best = key[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (key[v] == best) key[v] = 0;
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    const float z = from_ord_bits(static_cast<uint32_t>(best >> 32));
    // every lane holds the same (z, e); all lanes store the same value
    zsel[wave][s] = z;
    esel[wave][s] = e;
    if (s == 0) z0 = static_cast<double>(z);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // The k terms exp(z_s - z0) in float64, slot s on lane s % 64, summed in
  // slot order (the same sum, term for term, as a serial loop over s).
  double total = 0.0;
  for (int s0 = 0; s0 < k; s0 += kWave) {
    const int s = s0 + lane;
    const double ex = s < k ? exp(static_cast<double>(zsel[wave][s]) - z0) : 0.0;
    const int m = min(kWave, k - s0);
    for (int q = 0; q < m; ++q) total += __shfl(ex, q, kWave);
  }

  int* irow = idx + static_cast<int64_t>(t) * k;
  float* grow = gate + static_cast<int64_t>(t) * k;
  for (int s = lane; s < k; s += kWave) {
    const double ex = exp(static_cast<double>(zsel[wave][s]) - z0);
    grow[s] = static_cast<float>(ex / total);
    irow[s] = esel[wave][s];
  }
}

}  // namespace
}  // namespace cle

namespace cle {
namespace {

template <typename NT>
void launch_route_kernel(const RouteArgs& a, int n, int T, int E, int k, hipStream_t s) {
  const int rb = (T + kRouteWaves - 1) / kRouteWaves;
  const dim3 grid(std::is_void<NT>::value ? rb : 2 * rb, n), block(256);
  const int vpl = (E + kWave - 1) / kWave;
  if (k <= kWave && vpl <= 2) {  // the common shapes: 2 KiB of LDS per block
    if (vpl <= 1)
      route_kernel<1, NT, kWave><<<grid, block, 0, s>>>(a, T, E, k);
    else
      route_kernel<2, NT, kWave><<<grid, block, 0, s>>>(a, T, E, k);
  } else if (vpl <= 1)
    route_kernel<1, NT><<<grid, block, 0, s>>>(a, T, E, k);
  else if (vpl <= 2)
    route_kernel<2, NT><<<grid, block, 0, s>>>(a, T, E, k);
  else if (vpl <= 4)
    route_kernel<4, NT><<<grid, block, 0, s>>>(a, T, E, k);
  else if (vpl <= 8)
    route_kernel<8, NT><<<grid, block, 0, s>>>(a, T, E, k);
  else
    route_kernel<16, NT><<<grid, block, 0, s>>>(a, T, E, k);
}

}  // namespace

cle_status launch_route(int n, const float* const* logits, int T, int E, int k, int* const* idx,
                        float* const* gate, const cle_loop_state* st, int64_t layer_stride,
                        hipStream_t s, const void* const* norm_x, void* const* norm_y, int H,
                        float eps, cle_dtype norm_dt) {
  RouteArgs a;
  for (int j = 0; j < n; ++j) {
    a.logits[j] = logits[j];
    a.idx[j] = idx[j];
    a.gate[j] = gate[j];
    a.nx[j] = norm_x ? norm_x[j] : nullptr;
    a.ny[j] = norm_y ? norm_y[j] : nullptr;
  }
  a.st = st;
  a.layer_stride = layer_stride;
  a.route_blocks = (T + kRouteWaves - 1) / kRouteWaves;
  a.H = H;
  a.eps = eps;
  if (!norm_x)
    launch_route_kernel<void>(a, n, T, E, k, s);
  else if (norm_dt == CLE_BF16)
    launch_route_kernel<uint16_t>(a, n, T, E, k, s);
  else
    launch_route_kernel<float>(a, n, T, E, k, s);
  return launch_status();
}

}  // namespace cle

extern "C" cle_status cle_route(const float* logits, int32_t T, int32_t E, int32_t k,
                                int32_t* topk_idx, float* topk_gate, void* stream) {
  return cle_route_many(1, &logits, T, E, k, &topk_idx, &topk_gate, stream);
}

extern "C" cle_status cle_route_many(int32_t n, const float* const* logits, int32_t T, int32_t E,
                                     int32_t k, int32_t* const* topk_idx,
                                     float* const* topk_gate, void* stream) {
  using namespace cle;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || !logits || !topk_idx || !topk_gate) return CLE_EINVAL;
  if (T < 0 || E < 1 || E > CLE_MAX_E || k < 1 || k > E) return CLE_EINVAL;
  if (T == 0) return CLE_OK;
  for (int j = 0; j < n; ++j)
    if (!logits[j] || !topk_idx[j] || !topk_gate[j]) return CLE_EINVAL;
  return launch_route(n, logits, T, E, k, topk_idx, topk_gate, nullptr, 0, as_stream(stream));
}
