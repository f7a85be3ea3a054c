// Gate-weighted combine of each token's expert outputs, plus shared experts
// and the residual.  "EasyBalance: Cross-Layer Load Balancing in Distributed
// MoE Inference", Eq. (1): MLP(h'_l) = sum_{i in I_l} W_{l,i} expert_i(h'_l),
// and §2.1: h_{l+1} = h'_l + MLP(h'_l).
//
// One wavefront per token; each lane owns 16-byte column groups.  The sum is
// taken in float32 in a fixed order (slots, shared experts, residual) and
// rounded once, so it is deterministic and a gather, never a scatter-add.
#include "cle_internal.h"

namespace cle {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  // 16 bytes as loaded: 8 bf16 values, widened only when used, so the k slot
  // rows in flight take 4 registers each instead of 8
  using Raw = uint4;
  __device__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  // a row no other wavefront reads: non-temporal (it does not displace reused lines)
  __device__ static Raw load_once(const uint16_t* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ static void unpack(const Raw& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void load(const uint16_t* p, float* f) { unpack(load_raw(p), f); }
  __device__ static void store(uint16_t* p, const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  using Raw = float4;
  __device__ static Raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static Raw load_once(const float* p) { return load_raw(p); }
  __device__ static void unpack(const Raw& v, float* f) {
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  }
  __device__ static void load(const float* p, float* f) { unpack(load_raw(p), f); }
  __device__ static void store(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

// Buffers of the micro-batches of one launch (blockIdx.y picks one).
struct CombineArgs {
  const void* yp[CLE_MAX_MICROBATCHES];
  const int* dest[CLE_MAX_MICROBATCHES];
  const float* gate[CLE_MAX_MICROBATCHES];
  const void* y_shared[CLE_MAX_MICROBATCHES];
  const void* residual[CLE_MAX_MICROBATCHES];
  void* y[CLE_MAX_MICROBATCHES];
  const cle_loop_state* st;  // non-NULL: only the members of st->runset
  // With a state and h0: in a step that restarted the loop, y_j = h0_j for
  // every micro-batch instead (the run starts over from the initial states).
  const void* h0[CLE_MAX_MICROBATCHES];
  bool restart;
};
static_assert(sizeof(CombineArgs) <= 4096, "kernel argument size");

// KMAX > 0: k <= KMAX slots, whose destinations and gates are held in
// registers so that all slot rows of a column chunk are requested before the
// first one is used.  KMAX == 0: any k, one slot at a time.  Both sum the
// slots in order 0..k-1.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs args, int T_, int k, int H,
                                                      int n_shared) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (args.st) {  // uniform over the block
    if (args.restart && args.st->restarted) {
      if (t >= T_) return;
      const int64_t nv = static_cast<int64_t>(H) * sizeof(T) / 16;
      const uint4* src = static_cast<const uint4*>(args.h0[blockIdx.y]) + t * nv;
      uint4* dst = static_cast<uint4*>(args.y[blockIdx.y]) + t * nv;
      for (int64_t c = lane; c < nv; c += kWave) dst[c] = src[c];
      return;
    }
    if (!(args.st->runset >> blockIdx.y & 1)) return;
  }
  const T* __restrict__ yp = static_cast<const T*>(args.yp[blockIdx.y]);
  const int* __restrict__ dest = args.dest[blockIdx.y];
  const float* __restrict__ gate = args.gate[blockIdx.y];
  const T* __restrict__ y_shared = static_cast<const T*>(args.y_shared[blockIdx.y]);
  const T* residual = static_cast<const T*>(args.residual[blockIdx.y]);
  T* y = static_cast<T*>(args.y[blockIdx.y]);
  constexpr int N = Vec<T>::N;
  if (t >= T_) return;
  const int* drow = dest + static_cast<int64_t>(t) * k;
  const float* grow = gate + static_cast<int64_t>(t) * k;
  int d[KMAX > 0 ? KMAX : 1];
  float g[KMAX > 0 ? KMAX : 1];
  if (KMAX > 0) {
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      d[s] = s < k ? drow[s] : -1;
      g[s] = s < k ? grow[s] : 0.0f;
    }
  }
  for (int c = lane * N; c < H; c += kWave * N) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    if (KMAX > 0) {
      typename Vec<T>::Raw raw[KMAX > 0 ? KMAX : 1];
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (d[s] >= 0) raw[s] = Vec<T>::load_once(yp + static_cast<int64_t>(d[s]) * H + c);
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (d[s] >= 0) {
          float v[N];
          Vec<T>::unpack(raw[s], v);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[i] = fmaf(g[s], v[i], acc[i]);
        }
    } else {
      for (int s = 0; s < k; ++s) {
        const int ds = drow[s];
        if (ds < 0) continue;
        const float gs = grow[s];
        float v[N];
        Vec<T>::load(yp + static_cast<int64_t>(ds) * H + c, v);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = fmaf(gs, v[i], acc[i]);
      }
    }
    for (int q = 0; q < n_shared; ++q) {
      float v[N];
      Vec<T>::load(y_shared + (static_cast<int64_t>(q) * T_ + t) * H + c, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    if (residual) {
      float v[N];
      Vec<T>::load(residual + static_cast<int64_t>(t) * H + c, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    Vec<T>::store(y + static_cast<int64_t>(t) * H + c, acc);
  }
}

template <typename T>
void launch_combine(const CombineArgs& a, int n, int T_, int k, int H, int ns, hipStream_t s) {
  const dim3 grid((T_ + 3) / 4, n);
  if (k <= 8)
    combine_kernel<T, 8><<<grid, dim3(256), 0, s>>>(a, T_, k, H, ns);
  else
    combine_kernel<T, 0><<<grid, dim3(256), 0, s>>>(a, T_, k, H, ns);
}

}  // namespace
}  // namespace cle

extern "C" cle_status cle_combine(const void* yp, const int32_t* dest, const float* topk_gate,
                                  int32_t T, int32_t k, int32_t H, const void* y_shared,
                                  int32_t n_shared, const void* residual, void* y, cle_dtype dt,
                                  void* stream) {
  return cle_combine_many(1, &yp, &dest, &topk_gate, T, k, H, &y_shared, n_shared, &residual, &y,
                          dt, stream);
}

extern "C" cle_status cle_combine_many(int32_t n, const void* const* yp,
                                       const int32_t* const* dest,
                                       const float* const* topk_gate, int32_t T, int32_t k,
                                       int32_t H, const void* const* y_shared, int32_t n_shared,
                                       const void* const* residual, void* const* y, cle_dtype dt,
                                       void* stream) {
  using namespace cle;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || !yp || !dest || !topk_gate || !y) return CLE_EINVAL;
  if (T < 0 || k < 1 || H < 8 || H % 8 || n_shared < 0) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  if (T == 0) return CLE_OK;
  if (n_shared > 0 && !y_shared) return CLE_EINVAL;
  for (int j = 0; j < n; ++j) {
    const void* ys = y_shared ? y_shared[j] : nullptr;
    const void* res = residual ? residual[j] : nullptr;
    if (!yp[j] || !dest[j] || !topk_gate[j] || !y[j]) return CLE_EINVAL;
    if (n_shared > 0 && !ys) return CLE_EINVAL;
    if (!aligned(yp[j], 16) || !aligned(y[j], 16) || (ys && !aligned(ys, 16)) ||
        (res && !aligned(res, 16)))
      return CLE_EINVAL;
  }
  return launch_combine_many(n, yp, dest, topk_gate, T, k, H, y_shared, n_shared, residual, y, dt,
                             nullptr, as_stream(stream));
}

namespace cle {

cle_status launch_combine_many(int n, const void* const* yp, const int* const* dest,
                               const float* const* gate, int T, int k, int H,
                               const void* const* y_shared, int n_shared,
                               const void* const* residual, void* const* y, cle_dtype dt,
                               const cle_loop_state* st, hipStream_t s, const void* const* h0) {
  CombineArgs a;
  for (int j = 0; j < n; ++j) {
    a.yp[j] = yp[j];
    a.dest[j] = dest[j];
    a.gate[j] = gate[j];
    a.y_shared[j] = y_shared ? y_shared[j] : nullptr;
    a.residual[j] = residual ? residual[j] : nullptr;
    a.y[j] = y[j];
    a.h0[j] = h0 ? h0[j] : nullptr;
  }
  a.st = st;
  a.restart = st && h0;
  if (dt == CLE_BF16)
    launch_combine<uint16_t>(a, n, T, k, H, n_shared, s);
  else
    launch_combine<float>(a, n, T, k, H, n_shared, s);
  return launch_status();
}

}  // namespace cle
