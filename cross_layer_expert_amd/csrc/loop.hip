// Device-driven loop: Algorithm 1 of "EasyBalance: Cross-Layer Load
// Balancing in Distributed MoE Inference" (§4.2) with Schedule(S, m) run on
// the device, and the device form of that schedule for callers that keep
// workloads in device memory.
//
// The schedule needs only n x D integers (the paper's "small-sized routing
// metadata"), so it runs as one workgroup between the dispatch and the
// expert launch.  A step is then a fixed sequence of launches whose
// membership masks live in device memory: the host enqueues steps without
// waiting for the stream.
//
// Policies (§4.2 for m; §5.2 for MaxUtil, CumUtil, DiffPeak) follow the
// readings of the host scheduler exactly: U = sum_d W_d / (D max_d W_d),
// compared by cross-multiplication (0 for an all-zero workload); CumUtil and
// DiffPeak scan ids upwards from the first ready one and pad to m with the
// lowest rejected ids; MaxUtil maximises U over subsets of S with |R| >= m,
// ties to the larger set, then to the lexicographically smallest sorted ids.
// The linear scans run on one wavefront, lane d holding group d (D <= 64);
// MaxUtil's subsets are spread over the workgroup and reduced with that
// total order, so the winner does not depend on how the subsets were split.
#include "cle_internal.h"

namespace cle {
namespace {

// MaxUtil spreads its subsets over 1024 threads; the other policies run on
// one wavefront (a smaller launch with less LDS to set up).
constexpr int kSchedThreads = 1024;
constexpr int kScanThreads = 64;
constexpr int kMaxD = CLE_MAX_LOOP_D;
constexpr int kMaxN = CLE_MAX_MICROBATCHES;

struct UtilD {
  int64_t num;  // sum_d W_d
  int64_t den;  // max_d W_d (1 with num 0 for an all-zero workload)
};

__device__ __forceinline__ bool util_gt(UtilD a, UtilD b) {
  return static_cast<__int128>(a.num) * b.den > static_cast<__int128>(b.num) * a.den;
}

// Shared memory of one schedule: workloads and the MaxUtil reduction.
template <int NT>
struct SchedLDS {
  int w[kMaxN][kMaxD];
  int ids[kMaxN];
  int64_t rnum[NT], rden[NT];
  uint64_t rmask[NT];
  int rsize[NT];
  uint64_t result;
};

__device__ uint64_t pad_to_m(uint64_t chosen, uint64_t ready, int m) {
  for (int j = 0; j < kMaxN && static_cast<int>(__popcll(chosen)) < m; ++j) {
    const uint64_t b = 1ull << j;
    if ((ready & b) && !(chosen & b)) chosen |= b;
  }
  return chosen;
}

// Wavefront reductions (every lane gets the result).
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += static_cast<int64_t>(shfl_xor64(v, off));
  return v;
}
__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = shfl_xor64(v, off);
    v = o > v ? o : v;
  }
  return v;
}
// w[j][lane] as a lane value (0 for lanes past D)
template <int NT>
__device__ __forceinline__ int64_t w_lane(const SchedLDS<NT>& L, int j, int D) {
  const int lane = threadIdx.x % kWave;
  return lane < D ? L.w[j][lane] : 0;
}

// First wavefront, lane d holding group d: CumUtil.
template <int NT>
__device__ uint64_t cumutil_wave(SchedLDS<NT>& L, int n, int D, uint64_t ready, int m) {
  uint64_t chosen = 0;
  int64_t W = 0;
  UtilD uw{0, 1};
  for (int j = 0; j < n; ++j) {
    if (!(ready >> j & 1)) continue;
    const int64_t t = W + w_lane(L, j, D);
    const int64_t s = wave_sum(t), mx = static_cast<int64_t>(wave_max(t));
    const UtilD ut = mx == 0 ? UtilD{0, 1} : UtilD{s, mx};
    if (!chosen || util_gt(ut, uw)) {
      W = t;
      uw = ut;
      chosen |= 1ull << j;
    }
  }
  return pad_to_m(chosen, ready, m);
}

// Peak group of micro-batch j (lowest index among equal maxima), on the
// first wavefront.
template <int NT>
__device__ __forceinline__ int peak_wave(const SchedLDS<NT>& L, int j, int D) {
  const int lane = threadIdx.x % kWave;
  const uint64_t key = lane < D ? (static_cast<uint64_t>(L.w[j][lane]) << 32) |
                                      static_cast<uint32_t>(kWave - 1 - lane)
                                : 0;
  return kWave - 1 - static_cast<int>(wave_max(key) & 0xffffffffu);
}

// First wavefront: DiffPeak.
template <int NT>
__device__ uint64_t diffpeak_wave(SchedLDS<NT>& L, int n, int D, uint64_t ready, int m) {
  uint64_t chosen = 0, taken = 0;  // taken: bit d = group d is a chosen member's peak
  for (int j = 0; j < n; ++j) {
    if (!(ready >> j & 1)) continue;
    const int p = peak_wave(L, j, D);
    if (!chosen || !(taken >> p & 1)) {
      chosen |= 1ull << j;
      taken |= 1ull << p;
    }
  }
  return pad_to_m(chosen, ready, m);
}

// a preferred over b (b.size < 0: no candidate yet)?
__device__ __forceinline__ bool better(UtilD ua, int sa, uint64_t ma, UtilD ub, int sb,
                                       uint64_t mb) {
  if (sa < 0) return false;
  if (sb < 0) return true;
  if (util_gt(ua, ub)) return true;
  if (util_gt(ub, ua)) return false;
  if (sa != sb) return sa > sb;
  const uint64_t diff = ma ^ mb;
  return diff && ((ma >> __builtin_ctzll(diff)) & 1);
}

// Whole workgroup: MaxUtil over the subsets of the pool with |R| >= m.
template <int NT>
__device__ void maxutil_block(SchedLDS<NT>& L, int D, uint64_t ready, int m) {
  const int tid = threadIdx.x;
  const int p = __popcll(ready);
  if (tid == 0) {
    int q = 0;
    for (int j = 0; j < kMaxN; ++j)
      if (ready >> j & 1) L.ids[q++] = j;
  }
  __syncthreads();
  UtilD bu{0, 1};
  int bs = -1;
  uint64_t bm = 0;
  const uint64_t count = 1ull << p;
  for (uint64_t i = 1 + tid; i < count; i += NT) {
    const int size = __popcll(i);
    if (size < m) continue;
    int64_t s = 0, mx = 0;
    for (int d = 0; d < D; ++d) {
      int64_t t = 0;
      for (uint64_t b = i; b; b &= b - 1) t += L.w[L.ids[__builtin_ctzll(b)]][d];
      s += t;
      mx = t > mx ? t : mx;
    }
    uint64_t mask = 0;
    for (uint64_t b = i; b; b &= b - 1) mask |= 1ull << L.ids[__builtin_ctzll(b)];
    const UtilD u = mx == 0 ? UtilD{0, 1} : UtilD{s, mx};
    if (better(u, size, mask, bu, bs, bm)) {
      bu = u;
      bs = size;
      bm = mask;
    }
  }
  L.rnum[tid] = bu.num;
  L.rden[tid] = bu.den;
  L.rsize[tid] = bs;
  L.rmask[tid] = bm;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (tid < off) {
      const int o = tid + off;
      if (better(UtilD{L.rnum[o], L.rden[o]}, L.rsize[o], L.rmask[o],
                 UtilD{L.rnum[tid], L.rden[tid]}, L.rsize[tid], L.rmask[tid])) {
        L.rnum[tid] = L.rnum[o];
        L.rden[tid] = L.rden[o];
        L.rsize[tid] = L.rsize[o];
        L.rmask[tid] = L.rmask[o];
      }
    }
    __syncthreads();
  }
  if (tid == 0) L.result = L.rmask[0];
  __syncthreads();
}

// Whole workgroup: RunSet of the pool `ready` (non-zero) from L.w; the result
// is returned to every thread.
template <int NT>
__device__ uint64_t schedule_block(SchedLDS<NT>& L, int n, int D, uint64_t ready, int m,
                                   int policy) {
  const int pool = __popcll(ready);
  if constexpr (NT == kSchedThreads) {  // only the wide launch carries MaxUtil's code
    if (policy == CLE_POLICY_MAXUTIL && pool > m) {
      maxutil_block(L, D, ready, m);
      return L.result;
    }
  }
  if (threadIdx.x < kWave) {  // the first wavefront, lane d for group d
    uint64_t r;
    switch (policy) {
      case CLE_POLICY_B0_ALONE: r = ready & (~ready + 1); break;
      case CLE_POLICY_B1_LOCKSTEP: r = ready; break;
      case CLE_POLICY_CUMUTIL: r = pool < m ? ready : cumutil_wave(L, n, D, ready, m); break;
      case CLE_POLICY_DIFFPEAK: r = pool < m ? ready : diffpeak_wave(L, n, D, ready, m); break;
      default: r = ready; break;  // MAXUTIL with |S| <= m: S itself
    }
    if (threadIdx.x == 0) L.result = r;
  }
  __syncthreads();
  return L.result;
}

template <int NT>
__global__ __launch_bounds__(NT) void schedule_w_kernel(const int* __restrict__ w, int n, int D,
                                                       uint64_t ready, int m, int policy,
                                                       uint64_t* __restrict__ out) {
  __shared__ SchedLDS<NT> L;
  for (int i = threadIdx.x; i < n * D; i += NT) {
    const int v = w[i];
    L.w[i / D][i % D] = v > 0 ? v : 0;
  }
  __syncthreads();
  const uint64_t r = schedule_block(L, n, D, ready, m, policy);
  if (threadIdx.x == 0) out[0] = r;
}

struct LoopSchedArgs {
  const int* offsets[kMaxN];  // [E + 1] per micro-batch, from the dispatch
  cle_loop_state* st;
  int* w_out;          // [n, D] or NULL
  uint64_t* log;       // ring or NULL
  int64_t log_cap;
  int n, E, D, m, policy, restart;
};

// One loop step's schedule: workloads from the expert offsets, RunSet, statistics,
// log, layer advance, pool update and the optional restart.  The state is
// read into LDS by many lanes at once; the one lane that updates it then
// only stores.
template <int NT>
__global__ __launch_bounds__(NT) void loop_schedule_kernel(LoopSchedArgs a) {
  __shared__ SchedLDS<NT> L;
  __shared__ int lay[kMaxN], beg[kMaxN];
  __shared__ int64_t acc0[4];
  __shared__ int nl;
  cle_loop_state* st = a.st;
  const int n = a.n, D = a.D, g = a.E / a.D;
  const uint64_t ready = st->ready;
  if (threadIdx.x < kMaxN) {
    lay[threadIdx.x] = st->layer[threadIdx.x];
    beg[threadIdx.x] = st->start[threadIdx.x];
    if (threadIdx.x < 4) acc0[threadIdx.x] = st->acc[threadIdx.x];
    if (threadIdx.x == 4) nl = st->L;
  }
  // w[j][d] = offsets[j][(d + 1) g] - offsets[j][d g]: the group's counts
  // summed by the dispatch scan, two loads per (j, d) lane
  for (int i = threadIdx.x; i < n * D; i += NT) {
    const int j = i / D, d = i % D;
    const int* o = a.offsets[j];
    const int w = o[(d + 1) * g] - o[d * g];
    L.w[j][d] = w;
    if (a.w_out) a.w_out[i] = w;
  }
  __syncthreads();
  uint64_t r = 0;
  if (ready) r = schedule_block(L, n, D, ready, a.m, a.policy);
  if (threadIdx.x >= kWave) return;
  // Eq. (2)/(3) statistics of the RunSet on the first wavefront (lane d =
  // group d): W_d summed over the members, each member's own peak
  int64_t Wd = 0, sep = 0;
  for (int j = 0; j < n; ++j) {
    if (!(r >> j & 1)) continue;
    const int64_t x = w_lane(L, j, D);
    Wd += x;
    sep += static_cast<int64_t>(wave_max(x));
  }
  const int64_t sum = wave_sum(Wd), mx = static_cast<int64_t>(wave_max(Wd));
  if (threadIdx.x != 0) return;
  st->restarted = 0;
  st->runset = r;
  if (!r) {
    st->todo = 0;
    return;
  }
  const int Lyr = nl;
  if (a.log) a.log[acc0[3] % a.log_cap] = r;
  st->acc[0] = acc0[0] + sum;
  st->acc[1] = acc0[1] + mx;
  st->acc[2] = acc0[2] + sep;
  st->acc[3] = acc0[3] + 1;
  uint64_t left = ready;
  for (int j = 0; j < n; ++j) {
    if (!(r >> j & 1)) continue;
    st->run_layer[j] = lay[j];
    st->layer[j] = lay[j] + 1;
    if (lay[j] + 1 >= Lyr) left &= ~(1ull << j);
  }
  st->ready = left;
  st->todo = r & left;
  if (!left && a.restart) {
    uint64_t all = 0;
    for (int j = 0; j < n; ++j) {
      st->layer[j] = beg[j];
      if (beg[j] < Lyr) all |= 1ull << j;
    }
    st->ready = all;
    st->todo = all;
    st->restarts += 1;
    st->restarted = 1;
  }
}

struct LoopInitArgs {
  int start[kMaxN];
  cle_loop_state* st;
  int n, L;
};

__global__ void loop_init_kernel(LoopInitArgs a) {
  cle_loop_state* st = a.st;
  const int j = threadIdx.x;
  if (j < kMaxN) {
    const int s = j < a.n ? a.start[j] : a.L;
    st->layer[j] = s;
    st->start[j] = s;
    st->run_layer[j] = 0;
  }
  if (j == 0) {
    uint64_t ready = 0;
    for (int q = 0; q < a.n; ++q)
      if (a.start[q] < a.L) ready |= 1ull << q;
    st->ready = ready;
    st->todo = ready;
    st->runset = 0;
    for (int q = 0; q < 4; ++q) st->acc[q] = 0;
    st->n = a.n;
    st->L = a.L;
    st->restarts = 0;
    st->restarted = 0;
  }
}

bool valid_policy(int p) { return p >= CLE_POLICY_B0_ALONE && p <= CLE_POLICY_DIFFPEAK; }

}  // namespace
}  // namespace cle

extern "C" cle_status cle_schedule_step_device(const int32_t* w, int32_t n, int32_t D,
                                               uint64_t ready_mask, int32_t m, int32_t policy,
                                               uint64_t* runset, void* stream) {
  using namespace cle;
  if (!w || !runset) return CLE_EINVAL;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || D < 1 || D > CLE_MAX_LOOP_D) return CLE_EINVAL;
  if (m < 1 || m > n || !valid_policy(policy)) return CLE_EINVAL;
  if (ready_mask == 0) return CLE_EINVAL;
  if (n < 64 && (ready_mask >> n) != 0) return CLE_EINVAL;
  if (policy == CLE_POLICY_MAXUTIL && __builtin_popcountll(ready_mask) > m &&
      __builtin_popcountll(ready_mask) > CLE_MAX_MAXUTIL_POOL)
    return CLE_EUNSUPPORTED;
  if (policy == CLE_POLICY_MAXUTIL)
    schedule_w_kernel<kSchedThreads><<<dim3(1), dim3(kSchedThreads), 0, as_stream(stream)>>>(
        w, n, D, ready_mask, m, policy, runset);
  else
    schedule_w_kernel<kScanThreads><<<dim3(1), dim3(kScanThreads), 0, as_stream(stream)>>>(
        w, n, D, ready_mask, m, policy, runset);
  return launch_status();
}

extern "C" cle_status cle_loop_init(cle_loop_state* state, int32_t n, int32_t L,
                                    const int32_t* start, void* stream) {
  using namespace cle;
  if (!state || !aligned(state, 8) || n < 1 || n > CLE_MAX_MICROBATCHES || L < 1)
    return CLE_EINVAL;
  LoopInitArgs a;
  for (int j = 0; j < kMaxN; ++j) a.start[j] = 0;
  for (int j = 0; j < n; ++j) {
    const int s = start ? start[j] : 0;
    if (s < 0 || s > L) return CLE_EINVAL;
    a.start[j] = s;
  }
  a.st = state;
  a.n = n;
  a.L = L;
  loop_init_kernel<<<dim3(1), dim3(64), 0, as_stream(stream)>>>(a);
  return launch_status();
}

extern "C" cle_status cle_loop_step(const cle_loop_desc* d, void* const* phase_events,
                                    void* stream) {
  using namespace cle;
  if (!d || !d->state || !aligned(d->state, 8)) return CLE_EINVAL;
  const int n = d->n, T = d->T, E = d->E, k = d->k, H = d->H, D = d->D, ns = d->n_shared;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || d->L < 1 || T < 1) return CLE_EINVAL;
  if (E < 1 || E > CLE_MAX_E || k < 1 || k > E || H < 8 || H % 8 || ns < 0) return CLE_EINVAL;
  if (D < 1 || D > CLE_MAX_LOOP_D || E % D) return CLE_EINVAL;
  if (d->m < 1 || d->m > n || !valid_policy(d->policy)) return CLE_EINVAL;
  if (d->policy == CLE_POLICY_MAXUTIL && n > d->m && n > CLE_MAX_MAXUTIL_POOL)
    return CLE_EUNSUPPORTED;
  if (d->dtype != CLE_BF16 && d->dtype != CLE_F32) return CLE_EINVAL;
  if (d->restart != 0 && d->restart != 1) return CLE_EINVAL;
  if (d->log && d->log_cap < 1) return CLE_EINVAL;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A > INT32_MAX) return CLE_EUNSUPPORTED;
  const bool gated = d->w_gate != nullptr;
  if (d->prenorm != 0 && d->prenorm != 1) return CLE_EINVAL;
  if (d->prenorm && !(d->norm_eps >= 0.0f)) return CLE_EINVAL;
  if (gated) {
    const cle_status c = check_gate(T, H, E, static_cast<cle_dtype>(d->dtype), d->w_layout);
    if (c != CLE_OK) return c;
    if (!aligned(d->w_gate, 16)) return CLE_EINVAL;
  }
  for (int j = 0; j < n; ++j) {
    if (gated ? !d->gate_logits[j] : !d->logits[j]) return CLE_EINVAL;
    if (!d->h[j] || !d->idx[j] || !d->gate[j] || !d->counts[j] ||
        !d->offsets[j] || !d->dest[j] || !d->src[j] || !d->act[j] || !d->yp[j])
      return CLE_EINVAL;
    if (!aligned(d->h[j], 16) || !aligned(d->yp[j], 16)) return CLE_EINVAL;
    if (ns > 0 && (!d->act_shared[j] || !d->y_shared[j] || !aligned(d->y_shared[j], 16)))
      return CLE_EINVAL;
    if (d->restart && (!d->h0[j] || !aligned(d->h0[j], 16))) return CLE_EINVAL;
    if (d->prenorm && (!d->xn[j] || !aligned(d->xn[j], 16))) return CLE_EINVAL;
  }
  const size_t need = cle_workspace_bytes(CLE_OP_DISPATCH_MANY, T, E, k, 0, n);
  if (!d->ws_dispatch || d->ws_dispatch_bytes < need || !aligned(d->ws_dispatch, 256))
    return CLE_EWORKSPACE;
  cle_ffn_desc fd[CLE_MAX_MICROBATCHES];
  for (int j = 0; j < n; ++j) {
    cle_ffn_desc& q = fd[j];
    q.layer = 0;  // the planner takes the member's layer from the state
    q.rows = static_cast<int32_t>(A);
    q.offsets = d->offsets[j];
    q.xp = nullptr;
    q.act = d->act[j];
    q.yp = d->yp[j];
    const void* xin = d->prenorm ? d->xn[j] : d->h[j];  // what the experts read
    q.shared_rows = ns > 0 ? T : 0;
    q.x_shared = ns > 0 ? xin : nullptr;
    q.act_shared = ns > 0 ? d->act_shared[j] : nullptr;
    q.y_shared = ns > 0 ? d->y_shared[j] : nullptr;
    q.x = xin;
    q.src = d->src[j];
    q.k = k;
  }
  const cle_dtype dt = static_cast<cle_dtype>(d->dtype);
  cle_status rc = grouped_ffn(fd, n, d->w13, d->w2, d->w13_shared, d->w2_shared, d->L, E, ns, H,
                              d->I, dt, d->w_layout, d->ws_ffn, d->ws_ffn_bytes, phase_events,
                              d->state, false, stream);
  if (rc != CLE_OK) return rc;

  hipStream_t s = as_stream(stream);
  const cle_loop_state* st = d->state;
  const void* hs[CLE_MAX_MICROBATCHES];
  for (int j = 0; j < n; ++j) hs[j] = d->h[j];
  // with given scores the normalisation rides in the routing launch; the
  // router GEMM reads the normalised rows, so there it runs first
  if (d->prenorm && gated) {
    rc = launch_rmsnorm(n, hs, d->xn, T, H, d->norm_eps, dt, st, s);
    if (rc != CLE_OK) return rc;
  }
  if (gated) {
    const void* xs[CLE_MAX_MICROBATCHES];
    const void* wgs[CLE_MAX_MICROBATCHES];
    const float* bs[CLE_MAX_MICROBATCHES];
    for (int j = 0; j < n; ++j) {
      xs[j] = d->prenorm ? d->xn[j] : d->h[j];
      wgs[j] = d->w_gate;
      bs[j] = d->gate_bias;
    }
    rc = launch_gate(n, xs, wgs, bs, T, H, E, dt, d->w_layout == CLE_W_PACKED, d->gate_logits, st,
                     s);
    if (rc != CLE_OK) return rc;
    rc = launch_route(n, const_cast<const float* const*>(d->gate_logits), T, E, k, d->idx,
                      d->gate, st, 0, s);
  } else {
    rc = launch_route(n, d->logits, T, E, k, d->idx, d->gate, st, static_cast<int64_t>(T) * E, s,
                      d->prenorm ? hs : nullptr, d->prenorm ? d->xn : nullptr, H, d->norm_eps,
                      dt);
  }
  if (rc != CLE_OK) return rc;
  rc = launch_dispatch_many(n, d->idx, T, k, E, d->counts, d->offsets, d->dest, d->src,
                            d->ws_dispatch, st, s);
  if (rc != CLE_OK) return rc;
  LoopSchedArgs sa;
  for (int j = 0; j < n; ++j) sa.offsets[j] = d->offsets[j];
  sa.st = d->state;
  sa.w_out = d->w;
  sa.log = d->log;
  sa.log_cap = d->log_cap;
  sa.n = n;
  sa.E = E;
  sa.D = D;
  sa.m = d->m;
  sa.policy = d->policy;
  sa.restart = d->restart;
  if (d->policy == CLE_POLICY_MAXUTIL)
    loop_schedule_kernel<kSchedThreads><<<dim3(1), dim3(kSchedThreads), 0, s>>>(sa);
  else
    loop_schedule_kernel<kScanThreads><<<dim3(1), dim3(kScanThreads), 0, s>>>(sa);
  rc = grouped_ffn(fd, n, d->w13, d->w2, d->w13_shared, d->w2_shared, d->L, E, ns, H, d->I, dt,
                   d->w_layout, d->ws_ffn, d->ws_ffn_bytes, phase_events, st, true, stream);
  if (rc != CLE_OK) return rc;
  const void* ysh[CLE_MAX_MICROBATCHES];
  const void* res[CLE_MAX_MICROBATCHES];
  for (int j = 0; j < n; ++j) {
    ysh[j] = ns > 0 ? d->y_shared[j] : nullptr;
    res[j] = d->h[j];
  }
  rc = launch_combine_many(n, const_cast<const void* const*>(reinterpret_cast<void* const*>(d->yp)),
                           d->dest, d->gate, T, k, H, ns > 0 ? ysh : nullptr, ns, res, d->h, dt,
                           st, s, d->restart ? d->h0 : nullptr);
  if (rc != CLE_OK) return rc;
  return launch_status();
}
