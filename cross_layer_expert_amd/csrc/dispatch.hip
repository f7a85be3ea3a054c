// Dispatch: per-expert histogram, exclusive scan, stable permutation and row
// gather -- the single-GPU form of the expert-parallel all-to-all dispatch
// ("EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.2; per-expert token counts T_e as in section 1 of the EP load-balancing
// atlas page "系统侧负载均衡：EPLB、LPLB、UltraEP 与 MoonEP").
//
// Assignment a = t*k + s goes to row dest[a] = offsets[e] + (number of
// earlier assignments to the same expert): a stable counting sort.
//
//   1. count   one block per 1024-assignment chunk: LDS histogram
//   2. scan    one block: per-expert prefix over chunks, prefix over experts
//              (when the chunk histograms are small, each scatter block
//              computes the prefixes it needs itself: one launch fewer)
//   3. scatter one block per chunk: in-order ranks from wavefront ballots
//              (lanes that share an expert id find each other with one ballot
//              per id bit; rank = popcount of the lower lanes in the group)
//   4. gather  one wavefront per destination row: xp[p] = x[src[p] / k]
// Integer only; every output is exact and deterministic.
#include "cle_internal.h"

namespace cle {
namespace {

constexpr int kChunkWaves = 4;
constexpr int kPerWave = kDispatchChunk / kChunkWaves;  // 256 assignments per wave

// Buffers of the micro-batches of one launch (blockIdx.y picks one); each has
// its own chunk-histogram region of the workspace, hist_stride ints apart.
struct DispatchArgs {
  const int* idx[CLE_MAX_MICROBATCHES];
  int* counts[CLE_MAX_MICROBATCHES];
  int* offsets[CLE_MAX_MICROBATCHES];
  int* dest[CLE_MAX_MICROBATCHES];
  int* src[CLE_MAX_MICROBATCHES];
  int* hist;
  int64_t hist_stride;
  const cle_loop_state* st;  // non-NULL: only micro-batches in st->todo
};

__device__ __forceinline__ bool skip(const DispatchArgs& a, int j) {
  return a.st && !(a.st->todo >> j & 1);
}

__global__ __launch_bounds__(256) void dispatch_count(DispatchArgs args, int64_t A, int E) {
  if (skip(args, blockIdx.y)) return;
  const int* __restrict__ idx = args.idx[blockIdx.y];
  int* __restrict__ chunk_hist = args.hist + blockIdx.y * args.hist_stride;
  __shared__ int hist[CLE_MAX_E];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  for (int i = threadIdx.x; i < kDispatchChunk; i += blockDim.x) {
    const int64_t a = base + i;
    if (a < A) {
      const int e = idx[a];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  int* out = chunk_hist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

// Turns chunk counts into absolute chunk bases in place and writes counts
// and offsets.  Thread (s, e) of S = 1024 / E slices owns expert e in a
// contiguous run of chunks, so the chunk counts are read and rewritten by
// all threads at once: sums per (slice, expert), a prefix over slices, the
// exclusive scan over experts, then the chunk bases.
__global__ __launch_bounds__(1024) void dispatch_scan(DispatchArgs args, int64_t chunks, int E,
                                                      int64_t A) {
  if (skip(args, blockIdx.x)) return;
  int* __restrict__ chunk_hist = args.hist + blockIdx.x * args.hist_stride;
  int* __restrict__ counts = args.counts[blockIdx.x];
  int* __restrict__ offsets = args.offsets[blockIdx.x];
  int* __restrict__ src = args.src[blockIdx.x];
  __shared__ int ps[1024];  // [slice][expert]: chunk-count sums, then their prefix over slices
  __shared__ int tot[CLE_MAX_E];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int S = 1024 / E;
  const int64_t cps = (chunks + S - 1) / S;
  const int sl = tid / E, e = tid % E;
  const bool owner = sl < S;
  const int64_t c0 = owner ? min(chunks, sl * cps) : chunks;
  const int64_t c1 = owner ? min(chunks, c0 + cps) : chunks;
  if (owner) {
    int sum = 0;
    for (int64_t c = c0; c < c1; ++c) sum += chunk_hist[c * E + e];
    ps[tid] = sum;
  }
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int q = 0; q < S; ++q) {
      const int v = ps[q * E + tid];
      ps[q * E + tid] = run;
      run += v;
    }
    tot[tid] = run;
  }
  __syncthreads();
  // exclusive scan of tot[0..E) with one value per thread (E <= 1024)
  const int v = tid < E ? tot[tid] : 0;
  part[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int excl = part[tid] - v;
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = excl;
  }
  if (tid == E - 1) offsets[E] = part[tid];
  // positions past the valid assignments (dropped ids) have no source
  for (int64_t p = part[E - 1] + tid; p < A; p += blockDim.x) src[p] = -1;
  __syncthreads();
  if (tid < E) tot[tid] = excl;
  __syncthreads();
  if (owner) {
    int run = tot[e] + ps[tid];
    for (int64_t c = c0; c < c1; ++c) {
      int* p = chunk_hist + c * E + e;
      const int cnt = *p;
      *p = run;
      run += cnt;
    }
  }
}

// SCAN: the chunk histograms hold raw counts (no scan launch ran): every block
// computes the expert totals, their exclusive scan and its own chunk's prefix
// from them (chunks * E <= kScatterScanMax ints: a few dozen reads per thread
// at most), and block 0 also writes
// counts, offsets and the source-less tail.  Otherwise they hold the chunk
// bases that dispatch_scan wrote.
template <bool SCAN>
__global__ __launch_bounds__(256) void dispatch_scatter(DispatchArgs args, int64_t A, int E,
                                                        int id_bits, int chunks) {
  if (skip(args, blockIdx.y)) return;
  const int* __restrict__ idx = args.idx[blockIdx.y];
  const int* __restrict__ chunk_base = args.hist + blockIdx.y * args.hist_stride;
  int* __restrict__ dest = args.dest[blockIdx.y];
  int* __restrict__ src = args.src[blockIdx.y];
  __shared__ int wcount[kChunkWaves][CLE_MAX_E];
  __shared__ int base_s[SCAN ? CLE_MAX_E : 1];  // (also the prefix partial sums)
  __shared__ int part[SCAN ? 256 : 1];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  for (int i = tid; i < kChunkWaves * E; i += blockDim.x) wcount[i / E][i % E] = 0;
  __syncthreads();
  const int64_t wbase = static_cast<int64_t>(blockIdx.x) * kDispatchChunk +
                        static_cast<int64_t>(wave) * kPerWave;
  // pass 1: per-wave counts
  for (int it = 0; it < kPerWave / kWave; ++it) {
    const int64_t a = wbase + it * kWave + lane;
    if (a < A) {
      const int e = idx[a];
      if (e >= 0 && e < E) atomicAdd(&wcount[wave][e], 1);
    }
  }
  if constexpr (SCAN) {
    // Thread t owns the experts [t R, t R + R), R = ceil(E / 256): their
    // totals over all chunks and prefixes over the chunks before this one,
    // then the exclusive scan of the totals over the 256 runs.  With E <= 256
    // the chunks are first split over G = 256 / E thread groups (partial sums
    // in LDS), so each thread reads at most ceil(chunks / G) entries.
    const int bx = static_cast<int>(blockIdx.x);
    const int R = (E + 255) / 256;
    const int e0 = min(E, tid * R), e1 = min(E, e0 + R);
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};  // R <= 4 (E <= 1024)
    if (E <= 256) {
      const int G = 256 / E, e = tid % E, g = tid / E;
      int t = 0, p = 0;
      if (g < G) {
#pragma unroll 4
        for (int c = g; c < chunks; c += G) {
          const int v = chunk_base[static_cast<int64_t>(c) * E + e];
          t += v;
          p += c < bx ? v : 0;
        }
      }
      part[tid] = t;
      base_s[tid] = p;
      __syncthreads();
      if (tid < E)
        for (int q = 0; q < G; ++q) {
          tot[0] += part[q * E + tid];
          pre[0] += base_s[q * E + tid];
        }
      __syncthreads();  // part and base_s are reused below
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + q;
        if (e < e1)
          for (int c = 0; c < chunks; ++c) {
            const int v = chunk_base[static_cast<int64_t>(c) * E + e];
            tot[q] += v;
            pre[q] += c < bx ? v : 0;
          }
      }
    }
    const int run_sum = tot[0] + tot[1] + tot[2] + tot[3];
    part[tid] = run_sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    int excl = part[tid] - run_sum;
    const int nvalid = part[255];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + q;
      if (e < e1) {
        base_s[e] = excl + pre[q];
        if (blockIdx.x == 0) {
          args.counts[blockIdx.y][e] = tot[q];
          args.offsets[blockIdx.y][e] = excl;
        }
        excl += tot[q];
      }
    }
    if (blockIdx.x == 0) {
      if (tid == 0) args.offsets[blockIdx.y][E] = nvalid;
      // positions past the valid assignments (dropped ids) have no source
      for (int64_t p = nvalid + tid; p < A; p += blockDim.x) src[p] = -1;
    }
  }
  __syncthreads();
  // per expert: absolute base of each wave's sub-range
  const int* cb = chunk_base + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = tid; e < E; e += blockDim.x) {
    int run = SCAN ? base_s[e] : cb[e];
    for (int w = 0; w < kChunkWaves; ++w) {
      const int v = wcount[w][e];
      wcount[w][e] = run;
      run += v;
    }
  }
  __syncthreads();
  // pass 2: ranks in assignment order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int it = 0; it < kPerWave / kWave; ++it) {
    const int64_t a = wbase + it * kWave + lane;
    const bool in = a < A;
    const int e = in ? idx[a] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    int d = -1;
    if (valid) {
      const int rank = __popcll(match & lt_mask);
      d = wcount[wave][e] + rank;
    }
    // all lanes have read their base before the group leaders advance it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid) {
      const bool leader = (match >> lane) == 1ull;  // highest lane of its group
      if (leader) wcount[wave][e] += __popcll(match);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (in) {
      dest[a] = d;
      if (valid) src[d] = static_cast<int>(a);
    }
  }
}

// One wavefront per destination row; VEC elements of T per 16-byte access.
template <typename T>
__global__ __launch_bounds__(256) void dispatch_gather(const T* __restrict__ x, int64_t A, int k,
                                                       int H, const int* __restrict__ offsets,
                                                       int E, const int* __restrict__ src,
                                                       T* __restrict__ xp) {
  constexpr int VEC = 16 / sizeof(T);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (p >= A) return;
  const int64_t valid_rows = offsets[E];
  uint4* out = reinterpret_cast<uint4*>(xp + p * H);
  const int nvec = H / VEC;
  if (p < valid_rows) {
    const int64_t t = src[p] / k;
    const uint4* in = reinterpret_cast<const uint4*>(x + t * H);
    for (int c = lane; c < nvec; c += kWave) out[c] = in[c];
  } else {
    for (int c = lane; c < nvec; c += kWave) out[c] = make_uint4(0, 0, 0, 0);
  }
}

}  // namespace
}  // namespace cle

namespace cle {
namespace {

// count, scan and scatter for n micro-batches of A assignments each
// chunk histogram entries up to which every scatter block does the scan itself
constexpr int64_t kScatterScanMax = 4096;

cle_status launch_dispatch(const DispatchArgs& a, int n, int64_t A, int E, hipStream_t s) {
  const int64_t chunks = dispatch_chunks(A);
  if (chunks > 0)
    dispatch_count<<<dim3(static_cast<unsigned>(chunks), n), dim3(256), 0, s>>>(a, A, E);
  const bool scan_in_scatter = A > 0 && chunks * E <= kScatterScanMax;
  if (!scan_in_scatter) dispatch_scan<<<dim3(n), dim3(1024), 0, s>>>(a, chunks, E, A);
  if (A == 0) return launch_status();
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  const dim3 grid(static_cast<unsigned>(chunks), n);
  if (scan_in_scatter)
    dispatch_scatter<true><<<grid, dim3(256), 0, s>>>(a, A, E, id_bits, static_cast<int>(chunks));
  else
    dispatch_scatter<false><<<grid, dim3(256), 0, s>>>(a, A, E, id_bits, static_cast<int>(chunks));
  return launch_status();
}

}  // namespace
}  // namespace cle

extern "C" cle_status cle_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                   const void* x, int32_t H, cle_dtype dt, int32_t* counts,
                                   int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                                   void* ws, size_t ws_bytes, void* stream) {
  using namespace cle;
  if (T < 0 || k < 1 || E < 1 || E > CLE_MAX_E || H < 8 || H % 8) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  if (!counts || !offsets) return CLE_EINVAL;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A > INT32_MAX) return CLE_EUNSUPPORTED;
  if (A > 0 && (!topk_idx || !dest || !src)) return CLE_EINVAL;
  if (A > 0 && xp && !x) return CLE_EINVAL;
  if (!aligned(x, 16) || !aligned(xp, 16)) return CLE_EINVAL;
  const size_t need = cle_workspace_bytes(CLE_OP_DISPATCH, T, E, k, 0, 1);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return CLE_EWORKSPACE;
  hipStream_t s = as_stream(stream);
  DispatchArgs a;
  a.idx[0] = topk_idx;
  a.counts[0] = counts;
  a.offsets[0] = offsets;
  a.dest[0] = dest;
  a.src[0] = src;
  a.hist = static_cast<int*>(ws);
  a.hist_stride = 0;
  a.st = nullptr;
  const cle_status st = launch_dispatch(a, 1, A, E, s);
  if (st != CLE_OK || A == 0 || !xp) return st;
  const dim3 ggrid(static_cast<unsigned>((A + 3) / 4));
  if (dt == CLE_BF16)
    dispatch_gather<uint16_t><<<ggrid, dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(x), A, k, H, offsets, E, src, static_cast<uint16_t*>(xp));
  else
    dispatch_gather<float><<<ggrid, dim3(256), 0, s>>>(static_cast<const float*>(x), A, k, H,
                                                       offsets, E, src, static_cast<float*>(xp));
  return launch_status();
}

extern "C" cle_status cle_dispatch_many(int32_t n, const int32_t* const* topk_idx, int32_t T,
                                        int32_t k, int32_t E, int32_t* const* counts,
                                        int32_t* const* offsets, int32_t* const* dest,
                                        int32_t* const* src, void* ws, size_t ws_bytes,
                                        void* stream) {
  using namespace cle;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || !topk_idx || !counts || !offsets || !dest || !src)
    return CLE_EINVAL;
  if (T < 0 || k < 1 || E < 1 || E > CLE_MAX_E) return CLE_EINVAL;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A > INT32_MAX) return CLE_EUNSUPPORTED;
  DispatchArgs a;
  for (int j = 0; j < n; ++j) {
    if (!counts[j] || !offsets[j]) return CLE_EINVAL;
    if (A > 0 && (!topk_idx[j] || !dest[j] || !src[j])) return CLE_EINVAL;
    a.idx[j] = topk_idx[j];
    a.counts[j] = counts[j];
    a.offsets[j] = offsets[j];
    a.dest[j] = dest[j];
    a.src[j] = src[j];
  }
  const size_t one = cle_workspace_bytes(CLE_OP_DISPATCH, T, E, k, 0, 1);
  const size_t need = cle_workspace_bytes(CLE_OP_DISPATCH_MANY, T, E, k, 0, n);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return CLE_EWORKSPACE;
  a.hist = static_cast<int*>(ws);
  a.hist_stride = static_cast<int64_t>(one / sizeof(int));
  a.st = nullptr;
  return launch_dispatch(a, n, A, E, as_stream(stream));
}

namespace cle {

cle_status launch_dispatch_many(int n, const int* const* idx, int T, int k, int E,
                                int* const* counts, int* const* offsets, int* const* dest,
                                int* const* src, void* ws, const cle_loop_state* st,
                                hipStream_t s) {
  DispatchArgs a;
  for (int j = 0; j < n; ++j) {
    a.idx[j] = idx[j];
    a.counts[j] = counts[j];
    a.offsets[j] = offsets[j];
    a.dest[j] = dest[j];
    a.src[j] = src[j];
  }
  a.hist = static_cast<int*>(ws);
  a.hist_stride =
      static_cast<int64_t>(cle_workspace_bytes(CLE_OP_DISPATCH, T, E, k, 0, 1) / sizeof(int));
  a.st = st;
  return launch_dispatch(a, n, static_cast<int64_t>(T) * k, E, s);
}

}  // namespace cle
