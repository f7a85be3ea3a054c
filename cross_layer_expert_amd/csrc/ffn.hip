// Grouped SwiGLU expert FFN over micro-batches at different layers.
// "EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference":
// §4.1 -- the workloads of several micro-batches, each at its own layer, are
// executed in one step; Eq. (1) -- expert_i applied to the tokens routed to
// it.  The expert form (SwiGLU, intermediate I) is the workload's:
//   [G | U] = X_s W13^T,  Act = silu(G) * U,  Y = Act W2^T.
//
// Layout of the work:
//   plan     one block per 16 descriptors: builds the segment table (one
//            segment per (micro-batch, routed expert) and per shared expert)
//            in the workspace, with an exclusive prefix of the tile counts of
//            both phases; totals go to the workspace header.
//   phase 1  persistent kernel over all (segment, n-tile, m-tile) tiles:
//            64 rows x 64 act columns, K = H; gate and up rows of the same
//            act columns in one tile, so the SwiGLU epilogue is local.
//   phase 2  same scheduler: 64 rows x 128 output columns, K = I.
// bf16 path: v_mfma_f32_16x16x32_bf16 (gfx950), fp32 accumulation, one fixed
// K order for every tile, no split-K, so a row's result does not depend on
// which other segments share the launch.  A (activation) tiles are staged in
// LDS and shared by the four wavefronts; each wavefront streams its own
// weight rows straight into registers in the MFMA operand layout.
// Consecutive logical tiles go to one XCD (workgroups are dealt round-robin
// over the 8 XCDs) so tiles reading the same weight rows share that XCD's L2.
#include "cle_internal.h"

namespace cle {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;        // rows per tile (both phases, both dtypes)
constexpr int kBN1 = 64;       // act columns per phase-1 tile
constexpr int kBN2 = 128;      // output columns per phase-2 tile (bf16)
constexpr int kBN2F = 64;      // output columns per phase-2 tile (f32)
constexpr int kBK = 64;        // K per pipeline step
constexpr int kPlanDescs = 16;
constexpr int kXcds = 8;

struct DescDev {
  int layer, rows;
  const int* offsets;
  const void* xp;
  void* act;
  void* yp;
  int shared_rows;
  const void* x_shared;
  void* act_shared;
  void* y_shared;
};

struct PlanArgs {
  DescDev d[kPlanDescs];
  const void* w13;
  const void* w2;
  const void* w13s;
  const void* w2s;
  int nd, seg_base, first;
  int E, ns, H, I, esz, bn2;
};

// ---------------------------------------------------------------- planning
// Row range [lo, hi) of routed expert e, clamped to the descriptor's rows so
// that inconsistent offsets can never reach outside the caller's buffers.
__device__ __forceinline__ void seg_range(const DescDev& d, int e, int& lo, int& hi) {
  lo = min(max(d.offsets[e], 0), d.rows);
  hi = min(max(d.offsets[e + 1], lo), d.rows);
}

__device__ __forceinline__ int seg_rows(const PlanArgs& p, int s) {
  const int j = s / (p.E + p.ns), e = s % (p.E + p.ns);
  if (e < p.E) {
    int lo, hi;
    seg_range(p.d[j], e, lo, hi);
    return hi - lo;
  }
  return p.d[j].shared_rows;
}

__global__ __launch_bounds__(1024) void ffn_plan(PlanArgs p, Seg* __restrict__ segs,
                                                 int* __restrict__ totals) {
  __shared__ int s1[1024], s2[1024];
  __shared__ int base1, base2;
  const int tid = threadIdx.x;
  const int nseg = p.nd * (p.E + p.ns);
  const int per = (nseg + 1023) / 1024;
  const int lo = min(nseg, tid * per), hi = min(nseg, lo + per);
  const int n1 = p.I / kBN1, n2 = p.H / p.bn2;
  int c1 = 0, c2 = 0;
  for (int s = lo; s < hi; ++s) {
    const int mt = (seg_rows(p, s) + kBM - 1) / kBM;
    c1 += mt * n1;
    c2 += mt * n2;
  }
  if (tid == 0) {
    base1 = p.first ? 0 : totals[0];
    base2 = p.first ? 0 : totals[1];
  }
  s1[tid] = c1;
  s2[tid] = c2;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a1 = tid >= off ? s1[tid - off] : 0;
    const int a2 = tid >= off ? s2[tid - off] : 0;
    __syncthreads();
    s1[tid] += a1;
    s2[tid] += a2;
    __syncthreads();
  }
  int t1 = base1 + s1[tid] - c1, t2 = base2 + s2[tid] - c2;
  const int64_t H = p.H, I = p.I, esz = p.esz;
  for (int s = lo; s < hi; ++s) {
    const int j = s / (p.E + p.ns), e = s % (p.E + p.ns);
    const DescDev& d = p.d[j];
    Seg g;
    if (e < p.E) {
      int lo, hi;
      seg_range(d, e, lo, hi);
      const int64_t off = lo;
      g.rows = hi - lo;
      g.a = reinterpret_cast<const uint16_t*>(static_cast<const char*>(d.xp) + off * H * esz);
      g.act = static_cast<char*>(d.act) + off * I * esz;
      g.y = static_cast<char*>(d.yp) + off * H * esz;
      const int64_t we = static_cast<int64_t>(d.layer) * p.E + e;
      g.w13 = static_cast<const char*>(p.w13) + we * 2 * I * H * esz;
      g.w2 = static_cast<const char*>(p.w2) + we * H * I * esz;
    } else {
      const int64_t q = e - p.E, R = d.shared_rows;
      g.rows = d.shared_rows;
      g.a = reinterpret_cast<const uint16_t*>(d.x_shared);
      g.act = static_cast<char*>(d.act_shared) + q * R * I * esz;
      g.y = static_cast<char*>(d.y_shared) + q * R * H * esz;
      const int64_t we = static_cast<int64_t>(d.layer) * p.ns + q;
      g.w13 = static_cast<const char*>(p.w13s) + we * 2 * I * H * esz;
      g.w2 = static_cast<const char*>(p.w2s) + we * H * I * esz;
    }
    g.t1 = t1;
    g.t2 = t2;
    g.pad_ = 0;
    segs[p.seg_base + s] = g;
    const int mt = (g.rows + kBM - 1) / kBM;
    t1 += mt * n1;
    t2 += mt * n2;
  }
  if (tid == 1023) {
    totals[0] = t1;
    totals[1] = t2;
  }
}

// Segment owning a tile: the last segment whose first tile is <= tile.
template <int PHASE>
__device__ __forceinline__ int find_seg(const Seg* segs, int nseg, int tile) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int t = PHASE == 1 ? segs[mid].t1 : segs[mid].t2;
    if (t <= tile) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int logical_tile_base(int grid) {
  // grid is a multiple of kXcds; workgroup b runs on XCD b % kXcds
  const int b = blockIdx.x;
  return (b % kXcds) * (grid / kXcds) + b / kXcds;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------- bf16 MFMA tiles
// A tile in LDS: [kBM rows][8 chunks of 16 bytes], chunk c of row r stored at
// c ^ (r & 7) to spread the column reads of 16 rows over the banks.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

template <int PHASE>
__global__ __launch_bounds__(256) void ffn_gemm_bf16(const Seg* __restrict__ segs, int nseg,
                                                     const int* __restrict__ totals, int H,
                                                     int I) {
  __shared__ uint4 a_lds[2][kBM * 8];
  const int total = totals[PHASE - 1];
  const int grid = gridDim.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16, g4 = lane / 16;
  const int K = PHASE == 1 ? H : I;                 // reduction length = row stride of A and W
  const int KT = K / kBK;
  // A staging: thread -> (row, 32-byte quarter)
  const int ar = threadIdx.x / 4, aq = threadIdx.x % 4;

  for (int tile = logical_tile_base(grid); tile < total; tile += grid) {
    const int si = find_seg<PHASE>(segs, nseg, tile);
    const Seg sg = segs[si];
    const int mt = (sg.rows + kBM - 1) / kBM;
    const int r = tile - (PHASE == 1 ? sg.t1 : sg.t2);
    const int nt = r / mt, mi = r % mt;
    const int row0 = mi * kBM;
    const uint16_t* A = PHASE == 1 ? sg.a : static_cast<const uint16_t*>(sg.act);
    const uint16_t* W = static_cast<const uint16_t*>(PHASE == 1 ? sg.w13 : sg.w2);
    // this lane's two weight rows (operand B of the two MFMA column blocks)
    int wrow0, wrow1;
    if (PHASE == 1) {
      wrow0 = nt * kBN1 + wave * 16 + l16;  // gate row
      wrow1 = I + wrow0;                    // up row of the same act column
    } else {
      wrow0 = nt * kBN2 + wave * 32 + l16;
      wrow1 = wrow0 + 16;
    }
    const uint16_t* w0p = W + static_cast<int64_t>(wrow0) * K + g4 * 8;
    const uint16_t* w1p = W + static_cast<int64_t>(wrow1) * K + g4 * 8;
    // Rows past the segment end load the last valid row instead: an MFMA
    // output row depends only on its own A row, and those rows are never
    // stored, so no masking is needed.
    const int arow = min(row0 + ar, sg.rows - 1);
    const uint16_t* ap = A + static_cast<int64_t>(arow) * K + aq * 16;

    f32x4 acc0[4], acc1[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      acc0[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint4 b00 = *reinterpret_cast<const uint4*>(w0p);
    uint4 b01 = *reinterpret_cast<const uint4*>(w0p + 32);
    uint4 b10 = *reinterpret_cast<const uint4*>(w1p);
    uint4 b11 = *reinterpret_cast<const uint4*>(w1p + 32);
    a_lds[0][a_slot(ar, 2 * aq)] = *reinterpret_cast<const uint4*>(ap);
    a_lds[0][a_slot(ar, 2 * aq + 1)] = *reinterpret_cast<const uint4*>(ap + 8);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      // prefetch step kt+1 (the last step re-reads itself; never consumed)
      const int ko = min(kt + 1, KT - 1) * kBK;
      const uint4 na0 = *reinterpret_cast<const uint4*>(ap + ko);
      const uint4 na1 = *reinterpret_cast<const uint4*>(ap + ko + 8);
      const uint4 n00 = *reinterpret_cast<const uint4*>(w0p + ko);
      const uint4 n01 = *reinterpret_cast<const uint4*>(w0p + ko + 32);
      const uint4 n10 = *reinterpret_cast<const uint4*>(w1p + ko);
      const uint4 n11 = *reinterpret_cast<const uint4*>(w1p + ko + 32);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 B0 = __builtin_bit_cast(bf16x8, s == 0 ? b00 : b01);
        const bf16x8 B1 = __builtin_bit_cast(bf16x8, s == 0 ? b10 : b11);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const bf16x8 Af =
              __builtin_bit_cast(bf16x8, a_lds[cur][a_slot(mb * 16 + l16, s * 4 + g4)]);
          acc0[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af, B0, acc0[mb], 0, 0, 0);
          acc1[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af, B1, acc1[mb], 0, 0, 0);
        }
      }
      // buffer cur^1 was last read before the previous barrier
      a_lds[cur ^ 1][a_slot(ar, 2 * aq)] = na0;
      a_lds[cur ^ 1][a_slot(ar, 2 * aq + 1)] = na1;
      b00 = n00;
      b01 = n01;
      b10 = n10;
      b11 = n11;
      __syncthreads();
    }

    // epilogue: lane holds rows mb*16 + g4*4 + i, column l16 of each block
    if (PHASE == 1) {
      uint16_t* out = static_cast<uint16_t*>(sg.act);
      const int col = nt * kBN1 + wave * 16 + l16;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + mb * 16 + g4 * 4 + i;
          if (row < sg.rows)
            out[static_cast<int64_t>(row) * I + col] = f32_to_bf16(silu(acc0[mb][i]) * acc1[mb][i]);
        }
    } else {
      uint16_t* out = static_cast<uint16_t*>(sg.y);
      const int col = nt * kBN2 + wave * 32 + l16;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + mb * 16 + g4 * 4 + i;
          if (row < sg.rows) {
            out[static_cast<int64_t>(row) * H + col] = f32_to_bf16(acc0[mb][i]);
            out[static_cast<int64_t>(row) * H + col + 16] = f32_to_bf16(acc1[mb][i]);
          }
        }
    }
  }
}

// ---------------------------------------------------------------- f32 tiles (exact-order reference path)
template <int PHASE>
__global__ __launch_bounds__(256) void ffn_gemm_f32(const Seg* __restrict__ segs, int nseg,
                                                    const int* __restrict__ totals, int H, int I) {
  const int total = totals[PHASE - 1];
  const int grid = gridDim.x;
  const int K = PHASE == 1 ? H : I;
  for (int tile = logical_tile_base(grid); tile < total; tile += grid) {
    const int si = find_seg<PHASE>(segs, nseg, tile);
    const Seg sg = segs[si];
    const int mt = (sg.rows + kBM - 1) / kBM;
    const int r = tile - (PHASE == 1 ? sg.t1 : sg.t2);
    const int nt = r / mt, mi = r % mt;
    const float* A = static_cast<const float*>(PHASE == 1 ? static_cast<const void*>(sg.a) : sg.act);
    const float* W = static_cast<const float*>(PHASE == 1 ? sg.w13 : sg.w2);
    for (int e = threadIdx.x; e < kBM * 64; e += blockDim.x) {
      const int row = mi * kBM + e / 64;
      const int col = nt * 64 + e % 64;
      if (row >= sg.rows) continue;
      const float* a = A + static_cast<int64_t>(row) * K;
      if (PHASE == 1) {
        const float* wg = W + static_cast<int64_t>(col) * K;
        const float* wu = W + static_cast<int64_t>(I + col) * K;
        float g = 0.f, u = 0.f;
        for (int kk = 0; kk < K; ++kk) {
          g = fmaf(a[kk], wg[kk], g);
          u = fmaf(a[kk], wu[kk], u);
        }
        static_cast<float*>(sg.act)[static_cast<int64_t>(row) * I + col] = silu(g) * u;
      } else {
        const float* wd = W + static_cast<int64_t>(col) * K;
        float y = 0.f;
        for (int kk = 0; kk < K; ++kk) y = fmaf(a[kk], wd[kk], y);
        static_cast<float*>(sg.y)[static_cast<int64_t>(row) * H + col] = y;
      }
    }
  }
}

int persistent_grid(int64_t upper_bound_tiles) {
  int64_t g = static_cast<int64_t>(device_cu_count()) * 4;
  if (upper_bound_tiles < g) g = upper_bound_tiles;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return static_cast<int>(g);
}

}  // namespace
}  // namespace cle

extern "C" cle_status cle_grouped_expert_ffn(const cle_ffn_desc* d, int32_t n_desc,
                                             const void* w13, const void* w2,
                                             const void* w13_shared, const void* w2_shared,
                                             int32_t L, int32_t E, int32_t n_shared, int32_t H,
                                             int32_t I, cle_dtype dt, void* ws, size_t ws_bytes,
                                             void* const* phase_events, void* stream) {
  using namespace cle;
  if (!d || n_desc < 1 || n_desc > CLE_MAX_DESC) return CLE_EINVAL;
  if (!w13 || !w2 || L < 1 || E < 1 || E > CLE_MAX_E || n_shared < 0) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  const int bn2 = dt == CLE_BF16 ? kBN2 : kBN2F;
  if (H < bn2 || H % bn2 || I < kBN1 || I % kBN1) return CLE_EINVAL;
  if (n_shared > 0 && (!w13_shared || !w2_shared)) return CLE_EINVAL;
  const int esz = dt == CLE_BF16 ? 2 : 4;
  if (!aligned(w13, 16) || !aligned(w2, 16)) return CLE_EINVAL;
  int64_t ub1 = 0, ub2 = 0;
  for (int j = 0; j < n_desc; ++j) {
    const cle_ffn_desc& q = d[j];
    if (q.layer < 0 || q.layer >= L || q.rows < 0 || !q.offsets) return CLE_EINVAL;
    if (q.rows > 0 && (!q.xp || !q.act || !q.yp)) return CLE_EINVAL;
    if (!aligned(q.xp, 16) || !aligned(q.act, 16) || !aligned(q.yp, 16)) return CLE_EINVAL;
    if (n_shared > 0) {
      if (q.shared_rows < 0) return CLE_EINVAL;
      if (q.shared_rows > 0 && (!q.x_shared || !q.act_shared || !q.y_shared)) return CLE_EINVAL;
      if (!aligned(q.x_shared, 16) || !aligned(q.act_shared, 16) || !aligned(q.y_shared, 16))
        return CLE_EINVAL;
    }
    // sum over experts of ceil(c_e / BM) <= rows / BM + (non-empty experts)
    const int64_t mt = q.rows / kBM + (q.rows < E ? q.rows : E);
    const int64_t mts = n_shared > 0 ? static_cast<int64_t>(n_shared) * ((q.shared_rows + kBM - 1) / kBM) : 0;
    ub1 += (mt + mts) * (I / kBN1);
    ub2 += (mt + mts) * (H / bn2);
  }
  if (ub1 > INT32_MAX || ub2 > INT32_MAX) return CLE_EUNSUPPORTED;
  const size_t need = cle_workspace_bytes(CLE_OP_FFN, 0, E, 1, n_shared, n_desc);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return CLE_EWORKSPACE;

  hipStream_t s = as_stream(stream);
  int* totals = static_cast<int*>(ws);
  Seg* segs = reinterpret_cast<Seg*>(static_cast<char*>(ws) + kFfnHeader);
  const int nseg = n_desc * (E + n_shared);
  for (int c = 0; c < n_desc; c += kPlanDescs) {
    PlanArgs p;
    p.nd = n_desc - c < kPlanDescs ? n_desc - c : kPlanDescs;
    for (int j = 0; j < p.nd; ++j) {
      const cle_ffn_desc& q = d[c + j];
      p.d[j] = DescDev{q.layer, q.rows, q.offsets, q.xp, q.act, q.yp,
                       n_shared > 0 ? q.shared_rows : 0, q.x_shared, q.act_shared, q.y_shared};
    }
    p.w13 = w13;
    p.w2 = w2;
    p.w13s = w13_shared;
    p.w2s = w2_shared;
    p.seg_base = c * (E + n_shared);
    p.first = c == 0;
    p.E = E;
    p.ns = n_shared;
    p.H = H;
    p.I = I;
    p.esz = esz;
    p.bn2 = bn2;
    ffn_plan<<<dim3(1), dim3(1024), 0, s>>>(p, segs, totals);
  }
  if (phase_events && hipEventRecord(static_cast<hipEvent_t>(phase_events[0]), s) != hipSuccess)
    return CLE_EHIP;
  if (ub1 > 0) {
    const int g = persistent_grid(ub1);
    if (dt == CLE_BF16)
      ffn_gemm_bf16<1><<<dim3(g), dim3(256), 0, s>>>(segs, nseg, totals, H, I);
    else
      ffn_gemm_f32<1><<<dim3(g), dim3(256), 0, s>>>(segs, nseg, totals, H, I);
  }
  if (phase_events && hipEventRecord(static_cast<hipEvent_t>(phase_events[1]), s) != hipSuccess)
    return CLE_EHIP;
  if (ub2 > 0) {
    const int g = persistent_grid(ub2);
    if (dt == CLE_BF16)
      ffn_gemm_bf16<2><<<dim3(g), dim3(256), 0, s>>>(segs, nseg, totals, H, I);
    else
      ffn_gemm_f32<2><<<dim3(g), dim3(256), 0, s>>>(segs, nseg, totals, H, I);
  }
  if (phase_events && hipEventRecord(static_cast<hipEvent_t>(phase_events[2]), s) != hipSuccess)
    return CLE_EHIP;
  return launch_status();
}
