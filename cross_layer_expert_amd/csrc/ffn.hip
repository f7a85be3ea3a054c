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
//   phase 1  persistent kernel over all (segment, n-tile, m-tile) tiles,
//            K = H.  bf16: 128 rows x 128 act columns (the gate and up rows
//            of the same act columns are in one tile, so the SwiGLU epilogue
//            is local); f32: 64 x 64.
//   phase 2  same scheduler, K = I.  bf16: 128 rows x 256 output columns.
// bf16 path: v_mfma_f32_16x16x32_bf16 (gfx950), fp32 accumulation, no
// split-K.  The K loop over one weight block starts at a stage picked by the
// block's (layer, expert) alone and wraps around, so a row's result does not
// depend on which other segments share the launch, while tiles of different
// experts read different K offsets at the same time (tiles that all started
// at K = 0 would read addresses with equal low bits from thousands of rows at
// once and crowd the same HBM channels).
// Consecutive logical tiles go to one XCD (workgroups are dealt round-robin
// over the 8 XCDs) so tiles reading the same weight rows share that XCD's L2.
#include <hip/hip_ext.h>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "cle_internal.h"

namespace cle {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;        // rows per tile of the f32 path
constexpr int kBNF = 64;       // columns per tile of the f32 path (both phases)
constexpr int kPlanDescs = 16;
constexpr int kXcds = 8;
// the per-XCD tile claim counters of the two phases sit in the workspace
// header after the tile totals: ints [kClaimsOffset, kClaimsOffset + 16)
constexpr int kClaimsOffset = 16;
// then the segment counter of the fused thin-segment launch: int [kClaimsOffset + 16]
constexpr int kFusedCounter = kClaimsOffset + 2 * kXcds;
static_assert((kFusedCounter + 1) * sizeof(int) <= kFfnHeader, "workspace header");

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
  const void* x;      // token rows, read through src when xp is NULL
  const int* src;
  int k;
};

struct PlanArgs {
  DescDev d[kPlanDescs];
  int layer_all[CLE_MAX_DESC];  // layer of every descriptor of the launch (no loop state)
  int c0, nd, n_all;            // descriptors [c0, c0 + nd) of n_all are planned here
  int E, ns, H, I, esz, L;
  // non-NULL: descriptor j runs only if it is in st->runset, at layer
  // st->run_layer[j] (its own layer field and layer_all are unused)
  const cle_loop_state* st;
  // the launch that plans the last descriptors also orders the whole table
  // (see order_segments); earlier launches leave these unused
  int order, nseg, tm, n1, n2;
  int thin;  // > 0: routed segments of 1 .. thin rows go to the fused thin-segment launch
  int* totals;
  int* mscan;
};

// Expert weight tensors of a launch; a segment names its matrices by index.
struct Weights {
  const void* w13;
  const void* w2;
  const void* w13s;
  const void* w2s;
};
static_assert(sizeof(PlanArgs) <= 4096, "kernel argument size");

// ---------------------------------------------------------------- planning
// Row range [lo, hi) of routed expert e, clamped to the descriptor's rows so
// that inconsistent offsets can never reach outside the caller's buffers.
__device__ __forceinline__ void seg_range(const DescDev& d, int e, int& lo, int& hi) {
  lo = min(max(d.offsets[e], 0), d.rows);
  hi = min(max(d.offsets[e + 1], lo), d.rows);
}

// Row tiles of a segment in the two GEMM phases (none for a segment the fused
// thin-segment launch runs).
__device__ __forceinline__ int seg_tiles(int rows, int fused, int tm) {
  return fused ? 0 : (rows + tm - 1) / tm;
}

// One block over the grouped segment table: the row-tile prefix M over the
// segments (mscan[s] = row tiles of segments before s), then per segment its
// group's start m0 = M at the group's first segment, the group's row tiles
// gmt and its own offset moff in the group.  Group g of m-tile start m0
// owns tiles [N * m0, N * (m0 + gmt)) of a phase with N column tiles, in
// the order locate_tile gives.  Runs at the end of the last planning launch,
// after a block barrier, so the segments this block wrote are visible.
__device__ __forceinline__ void order_segments(Seg* __restrict__ segs, int nseg, int tm, int n1,
                                               int n2, int* __restrict__ totals,
                                               int* __restrict__ mscan, int* part) {
  const int tid = threadIdx.x;
  const int per = (nseg + 1023) / 1024;
  const int lo = min(nseg, tid * per), hi = min(nseg, lo + per);
  int c = 0;
  for (int s = lo; s < hi; ++s) c += seg_tiles(segs[s].rows, segs[s].fused, tm);
  part[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += a;
    __syncthreads();
  }
  int m = part[tid] - c;
  for (int s = lo; s < hi; ++s) {
    mscan[s] = m;
    m += seg_tiles(segs[s].rows, segs[s].fused, tm);
  }
  if (tid == 1023) {
    mscan[nseg] = m;
    totals[0] = n1 * m;
    totals[1] = n2 * m;
  }
  __syncthreads();
  for (int s = lo; s < hi; ++s) {
    const int s0 = s - segs[s].grank, s1 = s0 + segs[s].gsize;
    const int m0 = mscan[s0];
    segs[s].m0 = m0;
    segs[s].gmt = mscan[s1] - m0;
    segs[s].moff = mscan[s] - m0;
  }
}

// order_segments for a table planned by this one block (at most kPlanLds
// segments), from the rows and group fields the block kept in LDS: no
// global round trips between the passes.
constexpr int kPlanLds = 2048;
__device__ __forceinline__ void order_segments_lds(Seg* __restrict__ segs, int nseg, int tm,
                                                   int n1, int n2, int* __restrict__ totals,
                                                   const int* rows_l, const int* grp_l,
                                                   int* mscan_l, int* part) {
  const int tid = threadIdx.x;
  const int per = (nseg + 1023) / 1024;
  const int lo = min(nseg, tid * per), hi = min(nseg, lo + per);
  int c = 0;
  for (int s = lo; s < hi; ++s) c += (rows_l[s] + tm - 1) / tm;
  part[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += a;
    __syncthreads();
  }
  int m = part[tid] - c;
  for (int s = lo; s < hi; ++s) {
    mscan_l[s] = m;
    m += (rows_l[s] + tm - 1) / tm;
  }
  if (tid == 1023) {
    mscan_l[nseg] = m;
    totals[0] = n1 * m;
    totals[1] = n2 * m;
  }
  __syncthreads();
  for (int s = lo; s < hi; ++s) {
    const int grank = static_cast<int16_t>(grp_l[s] & 0xffff), gsize = grp_l[s] >> 16;
    const int s0 = s - grank, s1 = s0 + gsize;
    const int m0 = mscan_l[s0];
    segs[s].m0 = m0;
    segs[s].gmt = mscan_l[s1] - m0;
    segs[s].moff = mscan_l[s] - m0;
  }
}

// Writes the segments of descriptors [c0, c0 + nd) at their grouped
// positions.  Descriptors are grouped by layer (ascending; micro-batches not
// in the loop state's RunSet form a last, empty group); within the group of
// layer u, holding cnt micro-batches of which j is the rank-th, segment
// (j, e) sits at  base(u) + e * cnt + rank,  base(u) = (E + ns) * (number of
// descriptors at layers below u).  So the segments of one (layer, expert) are
// adjacent, ordered by micro-batch.
__global__ __launch_bounds__(1024) void ffn_plan(PlanArgs p, Seg* __restrict__ segs) {
  __shared__ DescDev dd[kPlanDescs];
  __shared__ int lay[CLE_MAX_DESC];
  __shared__ int pbase[kPlanDescs], pcnt[kPlanDescs], prank[kPlanDescs];
  const int tid = threadIdx.x;
  if (tid < p.n_all) {
    if (p.st)
      lay[tid] = (p.st->runset >> tid & 1) ? p.st->run_layer[tid] : p.L;
    else
      lay[tid] = p.layer_all[tid];
  }
  if (tid < p.nd) {
    DescDev d = p.d[tid];
    if (p.st) {
      const int j = p.c0 + tid;
      if (p.st->runset >> j & 1) {
        d.layer = p.st->run_layer[j];
      } else {
        d.rows = 0;
        d.shared_rows = 0;
        d.layer = 0;
      }
    }
    dd[tid] = d;
  }
  __syncthreads();
  if (tid < p.nd) {
    const int j = p.c0 + tid, u = lay[j];
    int below = 0, cnt = 0, rank = 0;
    for (int q = 0; q < p.n_all; ++q) {
      below += lay[q] < u;
      cnt += lay[q] == u;
      rank += lay[q] == u && q < j;
    }
    pbase[tid] = below * (p.E + p.ns);
    pcnt[tid] = cnt;
    prank[tid] = rank;
  }
  __syncthreads();
  // one launch plans the whole table: its rows and group fields stay in LDS
  // for the ordering pass
  __shared__ int rows_l[kPlanLds], grp_l[kPlanLds], mscan_l[kPlanLds + 1];
  const bool in_lds = p.order && p.c0 == 0 && p.nseg <= kPlanLds;
  const int64_t H = p.H, I = p.I, esz = p.esz;
  for (int s = tid; s < p.nd * (p.E + p.ns); s += 1024) {
    const int jl = s / (p.E + p.ns), e = s % (p.E + p.ns);
    const DescDev& d = dd[jl];
    Seg g;
    if (e < p.E) {
      int lo, hi;
      seg_range(d, e, lo, hi);
      const int64_t off = lo;
      g.rows = hi - lo;
      if (d.xp) {
        g.a = reinterpret_cast<const uint16_t*>(static_cast<const char*>(d.xp) + off * H * esz);
        g.rmap = nullptr;
        g.kdiv = 1;
      } else {
        g.a = static_cast<const uint16_t*>(d.x);
        g.rmap = d.src + off;
        g.kdiv = static_cast<int16_t>(d.k);
      }
      g.act = static_cast<char*>(d.act) + off * I * esz;
      g.y = static_cast<char*>(d.yp) + off * H * esz;
      g.widx = d.layer * p.E + e;
    } else {
      const int64_t q = e - p.E, R = d.shared_rows;
      g.rows = d.shared_rows;
      g.a = reinterpret_cast<const uint16_t*>(d.x_shared);
      g.rmap = nullptr;
      g.kdiv = 1;
      g.act = static_cast<char*>(d.act_shared) + q * R * I * esz;
      g.y = static_cast<char*>(d.y_shared) + q * R * H * esz;
      g.widx = -1 - (d.layer * p.ns + static_cast<int>(q));
    }
    g.kkey = static_cast<uint16_t>(d.layer * 7 + e * 5);  // e counts shared experts after E
    g.m0 = g.gmt = g.moff = 0;
    g.grank = static_cast<int16_t>(prank[jl]);
    g.gsize = static_cast<int16_t>(pcnt[jl]);
    g.fused = p.thin > 0 && g.rows >= 1 && g.rows <= p.thin && g.widx >= 0;
    const int pos = pbase[jl] + e * pcnt[jl] + prank[jl];
    segs[pos] = g;
    if (in_lds) {
      rows_l[pos] = g.fused ? 0 : g.rows;  // tiles of the two phases
      grp_l[pos] = (static_cast<int>(g.gsize) << 16) | static_cast<uint16_t>(g.grank);
    }
  }
  if (p.order) {
    __shared__ int part[1024];
    if (tid < 2 * kXcds + 1) p.totals[kClaimsOffset + tid] = 0;  // tile claims, fused counter
    __syncthreads();
    if (in_lds)
      order_segments_lds(segs, p.nseg, p.tm, p.n1, p.n2, p.totals, rows_l, grp_l, mscan_l, part);
    else
      order_segments(segs, p.nseg, p.tm, p.n1, p.n2, p.totals, p.mscan, part);
  }
}

// Tile -> (segment, column tile, row tile) in a phase with N column tiles
// and tm-row tiles: the group is found by binary search on m0 (the last
// segment with m0 <= tile / N is its group's last segment), the segment by a
// walk through the group.  Within a group the tiles run in blocks of C
// column tiles (the last block may be narrower): block by block, and in a
// block row tile by row tile, its C column tiles back to back.  C = 1 is
// column-tile-major order (every tile reading one block of weight rows runs
// back to back); C > 1 has the C column tiles that read the same A rows run
// one after another, so those rows are still in L2 for the later ones.
struct TilePos {
  int si, nt, mi;
};

__device__ __forceinline__ TilePos locate_tile(const Seg* segs, int nseg, int tile, int N,
                                               int tm, int C = 1) {
  const int x = tile / N;
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].m0 <= x) lo = mid;
    else hi = mid - 1;
  }
  const int m0 = segs[lo].m0, gmt = segs[lo].gmt;
  const int r = tile - N * m0;
  const int p = r / (C * gmt);            // block of column tiles
  const int cb = min(C, N - p * C);       // its width
  const int w = r - p * C * gmt;
  const int nt = p * C + w % cb, q = w / cb;
  // grank is read with its neighbour as one 32-bit word: a 16-bit load would
  // be a vector load, whose wait would also wait for every operand load in flight
  int32_t gw;
  __builtin_memcpy(&gw, &segs[lo].grank, sizeof(gw));
  int s = lo - static_cast<int16_t>(gw & 0xffff);
  while (q >= segs[s].moff + seg_tiles(segs[s].rows, segs[s].fused, tm)) ++s;
  return TilePos{s, nt, q - segs[s].moff};
}

__device__ __forceinline__ const void* seg_weights(const Weights& w, const Seg& g, int PHASE,
                                                   int64_t H, int64_t I, int esz) {
  const int64_t mat = PHASE == 1 ? 2 * I * H : H * I;
  const void* base = g.widx >= 0 ? (PHASE == 1 ? w.w13 : w.w2) : (PHASE == 1 ? w.w13s : w.w2s);
  const int64_t idx = g.widx >= 0 ? g.widx : -1 - static_cast<int64_t>(g.widx);
  return static_cast<const char*>(base) + idx * mat * esz;
}

__device__ __forceinline__ int logical_tile_base(int grid) {
  // grid is a multiple of kXcds; workgroup b runs on XCD b % kXcds
  const int b = blockIdx.x;
  return (b % kXcds) * (grid / kXcds) + b / kXcds;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// The bf16 tiles' SwiGLU epilogue: silu(g) = g / (1 + e^-g) evaluated as
// g * rcp(1 + 2^(-g log2 e)) with the hardware exp2 and reciprocal (each about
// 1 ulp of float32, far below the bf16 rounding of Act), and the hardware
// round-to-nearest-even conversion to bf16.  Six VALU instructions per act
// value instead of about thirty for expf and an IEEE division, which made the
// epilogue of a full tile cost several microseconds.
__device__ __forceinline__ float silu_hw(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}
__device__ __forceinline__ uint16_t bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ---------------------------------------------------------------- bf16 MFMA tiles
// A tile in LDS: [kBM rows][8 chunks of 16 bytes], chunk c of row r stored at
// c ^ (r & 7) to spread the column reads of 16 rows over the banks.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Workgroup barrier for LDS hand-off only.  __syncthreads() also orders
// global memory, which on gfx9 means waiting for every outstanding vector
// load -- including the prefetches of later K steps -- so it would drain the
// software pipeline at every step.  Here only LDS traffic is waited for.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte load from global memory.  The pointers come out of the segment
// table, so the compiler cannot see their address space and would emit flat
// loads, which also count against the LDS counter and would make every
// LDS barrier wait for the prefetches; the cast makes them global loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  const u32x4 v = *(gu32x4*)(p);
  return __builtin_bit_cast(uint4, v);
}

// Grouped GEMM tile kernel (bf16, gfx950).
//
// A tile is 128 rows x (WN * NB) weight blocks of 16 rows.  Wavefront w
// loads NB consecutive weight blocks -- phase 1: NB/2 blocks of gate rows and
// the NB/2 blocks of up rows of the same act columns; phase 2: NB blocks of
// output columns -- and 128/WN rows of A per stage.  For the MFMAs the
// standard 8-wavefront tile (NB = 2: 128 act columns / 256 output columns) is
// split 2 x 4: wavefront (rg, cg) computes rows 64*rg .. 64*rg+63 of the four
// blocks loaded by wavefronts 2cg and 2cg+1 (gate/up pairs stay together, so
// the SwiGLU epilogue is local).  Per K slice a wavefront then reads 4 A and
// 4 weight fragments from LDS instead of 8 + 2, which takes a fifth off the
// LDS reads that compete with the direct loads for the LDS port (measured
// together with the exact K-loop tail below: gate/up unchanged on the Qwen3
// step, down 4 % and long-prefill phases 5-7 % faster).  Shapes that do not
// divide into it use WN = 4 x NB = 2, one row group.  (Four wavefronts x four blocks, one wavefront per SIMD, measured
// slower: the memory and barrier stalls of a stage are not hidden.)
//
//  * Operands move with direct global->LDS loads (global_load_lds_dwordx4, no
//    registers) into a ring of kStages LDS stages, two stages in flight.
//  * Every load instruction covers 8 rows x 128 contiguous bytes (64 K
//    elements), i.e. 8 whole cache lines: the vector memory path takes 16
//    bytes per lane at full rate only when each quad of lanes reads 64
//    contiguous bytes, which the 16-rows-per-instruction MFMA operand layout
//    does not, so the operands are re-laid out through LDS.  Lane p writes
//    LDS position 16*p of its 1 KiB slot and fetches row p/8, 16-byte chunk
//    (p%8) ^ (p/8) of the 8-row group: an XOR swizzle under which the operand
//    reads (16 rows x one chunk per quarter-wave) hit distinct banks.
// Row blocks past the end of a segment cost no MFMAs or stores; their loads
// repeat the segment's last row.
constexpr int kTM = 128;
constexpr int kMB = kTM / 16;   // 16-row blocks per tile
constexpr int kKS = 64;         // K per stage (two MFMA K slices)
constexpr int kStages = 3;
constexpr int kBlocks = 16;     // most weight blocks per tile (WN * NB)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gvoid;
// Global-address-space views for the tile's row-map loads and output stores:
// through a generic pointer they would be flat instructions, which also count
// against the LDS counter, so every LDS barrier would wait for them.
typedef __attribute__((address_space(1))) const int gcint;
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef __attribute__((address_space(1))) float gf32;
typedef __attribute__((address_space(1))) int gint;

// AUX: the load's cache policy (0: default; kLoadNT: non-temporal, for lines
// that no other tile reads, so they do not displace lines that will be reused;
// plain streaming also runs faster with it, 7.2 against 6.2 TB/s measured)
constexpr int kLoadNT = 2;
template <int AUX = 0>
__device__ __forceinline__ void dma16(const uint16_t* src, uint4* lds_slot) {
  __builtin_amdgcn_global_load_lds((gvoid*)(src), (lds_void*)(lds_slot), 16, 0, AUX);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Barrier once this wavefront's LDS reads have completed; the empty asm keeps
// the compiler from moving LDS reads above it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One pipeline stage: a 16-row x 64-K operand block is two 1 KiB slots
// (rows 0-7, rows 8-15) of 64 lane positions.
struct StageLDS {
  uint4 w[kBlocks][2][64];  // [wave * NB + block][row group][position]
  uint4 x[kMB][2][64];      // [row block][row group][position]
};
// The stages, referenced by name (one set per kernel instantiation), so the
// compiler can tell which stage each direct load writes and each read reads,
// and waits only for the loads a read depends on.
template <int PHASE, int WN, int NB, bool PACKED> __shared__ StageLDS g_st0;
template <int PHASE, int WN, int NB, bool PACKED> __shared__ StageLDS g_st1;
template <int PHASE, int WN, int NB, bool PACKED> __shared__ StageLDS g_st2;

// Everything one tile needs, resolved from the segment table.
struct TileArgs {
  const uint16_t* wlo;  // first weight row of this wavefront's blocks 0 .. NB/2-1
  const uint16_t* whi;  // first weight row of its blocks NB/2 .. NB-1
  const uint16_t* A;    // first row of the tile's A operand (rmap == NULL), or the
                        // token rows the row map points into
  const int* rmap;      // NULL, or the row map from this tile's first row
  int kdiv;             // row r of the tile is token rmap[r] / kdiv of A
  uint16_t* out;        // first row of the tile's output
  int K;                // reduction length (row stride of A and W)
  int rot;              // first K stage of the loop (it wraps around at K)
  int ldo;              // output row stride
  int col;              // this lane's output column in the wavefront's first block
  int nrows;            // valid rows of the tile (1..kTM)
  const float* bias;    // phase 3: per-column bias added to the float32 output, or NULL
};

// Instruction order of one half step, for the scheduler: the NB weight
// fragment reads, then NMB times (NB MFMAs, one A fragment read).  The MFMAs
// of a half step use operands read in the previous half step, so each read
// has the MFMAs issued after it to land.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
template <int I, int N, int NB>
__device__ __forceinline__ void mfma_read_pairs() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, NB, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    mfma_read_pairs<I + 1, N, NB>();
  }
}
template <int NMB, int NB>
__device__ __forceinline__ void half_step_order() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NB, 0);
  mfma_read_pairs<0, NMB, NB>();
}

// The K loop and epilogue of one tile.  Loading and computing are split
// differently: wavefront w loads weight blocks w*NB .. w*NB+NB-1 and A row
// blocks w*XB .. w*XB+XB-1 of every stage, while for the MFMAs the WN
// wavefronts form RH row groups x WN/RH column groups.  Wavefront (rh, cg)
// computes rows rh*128/RH .. +128/RH of weight blocks cg*RB .. cg*RB+RB-1
// (RB = NB*RH; those are the blocks loaded by wavefronts cg*RH .. cg*RH+RH-1).
// RH = 2 reads 4 A + 4 weight fragments per K slice where RH = 1 reads 8 + 2,
// a fifth fewer LDS operand bytes per stage, with the same loads and MFMAs.
// RG is this wavefront's row group and NMB the number of 16-row blocks it
// computes (0 .. 8/RH); both are compile-time values, so the MFMA sequence
// has no data-dependent branches and every LDS operand offset is a constant.
// TR is the number of K-loop steps left after the last whole round (2 .. 4,
// fixed by K: 2 + (K/64 - 3) mod 3 for K >= 192), or -1 for code that takes
// any K; one tail per kernel keeps the register footprint of the loop low.
// hook() runs once the tile's first three stages are requested, while they
// are in flight (the persistent loop looks up its next tile there).
struct NoHook {
  __device__ void operator()() const {}
};

template <int PHASE, int WN, int NB, bool PACKED, int RH, int RG, int NMB, int TR,
          int BUF = PHASE, bool WNT = false, typename Hook = NoHook>
__device__ __forceinline__ void tile_nmb(const TileArgs& t, int wave, int lane,
                                         const Hook& hook = Hook()) {
  // lane-derived offsets (operand positions, epilogue rows) are recomputed per
  // tile: hoisted out of the persistent loop they would hold a register each
  // for the whole kernel
  asm volatile("" : "+v"(lane));
  static_assert(WN * NB <= kBlocks && WN % RH == 0 && kMB % RH == 0, "weight blocks per tile");
  static_assert(NMB >= 0 && NMB <= kMB / RH && RG >= 0 && RG < RH, "row blocks per wavefront");
  constexpr int XB = kMB / WN;  // A row blocks loaded by each wavefront
  constexpr int HB = NB / 2;
  constexpr int RB = NB * RH;   // weight blocks each wavefront computes
  constexpr int AM = NMB > 0 ? NMB : 1;
  const int cg = wave % (WN / RH);
  constexpr int xb0 = RG * (kMB / RH);  // first A row block of this wavefront
  const int KT = t.K / kKS;
  // load side: this lane fetches row lr of each 8-row group, chunk lc
  const int lr = lane / 8, lc = (lane % 8) ^ (lane / 8);
  const uint16_t* wp[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g = 0; g < 2; ++g)
      wp[b][g] = (b < HB ? t.wlo : t.whi) + (b % HB) * 16 * t.K +
                 (PACKED ? g * 512 + lane * 8 : (g * 8 + lr) * t.K + lc * 8);
  const uint16_t* xp[XB][2];
#pragma unroll
  for (int b = 0; b < XB; ++b)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // rows past the tile repeat its last row (never stored)
      const int row = min((wave * XB + b) * 16 + g * 8 + lr, t.nrows - 1);
      const int64_t arow =
          t.rmap ? static_cast<int64_t>(*(gcint*)(t.rmap + row) / t.kdiv) : row;
      xp[b][g] = t.A + arow * t.K + lc * 8;
    }
  // read side: MFMA operand of lane `lane` for K slice h is row lane%16,
  // chunk 4h + lane/16: row group rg, position (lane%8)*8 + (chunk ^ lane%8)
  const int rg = (lane % 16) / 8, r8 = lane % 8;
  const int pos0 = r8 * 8 + ((0 + lane / 16) ^ r8);
  const int pos1 = r8 * 8 + ((4 + lane / 16) ^ r8);

  f32x4 acc[RB][AM];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int mb = 0; mb < AM; ++mb) acc[b][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // request K stage KT_ (of the rotated order) into ST
#define CLE_ISSUE(ST, KT_)                                                          \
  {                                                                                 \
    int kr = (KT_) + t.rot;                                                         \
    kr -= kr >= KT ? KT : 0;                                                        \
    const int ko = kr * kKS;                                                        \
    if constexpr (WNT) {                                                            \
      _Pragma("unroll") for (int b = 0; b < NB; ++b)                                \
        _Pragma("unroll") for (int g = 0; g < 2; ++g)                               \
          dma16<kLoadNT>(wp[b][g] + (PACKED ? kr * 1024 : ko), &ST.w[wave * NB + b][g][0]); \
    } else {                                                                        \
      _Pragma("unroll") for (int b = 0; b < NB; ++b)                                \
        _Pragma("unroll") for (int g = 0; g < 2; ++g)                               \
          dma16(wp[b][g] + (PACKED ? kr * 1024 : ko), &ST.w[wave * NB + b][g][0]);   \
    }                                                                               \
    _Pragma("unroll") for (int b = 0; b < XB; ++b)                                  \
      _Pragma("unroll") for (int g = 0; g < 2; ++g)                                 \
        dma16(xp[b][g] + ko, &ST.x[wave * XB + b][g][0]);                           \
  }
  // The operands of one K slice of a stage: RB weight fragments and NMB A
  // fragments, read from LDS into registers.  Slice 0 and slice 1 have their
  // own registers.  A wavefront with no row blocks reads and computes nothing.
  bf16x8 fb[2][RB], fa[2][AM];
#define CLE_READ(ST, H)                                                             \
  if constexpr (NMB > 0) {                                                          \
    const int pos = (H) == 0 ? pos0 : pos1;                                         \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      fb[H][b] = __builtin_bit_cast(bf16x8, ST.w[cg * RB + b][rg][pos]);            \
    _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                              \
      fa[H][mb] = __builtin_bit_cast(bf16x8, ST.x[xb0 + mb][rg][pos]);              \
  }
#define CLE_MFMA(H)                                                                 \
  _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                                \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      acc[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[H][mb], fb[H][b], acc[b][mb], 0, 0, 0);
  // Software pipeline by half a stage.  On entry to step KT_ the slice-0
  // MFMAs of stage KT_ are issued and its slice-1 operands are in registers;
  // stage KT_ sits in buffer CUR and stage KT_+1 in NXT.  The step waits for
  // this wavefront's loads of stage KT_+1 (W = the loads it may leave in
  // flight: stage KT_+2 if that exists), synchronises (every wavefront's
  // loads of KT_+1 have landed, and every wavefront has finished reading
  // CUR), requests stage KT_+3 into CUR if that exists, then issues the
  // slice-1 MFMAs of KT_ while reading slice 0 of KT_+1, and the slice-0
  // MFMAs of KT_+1 while reading its slice 1, so the LDS reads of a stage
  // overlap the MFMAs of its neighbours.  The main loop runs whole rounds of
  // three steps that all request a stage; the last two to four steps are
  // straight-line code with the exact request and wait pattern, so no stage is
  // requested twice and the compiler sees which buffer every request writes.
  constexpr int kPerStep = 2 * NB + 2 * XB;
#define CLE_STEP_TAIL(NXT)                                                          \
    CLE_MFMA(1);                                                                    \
    CLE_READ(NXT, 0);                                                               \
    half_step_order<NMB, RB>();                                                     \
    CLE_MFMA(0);                                                                    \
    CLE_READ(NXT, 1);                                                               \
    half_step_order<NMB, RB>();
#define CLE_STEP(CUR, NXT, KT_)                                                     \
  {                                                                                 \
    wait_vmcnt<kPerStep>();                                                         \
    stage_barrier();                                                                \
    CLE_ISSUE(CUR, (KT_) + 3);                                                      \
    CLE_STEP_TAIL(NXT)                                                              \
  }
#define CLE_STEP_NOREQ(NXT, W)                                                      \
  {                                                                                 \
    wait_vmcnt<W>();                                                                \
    stage_barrier();                                                                \
    CLE_STEP_TAIL(NXT)                                                              \
  }

  static_assert(kStages == 3, "the pipeline below is written for 3 buffers");
  // BUF names the stage buffers (a kernel that runs both phases shares one set)
  auto& st0 = g_st0<BUF, WN, NB, PACKED>;
  auto& st1 = g_st1<BUF, WN, NB, PACKED>;
  auto& st2 = g_st2<BUF, WN, NB, PACKED>;
  // (K / 64 < 3 only on small shapes: the prologue then re-requests the last
  // stage into a buffer no step reads; the final wait covers it.)
  CLE_ISSUE(st0, 0);
  CLE_ISSUE(st1, min(1, KT - 1));
  CLE_ISSUE(st2, min(2, KT - 1));
  hook();
  wait_vmcnt<2 * kPerStep>();
  stage_barrier();
  CLE_READ(st0, 0);
  CLE_MFMA(0);
  CLE_READ(st0, 1);
  int kt = 0;
  for (; kt + 5 < KT; kt += 3) {
    CLE_STEP(st0, st1, kt);
    CLE_STEP(st1, st2, kt + 1);
    CLE_STEP(st2, st0, kt + 2);
  }
  // stage kt is in st0; steps kt .. KT-2 remain (stages up to min(kt+2, KT-1)
  // requested)
  switch (TR >= 0 ? TR : KT - 1 - kt) {
    case 4:
      CLE_STEP(st0, st1, kt);
      CLE_STEP(st1, st2, kt + 1);
      CLE_STEP_NOREQ(st0, kPerStep);
      CLE_STEP_NOREQ(st1, 0);
      break;
    case 3:
      CLE_STEP(st0, st1, kt);
      CLE_STEP_NOREQ(st2, kPerStep);
      CLE_STEP_NOREQ(st0, 0);
      break;
    case 2:
      CLE_STEP_NOREQ(st1, kPerStep);
      CLE_STEP_NOREQ(st2, 0);
      break;
    case 1:
      CLE_STEP_NOREQ(st1, 0);
      break;
    default:
      break;
  }
  CLE_MFMA(1);  // slice 1 of the last stage
#undef CLE_ISSUE
#undef CLE_READ
#undef CLE_MFMA
#undef CLE_STEP
#undef CLE_STEP_NOREQ
#undef CLE_STEP_TAIL
  wait_vmcnt<0>();  // every request has landed before the buffers are reused

  // epilogue: lane holds rows (xb0+mb)*16 + (lane/16)*4 + i, column lane%16 of
  // each block.  Phase 1 pairs gate block b with up block HB+b of each loading
  // wavefront; the act columns of consecutive pairs are 16 apart.
  const int g4 = lane / 16;
  const int col = t.col + cg * RH * 16 * (PHASE == 1 ? HB : NB);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (xb0 + mb) * 16 + g4 * 4 + i;
      if (row < t.nrows) {
        gu16* o = (gu16*)(t.out + row * t.ldo + col);
        if (PHASE == 1) {
#pragma unroll
          for (int u = 0; u < RH; ++u)
#pragma unroll
            for (int b = 0; b < HB; ++b)
              o[(u * HB + b) * 16] =
                  bf16_hw(silu_hw(acc[u * NB + b][mb][i]) * acc[u * NB + HB + b][mb][i]);
        } else if (PHASE == 3) {
          gf32* of = (gf32*)(reinterpret_cast<float*>(t.out) + row * t.ldo + col);
#pragma unroll
          for (int b = 0; b < RB; ++b)
            of[b * 16] = t.bias ? acc[b][mb][i] + t.bias[col + b * 16] : acc[b][mb][i];
        } else {
#pragma unroll
          for (int b = 0; b < RB; ++b) o[b * 16] = bf16_hw(acc[b][mb][i]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // store block by block (bounded live ranges)
  }
}

// ---------------------------------------------------------------- 256-row tiles
// The 8-wavefront tile with twice the rows: 256 rows x 256 weight rows.  Every
// CU fetches its operands through its vector L1, whose outstanding misses are
// limited, so on the large segments the rate at which a CU can bring operands
// in (tens of bytes per clock, set by that limit and the L2 latency) rather
// than the matrix cores sets the tile's time; this tile fetches (256 + 256) x K
// operand elements per 256 x 256 x K products, two thirds of the 128-row
// tile's bytes per FLOP.  A stage (K = 64) is 64 KiB, so the ring holds two:
// stage k+2 is requested into stage k's buffer once every wavefront has read
// stage k, and has the MFMAs of one stage to land.  K / 64 is even for every
// shape this tile takes (K = H with H % 256 == 0, or K = I with I % 128 ==
// 0), so the loop runs whole pairs of steps and needs no tail variants.  The
// compute layout is the 128-row tile's 2 x 4 with 128 rows per row group.
constexpr int kTM2 = 256;
constexpr int kMB2 = kTM2 / 16;  // 16-row blocks per 256-row tile
struct StageLDS2 {
  uint4 w[kBlocks][2][64];  // [wave * 2 + block][row group][position]
  uint4 x[kMB2][2][64];     // [row block][row group][position]
};
template <int PHASE, bool PACKED> __shared__ StageLDS2 g_sb0;
template <int PHASE, bool PACKED> __shared__ StageLDS2 g_sb1;

template <int PHASE, bool PACKED, int RG, int NMB, typename Hook = NoHook>
__device__ __forceinline__ void tile256_nmb(const TileArgs& t, int wave, int lane,
                                            const Hook& hook = Hook()) {
  asm volatile("" : "+v"(lane));  // recomputed per tile, as in tile_nmb
  constexpr int WN = 8, NB = 2, RH = 2;
  constexpr int XB = kMB2 / WN;  // A row blocks loaded by each wavefront
  constexpr int HB = NB / 2;
  constexpr int RB = NB * RH;    // weight blocks each wavefront computes
  constexpr int AM = NMB > 0 ? NMB : 1;
  static_assert(NMB >= 0 && NMB <= kMB2 / RH && RG >= 0 && RG < RH, "row blocks per wavefront");
  const int cg = wave % (WN / RH);
  constexpr int xb0 = RG * (kMB2 / RH);  // first A row block of this wavefront
  const int KT = t.K / kKS;
  // load side: this lane fetches row lr of each 8-row group, chunk lc
  const int lr = lane / 8, lc = (lane % 8) ^ (lane / 8);
  // Which wavefronts request a stage.  The two wavefronts of a SIMD belong to
  // different row groups, and the SIMD issues for the first row group's
  // wavefront first, so the second one finishes every step alone.  In the
  // gate/up phase (K = H, long K loops) the first row group's wavefronts
  // request the whole stage, their own blocks and those of the wavefront four
  // above them, and the second row group's request nothing, which shifts
  // issue slots towards the wavefronts that finish last (gate/up 1-3 %
  // faster, measured; in the down phase, with 11-step K loops, it was 4 %
  // slower, so there every wavefront requests its own blocks).
  constexpr int LW = PHASE == 1 ? (RG == 0 ? 2 : 0) : 1;
  constexpr int LWA = LW > 0 ? LW : 1;
  const int64_t wshift = static_cast<int64_t>(4 * 16 * (PHASE == 1 ? HB : NB)) * t.K;
  const uint16_t* wp[LWA][NB][2];
#pragma unroll
  for (int v = 0; v < LWA; ++v)
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g = 0; g < 2; ++g)
      wp[v][b][g] = (b < HB ? t.wlo : t.whi) + v * wshift + (b % HB) * 16 * t.K +
                    (PACKED ? g * 512 + lane * 8 : (g * 8 + lr) * t.K + lc * 8);
  const uint16_t* xp[LWA][XB][2];
#pragma unroll
  for (int v = 0; v < LWA; ++v)
#pragma unroll
  for (int b = 0; b < XB; ++b)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // rows past the tile repeat its last row (never stored)
      const int row = min(((wave + 4 * v) * XB + b) * 16 + g * 8 + lr, t.nrows - 1);
      const int64_t arow =
          t.rmap ? static_cast<int64_t>(*(gcint*)(t.rmap + row) / t.kdiv) : row;
      xp[v][b][g] = t.A + arow * t.K + lc * 8;
    }
  const int rg = (lane % 16) / 8, r8 = lane % 8;
  const int pos0 = r8 * 8 + ((0 + lane / 16) ^ r8);
  const int pos1 = r8 * 8 + ((4 + lane / 16) ^ r8);

  f32x4 acc[RB][AM];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int mb = 0; mb < AM; ++mb) acc[b][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

#define CLE_ISSUE(ST, KT_)                                                          \
  {                                                                                 \
    int kr = (KT_) + t.rot;                                                         \
    kr -= kr >= KT ? KT : 0;                                                        \
    const int ko = kr * kKS;                                                        \
    _Pragma("unroll") for (int v = 0; v < LW; ++v) {                                \
      _Pragma("unroll") for (int b = 0; b < NB; ++b)                                \
        _Pragma("unroll") for (int g = 0; g < 2; ++g)                               \
          dma16(wp[v][b][g] + (PACKED ? kr * 1024 : ko), &ST.w[(wave + 4 * v) * NB + b][g][0]); \
      _Pragma("unroll") for (int b = 0; b < XB; ++b)                                \
        _Pragma("unroll") for (int g = 0; g < 2; ++g)                               \
          dma16(xp[v][b][g] + ko, &ST.x[(wave + 4 * v) * XB + b][g][0]);            \
    }                                                                               \
  }
  bf16x8 fb[2][RB], fa[2][AM];
#define CLE_READ(ST, H)                                                             \
  if constexpr (NMB > 0) {                                                          \
    const int pos = (H) == 0 ? pos0 : pos1;                                         \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      fb[H][b] = __builtin_bit_cast(bf16x8, ST.w[cg * RB + b][rg][pos]);            \
    _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                              \
      fa[H][mb] = __builtin_bit_cast(bf16x8, ST.x[xb0 + mb][rg][pos]);              \
  }
#define CLE_MFMA(H)                                                                 \
  _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                                \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      acc[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[H][mb], fb[H][b], acc[b][mb], 0, 0, 0);
  // Step KT_ (stage KT_ in CUR, KT_+1 in NXT): on entry the slice-0 MFMAs of
  // stage KT_ are issued and its slice-1 operands are in registers.  Wait for
  // this wavefront's loads of stage KT_+1 (the only ones in flight), barrier
  // (every wavefront's loads of KT_+1 have landed and every wavefront has read
  // all of CUR), request stage KT_+2 into CUR, then the slice-1 MFMAs of KT_
  // while reading slice 0 of KT_+1, and the slice-0 MFMAs of KT_+1 while
  // reading its slice 1.
#define CLE_STEP2(CUR, NXT, KT_, ISS)                                               \
  {                                                                                 \
    wait_vmcnt<0>();                                                                \
    stage_barrier();                                                                \
    if constexpr (ISS) CLE_ISSUE(CUR, (KT_) + 2);                                   \
    CLE_MFMA(1);                                                                    \
    CLE_READ(NXT, 0);                                                               \
    half_step_order<NMB, RB>();                                                     \
    CLE_MFMA(0);                                                                    \
    CLE_READ(NXT, 1);                                                               \
    half_step_order<NMB, RB>();                                                     \
  }
  constexpr int kPerStep = LW * (2 * NB + 2 * XB);
  auto& sa = g_sb0<PHASE, PACKED>;
  auto& sb = g_sb1<PHASE, PACKED>;
  CLE_ISSUE(sa, 0);
  CLE_ISSUE(sb, 1);
  hook();
  wait_vmcnt<kPerStep>();
  stage_barrier();
  CLE_READ(sa, 0);
  CLE_MFMA(0);
  CLE_READ(sa, 1);
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    CLE_STEP2(sa, sb, kt, true);
    CLE_STEP2(sb, sa, kt + 1, true);
  }
  CLE_STEP2(sa, sb, kt, false);  // stage KT-2 in sa, KT-1 in sb
  CLE_MFMA(1);                   // slice 1 of the last stage
#undef CLE_ISSUE
#undef CLE_READ
#undef CLE_MFMA
#undef CLE_STEP2
  wait_vmcnt<0>();

  // The down phase's output rows are stored non-temporally: only the combine
  // reads them, once, in a later launch, so they need not displace the weight
  // and A lines the next tiles reuse (long-prefill down 2-3 % faster, its
  // combine unchanged; on the 128-row tiles of the thinner shapes the same
  // stores sped the down launch by 2 % but slowed the combine by more, since
  // its rows were then no longer in the last-level cache).
  const int g4 = lane / 16;
  const int col = t.col + cg * RH * 16 * (PHASE == 1 ? HB : NB);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (xb0 + mb) * 16 + g4 * 4 + i;
      if (row < t.nrows) {
        gu16* o = (gu16*)(t.out + row * t.ldo + col);
        if (PHASE == 1) {
#pragma unroll
          for (int u = 0; u < RH; ++u)
#pragma unroll
            for (int b = 0; b < HB; ++b)
              o[(u * HB + b) * 16] =
                  bf16_hw(silu_hw(acc[u * NB + b][mb][i]) * acc[u * NB + HB + b][mb][i]);
        } else {
#pragma unroll
          for (int b = 0; b < RB; ++b) __builtin_nontemporal_store(bf16_hw(acc[b][mb][i]), &o[b * 16]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- 512-wide tiles
// 128 rows x 512 weight rows (phase 1: 256 act columns, phase 2: 512 output
// columns): each wavefront loads four weight blocks per stage.  On large
// segments what bounds the expert launches is operand traffic, and most of
// what misses L2 is the A rows, which are read once per column tile (the
// concurrent tiles of one row tile start too far apart in time to share
// them in L2): twice the columns per tile halve those reads (3 instead of 6
// column tiles at I = 768, 4 instead of 8 at H = 2048; a third less fetched
// from HBM on the long-prefill launches).  What a CU can keep in flight is
// limited, so the ring stays deep: stages of K = 32 (40 KiB), four of them
// (the whole LDS), three in flight while one is computed.
// A stage slot is 16 rows x 64 bytes (1 KiB); 16-byte chunk i of row r sits
// at position r * 4 + (i ^ ((r >> 2) & 3)), so the MFMA operand reads (16
// rows x one chunk per quarter-wavefront) hit distinct banks; lane p of a
// load instruction fetches the chunk that belongs at its position p.
// Compute layout 1 x 8: each wavefront computes all 128 rows of the four
// weight blocks it loaded itself.
constexpr int kKS2 = 32;  // K per stage of the 512-wide tile
struct StageLDS4 {
  uint4 w[32][64];   // [wave * 4 + block][position]
  uint4 x[kMB][64];  // [row block][position]
};
template <int PHASE, bool PACKED> __shared__ StageLDS4 g_sw0;
template <int PHASE, bool PACKED> __shared__ StageLDS4 g_sw1;
template <int PHASE, bool PACKED> __shared__ StageLDS4 g_sw2;
template <int PHASE, bool PACKED> __shared__ StageLDS4 g_sw3;

template <int PHASE, bool PACKED, int NMB, typename Hook = NoHook>
__device__ __forceinline__ void tile512_nmb(const TileArgs& t, int wave, int lane,
                                            const Hook& hook = Hook()) {
  asm volatile("" : "+v"(lane));  // recomputed per tile, as in tile_nmb
  constexpr int WN = 8, NB = 4;
  constexpr int XB = kMB / WN;  // one A row block loaded per wavefront
  constexpr int HB = NB / 2;
  constexpr int RB = NB;        // weight blocks each wavefront computes (its own)
  constexpr int AM = NMB > 0 ? NMB : 1;
  static_assert(NMB >= 1 && NMB <= kMB, "row blocks per wavefront");
  const int KT = t.K / kKS2;
  // load side: lane p fetches row lr, chunk lc of a 16-row block (lc is the
  // chunk whose swizzled position is p)
  const int lr = lane >> 2, lc = (lane & 3) ^ ((lr >> 2) & 3);
  // the 64-K packed block holds K stage s in its half s & 1; chunk c of row
  // rr (of an 8-row group) at rr * 8 + (c ^ rr)
  const int pk = (lr >> 3) * 512 + (lr & 7) * 64;  // row lr's 128-byte run (elements)
  const uint16_t* wp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    wp[b] = (b < HB ? t.wlo : t.whi) + (b % HB) * 16 * t.K +
            (PACKED ? pk : lr * t.K + lc * 8);
  const uint16_t* xp[XB];
#pragma unroll
  for (int b = 0; b < XB; ++b) {
    const int row = min((wave * XB + b) * 16 + lr, t.nrows - 1);
    const int64_t arow = t.rmap ? static_cast<int64_t>(*(gcint*)(t.rmap + row) / t.kdiv) : row;
    xp[b] = t.A + arow * t.K + lc * 8;
  }
  // read side: MFMA operand of lane l is row l % 16, chunk l / 16
  const int rr = lane & 15;
  const int pos = rr * 4 + ((lane >> 4) ^ ((rr >> 2) & 3));

  f32x4 acc[RB][AM];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int mb = 0; mb < AM; ++mb) acc[b][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // request K stage KT_ (of the rotated order) into ST
#define CLE_ISSUE(ST, KT_)                                                          \
  {                                                                                 \
    int kr = (KT_) + t.rot;                                                         \
    kr -= kr >= KT ? KT : 0;                                                        \
    const int ko = kr * kKS2;                                                       \
    const int pkc = (kr >> 1) * 1024 + (((kr & 1) * 4 + lc) ^ (lr & 7)) * 8;         \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                                  \
      dma16(wp[b] + (PACKED ? pkc : ko), &ST.w[wave * NB + b][0]);                  \
    _Pragma("unroll") for (int b = 0; b < XB; ++b)                                  \
      dma16(xp[b] + ko, &ST.x[wave * XB + b][0]);                                   \
  }
  bf16x8 fb[2][RB], fa[2][AM];
#define CLE_READ(ST, H)                                                             \
  {                                                                                 \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      fb[H][b] = __builtin_bit_cast(bf16x8, ST.w[wave * NB + b][pos]);              \
    _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                              \
      fa[H][mb] = __builtin_bit_cast(bf16x8, ST.x[mb][pos]);                        \
  }
#define CLE_MFMA(H)                                                                 \
  _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                                \
    _Pragma("unroll") for (int b = 0; b < RB; ++b)                                  \
      acc[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[H][mb], fb[H][b], acc[b][mb], 0, 0, 0);
  // Step KT_: stage KT_'s operands are in registers (set KT_ & 1), stages
  // KT_+1 .. KT_+3 are in the other buffers.  Wait for this wavefront's loads
  // of stage KT_+1 (W: the loads it may leave in flight), barrier (everyone's
  // loads of KT_+1 have landed, everyone has read CUR), request stage KT_+4
  // into CUR, then the MFMAs of stage KT_ while reading stage KT_+1.
  constexpr int kPerStep = NB + XB;
#define CLE_STEP(CUR, NXT, KT_, W, ISS)                                             \
  {                                                                                 \
    wait_vmcnt<W>();                                                                \
    stage_barrier();                                                                \
    if constexpr (ISS) CLE_ISSUE(CUR, (KT_) + 4);                                   \
    CLE_MFMA((KT_) & 1);                                                            \
    CLE_READ(NXT, ((KT_) + 1) & 1);                                                 \
    half_step_order<NMB, RB>();                                                     \
  }
  auto& s0 = g_sw0<PHASE, PACKED>;
  auto& s1 = g_sw1<PHASE, PACKED>;
  auto& s2 = g_sw2<PHASE, PACKED>;
  auto& s3 = g_sw3<PHASE, PACKED>;
  CLE_ISSUE(s0, 0);
  CLE_ISSUE(s1, 1);
  CLE_ISSUE(s2, 2);
  CLE_ISSUE(s3, 3);
  hook();
  wait_vmcnt<3 * kPerStep>();
  stage_barrier();
  CLE_READ(s0, 0);
  int kt = 0;
  for (; kt + 4 < KT; kt += 4) {
    CLE_STEP(s0, s1, kt, 2 * kPerStep, true);
    CLE_STEP(s1, s2, kt + 1, 2 * kPerStep, true);
    CLE_STEP(s2, s3, kt + 2, 2 * kPerStep, true);
    CLE_STEP(s3, s0, kt + 3, 2 * kPerStep, true);
  }
  // stages KT-4 .. KT-1 sit in s0 .. s3 (KT % 4 == 0), all requested
  CLE_STEP(s0, s1, kt, 2 * kPerStep, false);
  CLE_STEP(s1, s2, kt + 1, kPerStep, false);
  CLE_STEP(s2, s3, kt + 2, 0, false);
  CLE_MFMA(1);  // stage KT-1 (odd)
#undef CLE_ISSUE
#undef CLE_READ
#undef CLE_MFMA
#undef CLE_STEP
  wait_vmcnt<0>();

  // lane holds rows mb*16 + (lane/16)*4 + i, column lane%16 of each of its
  // blocks; phase 1 pairs gate block b with up block HB + b (act columns of
  // consecutive pairs 16 apart)
  const int g4 = lane / 16;
  const int col = t.col + wave * 16 * (PHASE == 1 ? HB : NB);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mb * 16 + g4 * 4 + i;
      if (row < t.nrows) {
        gu16* o = (gu16*)(t.out + row * t.ldo + col);
        if (PHASE == 1) {
#pragma unroll
          for (int b = 0; b < HB; ++b)
            o[b * 16] = bf16_hw(silu_hw(acc[b][mb][i]) * acc[HB + b][mb][i]);
        } else {
#pragma unroll
          for (int b = 0; b < RB; ++b) o[b * 16] = bf16_hw(acc[b][mb][i]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int PHASE, int WN, int NB, bool PACKED, int TM> __shared__ int g_snext[2][4];

// Tiles go to XCDs in contiguous ranges of ceil(total / 8); within its XCD's
// range a workgroup takes the tile at (range start + its index among the XCD's
// workgroups) first, and then whichever tile the XCD's claim counter hands it,
// so the workgroups of an XCD finish within about one tile of each other
// whatever the tiles' lengths.  claims: this phase's 8 counters, zeroed by the
// planner.
template <int PHASE, int WN, int NB, bool PACKED, int TR, int TM = kTM>
__global__ __launch_bounds__(64 * WN, 1) void ffn_gemm_bf16(const Seg* __restrict__ segs,
                                                            int nseg,
                                                            const int* __restrict__ totals,
                                                            int* __restrict__ claims,
                                                            Weights wts, int H, int I) {
  constexpr bool kWide4 = NB == 4;  // the 512-wide tile (its stages fill the LDS)
  static_assert(kMB % WN == 0 && (WN * NB <= kBlocks || (kWide4 && WN == 8 && TM == kTM)) &&
                    NB % 2 == 0, "tile shape");
  static_assert(TM == kTM || (TM == kTM2 && WN == 8 && NB == 2), "tile height");
  constexpr int MBT = TM / 16;  // 16-row blocks per tile
  constexpr int HB = NB / 2;
  constexpr int RH = WN == 8 ? 2 : 1;  // row groups of the compute layout
  const int total = totals[PHASE - 1];
  const int grid = gridDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16;
  const int K = PHASE == 1 ? H : I;

  // column tiles of the phase: 16 * NB weight rows per wavefront (phase 1:
  // half gate, half up rows of 8 * NB act columns)
  const int ncols = PHASE == 1 ? I / (WN * 8 * NB) : H / (WN * 16 * NB);
  // grid is a multiple of kXcds; workgroup b runs on XCD b % kXcds
  const int xcd = blockIdx.x % kXcds, chunk = grid / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int lo = min(total, xcd * per), hi = min(total, lo + per);
  // by tile parity: next tile and its position (the 512-wide tile hands them
  // over through its stage buffer instead)
  auto& s_next = g_snext<PHASE, WN, NB, PACKED, TM>;
  // Tile order within a group (locate_tile): the 256-row gate/up tiles run
  // two column tiles at a time, so the second tile that reads a row tile's A
  // rows finds them in L2 (a quarter fewer bytes fetched from beyond L2 on
  // the long-prefill launches, gate/up 2-3 % faster, measured); other tiles
  // run column-tile-major (on the thin-segment shapes the pairs measured 2 %
  // slower, and in the down phase no faster).
  constexpr int kColBlock = TM == kTM2 && PHASE == 1 ? 2 : 1;
  int tile = lo + static_cast<int>(blockIdx.x) / kXcds;
  TilePos next =
      tile < hi ? locate_tile(segs, nseg, tile, ncols, TM, kColBlock) : TilePos{0, 0, 0};
  for (int par = 0; tile < hi; par ^= 1) {
    const TilePos tp = next;
    // Wavefront 0 claims the workgroup's next tile before this tile's first
    // requests (so the claim has returned once they are in flight), then in
    // the prologue locates it (scalar loads) and leaves both in LDS, where
    // the other wavefronts read them after this tile's barriers.
    int claim = 0;
    if (wave == 0 && lane == 0) {
      // a per-lane (vector) address: the counter is not folded into a
      // wave-aggregated atomic, whose result would be waited for at once
      gint* cp = (gint*)(claims + xcd);
      asm volatile("" : "+v"(cp));
      claim = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int tnext = hi;
    const auto look_ahead = [&]() {
      if (wave == 0) {
        tnext = lo + chunk + __builtin_amdgcn_readfirstlane(claim);
        if (tnext < hi) next = locate_tile(segs, nseg, tnext, ncols, TM, kColBlock);
        if (!kWide4 && lane == 0) {
          s_next[par][0] = tnext;
          s_next[par][1] = next.si;
          s_next[par][2] = next.nt;
          s_next[par][3] = next.mi;
        }
      }
    };
    const Seg sg = segs[tp.si];
    const int nt = tp.nt, mi = tp.mi;
    const int row0 = mi * TM;
    TileArgs t;
    t.K = K;
    // kdiv and kkey read as one 32-bit word (scalar load; see locate_tile)
    int32_t kw;
    __builtin_memcpy(&kw, &segs[tp.si].kdiv, sizeof(kw));
    const int kdiv = static_cast<int16_t>(kw & 0xffff), kkey = (kw >> 16) & 0xffff;
    t.rot = kkey % (K / kKS);
    if constexpr (kWide4) t.rot *= 2;  // the same K order counted in 32-K stages
    t.nrows = min(TM, sg.rows - row0);
    // The output row stride is laundered per tile: otherwise the compiler
    // hoists every per-row output offset (row * stride, one register per
    // row) out of the tile loop and keeps them all live.
    int ldo = PHASE == 1 ? I : H;
    asm volatile("" : "+s"(ldo));
    if (PHASE == 1 && sg.rmap) {
      t.A = sg.a;
      t.rmap = sg.rmap + row0;
      t.kdiv = kdiv;
    } else {
      t.A = (PHASE == 1 ? sg.a : static_cast<const uint16_t*>(sg.act)) +
            static_cast<int64_t>(row0) * K;
      t.rmap = nullptr;
      t.kdiv = 1;
    }
    const uint16_t* W = static_cast<const uint16_t*>(seg_weights(wts, sg, PHASE, H, I, 2));
    int wlo, whi;  // first weight rows of this wavefront's two half groups of blocks
    if (PHASE == 1) {
      wlo = (nt * WN + wave) * (16 * HB);  // gate rows
      whi = I + wlo;                       // up rows of the same act columns
      t.out = static_cast<uint16_t*>(sg.act) + static_cast<int64_t>(row0) * I;
      t.col = nt * WN * 16 * HB + l16;
    } else {
      wlo = (nt * WN + wave) * (16 * NB);
      whi = wlo + 16 * HB;
      t.out = static_cast<uint16_t*>(sg.y) + static_cast<int64_t>(row0) * H;
      t.col = nt * WN * 16 * NB + l16;
    }
    t.ldo = ldo;
    t.bias = nullptr;
    // one row tile in the group: no other tile reads this tile's weight rows,
    // which are then loaded non-temporally (WNT)
    const bool wnt = sg.gmt == 1;
    t.wlo = W + static_cast<int64_t>(wlo) * K;
    t.whi = W + static_cast<int64_t>(whi) * K;
    // row blocks this wavefront computes: its row group's share of the tile
    const int rg = wave / (WN / RH);
    const int nmb = min(max((t.nrows + 15) / 16 - rg * (MBT / RH), 0), MBT / RH);
    if constexpr (kWide4) {
      const int nall = (t.nrows + 15) / 16;
      switch (nall) {
        case 1: tile512_nmb<PHASE, PACKED, 1>(t, wave, lane, look_ahead); break;
        case 2: tile512_nmb<PHASE, PACKED, 2>(t, wave, lane, look_ahead); break;
        case 3: tile512_nmb<PHASE, PACKED, 3>(t, wave, lane, look_ahead); break;
        case 4: tile512_nmb<PHASE, PACKED, 4>(t, wave, lane, look_ahead); break;
        case 5: tile512_nmb<PHASE, PACKED, 5>(t, wave, lane, look_ahead); break;
        case 6: tile512_nmb<PHASE, PACKED, 6>(t, wave, lane, look_ahead); break;
        case 7: tile512_nmb<PHASE, PACKED, 7>(t, wave, lane, look_ahead); break;
        default: tile512_nmb<PHASE, PACKED, 8>(t, wave, lane, look_ahead); break;
      }
    } else if constexpr (TM == kTM2) {
#define CLE_T2(RG_, N_) tile256_nmb<PHASE, PACKED, RG_, N_>(t, wave, lane, look_ahead)
      if (rg == 0) {
        switch (nmb) {
          case 1: CLE_T2(0, 1); break;
          case 2: CLE_T2(0, 2); break;
          case 3: CLE_T2(0, 3); break;
          case 4: CLE_T2(0, 4); break;
          case 5: CLE_T2(0, 5); break;
          case 6: CLE_T2(0, 6); break;
          case 7: CLE_T2(0, 7); break;
          default: CLE_T2(0, 8); break;
        }
      } else {
        switch (nmb) {
          case 0: CLE_T2(1, 0); break;
          case 1: CLE_T2(1, 1); break;
          case 2: CLE_T2(1, 2); break;
          case 3: CLE_T2(1, 3); break;
          case 4: CLE_T2(1, 4); break;
          case 5: CLE_T2(1, 5); break;
          case 6: CLE_T2(1, 6); break;
          case 7: CLE_T2(1, 7); break;
          default: CLE_T2(1, 8); break;
        }
      }
#undef CLE_T2
    } else if constexpr (RH == 2) {
#define CLE_T1(RG_, N_)                                                                        \
  {                                                                                            \
    if (TR >= 0 && wnt) /* (not in the any-K variant: its registers are tight) */           \
      tile_nmb<PHASE, WN, NB, PACKED, RH, RG_, N_, TR, PHASE, true>(t, wave, lane, look_ahead);  \
    else                                                                                       \
      tile_nmb<PHASE, WN, NB, PACKED, RH, RG_, N_, TR, PHASE, false>(t, wave, lane, look_ahead); \
  }
      if (rg == 0) {
        switch (nmb) {
          case 1: CLE_T1(0, 1); break;
          case 2: CLE_T1(0, 2); break;
          case 3: CLE_T1(0, 3); break;
          default: CLE_T1(0, 4); break;
        }
      } else {
        switch (nmb) {
          case 0: CLE_T1(1, 0); break;
          case 1: CLE_T1(1, 1); break;
          case 2: CLE_T1(1, 2); break;
          case 3: CLE_T1(1, 3); break;
          default: CLE_T1(1, 4); break;
        }
      }
#undef CLE_T1
    } else {
      switch (nmb) {
        case 1: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 1, TR>(t, wave, lane, look_ahead); break;
        case 2: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 2, TR>(t, wave, lane, look_ahead); break;
        case 3: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 3, TR>(t, wave, lane, look_ahead); break;
        case 4: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 4, TR>(t, wave, lane, look_ahead); break;
        case 5: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 5, TR>(t, wave, lane, look_ahead); break;
        case 6: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 6, TR>(t, wave, lane, look_ahead); break;
        case 7: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 7, TR>(t, wave, lane, look_ahead); break;
        default: tile_nmb<PHASE, WN, NB, PACKED, RH, 0, 8, TR>(t, wave, lane, look_ahead); break;
      }
    }
    // every wavefront is done reading the stages before the next tile's
    // first requests overwrite them
    stage_barrier();
    if constexpr (kWide4) {
      // wavefront 0 leaves the next tile in the last stage buffer; every
      // wavefront has read it before the next tile requests a stage there
      uint4* hand = &g_sw3<PHASE, PACKED>.x[0][0];
      if (wave == 0 && lane == 0)
        *hand = make_uint4(static_cast<unsigned>(tnext), static_cast<unsigned>(next.si),
                           static_cast<unsigned>(next.nt), static_cast<unsigned>(next.mi));
      stage_barrier();
      if (wave != 0) {
        const uint4 v = *hand;
        tnext = __builtin_amdgcn_readfirstlane(static_cast<int>(v.x));
        next = TilePos{__builtin_amdgcn_readfirstlane(static_cast<int>(v.y)),
                       __builtin_amdgcn_readfirstlane(static_cast<int>(v.z)),
                       __builtin_amdgcn_readfirstlane(static_cast<int>(v.w))};
      }
      stage_barrier();
    } else if (wave != 0) {
      tnext = s_next[par][0];
      next = TilePos{s_next[par][1], s_next[par][2], s_next[par][3]};
    }
    tile = tnext;
  }
}

// ---------------------------------------------------------------- fused thin segments
// Gate/up and down of one thin segment (1 .. 16 rows) in one workgroup, in
// one launch: the six gate/up column tiles, then the eight down column tiles
// read the segment's Act rows this workgroup has just written (still in its
// L2), with no launch boundary between the phases.  Segments are taken from
// the table through a counter; the segment's tiles and K order are those of
// the two-phase kernels, so its outputs are bitwise the same.  Built for the
// K-loop tails of H = 2048 and I = 768 (4 and 2 steps).
template <bool PACKED, int TR1, int TR2>
__global__ __launch_bounds__(512, 1) void ffn_fused_thin(const Seg* __restrict__ segs, int nseg,
                                                        int* __restrict__ counter, Weights wts,
                                                        int H, int I) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int l16 = lane % 16;
  const int rg = wave / 4;  // row group of the 2 x 4 compute layout
  __shared__ int s_pick;
  for (;;) {
    if (threadIdx.x == 0) {
      gint* cp = (gint*)counter;
      asm volatile("" : "+v"(cp));
      s_pick = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int si = __builtin_amdgcn_readfirstlane(s_pick);
    __syncthreads();
    if (si >= nseg) break;
    if (!segs[si].fused) continue;
    const Seg sg = segs[si];
    int32_t kw;
    __builtin_memcpy(&kw, &segs[si].kdiv, sizeof(kw));
    const int kdiv = static_cast<int16_t>(kw & 0xffff), kkey = (kw >> 16) & 0xffff;
    TileArgs t;
    t.nrows = sg.rows;
    t.bias = nullptr;
    // gate/up: 128 act columns per column tile
    {
      const uint16_t* W = static_cast<const uint16_t*>(seg_weights(wts, sg, 1, H, I, 2));
      t.K = H;
      t.rot = kkey % (H / kKS);
      t.A = sg.a;
      t.rmap = sg.rmap;
      t.kdiv = sg.rmap ? kdiv : 1;
      t.out = static_cast<uint16_t*>(sg.act);
      int ldo = I;
      asm volatile("" : "+s"(ldo));
      t.ldo = ldo;
      for (int nt = 0; nt < I / 128; ++nt) {
        const int wlo = (nt * 8 + wave) * 16;
        t.wlo = W + static_cast<int64_t>(wlo) * H;
        t.whi = W + static_cast<int64_t>(I + wlo) * H;
        t.col = nt * 128 + l16;
        if (rg == 0)
          tile_nmb<1, 8, 2, PACKED, 2, 0, 1, TR1>(t, wave, lane);
        else
          tile_nmb<1, 8, 2, PACKED, 2, 1, 0, TR1>(t, wave, lane);
        stage_barrier();
      }
    }
    // every wavefront's Act stores have completed before any wavefront's
    // down loads read them, and the CU's L1 holds no older copy of those rows
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // down: 256 output columns per column tile
    {
      const uint16_t* W = static_cast<const uint16_t*>(seg_weights(wts, sg, 2, H, I, 2));
      t.K = I;
      t.rot = kkey % (I / kKS);
      t.A = static_cast<const uint16_t*>(sg.act);
      t.rmap = nullptr;
      t.kdiv = 1;
      t.out = static_cast<uint16_t*>(sg.y);
      int ldo = H;
      asm volatile("" : "+s"(ldo));
      t.ldo = ldo;
      for (int nt = 0; nt < H / 256; ++nt) {
        const int wlo = (nt * 8 + wave) * 32;
        t.wlo = W + static_cast<int64_t>(wlo) * I;
        t.whi = W + static_cast<int64_t>(wlo + 16) * I;
        t.col = nt * 256 + l16;
        if (rg == 0)
          tile_nmb<2, 8, 2, PACKED, 2, 0, 1, TR2, 1>(t, wave, lane);
        else
          tile_nmb<2, 8, 2, PACKED, 2, 1, 0, TR2, 1>(t, wave, lane);
        stage_barrier();
      }
    }
  }
}

// ---------------------------------------------------------------- f32 tiles (exact-order reference path)
template <int PHASE>
__global__ __launch_bounds__(256) void ffn_gemm_f32(const Seg* __restrict__ segs, int nseg,
                                                    const int* __restrict__ totals,
                                                    int* __restrict__ /*claims: unused*/,
                                                    Weights wts, int H, int I) {
  const int total = totals[PHASE - 1];
  const int grid = gridDim.x;
  const int K = PHASE == 1 ? H : I;
  for (int tile = logical_tile_base(grid); tile < total; tile += grid) {
    const TilePos tp = locate_tile(segs, nseg, tile, (PHASE == 1 ? I : H) / kBNF, kBM);
    const Seg sg = segs[tp.si];
    const int nt = tp.nt, mi = tp.mi;
    const float* A = static_cast<const float*>(PHASE == 1 ? static_cast<const void*>(sg.a) : sg.act);
    const float* W = static_cast<const float*>(seg_weights(wts, sg, PHASE, H, I, 4));
    for (int e = threadIdx.x; e < kBM * 64; e += blockDim.x) {
      const int row = mi * kBM + e / 64;
      const int col = nt * 64 + e % 64;
      if (row >= sg.rows) continue;
      const float* a =
          (PHASE == 1 && sg.rmap)
              ? static_cast<const float*>(static_cast<const void*>(sg.a)) +
                    static_cast<int64_t>(sg.rmap[row] / sg.kdiv) * K
              : A + static_cast<int64_t>(row) * K;
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

// ---------------------------------------------------------------- router gate
// Router logits z = x W_g^T + b of several micro-batches in one launch
// ("EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §2.1: the routing scores G(h') that top-k selects from).  bf16: the tile
// engine above as phase 3 (fp32 accumulation and output), one 32-row x
// (16 * WN * NB)-expert tile per workgroup, K = H in the same fixed order for
// every tile.  With a loop state, only micro-batches in its todo mask run,
// each with the weights and bias of its layer l_j.
constexpr int kGateRows = 32;

struct GateArgs {
  const uint16_t* x[CLE_MAX_MICROBATCHES];  // [T, H] (float for the f32 path)
  const uint16_t* wg[CLE_MAX_MICROBATCHES];  // [E, H], or with a loop state the base [L, E, H]
  const float* bias[CLE_MAX_MICROBATCHES];   // [E] / [L, E], or NULL
  float* out[CLE_MAX_MICROBATCHES];          // [T, E]
  const cle_loop_state* st;
};

__device__ __forceinline__ bool gate_member(const GateArgs& a, int j, const uint16_t*& wg,
                                            const float*& bias, int64_t wstride, int E) {
  wg = a.wg[j];
  bias = a.bias[j];
  if (a.st) {
    if (!(a.st->todo >> j & 1)) return false;
    const int l = a.st->layer[j];
    wg += static_cast<int64_t>(l) * wstride;
    if (bias) bias += static_cast<int64_t>(l) * E;
  }
  return true;
}

template <int WN, int NB, bool PACKED>
__global__ __launch_bounds__(64 * WN, 1) void gate_gemm_bf16(GateArgs a, int T, int H, int E) {
  constexpr int HB = NB / 2;
  const int j = blockIdx.y;
  const uint16_t* wg;
  const float* bias;
  if (!gate_member(a, j, wg, bias, static_cast<int64_t>(E) * H, E)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int ncols = E / (WN * 16 * NB);
  const int mt = blockIdx.x / ncols, nt = blockIdx.x % ncols;
  const int row0 = mt * kGateRows;
  TileArgs t;
  t.K = H;
  t.rot = 0;
  t.nrows = min(kGateRows, T - row0);
  t.A = a.x[j] + static_cast<int64_t>(row0) * H;
  t.rmap = nullptr;
  t.kdiv = 1;
  const int wlo = (nt * WN + wave) * (16 * NB);
  t.out = reinterpret_cast<uint16_t*>(a.out[j] + static_cast<int64_t>(row0) * E);
  t.ldo = E;
  t.col = nt * WN * 16 * NB + lane % 16;
  t.bias = bias;
  t.wlo = wg + static_cast<int64_t>(wlo) * H;
  t.whi = wg + static_cast<int64_t>(wlo + 16 * HB) * H;
  if (t.nrows > 16)
    tile_nmb<3, WN, NB, PACKED, 1, 0, 2, -1>(t, wave, lane);
  else
    tile_nmb<3, WN, NB, PACKED, 1, 0, 1, -1>(t, wave, lane);
}

// f32: one thread per logit, sequential K (the small fp32 shapes).
__global__ __launch_bounds__(256) void gate_f32(GateArgs a, int T, int H, int E) {
  const int j = blockIdx.y;
  const uint16_t* wg16;
  const float* bias;
  if (!gate_member(a, j, wg16, bias, static_cast<int64_t>(E) * H * 2, E)) return;
  const float* x = reinterpret_cast<const float*>(a.x[j]);
  const float* wg = reinterpret_cast<const float*>(wg16);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < static_cast<int64_t>(T) * E; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / E;
    const int e = static_cast<int>(i % E);
    float z = 0.f;
    for (int h = 0; h < H; ++h) z = fmaf(x[t * H + h], wg[static_cast<int64_t>(e) * H + h], z);
    a.out[j][i] = bias ? z + bias[e] : z;
  }
}

// Workgroups that fit on the device at once for `kernel` (cached per device).
template <typename Kernel>
int resident_blocks(Kernel kernel, int* cache, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  cache[dev] = per_cu * device_cu_count();
  return cache[dev];
}

// Tile of the 8-wavefront bf16 kernels (cle_set_expert_tile): an explicit
// choice, else the environment's CLE_TILE read once, else 128 x 256.
enum WideTile { kTile128x256 = CLE_TILE_128X256, kTile256x256 = CLE_TILE_256X256,
                kTile128x512 = CLE_TILE_128X512 };
int g_tile_choice = CLE_TILE_DEFAULT;

// The tile of a launch whose descriptors hold `rows` rows in all over
// n_desc x E experts: an explicit choice, else the environment's CLE_TILE
// read once, else 256 x 256 when the segments average at least 512 rows (the
// long-prefill shapes: each weight block is read by half as many tiles; 2-3 %
// faster there, measured) and 128 x 256 otherwise (thin segments would leave
// most of a 256-row tile empty).
WideTile wide_tile_shape(int64_t rows, int n_desc, int E) {
  static const int env = [] {
    const char* v = getenv("CLE_TILE");
    if (v && !strcmp(v, "128x256")) return static_cast<int>(kTile128x256);
    if (v && !strcmp(v, "256x256")) return static_cast<int>(kTile256x256);
    if (v && !strcmp(v, "128x512")) return static_cast<int>(kTile128x512);
    return 0;
  }();
  const int c = g_tile_choice != CLE_TILE_DEFAULT ? g_tile_choice : env;
  if (c != 0) return static_cast<WideTile>(c);
  return rows >= static_cast<int64_t>(512) * n_desc * E ? kTile256x256 : kTile128x256;
}

// Fused thin-segment launch (cle_set_fused_thin_rows): routed segments of 1
// .. r rows go to ffn_fused_thin; an explicit choice, else the environment's
// CLE_FUSE_THIN read once, else off.
int g_fuse_choice = -1;

int fuse_thin_rows() {
  static const int env = [] {
    const char* v = getenv("CLE_FUSE_THIN");
    const int r = v ? atoi(v) : 0;
    return r < 0 ? 0 : (r > 16 ? 16 : r);
  }();
  return g_fuse_choice >= 0 ? g_fuse_choice : env;
}

int persistent_grid(int64_t upper_bound_tiles, int resident) {
  int64_t g = resident;
  if (upper_bound_tiles < g) g = upper_bound_tiles;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return static_cast<int>(g);
}

}  // namespace
}  // namespace cle

// ---------------------------------------------------------------- no-allocation variant
// cle_grouped_expert_ffn_noalloc keeps its workspace (tile totals, per-XCD
// claims, segment table, row-tile prefix) in this file-scope array: one copy
// per GPU, held until the process ends.  Host code never takes the array's
// name as an address: the device address is looked up once per device with
// hipGetSymbolAddress and used from then on.
namespace cle {
namespace {
constexpr size_t kNoAllocScratchBytes = CLE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device, set on the first call there

cle_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return CLE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CLE_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CLE_OK;
}
}  // namespace
}  // namespace cle

extern "C" cle_status cle_grouped_expert_ffn_noalloc(
    const cle_ffn_desc* d, int32_t n_desc, const void* w13, const void* w2,
    const void* w13_shared, const void* w2_shared, int32_t L, int32_t E, int32_t n_shared,
    int32_t H, int32_t I, cle_dtype dt, int32_t w_layout, void* const* phase_events,
    void* stream) {
  // the sizes are checked before the scratch is touched; grouped_ffn checks
  // every other argument
  if (!d || n_desc < 1 || n_desc > CLE_MAX_DESC || E < 1 || E > CLE_MAX_E || n_shared < 0)
    return CLE_EINVAL;
  if (cle_workspace_bytes(CLE_OP_FFN, 0, E, 1, n_shared, n_desc) > cle::kNoAllocScratchBytes)
    return CLE_EUNSUPPORTED;
  void* ws = nullptr;
  const cle_status st = cle::noalloc_scratch(&ws);
  if (st != CLE_OK) return st;
  return cle::grouped_ffn(d, n_desc, w13, w2, w13_shared, w2_shared, L, E, n_shared, H, I, dt,
                          w_layout, ws, cle::kNoAllocScratchBytes, phase_events, nullptr, true,
                          stream);
}

extern "C" cle_status cle_set_fused_thin_rows(int32_t rows) {
  if (rows < -1 || rows > 16) return CLE_EINVAL;
  cle::g_fuse_choice = rows;
  return CLE_OK;
}

extern "C" cle_status cle_set_expert_tile(int32_t tile) {
  if (tile < CLE_TILE_DEFAULT || tile > CLE_TILE_128X512) return CLE_EINVAL;
  cle::g_tile_choice = tile;
  return CLE_OK;
}

extern "C" cle_status cle_grouped_expert_ffn(const cle_ffn_desc* d, int32_t n_desc,
                                             const void* w13, const void* w2,
                                             const void* w13_shared, const void* w2_shared,
                                             int32_t L, int32_t E, int32_t n_shared, int32_t H,
                                             int32_t I, cle_dtype dt, int32_t w_layout, void* ws,
                                             size_t ws_bytes, void* const* phase_events,
                                             void* stream) {
  return cle::grouped_ffn(d, n_desc, w13, w2, w13_shared, w2_shared, L, E, n_shared, H, I, dt,
                          w_layout, ws, ws_bytes, phase_events, nullptr, true, stream);
}

namespace cle {

cle_status grouped_ffn(const cle_ffn_desc* d, int32_t n_desc, const void* w13, const void* w2,
                       const void* w13_shared, const void* w2_shared, int32_t L, int32_t E,
                       int32_t n_shared, int32_t H, int32_t I, cle_dtype dt, int32_t w_layout,
                       void* ws, size_t ws_bytes, void* const* phase_events,
                       const cle_loop_state* st, bool launch, void* stream) {
  if (!d || n_desc < 1 || n_desc > CLE_MAX_DESC) return CLE_EINVAL;
  if (!w13 || !w2 || L < 1 || E < 1 || E > CLE_MAX_E || n_shared < 0) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  if (w_layout != CLE_W_ROWMAJOR && !(w_layout == CLE_W_PACKED && dt == CLE_BF16))
    return CLE_EINVAL;
  const bool packed = w_layout == CLE_W_PACKED;
  // bf16: 128-row tiles of 16 weight blocks (8 wavefronts x 2; 128 act
  // columns, 256 output columns) when the shape allows it, else of 8 blocks
  // (4 wavefronts x 2).  f32: 64 x 64 tiles.
  if (I < 64 || I % 64) return CLE_EINVAL;
  if (dt == CLE_BF16 ? (H < 128 || H % 128) : (H < 64 || H % 64)) return CLE_EINVAL;
  const bool wide = dt == CLE_BF16 && I % 128 == 0 && H % 256 == 0;
  int64_t all_rows = 0;
  for (int j = 0; j < n_desc; ++j) all_rows += d[j].rows > 0 ? d[j].rows : 0;
  const WideTile shape = wide_tile_shape(all_rows, n_desc, E);
  const bool tall = wide && shape == kTile256x256;
  // the fused thin-segment launch: 128 x 256 tiles with the K-loop tails of
  // H = 2048 and I = 768 (K / 64 = 32 and 12)
  const auto tail_of = [](int K) { return 2 + (K / kKS - 3) % 3; };
  const bool wide4 = wide && shape == kTile128x512 && I % 256 == 0 && H % 512 == 0;
  const int tm = dt == CLE_BF16 ? (tall ? kTM2 : kTM) : kBM;
  const int thin = wide && !tall && !wide4 && H / kKS >= 3 && I / kKS >= 3 &&
                           tail_of(H) == 4 && tail_of(I) == 2 ? fuse_thin_rows() : 0;
  const int tn1 = dt == CLE_BF16 ? (wide4 ? 256 : wide ? 128 : 64) : kBNF;
  const int tn2 = dt == CLE_BF16 ? (wide4 ? 512 : wide ? 256 : 128) : kBNF;
  if (n_shared > 0 && (!w13_shared || !w2_shared)) return CLE_EINVAL;
  const int esz = dt == CLE_BF16 ? 2 : 4;
  if (!aligned(w13, 16) || !aligned(w2, 16)) return CLE_EINVAL;
  int64_t ub1 = 0, ub2 = 0;
  for (int j = 0; j < n_desc; ++j) {
    const cle_ffn_desc& q = d[j];
    if (q.layer < 0 || q.layer >= L || q.rows < 0 || !q.offsets) return CLE_EINVAL;
    if (q.rows > 0 && (!q.act || !q.yp)) return CLE_EINVAL;
    if (q.rows > 0 && !q.xp && (!q.x || !q.src || q.k < 1)) return CLE_EINVAL;
    if (!aligned(q.xp, 16) || !aligned(q.x, 16) || !aligned(q.act, 16) || !aligned(q.yp, 16))
      return CLE_EINVAL;
    if (n_shared > 0) {
      if (q.shared_rows < 0) return CLE_EINVAL;
      if (q.shared_rows > 0 && (!q.x_shared || !q.act_shared || !q.y_shared)) return CLE_EINVAL;
      if (!aligned(q.x_shared, 16) || !aligned(q.act_shared, 16) || !aligned(q.y_shared, 16))
        return CLE_EINVAL;
    }
    // sum over experts of ceil(c_e / BM) <= rows / BM + (non-empty experts)
    const int64_t mt = q.rows / tm + (q.rows < E ? q.rows : E);
    const int64_t mts =
        n_shared > 0 ? static_cast<int64_t>(n_shared) * ((q.shared_rows + tm - 1) / tm) : 0;
    ub1 += (mt + mts) * (I / tn1);
    ub2 += (mt + mts) * (H / tn2);
  }
  if (ub1 > INT32_MAX || ub2 > INT32_MAX) return CLE_EUNSUPPORTED;
  const size_t need = cle_workspace_bytes(CLE_OP_FFN, 0, E, 1, n_shared, n_desc);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return CLE_EWORKSPACE;
  if (!launch) return CLE_OK;

  hipStream_t s = as_stream(stream);
  int* totals = static_cast<int*>(ws);
  int* claims1 = totals + kClaimsOffset;  // per-XCD tile claims of each phase
  int* claims2 = claims1 + kXcds;
  Seg* segs = reinterpret_cast<Seg*>(static_cast<char*>(ws) + kFfnHeader);
  const int nseg = n_desc * (E + n_shared);
  int* mscan = reinterpret_cast<int*>(segs + nseg);
  for (int c = 0; c < n_desc; c += kPlanDescs) {
    PlanArgs p;
    p.nd = n_desc - c < kPlanDescs ? n_desc - c : kPlanDescs;
    for (int j = 0; j < p.nd; ++j) {
      const cle_ffn_desc& q = d[c + j];
      p.d[j] = DescDev{q.layer, q.rows, q.offsets, q.xp, q.act, q.yp,
                       n_shared > 0 ? q.shared_rows : 0, q.x_shared, q.act_shared, q.y_shared,
                       q.x, q.src, q.k};
    }
    for (int j = 0; j < CLE_MAX_DESC; ++j) p.layer_all[j] = j < n_desc ? d[j].layer : 0;
    p.c0 = c;
    p.n_all = n_desc;
    p.E = E;
    p.ns = n_shared;
    p.H = H;
    p.I = I;
    p.esz = esz;
    p.L = L;
    p.st = st;
    p.order = c + kPlanDescs >= n_desc;
    p.nseg = nseg;
    p.tm = tm;
    p.n1 = I / tn1;
    p.n2 = H / tn2;
    p.thin = thin;
    p.totals = totals;
    p.mscan = mscan;
    ffn_plan<<<dim3(1), dim3(1024), 0, s>>>(p, segs);
  }
  const Weights wts{w13, w2, w13_shared, w2_shared};
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (phase_events)
    for (int q = 0; q < 4; ++q) ev[q] = static_cast<hipEvent_t>(phase_events[q]);
  // One persistent launch of `kernel` over `ub` tiles at most; the events (if
  // any) are taken by the launch itself, so timing adds no marker between
  // kernels.  A phase without tiles records its event pair back to back.
  auto run_phase = [&](auto kernel, int* occ, int threads, int64_t ub, hipEvent_t e0,
                       hipEvent_t e1, int* claims) -> bool {
    if (ub > 0) {
      const int g = persistent_grid(ub, resident_blocks(kernel, occ, threads));
      hipExtLaunchKernelGGL(kernel, dim3(g), dim3(threads), 0, s, e0, e1, 0,
                            static_cast<const Seg*>(segs), nseg,
                            static_cast<const int*>(totals), claims, wts, H, I);
      return true;
    }
    // no tiles: the events this phase was given are recorded back to back
    bool rec = true;
    if (e0) rec = rec && hipEventRecord(e0, s) == hipSuccess;
    if (e1) rec = rec && hipEventRecord(e1, s) == hipSuccess;
    return rec;
  };
  // The 8-wavefront bf16 kernel of a phase, with the K-loop tail its K needs.
  auto run_wide = [&](auto phase, auto pk, int K, int64_t ub, hipEvent_t e0, hipEvent_t e1,
                      int* claims) {
    constexpr int P = decltype(phase)::value;
    constexpr bool PK = decltype(pk)::value;
    static int occ_t2[64], occ_t3[64], occ_t4[64], occ_any[64], occ_256[64];
    static int occ_512[64];
    if (tall) return run_phase(ffn_gemm_bf16<P, 8, 2, PK, 0, kTM2>, occ_256, 512, ub, e0, e1, claims);
    if (wide4) return run_phase(ffn_gemm_bf16<P, 8, 4, PK, 0>, occ_512, 512, ub, e0, e1, claims);
    const int kt = K / kKS;
    switch (kt >= 3 ? 2 + (kt - 3) % 3 : -1) {
      case 2: return run_phase(ffn_gemm_bf16<P, 8, 2, PK, 2>, occ_t2, 512, ub, e0, e1, claims);
      case 3: return run_phase(ffn_gemm_bf16<P, 8, 2, PK, 3>, occ_t3, 512, ub, e0, e1, claims);
      case 4: return run_phase(ffn_gemm_bf16<P, 8, 2, PK, 4>, occ_t4, 512, ub, e0, e1, claims);
      default: return run_phase(ffn_gemm_bf16<P, 8, 2, PK, -1>, occ_any, 512, ub, e0, e1, claims);
    }
  };
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using PKT = std::true_type;
  using PKF = std::false_type;
  static int occ_c1[64], occ_c2[64], occ_f1[64], occ_f2[64], occ_c1p[64], occ_c2p[64];
  bool ok;
  if (thin > 0) {
    // the fused thin segments first (the gate/up events bracket both launches)
    static int occ_ft[64], occ_ff[64];
    int* counter = totals + kFusedCounter;
    if (packed)
      hipExtLaunchKernelGGL(ffn_fused_thin<true, 4, 2>, dim3(resident_blocks(
                                ffn_fused_thin<true, 4, 2>, occ_ft, 512)),
                            dim3(512), 0, s, ev[0], nullptr, 0, static_cast<const Seg*>(segs),
                            nseg, counter, wts, H, I);
    else
      hipExtLaunchKernelGGL(ffn_fused_thin<false, 4, 2>, dim3(resident_blocks(
                                ffn_fused_thin<false, 4, 2>, occ_ff, 512)),
                            dim3(512), 0, s, ev[0], nullptr, 0, static_cast<const Seg*>(segs),
                            nseg, counter, wts, H, I);
    ev[0] = nullptr;
  }
  if (wide)
    ok = packed ? run_wide(P1(), PKT(), H, ub1, ev[0], ev[1], claims1)
                : run_wide(P1(), PKF(), H, ub1, ev[0], ev[1], claims1);
  else if (dt == CLE_BF16)
    ok = packed ? run_phase(ffn_gemm_bf16<1, 4, 2, true, -1>, occ_c1p, 256, ub1, ev[0], ev[1], claims1)
                : run_phase(ffn_gemm_bf16<1, 4, 2, false, -1>, occ_c1, 256, ub1, ev[0], ev[1], claims1);
  else
    ok = run_phase(ffn_gemm_f32<1>, occ_f1, 256, ub1, ev[0], ev[1], claims1);
  if (!ok) return CLE_EHIP;
  if (wide)
    ok = packed ? run_wide(P2(), PKT(), I, ub2, ev[2], ev[3], claims2)
                : run_wide(P2(), PKF(), I, ub2, ev[2], ev[3], claims2);
  else if (dt == CLE_BF16)
    ok = packed ? run_phase(ffn_gemm_bf16<2, 4, 2, true, -1>, occ_c2p, 256, ub2, ev[2], ev[3], claims2)
                : run_phase(ffn_gemm_bf16<2, 4, 2, false, -1>, occ_c2, 256, ub2, ev[2], ev[3], claims2);
  else
    ok = run_phase(ffn_gemm_f32<2>, occ_f2, 256, ub2, ev[2], ev[3], claims2);
  if (!ok) return CLE_EHIP;
  return launch_status();
}

}  // namespace cle

namespace cle {

cle_status launch_gate(int n, const void* const* x, const void* const* wg,
                       const float* const* bias, int T, int H, int E, cle_dtype dt, bool packed,
                       float* const* logits, const cle_loop_state* st, hipStream_t s) {
  if (T == 0) return CLE_OK;
  GateArgs a;
  for (int j = 0; j < n; ++j) {
    a.x[j] = static_cast<const uint16_t*>(x[j]);
    a.wg[j] = static_cast<const uint16_t*>(wg[j]);
    a.bias[j] = bias ? bias[j] : nullptr;
    a.out[j] = logits[j];
  }
  a.st = st;
  if (dt == CLE_F32) {
    const int64_t blocks = (static_cast<int64_t>(T) * E + 255) / 256;
    gate_f32<<<dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096), n), dim3(256), 0, s>>>(
        a, T, H, E);
    return launch_status();
  }
  const unsigned mts = static_cast<unsigned>((T + kGateRows - 1) / kGateRows);
  if (E % 128 == 0) {
    const dim3 grid(mts * (E / 128), n);
    if (packed)
      gate_gemm_bf16<4, 2, true><<<grid, dim3(256), 0, s>>>(a, T, H, E);
    else
      gate_gemm_bf16<4, 2, false><<<grid, dim3(256), 0, s>>>(a, T, H, E);
  } else {
    const dim3 grid(mts * (E / 64), n);
    if (packed)
      gate_gemm_bf16<2, 2, true><<<grid, dim3(128), 0, s>>>(a, T, H, E);
    else
      gate_gemm_bf16<2, 2, false><<<grid, dim3(128), 0, s>>>(a, T, H, E);
  }
  return launch_status();
}

cle_status check_gate(int T, int H, int E, cle_dtype dt, int32_t w_layout) {
  if (T < 0 || H < 1 || E < 1 || E > CLE_MAX_E) return CLE_EINVAL;
  if (dt != CLE_BF16 && dt != CLE_F32) return CLE_EINVAL;
  if (w_layout != CLE_W_ROWMAJOR && !(w_layout == CLE_W_PACKED && dt == CLE_BF16))
    return CLE_EINVAL;
  if (dt == CLE_BF16 && (H % 128 || E % 64)) return CLE_EINVAL;
  return CLE_OK;
}

}  // namespace cle

extern "C" cle_status cle_gate_logits_many(int32_t n, const void* const* x,
                                           const void* const* w_gate,
                                           const float* const* bias, int32_t T, int32_t H,
                                           int32_t E, cle_dtype dt, int32_t w_layout,
                                           float* const* logits, void* stream) {
  using namespace cle;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || !x || !w_gate || !logits) return CLE_EINVAL;
  const cle_status c = check_gate(T, H, E, dt, w_layout);
  if (c != CLE_OK) return c;
  for (int j = 0; j < n; ++j) {
    if (!x[j] || !w_gate[j] || !logits[j]) return CLE_EINVAL;
    if (!aligned(x[j], 16) || !aligned(w_gate[j], 16) || !aligned(logits[j], 4)) return CLE_EINVAL;
  }
  return launch_gate(n, x, w_gate, bias, T, H, E, dt, w_layout == CLE_W_PACKED, logits, nullptr,
                     as_stream(stream));
}
