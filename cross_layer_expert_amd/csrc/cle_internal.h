// Internal helpers shared by the libcle translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cle.h"

namespace cle {

constexpr int kWave = 64;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Launch-status helper: any error left by the launches maps to CLE_EHIP.
inline cle_status launch_status() {
  return hipGetLastError() == hipSuccess ? CLE_OK : CLE_EHIP;
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Launchers behind the batched entry points, for callers that validated
// their arguments already.  `st` (may be NULL) restricts a launch to the
// micro-batches of the loop state's todo (route, dispatch) or runset
// (combine, expert FFN) mask; the kernels read the mask on the device.
// With norm_x, the same launch also writes norm_y[j] = rmsnorm(norm_x[j]) (rows
// of H elements of norm_dt; the rows of cle_rmsnorm_many, bit for bit).
cle_status launch_route(int n, const float* const* logits, int T, int E, int k, int* const* idx,
                        float* const* gate, const cle_loop_state* st, int64_t layer_stride,
                        hipStream_t s, const void* const* norm_x = nullptr,
                        void* const* norm_y = nullptr, int H = 0, float eps = 0.0f,
                        cle_dtype norm_dt = CLE_BF16);
cle_status launch_dispatch_many(int n, const int* const* idx, int T, int k, int E,
                                int* const* counts, int* const* offsets, int* const* dest,
                                int* const* src, void* ws, const cle_loop_state* st,
                                hipStream_t s);
cle_status launch_combine_many(int n, const void* const* yp, const int* const* dest,
                               const float* const* gate, int T, int k, int H,
                               const void* const* y_shared, int n_shared,
                               const void* const* residual, void* const* y, cle_dtype dt,
                               const cle_loop_state* st, hipStream_t s,
                               const void* const* h0 = nullptr);
// Row RMS normalisation of cle_rmsnorm_many (todo micro-batches only with a state).
cle_status launch_rmsnorm(int n, const void* const* x, void* const* y, int T, int H, float eps,
                          cle_dtype dt, const cle_loop_state* st, hipStream_t s);
// Router logits of cle_gate_logits_many (validated by check_gate); with a
// loop state, w_gate / bias entries are the bases [L, E, H] / [L, E].
cle_status launch_gate(int n, const void* const* x, const void* const* w_gate,
                       const float* const* bias, int T, int H, int E, cle_dtype dt, bool packed,
                       float* const* logits, const cle_loop_state* st, hipStream_t s);
cle_status check_gate(int T, int H, int E, cle_dtype dt, int32_t w_layout);
// cle_grouped_expert_ffn with an optional loop state; launch = false only
// validates the arguments.
cle_status grouped_ffn(const cle_ffn_desc* d, int32_t n_desc, const void* w13, const void* w2,
                       const void* w13_shared, const void* w2_shared, int32_t L, int32_t E,
                       int32_t n_shared, int32_t H, int32_t I, cle_dtype dt, int32_t w_layout,
                       void* ws, size_t ws_bytes, void* const* phase_events,
                       const cle_loop_state* st, bool launch, void* stream);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- bf16
// IEEE bfloat16 held as its 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- workspace layout
// Dispatch workspace: per-chunk per-expert counts, then bases.
constexpr int kDispatchChunk = 1024;  // assignments per histogram block

inline int64_t dispatch_chunks(int64_t A) { return (A + kDispatchChunk - 1) / kDispatchChunk; }

// FFN workspace: segment table + totals.
// One (micro-batch, expert) segment of a grouped expert launch.  Segments
// are stored grouped by (layer, expert): the segments of the micro-batches at
// the same layer using the same expert sit next to each other, ordered by
// micro-batch, and a group's tiles are ordered by column tile (or by blocks
// of a few column tiles), then by the group's row tiles, so the tiles that
// read one block of weight rows run close together (on one XCD) whichever
// micro-batch their rows come from.
struct Seg {
  const uint16_t* a;    // phase-1 A rows (bf16 or f32 storage; byte pointer semantics by dtype)
  void* act;            // phase-1 output / phase-2 A rows
  void* y;              // phase-2 output rows
  const int32_t* rmap;  // NULL: A row r is a + r*H; else token rmap[r] / kdiv of a
  int32_t widx;         // weights: layer * E + e, or -1 - (layer * n_shared + q) (shared q)
  int32_t rows;
  int32_t m0;           // row tiles of all groups before this segment's group
  int32_t gmt;          // row tiles of this segment's group
  int32_t moff;         // row tiles of the group's segments before this one
  int16_t kdiv;
  uint16_t kkey;        // K-order key of the segment's weights (a function of
                        // layer and expert only)
  int16_t grank;        // position of the segment in its group
  int16_t gsize;        // segments in the group
  int32_t fused;        // 1: run by the fused thin-segment launch, no tiles in the two phases
};
// (kdiv/kkey and grank/gsize are read in pairs as 32-bit words, low half first)
static_assert(sizeof(Seg) == 64 && offsetof(Seg, kdiv) % 4 == 0 &&
                  offsetof(Seg, kkey) == offsetof(Seg, kdiv) + 2 &&
                  offsetof(Seg, grank) % 4 == 0 && offsetof(Seg, gsize) == offsetof(Seg, grank) + 2,
              "Seg layout");

constexpr size_t kFfnHeader = 256;  // totals live in the first 256 bytes

}  // namespace cle
