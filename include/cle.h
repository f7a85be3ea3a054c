/*
 * cle.h -- C ABI of libcle.so, the cross-layer MoE expert step for AMD
 * Instinct MI355X (gfx950).
 *
 * The step is the hot path of EasyBalance ("EasyBalance: Cross-Layer Load
 * Balancing in Distributed MoE Inference", arXiv 2608.07964v1): route the
 * tokens of several micro-batches, dispatch them to expert-grouped buffers,
 * measure the per-device-group workload, pick which micro-batches run now
 * (Algorithm 1, Schedule(S, m)), run one grouped SwiGLU expert launch that
 * covers micro-batches sitting at different layers, and combine the expert
 * outputs with the routing weights (Eq. (1)).
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    never allocates device memory; scratch comes from a caller workspace
 *    sized by cle_workspace_bytes(), except in
 *    cle_grouped_expert_ffn_noalloc, whose scratch is a fixed array in the
 *    library's device code (one per GPU, for the life of the process).
 *  - Pointers are device pointers unless marked HOST.
 *  - Tensors are dense row-major.  bf16 tensors hold IEEE bfloat16 bit
 *    patterns; gates are float32; indices are int32.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every entry point
 *    except cle_schedule_step, cle_workspace_bytes and cle_status_string only
 *    enqueues work on that stream and returns without waiting.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued; on error nothing is written and a negative status returns.
 *    Device-side contents (expert ids) cannot be validated on the host; the
 *    kernels stay in bounds whatever they hold (see cle_dispatch).
 *  - Determinism: every output is bitwise reproducible and independent of how
 *    micro-batches are grouped into one cle_grouped_expert_ffn call.  No
 *    floating-point atomics are used.
 */
#ifndef CLE_H
#define CLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cle_status;
#define CLE_OK 0
#define CLE_EINVAL (-1)        /* bad argument (shape, size, null pointer, enum) */
#define CLE_EHIP (-2)          /* a HIP runtime call failed */
#define CLE_EWORKSPACE (-3)    /* workspace missing or too small */
#define CLE_EUNSUPPORTED (-4)  /* valid but beyond this build's limits */

typedef enum { CLE_BF16 = 0, CLE_F32 = 1 } cle_dtype;

/* RunSet policies.  B0 and B1 are baselines; the others are the three
 * heuristics of the paper, §5.2. */
typedef enum {
  CLE_POLICY_B0_ALONE = 0,     /* one micro-batch per step: no cross-layer combination */
  CLE_POLICY_B1_LOCKSTEP = 1,  /* every ready micro-batch */
  CLE_POLICY_CUMUTIL = 2,
  CLE_POLICY_MAXUTIL = 3,
  CLE_POLICY_DIFFPEAK = 4
} cle_policy;

/* Layout of the expert weight tensors given to cle_grouped_expert_ffn. */
typedef enum {
  CLE_W_ROWMAJOR = 0, /* each [rows, K] matrix row-major */
  CLE_W_PACKED = 1    /* bf16 only: as written by cle_pack_weights */
} cle_w_layout;

/* Workspace-owning operations, for cle_workspace_bytes(). */
typedef enum { CLE_OP_DISPATCH = 1, CLE_OP_FFN = 2, CLE_OP_DISPATCH_MANY = 3 } cle_op;

/* Library limits. */
#define CLE_MAX_E 1024            /* experts per layer */
#define CLE_MAX_MICROBATCHES 64   /* n: bits of a RunSet mask */
#define CLE_MAX_MAXUTIL_POOL 20   /* MaxUtil enumerates 2^|S| subsets */
#define CLE_MAX_DESC 64           /* micro-batches in one grouped FFN call */

/*
 * cle_route -- router top-k with renormalised softmax gates.
 * Paper §2.1: W_l, I_l = topk(G(h'_l)); the router scores (logits) are given.
 *
 *   logits    [T, E] float32, finite.
 *   topk_idx  [T, k] int32 out: slot s holds the s-th expert in the order
 *             (logit descending, expert id ascending); -0.0 equals +0.0.
 *   topk_gate [T, k] float32 out: g_s = exp(z_s - z_0) / sum_r exp(z_r - z_0)
 *             over the k selected logits, evaluated in float64 (sum in slot
 *             order) and rounded once to float32.
 * Requires 1 <= k <= E <= CLE_MAX_E, T >= 0 (T == 0 enqueues nothing).
 */
cle_status cle_route(const float* logits, int32_t T, int32_t E, int32_t k,
                     int32_t* topk_idx, float* topk_gate, void* stream);

/*
 * cle_route_many -- cle_route for n micro-batches of T tokens each, in one
 * launch (Algorithm 1 routes every micro-batch of the previous RunSet).
 *   logits, topk_idx, topk_gate: HOST arrays of n device pointers, entry j
 *   laid out as in cle_route.  Results are those of n cle_route calls.
 * Requires 1 <= n <= CLE_MAX_MICROBATCHES and cle_route's conditions; a NULL
 * entry (when T > 0) returns CLE_EINVAL before anything is enqueued.
 */
cle_status cle_route_many(int32_t n, const float* const* logits, int32_t T, int32_t E,
                          int32_t k, int32_t* const* topk_idx, float* const* topk_gate,
                          void* stream);

/*
 * cle_dispatch -- per-expert histogram, exclusive scan, stable permutation
 * and row gather: the local form of the expert-parallel all-to-all dispatch
 * (paper §2.2; per-expert token counts T_e as in the EP load-balancing atlas
 * page, section 1).
 *
 *   topk_idx [T, k] int32: expert of assignment a = t*k + s.
 *   x        [T, H] (dt): token rows.
 *   counts   [E] int32 out: assignments per expert.
 *   offsets  [E+1] int32 out: exclusive prefix sum of counts.
 *   dest     [T*k] int32 out: dest[a] = offsets[e] + #{a' < a : idx[a'] = e}.
 *   src      [T*k] int32 out: inverse permutation, src[dest[a]] = a.
 *   xp       [T*k, H] (dt) out: xp[p] = x[src[p] / k]; may be NULL, then the row
 *            copy is skipped (cle_grouped_expert_ffn can read the rows of x
 *            through src instead, see cle_ffn_desc).
 *   ws       workspace of at least cle_workspace_bytes(CLE_OP_DISPATCH, T, E, k, ...).
 * An expert id outside [0, E) is dropped: it is counted nowhere, its dest is
 * -1, and the trailing positions p >= offsets[E] get src = -1 (and zero xp
 * rows).
 * Requires H % 8 == 0, 1 <= k, 1 <= E <= CLE_MAX_E.
 */
cle_status cle_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                        const void* x, int32_t H, cle_dtype dt,
                        int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                        void* xp, void* ws, size_t ws_bytes, void* stream);

/*
 * cle_dispatch_many -- counts, offsets, dest and src of cle_dispatch for n
 * micro-batches of T tokens each, one launch per pass.  No row copy: the
 * expert launch reads the rows through src (cle_ffn_desc.x / .src).
 *   topk_idx, counts, offsets, dest, src: HOST arrays of n device pointers,
 *   entry j laid out as in cle_dispatch.
 *   ws: at least cle_workspace_bytes(CLE_OP_DISPATCH_MANY, T, E, k, 0, n) bytes,
 *   256-byte aligned (one cle_dispatch workspace per micro-batch).
 * Results are those of n cle_dispatch calls.  Requires 1 <= n <=
 * CLE_MAX_MICROBATCHES, 1 <= k, 1 <= E <= CLE_MAX_E.
 */
cle_status cle_dispatch_many(int32_t n, const int32_t* const* topk_idx, int32_t T, int32_t k,
                             int32_t E, int32_t* const* counts, int32_t* const* offsets,
                             int32_t* const* dest, int32_t* const* src, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * One micro-batch of a grouped expert launch.  `layer` selects that layer's
 * expert weights, so micro-batches at different layers share one launch
 * (paper §4.1: workloads of several layers executed in one step).
 */
typedef struct {
  int32_t layer;            /* in [0, L) */
  int32_t rows;             /* rows of xp / act / yp (= T*k of the micro-batch) */
  const int32_t* offsets;   /* [E+1] from cle_dispatch */
  const void* xp;           /* [rows, H] (dt) expert-sorted rows, or NULL (see x) */
  void* act;                /* [rows, I] (dt) out: silu(G) * U */
  void* yp;                 /* [rows, H] (dt) out: expert outputs, one per assignment */
  int32_t shared_rows;      /* rows of x_shared (0 when n_shared == 0) */
  const void* x_shared;     /* [shared_rows, H] (dt), rows for the shared experts */
  void* act_shared;         /* [n_shared, shared_rows, I] (dt) out */
  void* y_shared;           /* [n_shared, shared_rows, H] (dt) out */
  /* Used when xp is NULL: expert-sorted row p is x[src[p] / k], read in place
   * (the dispatch row copy fused into the expert launch; same results). */
  const void* x;            /* [rows / k, H] (dt) token rows */
  const int32_t* src;       /* [rows] from cle_dispatch */
  int32_t k;                /* experts per token */
} cle_ffn_desc;

/*
 * cle_grouped_expert_ffn -- SwiGLU experts for every (micro-batch, expert)
 * segment of all descs, in one grouped launch per GEMM phase.
 * The expert form is SwiGLU with intermediate I, no biases:
 *   [G | U] = X_s W13[l,e]^T,  Act = silu(G) * U,  Y = Act W2[l,e]^T,
 * silu(v) = v / (1 + exp(-v)); segment X_s = xp[offsets[e] : offsets[e+1]].
 * Paper Eq. (1) leaves expert_i abstract; the SwiGLU form is the workload's.
 *
 *   d          HOST array of n_desc descriptors (1 <= n_desc <= CLE_MAX_DESC).
 *   w13        [L, E, 2I, H] (dt): rows [0, I) gate, rows [I, 2I) up.
 *   w2         [L, E, H, I] (dt).
 *   w13_shared [L, n_shared, 2I, H], w2_shared [L, n_shared, H, I]: always-on
 *              shared experts (gate weight 1), applied to every x_shared row;
 *              NULL when n_shared == 0.
 *   bf16: fp32 accumulation; silu from the hardware exp2 and reciprocal
 *         (about 2 ulp of fp32); Act and Y rounded to bf16 (nearest even).
 *   f32 : fp32 throughout.
 *   w_layout   CLE_W_ROWMAJOR, or CLE_W_PACKED (bf16 only) for all four weight
 *              tensors (see cle_pack_weights).
 *   phase_events: NULL, or HOST array of 4 hipEvent_t (for measurement):
 *              [0], [1] take the start and end of the gate/up kernel, [2], [3]
 *              those of the down kernel.  They are recorded by the launches
 *              themselves (no separate marker on `stream`); a phase with no
 *              tiles records its pair back to back.
 * Rows of each segment are computed with one fixed instruction sequence and
 * a K order that depends only on the segment's layer and expert, so a row's
 * result does not depend on the other segments in the launch.
 * Requires I % 64 == 0, and H % 128 == 0 for bf16 or H % 64 == 0 for f32.
 */
cle_status cle_grouped_expert_ffn(const cle_ffn_desc* d, int32_t n_desc,
                                  const void* w13, const void* w2,
                                  const void* w13_shared, const void* w2_shared,
                                  int32_t L, int32_t E, int32_t n_shared, int32_t H, int32_t I,
                                  cle_dtype dt, int32_t w_layout, void* ws, size_t ws_bytes,
                                  void* const* phase_events, void* stream);

/*
 * cle_grouped_expert_ffn_noalloc -- cle_grouped_expert_ffn without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same kernels and the same results, bit for bit.
 * Its scratch is a file-scope device array of CLE_NOALLOC_SCRATCH_BYTES
 * (1 MiB) in the library, one per GPU, held until the process ends; the
 * call allocates and frees nothing, and the kernels set every byte of scratch
 * they read on the same call (no clearing between calls).  Calls that overlap
 * on one GPU (on different streams, or from different host threads) share
 * that array and race: serialise them.  Arguments as cle_grouped_expert_ffn.
 * Returns CLE_EUNSUPPORTED when cle_workspace_bytes(CLE_OP_FFN, 0, E, 1,
 * n_shared, n_desc) exceeds CLE_NOALLOC_SCRATCH_BYTES (e.g. 64 descriptors x
 * 128 experts fit; 64 x 1024 do not), CLE_EHIP if the array's device address
 * cannot be found.
 */
#define CLE_NOALLOC_SCRATCH_BYTES (1u << 20)
cle_status cle_grouped_expert_ffn_noalloc(const cle_ffn_desc* d, int32_t n_desc,
                                          const void* w13, const void* w2,
                                          const void* w13_shared, const void* w2_shared,
                                          int32_t L, int32_t E, int32_t n_shared, int32_t H,
                                          int32_t I, cle_dtype dt, int32_t w_layout,
                                          void* const* phase_events, void* stream);

/*
 * cle_set_expert_tile -- the output tile of the bf16 expert launches
 * (process-wide; takes effect at the next cle_grouped_expert_ffn or
 * cle_loop_step call).  A tuning choice only: the results are bitwise the
 * same for every tile, since each output element is the same sequence of
 * MFMAs over the same K order.
 *   CLE_TILE_DEFAULT  (0) the library's choice per launch: CLE_TILE_256X256
 *                     when the descriptors' rows average at least 512 per
 *                     expert (rows summed over the descriptors, divided by
 *                     n_desc * E), else CLE_TILE_128X256; or the shape named
 *                     by the environment variable CLE_TILE, "128x256" /
 *                     "256x256" / "128x512", when it is set;
 *   CLE_TILE_128X256  (1) 128 rows x 256 weight rows;
 *   CLE_TILE_256X256  (2) 256 rows x 256 weight rows;
 *   CLE_TILE_128X512  (3) 128 rows x 512 weight rows, used where I % 256 == 0
 *                     and H % 512 == 0 (otherwise 128 x 256).
 * The 8-wavefront tiles need I % 128 == 0 and H % 256 == 0; other shapes use
 * 128 x 128 tiles whatever the setting.  Not synchronised with launches in
 * flight on other host threads.  Returns CLE_EINVAL for an unknown value.
 */
#define CLE_TILE_DEFAULT 0
#define CLE_TILE_128X256 1
#define CLE_TILE_256X256 2
#define CLE_TILE_128X512 3
cle_status cle_set_expert_tile(int32_t tile);

/*
 * cle_set_fused_thin_rows -- the fused gate/up -> down launch for thin
 * segments (process-wide; takes effect at the next expert launch).  With
 * rows in 1 .. 16, routed segments of 1 .. rows rows run in one extra launch
 * in which one workgroup computes a segment's gate/up column tiles and then
 * its down column tiles, reading the Act rows it has just written, instead
 * of in the two phase launches (the paper's expert FFN per segment, fused
 * across the phases).  0: off; -1 (the default): the environment variable
 * CLE_FUSE_THIN decides (off when unset).  Used only with 128 x 256 tiles
 * where H / 64 and I / 64 leave K-loop tails of 4 and 2 steps (H = 2048,
 * I = 768 among them); results are bitwise the same either way.  Not
 * synchronised with launches in flight on other host threads.  Returns
 * CLE_EINVAL for rows outside -1 .. 16.
 */
cle_status cle_set_fused_thin_rows(int32_t rows);

/*
 * cle_pack_weights -- re-lays out n_mat row-major bf16 matrices [R, K] (src)
 * into the CLE_W_PACKED layout (dst, same size, must not overlap src), for
 * cle_grouped_expert_ffn with w_layout = CLE_W_PACKED.  Pack each of w13
 * ([L*E] matrices of [2I, H]), w2 ([L*E] of [H, I]) and the shared-expert
 * tensors once, when the weights are loaded.
 * Layout: blocks of 16 rows x 64 K (2 KiB) in (row block, K block) order; a
 * block holds two 1 KiB groups (rows 0-7, rows 8-15); in a group, the 16-byte
 * chunk c (K elements 8c .. 8c+7 of the block) of row r is at position
 * r * 8 + (c ^ r).  Results of the expert launch are bitwise the same for
 * both layouts.
 * Requires dt == CLE_BF16, R % 16 == 0, K % 64 == 0, 16-byte aligned pointers.
 */
cle_status cle_pack_weights(const void* src, void* dst, int64_t n_mat, int32_t R, int32_t K,
                            cle_dtype dt, void* stream);

/*
 * cle_combine -- gate-weighted sum of each token's expert outputs (paper
 * Eq. (1)), plus shared experts and the residual (paper §2.1,
 * h_{l+1} = h'_l + MLP(h'_l)):
 *   y[t] = round( sum_{s<k} gate[t,s] * yp[dest[t*k+s]]
 *                 + sum_{q<n_shared} y_shared[q, t] + residual[t] ),
 * accumulated in float32 in exactly that order; a slot with dest < 0
 * contributes nothing.  y may alias residual (each element is read before
 * it is written by the same thread); it must not overlap anything else.
 *   y_shared [n_shared, T, H] or NULL; residual [T, H] or NULL.
 * Requires H % 8 == 0.
 */
cle_status cle_combine(const void* yp, const int32_t* dest, const float* topk_gate,
                       int32_t T, int32_t k, int32_t H,
                       const void* y_shared, int32_t n_shared, const void* residual,
                       void* y, cle_dtype dt, void* stream);

/*
 * cle_combine_many -- cle_combine for n micro-batches of T tokens each, in
 * one launch (MoECompute_Combine of Algorithm 1 for a whole RunSet).
 *   yp, dest, topk_gate, y: HOST arrays of n device pointers, entry j laid
 *   out as in cle_combine.  y_shared, residual: HOST arrays of n device
 *   pointers (entries may be NULL as in cle_combine), or NULL for none.
 * Entry j of y may alias entry j of residual only.  Results are those of n
 * cle_combine calls.  Requires 1 <= n <= CLE_MAX_MICROBATCHES, H % 8 == 0.
 */
cle_status cle_combine_many(int32_t n, const void* const* yp, const int32_t* const* dest,
                            const float* const* topk_gate, int32_t T, int32_t k, int32_t H,
                            const void* const* y_shared, int32_t n_shared,
                            const void* const* residual, void* const* y, cle_dtype dt,
                            void* stream);

/*
 * cle_rmsnorm_many -- the MoE block's normalised input, for n micro-batches in
 * one launch: y[t] = x[t] / sqrt(mean_h x[t][h]^2 + eps).
 * Paper §2.1: the MoE of layer l takes the post-attention state h'_l and its
 * output is added back to it; the experts (and the router) read the
 * unit-weight RMS-normalised rows while the residual keeps h'_l.
 *   x, y  HOST arrays of n pointers to [T, H] (dt); y may alias x.
 * The sum of squares is taken in float32 in a fixed order and the row is
 * rounded once to dt (bitwise reproducible).
 * Requires 1 <= n <= CLE_MAX_MICROBATCHES, T >= 0, H % 8 == 0, eps >= 0.
 */
cle_status cle_rmsnorm_many(int32_t n, const void* const* x, void* const* y, int32_t T,
                            int32_t H, float eps, cle_dtype dt, void* stream);

/*
 * cle_gate_logits_many -- router logits from the hidden states, for n
 * micro-batches in one launch: z_j = x_j W_g,j^T + b_j.
 * Paper §2.1: the routing scores G(h'_l) that top-k selects from, with G a
 * linear router (no activation); the optional per-expert bias is a fixed
 * offset of each expert's score.  Route the result with cle_route_many.
 *   x       HOST array of n pointers to [T, H] (dt) hidden states.
 *   w_gate  HOST array of n pointers to [E, H] (dt) router weights (each
 *           micro-batch's own layer), row-major or packed (see
 *           cle_pack_weights; bf16 only).
 *   bias    NULL, or HOST array of n pointers to [E] float32 (entries may be NULL).
 *   logits  HOST array of n pointers to [T, E] float32 out.
 * bf16: products of bf16 values summed in float32 over H in one fixed order
 * (results are bitwise reproducible); f32: float32 throughout.
 * Requires 1 <= n <= CLE_MAX_MICROBATCHES, 1 <= E <= CLE_MAX_E, T >= 0
 * (T == 0 enqueues nothing); bf16: H % 128 == 0, E % 64 == 0.
 */
cle_status cle_gate_logits_many(int32_t n, const void* const* x, const void* const* w_gate,
                                const float* const* bias, int32_t T, int32_t H, int32_t E,
                                cle_dtype dt, int32_t w_layout, float* const* logits,
                                void* stream);

/*
 * cle_workload_stats -- per-group workloads and their step statistics.
 * Paper §2.3, Eq. (2) and Eq. (3); the even expert-device mapping (Figure 1)
 * gives group d the experts [d*E/D, (d+1)*E/D).
 *
 *   counts [n, E] int32: row j = counts of micro-batch j.
 *   w      [n, D] int32 out: w[j][d] = sum of counts[j][e] over group d.
 *   acc    [4] int64, accumulated only when runset_mask != 0 (may then not
 *          be NULL).  With W_d = sum_{j in mask} w[j][d]:
 *            acc[0] += sum_d W_d            (work done)
 *            acc[1] += max_d W_d            (effective workload, Eq. (2))
 *            acc[2] += sum_{j in mask} max_d w[j][d]  (the same work run alone)
 *            acc[3] += 1                    (steps)
 *          u = acc[0] / (D * acc[1]) is Eq. (3) over the accumulated steps.
 * Requires 1 <= n <= 64, 1 <= D, E % D == 0, n*D <= 8192, mask bits < n.
 */
cle_status cle_workload_stats(const int32_t* counts, int32_t n, int32_t E, int32_t D,
                              uint64_t runset_mask, int32_t* w, int64_t* acc, void* stream);

/*
 * cle_schedule_step -- Schedule(S, m) of Algorithm 1 (paper §4.2; policies
 * §5.2).  Synchronous, pure host code; touches no device.
 *
 *   w          HOST [n, D] int32 workloads (row j = micro-batch j).
 *   ready_mask bit j set = micro-batch j is in the pool S.
 *   m          minimum RunSet size (1 <= m <= n); if |S| < m all of S runs.
 *   runset_mask HOST out.
 * With U(R) = sum_d W_d / (D * max_d W_d) of the combined workload (0 when
 * it is all zero), compared exactly by cross-multiplication:
 *   B0_ALONE    lowest ready id (m ignored);
 *   B1_LOCKSTEP all of S (m ignored);
 *   CUMUTIL     scan ready ids ascending, take the first, add a later id iff
 *               U rises strictly; then pad to m with the lowest rejected ids;
 *   MAXUTIL     argmax of U over subsets R of S with |R| >= m; ties to the
 *               larger |R|, then to the lexicographically smallest sorted ids;
 *               |S| <= CLE_MAX_MAXUTIL_POOL;
 *   DIFFPEAK    scan ascending, take the first, add an id iff its peak group
 *               (lowest index among maxima) is not a chosen id's peak; pad to m.
 * Requires 1 <= n <= 64, D >= 1, ready_mask != 0 with bits < n.
 */
cle_status cle_schedule_step(const int32_t* w, int32_t n, int32_t D, uint64_t ready_mask,
                             int32_t m, int32_t policy, uint64_t* runset_mask);

/*
 * cle_schedule_step_device -- cle_schedule_step computed on the device, for
 * callers that keep the workloads in device memory (no copy to the host and
 * no wait on the stream).  Same policies, readings and results, bit for bit.
 *
 *   w          [n, D] int32 device workloads.
 *   ready_mask HOST value, as in cle_schedule_step.
 *   runset     [1] uint64 device out.
 * Requires cle_schedule_step's conditions on the host-visible arguments,
 * D <= CLE_MAX_LOOP_D, and n <= CLE_MAX_MAXUTIL_POOL for MAXUTIL (the pool
 * is only known on the device).  Negative workloads count as 0.
 */
#define CLE_MAX_LOOP_D 64
cle_status cle_schedule_step_device(const int32_t* w, int32_t n, int32_t D, uint64_t ready_mask,
                                    int32_t m, int32_t policy, uint64_t* runset, void* stream);

/*
 * The device-driven loop: Algorithm 1 (paper §4.2) with Schedule(S, m)
 * computed on the device, so a step is a fixed sequence of launches and the
 * host never waits for the stream between steps.
 *
 * cle_loop_state -- the loop's state in DEVICE memory that the caller
 * allocates (sizeof(cle_loop_state) bytes, 8-byte aligned); written by
 * cle_loop_init and cle_loop_step, readable by copying it back.
 */
typedef struct {
  int32_t layer[64];      /* l_j: the layer micro-batch j runs next; L once finished */
  int32_t run_layer[64];  /* the layer at which each member of `runset` ran */
  int32_t start[64];      /* starting layers (used again by a restart) */
  uint64_t ready;         /* the pool S: bit j set iff l_j < L */
  uint64_t todo;          /* routed at the start of the next step: the last RunSet's
                             members that are still ready (all of S at first: RunSet_0 = S) */
  uint64_t runset;        /* RunSet of the last step (0 when nothing ran) */
  int64_t acc[4];         /* as cle_workload_stats' acc, over every step that ran */
  int32_t n, L;
  int32_t restarts;       /* how many times every micro-batch finished and the loop restarted */
  int32_t restarted;      /* 1 from a restart until the next step begins */
} cle_loop_state;

/*
 * cle_loop_init -- set the state for n micro-batches of an L-layer stack:
 * l_j = start[j] (HOST array of n, or NULL for all 0), S = {j : l_j < L},
 * todo = S, runset = 0, acc = 0.  Requires 1 <= n <= CLE_MAX_MICROBATCHES,
 * L >= 1, 0 <= start[j] <= L.
 */
cle_status cle_loop_init(cle_loop_state* state, int32_t n, int32_t L, const int32_t* start,
                         void* stream);

/*
 * cle_loop_desc -- everything one loop step touches (HOST struct; the
 * pointers are device pointers, per micro-batch j < n).  Layouts are those
 * of cle_route, cle_dispatch (fused row gather: no xp), cle_grouped_expert_ffn
 * and cle_combine.
 */
typedef struct {
  int32_t n, L, T, E, k, H, I, D, m, policy, n_shared;
  int32_t dtype;         /* cle_dtype */
  int32_t w_layout;      /* cle_w_layout */
  int32_t restart;       /* 1: when every micro-batch has finished, start over
                            (l_j = start_j, h_j = h0_j) in the same step */
  const float* logits[64];          /* [L, T, E]: router logits of every layer */
  void* h[64];                      /* [T, H]: hidden state, updated in place */
  const void* h0[64];               /* [T, H]: restart source (restart only) */
  int32_t* idx[64];                 /* [T, k] */
  float* gate[64];                  /* [T, k] */
  int32_t* counts[64];              /* [E] */
  int32_t* offsets[64];             /* [E + 1] */
  int32_t* dest[64];                /* [T * k] */
  int32_t* src[64];                 /* [T * k] */
  void* act[64];                    /* [T * k, I] */
  void* yp[64];                     /* [T * k, H] */
  void* act_shared[64];             /* [n_shared, T, I] (n_shared > 0) */
  void* y_shared[64];               /* [n_shared, T, H] (n_shared > 0) */
  const void* w13;                  /* [L, E, 2I, H] */
  const void* w2;                   /* [L, E, H, I] */
  const void* w13_shared;           /* [L, n_shared, 2I, H] or NULL */
  const void* w2_shared;            /* [L, n_shared, H, I] or NULL */
  void* ws_dispatch;                /* CLE_OP_DISPATCH_MANY workspace, n_desc = n */
  size_t ws_dispatch_bytes;
  void* ws_ffn;                     /* CLE_OP_FFN workspace, n_desc = n */
  size_t ws_ffn_bytes;
  int32_t* w;                       /* [n, D] out or NULL: workloads the last schedule saw */
  uint64_t* log;                    /* NULL, or a ring of log_cap RunSet masks: the step that
                                       ran as the s-th (acc[3] = s before it) writes entry
                                       s % log_cap */
  int64_t log_cap;
  cle_loop_state* state;
  /* Routing from the hidden state (optional): when w_gate is not NULL, the
   * router logits of micro-batch j at layer l are computed from h_j by
   * cle_gate_logits_many (weights w_gate[l], bias gate_bias[l]) into
   * gate_logits[j], and `logits` is not read. */
  const void* w_gate;               /* [L, E, H] (dtype, w_layout) or NULL */
  const float* gate_bias;           /* [L, E] float32 or NULL */
  float* gate_logits[64];           /* [T, E] float32 scratch (w_gate only) */
  /* Normalised MoE input (optional): with prenorm = 1 each routed micro-batch's
   * rows are first RMS-normalised (cle_rmsnorm_many, norm_eps) into xn[j];
   * the router and the experts read xn[j], the combine adds to h[j]. */
  int32_t prenorm;
  float norm_eps;
  void* xn[64];                     /* [T, H] (prenorm only) */
} cle_loop_desc;

/*
 * cle_loop_step -- enqueue one iteration of Algorithm 1 on `stream`:
 *   1. route and dispatch the micro-batches in state->todo, each at its l_j
 *      (from logits[j] at layer l_j, or with w_gate from h_j -- xn_j with
 *      prenorm -- through the router of layer l_j);
 *   2. on the device: w[j][d] for j in S, RunSet = Schedule(S, m) as in
 *      cle_schedule_step, acc as in cle_workload_stats, the log entry,
 *      run_layer = l_j and l_j += 1 for the members, S and todo updated
 *      (and the restart, if asked for and S became empty);
 *   3. the grouped expert FFN of every member at its run_layer (as
 *      cle_grouped_expert_ffn, whose phase_events it takes);
 *   4. h_j = h_j + combine (Eq. (1)) for every member;
 *   5. on a restart, h_j = h0_j for every j.
 * A step with S empty (and no restart) does nothing.  Results, state and
 * statistics are bitwise those of the host-driven sequence of the same calls.
 * Requires the conditions of the calls above, E % D == 0, D <= CLE_MAX_LOOP_D,
 * 1 <= m <= n, and n <= CLE_MAX_MAXUTIL_POOL for MAXUTIL.
 */
cle_status cle_loop_step(const cle_loop_desc* d, void* const* phase_events, void* stream);

/*
 * cle_workspace_bytes -- device workspace, in bytes, that `op` needs:
 *   CLE_OP_DISPATCH: depends on T, E, k (n_shared, n_desc ignored);
 *   CLE_OP_DISPATCH_MANY: n_desc (= n of cle_dispatch_many) times that;
 *   CLE_OP_FFN:      depends on E, n_shared, n_desc (T, k ignored).
 * The workspace must be 256-byte aligned.  Returns 0 for an unknown op or
 * out-of-range sizes.
 */
size_t cle_workspace_bytes(int32_t op, int32_t T, int32_t E, int32_t k, int32_t n_shared,
                           int32_t n_desc);

/* Static string for a status code. */
const char* cle_status_string(cle_status s);

/* Library version, "major.minor.patch". */
const char* cle_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CLE_H */
