/*
 * beam_moe.h -- C ABI of libbeam_moe.so, one Beam Mixture-of-Experts block on
 * an AMD Instinct MI355X (gfx950).
 *
 * Source pages (cited by title and section):
 *   [MoE] "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen,
 *         anpassen und skalieren können" (spke.com), section "Mixture of
 *         Experts"; the same paragraph on "Reflection 发布 501B 开放模型 Beam，
 *         支持自托管定制与扩展" (sihot.dev), section 混合专家（Mixture of Experts）.
 *   [RES] the same pages, section "Residual Stream".
 *
 * Conventions shared by every entry point
 *   - Tensors are DEVICE pointers, row-major and contiguous.  "bf16" tensors
 *     are uint16_t bit patterns.  Every pointer must be 16-byte aligned.
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates, frees or synchronises device memory.  Work is enqueued
 *     on `stream` (a hipStream_t; NULL = the default stream) and is complete
 *     when that stream is synchronised.  Inputs are never written; outputs
 *     are overwritten in full; outputs must not alias inputs.  Workspace
 *     contents are not preserved between calls, so two calls in flight at the
 *     same time must use different workspaces.
 *   - Return value: 0 on success, a negative BEAM_MOE_ERR_* code otherwise.
 *     Every argument check runs on the host before any HIP call, so a call
 *     that fails validation enqueues nothing.  T == 0 with valid dimensions
 *     returns 0 and enqueues nothing; pointers and workspace size are not
 *     examined then (empty tensors may have NULL data pointers).  HIP_ERROR reports a launch failure (hipGetLastError); a fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Dimension rules (the Beam shapes satisfy all of them):
 *       0 <= T <= 2^24;  H, I in [64, 32768] and multiples of 64;
 *       1 <= E <= 512;  E % groups == 0 and E / groups >= 2;
 *       1 <= topk_groups <= groups;  1 <= k <= min(32, topk_groups * E / groups)
 *       (route / block); 1 <= k <= 32 (forward / permute); scale finite.
 *   - Device data (id range, weight values) is not validated: routing ids
 *     outside [0, E) are dropped (they contribute nothing and are not counted).
 *   - The first compute call on a device checks that it is gfx950
 *     (UNSUPPORTED_DEVICE otherwise).
 *   - The library is stateless apart from a per-device property cache and the
 *     optional stage timer; calls from several host threads are safe.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BEAM_MOE_OK 0
#define BEAM_MOE_ERR_INVALID_DIM (-1)
#define BEAM_MOE_ERR_NULL_POINTER (-2)
#define BEAM_MOE_ERR_MISALIGNED (-3)
#define BEAM_MOE_ERR_WORKSPACE_TOO_SMALL (-4)
#define BEAM_MOE_ERR_UNSUPPORTED_DEVICE (-5)
#define BEAM_MOE_ERR_HIP (-6)

/* Human-readable name of a status code (static string, never NULL). */
const char* beam_moe_status_string(int status);

/* Library version, "major.minor.patch" (static string). */
const char* beam_moe_version(void);

/* Bytes of workspace that route, permute, forward, block and sublayer need
 * for these sizes (the maximum over all of them).  Returns 0 if the sizes
 * break the dimension rules. */
size_t beam_moe_workspace_bytes(int64_t T, int H, int I, int E, int k);

/*
 * Packed expert weights.  forward, block and sublayer read the expert weight
 * matrices in a packed block layout, produced once (at model load) by
 * beam_moe_pack_weights from the nn.Linear layout W[e][n][k] (k contiguous):
 *   - each expert matrix W[e] (N x K) becomes ceil(N/128) row blocks x K/32
 *     k-blocks of 128 rows x 32 k = 8192 bytes; block (rb, kb) starts at
 *     byte (rb * K/32 + kb) * 8192 of the expert; experts follow each other,
 *     each taking beam_moe_packed_weight_bytes(N, K) bytes;
 *   - row j (0..127) of a block takes 64 bytes at byte j*64; its 16-byte
 *     chunk c (0..3), holding k = kb*32 + 8c .. kb*32 + 8c + 7, is stored at
 *     chunk position c XOR (((j >> 1) XOR (j >> 2)) AND 3);
 *   - rows rb*128 + j >= N are zero.
 * One k-step of a weight tile is then one contiguous stretch of memory that
 * lands in on-chip memory exactly as the matrix-core reads want it.
 *
 * beam_moe_packed_weight_bytes: bytes of one packed N x K expert matrix
 *   (N, K multiples of 64 in [64, 32768]); 0 if the sizes break that rule.
 * beam_moe_pack_weights: dst [E * packed bytes] = packed copy of src [E,N,K]
 *   bf16.  src and dst must not overlap (INVALID_DIM otherwise).  Enqueued on
 *   `stream`, like every compute call; the caller owns both buffers.
 */
size_t beam_moe_packed_weight_bytes(int N, int K);
int beam_moe_pack_weights(void* stream, int E, int N, int K, const uint16_t* src, uint16_t* dst);

/*
 * FP8 expert weights (OCP E4M3), for the *_fp8 compute calls.  The pages
 * state that an FP8 checkpoint of the model exists ([MoE]; section on
 * hardware requirements) but not its scaling; this library's encoding is:
 *   - one scale per output row r of each expert matrix: 2^e_r with e_r the
 *     smallest integer such that max_k |W[r,k]| <= 448 * 2^e_r (e_r = 0 for
 *     an all-zero row); scales[e][r] holds 2^e_r as fp32;
 *   - code[r,k] = the E4M3 value nearest to W[r,k] * 2^-e_r, ties to the even
 *     mantissa (the scaling by a power of two is exact); the weight the
 *     kernels use is value(code) * 2^e_r;
 *   - layout: the packed block grid above with one byte per weight: blocks of
 *     128 rows x 32 k = 4096 bytes at (rb * K/32 + kb) * 4096; row j takes
 *     32 bytes at j*32; its 8-byte chunk c (k = kb*32 + 8c .. + 7) is stored
 *     at chunk position c XOR ((j >> 3) AND 3); rows past N are zero.
 * beam_moe_packed_fp8_bytes: bytes of one packed N x K FP8 expert matrix (0
 *   if the sizes break the rule above).
 * beam_moe_pack_weights_fp8: dst [E * packed bytes] and scales [E,N] fp32
 *   from src [E,N,K] bf16 (finite values).  No two of the buffers may overlap.
 */
size_t beam_moe_packed_fp8_bytes(int N, int K);
int beam_moe_pack_weights_fp8(void* stream, int E, int N, int K, const uint16_t* src,
                              uint8_t* dst, float* scales);

/*
 * Router + group-limited top-k  ([MoE]; router in FP32 per [RES]).
 *   z[t,e]  = sum_h x[t,h] * w_router[e,h]  (+ logit_offset[e])   FP32 accumulate
 *   s[t,e]  = 1 / (1 + exp(-z[t,e]))                               FP32
 *   group g = experts [g*E/groups, (g+1)*E/groups); its score is the sum of its
 *             two largest s; the topk_groups best groups are kept;
 *   the k largest s among experts of kept groups are selected (exact ties go
 *   to the lower index), ordered by decreasing s;
 *   topk_weights[t,j] = scale * (s_j / sum of the k selected s).
 * x            [T,H] bf16          w_router [E,H] bf16
 * logit_offset [E] fp32 or NULL (added to the logit before the sigmoid)
 * topk_ids     [T,k] int32 out     topk_weights [T,k] fp32 out
 * expert_counts[E] int32 out or NULL (number of tokens that picked each expert)
 */
int beam_moe_route(void* stream, int64_t T, int H, int E, int groups, int topk_groups, int k,
                   float scale, const uint16_t* x, const uint16_t* w_router,
                   const float* logit_offset, int32_t* topk_ids, float* topk_weights,
                   int32_t* expert_counts, void* workspace, size_t workspace_bytes);

/*
 * Token permutation: the (token, slot) assignments a = t*k + j sorted by
 * expert id with a stable sort (ascending token order inside an expert).
 * topk_ids       [T,k] int32 in
 * expert_counts  [E] int32 out      expert_offsets [E+1] int32 out (exclusive scan)
 * sorted_tokens  [T*k] int32 out    token of each expert-major row; entries
 *                                   past expert_offsets[E] are left untouched
 * row_of         [T*k] int32 out    expert-major row of each assignment, -1 for
 *                                   an id outside [0, E)
 */
int beam_moe_permute(void* stream, int64_t T, int E, int k, const int32_t* topk_ids,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_tokens,
                     int32_t* row_of, void* workspace, size_t workspace_bytes);

/*
 * Experts + combine with given routing  ([MoE]; SwiGLU product in FP32 per [RES]).
 *   for each assignment (t, j) with e = topk_ids[t,j] in [0, E):
 *     g = w_gate[e] . x[t],  u = w_up[e] . x[t]              (FP32 accumulate)
 *     h = bf16( g / (1 + exp(-g)) * u )                       (FP32, one rounding)
 *     o = w_down[e] . h                                       (FP32 accumulate)
 *   y[t] = bf16( sum_j topk_weights[t,j] * o_j )   FP32 sum in slot order j = 0..k-1
 * topk_weights are used as given (the router's weights already hold the scale).
 * x [T,H] bf16; w_gate, w_up: the packed I x H matrices of the E experts,
 * w_down: the packed H x I matrices (see beam_moe_pack_weights); y [T,H] bf16
 * out; expert_counts [E] int32 out or NULL.
 */
int beam_moe_forward(void* stream, int64_t T, int H, int I, int E, int k, const uint16_t* x,
                     const int32_t* topk_ids, const float* topk_weights, const uint16_t* w_gate,
                     const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes);

/*
 * Whole block: route -> permute -> gate/up GEMM + SwiGLU -> down GEMM -> combine.
 * Same arguments and meaning as route and forward (expert weights packed).
 * topk_ids / topk_weights /
 * expert_counts are outputs and may each be NULL (then they live in the
 * workspace and are not returned).
 */
int beam_moe_block(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                   int k, float scale, const uint16_t* x, const uint16_t* w_router,
                   const float* logit_offset, const uint16_t* w_gate, const uint16_t* w_up,
                   const uint16_t* w_down, uint16_t* y, int32_t* topk_ids, float* topk_weights,
                   int32_t* expert_counts, void* workspace, size_t workspace_bytes);

/*
 * The same two calls with FP8 expert weights (see beam_moe_pack_weights_fp8):
 * w_* are the packed E4M3 codes and s_* the [E,N] fp32 row scales of gate,
 * up and down.  Each expert computes with the weights value(code) * scale
 * (dequantised exactly to bf16 operands, the scale applied to the FP32
 * accumulators); everything else is as in forward / block.
 */
int beam_moe_forward_fp8(void* stream, int64_t T, int H, int I, int E, int k, const uint16_t* x,
                         const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                         const float* s_up, const uint8_t* w_down, const float* s_down,
                         uint16_t* y, int32_t* expert_counts, void* workspace,
                         size_t workspace_bytes);
int beam_moe_block_fp8(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                       int k, float scale, const uint16_t* x, const uint16_t* w_router,
                       const float* logit_offset, const uint8_t* w_gate, const float* s_gate,
                       const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                       const float* s_down, uint16_t* y, int32_t* topk_ids, float* topk_weights,
                       int32_t* expert_counts, void* workspace, size_t workspace_bytes);

/*
 * beam_moe_block without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP-graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a static
 * device array of BEAM_MOE_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held from the first call on that GPU until the process ends.
 * Everything else (arguments, layouts, results, bf16 packed weights) is as
 * in beam_moe_block; the results are bit-identical to its.
 *   - The call allocates nothing: no hipMalloc / hipFree, no allocating
 *     library routine.  Its first call on a device looks up the array's
 *     device address (hipGetSymbolAddress) and caches it.
 *   - All calls on one GPU share its array, which keeps the last call's
 *     contents; everything a call needs zeroed it clears itself with a fill
 *     kernel.  Calls that overlap on one GPU (different streams or threads
 *     without ordering) race on the array and give undefined results.
 *   - WORKSPACE_TOO_SMALL when the sizes need more scratch than the array
 *     holds (beam_moe_workspace_bytes(T, H, I, E, k) > the maximum); it is
 *     checked before anything is enqueued.  At the Beam shape (H 5120,
 *     I 2560, E 256, k 8) T up to 259 fits: decode and speculative-verify
 *     batches; prefill batches take beam_moe_block.
 */
#define BEAM_MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int beam_moe_block_noalloc(void* stream, int64_t T, int H, int I, int E, int groups,
                           int topk_groups, int k, float scale, const uint16_t* x,
                           const uint16_t* w_router, const float* logit_offset,
                           const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                           uint16_t* y, int32_t* topk_ids, float* topk_weights,
                           int32_t* expert_counts);

/*
 * Residual stream helpers  ([RES]: every sublayer is normalised before and
 * after; the embedding is residual step 1; at step >= 2 the stream keeps
 * sqrt((step-1)/step) of itself and adds 1/sqrt(step) of the sublayer output).
 * RMSNorm here is v / sqrt(mean(v^2) + eps) with unit gain, in FP32.
 *
 * beam_moe_stream_init:    stream[T,H] fp32 out = x[T,H] bf16 widened.
 * beam_moe_rmsnorm:        out[T,H] bf16 = bf16(RMSNorm(in[T,H] fp32)).
 * beam_moe_residual_update: stream[T,H] fp32 in/out =
 *                   sqrt((step-1)/step)*stream + RMSNorm(float(y)) / sqrt(step),
 *                   y [T,H] bf16; step >= 2.
 * beam_moe_sublayer: one sandwich-normed MoE sublayer at residual step `step`:
 *                   x_in = rmsnorm(stream); y = block(x_in); residual_update(y)
 *                   (expert weights packed, as for block).
 *                   moe_input / moe_output [T,H] bf16 receive x_in and y when
 *                   not NULL; topk_ids / topk_weights / expert_counts as in block.
 */
int beam_moe_stream_init(void* stream, int64_t T, int H, const uint16_t* x, float* stream_out);
int beam_moe_rmsnorm(void* stream, int64_t T, int H, float eps, const float* in, uint16_t* out);
int beam_moe_residual_update(void* stream, int64_t T, int H, float eps, int step,
                             const uint16_t* y, float* stream_io);
int beam_moe_sublayer(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                      int k, float scale, float eps, int step, float* stream_io,
                      const uint16_t* w_router, const uint16_t* w_gate, const uint16_t* w_up,
                      const uint16_t* w_down, uint16_t* moe_input, uint16_t* moe_output,
                      int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                      void* workspace, size_t workspace_bytes);
/* beam_moe_sublayer with FP8 (E4M3) expert weights and per-row scales, as
 * beam_moe_block_fp8.  Scale pointers must not be NULL. */
int beam_moe_sublayer_fp8(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                          int k, float scale, float eps, int step, float* stream_io,
                          const uint16_t* w_router, const uint8_t* w_gate, const float* s_gate,
                          const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                          const float* s_down, uint16_t* moe_input, uint16_t* moe_output,
                          int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                          void* workspace, size_t workspace_bytes);

/*
 * Attention sublayer of one sequence (prefill): page "Willkommen Beam: ein
 * offenes 501B-Modell, das Sie besitzen, anpassen und skalieren können",
 * section "Attention" (grouped-query attention, 48 query heads and 8
 * key/value heads, RMSNorm on queries and keys, RoPE on the sliding-window
 * layers, the query scaling (1 + (pos + 1) / 2048)^0.1 on the global layers,
 * a sigmoid gate from the layer input on every channel of every head before
 * the output projection); section "Long Context" (head size 128); section
 * "Residual Stream" (RoPE and the query scaling in FP32).
 *
 *   u       [T, H] bf16, the layer input at positions 0 .. T-1
 *   w_qkvg  [Wq; Wk; Wv; Wg] stacked into one [14336, H] matrix (rows 0..6143
 *           Wq, 6144..7167 Wk, 7168..8191 Wv, 8192..14335 Wg), packed with
 *           beam_moe_pack_weights(E = 1, N = 14336, K = H)
 *   w_o     Wo [H, 6144] packed with beam_moe_pack_weights(E = 1, N = H, K = 6144)
 *   y       [T, H] bf16 out
 *   global_layer  1: no position encoding, queries scaled; 0: RoPE with base
 *           theta on dims (i, i + 64), keys j with i - window < j <= i
 *
 * Per head: q and k are RMSNorm-ed over their 128 dims (eps 1e-6, unit gain,
 * FP32), then rotated or scaled, and rounded to bf16; v is rounded to bf16;
 * scores are scaled by 1/sqrt(128); softmax in FP32; query head h reads
 * key/value head h / 6; the gated head outputs are rounded to bf16 before the
 * output projection.  Constraints: 0 <= T <= 65536, H a multiple of 64
 * in [64, 32768], T * H < 2^30,
 * window >= 1 and theta > 0 on sliding-window layers.  Workspace:
 * beam_attn_workspace_bytes(T, H) bytes (0 for invalid sizes), 16-byte
 * aligned, contents not preserved.  Errors as for the MoE calls.
 */
size_t beam_attn_workspace_bytes(int64_t T, int H);
int beam_attn_forward(void* stream, int64_t T, int H, int global_layer, int window, float theta,
                      const uint16_t* u, const uint16_t* w_qkvg, const uint16_t* w_o, uint16_t* y,
                      void* workspace, size_t workspace_bytes);

/*
 * Dense SwiGLU layer (the first three layers): page "Willkommen Beam: ein
 * offenes 501B-Modell, das Sie besitzen, anpassen und skalieren können",
 * section "Mixture of Experts" (dense layers before the expert layers), with
 * the expert's SwiGLU and rounding: y = bf16( down( bf16( SiLU(gate x) *
 * (up x) ) ) ), gate/up and the product in FP32, down accumulated in FP32.
 * The pages give no intermediate size; I = 20480 (8 x 2560) is the reading
 * the tests and benchmark use, any I with I / chunks a multiple of 64 works.
 *
 *   x        [T, H] bf16
 *   w_gate   gate [I, H] split into `chunks` row blocks of I / chunks rows,
 *            i.e. [chunks, I/chunks, H], packed with beam_moe_pack_weights
 *            (E = chunks, N = I / chunks, K = H); likewise w_up
 *   w_down   down [H, I] split into column blocks: chunk c is columns
 *            c*I/chunks .. (c+1)*I/chunks - 1, i.e. [chunks, H, I/chunks],
 *            packed with E = chunks, N = H, K = I / chunks
 *   y        [T, H] bf16 out
 *
 * The layer runs as the expert path with `chunks` experts, every token sent
 * to all of them with weight 1: each chunk's down output stays FP32 and the
 * chunks are summed in order in FP32 before the one bf16 rounding of y (the
 * same value as one down product over I, up to FP32 summation order).  More
 * chunks give decode-size batches more parallel work.  Constraints: 1 <=
 * chunks <= 32, I % chunks == 0, H and I / chunks multiples of 64 in [64,
 * 32768], 0 <= T <= 2^24.  Workspace: beam_dense_workspace_bytes(T, H, I,
 * chunks) bytes (0 for invalid sizes).  Errors as for the MoE calls.
 */
size_t beam_dense_workspace_bytes(int64_t T, int H, int I, int chunks);
int beam_dense_mlp(void* stream, int64_t T, int H, int I, int chunks, const uint16_t* x,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                   void* workspace, size_t workspace_bytes);
/*
 * The dense layer with FP8 (E4M3) weights: each chunk matrix packed with
 * beam_moe_pack_weights_fp8 (E = chunks; one power-of-two scale per row of
 * each chunk, so the down matrix's scales depend on the chunking), as the
 * FP8 expert path (beam_moe_forward_fp8).  Same rules and errors.
 */
int beam_dense_mlp_fp8(void* stream, int64_t T, int H, int I, int chunks, const uint16_t* x,
                       const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                       const float* s_up, const uint8_t* w_down, const float* s_down, uint16_t* y,
                       void* workspace, size_t workspace_bytes);

/*
 * Expert-GEMM schedule for later calls in this process: 0 = automatic (the
 * weight-streaming schedule when there are fewer than 20 assignments per
 * expert on average, the LDS-tiled schedule otherwise), 1 = always
 * streaming, 2 = always tiled.  Both give the same results up to FP32
 * summation order inside the MFMA accumulations.  Returns INVALID_DIM for
 * another mode.
 */
int beam_moe_set_schedule(int mode);

/*
 * Stage timer (measurement aid).  After beam_moe_timer_begin(max_calls), each
 * block / forward / attention call (up to max_calls of them) records a hipEvent before
 * and after each of its stages on its stream.  beam_moe_timer_end
 * synchronises those events, writes the summed milliseconds of each stage
 * into stage_ms[0 .. n_stages-1] (n_stages >= beam_moe_stage_count()), the
 * number of timed calls into *n_calls, and releases the events.  One timer
 * per process; not for concurrent use from several threads.
 * beam_moe_timer_begin_stages(max_calls, stage_mask) records events only for
 * the stages whose bit (1u << stage) is set, so that a timed loop carries no
 * more events than it needs; the other stages read 0 at the end.
 * beam_moe_timer_begin(n) is beam_moe_timer_begin_stages(n, all stages).
 * INVALID_DIM for max_calls outside [1, 100000], an empty mask, a bit at or
 * above beam_moe_stage_count(), or a timer already running.
 */
int beam_moe_stage_count(void);
const char* beam_moe_stage_name(int stage);
int beam_moe_timer_begin(int max_calls);
int beam_moe_timer_begin_stages(int max_calls, unsigned stage_mask);
int beam_moe_timer_end(double* stage_ms, int n_stages, int* n_calls);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
