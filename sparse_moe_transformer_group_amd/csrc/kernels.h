// Internal launchers of libbeam_moe (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace beam {

// ---- router (router.hip) ----
// Number of K-slices the router logit GEMM is split into for T tokens; the
// slices' partial sums are added in slice order by the selection kernel.
int router_splits(int64_t T, int H, int E);
hipError_t launch_router_logits(hipStream_t s, const uint16_t* x, const uint16_t* wr, float* zpart,
                                int T, int H, int E, int S);
hipError_t launch_select(hipStream_t s, const float* zpart, int S, const float* offset, int T, int E,
                         int groups, int topk_groups, int k, float scale, int32_t* ids, float* w,
                         int32_t* counts);
hipError_t launch_fill_i32(hipStream_t s, int32_t* p, int64_t n, int32_t v);

// ---- permutation (permute.hip) ----
constexpr int kPermChunk = 512;  // assignments per permutation block
inline int64_t perm_blocks(int64_t Tk) { return (Tk + kPermChunk - 1) / kPermChunk; }
hipError_t launch_permute(hipStream_t s, const int32_t* ids, int64_t Tk, int k, int E,
                          int32_t* block_hist, int32_t* block_base, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_tokens, int32_t* row_of,
                          int32_t* user_counts);

// ---- grouped expert GEMMs (gemm_stream.hip, gemm_tiled.hip) ----
struct GroupedArgs {
  const uint16_t* act;          // activations: x [T,H] (gate/up) or h [Tk,I] (down)
  const int32_t* sorted_tokens; // row indirection for x (gate/up); NULL for h
  const uint16_t* w0;           // gate [E,I,H] or down [E,H,I]
  const uint16_t* w1;           // up [E,I,H] or NULL
  const int32_t* counts;        // [E]
  const int32_t* offsets;       // [E+1]
  void* out;                    // h [Tk,I] bf16 or o [Tk,H] fp32
  int N;                        // output features (I or H)
  int K;                        // reduction length (H or I)
  int E;
  int64_t Tk;                   // number of assignments (rows of h / o)
};
// Decode-size batches: every weight row is streamed once per <= 16*mt tokens.
hipError_t launch_gateup_stream(hipStream_t s, const GroupedArgs& a, int64_t T, int k);
hipError_t launch_down_stream(hipStream_t s, const GroupedArgs& a, int64_t T, int k);
// Prefill-size batches: LDS-staged tiles on MFMA, persistent XCD-aware schedule.
hipError_t launch_gateup_tiled(hipStream_t s, const GroupedArgs& a, int num_cu);
hipError_t launch_down_tiled(hipStream_t s, const GroupedArgs& a, int num_cu);

// ---- combine / norms (combine.hip) ----
hipError_t launch_combine(hipStream_t s, const float* o, const int32_t* row_of, const float* w,
                          int T, int H, int k, uint16_t* y);
hipError_t launch_stream_init(hipStream_t s, const uint16_t* x, float* out, int64_t T, int H);
hipError_t launch_rmsnorm(hipStream_t s, const float* in, uint16_t* out, int64_t T, int H, float eps);
hipError_t launch_residual(hipStream_t s, const uint16_t* y, float* stream, int64_t T, int H,
                           float eps, int step);

}  // namespace beam
