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
// ids[t*C + j] = j, w = 1 (a dense layer as C chunks of its intermediate dimension)
hipError_t launch_dense_routing(hipStream_t s, int32_t* ids, float* w, int64_t T, int C);

// ---- permutation (permute.hip) ----
constexpr int kPermChunk = 512;  // assignments per permutation block
inline int64_t perm_blocks(int64_t Tk) { return (Tk + kPermChunk - 1) / kPermChunk; }
// clear16: 16 counters the permutation's single-workgroup kernel sets to 0
// (the expert GEMMs' tile-claim counters), or null.
hipError_t launch_permute(hipStream_t s, const int32_t* ids, int64_t Tk, int k, int E,
                          int32_t* block_hist, int32_t* block_base, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_tokens, int32_t* row_of,
                          int32_t* user_counts, int32_t* clear16);

// ---- packed expert weights (pack.hip) ----
// An expert matrix W[N][K] (bf16, K contiguous) is stored as ceil(N/128) row
// blocks x K/32 k-blocks of 128 rows x 32 k (8 KB each); block (rb, kb) sits
// at byte (rb * K/32 + kb) * 8192 of the expert, experts back to back.  Row j
// of a block takes 64 bytes at j * 64; its logical 16-byte chunk c (k = 32 kb
// + 8c .. 32 kb + 8c + 7) is stored at physical chunk c ^ pack_swz(j).  Rows
// past N are zero.  A k-step of a tile is then one contiguous stretch of
// memory, already in the LDS layout the MFMA reads conflict-free.
constexpr int kPackRows = 128;
constexpr int kPackK = 32;
constexpr int kPackBlockBytes = kPackRows * kPackK * 2;
__host__ __device__ inline int pack_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
__host__ __device__ inline int64_t packed_expert_bytes(int N, int K) {
  return (int64_t)((N + kPackRows - 1) / kPackRows) * (K / kPackK) * kPackBlockBytes;
}
hipError_t launch_pack(hipStream_t s, const uint16_t* src, uint16_t* dst, int E, int N, int K);

// FP8 (OCP E4M3) expert weights: the same block grid with one byte per
// weight, i.e. blocks of 128 rows x 32 k = 4 KB; row j takes 32 bytes and
// its logical 8-byte chunk c (k = 32 kb + 8c .. + 7) sits at chunk position
// c ^ pack8_swz(j).  Each row r has a scale 2^e_r (fp32, [E][N]): the
// smallest power of two with max|W[r,:]| <= 448 * 2^e_r; a code is the E4M3
// value nearest to W * 2^-e_r (ties to even); the weight is value * 2^e_r.
constexpr int kPack8BlockBytes = kPackRows * kPackK;
// The swizzle depends on row bits 2..4 only (so it is the same for row r of
// every 32-row block): the four rows that share a bank set under 8-byte
// operand reads -- rows r, r+4, r+8, r+12 when 16 lanes are served over 32
// banks, rows r, r+8, r+16, r+24 when 32 lanes are served over 64 -- get
// four different chunk positions.  A swizzle by bits 3..4 alone leaves the
// first case 2-way conflicted (measured: SQ_LDS_BANK_CONFLICT).
__host__ __device__ inline int pack8_swz(int row) {
  return (((row >> 2) ^ (row >> 4)) & 1) | ((row >> 2) & 2);
}
__host__ __device__ inline int64_t packed8_expert_bytes(int N, int K) {
  return (int64_t)((N + kPackRows - 1) / kPackRows) * (K / kPackK) * kPack8BlockBytes;
}
hipError_t launch_pack_fp8(hipStream_t s, const uint16_t* src, uint8_t* dst, float* scales, int E,
                           int N, int K);

// ---- grouped expert GEMMs (gemm_stream.hip, gemm_tiled.hip) ----
struct GroupedArgs {
  const uint16_t* act;          // activations: x [T,H] (gate/up) or h (down): [Tk,I] row-major
                                // on the stream path, k-major on the tiled path (see gemm_tiled.hip)
  const int32_t* sorted_tokens; // row indirection for x (gate/up); NULL for h
  const uint16_t* w0;           // packed gate [E,I,H] or down [E,H,I] (bf16, or FP8 bytes)
  const uint16_t* w1;           // packed up [E,I,H] or NULL
  const float* s0;              // FP8 row scales of w0 [E][N], NULL for bf16 weights
  const float* s1;              // FP8 row scales of w1, or NULL
  const int32_t* counts;        // [E]
  const int32_t* offsets;       // [E+1]
  void* out;                    // h bf16 (layout as for act) or o [Tk,H] fp32
  int N;                        // output features (I or H)
  int K;                        // reduction length (H or I)
  int E;
  int64_t Tk;                   // number of assignments (rows of h / o)
  int* tile_ctr;                // tiled schedule: 8 per-XCD tile-claim counters, zero at
                                // launch (NULL: static round-robin); unused by the stream path
  int out_bf16;                 // plain tiled GEMM only: 1 = bf16 result, 0 = FP32
  int m_tiles;                  // tiled schedule, one matrix (E = 1): token tiles to split the
                                // rows over (0: ceil(rows / tile height)); set by the launcher
};
// Decode-size batches: every weight row is streamed once per <= 16*mt tokens.
hipError_t launch_gateup_stream(hipStream_t s, const GroupedArgs& a, int64_t T, int k);
hipError_t launch_down_stream(hipStream_t s, const GroupedArgs& a, int64_t T, int k);
// Prefill-size batches: LDS-staged tiles on MFMA, persistent XCD-aware schedule.
hipError_t launch_gateup_tiled(hipStream_t s, const GroupedArgs& a, int num_cu);
hipError_t launch_down_tiled(hipStream_t s, const GroupedArgs& a, int num_cu);
// Token-tile count for one matrix (E = 1) over exactly `rows` rows (GroupedArgs::m_tiles).
int tiled_token_tiles(int64_t rows, int N, int MAT, int num_cu);
// ---- attention sublayer (attention.hip) ----
constexpr int kAttnQHeads = 48, kAttnKVHeads = 8, kAttnHeadDim = 128;
constexpr int kAttnProjRows = 2 * kAttnQHeads * kAttnHeadDim + 2 * kAttnKVHeads * kAttnHeadDim;  // q,k,v,gate
struct AttnArgs {
  int64_t T;
  int H;
  int global_layer;             // 1: no RoPE, query scaling; 0: RoPE, sliding window
  int window;                   // keys j with i - window < j <= i (sliding-window layers)
  float theta;                  // RoPE base
  const uint16_t* u;            // [T, H] bf16 layer input
  const uint16_t* w_qkvg;       // packed [Wq; Wk; Wv; Wg] ([14336, H], one expert)
  const uint16_t* w_o;          // packed Wo ([H, 6144])
  uint16_t* y;                  // [T, H] bf16 out
  // workspace
  float* qkvg;                  // [T, 14336] fp32
  uint16_t* qn;                 // [48][Tp][128], Tp = T rounded up to 128
  uint16_t* kn;                 // [8][Tp][128]
  uint16_t* vb;                 // [T][1024]
  uint16_t* vt;                 // [8][128][Tp] FP16, scaled per kv head
  uint16_t* o;                  // [T][6144]
  float* vmx;                   // [T][8] largest |v| of each kv head per token
  int32_t* counts;              // [1]
  int32_t* offsets;             // [2]
  int32_t* tile_ctr;            // [32]
};
hipError_t launch_attn_proj(hipStream_t s, const AttnArgs& a, int num_cu);
hipError_t launch_attn_prep(hipStream_t s, const AttnArgs& a);   // q/k norm + position, v^T
hipError_t launch_attn_flash(hipStream_t s, const AttnArgs& a);  // attention + gate -> o
hipError_t launch_attn_out(hipStream_t s, const AttnArgs& a, int num_cu);

// Plain GEMM on the tiled kernel (one "expert" with every row): out[T, N] =
// act[T, K] (row-major bf16) x W^T, W packed; FP32 or bf16 out.
hipError_t launch_plain_tiled(hipStream_t s, const GroupedArgs& a, int num_cu);

// ---- combine / norms (combine.hip) ----
hipError_t launch_combine(hipStream_t s, const float* o, const int32_t* row_of, const float* w,
                          int T, int H, int k, uint16_t* y);
hipError_t launch_stream_init(hipStream_t s, const uint16_t* x, float* out, int64_t T, int H);
hipError_t launch_rmsnorm(hipStream_t s, const float* in, uint16_t* out, int64_t T, int H, float eps);
hipError_t launch_residual(hipStream_t s, const uint16_t* y, float* stream, int64_t T, int H,
                           float eps, int step);

}  // namespace beam
