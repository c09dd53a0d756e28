// Grouped expert GEMMs of the Beam MoE block on gfx950 MFMA.
//
// Every expert is a SwiGLU MLP, hidden 5120 -> intermediate 2560 -> hidden
// (page "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen, anpassen
// und skalieren können", section "Mixture of Experts"); the SwiGLU product is
// formed in FP32 (same page, section "Residual Stream").
//
//   gate/up:  h[row, n] = bf16( SiLU(sum_k Wg[e,n,k] x[tok,k]) * sum_k Wu[e,n,k] x[tok,k] )
//   down:     o[row, n] = sum_k Wd[e,n,k] h[row,k]                       (FP32 out)
// where row runs over the expert-major rows of expert e and tok is the token
// of that row.  Weights are the MFMA A operand, tokens the B operand; both
// are K-contiguous.
//
// This file: the tiled schedule, for prefill-size batches, on 32x32x16
// MFMAs.  A persistent grid walks the (expert, feature tile, token tile)
// space in XCD-contiguous ranges; weight and token slabs go straight from
// memory into a 4-stage LDS ring with direct-to-LDS buffer loads.  The
// decode-size schedule is in gemm_stream.hip.
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace beam {


// ===========================================================================
// Tiled schedule
// ===========================================================================
// One 32x32x16 bf16 MFMA (gfx950): lane l supplies row (l % 32) of A and
// column (l % 32) of B with the 8 k-values of its k-group (l / 32); result
// element i of lane l is row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The same MFMA with its accumulator pinned to 16 architectural VGPRs.  A
// wave has 256 accumulation registers (AGPRs); a tile of 320 tokens needs 320
// accumulators per lane, so token blocks 8 and 9 accumulate in VGPRs through
// the VGPR form of the instruction.  (Left to itself the register allocator
// shuttles accumulators between the two files every k-step.)  The compiler
// does not see the MFMA behind the asm, so the caller covers the hazards it
// would have covered: no VALU write of an operand right before it (operands
// come from LDS reads or from conversions that precede a run of builtin
// MFMAs) and a wait-state pad before any VALU read of the result.
typedef unsigned int u32x4e __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x16 mfma32_vacc(uint4 a, uint4 b, f32x16 c) {
  const u32x4e av = __builtin_bit_cast(u32x4e, a), bv = __builtin_bit_cast(u32x4e, b);
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(av), "v"(bv));
  return c;
}
// FP8 (E4M3) -> bf16 of 8 weights (exact), as volatile asm: volatile asm
// keeps its place among the k-loop's other volatile asm (the direct-to-LDS
// loads), so the conversion stays where it is put instead of being hoisted
// next to the LDS read it waits on.  Byte 2i+h of the input is element 2i+h.
// The trailing s_nop covers a VALU write -> MFMA operand read that follows.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8_pinned(uint2 v) {
  uint4 o;
  asm volatile(
      "v_cvt_scalef32_pk_bf16_fp8 %0, %4, 1.0\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %1, %4, 1.0 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %2, %5, 1.0\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %3, %5, 1.0 op_sel:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(o.x), "=&v"(o.y), "=&v"(o.z), "=&v"(o.w)
      : "v"(v.x), "v"(v.y));
  return o;
}

// Wait states between the last VGPR-accumulator MFMA and a VALU read of its
// result (more than the 8-pass XDL write -> VALU read requirement).
__device__ __forceinline__ void mfma_vacc_drain(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

constexpr int kMaxE = 512;
constexpr int kBW = 256;                 // weight rows per tile (8 MFMA row blocks of 32)
constexpr int kBK = 32;                  // k per pipeline step (64 bytes per row)
static_assert(kBK == kPackK && kBW == 2 * kPackRows, "a k-step is one packed k-block");
constexpr int kWBytes = kBW * kBK * 2;   // weight slab per step (16 KB)

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Physical 16-byte chunk of logical chunk c (0..3) in 64-byte row `row`:
// XOR by ((row >> 1) ^ (row >> 2)) & 3 keeps the 8-lane and the 16-lane
// groups of ds_read_b128 conflict-free (32 or 64 banks).
__device__ __forceinline__ int rchunk(int row, int c) { return c ^ pack_swz(row); }


// Wait for this wave's direct-to-LDS loads of the current step (at most N
// younger ones outstanding) and for its LDS reads, then a workgroup barrier
// that does not wait for anything else (__syncthreads() would also drain the
// prefetch pipeline through its release fence).
// The scheduling barriers keep the compiler from moving MFMAs (which touch
// no memory) across it: work meant to overlap the wait stays in front.
#define BEAM_STEP_BARRIER(N)                                                    \
  do {                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                          \
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");        \
    __builtin_amdgcn_s_barrier();                                               \
    asm volatile("" ::: "memory");                                              \
    __builtin_amdgcn_sched_barrier(0);                                          \
  } while (0)

// Workgroup tile: 256 weight rows x up to BM = 320 tokens of one expert, 4 waves.
// Wave w owns 64 weight rows and every token of the tile, so the MFMA work
// of a tile is proportional to its token blocks (32 tokens each) and equal on
// the 4 SIMDs:
//   gate/up (MAT = 2): wave w holds the gate rows (block 0) and the up rows
//     (block 1) of features [f0 + 32w, f0 + 32w + 32), so SiLU(g)*u pairs sit
//     in one lane; a tile covers 128 features;
//   down (MAT = 1): rows [f0 + 64w, f0 + 64w + 64); a tile covers 256;
//   plain GEMM (MAT = 0): the down layout of one weight matrix over
//     row-major token rows (the attention projections): FP32 or bf16 out.
// Accumulators: 2 x NB blocks of 32x32 FP32 (NB = token blocks, 1..10);
// blocks 0..7 in AGPRs, blocks 8 and 9 in VGPRs.  320 tokens cover every
// expert of a near-uniform 8192-token batch (200 to 300 tokens each) with
// one tile, so no expert's weights are streamed into two CUs: what bounds
// this kernel is the rate at which one CU's direct-to-LDS loads complete,
// and two half-full tiles move 1.4x the bytes of one full tile per FLOP.
//
// At prefill sizes an expert's weights feed only ~256 tokens, about 256
// FLOP per weight byte -- near MI355X's MFMA/HBM ridge -- so the tile is
// built to keep HBM busy.  Each k-step (32 wide) moves the 16 KB weight slab
// and the tile's token slab (64 bytes per token) straight into an LDS ring of
// STAGES stages with direct-to-LDS buffer loads -- no vector registers are
// spent on staging.  A load instruction fills 16 rows x 64 bytes; lane l
// takes the 16-byte chunk that lands in physical slot l%4 of its row.  The
// loads of a step go out one instruction every few MFMAs of an earlier step
// (a full address queue then stalls a wave only briefly while its MFMAs keep
// the pipe busy).  One wait + barrier per step publishes a stage and frees
// the one read a step earlier.
//
// MFMA s (0..1) of a step uses 16-byte chunk 2s+g of each row for lane group
// g = l/32 of both operands.
//
// W8: FP8 (E4M3) weights with per-row scales.  The weight slab of a step is
// 8 KB (32 bytes per row, two 1 KB loads per wave), so a stage is 28 KB and
// the ring one stage deeper; an MFMA weight operand is an 8-byte LDS read
// converted to bf16 in registers (exactly), and the row scales multiply the
// FP32 accumulators in the epilogue.
template <int MAT, int BM, int STAGES, int OCC, bool W8>
__global__ __launch_bounds__(256, OCC) void grouped_tiled_kernel(GroupedArgs a) {
  static_assert(BM == 256 || BM == 320, "tokens per tile");
  constexpr int WB = W8 ? kWBytes / 2 : kWBytes;  // weight slab per step
  constexpr int TBytes = BM * kBK * 2;         // token slab per step
  constexpr int Stage = WB + TBytes;
  constexpr int F = (MAT == 2) ? kBW / 2 : kBW;  // output features per tile
  static_assert(STAGES >= 3 && STAGES * Stage <= 160 * 1024 / OCC - 4096, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * Stage];
  __shared__ int s_start[kMaxE + 1];
  __shared__ int s_scan[256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = lane & 31, g = lane >> 5;
  const int N = a.N, K = a.K, E = a.E;
  const int NF = (N + F - 1) / F;

  // Tile prefix over experts: expert e owns NF * ceil(n_e / BM) tiles.
  {
    const int e0 = tid * 2;
    int c0 = 0, c1 = 0;
    if (e0 < E) c0 = NF * (a.m_tiles > 0 ? a.m_tiles : (a.counts[e0] + BM - 1) / BM);
    if (e0 + 1 < E) c1 = NF * ((a.counts[e0 + 1] + BM - 1) / BM);
    s_scan[tid] = c0 + c1;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int v = (tid >= off) ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int incl = s_scan[tid];
    if (e0 < E) s_start[e0] = incl - c0 - c1;
    if (e0 + 1 < E) s_start[e0 + 1] = incl - c1;
    if (tid == 255) s_start[E] = incl;
    __syncthreads();
  }
  const int total = s_start[E];
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = nwg >> 3;
  const int span = (total + 7) / 8;
  const int lo = xcd * span, hi = min(total, lo + span);
  const int nk = K / kBK;
  const uint32_t wbytes =  // one packed expert matrix (< 2^31)
      (uint32_t)(W8 ? packed8_expert_bytes(N, K) : packed_expert_bytes(N, K));
  const __amdgpu_buffer_rsrc_t rs_act = buf_rsrc(a.act, 0x7fffffffu);
  const uint32_t tk64 = (uint32_t)a.Tk * 64u;  // one k-block of the k-major h
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)ring;

  // Per-lane byte offsets inside a stage (same for every stage).  The chunk
  // swizzle depends on the row's low bits only, so it is the same for row r
  // of every 32-row block.
  const int lrow = lane >> 2, lpc = lane & 3;  // DMA: row within a 16-row group, physical chunk
  const uint32_t c_rd0 = r * 64 + (rchunk(r, g) << 4);      // MFMA s = 0, row r of a block
  const uint32_t c_rd1 = r * 64 + (rchunk(r, 2 + g) << 4);  // MFMA s = 1
  const uint32_t c8_rd0 = r * 32 + ((g ^ pack8_swz(r)) << 3);        // FP8 weights, s = 0
  const uint32_t c8_rd1 = r * 32 + (((2 + g) ^ pack8_swz(r)) << 3);  // s = 1
  const uint32_t w_base = wave * (WB / 4);                   // this wave's 64 weight rows

  // Tiles of an XCD's range go to its workgroups in order.  With a claim
  // counter (one per XCD, zero at launch) each workgroup takes the next
  // unclaimed tile when it starts one, so the 32 CUs of an XCD always work on
  // neighbouring tiles -- the feature tiles of one expert, which read the
  // same token slab -- however unequal the tiles are; without one, workgroup
  // `slot` takes every per_xcd-th tile.  The next tile is claimed at the start
  // of the current one, hiding the atomic's latency.
  int* const ctr = a.tile_ctr ? a.tile_ctr + xcd : nullptr;
  __shared__ int s_tile;
  int tile = lo + slot;
  if (ctr) {
    if (tid == 0) s_tile = lo + __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(s_tile);
  }
  while (tile < hi) {
    int next = tile + per_xcd;
    if (ctr && tid == 0)
      next = lo + __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // expert: largest e with s_start[e] <= tile
    int elo = 0, ehi = E - 1;
    while (elo < ehi) {
      const int mid = (elo + ehi + 1) >> 1;
      if (s_start[mid] <= tile) elo = mid;
      else ehi = mid - 1;
    }
    // tile coordinates are wave-uniform: keep them in scalar registers so the
    // k-loop has no divergent branches
    const int e = __builtin_amdgcn_readfirstlane(elo);
    const int n_e = __builtin_amdgcn_readfirstlane(a.counts[e]);
    const int row0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
    const int mt_e = a.m_tiles > 0 ? a.m_tiles : (n_e + BM - 1) / BM;
    const int rel = tile - __builtin_amdgcn_readfirstlane(s_start[e]);
    // Order of an expert's NF x mt_e tiles.  The 32 CUs of an XCD work on 32
    // consecutive tiles at a time, so consecutive tiles should share data in
    // L2: tiles of one feature tile share its weight slab, tiles of one token
    // tile share its token slab.  Experts with few token tiles (near-uniform
    // loads) go feature tile by feature tile, token tile fastest; for hot
    // experts (>= 8 token tiles) a run of 32 tiles is a 4 x 8 block of
    // feature x token tiles: 12 slabs per 32 tiles instead of 33.
    int ftile, mtile;
    {
      const int MB = min(mt_e, 8);
      const int chunk = rel / (MB * NF);                 // token-tile chunk
      const int m_lo = chunk * MB, mb = min(MB, mt_e - m_lo);
      const int r2 = rel - chunk * MB * NF;              // [0, mb * NF)
      const int FB = (MB >= 8) ? 4 : NF;                 // feature tiles per block
      const int grp = r2 / (FB * mb);
      const int r3 = r2 - grp * FB * mb;                 // [0, fb * mb)
      ftile = grp * FB + r3 / mb;
      mtile = m_lo + r3 % mb;
    }
    const int fbase = ftile * F;
    // The expert's tokens are split evenly over its mt_e token tiles (each at
    // most BM): sibling tiles of one weight tile then do equal work, run side
    // by side on one XCD (adjacent tile ids) and share the weight stream
    // through L2 instead of each reading it from HBM.
    const int m0 = __builtin_amdgcn_readfirstlane((int)((int64_t)mtile * n_e / mt_e));
    const int m1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(mtile + 1) * n_e / mt_e));
    const int nb = (m1 - m0 + 31) / 32;  // token blocks of the tile, 1..BM/32

    // Weight DMA from the packed layout: instruction i (0..3) copies 16 rows
    // x 64 bytes (1 KB, contiguous) of this wave's 128-row block into its
    // rows 16i .. 16i+15; the packed chunk order is already the LDS order.
    // Gate/up: rows 0..31 are gate rows, 32..63 the up rows of the same
    // features (block ftile, rows 32w ..); down: block 2*ftile + w/2, rows
    // 64*(w%2) ...  A block past the matrix (odd block count, down) reads
    // as zeros through the buffer bounds.
    const int fw = (MAT == 2) ? fbase + 32 * wave : fbase + 64 * wave;  // this wave's first feature
    const char* wexp0 = reinterpret_cast<const char*>(a.w0) + (int64_t)e * wbytes;
    const char* wexp1 = reinterpret_cast<const char*>(MAT == 2 ? a.w1 : a.w0) + (int64_t)e * wbytes;
    const __amdgpu_buffer_rsrc_t rs_w0 = buf_rsrc(wexp0, wbytes);
    const __amdgpu_buffer_rsrc_t rs_w1 = buf_rsrc(wexp1, wbytes);
    // FP8: load d (0, 1) copies 32 rows x 32 bytes (1 KB): gate/up rows 32w
    // of the gate (d = 0) or up (d = 1) block; down rows 64(w%2) + 32d.
    constexpr int WPW = W8 ? 2 : 4;  // weight loads per step and wave
    uint32_t woff[WPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int blk = (MAT == 2) ? ftile : 2 * ftile + (wave >> 1);
      if constexpr (W8) {
        const int brow = (MAT == 2) ? 32 * wave : 64 * (wave & 1) + 32 * i;
        woff[i] = ((uint32_t)blk * (uint32_t)nk * kPackRows + (uint32_t)brow) * 32u + lane * 16u;
      } else {
        const int brow = (MAT == 2) ? 32 * wave + 16 * (i & 1) : 64 * (wave & 1) + 16 * i;
        woff[i] = ((uint32_t)blk * (uint32_t)nk * kPackRows + (uint32_t)brow) * 64u + lane * 16u;
      }
    }

    // k-loop and epilogue, specialised on the number of token blocks
    auto run = [&](auto NBc) {
      constexpr int NB = decltype(NBc)::value;
      // Token DMA: 2*NB instructions of 16 rows, instruction 4q + w issued
      // by wave w; every wave issues TPW of them (rows past the tile's last
      // token load that token again and are never read).
      constexpr int TPW = (2 * NB + 3) / 4;
      constexpr int LPS = WPW + TPW;  // direct-to-LDS loads per step and wave
      uint32_t toff[TPW];
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int trow = 16 * (4 * q + wave) + lrow;
        const int tok = min(m0 + trow, m1 - 1);
        const int rr = row0 + tok;
        if constexpr (MAT != 1) {
          // x rows (row-major, gathered through sorted_tokens; in order when
          // there is no indirection)
          const uint32_t src = a.sorted_tokens ? (uint32_t)a.sorted_tokens[rr] : (uint32_t)rr;
          toff[q] = src * (uint32_t)K * 2u + (rchunk(trow, lpc) << 4);
        } else {
          // h in k-major order (written so by the gate/up epilogue): row rr
          // of k-block kb at (kb * Tk + rr) * 64, chunks swizzled by rr; the
          // lane fetches the chunk that belongs in LDS slot lpc of row trow.
          toff[q] = (uint32_t)rr * 64u + ((lpc ^ pack_swz(trow) ^ pack_swz(rr)) << 4);
        }
      }

      f32x16 acc[2][NB];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[b][j][i] = 0.f;
      // VGPR accumulators: materialise the zeros, then pad the VALU write ->
      // MFMA srcC read before the first asm MFMA (volatile asm keeps order)
      if constexpr (NB > 8) {
#pragma unroll
        for (int j = 8; j < NB; ++j) {
          asm volatile("" : "+v"(acc[0][j]));
          asm volatile("" : "+v"(acc[1][j]));
        }
        asm volatile("s_nop 4");
      }

      auto dma_op = [&](int d, uint32_t st, uint32_t so) {
        if (d < WPW) {  // weights: k-block kt of the packed block (so = kt * 64)
          if constexpr (W8)
            dma16(__builtin_amdgcn_readfirstlane(st + w_base + 1024 * d), woff[d],
                  (MAT == 2 && d == 1) ? rs_w1 : rs_w0, so * (kPack8BlockBytes / (kBK * 2)));
          else
            dma16(__builtin_amdgcn_readfirstlane(st + w_base + 16 * d * 64), woff[d],
                  (MAT == 2 && d >= 2) ? rs_w1 : rs_w0, so * (kPackBlockBytes / (kBK * 2)));
        } else {  // tokens: x step offset kt * 64, or k-major h block kt * Tk * 64
          dma16(__builtin_amdgcn_readfirstlane(st + WB + 16 * (4 * (d - WPW) + wave) * 64),
                toff[d - WPW], rs_act, (MAT != 1) ? so : (so >> 6) * tk64);
        }
      };
      auto issue = [&](int kt) {  // loads of step kt into stage kt % STAGES
        const uint32_t st = ring_lds + (kt % STAGES) * Stage;
        const uint32_t so = (uint32_t)kt * (kBK * 2);
#pragma unroll
        for (int d = 0; d < LPS; ++d) dma_op(d, st, so);
      };

      // Step s may load into the stage of step s-1 (fully read before the
      // barrier of step s-1), so loads run STAGES-1 steps ahead.  Step
      // min(s+STAGES-1, nk-1) goes out during step s: past the last step the
      // clamp re-loads step nk-1 into its own stage (identical bytes, so its
      // readers see the same values), and every step issues LPS loads, which
      // keeps the wait counts exact.  Step s+1 must have landed at the
      // barrier of step s; the STAGES-2 steps issued after it may still be in
      // flight.  Prologue: steps 0 .. STAGES-2, step 0 published.
#pragma unroll
      for (int q = 0; q < STAGES - 1; ++q) issue(min(q, nk - 1));
      BEAM_STEP_BARRIER((STAGES - 2) * LPS);

      // Operands of MFMA s of the step whose stage starts at sb.
      // FP8 weights: the raw 8-byte codes are read here and converted to bf16
      // halfway through the MFMA group that precedes their use (to_bf16),
      // so the conversion never waits on a read that was just issued.
      auto read_ops = [&](const unsigned char* sb, int s, uint4 (&af)[2], uint2 (&ar)[2],
                          uint4 (&bf)[NB]) {
        const uint32_t c = s ? c_rd1 : c_rd0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if constexpr (W8)
            ar[b] = *reinterpret_cast<const uint2*>(sb + w_base + 1024 * b + (s ? c8_rd1 : c8_rd0));
          else
            af[b] = *reinterpret_cast<const uint4*>(sb + w_base + 2048 * b + c);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bf[j] = *reinterpret_cast<const uint4*>(sb + WB + 2048 * j + c);
        __builtin_amdgcn_sched_barrier(0);  // reads go out before the MFMAs that follow
      };

      // Software pipeline: the barrier publishing step kt+1 sits between
      // the two MFMA groups of step kt, so the reads of the next group are
      // always in flight while the current one runs.
      uint4 af0[2], bf0[NB], af1[2], bf1[NB];
      uint2 ar0[2], ar1[2];
      auto to_bf16 = [&](uint4 (&af)[2], const uint2 (&ar)[2]) {
        if constexpr (W8) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int b = 0; b < 2; ++b) af[b] = fp8x8_to_bf16x8_pinned(ar[b]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      read_ops(ring, 0, af0, ar0, bf0);
      to_bf16(af0, ar0);
      for (int kt = 0; kt < nk; ++kt) {
        // stage offsets pass through readfirstlane: it keeps the compiler from
        // strength-reducing kt % STAGES (STAGES = 5) into one loop-carried
        // address per token block, which spills and then makes every step
        // wait for all loads in flight (its wait counts do not see the
        // direct-to-LDS loads); each read is then base + immediate offset
        const unsigned char* sb = ring + __builtin_amdgcn_readfirstlane((kt % STAGES) * Stage);
        const int ki = min(kt + STAGES - 1, nk - 1);
        const uint32_t st = ring_lds + (ki % STAGES) * Stage;
        const uint32_t so = (uint32_t)ki * (kBK * 2);
        read_ops(sb, 1, af1, ar1, bf1);
        {
          constexpr int NM = 2 * NB;
          constexpr int EVERY = NM / LPS > 0 ? NM / LPS : 1;
          int d = 0;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            if ((m >> 1) >= 8)
              acc[m & 1][m >> 1] = mfma32_vacc(af0[m & 1], bf0[m >> 1], acc[m & 1][m >> 1]);
            else
              acc[m & 1][m >> 1] = mfma32(af0[m & 1], bf0[m >> 1], acc[m & 1][m >> 1]);
            if (m == NM / 2 - 1) to_bf16(af1, ar1);
            if (m % EVERY == EVERY - 1 && d < LPS) {
              dma_op(d, st, so);
              ++d;
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (; d < LPS; ++d) dma_op(d, st, so);
        }
        // this wave's loads of step kt+1 have landed and its reads of stage
        // kt are done; after the barrier, the same holds for every wave
        BEAM_STEP_BARRIER((STAGES - 2) * LPS);
        // next step's first operands (after the last step: a stale stage, unused)
        read_ops(ring + __builtin_amdgcn_readfirstlane(((kt + 1) % STAGES) * Stage), 0, af0, ar0, bf0);
#pragma unroll
        for (int m = 0; m < 2 * NB; ++m) {
          if ((m >> 1) >= 8)
            acc[m & 1][m >> 1] = mfma32_vacc(af1[m & 1], bf1[m >> 1], acc[m & 1][m >> 1]);
          else
            acc[m & 1][m >> 1] = mfma32(af1[m & 1], bf1[m >> 1], acc[m & 1][m >> 1]);
          if (m == NB - 1) to_bf16(af0, ar0);
        }
      }
      BEAM_STEP_BARRIER(0);  // drain the clamped prefetches; the next tile may refill the ring
#pragma unroll
      for (int j = 8; j < NB; ++j) {
        mfma_vacc_drain(acc[0][j]);
        mfma_vacc_drain(acc[1][j]);
      }

      // Epilogue: acc[b][j][i] is row 8*(i/4) + 4*g + (i%4) of this wave's
      // weight block b, token m0 + 32*j + r.  The lane coordinates are
      // recomputed here (lane_here) and the FP8 row scales are loaded before
      // the first store: a load issued after stores (a spill reload
      // included) waits for all of them.
      const int ln = lane_here();
      const int er = ln & 31, eg = ln >> 5;
      if constexpr (MAT == 2) {
      f32x4 sg[4], su[4];  // FP8 row scales of the lane's 4 x 4 gate and up rows
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        sg[q4] = f32x4{1.f, 1.f, 1.f, 1.f};
        su[q4] = sg[q4];
        const int f = fw + 8 * q4 + 4 * eg;
        if constexpr (W8) {
          if (f < N) {
            sg[q4] = *reinterpret_cast<const f32x4*>(a.s0 + (int64_t)e * N + f);
            su[q4] = *reinterpret_cast<const f32x4*>(a.s1 + (int64_t)e * N + f);
          }
        }
      }
      // one wait for the scales here, on every path, rather than one in
      // front of each guarded store block
      if constexpr (W8) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) asm volatile("" ::"v"(sg[q4]), "v"(su[q4]));
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int tok = m0 + 32 * j + er;
        if (tok >= m1) continue;
        const int64_t row = row0 + tok;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // h k-major: feature f of row `row` sits in k-block f/32, chunk
          // (f%32)/8 (swizzled by the row), element f%8; the 4 features
          // f..f+3 share one chunk.
          const int f = fw + 8 * q4 + 4 * eg;
          if (f >= N) continue;
          float h4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            h4[c] = swiglu(acc[0][j][4 * q4 + c] * sg[q4][c], acc[1][j][4 * q4 + c] * su[q4][c]);
          const int64_t off = ((int64_t)(f >> 5) * a.Tk + row) * 32 +
                              ((((f & 31) >> 3) ^ pack_swz((int)row)) << 3) + (f & 7);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
              make_uint2(pack_bf16x2_rne(h4[0], h4[1]), pack_bf16x2_rne(h4[2], h4[3]));
        }
      }
      } else {
        // Down: a tile's output row is 256 contiguous FP32 features (1 KB) per
        // token.  Each 32-token block is staged through LDS so that one store
        // instruction writes one whole row (64 lanes x 16 B) rather than 32
        // rows x 32 B.  Two staging areas alternate in the idle ring, so one
        // barrier per block keeps writers of block j+2 behind the readers of
        // block j; rows are padded by 16 B so the column writes of a wave
        // spread over all banks.
        constexpr int RS = 1024 + 16;  // staging row stride, bytes
        static_assert(2 * 32 * RS <= STAGES * Stage, "staging fits the ring");
        f32x4 sd[2][4];  // FP8 row scales of the lane's features (1 past N)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            sd[b][q4] = f32x4{1.f, 1.f, 1.f, 1.f};
            const int f = fbase + 64 * wave + 32 * b + 8 * q4 + 4 * eg;
            if constexpr (W8) {
              if (f < N) sd[b][q4] = *reinterpret_cast<const f32x4*>(a.s0 + (int64_t)e * N + f);
            }
          }
        if constexpr (W8) {  // one wait for the scales, on every path
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) asm volatile("" ::"v"(sd[b][q4]));
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          unsigned char* stg = ring + (j & 1) * (32 * RS);
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int fl = 64 * wave + 32 * b + 8 * q4 + 4 * eg;  // feature within the tile
              f32x4 v = f32x4{acc[b][j][4 * q4], acc[b][j][4 * q4 + 1], acc[b][j][4 * q4 + 2],
                              acc[b][j][4 * q4 + 3]};
              if constexpr (W8) v *= sd[b][q4];
              *reinterpret_cast<f32x4*>(stg + er * RS + fl * 4) = v;
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          const int f = fbase + 4 * ln;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int rr = 8 * wave + i;  // token of the block, wave-uniform
            const int tok = m0 + 32 * j + rr;
            if (tok < m1 && f < N) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rr * RS + ln * 16);
              const int64_t at = (int64_t)(row0 + tok) * N + f;
              if (a.out_bf16)  // plain GEMM with a bf16 result (one RNE per value)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + at) =
                    make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
              else
                *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + at) = v;
            }
          }
        }
        // every wave is done with the staging rows before the next tile's
        // loads refill the ring
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    };  // run
    if constexpr (BM == 320) {
      switch (nb) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        case 8: run(std::integral_constant<int, 8>{}); break;
        case 9: run(std::integral_constant<int, 9>{}); break;
        default: run(std::integral_constant<int, 10>{}); break;
      }
    } else {
      switch (nb) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        default: run(std::integral_constant<int, 8>{}); break;
      }
    }
    if (ctr) {  // hand thread 0's claim to the workgroup (LDS only: the h stores may stay in flight)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();  // every wave has read s_tile of this tile
      asm volatile("" ::: "memory");
      if (tid == 0) s_tile = next;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      next = s_tile;
    }
    tile = __builtin_amdgcn_readfirstlane(next);
  }
}

// Tile configuration: tokens per tile, ring depth, workgroups per CU.
#ifndef BEAM_TILED_CFG
#define BEAM_TILED_CFG 320, 4, 1
#endif

// FP8 weights (recognised by their row scales) use a 5-stage ring of 28 KB.
#ifndef BEAM_TILED_FP8_STAGES
#define BEAM_TILED_FP8_STAGES 5
#endif

template <int MAT, bool W8, int BM, int STAGES, int OCC>
static hipError_t launch_tiled_cfg(hipStream_t st, const GroupedArgs& a, int num_cu) {
  const int nwg = ((num_cu * OCC + 7) / 8) * 8;  // persistent grid, a multiple of the 8 XCDs
  hipLaunchKernelGGL((grouped_tiled_kernel<MAT, BM, STAGES, OCC, W8>), dim3(nwg), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

template <int MAT>
static hipError_t launch_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  if (a.s0) return launch_tiled_cfg<MAT, true, 320, BEAM_TILED_FP8_STAGES, 1>(st, a, num_cu);
  return launch_tiled_cfg<MAT, false, BEAM_TILED_CFG>(st, a, num_cu);
}

hipError_t launch_gateup_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<2>(st, a, num_cu);
}

hipError_t launch_down_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<1>(st, a, num_cu);
}

#ifndef BEAM_PLAIN_CFG
#define BEAM_PLAIN_CFG BEAM_TILED_CFG
#endif
template <int BM, int STAGES, int OCC>
struct PlainBM {
  static constexpr int value = BM;
};

// Token tiles of a one-matrix GEMM over T rows: the count mt (tiles of
// ceil(T / mt) rows or one fewer, at most BM) that minimises the persistent
// grid's rounds times the tile height, each tile also costing a fixed
// overhead worth about one 32-row block (prologue, epilogue).
static int plain_token_tiles(int64_t T, int NF, int nwg, int bm) {
  const int lo = (int)((T + bm - 1) / bm), hi = (int)std::min<int64_t>((T + 31) / 32, 4 * lo + 64);
  int best = lo;
  int64_t best_cost = INT64_MAX;
  for (int mt = lo; mt <= hi; ++mt) {
    const int64_t rounds = ((int64_t)NF * mt + nwg - 1) / nwg;
    const int64_t blocks = ((T + mt - 1) / mt + 31) / 32;
    const int64_t cost = rounds * (blocks + 1);
    if (cost < best_cost) {
      best_cost = cost;
      best = mt;
    }
  }
  return best;
}

hipError_t launch_plain_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  GroupedArgs b = a;
  constexpr int kPlainBM = PlainBM<BEAM_PLAIN_CFG>::value;
  const int nwg = ((num_cu + 7) / 8) * 8;
  if (b.E == 1 && b.Tk > 0) b.m_tiles = plain_token_tiles(b.Tk, (b.N + kBW - 1) / kBW, nwg, kPlainBM);
  return launch_tiled_cfg<0, false, BEAM_PLAIN_CFG>(st, b, num_cu);
}

int tiled_token_tiles(int64_t rows, int N, int MAT, int num_cu) {
  const int F = (MAT == 2) ? kBW / 2 : kBW;
  const int nwg = ((num_cu + 7) / 8) * 8;
  return plain_token_tiles(rows, (N + F - 1) / F, nwg, 320);
}

}  // namespace beam
