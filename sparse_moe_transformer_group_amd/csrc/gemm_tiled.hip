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

constexpr int kMaxE = 512;
constexpr int kBW = 256;                 // weight rows per tile (8 MFMA row blocks of 32)
constexpr int kBK = 32;                  // k per pipeline step (64 bytes per row)
constexpr int kWBytes = kBW * kBK * 2;   // weight slab per step (16 KB)

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (raw access; word 3 is the
// gfx9-family raw-buffer format).  Accesses past the end read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Physical 16-byte chunk of logical chunk c (0..3) in 64-byte row `row`:
// XOR by ((row >> 1) ^ (row >> 2)) & 3 keeps the 8-lane and the 16-lane
// groups of ds_read_b128 conflict-free (32 or 64 banks).
__device__ __forceinline__ int rchunk(int row, int c) { return c ^ (((row >> 1) ^ (row >> 2)) & 3); }

// One direct-to-LDS 16-byte-per-lane buffer load: lane l's 16 bytes at
// rsrc + voff + soff land at LDS byte lds + 16 l.  Issued from inline asm so
// the compiler does not track it: its own wait insertion would otherwise
// order every later LDS read after all of these loads (it cannot tell the
// ring stages apart), draining the pipeline.  The k-loop orders them itself
// with an explicit vmcnt wait and a barrier.  No register is written.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t rs, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

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

// Workgroup tile: 256 weight rows x BM tokens, 4 waves; wave w owns tokens
// [w*BM/4, (w+1)*BM/4) of the tile (NB = BM/128 MFMA column blocks of 32)
// and all 256 weight rows (8 MFMA row blocks):
// gate/up (MAT = 2): blocks 0-3 = gate rows of features [f, f+128) and
// blocks 4-7 = the up rows of the same features, so SiLU(g)*u pairs sit in
// one lane; down (MAT = 1): 256 features.  Accumulators: 8 x NB 32x32 blocks.
//
// At prefill sizes an expert's weights feed only ~256 tokens, about 256
// FLOP per weight byte -- below MI355X's MFMA/HBM ridge -- so the tile is
// built to keep HBM busy.  Each k-step (32 wide) moves a 16 KB weight slab
// and each wave's BM/4 x 64-byte token slab straight into an LDS ring of
// STAGES stages with direct-to-LDS buffer loads -- no vector registers are
// spent on staging.  A wave instruction fills 16 rows x 64 bytes; lane l
// takes the 16-byte chunk that lands in physical slot l%4 of its row.  One
// wait + barrier per step publishes a stage and frees the one read a step
// earlier.  With PAIR = 2 loads go out two steps at a time, so each weight
// row sees back-to-back requests for 128 contiguous bytes.  Token blocks
// past the tile's last token skip their loads and MFMAs: the k-loop is
// specialised on the number of valid blocks (wave-uniform).  With OCC = 2
// two workgroups share a CU, so one's waits overlap the other's MFMAs.
//
// MFMA s (0..1) of a step uses 16-byte chunk 2s+g of each row for lane group
// g = l/32 of both operands.
template <int MAT, int BM, int STAGES, int PAIR, int OCC>
__global__ __launch_bounds__(256, OCC) void grouped_tiled_kernel(GroupedArgs a) {
  static_assert(BM == 128 || BM == 256, "4 waves x 32 or 64 tokens");
  static_assert(PAIR == 1 || (PAIR == 2 && STAGES == 4), "paired issue needs 4 stages");
  static_assert(STAGES >= 2 && STAGES * (kWBytes + BM * kBK * 2) <= 160 * 1024 - 4096, "LDS");
  constexpr int NB = BM / 128;                 // 32-token MFMA blocks per wave
  constexpr int TBytes = BM * kBK * 2;         // token slab per step
  constexpr int Stage = kWBytes + TBytes;
  constexpr int F = (MAT == 2) ? kBW / 2 : kBW;  // output features per tile
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
    if (e0 < E) c0 = NF * ((a.counts[e0] + BM - 1) / BM);
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
  const uint32_t wbytes = (uint32_t)N * (uint32_t)K * 2u;  // one expert matrix (< 2^31)
  const __amdgpu_buffer_rsrc_t rs_act = buf_rsrc(a.act, 0x7fffffffu);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)ring;

  // Per-lane byte offsets inside a stage (same for every stage).
  const int lrow = lane >> 2, lpc = lane & 3;  // DMA: row within a 16-row group, physical chunk
  const uint32_t a_rd = r * 64 + (rchunk(r, g) << 4);          // weight operand, s = 0, block 0
  const uint32_t a_rd1 = r * 64 + (rchunk(r, 2 + g) << 4);     // s = 1
  const uint32_t t_rd = kWBytes + wave * (TBytes / 4);         // this wave's token region

  for (int tile = lo + slot; tile < hi; tile += per_xcd) {
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
    const int mt_e = (n_e + BM - 1) / BM;
    const int rel = tile - __builtin_amdgcn_readfirstlane(s_start[e]);
    const int ftile = rel / mt_e, mtile = rel % mt_e;
    const int fbase = ftile * F;
    // The expert's tokens are split evenly over its mt_e token tiles (each at
    // most BM): sibling tiles of one weight tile then do equal work, run side
    // by side on one XCD (adjacent tile ids) and share the weight stream
    // through L2 instead of each reading it from HBM.
    const int m0 = (int)((int64_t)mtile * n_e / mt_e);
    const int m1 = (int)((int64_t)(mtile + 1) * n_e / mt_e);
    const int tw0 = __builtin_amdgcn_readfirstlane(m0 + wave * (BM / 4));  // this wave's first token
    const int nbv = max(0, min(NB, (m1 - tw0 + 31) / 32));             // its blocks holding a token

    // Weight DMA: wave instruction i (0..3) fills tile rows 64w + 16i .. +16.
    // Rows 0..127 of a gate/up tile are gate rows (waves 0, 1), 128..255 up rows.
    const __amdgpu_buffer_rsrc_t rs_w =
        buf_rsrc(((MAT == 2 && wave >= 2) ? a.w1 : a.w0) + (int64_t)e * N * K, wbytes);
    uint32_t woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wave + 16 * i + lrow;
      const int f = (MAT == 2) ? fbase + (row % F) : fbase + row;
      woff[i] = ((uint32_t)min(f, N - 1) * (uint32_t)K) * 2u + (rchunk(row, lpc) << 4);
    }
    // Token DMA: wave instruction i fills this wave's token rows 16i .. +16.
    uint32_t toff[2 * NB];
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      const int trow = 16 * i + lrow;
      const int tok = max(0, min(tw0 + trow, m1 - 1));
      const int rr = row0 + tok;
      const uint32_t src = a.sorted_tokens ? (uint32_t)a.sorted_tokens[rr] : (uint32_t)rr;
      toff[i] = src * (uint32_t)K * 2u + (rchunk(trow, lpc) << 4);
    }

    // k-loop and epilogue, specialised on the number of valid token blocks
    auto run = [&](auto NBVc) {
      constexpr int NBV = decltype(NBVc)::value;
      constexpr int LPS = 4 + 2 * NBV;  // direct-to-LDS loads per step and wave
      f32x16 acc[8][NB];
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[b][j][i] = 0.f;

      auto issue = [&](int kt) {  // loads of step kt into stage kt % STAGES
        const uint32_t st = ring_lds + (kt % STAGES) * Stage;
        const uint32_t so = (uint32_t)kt * (kBK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16(__builtin_amdgcn_readfirstlane(st + (64 * wave + 16 * i) * 64), woff[i], rs_w, so);
#pragma unroll
        for (int i = 0; i < 2 * NBV; ++i)
          dma16(__builtin_amdgcn_readfirstlane(st + t_rd + 16 * i * 64), toff[i], rs_act, so);
      };

      // Step s may load into the stage of step s-1 (fully read before the
      // barrier of step s-1), so loads run up to STAGES-1 steps ahead.  Issue
      // points are the steps s with s % PAIR == 0; each issues steps
      // s+STAGES-PAIR .. s+STAGES-1 (clamped to the last step, so every issue
      // point issues PAIR steps and the wait counts below stay exact).  Step
      // s+1 must have landed at the barrier of step s; the steps issued after
      // it are still allowed in flight: STAGES-2-(s % PAIR) of them.
      // Prologue: steps 0 .. STAGES-PAIR-1, step 0 published.
#pragma unroll
      for (int q = 0; q < STAGES - PAIR; ++q) issue(min(q, nk - 1));
      BEAM_STEP_BARRIER((STAGES - PAIR - 1) * LPS);

      // Operands of MFMA s of the step whose stage starts at sb.
      auto read_ops = [&](const unsigned char* sb, int s, uint4 (&af)[8], uint4 (&bf)[NB]) {
        const unsigned char* wa = sb + (s ? a_rd1 : a_rd);
#pragma unroll
        for (int b = 0; b < 8; ++b) af[b] = *reinterpret_cast<const uint4*>(wa + 2048 * b);
#pragma unroll
        for (int j = 0; j < NBV; ++j) bf[j] = *reinterpret_cast<const uint4*>(wa + t_rd + 2048 * j);
        __builtin_amdgcn_sched_barrier(0);  // reads go out before the MFMAs that follow
      };
      auto mfmas = [&](const uint4 (&af)[8], const uint4 (&bf)[NB]) {
#pragma unroll
        for (int j = 0; j < NBV; ++j)
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[b][j] = mfma32(af[b], bf[j], acc[b][j]);
      };

      // Software pipeline: the barrier publishing step kt+1 sits between
      // the two MFMA groups of step kt, so the reads of the next group are
      // always in flight while the current one runs.
      uint4 af0[8], bf0[NB], af1[8], bf1[NB];
      if constexpr (NBV > 0) read_ops(ring, 0, af0, bf0);
      auto kstep = [&](auto PHASE, int kt) {
        constexpr int ph = decltype(PHASE)::value;  // kt % PAIR
        const unsigned char* sb = ring + (kt % STAGES) * Stage;
        if constexpr (PAIR == 1) {
          // Single issue, spread over the MFMAs: step min(kt+STAGES-1, nk-1)
          // goes out one instruction every few MFMAs, so a full address queue
          // stalls this wave only briefly while its MFMAs keep the pipe busy.
          // Past the last step the clamp re-loads step nk-1 into its own
          // stage: identical bytes, so the readers of that stage see the same
          // values, and every step issues LPS loads (exact wait counts).
          const int ki = min(kt + STAGES - 1, nk - 1);
          const uint32_t st = ring_lds + (ki % STAGES) * Stage;
          const uint32_t so = (uint32_t)ki * (kBK * 2);
          auto dma_op = [&](int d) {
            if (d < 4) dma16(__builtin_amdgcn_readfirstlane(st + (64 * wave + 16 * d) * 64), woff[d], rs_w, so);
            else dma16(__builtin_amdgcn_readfirstlane(st + t_rd + 16 * (d - 4) * 64), toff[d - 4], rs_act, so);
          };
          if constexpr (NBV > 0) {
            read_ops(sb, 1, af1, bf1);
            constexpr int NM = 8 * NBV;
            constexpr int EVERY = NM / LPS > 0 ? NM / LPS : 1;
            int d = 0;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              acc[m % 8][m / 8] = mfma32(af0[m % 8], bf0[m / 8], acc[m % 8][m / 8]);
              if (m % EVERY == EVERY - 1 && d < LPS) {
                dma_op(d);
                ++d;
                __builtin_amdgcn_sched_barrier(0);
              }
            }
#pragma unroll
            for (; d < LPS; ++d) dma_op(d);
          } else {
#pragma unroll
            for (int d = 0; d < LPS; ++d) dma_op(d);
          }
          // this wave's loads of step kt+1 have landed and its reads of stage
          // kt are done; after the barrier, the same holds for every wave
          BEAM_STEP_BARRIER((STAGES - 2) * LPS);
        } else {
          const bool issued = kt - ph + STAGES - PAIR < nk;  // this step's issue point issued
          if (ph == 0 && issued) {
#pragma unroll
            for (int q = STAGES - PAIR; q < STAGES; ++q) issue(min(kt + q, nk - 1));
          }
          if constexpr (NBV > 0) {
            read_ops(sb, 1, af1, bf1);
            mfmas(af0, bf0);
          }
          if (issued) BEAM_STEP_BARRIER((STAGES - 2 - ph) * LPS);
          else BEAM_STEP_BARRIER(0);
        }
        if constexpr (NBV > 0) {
          // next step's first operands (after the last step: a stale stage, unused)
          read_ops(ring + ((kt + 1) % STAGES) * Stage, 0, af0, bf0);
          mfmas(af1, bf1);
        }
      };
      int kt = 0;
      if constexpr (PAIR == 2) {
        for (; kt + 2 <= nk; kt += 2) {
          kstep(std::integral_constant<int, 0>{}, kt);
          kstep(std::integral_constant<int, 1>{}, kt + 1);
        }
        if (kt < nk) kstep(std::integral_constant<int, 0>{}, kt);
      } else {
        for (; kt < nk; ++kt) kstep(std::integral_constant<int, 0>{}, kt);
      }
      BEAM_STEP_BARRIER(0);  // drain the clamped prefetches; the next tile may refill the ring

      // Epilogue: acc[b][j][i] is row 8*(i/4) + 4*g + (i%4) of weight block
      // b, token tw0 + 32*j + r.
#pragma unroll
      for (int j = 0; j < NBV; ++j) {
        const int tok = tw0 + 32 * j + r;
        if (tok >= m1) continue;
        const int64_t row = row0 + tok;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if constexpr (MAT == 2) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int f = fbase + 32 * b + 8 * q4 + 4 * g;
              if (f >= N) continue;
              uint32_t p[4];
#pragma unroll
              for (int c = 0; c < 4; ++c)
                p[c] = f32_to_bf16_rne(swiglu(acc[b][j][4 * q4 + c], acc[b + 4][j][4 * q4 + c]));
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + f) =
                  make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
            }
          } else {
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              const int f = fbase + 32 * b + 8 * q4 + 4 * g;
              if (f >= N) continue;
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * N + f) =
                  f32x4{acc[b][j][4 * q4], acc[b][j][4 * q4 + 1], acc[b][j][4 * q4 + 2],
                        acc[b][j][4 * q4 + 3]};
            }
          }
        }
      }
    };  // run
    if constexpr (NB == 2) {
      if (nbv == 2) run(std::integral_constant<int, 2>{});
      else if (nbv == 1) run(std::integral_constant<int, 1>{});
      else run(std::integral_constant<int, 0>{});
    } else {
      if (nbv == 1) run(std::integral_constant<int, 1>{});
      else run(std::integral_constant<int, 0>{});
    }
  }
}

// Tile configuration: BM tokens per tile, ring depth, issue pairing,
// workgroups per CU.
#ifndef BEAM_TILED_CFG
#define BEAM_TILED_CFG 256, 4, 1, 1
#endif

template <int MAT, int BM, int STAGES, int PAIR, int OCC>
static hipError_t launch_tiled_cfg(hipStream_t st, const GroupedArgs& a, int num_cu) {
  const int nwg = ((num_cu * OCC + 7) / 8) * 8;  // persistent grid, a multiple of the 8 XCDs
  hipLaunchKernelGGL((grouped_tiled_kernel<MAT, BM, STAGES, PAIR, OCC>), dim3(nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled_cfg<2, BEAM_TILED_CFG>(st, a, num_cu);
}

hipError_t launch_down_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled_cfg<1, BEAM_TILED_CFG>(st, a, num_cu);
}

}  // namespace beam
