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
// of that row.  Weights are the MFMA A operand (16 output features per
// block), tokens the B operand (16 tokens per block); both are K-contiguous,
// so each lane's operand is one 16-byte load.  A lane's results are 4
// consecutive features of one token, stored as one 8- or 16-byte vector.
//
// Two schedules share this arithmetic:
//  * stream: decode-size batches (a handful of tokens per expert).  Bound by
//    reading the active experts' weights once from HBM.  Each wave streams
//    its own weight rows straight into registers (64 contiguous bytes per
//    lane per step, 256 bytes per row segment, nontemporal loads since each
//    byte is used once), double-buffered, with the expert's tokens as up to
//    16*MT MFMA columns.  No LDS, no barriers.
//  * tiled: prefill-size batches, on 32x32x16 MFMAs.  Weight rows go straight
//    from L2 into registers (each is used by one wave only); the token tile,
//    shared by the 4 waves, is staged through LDS.  A persistent grid walks
//    the (expert, feature tile, token tile) space in XCD-contiguous ranges so
//    that the token tiles of one weight tile run back to back on one XCD and
//    share its L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace beam {

// ===========================================================================
// Stream schedule
// ===========================================================================
// MAT = 2: gate+up with SwiGLU epilogue (bf16 out); MAT = 1: down (fp32 out).
// RB  = 16-row weight blocks per wave per matrix; MT = 16-token tiles held.
//
// Each wave owns ROWS = MAT*RB*16 weight rows and walks K in steps of 128
// (256 bytes per row).  A step's weight slab (ROWS x 256 B) is read with
// fully coalesced nontemporal 16-byte loads, 16 lanes per row segment, so
// every load instruction covers whole cache lines; it is then re-laid into
// the MFMA operand layout through a wave-private LDS tile (16-byte chunks
// XOR-swizzled by row, conflict-free).  The next step's slab is in flight
// while the current one is multiplied.  Within a step, MFMA j (0..3) takes
// 16-byte chunk 4j+q of the row segment for lane group q; the token operand
// uses the same k mapping.
template <int MAT, int RB, int MT>
__global__ __launch_bounds__(256) void grouped_stream_kernel(GroupedArgs a) {
  constexpr int ROWS = MAT * RB * 16;
  constexpr int LD = ROWS / 4;  // 16-byte loads per lane per step (4 rows per wave load)
  __shared__ __attribute__((aligned(16))) unsigned char lds[4][ROWS * 256];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int e = blockIdx.y;
  const int n_e = a.counts[e];
  if (n_e <= 0) return;
  const int f0 = (blockIdx.x * 4 + wave) * (RB * 16);
  if (f0 >= a.N) return;  // no workgroup barriers in this kernel
  const int row0 = a.offsets[e];
  const int N = a.N, K = a.K;
  unsigned char* tile = lds[wave];

  // Load slot i of this lane: wave row rw = 4i + lane/16, 16-byte chunk lane%16.
  const uint16_t* lp[LD];
  int lo[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int rw = 4 * i + (lane >> 4);
    const int c = lane & 15;
    const int m = rw / (RB * 16);
    const int fr = rw % (RB * 16);
    const int f = min(f0 + fr, N - 1);
    const uint16_t* base = (m == 0) ? a.w0 : a.w1;
    lp[i] = base + ((int64_t)e * N + f) * K + c * 8;
    lo[i] = rw * 256 + ((c ^ (rw & 15)) << 4);
  }

  for (int c0 = 0; c0 < n_e; c0 += 16 * MT) {
    const uint16_t* bp[MT];
    bool bv[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tok = c0 + 16 * j + r;
      bv[j] = tok < n_e;
      const int rr = row0 + (bv[j] ? tok : 0);
      const int64_t src = a.sorted_tokens ? (int64_t)a.sorted_tokens[rr] : (int64_t)rr;
      bp[j] = a.act + src * K + q * 8;
    }
    f32x4 acc[MAT][RB][MT];
#pragma unroll
    for (int m = 0; m < MAT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = K / 128;  // K is a multiple of 64; a 64-wide tail is handled below
    uint4 R[LD];
    uint4 B[2][MT][4];
    auto load_w = [&](int ks) {
#pragma unroll
      for (int i = 0; i < LD; ++i) R[i] = ld16_nt(lp[i] + ks * 128);
    };
    auto load_b = [&](int buf, int ks) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          B[buf][t][j] = bv[t] ? ld16(bp[t] + ks * 128 + j * 32) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto step = [&](int buf, int ks) {
      // slab of step ks: registers -> LDS tile, then prefetch step ks+1
#pragma unroll
      for (int i = 0; i < LD; ++i) st16(tile + lo[i], R[i]);
      __builtin_amdgcn_wave_barrier();
      if (ks + 1 < nsteps) {
        load_w(ks + 1);
        load_b(buf ^ 1, ks + 1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int m = 0; m < MAT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const int rw = m * RB * 16 + i * 16 + r;
            const uint4 av = *reinterpret_cast<const uint4*>(tile + rw * 256 + (((4 * j + q) ^ r) << 4));
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[m][i][t] = mfma16(av, B[buf][t][j], acc[m][i][t]);
          }
      }
      __builtin_amdgcn_wave_barrier();
    };

    if (nsteps > 0) {
      load_w(0);
      load_b(0, 0);
    }
    int ks = 0;
    for (; ks + 2 <= nsteps; ks += 2) {
      step(0, ks);
      step(1, ks + 1);
    }
    if (ks < nsteps) step(0, ks);

    if (K % 128) {
      // 64-wide tail: ordinary loads straight into the operand layout; lane
      // group q covers k in [kt + 16q, kt + 16q + 16) as two 8-wide pieces.
      const int kt = nsteps * 128;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 bt[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t)
          bt[t] = bv[t] ? ld16(bp[t] - q * 8 + kt + q * 16 + c * 8) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int m = 0; m < MAT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const int f = min(f0 + 16 * i + r, N - 1);
            const uint16_t* base = (m == 0) ? a.w0 : a.w1;
            const uint4 at = ld16(base + ((int64_t)e * N + f) * K + kt + q * 16 + c * 8);
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[m][i][t] = mfma16(at, bt[t], acc[m][i][t]);
          }
      }
    }

    // Epilogue: lane holds features f0+16i+4q+c (c = 0..3) of token c0+16t+r.
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int f = f0 + 16 * i + 4 * q;
      if (f >= N) continue;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int tok = c0 + 16 * t + r;
        if (tok >= n_e) continue;
        const int64_t row = row0 + tok;
        if constexpr (MAT == 2) {
          uint32_t p[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) p[c] = f32_to_bf16_rne(swiglu(acc[0][i][t][c], acc[1][i][t][c]));
          uint2 v = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + f) = v;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * N + f) = acc[0][i][t];
        }
      }
    }
  }
}

// Token tiles held per pass: enough for the expected tokens per expert, so
// that the weights are usually streamed exactly once.
static int stream_mt(int64_t T, int k, int E) {
  const double avg = (double)T * k / E;
  if (avg <= 6.0) return 1;
  if (avg <= 16.0) return 2;
  return 4;
}

template <int MAT, int RB>
static hipError_t launch_stream(hipStream_t st, const GroupedArgs& a, int mt) {
  dim3 grid((a.N + 4 * RB * 16 - 1) / (4 * RB * 16), a.E), block(256);
  if (mt == 1) hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 1>), grid, block, 0, st, a);
  else if (mt == 2) hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 2>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 4>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gateup_stream(hipStream_t st, const GroupedArgs& a, int64_t T, int k) {
  return launch_stream<2, 1>(st, a, stream_mt(T, k, a.E));
}

hipError_t launch_down_stream(hipStream_t st, const GroupedArgs& a, int64_t T, int k) {
  return launch_stream<1, 2>(st, a, stream_mt(T, k, a.E));
}

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
constexpr int kBM = 256;                 // tokens per tile (each of the 4 waves owns 64)
constexpr int kBK = 32;                  // k per pipeline step (64 bytes per row)
constexpr int kStages = 4;               // ring depth: loads run three steps ahead
constexpr int kWBytes = kBW * kBK * 2;   // weight slab per step (16 KB)
constexpr int kTBytes = kBM * kBK * 2;   // token slab per step (16 KB, 4 KB per wave)
constexpr int kStage = kWBytes + kTBytes;

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

// Workgroup tile: 256 weight rows x 256 tokens, 4 waves; wave w owns tokens
// [64w, 64w+64) of the tile and all 256 weight rows (8 MFMA row blocks):
// gate/up (MAT = 2): blocks 0-3 = gate rows of features [f, f+128) and
// blocks 4-7 = the up rows of the same features, so SiLU(g)*u pairs sit in
// one lane; down (MAT = 1): 256 features.  Accumulators: 8 x 2 32x32 blocks.
//
// At prefill sizes an expert's weights feed only ~256 tokens, about 256
// FLOP per weight byte -- below MI355X's MFMA/HBM ridge -- so the tile is
// built to keep HBM busy.  Each k-step (32 wide) moves a 16 KB weight slab
// and each wave's 4 KB token slab straight into a 4-stage LDS ring with
// direct-to-LDS buffer loads issued three steps ahead (~96 KB in flight per
// CU) -- no vector registers are spent on staging.  A wave instruction fills
// 16 rows x 64 bytes; lane l takes the 16-byte chunk that lands in physical
// slot l%4 of its row.  One wait + barrier per step publishes a stage and
// frees the one read a step earlier.  Token blocks past the expert's last
// token skip their loads and MFMAs: the k-loop is specialised on the number
// of valid blocks (wave-uniform).
//
// MFMA s (0..1) of a step uses 16-byte chunk 2s+g of each row for lane group
// g = l/32 of both operands.
template <int MAT, int OCC>
__global__ __launch_bounds__(256, OCC) void grouped_tiled_kernel(GroupedArgs a) {
  constexpr int F = (MAT == 2) ? kBW / 2 : kBW;  // output features per tile
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStage];
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
    if (e0 < E) c0 = NF * ((a.counts[e0] + kBM - 1) / kBM);
    if (e0 + 1 < E) c1 = NF * ((a.counts[e0 + 1] + kBM - 1) / kBM);
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
  const uint32_t t_rd = kWBytes + wave * (kTBytes / 4);        // this wave's token region

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
    const int mt_e = (n_e + kBM - 1) / kBM;
    const int rel = tile - __builtin_amdgcn_readfirstlane(s_start[e]);
    const int ftile = rel / mt_e, mtile = rel % mt_e;
    const int fbase = ftile * F;
    // The expert's tokens are split evenly over its mt_e token tiles (each at
    // most BM): sibling tiles of one weight tile then do equal work, run side
    // by side on one XCD (adjacent tile ids) and share the weight stream
    // through L2 instead of each reading it from HBM.
    const int m0 = (int)((int64_t)mtile * n_e / mt_e);
    const int m1 = (int)((int64_t)(mtile + 1) * n_e / mt_e);
    const int tw0 = __builtin_amdgcn_readfirstlane(m0 + wave * 64);  // this wave's first token
    const int nbv = max(0, min(2, (m1 - tw0 + 31) / 32));            // its token blocks holding a token

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
    uint32_t toff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
      f32x16 acc[8][2];
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[b][j][i] = 0.f;

      auto issue = [&](int kt) {  // loads of step kt into stage kt % 4
        const uint32_t st = ring_lds + (kt & (kStages - 1)) * kStage;
        const uint32_t so = (uint32_t)kt * (kBK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16(__builtin_amdgcn_readfirstlane(st + (64 * wave + 16 * i) * 64), woff[i], rs_w, so);
#pragma unroll
        for (int i = 0; i < 2 * NBV; ++i)
          dma16(__builtin_amdgcn_readfirstlane(st + t_rd + 16 * i * 64), toff[i], rs_act, so);
      };

      // Loads go out two steps at a time (steps s+2 and s+3 at every even
      // step s), so each row sees back-to-back requests for 128 contiguous
      // bytes.  Step s+1 must have landed at the barrier of step s: at an
      // even step s+2 and s+3 may still be in flight (vmcnt 2 LPS), at an odd
      // step s+2 (vmcnt LPS).  Prologue: steps 0 and 1, step 0 published.
      issue(0);
      issue(min(1, nk - 1));
      BEAM_STEP_BARRIER(LPS);

      // Operands of MFMA s of the step whose stage starts at sb.
      auto read_ops = [&](const unsigned char* sb, int s, uint4 (&af)[8], uint4 (&bf)[2]) {
        const unsigned char* wa = sb + (s ? a_rd1 : a_rd);
#pragma unroll
        for (int b = 0; b < 8; ++b) af[b] = *reinterpret_cast<const uint4*>(wa + 2048 * b);
#pragma unroll
        for (int j = 0; j < NBV; ++j) bf[j] = *reinterpret_cast<const uint4*>(wa + t_rd + 2048 * j);
        __builtin_amdgcn_sched_barrier(0);  // reads go out before the MFMAs that follow
      };
      auto mfmas = [&](const uint4 (&af)[8], const uint4 (&bf)[2]) {
#pragma unroll
        for (int j = 0; j < NBV; ++j)
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[b][j] = mfma32(af[b], bf[j], acc[b][j]);
      };

      // Software pipeline: the barrier publishing step kt+1 sits between
      // the two MFMA groups of step kt, so the reads of the next group are
      // always in flight while the current one runs.  Stage kt % 4 is fully
      // read before that barrier, so an even step kt may refill the stages of
      // steps kt-2 and kt-1 with steps kt+2 and kt+3.
      uint4 af0[8], bf0[2], af1[8], bf1[2];
      if constexpr (NBV > 0) read_ops(ring, 0, af0, bf0);
      auto kstep = [&](auto ODD, int kt) {
        constexpr bool odd = decltype(ODD)::value;
        const unsigned char* sb = ring + (kt & (kStages - 1)) * kStage;
        if (!odd && kt + 2 < nk) {
          issue(kt + 2);
          issue(min(kt + 3, nk - 1));
        }
        if constexpr (NBV > 0) {
          read_ops(sb, 1, af1, bf1);
          mfmas(af0, bf0);
        }
        // this wave's loads of step kt+1 have landed and its reads of stage
        // kt are done; after the barrier, the same holds for every wave
        if (kt + 2 < nk) {
          if constexpr (odd) BEAM_STEP_BARRIER(LPS);
          else BEAM_STEP_BARRIER(2 * LPS);
        } else {
          BEAM_STEP_BARRIER(0);
        }
        if constexpr (NBV > 0) {
          // next step's first operands (after the last step: a stale stage, unused)
          read_ops(ring + ((kt + 1) & (kStages - 1)) * kStage, 0, af0, bf0);
          mfmas(af1, bf1);
        }
      };
      int kt = 0;
      for (; kt + 2 <= nk; kt += 2) {
        kstep(std::false_type{}, kt);
        kstep(std::true_type{}, kt + 1);
      }
      if (kt < nk) kstep(std::false_type{}, kt);
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
    if (nbv == 2) run(std::integral_constant<int, 2>{});
    else if (nbv == 1) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
  }
}

template <int MAT>
static hipError_t launch_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  constexpr int OCC = 1;
  const int nwg = ((num_cu * OCC + 7) / 8) * 8;  // persistent grid, a multiple of the 8 XCDs
  hipLaunchKernelGGL((grouped_tiled_kernel<MAT, OCC>), dim3(nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<2>(st, a, num_cu);
}

hipError_t launch_down_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<1>(st, a, num_cu);
}

}  // namespace beam
