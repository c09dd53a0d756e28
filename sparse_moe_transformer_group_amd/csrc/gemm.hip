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
//    lane per step, 256 bytes per row segment), double-buffered, with the
//    expert's tokens as up to 16*MT MFMA columns.  No LDS, no barriers.
//  * tiled: prefill-size batches.  Weight and token tiles are staged through
//    LDS (XOR-swizzled 16-byte chunks, conflict-free for ds_read_b128),
//    double-buffered, and a persistent grid walks the (expert, feature tile,
//    token tile) space in XCD-contiguous ranges so that the token tiles of
//    one weight tile run back to back on one XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace beam {

// ===========================================================================
// Stream schedule
// ===========================================================================
// MAT = 2: gate+up with SwiGLU epilogue (bf16 out); MAT = 1: down (fp32 out).
// RB  = 16-row weight blocks per wave per matrix; MT = 16-token tiles held.
template <int MAT, int RB, int MT>
__global__ __launch_bounds__(256) void grouped_stream_kernel(GroupedArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int e = blockIdx.y;
  const int n_e = a.counts[e];
  if (n_e <= 0) return;
  const int f0 = (blockIdx.x * 4 + wave) * (RB * 16);
  if (f0 >= a.N) return;  // no barriers in this kernel
  const int row0 = a.offsets[e];
  const int N = a.N, K = a.K;

  // Lane (r, q) reads weight row f0+16i+r, k in [k0 + 32q, k0 + 32q + 32) per
  // 128-wide step; MFMA c of the step uses its 8-value piece c.  The token
  // operand uses the same k mapping.
  const uint16_t* wp[MAT][RB];
#pragma unroll
  for (int m = 0; m < MAT; ++m)
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int f = min(f0 + 16 * i + r, N - 1);
      const uint16_t* base = (m == 0) ? a.w0 : a.w1;
      wp[m][i] = base + ((int64_t)e * N + f) * K + q * 32;
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
      bp[j] = a.act + src * K + q * 32;
    }
    f32x4 acc[MAT][RB][MT];
#pragma unroll
    for (int m = 0; m < MAT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 A[2][MAT][RB][4];
    uint4 B[2][MT][4];
    auto load = [&](int buf, int k0) {
#pragma unroll
      for (int m = 0; m < MAT; ++m)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) A[buf][m][i][c] = ld16(wp[m][i] + k0 + c * 8);
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          B[buf][j][c] = bv[j] ? ld16(bp[j] + k0 + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int m = 0; m < MAT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j)
              acc[m][i][j] = mfma16(A[buf][m][i][c], B[buf][j][c], acc[m][i][j]);
    };

    const int nsteps = K / 128;  // K is a multiple of 64; a 64 tail is handled below
    load(0, 0);
    int ks = 0;
    for (; ks + 2 <= nsteps; ks += 2) {
      load(1, (ks + 1) * 128);
      compute(0);
      if (ks + 2 < nsteps) load(0, (ks + 2) * 128);
      compute(1);
    }
    if (ks < nsteps) compute(0);
    if (K % 128) {
      // 64-wide tail: lane q covers k in [kt + 16q, kt + 16q + 16) as two pieces
      const int kt = nsteps * 128;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 at[MAT][RB], bt[MT];
#pragma unroll
        for (int m = 0; m < MAT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i) at[m][i] = ld16(wp[m][i] - q * 32 + kt + q * 16 + c * 8);
#pragma unroll
        for (int j = 0; j < MT; ++j)
          bt[j] = bv[j] ? ld16(bp[j] - q * 32 + kt + q * 16 + c * 8) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int m = 0; m < MAT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j) acc[m][i][j] = mfma16(at[m][i], bt[j], acc[m][i][j]);
      }
    }

    // Epilogue: lane holds features f0+16i+4q+c (c = 0..3) of token c0+16j+r.
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int f = f0 + 16 * i + 4 * q;
      if (f >= N) continue;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int tok = c0 + 16 * j + r;
        if (tok >= n_e) continue;
        const int64_t row = row0 + tok;
        if constexpr (MAT == 2) {
          uint32_t p[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) p[c] = f32_to_bf16_rne(swiglu(acc[0][i][j][c], acc[1][i][j][c]));
          uint2 v = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + f) = v;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * N + f) = acc[0][i][j];
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
constexpr int kMaxE = 512;
constexpr int kBK = 64;  // k per LDS stage (128 bytes per row)

// MAT matrices of F = WF*FW features each form the weight tile (AR rows);
// BM = WT*TW tokens form the token tile.  4 waves as WF x WT.
template <int MAT, int FW, int TW, int WF, int WT>
struct TileCfg {
  static constexpr int F = WF * FW;
  static constexpr int AR = MAT * F;
  static constexpr int BM = WT * TW;
  static constexpr int ROWS = AR + BM;
  static constexpr int PASSES = ROWS * 8 / 256;  // 16-byte chunks per thread per stage
  static constexpr int STAGE_BYTES = ROWS * kBK * 2;
  static_assert(WF * WT == 4, "4 waves");
  static_assert((ROWS * 8) % 256 == 0, "whole passes");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int MAT, int FW, int TW, int WF, int WT>
__global__ __launch_bounds__(256, 2) void grouped_tiled_kernel(GroupedArgs a) {
  using C = TileCfg<MAT, FW, TW, WF, WT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_start[kMaxE + 1];
  __shared__ int s_scan[256];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int wf = wave % WF, wt = wave / WF;
  const int N = a.N, K = a.K, E = a.E;
  const int NF = (N + C::F - 1) / C::F;

  // Tile prefix over experts: expert e owns NF * ceil(n_e / BM) tiles.
  {
    const int e0 = tid * 2;
    int c0 = 0, c1 = 0;
    if (e0 < E) c0 = NF * ((a.counts[e0] + C::BM - 1) / C::BM);
    if (e0 + 1 < E) c1 = NF * ((a.counts[e0 + 1] + C::BM - 1) / C::BM);
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

  for (int tile = lo + slot; tile < hi; tile += per_xcd) {
    // expert: largest e with s_start[e] <= tile
    int elo = 0, ehi = E - 1;
    while (elo < ehi) {
      const int mid = (elo + ehi + 1) >> 1;
      if (s_start[mid] <= tile) elo = mid;
      else ehi = mid - 1;
    }
    const int e = elo;
    const int n_e = a.counts[e];
    const int row0 = a.offsets[e];
    const int mt_e = (n_e + C::BM - 1) / C::BM;
    const int rel = tile - s_start[e];
    const int ftile = rel / mt_e, mtile = rel % mt_e;
    const int fbase = ftile * C::F, m0 = mtile * C::BM;

    // Per-thread source rows for the global->LDS copy.
    const uint16_t* src[C::PASSES];
    int dst[C::PASSES];
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int idx = tid + 256 * p;
      const int row = idx >> 3, chunk = idx & 7;
      dst[p] = swz(row, chunk);
      if (row < C::AR) {
        const int m = row / C::F;
        const int f = min(fbase + row % C::F, N - 1);
        const uint16_t* base = (m == 0) ? a.w0 : a.w1;
        src[p] = base + ((int64_t)e * N + f) * K + chunk * 8;
      } else {
        const int tok = min(m0 + row - C::AR, n_e - 1);
        const int rr = row0 + tok;
        const int64_t s = a.sorted_tokens ? (int64_t)a.sorted_tokens[rr] : (int64_t)rr;
        src[p] = a.act + s * K + chunk * 8;
      }
    }

    constexpr int NA = MAT * (FW / 16), NB = TW / 16;
    f32x4 acc[NA][NB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 stg[C::PASSES];
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) stg[p] = ld16(src[p]);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) st16(smem + dst[p], stg[p]);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) {
#pragma unroll
        for (int p = 0; p < C::PASSES; ++p) stg[p] = ld16(src[p] + (kt + 1) * kBK);
      }
      const unsigned char* sa = smem + (kt & 1) * C::STAGE_BYTES;
      const unsigned char* sb = sa + C::AR * 128;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int chunk = s * 4 + q;
        uint4 af[NA], bf[NB];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const int m = i / (FW / 16), ib = i % (FW / 16);
          const int row = m * C::F + wf * FW + ib * 16 + r;
          af[i] = *reinterpret_cast<const uint4*>(sa + swz(row, chunk));
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int row = wt * TW + j * 16 + r;
          bf[j] = *reinterpret_cast<const uint4*>(sb + swz(row, chunk));
        }
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
      }
      if (more) {
        unsigned char* nxt = smem + ((kt + 1) & 1) * C::STAGE_BYTES;
#pragma unroll
        for (int p = 0; p < C::PASSES; ++p) st16(nxt + dst[p], stg[p]);
      }
      __syncthreads();
    }

    // Epilogue.
    constexpr int FB = FW / 16;
#pragma unroll
    for (int ib = 0; ib < FB; ++ib) {
      const int f = fbase + wf * FW + ib * 16 + 4 * q;
      if (f >= N) continue;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int tok = m0 + wt * TW + j * 16 + r;
        if (tok >= n_e) continue;
        const int64_t row = row0 + tok;
        if constexpr (MAT == 2) {
          uint32_t p[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) p[c] = f32_to_bf16_rne(swiglu(acc[ib][j][c], acc[FB + ib][j][c]));
          uint2 v = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + f) = v;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * N + f) = acc[ib][j];
        }
      }
    }
  }
}

template <int MAT, int FW, int TW, int WF, int WT>
static hipError_t launch_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  using C = TileCfg<MAT, FW, TW, WF, WT>;
  const int lds = 2 * C::STAGE_BYTES;
  auto kern = grouped_tiled_kernel<MAT, FW, TW, WF, WT>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int nwg = ((num_cu * 2 + 7) / 8) * 8;  // 2 workgroups per CU, multiple of 8 XCDs
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(256), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<2, 32, 64, 2, 2>(st, a, num_cu);
}

hipError_t launch_down_tiled(hipStream_t st, const GroupedArgs& a, int num_cu) {
  return launch_tiled<1, 64, 64, 2, 2>(st, a, num_cu);
}

}  // namespace beam
