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
// This file: the stream schedule, for decode-size batches (a handful of
// tokens per expert).  Bound by reading the active experts' weights once
// from HBM.  Each wave streams its own weight rows with coalesced
// nontemporal loads (16 lanes cover a 256-byte row segment; each byte is
// used once), re-lays them out through a wave-private LDS tile into the
// 16x16x32 MFMA operand layout, and multiplies them with the expert's tokens
// (up to 16*MT MFMA columns, read from L2).  No workgroup barriers.
// The prefill-size schedule is in gemm_tiled.hip.
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
//
// W8: FP8 (E4M3) weights with per-row scales.  A step's slab is half the
// bytes (ROWS x 128 B), read as 8-byte chunks; each MFMA operand is 8 codes
// converted to bf16 in registers (exactly); the row scales multiply the FP32
// accumulators in the epilogue.
template <int MAT, int RB, int MT, bool W8>
__global__ __launch_bounds__(256) void grouped_stream_kernel(GroupedArgs a) {
  constexpr int ROWS = MAT * RB * 16;
  constexpr int LD = ROWS / 4;  // loads per lane per step (16 or 8 bytes each)
  constexpr int RB8 = W8 ? 128 : 256;  // LDS tile bytes per row
  __shared__ __attribute__((aligned(16))) unsigned char lds[4][ROWS * RB8];

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

  // Weights come in the packed block layout: a 128-k step of the wave's
  // ROWS rows is ROWS/16 row groups x 4 k-blocks, each 16 rows x 64 bytes
  // contiguous (1 KB, one wave load).  Load i covers row group i/4 and
  // k-block i%4; lane l takes row l/4 of the group and physical chunk l%4,
  // i.e. logical chunk (l%4) ^ swz(row).  f0 is a multiple of 16, so the
  // row groups never cross a 128-row block.
  // FP8: the same grid of loads with 8-byte chunks (16 rows x 32 bytes =
  // 512 bytes per wave load), chunk c of block row j at c ^ pack8_swz(j).
  const int64_t ebytes = W8 ? packed8_expert_bytes(N, K) : packed_expert_bytes(N, K);
  constexpr int RBYTES = W8 ? 32 : 64;       // bytes of a packed block row
  constexpr int CH = W8 ? 8 : 16;            // bytes of a chunk (8 k-values)
  constexpr int64_t BLK = W8 ? kPack8BlockBytes : kPackBlockBytes;
  const int nkb = K / kPackK;
  const int rb = f0 / kPackRows, rib0 = f0 % kPackRows;
  const unsigned char* lp[LD];
  int lo[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int grp = i >> 2, kbl = i & 3;
    const int j = lane >> 2, pc = lane & 3;
    const int m = (grp * 16) / (RB * 16);           // matrix (gate / up) of this row group
    const int rib = rib0 + (grp * 16) % (RB * 16) + j;  // row inside the 128-row block
    const int c = pc ^ (W8 ? pack8_swz(rib) : pack_swz(rib));
    const unsigned char* base = reinterpret_cast<const unsigned char*>(m == 0 ? a.w0 : a.w1);
    lp[i] = base + e * ebytes + ((int64_t)(rb * nkb + kbl) * kPackRows + rib) * RBYTES + pc * CH;
    const int rw = grp * 16 + j;                      // row of the wave's LDS tile
    lo[i] = rw * RB8 + (((4 * kbl + c) ^ (rw & 15)) * CH);
  }
  // FP8: 16-byte loads instead -- load i covers k-block i of all 32 rows
  // (1 KB): lane l takes row l/2 and physical chunks 2(l%2), 2(l%2)+1 of it,
  // stored to the LDS slots of their logical chunks (same tile layout).
  constexpr int LD8 = 4;
  const unsigned char* lp8[LD8];
  int lo8[LD8][2];
  if constexpr (W8) {
    static_assert(ROWS == 32, "32 rows per wave");
    const int j = lane >> 1, hh = lane & 1;
    const int m = j / (RB * 16), rib = rib0 + j % (RB * 16);
    const unsigned char* base = reinterpret_cast<const unsigned char*>(m == 0 ? a.w0 : a.w1);
#pragma unroll
    for (int i = 0; i < LD8; ++i) {
      lp8[i] = base + e * ebytes + ((int64_t)(rb * nkb + i) * kPackRows + rib) * RBYTES + hh * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = (2 * hh + u) ^ pack8_swz(rib);
        lo8[i][u] = j * RB8 + (((4 * i + c) ^ (j & 15)) * CH);
      }
    }
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
    uint4 R[W8 ? LD8 : LD];
    uint4 B[2][MT][4];
    auto load_w = [&](int ks) {
      if constexpr (W8) {
#pragma unroll
        for (int i = 0; i < LD8; ++i) R[i] = ld16_nt(lp8[i] + (int64_t)ks * 4 * BLK);
      } else {
#pragma unroll
        for (int i = 0; i < LD; ++i) R[i] = ld16_nt(lp[i] + (int64_t)ks * 4 * BLK);
      }
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
      if constexpr (W8) {
#pragma unroll
        for (int i = 0; i < LD8; ++i) {
          *reinterpret_cast<uint2*>(tile + lo8[i][0]) = make_uint2(R[i].x, R[i].y);
          *reinterpret_cast<uint2*>(tile + lo8[i][1]) = make_uint2(R[i].z, R[i].w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < LD; ++i) st16(tile + lo[i], R[i]);
      }
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
            uint4 av;
            if constexpr (W8)
              av = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(tile + rw * RB8 + ((4 * j + q) ^ r) * CH));
            else
              av = *reinterpret_cast<const uint4*>(tile + rw * RB8 + ((4 * j + q) ^ r) * CH);
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
            // k = kt + 16q + 8c: k-block kt/32 + q/2, logical chunk 2(q%2) + c
            const int rib = rib0 + 16 * i + r;
            const int kb = kt / kPackK + (q >> 1);
            const int pc = (2 * (q & 1) + c) ^ (W8 ? pack8_swz(rib) : pack_swz(rib));
            const unsigned char* base = reinterpret_cast<const unsigned char*>(m == 0 ? a.w0 : a.w1);
            const unsigned char* ap =
                base + e * ebytes + ((int64_t)(rb * nkb + kb) * kPackRows + rib) * RBYTES + pc * CH;
            uint4 at;
            if constexpr (W8) at = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(ap));
            else at = ld16(ap);
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[m][i][t] = mfma16(at, bt[t], acc[m][i][t]);
          }
      }
    }

    // Epilogue: lane holds features f0+16i+4q+c (c = 0..3) of token c0+16t+r
    // (FP8: times the features' row scales first).
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int f = f0 + 16 * i + 4 * q;
      if (f >= N) continue;
      f32x4 sc0 = f32x4{1.f, 1.f, 1.f, 1.f}, sc1 = sc0;
      if constexpr (W8) {
        sc0 = *reinterpret_cast<const f32x4*>(a.s0 + (int64_t)e * N + f);
        if constexpr (MAT == 2) sc1 = *reinterpret_cast<const f32x4*>(a.s1 + (int64_t)e * N + f);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int tok = c0 + 16 * t + r;
        if (tok >= n_e) continue;
        const int64_t row = row0 + tok;
        if constexpr (MAT == 2) {
          float h4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) h4[c] = swiglu(acc[0][i][t][c] * sc0[c], acc[1][i][t][c] * sc1[c]);
          uint2 v = make_uint2(pack_bf16x2_rne(h4[0], h4[1]), pack_bf16x2_rne(h4[2], h4[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + f) = v;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * N + f) = acc[0][i][t] * sc0;
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

template <int MAT, int RB, bool W8>
static hipError_t launch_stream_w(hipStream_t st, const GroupedArgs& a, int mt) {
  dim3 grid((a.N + 4 * RB * 16 - 1) / (4 * RB * 16), a.E), block(256);
  if (mt == 1) hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 1, W8>), grid, block, 0, st, a);
  else if (mt == 2) hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 2, W8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((grouped_stream_kernel<MAT, RB, 4, W8>), grid, block, 0, st, a);
  return hipGetLastError();
}

// FP8 weights are recognised by their row scales.
template <int MAT, int RB>
static hipError_t launch_stream(hipStream_t st, const GroupedArgs& a, int mt) {
  return a.s0 ? launch_stream_w<MAT, RB, true>(st, a, mt) : launch_stream_w<MAT, RB, false>(st, a, mt);
}

hipError_t launch_gateup_stream(hipStream_t st, const GroupedArgs& a, int64_t T, int k) {
  return launch_stream<2, 1>(st, a, stream_mt(T, k, a.E));
}

hipError_t launch_down_stream(hipStream_t st, const GroupedArgs& a, int64_t T, int k) {
  return launch_stream<1, 2>(st, a, stream_mt(T, k, a.E));
}

}  // namespace beam
