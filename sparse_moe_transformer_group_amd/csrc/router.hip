// Router of the Beam MoE block on gfx950: FP32 logits on MFMA, FP32 sigmoid,
// group-limited top-k with wavefront shuffle reductions.
//
// Method (page "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen,
// anpassen und skalieren können", section "Mixture of Experts"; router in FP32
// per section "Residual Stream"): every expert gets a sigmoid score; experts
// form contiguous groups; a group's score is the sum of its two best expert
// scores; the best topk_groups groups are kept and the k best experts inside
// them are chosen; their scores are normalised to sum to one and scaled.
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Logits: zpart[s][t][e] = sum over K-slice s of x[t,h] * wr[e,h].
// bf16 x bf16 products are exact; MFMA accumulates them in FP32.
// Each wave computes 64 experts x 64 tokens (4 x 4 MFMA blocks), loading its
// operands straight from global memory (Wr is 2.6 MB at Beam shape and stays
// in L2); a workgroup's waves (4, or 1 for decode-size batches, which then
// spread over 4x as many CUs) cover 64 experts each.  Expert rows are the MFMA
// A side, tokens the B side, so each lane ends with 4 consecutive experts of
// one token and stores them as one 16-byte vector.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ zpart, int T, int H,
                                                            int E, int S) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 64;
  const int e0 = (blockIdx.y * (int)(blockDim.x >> 6) + wave) * 64;
  if (e0 >= E) return;  // no barriers below
  const int s = blockIdx.z;
  const int nk = H / 32;
  const int kb = (int)((int64_t)s * nk / S), ke = (int)((int64_t)(s + 1) * nk / S);

  const uint16_t* ap[4];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = min(e0 + 16 * i + r, E - 1);
    ap[i] = wr + (int64_t)e * H + q * 8;
    int t = min(t0 + 16 * i + r, T - 1);
    bp[i] = x + (int64_t)t * H + q * 8;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // software-pipelined: the next k-step's operands are in flight while the
  // current one is multiplied
  uint4 a[2][4], b[2][4];
  auto load = [&](int buf, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[buf][i] = ld16(ap[i] + kk * 32);
      b[buf][i] = ld16(bp[i] + kk * 32);
    }
  };
  auto mult = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[buf][i], b[buf][j], acc[i][j]);
  };
  if (kb < ke) load(0, kb);
  int kk = kb;
  for (; kk + 2 <= ke; kk += 2) {
    load(1, kk + 1);
    mult(0);
    if (kk + 2 < ke) load(0, kk + 2);
    mult(1);
  }
  if (kk < ke) mult(0);

  float* zs = zpart + (int64_t)s * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 16 * i + q * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 16 * j + r;
      if (t >= T) continue;
      float* dst = zs + (int64_t)t * E + e;
      if (e + 3 < E && (E & 3) == 0) {
        *reinterpret_cast<f32x4*>(dst) = acc[i][j];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < E) dst[c] = acc[i][j][c];
      }
    }
  }
}

// Prefill-size batches: a workgroup computes 256 experts x 128 tokens of a
// K-slice.  The 128-token x slab of a k-step (8 KB) is loaded once per
// workgroup into LDS (double-buffered, one barrier per step) and shared by
// the 4 waves; each wave loads its own 64 expert rows from global memory as
// above.  Per k-step a CU then reads 24 KB for 32 MFMAs per wave instead of
// 8 KB for 16 (4 waves each loading the same token rows), which kept the
// kernel on the cache bandwidth.  The k-steps of a slice run in the same
// order, so the logits are bit-identical to the kernel above.
__device__ __forceinline__ int xs_swz(int row) { return (row >> 2) & 3; }

__global__ __launch_bounds__(256) void router_logits_wide_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr,
                                                                 float* __restrict__ zpart, int T,
                                                                 int H, int E, int S) {
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][128 * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 128;
  const int e0 = (blockIdx.y * 4 + wave) * 64;  // may be >= E: computes, stores nothing
  const int s = blockIdx.z;
  const int nk = H / 32;
  const int kb = (int)((int64_t)s * nk / S), ke = (int)((int64_t)(s + 1) * nk / S);

  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ap[i] = wr + (int64_t)min(e0 + 16 * i + r, E - 1) * H + q * 8;
  // x slab loads: thread tid copies chunks tid and tid + 256 (row c/4, chunk c%4)
  const uint16_t* xp[2];
  int xo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + 256 * u, row = c >> 2, ch = c & 3;
    xp[u] = x + (int64_t)min(t0 + row, T - 1) * H + ch * 8;
    xo[u] = row * 64 + ((ch ^ xs_swz(row)) << 4);
  }
  int bo[8];  // this lane's operand of token block j: row 16 j + r, chunk q
#pragma unroll
  for (int j = 0; j < 8; ++j) bo[j] = (16 * j + r) * 64 + ((q ^ xs_swz(16 * j + r)) << 4);

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 a_cur[4], a_nxt[4], x_nxt[2];
  if (kb < ke) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a_cur[i] = ld16(ap[i] + kb * 32);
#pragma unroll
    for (int u = 0; u < 2; ++u) st16(xs[0] + xo[u], ld16(xp[u] + kb * 32));
  }
  __syncthreads();
  for (int kk = kb; kk < ke; ++kk) {
    const int buf = (kk - kb) & 1;
    const bool more = kk + 1 < ke;
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a_nxt[i] = ld16(ap[i] + (kk + 1) * 32);
#pragma unroll
      for (int u = 0; u < 2; ++u) x_nxt[u] = ld16(xp[u] + (kk + 1) * 32);
    }
    uint4 b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = *reinterpret_cast<const uint4*>(xs[buf] + bo[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(a_cur[i], b[j], acc[i][j]);
    if (more) {
      // the other buffer was last read before the previous barrier
#pragma unroll
      for (int u = 0; u < 2; ++u) st16(xs[buf ^ 1] + xo[u], x_nxt[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) a_cur[i] = a_nxt[i];
    }
    __syncthreads();
  }

  if (e0 >= E) return;  // after the last barrier
  float* zs = zpart + (int64_t)s * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 16 * i + q * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + 16 * j + r;
      if (t >= T) continue;
      float* dst = zs + (int64_t)t * E + e;
      if (e + 3 < E && (E & 3) == 0) {
        *reinterpret_cast<f32x4*>(dst) = acc[i][j];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < E) dst[c] = acc[i][j][c];
      }
    }
  }
}

// Decode-size batches (one 64-token tile) run the logits with one-wave
// workgroups of 64 experts: the same per-wave work on 4x as many CUs.
static bool router_small(int64_t T) { return T <= 64; }

int router_splits(int64_t T, int H, int E) {
  const int64_t blocks = ((T + 63) / 64) * ((E + 255) / 256);
  const int nk = H / 32;
  int S = 1;
  while (blocks * S < 512 && S * 2 * 4 <= nk) S *= 2;
  return S;
}

hipError_t launch_router_logits(hipStream_t st, const uint16_t* x, const uint16_t* wr, float* zpart,
                                int T, int H, int E, int S) {
  if (T >= 1024) {  // prefill sizes: the 128-token tiles with the x slab in LDS
    dim3 grid((T + 127) / 128, (E + 255) / 256, S);
    hipLaunchKernelGGL(router_logits_wide_kernel, grid, dim3(256), 0, st, x, wr, zpart, T, H, E, S);
  } else {
    const int W = router_small(T) ? 1 : 4;  // waves per workgroup
    dim3 grid((T + 63) / 64, (E + 64 * W - 1) / (64 * W), S);
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(64 * W), 0, st, x, wr, zpart, T, H, E, S);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection: one wavefront per token.
// ---------------------------------------------------------------------------

// (value, index) total order: larger value first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Butterfly all-reduce of the best (value, index) pair over the wavefront.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, 64);
    int oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Merge two descending top-2 lists (a1 >= a2, b1 >= b2).
__device__ __forceinline__ void merge_top2(float& a1, float& a2, float b1, float b2) {
  float n1 = fmaxf(a1, b1);
  float n2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
  a1 = n1;
  a2 = n2;
}

constexpr int kMaxE = 512;
constexpr int kMaxG = 256;

// EPL = experts held per lane (lane l holds experts l*EPL .. l*EPL+EPL-1);
// W = waves (tokens) per workgroup: 4, or 1 for decode-size batches.
template <int EPL, int W>
__global__ __launch_bounds__(64 * W) void select_kernel(const float* __restrict__ zpart, int S,
                                                         const float* __restrict__ offset, int T, int E,
                                                         int G, int KG, int k, float scale,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wout,
                                                         int32_t* __restrict__ counts) {
  __shared__ float lds_sc[W][kMaxE];
  __shared__ float lds_gs[W][kMaxG];
  __shared__ int lds_kept[W][kMaxG];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t_raw = blockIdx.x * W + wave;
  const bool active = t_raw < T;
  const int t = active ? t_raw : T - 1;
  const int GS = E / G;

  // 1. scores: FP32 sum of the K-slice partials in slice order, + offset, sigmoid.
  // The loads of up to 16 slices are issued together (one 16-byte load per
  // slice when the lane's 4 experts are contiguous and aligned), so the
  // latency is paid once per 16 slices; the sum stays in slice order.
  float z[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) z[i] = 0.f;
  {
    const float* zp = zpart + (int64_t)t * E + lane * EPL;
    const int64_t sstride = (int64_t)T * E;
    const bool vec4 = (EPL == 4) && (E % 4 == 0) && (lane * EPL + 3 < E);
    for (int s0 = 0; s0 < S; s0 += 16) {
      float v[16][EPL];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (s0 + u >= S) continue;
        const float* p = zp + (s0 + u) * sstride;
        if (vec4) {
          const f32x4 q4 = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
          for (int i = 0; i < EPL; ++i) v[u][i] = q4[i & 3];
        } else {
#pragma unroll
          for (int i = 0; i < EPL; ++i) v[u][i] = (lane * EPL + i < E) ? p[i] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (s0 + u >= S) continue;
#pragma unroll
        for (int i = 0; i < EPL; ++i) z[i] = (s0 + u == 0) ? v[u][i] : z[i] + v[u][i];
      }
    }
  }
  float sc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    if (e < E) {
      float zi = z[i];
      if (offset) zi += offset[e];
      sc[i] = 1.0f / (1.0f + expf(-zi));
    } else {
      sc[i] = -INFINITY;
    }
  }

  // 2. group scores = sum of the two largest scores of each group.
  const int LPG = GS / EPL;  // lanes per group when a group is whole lanes
  const bool lane_groups = (GS % EPL == 0) && LPG >= 1 && LPG <= 64 && ((LPG & (LPG - 1)) == 0) &&
                           (E == 64 * EPL);
  if (lane_groups) {
    float b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float v = sc[i];
      if (v > b1) {
        b2 = b1;
        b1 = v;
      } else if (v > b2) {
        b2 = v;
      }
    }
    for (int off = 1; off < LPG; off <<= 1) {
      float o1 = __shfl_xor(b1, off, 64);
      float o2 = __shfl_xor(b2, off, 64);
      merge_top2(b1, b2, o1, o2);
    }
    if ((lane % LPG) == 0) lds_gs[wave][(lane * EPL) / GS] = b1 + b2;
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (e < E) lds_sc[wave][e] = sc[i];
    }
    __syncthreads();
    for (int g = lane; g < G; g += 64) {
      float b1 = -INFINITY, b2 = -INFINITY;
      for (int m = 0; m < GS; ++m) {
        float v = lds_sc[wave][g * GS + m];
        if (v > b1) {
          b2 = b1;
          b1 = v;
        } else if (v > b2) {
          b2 = v;
        }
      }
      lds_gs[wave][g] = b1 + b2;
    }
  }
  __syncthreads();

  // 3. keep the KG best groups (iterative wavefront argmax).
  constexpr int GPL = kMaxG / 64;  // groups per lane: g = lane + 64 * j
  float gv[GPL];
  uint32_t kept = 0;
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int g = lane + 64 * j;
    gv[j] = (g < G) ? lds_gs[wave][g] : -INFINITY;
  }
  for (int rnd = 0; rnd < KG; ++rnd) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = lane + 64 * j;
      if (g < G && !((kept >> j) & 1u) && better(gv[j], g, bv, bi)) {
        bv = gv[j];
        bi = g;
      }
    }
    wave_argmax(bv, bi);
    if (bi < G && (bi & 63) == lane) kept |= 1u << (bi >> 6);
  }
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int g = lane + 64 * j;
    if (g < G) lds_kept[wave][g] = (kept >> j) & 1u;
  }
  __syncthreads();

  // 4. the k best experts of the kept groups.
  bool elig[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    elig[i] = (e < E) && lds_kept[wave][e / GS];
  }
  uint32_t taken = 0;
  float sum = 0.f, my_v = 0.f;
  int my_e = 0;
  for (int rnd = 0; rnd < k; ++rnd) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (elig[i] && !((taken >> i) & 1u) && better(sc[i], e, bv, bi)) {
        bv = sc[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (bi < E && bi / EPL == lane) taken |= 1u << (bi % EPL);
    sum += bv;  // same order in every lane: selection order
    if (lane == rnd) {
      my_v = bv;
      my_e = bi;
    }
  }

  // 5. normalise, then scale.
  if (active && lane < k) {
    ids[(int64_t)t * k + lane] = my_e;
    wout[(int64_t)t * k + lane] = scale * (my_v / sum);
    if (counts) atomicAdd(&counts[my_e], 1);
  }
}

hipError_t launch_select(hipStream_t st, const float* zpart, int S, const float* offset, int T, int E,
                         int groups, int topk_groups, int k, float scale, int32_t* ids, float* w,
                         int32_t* counts) {
  const int epl = (E + 63) / 64;
  const bool one = T <= 256;  // one token per workgroup: more CUs for a small batch
#define BEAM_SELECT(N)                                                                            \
  if (one)                                                                                        \
    hipLaunchKernelGGL((select_kernel<N, 1>), dim3(T), dim3(64), 0, st, zpart, S, offset, T, E,   \
                       groups, topk_groups, k, scale, ids, w, counts);                            \
  else                                                                                            \
    hipLaunchKernelGGL((select_kernel<N, 4>), dim3((T + 3) / 4), dim3(256), 0, st, zpart, S,      \
                       offset, T, E, groups, topk_groups, k, scale, ids, w, counts)
  if (epl <= 1) BEAM_SELECT(1);
  else if (epl <= 2) BEAM_SELECT(2);
  else if (epl <= 4) BEAM_SELECT(4);
  else BEAM_SELECT(8);
#undef BEAM_SELECT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(hipStream_t st, int32_t* p, int64_t n, int32_t v) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace beam
