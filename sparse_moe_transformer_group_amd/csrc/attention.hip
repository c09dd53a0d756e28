// Beam attention sublayer (prefill of one sequence) on gfx950.
//
// Page "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen, anpassen
// und skalieren können", section "Attention": grouped-query attention with 48
// query heads and 8 key/value heads, RMSNorm on queries and keys; sliding-
// window layers (the previous 512 tokens) use RoPE, global layers use no
// position encoding and multiply each query by (1 + (pos + 1) / 2048)^0.1; a
// sigmoid gate computed from the layer input scales every channel of every
// head before the output projection.  Section "Long Context" fixes the head
// size at 128 (2 x 8 KV heads x 128 dims cached per token); section "Residual
// Stream" puts RoPE and the query scaling in FP32.
//
// Path (one call of beam_attn_forward):
//   1. qkvg = u [T, H] x [Wq; Wk; Wv; Wg]^T      plain tiled GEMM, FP32 out
//   2. attn_prep:   per token and head, RMSNorm (FP32) of q and k, then RoPE
//      (sliding window) or the query scaling (global); q, k -> bf16 head-major
//      [head][T][128]; v -> bf16 [T][8*128]
//   3. attn_vt:     v -> per kv head [128 dims][Tp keys] in FP16, scaled by a
//      power of two (keys permuted inside each group of 16, see below), zero
//      past T
//   4. attn_flash:  softmax(q k^T / sqrt(128)) v per query head, causal and
//      windowed, online softmax in FP32, PV in FP16; x sigmoid(gate) -> o bf16
//      [T][6144]
//   5. y = o x Wo^T                                plain tiled GEMM, bf16 out
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace beam {

typedef float f32x16a __attribute__((__vector_size__(16 * sizeof(float))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16a mfma32a(uint4 a, uint4 b, f32x16a c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16a mfma32h(uint4 a, uint4 b, f32x16a c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_f16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// The PV product runs in FP16 (11 significant bits for the probabilities
// instead of bf16's 8).  v is bf16; multiplied by a power of two chosen per
// kv head so that the largest |v| lands in [2^14, 2^15), every normal value
// converts to FP16 exactly and none overflows.  vmax holds the per-head
// maximum |v| as float bits (non-negative floats order like their bits).
constexpr int kAttnVmaxSlot = 8;  // tile_ctr[8 .. 15]: the 8 kv heads' max |v| (float bits)
__device__ __forceinline__ float attn_v_scale(const int32_t* vmax, int g) {
  const float m = __int_as_float(vmax[g]);
  if (!(m > 0.f) || !isfinite(m)) return 1.f;
  int e;
  frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)
  return ldexpf(1.f, 15 - e);
}

// ---------------------------------------------------------------------------
// setup: the one-"expert" row bookkeeping of the two GEMMs and their tile
// counters (a kernel, not a memset, so the call can be graph-captured)
__global__ void attn_setup_kernel(int T, int32_t* counts, int32_t* offsets, int32_t* ctr, int nctr) {
  const int i = threadIdx.x;
  if (i == 0) {
    counts[0] = T;
    offsets[0] = 0;
    offsets[1] = T;
  }
  if (i < nctr) ctr[i] = 0;
}

// ---------------------------------------------------------------------------
// prep: one workgroup per token (rows T .. Tp-1 are written as zeros).  Each
// wave normalises pairs of heads: the 28 pairs (q heads 0..47, then k heads)
// are dealt to the 4 waves, lanes 0..31 taking the first head of a pair and
// 32..63 the second.  Lane l' = l % 32 holds dims 2l', 2l'+1 and their RoPE
// partners 2l'+64, 2l'+65, so the rotation needs no cross-lane step.  The
// largest |v| of each kv head at this token goes to vmx[t][8].
constexpr int kPrepPairsPerWave = (kAttnQHeads + kAttnKVHeads) / 8;  // 7
__global__ __launch_bounds__(256) void attn_prep_kernel(const float* __restrict__ qkvg, int T,
                                                        int global_layer, float theta,
                                                        uint16_t* __restrict__ qn,
                                                        uint16_t* __restrict__ kn,
                                                        uint16_t* __restrict__ vb, int Tp,
                                                        float* __restrict__ vmx) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l = lane & 31, half = lane >> 5;
  constexpr int QW = kAttnQHeads * kAttnHeadDim, KW = kAttnKVHeads * kAttnHeadDim;
  constexpr int NW = 2 * QW + 2 * KW;
  auto dst_of = [&](int h) {
    return (h < kAttnQHeads) ? qn + ((int64_t)h * Tp + t) * kAttnHeadDim
                             : kn + ((int64_t)(h - kAttnQHeads) * Tp + t) * kAttnHeadDim;
  };
  auto head_of = [&](int i) { return 2 * (wave + 4 * i) + half; };  // q heads 0..47, k heads 48..55
  if (t >= T) {  // padding rows of the head-major arrays
#pragma unroll
    for (int i = 0; i < kPrepPairsPerWave; ++i) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(dst_of(head_of(i)));
      dst[l] = 0u;
      dst[l + 32] = 0u;
    }
    return;
  }
  const float* row = qkvg + (int64_t)t * NW;
  // all of this wave's loads first (q and k heads: columns h * 128)
  float2 lo[kPrepPairsPerWave], hi[kPrepPairsPerWave];
#pragma unroll
  for (int i = 0; i < kPrepPairsPerWave; ++i) {
    const float* src = row + head_of(i) * kAttnHeadDim + 2 * l;
    lo[i] = *reinterpret_cast<const float2*>(src);
    hi[i] = *reinterpret_cast<const float2*>(src + 64);
  }
  const f32x4 v = *reinterpret_cast<const f32x4*>(row + QW + KW + threadIdx.x * 4);
  // rotations of pairs 2l' and 2l'+1 at position t: the angle is formed and
  // reduced in double precision (t * theta^(-i/64) exceeds FP32 resolution at
  // long positions), then sin/cos in FP32
  float cs0 = 1.f, sn0 = 0.f, cs1 = 1.f, sn1 = 0.f, qs = 1.f;
  if (global_layer) {
    qs = powf(1.f + (float)(t + 1) / 2048.f, 0.1f);
  } else {
    auto angle = [&](int i, float& sn, float& cs) {
      const double ang = (double)t * pow((double)theta, -(double)i / 64.0);
      const double red = ang - 6.283185307179586 * floor(ang / 6.283185307179586);
      sincosf((float)red, &sn, &cs);
    };
    angle(2 * l, sn0, cs0);
    angle(2 * l + 1, sn1, cs1);
  }
#pragma unroll
  for (int i = 0; i < kPrepPairsPerWave; ++i) {
    const int h = head_of(i);
    float a0 = lo[i].x, a1 = lo[i].y, b0 = hi[i].x, b1 = hi[i].y;  // dims 2l', 2l'+1, +64, +65
    float ss = a0 * a0 + a1 * a1 + b0 * b0 + b1 * b1;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kAttnHeadDim) + 1e-6f);
    a0 *= inv;
    a1 *= inv;
    b0 *= inv;
    b1 *= inv;
    if (global_layer) {
      if (h < kAttnQHeads) {
        a0 *= qs;
        a1 *= qs;
        b0 *= qs;
        b1 *= qs;
      }
    } else {
      const float r0 = a0 * cs0 - b0 * sn0, s0 = b0 * cs0 + a0 * sn0;
      const float r1 = a1 * cs1 - b1 * sn1, s1 = b1 * cs1 + a1 * sn1;
      a0 = r0;
      b0 = s0;
      a1 = r1;
      b1 = s1;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(dst_of(h));
    dst[l] = pack_bf16x2_rne(a0, a1);       // dims 2l', 2l'+1
    dst[l + 32] = pack_bf16x2_rne(b0, b1);  // dims 2l'+64, 2l'+65
  }
  // v -> bf16, row-major [T][8*128]; thread i holds dims 4i .. 4i+3, so the
  // 32 lanes of each half-wave hold one kv head
  const uint2 bv = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
  *reinterpret_cast<uint2*>(vb + (int64_t)t * KW + threadIdx.x * 4) = bv;
  float m = fmaxf(fmaxf(fabsf(__uint_as_float(bv.x << 16)), fabsf(__uint_as_float(bv.x & 0xffff0000u))),
                  fmaxf(fabsf(__uint_as_float(bv.y << 16)), fabsf(__uint_as_float(bv.y & 0xffff0000u))));
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 31) == 0) vmx[(int64_t)t * kAttnKVHeads + (threadIdx.x >> 5)] = m;
}

// vmax[g] = max over tokens of vmx[t][g] (as float bits, non-negative floats
// order like their bits): grid (8 kv heads, 16 token slices); each workgroup
// folds its slice and raises vmax[g] with one atomic (vmax zeroed by
// attn_setup_kernel).
constexpr int kVmaxSlices = 16;
__global__ __launch_bounds__(256) void attn_vmax_kernel(const float* __restrict__ vmx, int T,
                                                        int32_t* __restrict__ vmax) {
  __shared__ float part[4];
  const int g = blockIdx.x;
  float m = 0.f;
  for (int t = blockIdx.y * 256 + threadIdx.x; t < T; t += 256 * kVmaxSlices)
    m = fmaxf(m, vmx[(int64_t)t * kAttnKVHeads + g]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mm = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    if (mm > 0.f) atomicMax(vmax + g, __float_as_int(mm));
  }
}

// Key order inside each group of 16 in the transposed v: the attention
// kernel's PV product takes, for MFMA lane group g, the keys 4g..4g+3 and
// 8+4g..8+4g+3 of a group (the layout of its softmax registers), so keys
// 4..7 and 8..11 trade places: then each lane group reads 8 contiguous keys.
__device__ __forceinline__ int vt_slot(int key) {
  const int k = key & 15;
  const int s = (k >= 4 && k < 8) ? k + 4 : (k >= 8 && k < 12) ? k - 4 : k;
  return (key & ~15) | s;
}

// v^T tile-major: vt[g][kt][d][64 keys in vt_slot order] = FP16(v[t][g][d] *
// scale_g) for t = 64 kt + key < T, zero up to Tp, so one 64-key tile of a kv
// head is one contiguous 16 KB block.  64 x 64 tiles through LDS; grid
// (Tp/64, 8 heads x 2 dim halves).
__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t* __restrict__ vb, int T,
                                                      int Tp, const int32_t* __restrict__ vmax,
                                                      uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][66];
  const int t0 = blockIdx.x * 64;
  const int g = blockIdx.y >> 1, d0 = (blockIdx.y & 1) * 64;
  constexpr int KW = kAttnKVHeads * kAttnHeadDim;
  const float scale = attn_v_scale(vmax, g);
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int tt = i >> 6, dd = i & 63;
    const int t = t0 + tt;
    const float v = (t < T) ? __uint_as_float((uint32_t)vb[(int64_t)t * KW + g * kAttnHeadDim + d0 + dd] << 16)
                            : 0.f;
    tile[tt][dd] = __builtin_bit_cast(uint16_t, (_Float16)(v * scale));
  }
  __syncthreads();
  uint16_t* dst = vt + (((int64_t)g * (Tp / 64) + blockIdx.x) * kAttnHeadDim + d0) * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int dd = i >> 6, tt = i & 63;
    dst[dd * 64 + vt_slot(tt)] = tile[tt][dd];
  }
}

// ---------------------------------------------------------------------------
// Flash attention.  One workgroup per (query head, 128-query block), 4 waves;
// wave w owns queries q0 + 32w .. + 31, one per MFMA column (lane l: query l%32).
//   S^T = K Q^T:  A = 32 keys x 16 dims from LDS, B = the wave's queries from
//     registers; element i of lane l is key 8(i/4) + 4(l/32) + i%4 of the
//     32-key tile, query l%32 -- a query's scores sit in one lane and its
//     partner l^32, so the softmax needs one cross-lane step (permlane32 swap).
//   O^T = V^T P^T:  A = 32 dims x 16 keys of the scaled FP16 v^T from LDS
//     (keys in vt_slot order), B = the lane's own probabilities as FP16.
//     O^T's columns are queries, so the online-softmax rescale is lane-local.
// Keys go in 64-key tiles, double-buffered in LDS: the next tile's global
// loads are in flight while the current one is multiplied.  Only tiles that
// cross the diagonal, the window's edge or the sequence end are masked.
// The running max is raised lazily: probabilities are formed against a max
// that may trail the true one by up to 8 (log2 units), so they stay <= 256
// (exact in FP16 to the same relative precision) and the accumulators are
// rescaled only when some lane's max grows further; the final o / l is the
// same softmax.
// LDS per stage: K tile 64 keys x 256 B, 16-byte chunk c of key j at
// c ^ (j & 15); v^T tile 128 dims x 128 B, chunk c of dim d at c ^ vt_swz(d).
// Both are free of bank conflicts for these reads and writes.
__device__ __forceinline__ int vt_swz(int d) { return (d & 7) ^ (((d >> 2) ^ (d >> 3)) & 1); }

__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kFlashStage = 32768;  // bytes of one LDS stage (K 16 KB + v^T 16 KB)

__global__ __launch_bounds__(256, 2) void attn_flash_kernel(const uint16_t* __restrict__ qn,
                                                            const uint16_t* __restrict__ kn,
                                                            const uint16_t* __restrict__ vt,
                                                            const float* __restrict__ qkvg,
                                                            const int32_t* __restrict__ vmax,
                                                            int T, int Tp, int window,
                                                            uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kFlashStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, g = lane >> 5;
  constexpr int D = kAttnHeadDim;
  constexpr int NW = 2 * kAttnQHeads * D + 2 * kAttnKVHeads * D;
  constexpr int QPG = kAttnQHeads / kAttnKVHeads;  // query heads per kv head (6)
  // workgroup b runs on XCD b % 8: XCD x takes every query head of kv head x
  // (its K and v^T stay in that XCD's L2), longest query blocks first
  const int nqb = Tp / 128;
  const int kvh = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int h = kvh * QPG + bi % QPG;
  const int q0 = (nqb - 1 - bi / QPG) * 128;
  const int qi = q0 + 32 * wave + r;  // this lane's query

  // the wave's queries as the B operand: dims 16s + 8g .. + 7 of query qi
  uint4 qf[8];
  {
    const uint16_t* qp = qn + ((int64_t)h * Tp + qi) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const uint4*>(qp + 16 * s);
  }

  f32x16a o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max (log2 units), this lane's share of the sum
  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)

  const int j_hi = min(q0 + 128, T);  // keys [j_lo, j_hi)
  const int j_lo = window > 0 ? (max(0, q0 - window + 1) & ~63) : 0;
  const uint16_t* kbase = kn + (int64_t)kvh * Tp * D;
  const uint16_t* vbase = vt + (int64_t)kvh * Tp * D;  // [Tp/64][128][64]

  // global -> LDS copy of one tile by direct-to-LDS buffer loads: wave w
  // fills bytes 4096 w .. 4096 w + 4095 of the K tile and of the v^T tile,
  // 1 KB per load.  Lane l of a load lands at LDS offset 16 l of its 1 KB,
  // so each lane fetches the global chunk that belongs in that swizzled
  // slot: K rows 256 B (4 keys per load, slot l%16 of key l/16), v^T rows
  // 128 B (8 dims per load, slot l%8 of dim l/8).  Both tiles of 64 keys
  // start at byte 256 * j0 of their head's array.
  const __amdgpu_buffer_rsrc_t rs_k = buf_rsrc(kbase, (uint32_t)Tp * D * 2);
  const __amdgpu_buffer_rsrc_t rs_v = buf_rsrc(vbase, (uint32_t)Tp * D * 2);
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 4 * (4 * wave + i) + (lane >> 4), kc = lane & 15;
    koff[i] = (uint32_t)(key * 256 + ((kc ^ (key & 15)) << 4));
    const int d = 8 * (4 * wave + i) + (lane >> 3), vc = lane & 7;
    voff[i] = (uint32_t)(d * 128 + ((vc ^ vt_swz(d)) << 4));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds + 4096u * (uint32_t)wave;
  auto issue = [&](int j0, int stg) {
    const uint32_t kl = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)stg * kFlashStage);
    const uint32_t so = (uint32_t)j0 * (D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(kl + 1024u * i, koff[i], rs_k, so);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(kl + 16384u + 1024u * i, voff[i], rs_v, so);
  };

  // j_lo <= q0 < j_hi always (q0 < T), so the first tile exists
  issue(j_lo, 0);
  // the query registers are complete before the loop (otherwise their loads
  // sink into it and its MFMAs wait on every load in flight)
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(qf[s].x), "+v"(qf[s].y), "+v"(qf[s].z), "+v"(qf[s].w));
  int stage = 0;
  for (int j0 = j_lo; j0 < j_hi; j0 += 64, stage ^= 1) {
    // this wave's loads of tile j0 have landed; after the barrier every
    // wave's have, and nobody reads the other stage any more
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j0 + 64 < j_hi) issue(j0 + 64, stage ^ 1);
    const unsigned char* kl = lds + stage * kFlashStage;
    const unsigned char* vl = kl + 16384;

    // S^T for the 64 keys: two 32-key tiles
    f32x16a st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[t][i] = 0.f;
      const int key = 32 * t + r;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 kf = *reinterpret_cast<const uint4*>(kl + key * 256 + (((2 * s + g) ^ (key & 15)) << 4));
        st[t] = mfma32a(kf, qf[s], st[t]);
      }
    }
    // mask (edge tiles only) and this tile's max of the raw scores
    const bool full = j0 + 63 <= q0 && j0 + 63 < T && (window <= 0 || j0 >= q0 + 128 - window);
    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[t][i]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = j0 + 32 * t + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool ok = kj <= qi && kj < T && (window <= 0 || kj > qi - window);
          st[t][i] = ok ? st[t][i] : -INFINITY;
          mx = fmaxf(mx, st[t][i]);
        }
    }
    mx = swap_halves_max(mx) * sc;
    // lazy rescale, wave-uniform
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[t][i], sc, nm));
        st[t][i] = p;
        l_run += p;
      }

    // O^T += V^T P^T: MFMA (t, hf) covers keys 32t + 16hf + 0..15
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint4 pf = make_uint4(pack_f16x2_rne(st[t][8 * hf + 0], st[t][8 * hf + 1]),
                                    pack_f16x2_rne(st[t][8 * hf + 2], st[t][8 * hf + 3]),
                                    pack_f16x2_rne(st[t][8 * hf + 4], st[t][8 * hf + 5]),
                                    pack_f16x2_rne(st[t][8 * hf + 6], st[t][8 * hf + 7]));
        const int chunk = 4 * t + 2 * hf + g;  // 16-B chunk of the v^T row (slot order)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + r;
          const uint4 vf = *reinterpret_cast<const uint4*>(vl + d * 128 + ((chunk ^ vt_swz(d)) << 4));
          o[dt] = mfma32h(vf, pf, o[dt]);
        }
      }
  }

  // normalise, gate, store: o[dt][i] is dim 32dt + 8(i/4) + 4g + i%4 of query qi
  const float l_tot = swap_halves_sum(l_run);
  if (qi < T) {
    const float inv = 1.f / (l_tot * attn_v_scale(vmax, kvh));  // the scale is a power of two
    // gate logits: columns QW + 2 KW .. of the projection output
    const float* gl = qkvg + (int64_t)qi * NW + (kAttnQHeads + 2 * kAttnKVHeads) * D + h * D;
    uint16_t* dst = out + (int64_t)qi * (kAttnQHeads * D) + h * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        const f32x4 z = *reinterpret_cast<const f32x4*>(gl + d);
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = o[dt][4 * q4 + c] * inv / (1.f + expf(-z[c]));
        *reinterpret_cast<uint2*>(dst + d) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
  }
}

// ---------------------------------------------------------------------------
static int attn_tp(int64_t T) { return (int)((T + 127) / 128 * 128); }

// setup + 1. projections (FP32 q, k, v, gate logits)
hipError_t launch_attn_proj(hipStream_t st, const AttnArgs& a, int num_cu) {
  hipLaunchKernelGGL(attn_setup_kernel, dim3(1), dim3(64), 0, st, (int)a.T, a.counts, a.offsets,
                     a.tile_ctr, 32);
  GroupedArgs g{a.u, nullptr, a.w_qkvg, nullptr, nullptr, nullptr, a.counts, a.offsets,
                a.qkvg, kAttnProjRows, a.H, 1, a.T, a.tile_ctr, 0};
  return launch_plain_tiled(st, g, num_cu);
}

// 2-3. q/k norm and position, v layout
hipError_t launch_attn_prep(hipStream_t st, const AttnArgs& a) {
  const int Tp = attn_tp(a.T);
  int32_t* vmax = a.tile_ctr + kAttnVmaxSlot;
  hipLaunchKernelGGL(attn_prep_kernel, dim3(Tp), dim3(256), 0, st, a.qkvg, (int)a.T, a.global_layer,
                     a.theta, a.qn, a.kn, a.vb, Tp, a.vmx);
  hipLaunchKernelGGL(attn_vmax_kernel, dim3(kAttnKVHeads, kVmaxSlices), dim3(256), 0, st, a.vmx, (int)a.T, vmax);
  hipLaunchKernelGGL(attn_vt_kernel, dim3(Tp / 64, 2 * kAttnKVHeads), dim3(256), 0, st, a.vb,
                     (int)a.T, Tp, vmax, a.vt);
  return hipGetLastError();
}

// 4. attention with the gate
hipError_t launch_attn_flash(hipStream_t st, const AttnArgs& a) {
  const int Tp = attn_tp(a.T);
  const int32_t* vmax = a.tile_ctr + kAttnVmaxSlot;
  hipLaunchKernelGGL(attn_flash_kernel, dim3(Tp / 128 * kAttnQHeads), dim3(256), 0, st, a.qn, a.kn,
                     a.vt, a.qkvg, vmax, (int)a.T, Tp, a.global_layer ? 0 : a.window, a.o);
  return hipGetLastError();
}

// 5. output projection, bf16 result
hipError_t launch_attn_out(hipStream_t st, const AttnArgs& a, int num_cu) {
  GroupedArgs g{a.o, nullptr, a.w_o, nullptr, nullptr, nullptr, a.counts, a.offsets,
                a.y, a.H, kAttnQHeads * kAttnHeadDim, 1, a.T, a.tile_ctr + 16, 1};
  return launch_plain_tiled(st, g, num_cu);
}

}  // namespace beam
