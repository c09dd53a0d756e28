// One-time re-layout of expert weight matrices into the packed block layout
// the grouped GEMMs stream (layout defined in kernels.h).  Not part of the
// per-call path: a model loader packs each expert matrix once.
#include "common.h"
#include "kernels.h"

namespace beam {

// Workgroup (b, e): block b = rb * KB + kb of expert e; thread t moves the
// 16-byte chunks t and t + 256 (row j = q / 4, physical chunk q % 4).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int N, int K) {
  const int KB = K / kPackK;
  const int rb = blockIdx.x / KB, kb = blockIdx.x % KB;
  const int64_t e = blockIdx.y;
  const int64_t ebytes = packed_expert_bytes(N, K);
  unsigned char* out = reinterpret_cast<unsigned char*>(dst) + e * ebytes +
                       (int64_t)blockIdx.x * kPackBlockBytes;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = threadIdx.x + 256 * h;
    const int j = q >> 2, pc = q & 3;
    const int c = pc ^ pack_swz(j);
    const int row = rb * kPackRows + j;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < N) v = ld16(src + (e * N + row) * K + kb * kPackK + c * 8);
    st16(out + j * 64 + pc * 16, v);
  }
}

hipError_t launch_pack(hipStream_t st, const uint16_t* src, uint16_t* dst, int E, int N, int K) {
  const int blocks = ((N + kPackRows - 1) / kPackRows) * (K / kPackK);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks, E), dim3(256), 0, st, src, dst, N, K);
  return hipGetLastError();
}

}  // namespace beam

namespace beam {

// E4M3 code of v (|v| <= 448, v exactly representable in fp32), nearest
// value with ties to the even mantissa.  Subnormal range (|v| < 2^-6): grid
// step 2^-9, and the rounded count 0..8 is the code itself (8 = smallest
// normal).  Normal range [2^E, 2^(E+1)): step 2^(E-3), count 8..16; 16
// carries into the next binade.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 0x1p9f);
  } else {
    int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    float r = __builtin_rintf(__builtin_ldexpf(a, 3 - E));  // 8 .. 16, exact scaling
    if (r >= 16.0f) {
      ++E;
      r = 8.0f;
    }
    code = (uint32_t)((E + 7) << 3) | ((uint32_t)r - 8u);
  }
  return code | sign;
}

// Workgroup (rb, e): 128 rows of expert e.  Pass 1: per-row max |w| (bf16
// magnitudes compare as integers) -> scale exponent.  Pass 2: quantise and
// write the row block's K/32 blocks.  Thread t: row t/2, half t%2.
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint16_t* __restrict__ src,
                                                       uint8_t* __restrict__ dst,
                                                       float* __restrict__ scales, int N, int K) {
  __shared__ uint32_t s_amax[256];
  __shared__ int s_exp[kPackRows];
  const int rb = blockIdx.x;
  const int64_t e = blockIdx.y;
  const int t = threadIdx.x, j = t >> 1, half = t & 1;
  const int row = rb * kPackRows + j;
  const bool live = row < N;
  const uint16_t* wrow = src + (e * N + (live ? row : 0)) * K;

  uint32_t m = 0;
  if (live) {
    for (int k = half * 8; k < K; k += 16) {
      const uint4 v = ld16(wrow + k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7fffu);
        m = max(m, (w[i] >> 16) & 0x7fffu);
      }
    }
  }
  s_amax[t] = m;
  __syncthreads();
  if (half == 0) {
    const uint32_t am = max(s_amax[t], s_amax[t + 1]);
    int ex = 0;
    if (am != 0) {
      int x;
      const float f = frexpf(bf16_to_f32(am), &x);  // am = f * 2^x, f in [0.5, 1)
      ex = x - 9 + (f > 0.875f ? 1 : 0);             // 448 = 0.875 * 2^9
    }
    s_exp[j] = ex;
    if (live) scales[e * N + row] = __builtin_ldexpf(1.0f, ex);
  }
  __syncthreads();
  const int ex = s_exp[j];

  const int KB = K / kPackK;
  uint8_t* out = dst + e * packed8_expert_bytes(N, K) + (int64_t)rb * KB * kPack8BlockBytes;
  for (int kb = 0; kb < KB; ++kb) {
    // this thread: logical chunks 2*half and 2*half + 1 (16 weights) of row j
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    if (live) {
      const uint16_t* p = wrow + kb * kPackK + half * 16;
      const uint4 v0 = ld16(p), v1 = ld16(p + 8);
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t b = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
        const uint32_t c = e4m3_code(__builtin_ldexpf(bf16_to_f32(b), -ex));
        q[i >> 2] |= c << (8 * (i & 3));
      }
    }
    uint8_t* blk = out + (int64_t)kb * kPack8BlockBytes + j * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * half + h;
      *reinterpret_cast<uint2*>(blk + ((c ^ pack8_swz(j)) << 3)) = make_uint2(q[2 * h], q[2 * h + 1]);
    }
  }
}

hipError_t launch_pack_fp8(hipStream_t st, const uint16_t* src, uint8_t* dst, float* scales, int E,
                           int N, int K) {
  const int nrb = (N + kPackRows - 1) / kPackRows;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3(nrb, E), dim3(256), 0, st, src, dst, scales, N, K);
  return hipGetLastError();
}

}  // namespace beam
