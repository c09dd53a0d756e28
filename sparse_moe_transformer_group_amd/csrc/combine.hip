// Combine, RMSNorm and scaled-residual kernels (gfx950).
//
// Combine (page "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen,
// anpassen und skalieren können", section "Mixture of Experts"): a token's
// output is the router-weighted sum of its experts' outputs; the weights
// arrive normalised and already multiplied by 2.5.
// Norms and residual (same page, section "Residual Stream"): each sublayer is
// normalised before and after, in FP32; the embedding is residual step 1 and
// step s >= 2 keeps sqrt((s-1)/s) of the stream and adds 1/sqrt(s) of the
// sublayer output.
#include "common.h"
#include "kernels.h"

namespace beam {

// 8-byte store marked nontemporal, for output written once and not re-read
// by this kernel.
__device__ __forceinline__ void st8_nt(void* p, uint2 v) {
  __builtin_nontemporal_store((uint64_t)v.x | ((uint64_t)v.y << 32), reinterpret_cast<uint64_t*>(p));
}

// y[t, :] = bf16( sum_j w[t,j] * o[row_of[t*k+j], :] ): FP32 fused multiply-adds
// in slot order j = 0..k-1, one rounding at the end.  Workgroup (c, t) covers
// 1024 columns of token t; each thread issues the loads of all its slots
// (16-byte loads of the FP32 partial rows) before summing them in order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int H, int k,
                                                      uint16_t* __restrict__ y) {
  const int64_t t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 v[8];
    float wj[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int row = (j < k) ? row_of[t * k + j] : -1;
      ok[u] = row >= 0;  // a dropped slot (id outside [0, E)) contributes nothing
      wj[u] = ok[u] ? w[t * k + j] : 0.f;
      // o is read exactly once: nontemporal loads keep it from displacing
      // cached data (measured 11% faster)
      v[u] = ok[u] ? __builtin_bit_cast(f32x4, ld16_nt(o + (int64_t)row * H + c))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!ok[u]) continue;
      a0 = fmaf(wj[u], v[u][0], a0);
      a1 = fmaf(wj[u], v[u][1], a1);
      a2 = fmaf(wj[u], v[u][2], a2);
      a3 = fmaf(wj[u], v[u][3], a3);
    }
  }
  // nontemporal store: 5% faster at T = 8192 (the 84 MB of y compete with
  // the 1.34 GB read of o; plain stores cost 0.053 ms over a store-free run)
  st8_nt(y + t * H + c, make_uint2(pack_bf16x2_rne(a0, a1), pack_bf16x2_rne(a2, a3)));
}

hipError_t launch_combine(hipStream_t st, const float* o, const int32_t* row_of, const float* w, int T,
                          int H, int k, uint16_t* y) {
  dim3 grid((H + 1023) / 1024, T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, o, row_of, w, H, k, y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_init_kernel(const uint16_t* __restrict__ x,
                                                          float* __restrict__ out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const uint2 v = *reinterpret_cast<const uint2*>(x + i);
  *reinterpret_cast<f32x4*>(out + i) =
      f32x4{bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffffu),
            bf16_to_f32(v.y >> 16)};
}

hipError_t launch_stream_init(hipStream_t st, const uint16_t* x, float* out, int64_t T, int H) {
  const int64_t n = T * H;  // multiple of 4 (H % 64 == 0)
  hipLaunchKernelGGL(stream_init_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, x,
                     out, n);
  return hipGetLastError();
}

// Block sum of one float per thread, in a fixed order (wave butterflies, then
// the 4 wave sums in wave order).
__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Inverse RMS of one row of H fp32 values held 4 per thread-iteration.
__device__ __forceinline__ float row_inv_rms(float ss, int H, float eps, float* red) {
  const float tot = block_sum_256(ss, red);
  return 1.0f / sqrtf(tot / (float)H + eps);
}

// out[t,:] = bf16( in[t,:] / sqrt(mean(in[t,:]^2) + eps) ).  One workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ in,
                                                      uint16_t* __restrict__ out, int H, float eps) {
  __shared__ float red[4];
  const float* row = in + (int64_t)blockIdx.x * H;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    ss = fmaf(v[0], v[0], ss);
    ss = fmaf(v[1], v[1], ss);
    ss = fmaf(v[2], v[2], ss);
    ss = fmaf(v[3], v[3], ss);
  }
  const float inv = row_inv_rms(ss, H, eps, red);
  uint16_t* orow = out + (int64_t)blockIdx.x * H;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    *reinterpret_cast<uint2*>(orow + c) =
        make_uint2(pack_bf16x2_rne(v[0] * inv, v[1] * inv), pack_bf16x2_rne(v[2] * inv, v[3] * inv));
  }
}

hipError_t launch_rmsnorm(hipStream_t st, const float* in, uint16_t* out, int64_t T, int H, float eps) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, st, in, out, H, eps);
  return hipGetLastError();
}

// stream[t,:] = keep * stream[t,:] + add * RMSNorm(float(y[t,:])).
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* __restrict__ y,
                                                       float* __restrict__ stream, int H, float eps,
                                                       float keep, float add) {
  __shared__ float red[4];
  const uint16_t* yr = y + (int64_t)blockIdx.x * H;
  float* sr = stream + (int64_t)blockIdx.x * H;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const uint2 v = *reinterpret_cast<const uint2*>(yr + c);
    const float f0 = bf16_to_f32(v.x & 0xffffu), f1 = bf16_to_f32(v.x >> 16);
    const float f2 = bf16_to_f32(v.y & 0xffffu), f3 = bf16_to_f32(v.y >> 16);
    ss = fmaf(f0, f0, ss);
    ss = fmaf(f1, f1, ss);
    ss = fmaf(f2, f2, ss);
    ss = fmaf(f3, f3, ss);
  }
  const float inv = row_inv_rms(ss, H, eps, red);
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const uint2 v = *reinterpret_cast<const uint2*>(yr + c);
    f32x4 s = *reinterpret_cast<const f32x4*>(sr + c);
    s[0] = keep * s[0] + add * (bf16_to_f32(v.x & 0xffffu) * inv);
    s[1] = keep * s[1] + add * (bf16_to_f32(v.x >> 16) * inv);
    s[2] = keep * s[2] + add * (bf16_to_f32(v.y & 0xffffu) * inv);
    s[3] = keep * s[3] + add * (bf16_to_f32(v.y >> 16) * inv);
    *reinterpret_cast<f32x4*>(sr + c) = s;
  }
}

hipError_t launch_residual(hipStream_t st, const uint16_t* y, float* stream, int64_t T, int H, float eps,
                           int step) {
  const float keep = (float)sqrt((double)(step - 1) / (double)step);
  const float add = (float)(1.0 / sqrt((double)step));
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)T), dim3(256), 0, st, y, stream, H, eps, keep, add);
  return hipGetLastError();
}

}  // namespace beam
