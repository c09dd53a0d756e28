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
