// Token permutation for the grouped expert GEMMs (gfx950).
//
// Each token runs only its k chosen experts (page "Willkommen Beam: ein
// offenes 501B-Modell, das Sie besitzen, anpassen und skalieren können",
// section "Mixture of Experts"), so the (token, slot) assignments are sorted
// by expert to give every expert a contiguous block of rows.  The sort is a
// stable counting sort, fully deterministic (integer atomics only count):
//   1. per chunk of 512 assignments, an LDS histogram over experts;
//   2. one workgroup scans the chunk histograms per expert (chunk-major) and
//      the expert totals (expert-major) -> counts, offsets, chunk bases;
//   3. per chunk, the rank of an assignment among the chunk's assignments to
//      the same expert is the popcount of a per-expert LDS bitmask below it;
//      row = offsets[e] + chunk base + rank.
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kMaxE = 512;
constexpr int kMaskWords = kPermChunk / 32;

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ ids, int64_t Tk,
                                                        int E, int32_t* __restrict__ block_hist) {
  __shared__ int h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int64_t a = base + i;
    if (a < Tk) {
      const int e = ids[a];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) block_hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One workgroup of 1024 threads: thread (slice, e) walks a contiguous range of
// chunks for expert e.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ block_hist,
                                                         int NB, int E,
                                                         int32_t* __restrict__ block_base,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ user_counts,
                                                         int32_t* __restrict__ clear16) {
  __shared__ int part[1024];
  __shared__ int scan[kMaxE];
  if (clear16 && threadIdx.x < 16) clear16[threadIdx.x] = 0;  // the GEMMs' tile-claim counters
  const int tid = threadIdx.x;
  const int SL = 1024 / E;  // >= 2 since E <= 512
  const int e = tid % E, sl = tid / E;
  const bool on = sl < SL;
  const int b0 = on ? (int)((int64_t)sl * NB / SL) : 0;
  const int b1 = on ? (int)((int64_t)(sl + 1) * NB / SL) : 0;

  int sum = 0;
#pragma unroll 8
  for (int b = b0; b < b1; ++b) sum += block_hist[(int64_t)b * E + e];
  if (on) part[tid] = sum;
  __syncthreads();

  int pre = 0, tot = 0;
  if (on) {
    for (int s = 0; s < SL; ++s) {
      const int v = part[s * E + e];
      if (s < sl) pre += v;
      tot += v;
    }
  }
  if (tid < E) scan[tid] = tot;
  __syncthreads();
  for (int off = 1; off < E; off <<= 1) {  // inclusive Hillis-Steele scan
    int v = 0;
    if (tid < E && tid >= off) v = scan[tid - off];
    __syncthreads();
    if (tid < E) scan[tid] += v;
    __syncthreads();
  }
  const int excl = (on ? scan[e] : 0) - tot;
  if (tid < E) {
    counts[e] = tot;
    offsets[e] = excl;
    if (user_counts) user_counts[e] = tot;
    if (e == E - 1) offsets[E] = scan[E - 1];
  }
  if (on) {
    int run = excl + pre;
    for (int b = b0; b < b1; ++b) {
      const int64_t idx = (int64_t)b * E + e;
      const int v = block_hist[idx];
      block_base[idx] = run;
      run += v;
    }
  }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                           int64_t Tk, int k, int E,
                                                           const int32_t* __restrict__ block_base,
                                                           int32_t* __restrict__ sorted_tokens,
                                                           int32_t* __restrict__ row_of) {
  __shared__ uint32_t mask[kMaxE * kMaskWords];
  for (int i = threadIdx.x; i < E * kMaskWords; i += 256) mask[i] = 0u;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPermChunk;
  int ev[kPermChunk / 256];
#pragma unroll
  for (int r = 0; r < kPermChunk / 256; ++r) {
    const int i = threadIdx.x + 256 * r;
    const int64_t a = base + i;
    const int e = (a < Tk) ? ids[a] : -1;
    ev[r] = e;
    if ((unsigned)e < (unsigned)E) atomicOr(&mask[e * kMaskWords + (i >> 5)], 1u << (i & 31));
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPermChunk / 256; ++r) {
    const int i = threadIdx.x + 256 * r;
    const int64_t a = base + i;
    if (a >= Tk) continue;
    const int e = ev[r];
    if ((unsigned)e >= (unsigned)E) {
      row_of[a] = -1;
      continue;
    }
    const uint32_t* m = mask + e * kMaskWords;
    const int w = i >> 5;
    int rank = __popc(m[w] & ((1u << (i & 31)) - 1u));
    for (int j = 0; j < w; ++j) rank += __popc(m[j]);
    const int pos = block_base[(int64_t)blockIdx.x * E + e] + rank;
    sorted_tokens[pos] = (int)(a / k);
    row_of[a] = pos;
  }
}

// Whole permutation in one workgroup when all assignments fit one chunk
// (decode-size batches): histogram, scan and ranked scatter without the two
// extra launches.  Same results as the three-kernel path.
__global__ __launch_bounds__(256) void perm_single_kernel(const int32_t* __restrict__ ids, int Tk, int k,
                                                          int E, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_tokens,
                                                          int32_t* __restrict__ row_of,
                                                          int32_t* __restrict__ user_counts,
                                                          int32_t* __restrict__ clear16) {
  __shared__ uint32_t mask[kMaxE * kMaskWords];
  __shared__ int hist[kMaxE];
  __shared__ int scan[kMaxE];
  if (clear16 && threadIdx.x < 16) clear16[threadIdx.x] = 0;  // the GEMMs' tile-claim counters
  for (int i = threadIdx.x; i < E * kMaskWords; i += 256) mask[i] = 0u;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  int ev[kPermChunk / 256];
#pragma unroll
  for (int r = 0; r < kPermChunk / 256; ++r) {
    const int i = threadIdx.x + 256 * r;
    const int e = (i < Tk) ? ids[i] : -1;
    ev[r] = e;
    if ((unsigned)e < (unsigned)E) {
      atomicOr(&mask[e * kMaskWords + (i >> 5)], 1u << (i & 31));
      atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) scan[e] = hist[e];
  __syncthreads();
  for (int off = 1; off < E; off <<= 1) {  // inclusive Hillis-Steele scan
    int v0 = 0, v1 = 0;
    const int e0 = threadIdx.x, e1 = threadIdx.x + 256;
    if (e0 < E && e0 >= off) v0 = scan[e0 - off];
    if (e1 < E && e1 >= off) v1 = scan[e1 - off];
    __syncthreads();
    if (e0 < E) scan[e0] += v0;
    if (e1 < E) scan[e1] += v1;
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += 256) {
    counts[e] = hist[e];
    offsets[e] = scan[e] - hist[e];
    if (user_counts) user_counts[e] = hist[e];
    if (e == E - 1) offsets[E] = scan[E - 1];
  }
#pragma unroll
  for (int r = 0; r < kPermChunk / 256; ++r) {
    const int i = threadIdx.x + 256 * r;
    if (i >= Tk) continue;
    const int e = ev[r];
    if ((unsigned)e >= (unsigned)E) {
      row_of[i] = -1;
      continue;
    }
    const uint32_t* m = mask + e * kMaskWords;
    const int w = i >> 5;
    int rank = __popc(m[w] & ((1u << (i & 31)) - 1u));
    for (int j = 0; j < w; ++j) rank += __popc(m[j]);
    const int pos = scan[e] - hist[e] + rank;
    sorted_tokens[pos] = i / k;
    row_of[i] = pos;
  }
}

hipError_t launch_permute(hipStream_t st, const int32_t* ids, int64_t Tk, int k, int E,
                          int32_t* block_hist, int32_t* block_base, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_tokens, int32_t* row_of,
                          int32_t* user_counts, int32_t* clear16) {
  const int64_t NB = perm_blocks(Tk);
  if (NB == 1) {
    hipLaunchKernelGGL(perm_single_kernel, dim3(1), dim3(256), 0, st, ids, (int)Tk, k, E, counts,
                       offsets, sorted_tokens, row_of, user_counts, clear16);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)NB), dim3(256), 0, st, ids, Tk, E, block_hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, block_hist, (int)NB, E, block_base,
                     counts, offsets, user_counts, clear16);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)NB), dim3(256), 0, st, ids, Tk, k, E,
                     block_base, sorted_tokens, row_of);
  return hipGetLastError();
}

// Routing of a dense layer split into C chunks of its intermediate dimension:
// every token goes to chunk j in slot j with weight 1.
__global__ __launch_bounds__(256) void dense_routing_kernel(int32_t* __restrict__ ids,
                                                            float* __restrict__ w, int64_t n, int C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    ids[i] = (int32_t)(i % C);
    w[i] = 1.0f;
  }
}

hipError_t launch_dense_routing(hipStream_t st, int32_t* ids, float* w, int64_t T, int C) {
  const int64_t n = T * C;
  hipLaunchKernelGGL(dense_routing_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids, w,
                     n, C);
  return hipGetLastError();
}

}  // namespace beam
