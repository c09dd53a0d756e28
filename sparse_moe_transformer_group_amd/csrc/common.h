// Shared device helpers for the gfx950 kernels of libbeam_moe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte streaming load with the nontemporal hint: for data read once
// (expert weights at decode sizes); measured ~12% more HBM read bandwidth on
// gfx950 than ordinary loads for a pure stream.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_nt(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// Eight FP8 (E4M3) codes, byte i = element i, -> eight bf16 (exact: every
// E4M3 value is a bf16 value), in the 16-byte MFMA operand order.
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

// Two fp32 values -> a packed bf16 pair (a in the low half), round to
// nearest, ties to even: one v_cvt_pk_bf16_f32.  For finite inputs it gives
// exactly the integer rounding (add 0x7fff plus the lowest kept bit, keep the
// high half) -- checked on the device over all finite exponents, exact ties
// and subnormals; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// One 16x16x32 bf16 MFMA (gfx950): D = A(16x32) * B(32x16) + C.
// Lane l supplies A row (l % 16) and B column (l % 16), each with the 8
// k-values of its 16-byte operand; the k-slot each lane group (l / 16)
// stands for only needs to agree between A and B, since the products are
// summed.  The result holds rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// SiLU(g) * u in fp32: g * u / (1 + exp(-g)), with the hardware exponential
// and reciprocal (a few ulp in fp32; the result is then rounded once to
// bf16, whose ulp is 2^16 times coarser).  exp(-g) = inf for very negative g
// gives a reciprocal of 0 and h = 0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & 63; }

// The lane index, computed where it is used.  The asm is volatile, so the
// compiler can neither hoist it nor merge it with an earlier lane index: a
// kernel-long copy would be spilled under register pressure, and each
// reload of it waits for every memory access in flight, stores included.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// ---- direct-to-LDS buffer loads (tiled GEMM, flash attention)
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base` (raw access; word 3 is the
// gfx9-family raw-buffer format).  Accesses past the end read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One direct-to-LDS 16-byte-per-lane buffer load: lane l's 16 bytes at
// rsrc + voff + soff land at LDS byte lds + 16 l (lds wave-uniform).  Issued
// from inline asm so the compiler does not track it: its own wait insertion
// would otherwise order every later LDS read after all of these loads (it
// cannot tell ring stages apart), draining the pipeline.  Callers order them
// with an explicit vmcnt wait and a barrier.  No register is written.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t rs, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

}  // namespace beam
