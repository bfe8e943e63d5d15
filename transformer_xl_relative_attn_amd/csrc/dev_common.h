// Device-side helpers shared by the libtxl HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "txl_internal.h"

namespace txl {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load element i of a tensor stored as dtype (f32 / bf16) and widen to f32.
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int32_t dtype) {
  if (dtype == TXL_F32) return static_cast<const float*>(p)[i];
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float x, int32_t dtype) {
  if (dtype == TXL_F32)
    static_cast<float*>(p)[i] = x;
  else
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
}

// Address of virtual row `v` of a GEMM operand (NULL = zero row).  `esize` is
// the element size in bytes of the source tensor.
__device__ __forceinline__ const char* row_address(const RowSrc& s, int32_t v, int esize) {
  const char* p = nullptr;
  switch (s.kind) {
    case ROW_PLAIN:
      if (v < s.rows) p = static_cast<const char*>(s.p0) + (int64_t)v * s.ld * esize;
      break;
    case ROW_HEADPAD: {
      const int32_t head = magic_quot(v, s.qmul, s.qshift), c = v - head * s.dp;
      if (c < s.dh) p = static_cast<const char*>(s.p0) + (int64_t)(head * s.dh + c) * s.ld * esize;
      break;
    }
    default: {  // ROW_HTILDE
      const int32_t b = magic_quot(v, s.qmul, s.qshift), r = v - b * s.np - s.lead;
      if (r < 0) {
      } else if (r < s.M) {
        int32_t slot = r + s.start;
        if (slot >= s.M) slot -= s.M;
        p = static_cast<const char*>(s.p0) + ((int64_t)b * s.M + slot) * s.ld * esize;
      } else if (r < s.M + s.L) {
        p = static_cast<const char*>(s.p1) + ((int64_t)b * s.L + (r - s.M)) * s.ld * esize;
      }
      break;
    }
  }
  return p;
}

__device__ __forceinline__ int64_t axis_off(const AxisMap& a, int32_t x) {
  return axis_offset(a, x);
}

__device__ __forceinline__ int64_t col_off(const OutDst& o, int32_t n) {
  return axis_offset(o.col, n) + axis_offset(o.col2, n);
}

// Epilogue store of one accumulator element.
__device__ __forceinline__ void epi_store(const OutDst& o, int64_t off, float x) {
  if (o.flags & EPI_RESID) x += o.resid[off];
  if (o.flags & EPI_RELU) x = fmaxf(x, 0.0f);
  store_from_f32(o.p, off, x, o.dtype);
}

// Wave-local LDS ordering: all LDS operations of this wave issued before are
// complete and the compiler may not move memory operations across.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
}

// Map a linear block id to a work item so that consecutive work items run on
// the same XCD (blocks are dealt to the 8 XCDs round-robin).  `total` work
// items, `padded` = total rounded up to a multiple of 8 blocks launched.
__device__ __forceinline__ int32_t xcd_swizzle(int32_t bid, int32_t padded) {
  int32_t per = padded >> 3;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace txl
