// Internal declarations shared by the HIP translation units of libmoe.so.
// Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- limits -------------------------------------------------------------
constexpr int kMaxExperts = 256;     // selection range of the fused router
constexpr int kMaxRouteK = 16;       // one 16-lane group keeps one pick per lane
#ifndef MOE_DISPATCH_TOKENS
#define MOE_DISPATCH_TOKENS 16
#endif
constexpr int kDispatchTokens = MOE_DISPATCH_TOKENS;  // tokens per dispatch sub-chunk

// ---- vector types -------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 (bf16 is the upper half of a binary32) ---------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- launchers (each validates nothing: the C ABI layer has done it) -----
// Router.  wgt is the fragment-major packed gate (bf16 path only).
int route_padded_experts(int E);
int route_gate_rows(int H);  // H rounded up to whole 64-wide steps (packed gate)
hipError_t launch_gate_transpose(const uint16_t* gate_w, int H, int E, uint16_t* wgt,
                                 int32_t* counts, hipStream_t s);
hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* wgt, const float* bias,
                             int64_t N, int H, int E, int K, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s);
hipError_t launch_route_f32(const float* x, const float* gate_w, const float* bias, int64_t N,
                            int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                            hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// Dispatch.
int64_t dispatch_num_sub(int64_t N);
hipError_t launch_dispatch(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                           int E, int K, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, void* x_perm, int32_t* blockcnt, hipStream_t s);

// Combine.
hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t N, int H,
                          int K, bool bf16, void* out, hipStream_t s);

}  // namespace moe
