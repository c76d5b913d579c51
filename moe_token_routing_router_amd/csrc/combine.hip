// Weighted MoE combine for gfx950: out[n,:] = sum_k w[n,k] * y[inv[n*K+k],:].
//
// Method: "Building a MoE training stack in 10k lines of Python", section 6.1
// "Model protocol first": forward_aggregate takes the expert outputs, the
// index that undoes the dispatch and the top-K weights and forms the weighted
// expert output (the residual add is not part of this call).
//
// One gather per token, no scatter-add: each output vector of 16 bytes is
// owned by one lane, which loads its K source vectors (independent 16-byte
// loads, all in flight together), accumulates in fp32 with k ascending from
// 0, rounds once and stores.  No float atomics, so the result is
// deterministic.  A row index outside [0, N*K) contributes nothing.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kCombineTokens = 8;  // tokens per workgroup

template <bool BF16>
__device__ __forceinline__ void fma_vec(float (&acc)[BF16 ? 8 : 4], float w, uint4 v) {
  if constexpr (BF16) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = fmaf(w, bf16_lo(u[j]), acc[2 * j]);
      acc[2 * j + 1] = fmaf(w, bf16_hi(u[j]), acc[2 * j + 1]);
    }
  } else {
    acc[0] = fmaf(w, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(w, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(w, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(w, __uint_as_float(v.w), acc[3]);
  }
}

template <bool BF16>
__device__ __forceinline__ uint4 pack_vec(const float (&acc)[BF16 ? 8 : 4]) {
  uint4 o;
  if constexpr (BF16) {
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
  } else {
    o.x = __float_as_uint(acc[0]);
    o.y = __float_as_uint(acc[1]);
    o.z = __float_as_uint(acc[2]);
    o.w = __float_as_uint(acc[3]);
  }
  return o;
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t N,
                                                      int K, int row_vecs,
                                                      uint4* __restrict__ out) {
  constexpr int L = BF16 ? 8 : 4;
  extern __shared__ int dyn[];  // rows[kCombineTokens*K] then weights
  int* lrow = dyn;
  float* lw = reinterpret_cast<float*>(dyn + kCombineTokens * K);
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * kCombineTokens;
  const int ntok = (int)min((int64_t)kCombineTokens, N - n0);
  const int64_t T = N * K;
  for (int j = tid; j < ntok * K; j += 256) {
    const int rrow = inv[n0 * K + j];
    lrow[j] = ((unsigned)rrow < (unsigned long long)T) ? rrow : -1;
    lw[j] = w[n0 * K + j];
  }
  __syncthreads();

  const int total = ntok * row_vecs;
  uint4* os = out + n0 * (int64_t)row_vecs;
  for (int idx = tid; idx < total; idx += 256) {
    const int tt = idx / row_vecs;
    const int c = idx - tt * row_vecs;
    float acc[L];
#pragma unroll
    for (int j = 0; j < L; ++j) acc[j] = 0.f;
    const int* rr = lrow + tt * K;
    const float* ww = lw + tt * K;
    int k = 0;
    // groups of 4 independent gathers in flight
    for (; k + 4 <= K; k += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rrow = rr[k + u];
        v[u] = rrow >= 0 ? y[(int64_t)rrow * row_vecs + c] : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (rr[k + u] >= 0) fma_vec<BF16>(acc, ww[k + u], v[u]);
    }
    for (; k < K; ++k) {
      const int rrow = rr[k];
      if (rrow >= 0) fma_vec<BF16>(acc, ww[k], y[(int64_t)rrow * row_vecs + c]);
    }
    os[(int64_t)tt * row_vecs + c] = pack_vec<BF16>(acc);
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t N, int H,
                          int K, bool bf16, void* out, hipStream_t s) {
  const int64_t blocks = (N + kCombineTokens - 1) / kCombineTokens;
  const int row_vecs = bf16 ? H / 8 : H / 4;
  const size_t dyn = (sizeof(int) + sizeof(float)) * (size_t)kCombineTokens * K;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), dyn, s,
                       reinterpret_cast<const uint4*>(y), inv, w, N, K, row_vecs,
                       reinterpret_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), dyn, s,
                       reinterpret_cast<const uint4*>(y), inv, w, N, K, row_vecs,
                       reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
