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
// deterministic.  A row index outside [0, N*K) contributes nothing.  For the
// common K (1, 2, 4, 8) each lane works on U output vectors at once, so
// U*K independent row gathers are in flight per lane.
#include "moe_internal.h"

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_COMBINE_TOKENS
#define MOE_COMBINE_TOKENS 2   // tokens per workgroup (K = 2: MOE_COMBINE_TOKENS2)
#endif
#ifndef MOE_COMBINE_TOKENS2
#define MOE_COMBINE_TOKENS2 1  // tokens per workgroup for K = 2
#endif
#ifndef MOE_COMBINE_U2
#define MOE_COMBINE_U2 2        // output vectors per lane in flight for K = 2
#endif
#ifndef MOE_COMBINE_U4
#define MOE_COMBINE_U4 2        // ... for K = 4
#endif
#ifndef MOE_COMBINE_U8
#define MOE_COMBINE_U8 4        // ... for K = 8
#endif
#ifndef MOE_COMBINE_CAP_KIB
#define MOE_COMBINE_CAP_KIB 144 // rows in flight per CU (KiB) for large batches (gather_lds_cap)
#endif
#ifndef MOE_COMBINE_NT_LOAD
#define MOE_COMBINE_NT_LOAD 1   // non-temporal loads of y (each row is read once)
#endif
#ifndef MOE_COMBINE_NT_STORE
#define MOE_COMBINE_NT_STORE 1  // non-temporal stores of out
#endif

namespace moe {

namespace {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_vec(const u32x4* p) {
#if MOE_COMBINE_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ void st_vec(u32x4* p, u32x4 v) {
#if MOE_COMBINE_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

template <bool BF16>
__device__ __forceinline__ void fma_vec(float (&acc)[BF16 ? 8 : 4], float w, u32x4 v) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = fmaf(w, bf16_lo(v[j]), acc[2 * j]);
      acc[2 * j + 1] = fmaf(w, bf16_hi(v[j]), acc[2 * j + 1]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, __uint_as_float(v[j]), acc[j]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack_vec(const float (&acc)[BF16 ? 8 : 4]) {
  u32x4 o;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(acc[j]);
  }
  return o;
}

// KT > 0: K known at compile time; U output vectors per iteration, so U*KT
// independent 16-byte gathers are in flight per lane.  KT == 0: any K, one
// output vector per iteration, gathers in groups of 4.
// With `res`, the residual row is added after the K expert terms (the
// forward_aggregate of the same page: weighted expert output + residual).
template <bool BF16>
__device__ __forceinline__ void add_vec(float (&acc)[BF16 ? 8 : 4], u32x4 v) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_lo(v[j]);
      acc[2 * j + 1] += bf16_hi(v[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += __uint_as_float(v[j]);
  }
}

template <bool BF16, int KT, int U, int TPW, bool RES>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t N,
                                                      int Krt, int row_vecs,
                                                      const u32x4* res,  // may alias out
                                                      u32x4* out) {
  constexpr int L = BF16 ? 8 : 4;
  const int K = KT > 0 ? KT : Krt;
  extern __shared__ int dyn[];  // rows[TPW*K] then weights
  int* lrow = dyn;
  float* lw = reinterpret_cast<float*>(dyn + TPW * K);
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * TPW;
  const int ntok = (int)min((int64_t)TPW, N - n0);
  const int64_t T = N * K;
  for (int j = tid; j < ntok * K; j += 256) {
    const int rrow = inv[n0 * K + j];
    lrow[j] = ((unsigned)rrow < (unsigned long long)T) ? rrow : -1;
    lw[j] = w ? w[n0 * K + j] : 1.f;  // no weights: the dispatch backward (a plain sum)
  }
  __syncthreads();

  const int total = ntok * row_vecs;
  u32x4* os = out + n0 * (int64_t)row_vecs;
  const u32x4* rs = RES ? res + n0 * (int64_t)row_vecs : nullptr;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if constexpr (KT > 0) {
    for (int base = tid; base < total; base += 256 * U) {
      u32x4 v[U][KT], rv[RES ? U : 1];
      int tt[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = min(base + u * 256, total - 1);
        tt[u] = idx / row_vecs;
        c[u] = idx - tt[u] * row_vecs;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const int rrow = lrow[tt[u] * KT + k];
          v[u][k] = rrow >= 0 ? ld_vec(y + (int64_t)rrow * row_vecs + c[u]) : zero;
        }
        if constexpr (RES) rv[u] = ld_vec(rs + idx);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float acc[L];
#pragma unroll
        for (int j = 0; j < L; ++j) acc[j] = 0.f;
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (lrow[tt[u] * KT + k] >= 0) fma_vec<BF16>(acc, lw[tt[u] * KT + k], v[u][k]);
        if constexpr (RES) add_vec<BF16>(acc, rv[u]);
        if (base + u * 256 < total) st_vec(os + (int64_t)tt[u] * row_vecs + c[u], pack_vec<BF16>(acc));
      }
    }
  } else {
    for (int idx = tid; idx < total; idx += 256) {
      const int tt = idx / row_vecs;
      const int c = idx - tt * row_vecs;
      float acc[L];
#pragma unroll
      for (int j = 0; j < L; ++j) acc[j] = 0.f;
      const int* rr = lrow + tt * K;
      const float* ww = lw + tt * K;
      int k = 0;
      for (; k + 4 <= K; k += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = rr[k + u] >= 0 ? ld_vec(y + (int64_t)rr[k + u] * row_vecs + c) : zero;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (rr[k + u] >= 0) fma_vec<BF16>(acc, ww[k + u], v[u]);
      }
      for (; k < K; ++k)
        if (rr[k] >= 0) fma_vec<BF16>(acc, ww[k], ld_vec(y + (int64_t)rr[k] * row_vecs + c));
      if constexpr (RES) add_vec<BF16>(acc, ld_vec(rs + idx));
      st_vec(os + (int64_t)tt * row_vecs + c, pack_vec<BF16>(acc));
    }
  }
}

template <bool BF16, int KT, int U, int TPW = MOE_COMBINE_TOKENS>
hipError_t launch_k(const void* y, const int32_t* inv, const float* w, int64_t N, int H, int K,
                    const void* res, void* out, hipStream_t s) {
  const int64_t blocks = (N + TPW - 1) / TPW;
  const int row_vecs = BF16 ? H / 8 : H / 4;
  size_t dyn = (sizeof(int) + sizeof(float)) * (size_t)TPW * K;
  // a workgroup moves TPW tokens' K rows read, the residual and the output:
  // at N = 16384, H = 4096, K = 2 (24 KiB) six workgroups per CU, with the
  // residual (32 KiB) four: combine 66.6 -> 65.1 us, aggregate
  // 88.3 -> 84.1 us
  const size_t row_bytes = (size_t)row_vecs * 16;
  dyn = std::max(dyn, gather_lds_cap(N, row_bytes, (size_t)TPW * (K + 1 + (res ? 1 : 0)),
                                     (size_t)MOE_COMBINE_CAP_KIB * 1024));
  if (res)
    hipLaunchKernelGGL((combine_kernel<BF16, KT, U, TPW, true>), dim3((unsigned)blocks), dim3(256),
                       dyn, s, reinterpret_cast<const u32x4*>(y), inv, w, N, K, row_vecs,
                       reinterpret_cast<const u32x4*>(res), reinterpret_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL((combine_kernel<BF16, KT, U, TPW, false>), dim3((unsigned)blocks),
                       dim3(256), dyn, s, reinterpret_cast<const u32x4*>(y), inv, w, N, K,
                       row_vecs, nullptr, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const void* y, const int32_t* inv, const float* w, int64_t N, int H,
                        int K, const void* res, void* out, hipStream_t s) {
  switch (K) {
    case 1: return launch_k<BF16, 1, 8>(y, inv, w, N, H, K, res, out, s);
    case 2:
      return launch_k<BF16, 2, MOE_COMBINE_U2, MOE_COMBINE_TOKENS2>(y, inv, w, N, H, K, res, out,
                                                                    s);
    case 4: return launch_k<BF16, 4, MOE_COMBINE_U4>(y, inv, w, N, H, K, res, out, s);
    case 8: return launch_k<BF16, 8, MOE_COMBINE_U8>(y, inv, w, N, H, K, res, out, s);
    default: return launch_k<BF16, 0, 1>(y, inv, w, N, H, K, res, out, s);
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t N, int H,
                          int K, bool bf16, void* out, hipStream_t s, const void* residual) {
  return bf16 ? launch_dtype<true>(y, inv, w, N, H, K, residual, out, s)
              : launch_dtype<false>(y, inv, w, N, H, K, residual, out, s);
}

}  // namespace moe
