// Fused MoE router for gfx950: logits = x @ gate_w (+ bias), top-K by K
// rounds of selection, renormalised softmax weights -- one pass over x, the
// logits never leave the chip.
//
// Method: "moe-engine: sparse MoE training infrastructure for 10k-GPU
// clusters", section "Fused Triton routing kernel" (融合Triton路由内核): the
// gate chain tokens @ gate_w -> softmax -> top-K -> renorm is done in one
// memory pass, with K rounds of selection (not a bitonic sort) for small K and
// E <= 256.  The pages' kernel is a Triton kernel on 64x64 SRAM tiles; this one
// is laid out for CDNA4 instead:
//  * the contraction runs on v_mfma_f32_16x16x32_bf16 (bf16 products are exact
//    in fp32, accumulation in fp32);
//  * the gate is first re-laid out expert-major (wgt[e][h], padded to a
//    multiple of 16 experts) so both MFMA operands are read straight from
//    global memory into registers with 16-byte loads -- x from HBM exactly
//    once, wgt from L2 -- and no LDS staging is needed for the contraction;
//  * a workgroup owns BM = 16*MT tokens; its NW waves split H and their fp32
//    partial logits are summed through LDS in a fixed order (deterministic);
//  * softmax/top-K/renorm happen in registers: a token's logits live in one
//    16-lane row of the wave (lane r holds experts r, r+16, ...), and each of
//    the K rounds is a 16-lane arg-max butterfly.
//
// Selection is on logits (softmax is monotone), ties go to the lower expert
// index, and since the renormalised weights equal a softmax over the K kept
// logits the full-E softmax denominator cancels and is not formed.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kSentinel = 0x7fffffff;

// K rounds of arg-max over one token's logits held by a 16-lane group, then
// w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0) for the K picks.  Lane r keeps
// round r's pick and writes ids[t*K + r], w[t*K + r].
// v[q] is the logit of expert 16*q + r (already biased); experts >= E are
// never candidates.
template <int NT>
__device__ __forceinline__ void select_topk_store(const float (&v)[NT], int r, int E, int K,
                                                  int64_t t, bool valid, int32_t* __restrict__ ids,
                                                  float* __restrict__ topw, int* hist) {
  uint32_t taken = 0;
  float my_val = 0.f, top = 0.f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -__builtin_inff();
    int bi = kSentinel;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      const bool cand = (e < E) && !((taken >> q) & 1u);
      // experts are visited in ascending index: strict '>' keeps the lower
      // index on ties; the first candidate always replaces the sentinel
      if (cand && (bi == kSentinel || v[q] > bv)) {
        bv = v[q];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 16);
      const int oi = __shfl_xor(bi, off, 16);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (k == 0) top = bv;
    if (r == k) {
      my_val = bv;
      my_id = bi;
    }
    if ((bi & 15) == r) taken |= 1u << (bi >> 4);
  }
  float ex = (r < K) ? expf(my_val - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 16);
  if (valid && r < K) {
    ids[t * K + r] = my_id;
    topw[t * K + r] = ex / sum;
    if (hist) atomicAdd(&hist[my_id], 1);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// ---------------------------------------------------------------- bf16 MFMA
// Grid: ceil(N / BM) workgroups of NW waves.  Each lane (r = lane%16,
// g = lane/16) loads, per 64-wide step of h, 32 contiguous bytes of a token
// row (A operand) and of an expert row of wgt (B operand):
//   A[r][8g + j] = x[t0 + 16m + r][h0 + 16g + j]        (first MFMA)
//   A[r][8g + j] = x[t0 + 16m + r][h0 + 16g + 8 + j]    (second MFMA)
// and the same h for B from wgt[16q + r][...].  Both operands use the same
// (lane group, element) -> h map, so each MFMA sums over 32 distinct h and
// every h in [h0, h0+64) is covered once.  Accumulator element i of lane l
// is D[4g + i][r]: token 16m + 4g + i, expert 16q + r.
template <int NT, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgt,
    const float* __restrict__ bias, int64_t N, int H, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ topw, int32_t* __restrict__ counts) {
  constexpr int BM = 16 * MT;
  constexpr int EP = 16 * NT;
  constexpr int ROWP = EP + 4;
  static_assert(BM % (4 * NW) == 0, "epilogue maps 4 tokens per wave per pass");
  __shared__ float part[NW][BM][ROWP];
  __shared__ int hist[EP];

  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BM;

  if (counts) {
    for (int e = tid; e < EP; e += NW * 64) hist[e] = 0;
  }

  const uint16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int64_t t = t0 + 16 * m + r;
    if (t > N - 1) t = N - 1;  // tail rows recompute the last token; never stored
    arow[m] = x + t * H + 16 * g;
  }
  const uint16_t* brow[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) brow[q] = wgt + (int64_t)(16 * q + r) * H + 16 * g;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nss = (H + 63) >> 6;
  const int s_begin = (wid * nss) / NW;
  const int s_end = ((wid + 1) * nss) / NW;
  const uint4 zero = {0u, 0u, 0u, 0u};

  uint4 a0[MT], a1[MT], b0[NT], b1[NT];
  auto load = [&](int s) {
    const int h = s * 64;          // this lane's columns: h + 16g + [0, 16)
    const int hl = h + 16 * g;
    const bool ok0 = hl < H;       // H % 8 == 0: each 8-wide half is all in or all out
    const bool ok1 = hl + 8 < H;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      a0[m] = ok0 ? *reinterpret_cast<const uint4*>(arow[m] + h) : zero;
      a1[m] = ok1 ? *reinterpret_cast<const uint4*>(arow[m] + h + 8) : zero;
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      b0[q] = ok0 ? *reinterpret_cast<const uint4*>(brow[q] + h) : zero;
      b1[q] = ok1 ? *reinterpret_cast<const uint4*>(brow[q] + h + 8) : zero;
    }
  };

  if (s_begin < s_end) load(s_begin);
  for (int s = s_begin; s < s_end; ++s) {
    uint4 c0[MT], c1[MT], d0[NT], d1[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      c0[m] = a0[m];
      c1[m] = a1[m];
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      d0[q] = b0[q];
      d1[q] = b1[q];
    }
    if (s + 1 < s_end) load(s + 1);  // next step's loads overlap this step's MFMAs
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(c0[m]), as_bf16x8(d0[q]),
                                                            acc[m][q], 0, 0, 0);
        acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(c1[m]), as_bf16x8(d1[q]),
                                                            acc[m][q], 0, 0, 0);
      }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wid][16 * m + 4 * g + i][16 * q + r] = acc[m][q][i];
  __syncthreads();

  for (int tl = wid * 4 + g; tl < BM; tl += NW * 4) {
    const int64_t t = t0 + tl;
    float v[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      float s = part[0][tl][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += part[w][tl][e];
      if (bias && e < E) s += bias[e];
      v[q] = s;
    }
    select_topk_store<NT>(v, r, E, K, t, t < N, ids, topw, counts ? hist : nullptr);
  }

  if (counts) {
    __syncthreads();
    for (int e = tid; e < E; e += NW * 64)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

// ---------------------------------------------------------------- fp32 VALU
// 16 tokens per 256-thread workgroup: wave w, lane group g owns token
// 16*blockIdx + 4w + g; lane r accumulates experts r, r+16, ... with one fp32
// FMA chain per expert in ascending h.
template <int NT>
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ gate_w,
                                                        const float* __restrict__ bias, int64_t N,
                                                        int H, int E, int K,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ topw,
                                                        int32_t* __restrict__ counts) {
  constexpr int EP = 16 * NT;
  __shared__ int hist[EP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t = (int64_t)blockIdx.x * 16 + (tid >> 6) * 4 + g;
  if (counts) {
    for (int e = tid; e < EP; e += 256) hist[e] = 0;
    __syncthreads();
  }
  const int64_t tc = t < N ? t : N - 1;
  const float* xr = x + tc * H;
  float acc[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) acc[q] = 0.f;
  for (int h = 0; h < H; h += 4) {
    const float4 xv = *reinterpret_cast<const float4*>(xr + h);
    const float* wr = gate_w + (int64_t)h * E;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      if (e < E) {
        acc[q] = fmaf(xv.x, wr[e], acc[q]);
        acc[q] = fmaf(xv.y, wr[E + e], acc[q]);
        acc[q] = fmaf(xv.z, wr[2 * E + e], acc[q]);
        acc[q] = fmaf(xv.w, wr[3 * E + e], acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int e = 16 * q + r;
    if (bias && e < E) acc[q] += bias[e];
  }
  select_topk_store<NT>(acc, r, E, K, t, t < N, ids, topw, counts ? hist : nullptr);
  if (counts) {
    __syncthreads();
    for (int e = tid; e < E; e += 256)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

// ------------------------------------------------------- gate re-layout
// wgt[e][h] = gate_w[h][e] for e < E, 0 for E <= e < EP; 64x64 tiles through
// LDS.  Block (0,0) also zeroes counts (the router then adds into it).
__global__ __launch_bounds__(256) void gate_transpose_kernel(const uint16_t* __restrict__ gate_w,
                                                             int H, int E, int EP,
                                                             uint16_t* __restrict__ wgt,
                                                             int32_t* __restrict__ counts) {
  __shared__ uint16_t tile[64][66];
  const int h0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int hh = i >> 6, ee = i & 63;
    const int h = h0 + hh, e = e0 + ee;
    tile[hh][ee] = (h < H && e < E) ? gate_w[(int64_t)h * E + e] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int ee = i >> 6, hh = i & 63;
    const int h = h0 + hh, e = e0 + ee;
    if (h < H && e < EP) wgt[(int64_t)e * H + h] = tile[hh][ee];
  }
  if (counts && blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < E; e += 256) counts[e] = 0;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int NT, int MT>
hipError_t launch_bf16_nt(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                          int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                          hipStream_t s) {
  constexpr int NW = 4;
  const int64_t blocks = (N + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL((route_bf16_kernel<NT, MT, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     s, x, wgt, bias, N, H, E, K, ids, w, counts);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_f32_nt(const float* x, const float* gw, const float* bias, int64_t N, int H,
                         int E, int K, int32_t* ids, float* w, int32_t* counts, hipStream_t s) {
  const int64_t blocks = (N + 15) / 16;
  hipLaunchKernelGGL((route_f32_kernel<NT>), dim3((unsigned)blocks), dim3(256), 0, s, x, gw,
                     bias, N, H, E, K, ids, w, counts);
  return hipGetLastError();
}

}  // namespace

int route_padded_experts(int E) {
  int ep = 16;
  while (ep < E) ep *= 2;
  return ep;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n,
                     v);
  return hipGetLastError();
}

hipError_t launch_gate_transpose(const uint16_t* gate_w, int H, int E, uint16_t* wgt,
                                 int32_t* counts, hipStream_t s) {
  const int EP = route_padded_experts(E);
  dim3 grid((unsigned)((H + 63) / 64), (unsigned)((EP + 63) / 64));
  hipLaunchKernelGGL(gate_transpose_kernel, grid, dim3(256), 0, s, gate_w, H, E, EP, wgt, counts);
  return hipGetLastError();
}

hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                             int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                             hipStream_t s) {
  switch (route_padded_experts(E)) {
    case 16: return launch_bf16_nt<1, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 32: return launch_bf16_nt<2, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 64: return launch_bf16_nt<4, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 128: return launch_bf16_nt<8, 2>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 256: return launch_bf16_nt<16, 1>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route_f32(const float* x, const float* gate_w, const float* bias, int64_t N,
                            int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                            hipStream_t s) {
  switch (route_padded_experts(E)) {
    case 16: return launch_f32_nt<1>(x, gate_w, bias, N, H, E, K, ids, w, counts, s);
    case 32: return launch_f32_nt<2>(x, gate_w, bias, N, H, E, K, ids, w, counts, s);
    case 64: return launch_f32_nt<4>(x, gate_w, bias, N, H, E, K, ids, w, counts, s);
    case 128: return launch_f32_nt<8>(x, gate_w, bias, N, H, E, K, ids, w, counts, s);
    case 256: return launch_f32_nt<16>(x, gate_w, bias, N, H, E, K, ids, w, counts, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
