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

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_ROUTE_NW
#define MOE_ROUTE_NW 4       // waves per workgroup, splitting H
#endif
#ifndef MOE_ROUTE_MT64
#define MOE_ROUTE_MT64 4     // 16-token M-tiles per workgroup for E <= 64
#endif
#ifndef MOE_ROUTE_MT128
#define MOE_ROUTE_MT128 2    // ... for 64 < E <= 128
#endif
#ifndef MOE_ROUTE_ROTATE
#define MOE_ROUTE_ROTATE 1   // stagger each workgroup's first H step
#endif
#ifndef MOE_ROUTE_DEPTH
#define MOE_ROUTE_DEPTH 2    // steps of register prefetch (1 or 2) for E <= 64
#endif
#ifndef MOE_GATE_PAD
#define MOE_GATE_PAD 128     // elements of padding per expert-major gate row
#endif

namespace moe {

namespace {

constexpr int kSentinel = 0x7fffffff;
constexpr int kGatePad = MOE_GATE_PAD;

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 u) {
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
template <int NT, int MT, int NW, int D>
__global__ __launch_bounds__(NW * 64) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgt, int ldw,
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
  for (int q = 0; q < NT; ++q) brow[q] = wgt + (int64_t)(16 * q + r) * ldw + 16 * g;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nss = (H + 63) >> 6;
  const int s_begin = (wid * nss) / NW;
  const int s_end = ((wid + 1) * nss) / NW;

  // One 64-wide step of h: per lane 2 x 16 bytes of each of its MT token rows
  // and NT expert rows.  Full steps use plain 16-byte loads that stay in
  // flight until the MFMAs consume them; only a ragged last step
  // (H % 64 != 0) takes the masked path, where a half beyond H reads column 0
  // of its row and is replaced by zeros.
  struct Buf {
    u32x4 a0[MT], a1[MT], b0[NT], b1[NT];
  };
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load = [&](Buf& bf, int s) {
    const int o = s * 64;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      bf.a0[m] = *reinterpret_cast<const u32x4*>(arow[m] + o);
      bf.a1[m] = *reinterpret_cast<const u32x4*>(arow[m] + o + 8);
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      bf.b0[q] = *reinterpret_cast<const u32x4*>(brow[q] + o);
      bf.b1[q] = *reinterpret_cast<const u32x4*>(brow[q] + o + 8);
    }
  };
  auto load_masked = [&](Buf& bf, int s) {
    const int hl = s * 64 + 16 * g;  // this lane's columns: hl + [0, 16)
    const bool ok0 = hl < H;         // H % 8 == 0: each 8-wide half is all in or all out
    const bool ok1 = hl + 8 < H;
    const int o0 = ok0 ? s * 64 : -16 * g;
    const int o1 = ok1 ? s * 64 + 8 : -16 * g;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(arow[m] + o0);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(arow[m] + o1);
      bf.a0[m] = ok0 ? v0 : zero;
      bf.a1[m] = ok1 ? v1 : zero;
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(brow[q] + o0);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(brow[q] + o1);
      bf.b0[q] = ok0 ? v0 : zero;
      bf.b1[q] = ok1 ? v1 : zero;
    }
  };
  // MT*NT independent accumulators: consecutive MFMAs never depend on each
  // other
  auto mma = [&](const Buf& bf) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < NT; ++q)
        acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bf.a0[m]), as_bf16x8(bf.b0[q]),
                                                            acc[m][q], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < NT; ++q)
        acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bf.a1[m]), as_bf16x8(bf.b1[q]),
                                                            acc[m][q], 0, 0, 0);
  };

  // Each workgroup walks its H range starting at a different step (rotated
  // by the workgroup index), so that at any moment the resident workgroups
  // read different column windows of their rows: all rows are H*2 bytes
  // apart, and reading the same window of every row at once would load only
  // a few memory channels.
  const int nfull = H >> 6;  // steps with all 64 columns inside H
  const int s_stop = s_end < nfull ? s_end : nfull;
  const int cnt = s_stop > s_begin ? s_stop - s_begin : 0;
  const int rot = (MOE_ROUTE_ROTATE && cnt > 0) ? (int)(blockIdx.x % (unsigned)cnt) : 0;
  auto step_of = [&](int i) {
    int s = s_begin + rot + i;
    return s >= s_stop ? s - cnt : s;
  };
  // Software pipeline over register buffers.  The loop bodies have no
  // branches (a branch there makes the compiler drain every outstanding load
  // at the loop head): the prefetch is always issued, clamped to the last
  // step, so the final iterations reload a step that is already cached.
  // Software pipeline over register buffers.  The loop bodies have no
  // branches (a branch there makes the compiler drain every outstanding load
  // at the loop head): the prefetch is always issued, clamped to the last
  // step, so the final iterations reload a step that is already cached.  A
  // scheduling barrier after each prefetch keeps its loads ahead of the
  // MFMAs, which then wait only for their own (older) loads.
  if (cnt > 0) {
    const int last = cnt - 1;
    if constexpr (D >= 2) {
      // three buffers: two steps of loads in flight during each step's MFMAs
      Buf p0, p1, p2;
      load(p0, step_of(0));
      load(p1, step_of(min(1, last)));
      int i = 0;
      for (; i + 3 <= cnt; i += 3) {
        load(p2, step_of(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        mma(p0);
        __builtin_amdgcn_sched_barrier(0);
        load(p0, step_of(min(i + 3, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(p1);
        __builtin_amdgcn_sched_barrier(0);
        load(p1, step_of(min(i + 4, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(p2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (cnt - i >= 1) mma(p0);
      if (cnt - i >= 2) mma(p1);
    } else {
      // two buffers: one step of loads in flight during each step's MFMAs
      Buf p, q;
      load(p, step_of(0));
      int i = 0;
      for (; i + 2 <= cnt; i += 2) {
        load(q, step_of(i + 1));
        __builtin_amdgcn_sched_barrier(0);
        mma(p);
        __builtin_amdgcn_sched_barrier(0);
        load(p, step_of(min(i + 2, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(q);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i < cnt) mma(p);
    }
  }
  if (s_end > nfull && nfull >= s_begin) {  // the ragged last step, if this wave owns it
    Buf t;
    load_masked(t, nfull);
    mma(t);
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
// wgt[e][h] = gate_w[h][e] for e < E and 0 for E <= e < EP, rows ldw
// elements apart (ldw = H + kGatePad: the pad staggers the rows over the
// memory channels).  Each thread moves one 8(h) x 8(e) block: eight 16-byte
// loads, a register transpose, eight 16-byte stores; consecutive threads take
// consecutive h blocks so the stores are contiguous.  Thread 0.. also zero
// `counts` (the router then adds into it).
__global__ __launch_bounds__(64) void gate_transpose_kernel(const uint16_t* __restrict__ gate_w,
                                                            int H, int E, int EP, int ldw,
                                                            uint16_t* __restrict__ wgt,
                                                            int32_t* __restrict__ counts) {
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (counts && idx < E) counts[idx] = 0;
  const int nhb = H / 8;
  if (idx >= (int64_t)nhb * (EP / 8)) return;
  const int eb = (int)(idx / nhb);
  const int hb = (int)(idx - (int64_t)eb * nhb);
  const int h0 = hb * 8, e0 = eb * 8;
  uint32_t v[8][4];  // v[i] = 8 bf16 of gate row h0+i, experts e0..e0+7 (2 per word)
  const bool vec = (E % 8 == 0) && (e0 + 8 <= E);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t* src = gate_w + (int64_t)(h0 + i) * E + e0;
    if (vec) {
      const uint4 u = *reinterpret_cast<const uint4*>(src);
      v[i][0] = u.x; v[i][1] = u.y; v[i][2] = u.z; v[i][3] = u.w;
    } else {
      uint16_t t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = (e0 + j < E) ? src[j] : (uint16_t)0;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i][j] = (uint32_t)t[2 * j] | ((uint32_t)t[2 * j + 1] << 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // expert e0+j: its 8 values of h0..h0+7
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = (v[2 * p][j >> 1] >> (16 * (j & 1))) & 0xffffu;
      const uint32_t hi = (v[2 * p + 1][j >> 1] >> (16 * (j & 1))) & 0xffffu;
      o[p] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(wgt + (int64_t)(e0 + j) * ldw + h0) = uint4{o[0], o[1], o[2], o[3]};
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int NT, int MT, int NW = MOE_ROUTE_NW, int D = (NT <= 4 ? MOE_ROUTE_DEPTH : 1)>
hipError_t launch_bf16_nt(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                          int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                          hipStream_t s) {
  const int64_t blocks = (N + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL((route_bf16_kernel<NT, MT, NW, D>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     s, x, wgt, route_gate_stride(H), bias, N, H, E, K, ids, w, counts);
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

int route_gate_stride(int H) { return H + kGatePad; }

hipError_t launch_gate_transpose(const uint16_t* gate_w, int H, int E, uint16_t* wgt,
                                 int32_t* counts, hipStream_t s) {
  const int EP = route_padded_experts(E);
  int64_t threads = (int64_t)(H / 8) * (EP / 8);
  if (threads < E) threads = E;
  hipLaunchKernelGGL(gate_transpose_kernel, dim3((unsigned)((threads + 63) / 64)), dim3(64), 0, s,
                     gate_w, H, E, EP, route_gate_stride(H), wgt, counts);
  return hipGetLastError();
}

hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                             int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                             hipStream_t s) {
  switch (route_padded_experts(E)) {
    case 16: return launch_bf16_nt<1, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 32: return launch_bf16_nt<2, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 64: return launch_bf16_nt<4, MOE_ROUTE_MT64>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 128: return launch_bf16_nt<8, MOE_ROUTE_MT128>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
    case 256: return launch_bf16_nt<16, 1, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, s);
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
