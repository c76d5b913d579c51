// Backward of the MoE routing path for gfx950: the gradients of the combine,
// of the row dispatch and of the router.
//
// Method: training runs the path's stages backward ("Building a MoE training
// stack in 10k lines of Python", section 6.2 "The five stages"); the forward
// they differentiate is the fused gate of "moe-engine: sparse MoE training
// infrastructure for 10k-GPU clusters", section "Fused Triton routing kernel"
// (tokens @ gate_w -> softmax -> top-K -> renorm), the counting-sort dispatch
// of the first page's section 8.2, and forward_aggregate of its section 6.1.
//
//  combine backward   (one workgroup per token)  dy[inv[n,k]] = w[n,k] *
//                     dout[n] rounded once (exactly: the fp32 product and its
//                     FMA error term decide bf16 midpoints), dw[n,k] =
//                     <dout[n], y[inv[n,k]]> in fp32 with a fixed-order block
//                     reduction; dout and each y row are read once.
//  dispatch backward  the combine kernel with unit weights.
//  router backward    dl[n,k] = w[n,k] (dw[n,k] - sum_j w[n,j] dw[n,j]) is
//                     the gradient of the logits at the kept experts, and 0
//                     elsewhere (the full-softmax denominator cancels in the
//                     renormalisation).  Because only K of the E logits of a
//                     token carry gradient:
//                     dx[n]     = sum_k dx_perm[inv[n,k]] + sum_k dl[n,k] *
//                                 gate_w[:, ids[n,k]]  -- a gather of 2K rows
//                                 per token (the gate's columns from an
//                                 expert-major copy, L2-resident), rounded once;
//                     dgate_w[:, e] = sum over the rows p of expert e's
//                                 dispatched segment of dl[perm[p]] *
//                                 x_perm[p]  -- partial sums over equal,
//                                 fixed ranges of dispatched rows (one per
//                                 expert a range meets), then the ranges of
//                                 each expert in order: deterministic, no
//                                 atomics;
//                     dbias[e]  = the same sums of dl.
//                     Two kernels: the partials (plus the gate's expert-major
//                     copy), then dx (plus the partials' reduction); dl is
//                     recomputed where it is used.
#include "moe_internal.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tuning knobs (compile-time).
#ifndef MOE_BWD_U
#define MOE_BWD_U 2        // row vectors per lane in flight for K <= 2 (dx backward)
#endif
#ifndef MOE_CBWD_U
#define MOE_CBWD_U 2       // ... in the combine backward
#endif
#ifndef MOE_BWD_ROWS
#define MOE_BWD_ROWS 8     // dispatched rows in flight per lane (gate partials)
#endif

#ifndef MOE_CBWD_CAP_KIB
#define MOE_CBWD_CAP_KIB 160  // combine backward: rows in flight per CU (KiB), large batches
#endif

#ifndef MOE_BWD_GROUPS
#define MOE_BWD_GROUPS 512 // gate-gradient partial-sum workgroups (about; see below)
#endif

#ifndef MOE_BWD_CHUNK
#define MOE_BWD_CHUNK 8
#endif
constexpr int kBwdChunk = MOE_BWD_CHUNK;  // fewest dispatched rows per partial-sum workgroup
constexpr int kBwdCoef = 256;   // most dispatched rows per partial-sum workgroup
constexpr int kBwdGroups = MOE_BWD_GROUPS;
#ifndef MOE_BWD_COPY_LAST
#define MOE_BWD_COPY_LAST 1 // the gate copy's workgroups after the partial sums'
#endif
#ifndef MOE_BWD_RED_LAST
#define MOE_BWD_RED_LAST 0  // the reduction's workgroups after dx's (1) or first (0)
#endif
constexpr bool kBwdCopyLast = MOE_BWD_COPY_LAST;
constexpr bool kBwdRedLast = MOE_BWD_RED_LAST;
constexpr int kBwdVPT = 2;     // 16-byte vectors per thread and row in the partial kernel
constexpr int kBwdU = MOE_BWD_U;
constexpr int kCbwdU = MOE_CBWD_U;
constexpr int kBwdRows = MOE_BWD_ROWS;

__device__ __forceinline__ u32x4 ldnt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void stnt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

template <bool BF16>
__device__ __forceinline__ void unpack(u32x4 v, float (&f)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_lo(v[j]);
      f[2 * j + 1] = bf16_hi(v[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(v[j]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack(const float (&f)[BF16 ? 8 : 4]) {
  u32x4 o;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(f[j]);
  }
  return o;
}

// w * g for the 8 (bf16) or 4 (fp32) elements of g, each rounded once
template <bool BF16>
__device__ __forceinline__ u32x4 scale_exact(float w, const float (&g)[BF16 ? 8 : 4]) {
  u32x4 o;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = bf16_of_product(w, g[2 * j]) | (bf16_of_product(w, g[2 * j + 1]) << 16);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(__fmul_rn(w, g[j]));
  }
  return o;
}

// ------------------------------------------------------------ combine backward
// KT > 0: all K rows of the token in one pass; KT == 0: one k per pass.
template <bool BF16, int KT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const u32x4* __restrict__ dout,
                                                          const u32x4* __restrict__ y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w, int64_t N,
                                                          int Krt, int row_vecs,
                                                          u32x4* __restrict__ dy,
                                                          float* __restrict__ dw) {
  constexpr int L = BF16 ? 8 : 4;
  constexpr int KR = KT > 0 ? KT : 1;
  __shared__ float red[4][KR];
  const int K = KT > 0 ? KT : Krt;
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t T = N * K;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const u32x4* grow = dout + n * row_vecs;
  for (int k0 = 0; k0 < K; k0 += KR) {
    int row[KR];
    float wk[KR], part[KR];
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      const int r = inv[n * K + k0 + kk];
      row[kk] = (unsigned)r < (unsigned long long)T ? r : -1;
      wk[kk] = w[n * K + k0 + kk];
      part[kk] = 0.f;
    }
    constexpr int U = KR <= 2 ? kCbwdU : 1;
    for (int c0 = tid; c0 < row_vecs; c0 += 256 * U) {
      // all loads of U vectors first (clamped: the extra ones are not used)
      u32x4 gv[U], yv[U][KR];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + u * 256, row_vecs - 1);
        gv[u] = ldnt(grow + c);
#pragma unroll
        for (int kk = 0; kk < KR; ++kk)
          yv[u][kk] = row[kk] >= 0 ? ldnt(y + (int64_t)row[kk] * row_vecs + c) : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 256;
        if (c >= row_vecs) break;
        float gf[L];
        unpack<BF16>(gv[u], gf);
#pragma unroll
        for (int kk = 0; kk < KR; ++kk) {
          float yf[L];
          unpack<BF16>(yv[u][kk], yf);
#pragma unroll
          for (int j = 0; j < L; ++j) part[kk] = fmaf(gf[j], yf[j], part[kk]);
          if (row[kk] >= 0)
            stnt(dy + (int64_t)row[kk] * row_vecs + c, scale_exact<BF16>(wk[kk], gf));
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      const float s = wave_sum_f32(part[kk]);
      if (lane == 0) red[wid][kk] = s;
    }
    __syncthreads();
    if (tid < KR) dw[n * K + k0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    __syncthreads();  // red is rewritten by the next pass
  }
}

template <bool BF16, int KT>
hipError_t launch_cbwd(const void* dout, const void* y, const int32_t* inv, const float* w,
                       int64_t N, int H, int K, void* dy, float* dw, hipStream_t s) {
  const int row_vecs = BF16 ? H / 8 : H / 4;
  // a workgroup moves one token's 2K + 1 rows: four workgroups per CU at
  // N = 16384, H = 4096, K = 2 (127.4 -> 121.7 us), three at N = 32768,
  // H = 2048, K = 8 (423 -> 410 us)
  const size_t dyn = gather_lds_cap(N, (size_t)H * (BF16 ? 2 : 4), (size_t)(2 * K + 1),
                                    (size_t)MOE_CBWD_CAP_KIB * 1024);
  hipLaunchKernelGGL((combine_bwd_kernel<BF16, KT>), dim3((unsigned)N), dim3(256), dyn, s,
                     reinterpret_cast<const u32x4*>(dout), reinterpret_cast<const u32x4*>(y),
                     inv, w, N, K, row_vecs, reinterpret_cast<u32x4*>(dy), dw);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_cbwd_dtype(const void* dout, const void* y, const int32_t* inv, const float* w,
                             int64_t N, int H, int K, void* dy, float* dw, hipStream_t s) {
  switch (K) {
    case 1: return launch_cbwd<BF16, 1>(dout, y, inv, w, N, H, K, dy, dw, s);
    case 2: return launch_cbwd<BF16, 2>(dout, y, inv, w, N, H, K, dy, dw, s);
    case 4: return launch_cbwd<BF16, 4>(dout, y, inv, w, N, H, K, dy, dw, s);
    case 8: return launch_cbwd<BF16, 8>(dout, y, inv, w, N, H, K, dy, dw, s);
    default: return launch_cbwd<BF16, 0>(dout, y, inv, w, N, H, K, dy, dw, s);
  }
}

// ------------------------------------------------------------ router backward
// dl of slot i = n*K + k: w[i] * (dw[i] - sum_j w[n*K+j] dw[n*K+j]), the sum
// over j ascending in fp32.  Both kernels that need dl call this same code,
// so they see the same values.
__device__ __forceinline__ float route_dl(const float* __restrict__ w,
                                          const float* __restrict__ dw, int64_t i, int K) {
  const int64_t n0 = i - i % K;
  float s = 0.f;
  for (int j = 0; j < K; ++j) s = fmaf(w[n0 + j], dw[n0 + j], s);
  return w[i] * (dw[i] - s);
}

// One element of the expert-major copy of the gate, gate_t[e][h] = gate_w[h][e].
__device__ __forceinline__ void gate_transpose_one(int64_t idx, const void* __restrict__ gate_w,
                                                   int H, int E, int esize,
                                                   void* __restrict__ gate_t) {
  if (idx >= (int64_t)E * H) return;
  const int64_t e = idx / H;
  const int64_t h = idx - e * H;
  if (esize == 2)
    reinterpret_cast<uint16_t*>(gate_t)[idx] = reinterpret_cast<const uint16_t*>(gate_w)[h * E + e];
  else
    reinterpret_cast<float*>(gate_t)[idx] = reinterpret_cast<const float*>(gate_w)[h * E + e];
}

// dgate_w[h][e] (and dbias[e] at h == 0) for idx = e*H + h: the partials of
// expert e's row ranges (rows g + e of part, g over the ranges that meet its
// segment) summed in range order.
__device__ __forceinline__ void wreduce_one(int64_t idx, const float* __restrict__ part,
                                            const float* __restrict__ part_b,
                                            const int32_t* __restrict__ offsets, int64_t T,
                                            int64_t RW, int H, int E, float* __restrict__ dgate_w,
                                            float* __restrict__ dbias) {
  if (idx >= (int64_t)H * E) return;
  const int64_t e = idx / H;
  const int64_t h = idx - e * H;
  const int64_t lo = min(max((int64_t)offsets[e], (int64_t)0), T);
  const int64_t hi = min(max((int64_t)offsets[e + 1], lo), T);
  const int64_t c0 = lo / RW + e;
  const int64_t c1 = hi > lo ? (hi - 1) / RW + e + 1 : c0;
  // in order; four loads in flight ahead of the (ordered) adds
  float s = 0.f;
  int64_t c = c0;
  for (; c + 4 <= c1; c += 4) {
    const float a0 = part[c * H + h], a1 = part[(c + 1) * H + h];
    const float a2 = part[(c + 2) * H + h], a3 = part[(c + 3) * H + h];
    s += a0;
    s += a1;
    s += a2;
    s += a3;
  }
  for (; c < c1; ++c) s += part[c * H + h];
  dgate_w[h * E + e] = s;
  if (dbias && h == 0) {
    float b = 0.f;
    for (int64_t c = c0; c < c1; ++c) b += part_b[c];
    dbias[e] = b;
  }
}

// Blocks [0, nred): the gate and bias gradients from the partials (one
// element per thread).  Blocks [nred, nred + N): dx[n] = sum_k
// dx_perm[inv[n,k]] (if given) + sum_k dl[n,k] gate_t[ids[n,k]], fp32, the
// dispatch terms first, k ascending in each; one rounding.
template <bool BF16, int KT>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(
    const u32x4* __restrict__ dx_perm, const int32_t* __restrict__ inv,
    const u32x4* __restrict__ gate_t, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const float* __restrict__ dw, int64_t N, int Krt, int E,
    int row_vecs, u32x4* __restrict__ dx, int nred, const float* __restrict__ part,
    const float* __restrict__ part_b, const int32_t* __restrict__ offsets, int64_t RW,
    float* __restrict__ dgate_w, float* __restrict__ dbias) {
  constexpr int L = BF16 ? 8 : 4;
  const int K = KT > 0 ? KT : Krt;
  const int tid = threadIdx.x;
  const int64_t T = N * K;
  const int64_t red0 = kBwdRedLast ? N : 0;  // the reduction's first workgroup
  if ((int64_t)blockIdx.x >= red0 && (int64_t)blockIdx.x < red0 + nred) {
    wreduce_one(((int64_t)blockIdx.x - red0) * 256 + tid, part, part_b, offsets, T, RW,
                row_vecs * L, E, dgate_w, dbias);
    return;
  }
  extern __shared__ int dyn[];  // prow[K], grow[K], gw[K]
  int* prow = dyn;
  int* grw = dyn + K;
  float* gw = reinterpret_cast<float*>(dyn + 2 * K);
  const int64_t n = (int64_t)blockIdx.x - (kBwdRedLast ? 0 : nred);
  for (int j = tid; j < K; j += 256) {
    const int r = dx_perm ? inv[n * K + j] : -1;
    prow[j] = (unsigned)r < (unsigned long long)T ? r : -1;
    const int e = ids[n * K + j];
    grw[j] = (unsigned)e < (unsigned)E ? e : -1;
    gw[j] = route_dl(w, dw, n * K + j, K);
  }
  __syncthreads();
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if constexpr (KT > 0) {
    constexpr int U = KT <= 2 ? kBwdU : 1;
    for (int c0 = tid; c0 < row_vecs; c0 += 256 * U) {
      u32x4 pv[U][KT], gv[U][KT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + u * 256, row_vecs - 1);
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          pv[u][k] = prow[k] >= 0 ? ldnt(dx_perm + (int64_t)prow[k] * row_vecs + c) : zero;
          gv[u][k] = grw[k] >= 0 ? gate_t[(int64_t)grw[k] * row_vecs + c] : zero;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 256;
        if (c >= row_vecs) break;
        float acc[L];
#pragma unroll
        for (int j = 0; j < L; ++j) acc[j] = 0.f;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          float f[L];
          unpack<BF16>(pv[u][k], f);
#pragma unroll
          for (int j = 0; j < L; ++j) acc[j] += f[j];
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          float f[L];
          unpack<BF16>(gv[u][k], f);
#pragma unroll
          for (int j = 0; j < L; ++j) acc[j] = fmaf(gw[k], f[j], acc[j]);
        }
        stnt(dx + n * row_vecs + c, pack<BF16>(acc));
      }
    }
    return;
  }
  // any K: one output vector per lane at a time
  for (int c = tid; c < row_vecs; c += 256) {
    float acc[L];
#pragma unroll
    for (int j = 0; j < L; ++j) acc[j] = 0.f;
    for (int k = 0; k < K; ++k) {
      if (prow[k] < 0) continue;
      float f[L];
      unpack<BF16>(ldnt(dx_perm + (int64_t)prow[k] * row_vecs + c), f);
#pragma unroll
      for (int j = 0; j < L; ++j) acc[j] += f[j];
    }
    for (int k = 0; k < K; ++k) {
      if (grw[k] < 0) continue;
      float f[L];
      unpack<BF16>(gate_t[(int64_t)grw[k] * row_vecs + c], f);
#pragma unroll
      for (int j = 0; j < L; ++j) acc[j] = fmaf(gw[k], f[j], acc[j]);
    }
    stnt(dx + n * row_vecs + c, pack<BF16>(acc));
  }
}

// Rows of x_perm per partial-sum workgroup: the N*K dispatched rows are cut
// into equal ranges, about kBwdGroups of them, of kBwdChunk..kBwdCoef rows,
// so every workgroup streams the same number of bytes.
__host__ __device__ inline int64_t route_bwd_rows_per_group(int64_t T) {
  const int64_t r = (T + kBwdGroups - 1) / kBwdGroups;
  return r < kBwdChunk ? kBwdChunk : (r > kBwdCoef ? kBwdCoef : r);
}

// Partial gate gradients: workgroup (g, slice) sums, over the columns of its
// slice, the rows p of its range [g*RW, (g+1)*RW) in ascending order,
// dl[perm[p]] * x_perm[p], one sum per expert segment the range meets:
// the partial of (range g, expert e) goes to row g + e of `part` (ranges and
// segments both ascend, so these rows are distinct and below G + E).
// Expert segments are [offsets[e], offsets[e+1]) clamped to [0, T] (rows
// outside every segment are skipped; inconsistent offsets give wrong sums,
// never an access outside x_perm, perm or the partials).
template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_wpart_kernel(
    const u32x4* __restrict__ x_perm, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ w,
    const float* __restrict__ dw, int64_t T, int K, int E, int row_vecs, int64_t RW,
    int64_t groups, float* __restrict__ part, float* __restrict__ part_b,
    const void* __restrict__ gate_w, void* __restrict__ gate_t, int ngt) {
  // the gate's expert-major copy, for the dx kernel: kBwdCopyLast puts its
  // workgroups after the partial-sum ones
  const int64_t side0 = kBwdCopyLast ? (int64_t)gridDim.x - ngt : 0;
  if ((int64_t)blockIdx.x >= side0 && (int64_t)blockIdx.x < side0 + ngt) {
    gate_transpose_one(((int64_t)blockIdx.x - side0) * 256 + threadIdx.x, gate_w,
                       row_vecs * (BF16 ? 8 : 4), E, BF16 ? 2 : 4, gate_t);
    return;
  }
  constexpr int L = BF16 ? 8 : 4;
  constexpr int V = kBwdVPT;
  __shared__ int64_t s_lo[kMaxExperts], s_hi[kMaxExperts];
  __shared__ float coef[kBwdCoef];
  const int tid = threadIdx.x;
  const int64_t b = (int64_t)blockIdx.x - (kBwdCopyLast ? 0 : ngt);
  const int64_t g = b % groups;  // row range
  const int slice = (int)(b / groups);  // 256*V-vector slice of the columns
  const int64_t pb = g * RW;
  const int64_t pe = min(pb + RW, T);
  const int64_t H = (int64_t)row_vecs * L;

  int cv[V];
  bool ok[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    cv[v] = (slice * V + v) * 256 + tid;
    ok[v] = cv[v] < row_vecs;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int RR = kBwdRows;
  u32x4 xv[RR][V];
  auto load_rows = [&](int64_t r) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int64_t p = min(r + rr, pe - 1);
#pragma unroll
      for (int v = 0; v < V; ++v) xv[rr][v] = ok[v] ? ldnt(x_perm + p * row_vecs + cv[v]) : zero;
    }
  };
  // the first rows' loads depend on nothing: issue them before the segment
  // bounds, the perm -> dl gather and their barriers
  load_rows(pb);

  int64_t lo = 0, hi = 0;
  if (tid < E) {
    lo = min(max((int64_t)offsets[tid], (int64_t)0), T);
    hi = min(max((int64_t)offsets[tid + 1], lo), T);
    s_lo[tid] = lo;
    s_hi[tid] = hi;
  }
  if (pb + tid < pe) {
    const int i = perm[pb + tid];
    coef[tid] = (unsigned)i < (unsigned long long)T ? route_dl(w, dw, i, K) : 0.f;
  }
  __syncthreads();
  // with ascending segments: experts [0, e_first) end at or before the range,
  // experts [0, e_end) start before its end (both counts also barrier)
  const int e_first = __syncthreads_count(tid < E && hi <= pb);
  const int e_end = __syncthreads_count(tid < E && lo < pe);

  float acc[V][L];
  float cs = 0.f;  // the bias partial: sum of the coefficients
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int j = 0; j < L; ++j) acc[v][j] = 0.f;
  bool touched = false;
  int e = e_first;
  auto flush = [&]() {
    if (!touched) return;
    float* prow = part + (g + e) * H;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!ok[v]) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(prow + (int64_t)cv[v] * L);
#pragma unroll
      for (int q = 0; q < L / 4; ++q)
        dst[q] = u32x4{__float_as_uint(acc[v][4 * q]), __float_as_uint(acc[v][4 * q + 1]),
                       __float_as_uint(acc[v][4 * q + 2]), __float_as_uint(acc[v][4 * q + 3])};
    }
    if (slice == 0 && tid == 0) part_b[g + e] = cs;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int j = 0; j < L; ++j) acc[v][j] = 0.f;
    cs = 0.f;
    touched = false;
  };
  for (int64_t r = pb; r < pe; r += RR) {
    if (r > pb) load_rows(r);
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int64_t p = r + rr;
      if (p >= pe) break;
      while (e < e_end && p >= s_hi[e]) {  // uniform: the segment ended
        flush();
        ++e;
      }
      if (e >= e_end || p < s_lo[e]) continue;  // in no segment
      const float c = coef[p - pb];
      cs += c;
      touched = true;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float f[L];
        unpack<BF16>(xv[rr][v], f);
#pragma unroll
        for (int j = 0; j < L; ++j) acc[v][j] = fmaf(c, f[j], acc[v][j]);
      }
    }
  }
  if (e < e_end) flush();
}

struct RouteBwdArgs {
  const void* x_perm;
  const void* gate_w;
  const int32_t* ids;
  const float* w;
  const float* dw;
  const int32_t* perm;
  const int32_t* offsets;
  const int32_t* inv;
  const void* dx_perm;
  int64_t N;
  int H, E, K;
  float* dgate_w;
  float* dbias;
  void* dx;
  void* gate_t;
  float* part;
  float* part_b;
};

template <bool BF16, int KT>
hipError_t launch_dx(const RouteBwdArgs& a, int64_t RW, hipStream_t s) {
  const int row_vecs = BF16 ? a.H / 8 : a.H / 4;
  const int nred = (int)(((int64_t)a.H * a.E + 255) / 256);
  hipLaunchKernelGGL((route_bwd_dx_kernel<BF16, KT>), dim3((unsigned)(nred + a.N)), dim3(256),
                     sizeof(int) * 3 * (size_t)a.K, s, reinterpret_cast<const u32x4*>(a.dx_perm),
                     a.inv, reinterpret_cast<const u32x4*>(a.gate_t), a.ids, a.w, a.dw, a.N, a.K,
                     a.E, row_vecs, reinterpret_cast<u32x4*>(a.dx), nred, a.part, a.part_b,
                     a.offsets, RW, a.dgate_w, a.dbias);
  return hipGetLastError();
}

// Two kernels: the gate's expert-major copy and the per-range partials of the
// gate gradient (reading x_perm), then dx (reading dx_perm and the copy) with
// the partials' ordered reduction in its first workgroups.  dl is computed
// where it is used.
template <bool BF16>
hipError_t launch_rbwd(const RouteBwdArgs& a, hipStream_t s) {
  const int row_vecs = BF16 ? a.H / 8 : a.H / 4;
  const int64_t T = a.N * a.K;
  const int ngt = (int)(((int64_t)a.E * a.H + 255) / 256);
  const int64_t RW = route_bwd_rows_per_group(T);
  const int64_t groups = (T + RW - 1) / RW;
  const int slices = (row_vecs + 256 * kBwdVPT - 1) / (256 * kBwdVPT);
  hipLaunchKernelGGL((route_bwd_wpart_kernel<BF16>), dim3((unsigned)(ngt + groups * slices)),
                     dim3(256), 0, s, reinterpret_cast<const u32x4*>(a.x_perm), a.perm, a.offsets,
                     a.w, a.dw, T, a.K, a.E, row_vecs, RW, groups, a.part, a.part_b, a.gate_w,
                     a.gate_t, ngt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (a.K) {
    case 1: return launch_dx<BF16, 1>(a, RW, s);
    case 2: return launch_dx<BF16, 2>(a, RW, s);
    case 4: return launch_dx<BF16, 4>(a, RW, s);
    case 8: return launch_dx<BF16, 8>(a, RW, s);
    default: return launch_dx<BF16, 0>(a, RW, s);
  }
}

}  // namespace

int64_t route_bwd_max_chunks(int64_t T, int E) {
  const int64_t RW = route_bwd_rows_per_group(T);
  return (T + RW - 1) / RW + E;
}

hipError_t launch_combine_backward(const void* dout, const void* y, const int32_t* inv,
                                   const float* w, int64_t N, int H, int K, bool bf16, void* dy,
                                   float* dw, hipStream_t s) {
  return bf16 ? launch_cbwd_dtype<true>(dout, y, inv, w, N, H, K, dy, dw, s)
              : launch_cbwd_dtype<false>(dout, y, inv, w, N, H, K, dy, dw, s);
}

hipError_t launch_route_backward(const void* x_perm, const void* gate_w, const int32_t* ids,
                                 const float* w, const float* dw, const int32_t* perm,
                                 const int32_t* offsets, const int32_t* inv, const void* dx_perm,
                                 int64_t N, int H, int E, int K, bool bf16, float* dgate_w,
                                 float* dbias, void* dx, void* gate_t, float* part, float* part_b,
                                 hipStream_t s) {
  const RouteBwdArgs a{x_perm, gate_w, ids, w, dw, perm, offsets, inv, dx_perm, N, H, E, K,
                       dgate_w, dbias, dx, gate_t, part, part_b};
  return bf16 ? launch_rbwd<true>(a, s) : launch_rbwd<false>(a, s);
}

}  // namespace moe
