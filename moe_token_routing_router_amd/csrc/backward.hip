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
//                                 x_perm[p]  -- segmented sums over fixed
//                                 chunks of 32 rows, then the chunks of each
//                                 expert in order: deterministic, no atomics;
//                     dbias[e]  = the same sums of dl.
#include "moe_internal.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tuning knobs (compile-time).
#ifndef MOE_BWD_U
#define MOE_BWD_U 2        // row vectors per lane in flight for K <= 2 (combine / dx backward)
#endif
#ifndef MOE_BWD_ROWS
#define MOE_BWD_ROWS 8     // dispatched rows in flight per lane (gate partials)
#endif

constexpr int kBwdChunk = 32;  // dispatched rows per gate-gradient partial
constexpr int kBwdVPT = 2;     // 16-byte vectors per thread and row in the partial kernel
constexpr int kBwdU = MOE_BWD_U;
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
    constexpr int U = KR <= 2 ? kBwdU : 1;
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
  hipLaunchKernelGGL((combine_bwd_kernel<BF16, KT>), dim3((unsigned)N), dim3(256), 0, s,
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
// Blocks [0, nbt): dl for 256 tokens each.  Blocks [nbt, ...): the
// expert-major copy of the gate, gate_t[e][h] = gate_w[h][e].
__global__ __launch_bounds__(256) void route_bwd_prep_kernel(
    const float* __restrict__ w, const float* __restrict__ dw, int64_t N, int K,
    float* __restrict__ dlsel, const void* __restrict__ gate_w, int H, int E, int esize,
    void* __restrict__ gate_t, int nbt) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < nbt) {
    const int64_t n = (int64_t)blockIdx.x * 256 + tid;
    if (n >= N) return;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(w[n * K + k], dw[n * K + k], s);
    for (int k = 0; k < K; ++k) dlsel[n * K + k] = w[n * K + k] * (dw[n * K + k] - s);
    return;
  }
  const int64_t idx = (int64_t)(blockIdx.x - nbt) * 256 + tid;
  if (idx >= (int64_t)E * H) return;
  const int64_t e = idx / H;
  const int64_t h = idx - e * H;
  if (esize == 2)
    reinterpret_cast<uint16_t*>(gate_t)[idx] = reinterpret_cast<const uint16_t*>(gate_w)[h * E + e];
  else
    reinterpret_cast<float*>(gate_t)[idx] = reinterpret_cast<const float*>(gate_w)[h * E + e];
}

// dx[n] = sum_k dx_perm[inv[n,k]] (if given) + sum_k dl[n,k] gate_t[ids[n,k]],
// fp32, the dispatch terms first, k ascending in each; one rounding.
template <bool BF16, int KT>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(
    const u32x4* __restrict__ dx_perm, const int32_t* __restrict__ inv,
    const u32x4* __restrict__ gate_t, const int32_t* __restrict__ ids,
    const float* __restrict__ dlsel, int64_t N, int Krt, int E, int row_vecs,
    u32x4* __restrict__ dx) {
  constexpr int L = BF16 ? 8 : 4;
  const int K = KT > 0 ? KT : Krt;
  extern __shared__ int dyn[];  // prow[K], grow[K], gw[K]
  int* prow = dyn;
  int* grw = dyn + K;
  float* gw = reinterpret_cast<float*>(dyn + 2 * K);
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t T = N * K;
  for (int j = tid; j < K; j += 256) {
    const int r = dx_perm ? inv[n * K + j] : -1;
    prow[j] = (unsigned)r < (unsigned long long)T ? r : -1;
    const int e = ids[n * K + j];
    grw[j] = (unsigned)e < (unsigned)E ? e : -1;
    gw[j] = dlsel[n * K + j];
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

// Partial gate gradients: workgroup (id, slice) sums kBwdChunk consecutive
// rows of one expert's dispatched segment, rows ascending, over the columns
// of its slice.  Chunk ids are numbered expert by expert (chunk_base[e] =
// sum over e' < e of ceil(count[e'] / kBwdChunk)); ids past the last chunk
// do nothing.
template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_wpart_kernel(
    const u32x4* __restrict__ x_perm, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ dlsel, int64_t T, int E,
    int row_vecs, int32_t* __restrict__ chunk_base, float* __restrict__ part,
    float* __restrict__ part_b) {
  constexpr int L = BF16 ? 8 : 4;
  constexpr int V = kBwdVPT;
  __shared__ int s_e, s_first;
  __shared__ int s_scan[4];
  __shared__ float coef[kBwdChunk];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int id = blockIdx.x;
  // chunk bases: exclusive scan of the chunk counts over the experts (E <= 256)
  // (offsets are clamped to [0, T]: inconsistent ones give wrong sums, never
  // an access outside x_perm, perm or the partials)
  const int64_t o0 = tid < E ? min(max((int64_t)offsets[tid], (int64_t)0), T) : 0;
  const int64_t o1 = tid < E ? min(max((int64_t)offsets[tid + 1], o0), T) : 0;
  const int cnt = (int)(o1 - o0);
  const int nch = (cnt + kBwdChunk - 1) / kBwdChunk;
  const int incl = wave_inclusive_sum(nch);
  if (lane == 63) s_scan[wid] = incl;
  if (tid == 0) s_e = -1;
  __syncthreads();
  int wbase = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) wbase += w < wid ? s_scan[w] : 0;
  const int cb = wbase + incl - nch;
  __shared__ int64_t s_p0, s_p1;
  if (tid < E && id >= cb && id < cb + nch) {
    s_e = tid;
    s_first = cb;
    s_p0 = o0;
    s_p1 = o1;
  }
  if (id == 0 && blockIdx.y == 0 && tid < E) {
    chunk_base[tid] = cb;
    if (tid == E - 1) chunk_base[E] = cb + nch;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int64_t p0 = s_p0 + (int64_t)(id - s_first) * kBwdChunk;
  const int rows = (int)min((int64_t)kBwdChunk, s_p1 - p0);

  int cv[V];
  bool ok[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    cv[v] = ((int)blockIdx.y * V + v) * 256 + tid;
    ok[v] = cv[v] < row_vecs;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int RR = kBwdRows;
  u32x4 xv[RR][V];
  auto load_rows = [&](int r) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int64_t p = p0 + min(r + rr, rows - 1);
#pragma unroll
      for (int v = 0; v < V; ++v) xv[rr][v] = ok[v] ? ldnt(x_perm + p * row_vecs + cv[v]) : zero;
    }
  };
  // the first rows' loads do not depend on the coefficients: issue them
  // before the perm -> dlsel gather and its barrier
  load_rows(0);
  if (tid < rows) {
    const int i = perm[p0 + tid];
    coef[tid] = (unsigned)i < (unsigned long long)T ? dlsel[i] : 0.f;
  }
  __syncthreads();

  float acc[V][L];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int j = 0; j < L; ++j) acc[v][j] = 0.f;
  for (int r = 0; r < rows; r += RR) {
    if (r > 0) load_rows(r);
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      if (r + rr >= rows) break;
      const float c = coef[r + rr];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float f[L];
        unpack<BF16>(xv[rr][v], f);
#pragma unroll
        for (int j = 0; j < L; ++j) acc[v][j] = fmaf(c, f[j], acc[v][j]);
      }
    }
  }
  const int64_t H = (int64_t)row_vecs * L;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (!ok[v]) continue;
    u32x4* dst = reinterpret_cast<u32x4*>(part + (int64_t)id * H + (int64_t)cv[v] * L);
#pragma unroll
    for (int q = 0; q < L / 4; ++q)
      dst[q] = u32x4{__float_as_uint(acc[v][4 * q]), __float_as_uint(acc[v][4 * q + 1]),
                     __float_as_uint(acc[v][4 * q + 2]), __float_as_uint(acc[v][4 * q + 3])};
  }
  if (blockIdx.y == 0 && tid == 0) {
    float sb = 0.f;
    for (int j = 0; j < rows; ++j) sb += coef[j];
    part_b[id] = sb;
  }
}

// dgate_w[h][e] = the partials of expert e's chunks summed in chunk order.
__global__ __launch_bounds__(256) void route_bwd_wreduce_kernel(
    const float* __restrict__ part, const float* __restrict__ part_b,
    const int32_t* __restrict__ chunk_base, int64_t nchunks, int H, int E,
    float* __restrict__ dgate_w, float* __restrict__ dbias) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)H * E) return;
  const int64_t e = idx / H;
  const int64_t h = idx - e * H;
  // chunks the partial kernel had no workgroup for (inconsistent offsets
  // only) are left out
  const int64_t c0 = min((int64_t)chunk_base[e], nchunks);
  const int64_t c1 = min((int64_t)chunk_base[e + 1], nchunks);
  // chunks in order; four loads in flight ahead of the (ordered) adds
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

template <bool BF16, int KT>
hipError_t launch_dx(const void* dx_perm, const int32_t* inv, const void* gate_t,
                     const int32_t* ids, const float* dlsel, int64_t N, int K, int E, int H,
                     void* dx, hipStream_t s) {
  const int row_vecs = BF16 ? H / 8 : H / 4;
  hipLaunchKernelGGL((route_bwd_dx_kernel<BF16, KT>), dim3((unsigned)N), dim3(256),
                     sizeof(int) * 3 * (size_t)K, s, reinterpret_cast<const u32x4*>(dx_perm), inv,
                     reinterpret_cast<const u32x4*>(gate_t), ids, dlsel, N, K, E, row_vecs,
                     reinterpret_cast<u32x4*>(dx));
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dx_dtype(const void* dx_perm, const int32_t* inv, const void* gate_t,
                           const int32_t* ids, const float* dlsel, int64_t N, int K, int E, int H,
                           void* dx, hipStream_t s) {
  switch (K) {
    case 1: return launch_dx<BF16, 1>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
    case 2: return launch_dx<BF16, 2>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
    case 4: return launch_dx<BF16, 4>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
    case 8: return launch_dx<BF16, 8>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
    default: return launch_dx<BF16, 0>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
  }
}

template <bool BF16>
hipError_t launch_rbwd(const void* x_perm, const void* gate_w, const int32_t* ids, const float* w,
                       const float* dw, const int32_t* perm, const int32_t* offsets,
                       const int32_t* inv, const void* dx_perm, int64_t N, int H, int E, int K,
                       float* dgate_w, float* dbias, void* dx, void* gate_t, float* dlsel,
                       int32_t* chunk_base, float* part, float* part_b, hipStream_t s) {
  const int row_vecs = BF16 ? H / 8 : H / 4;
  const int64_t T = N * K;
  const int nbt = (int)((N + 255) / 256);
  const int64_t ngt = ((int64_t)E * H + 255) / 256;
  hipLaunchKernelGGL(route_bwd_prep_kernel, dim3((unsigned)(nbt + ngt)), dim3(256), 0, s, w, dw,
                     N, K, dlsel, gate_w, H, E, BF16 ? 2 : 4, gate_t, nbt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_dx_dtype<BF16>(dx_perm, inv, gate_t, ids, dlsel, N, K, E, H, dx, s);
  if (err != hipSuccess) return err;
  const int64_t chunks = route_bwd_max_chunks(T, E);
  const int slices = (row_vecs + 256 * kBwdVPT - 1) / (256 * kBwdVPT);
  hipLaunchKernelGGL((route_bwd_wpart_kernel<BF16>), dim3((unsigned)chunks, (unsigned)slices),
                     dim3(256), 0, s, reinterpret_cast<const u32x4*>(x_perm), perm, offsets,
                     dlsel, T, E, row_vecs, chunk_base, part, part_b);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_bwd_wreduce_kernel, dim3((unsigned)(((int64_t)H * E + 255) / 256)),
                     dim3(256), 0, s, part, part_b, chunk_base, chunks, H, E, dgate_w, dbias);
  return hipGetLastError();
}

}  // namespace

int64_t route_bwd_max_chunks(int64_t T, int E) { return (T + kBwdChunk - 1) / kBwdChunk + E; }

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
                                 float* dbias, void* dx, void* gate_t, float* dlsel,
                                 int32_t* chunk_base, float* part, float* part_b, hipStream_t s) {
  return bf16 ? launch_rbwd<true>(x_perm, gate_w, ids, w, dw, perm, offsets, inv, dx_perm, N, H,
                                  E, K, dgate_w, dbias, dx, gate_t, dlsel, chunk_base, part,
                                  part_b, s)
              : launch_rbwd<false>(x_perm, gate_w, ids, w, dw, perm, offsets, inv, dx_perm, N, H,
                                   E, K, dgate_w, dbias, dx, gate_t, dlsel, chunk_base, part,
                                   part_b, s);
}

}  // namespace moe
