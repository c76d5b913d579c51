// Grouped expert linear layer over the dispatched rows for gfx950:
//   y[p, :] = weight[e] @ x_perm[p, :]   for offsets[e] <= p < offsets[e+1]
// with weight [E][F][H] (row f of expert e: the weights of output f).
//
// Method: the expert layer that runs between dispatch and combine ("Building
// a MoE training stack in 10k lines of Python", section 6.1: forward_mlp on
// the gathered tokens; the MoE GroupLinear of its layer list), one GEMM per
// expert over that expert's contiguous segment of the dispatched buffer --
// the expert-contiguous layout is what makes the rows of one expert a dense
// operand.  The pages' GroupLinear is an FP8 DeepGEMM kernel for NVIDIA
// parts; this one is bf16 on CDNA4 matrix cores:
//  * a workgroup computes a 128 x 128 tile of one expert's output; its
//    m-tiles are numbered expert by expert (the 128-row tiles of expert e
//    start at tile sum_{e'<e} ceil(count[e'] / 128)), so each expert's
//    ragged last tile stays inside its segment;
//  * both operands are K-contiguous rows (token rows of x_perm, weight rows
//    of one output each), loaded with coalesced 16-byte loads into LDS tiles
//    with an XOR swizzle (16-byte chunk c of row r at c ^ (r & 7)), double
//    buffered: the next 64-wide K step is loaded into registers while the
//    current one feeds the matrix cores;
//  * 4 waves, each a 64 x 64 quarter: 4 x 4 v_mfma_f32_16x16x32_bf16 tiles,
//    fp32 accumulation, one rounding to bf16 at the end.
// fp32 inputs use a plain fp32 FMA kernel (one output per thread).
#include "moe_internal.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 128;  // rows (tokens) per tile
constexpr int GBN = 128;  // outputs per tile
constexpr int GBK = 64;   // K step (h)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// This workgroup's expert and rows: tiles are numbered expert by expert.
// Offsets are clamped to [0, T] (inconsistent ones give wrong rows, never an
// access outside x_perm or y).  Returns false if the id is past the last tile.
__device__ __forceinline__ bool tile_of(const int32_t* offsets, int E, int64_t T, int id,
                                        int* s_e, int64_t* s_m0, int* s_rows, int* s_scan) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t o0 = tid < E ? min(max((int64_t)offsets[tid], (int64_t)0), T) : 0;
  const int64_t o1 = tid < E ? min(max((int64_t)offsets[tid + 1], o0), T) : 0;
  const int nt = (int)((o1 - o0 + GBM - 1) / GBM);
  const int incl = wave_inclusive_sum(nt);
  if (lane == 63) s_scan[wid] = incl;
  if (tid == 0) *s_e = -1;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) base += w < wid ? s_scan[w] : 0;
  const int cb = base + incl - nt;
  if (tid < E && id >= cb && id < cb + nt) {
    *s_e = tid;
    *s_m0 = o0 + (int64_t)(id - cb) * GBM;
    *s_rows = (int)min((int64_t)GBM, o1 - *s_m0);
  }
  __syncthreads();
  return *s_e >= 0;
}

__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ offsets, int E, int64_t T, int H, int F,
    uint16_t* __restrict__ y) {
  __shared__ __align__(16) char sA[2][GBM * 128];
  __shared__ __align__(16) char sB[2][GBN * 128];
  __shared__ int s_e, s_rows;
  __shared__ int64_t s_m0;
  __shared__ int s_scan[4];
  if (!tile_of(offsets, E, T, blockIdx.x, &s_e, &s_m0, &s_rows, s_scan)) return;
  const int e = s_e;
  const int64_t m0 = s_m0;
  const int rows = s_rows;
  const int n0 = blockIdx.y * GBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int wm = wid & 1;
  const int wn = wid >> 1;

  // global -> LDS mapping: 4 chunks of 16 bytes per thread and operand; 8
  // threads cover one 128-byte row segment.  Rows past the tile's valid rows
  // (outputs past F) reload the last valid one; they are never stored.
  const uint16_t* ap[4];
  const uint16_t* bp[4];
  int loff[4], lch[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int rr = idx >> 3;
    const int ch = idx & 7;
    lch[i] = ch;
    ap[i] = x + (m0 + min(rr, rows - 1)) * H + 8 * ch;
    bp[i] = w + ((int64_t)e * F + min(n0 + rr, F - 1)) * H + 8 * ch;
    loff[i] = rr * 128 + ((ch ^ (rr & 7)) << 4);
  }
  // fragment offsets: A rows 64*wm + 16*mi + r, B rows 64*wn + 16*ni + r,
  // chunk 4*kh + g of the 64-wide step
  int aoff[4][2], boff[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int ra = 64 * wm + 16 * t + r;
      const int rb = 64 * wn + 16 * t + r;
      aoff[t][kh] = ra * 128 + (((4 * kh + g) ^ (ra & 7)) << 4);
      boff[t][kh] = rb * 128 + (((4 * kh + g) ^ (rb & 7)) << 4);
    }

  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  // a full K step: plain loads, consumed only by the LDS stores
  auto gload = [&](u32x4 (&ra)[4], u32x4 (&rb)[4], int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + kt * GBK);
      rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + kt * GBK);
    }
  };
  // the ragged last K step (H % 64 != 0; H % 8 == 0): chunks with h >= H are
  // zero, their loads read column 0 of the row instead
  auto gload_masked = [&](u32x4 (&ra)[4], u32x4 (&rb)[4], int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = kt * GBK + 8 * lch[i] < H;
      const int ko = ok ? kt * GBK : -8 * lch[i];
      const u32x4 va = *reinterpret_cast<const u32x4*>(ap[i] + ko);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(bp[i] + ko);
      ra[i] = ok ? va : zero;
      rb[i] = ok ? vb : zero;
    }
  };
  auto lstore = [&](int buf, const u32x4 (&ra)[4], const u32x4 (&rb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(sA[buf] + loff[i]) = ra[i];
      *reinterpret_cast<u32x4*>(sB[buf] + loff[i]) = rb[i];
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = *reinterpret_cast<const u32x4*>(sA[buf] + aoff[t][kh]);
        bf[t] = *reinterpret_cast<const u32x4*>(sB[buf] + boff[t][kh]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[mi]),
                                                                as_bf16x8(bf[ni]), acc[mi][ni],
                                                                0, 0, 0);
    }
  };

  // Double-buffered over the full K steps.  The loop body has no branches
  // (a branch makes the compiler wait for every outstanding load at its
  // end): the next step's loads are always issued, clamped to the last step,
  // and always stored to the other buffer, which nothing reads after the
  // last step.  The loads stay in flight under the MFMAs of the current step.
  const int nfull = H / GBK;
  u32x4 ra[4], rb[4];
  if (nfull > 0) {
    gload(ra, rb, 0);
    lstore(0, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < nfull; ++kt) {
      const int cur = kt & 1;
      gload(ra, rb, min(kt + 1, nfull - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(cur);
      __builtin_amdgcn_sched_barrier(0);
      lstore(cur ^ 1, ra, rb);
      __syncthreads();
    }
  }
  if (H % GBK) {
    gload_masked(ra, rb, nfull);
    lstore(0, ra, rb);
    __syncthreads();
    compute(0);
  }

  // lane (g, r), tile (mi, ni), element i: output row 64*wm + 16*mi + 4*g + i,
  // column n0 + 64*wn + 16*ni + r
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = n0 + 64 * wn + 16 * ni + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 64 * wm + 16 * mi + 4 * g + i;
        if (row < rows && col < F)
          y[(m0 + row) * F + col] = (uint16_t)f32_to_bf16_rne(acc[mi][ni][i]);
      }
    }
}

// fp32: one output per thread, h ascending (small shapes).
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ offsets,
                                                               int E, int64_t T, int H, int F,
                                                               float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * F) return;
  const int64_t p = idx / F;
  const int f = (int)(idx - p * F);
  // the segment holding p (offsets clamped to [0, T]); rows past offsets[E]
  // belong to no expert
  int e = -1;
  int64_t lo = 0;
  for (int j = 0; j < E; ++j) {
    const int64_t hi = min(max((int64_t)offsets[j + 1], lo), T);
    if (e < 0 && p >= lo && p < hi) e = j;
    lo = hi;
  }
  if (e < 0) return;
  const float* xr = x + p * H;
  const float* wr = w + ((int64_t)e * F + f) * H;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
  y[p * F + f] = acc;
}

}  // namespace

int64_t grouped_gemm_max_tiles(int64_t T, int E) { return (T + GBM - 1) / GBM + E; }

hipError_t launch_grouped_linear(const void* x_perm, const void* weight, const int32_t* offsets,
                                 int64_t T, int H, int E, int F, bool bf16, void* y,
                                 hipStream_t s) {
  if (bf16) {
    const dim3 grid((unsigned)grouped_gemm_max_tiles(T, E), (unsigned)((F + GBN - 1) / GBN));
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel, grid, dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(x_perm),
                       reinterpret_cast<const uint16_t*>(weight), offsets, E, T, H, F,
                       reinterpret_cast<uint16_t*>(y));
  } else {
    hipLaunchKernelGGL(grouped_gemm_f32_kernel, dim3((unsigned)((T * F + 255) / 256)), dim3(256),
                       0, s, reinterpret_cast<const float*>(x_perm),
                       reinterpret_cast<const float*>(weight), offsets, E, T, H, F,
                       reinterpret_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
