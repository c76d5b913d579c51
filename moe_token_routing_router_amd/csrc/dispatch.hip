// Counting-sort MoE dispatch for gfx950: per-expert histogram, exclusive
// prefix sums, stable scatter of the N*K (token, expert) slots, and the copy
// of token rows into expert-contiguous order.
//
// Method: "Building a MoE training stack in 10k lines of Python", section 8.2
// "O(n) counting sort instead of O(n log n) argsort": an atomic-free parallel
// bincount over per-block private histograms, a reduction + prefix sum, and a
// counting-sort scatter producing the expand index -- replacing a chain of
// argsort / nonzero / searchsorted / repeat_interleave launches with fixed-size
// outputs.  This build keeps that three-kernel shape, on CDNA4:
//
//  hist  (grid = #sub-chunks, 1 wave each)  LDS-atomic histogram of the ids of
//        one sub-chunk of kDispatchTokens tokens -> blockcnt[e][sub]
//  scan  (grid = E, 256 threads)            exclusive scan of blockcnt[e][:]
//        across sub-chunks, in place; counts[e] = total
//  scatter (grid = #sub-chunks, 256 thr.)   offsets = exclusive scan of counts
//        (each block redoes this E-wide scan in LDS; block 0 stores it);
//        stable rank of every slot inside its sub-chunk; inv/perm; then the
//        block copies its tokens' rows, each row read once with 16-byte loads
//        and written K times with 16-byte stores.
//
// Atomics only ever produce counts; every position comes from a deterministic
// rank, so the output is bitwise reproducible and equal to a stable argsort.
// An id outside [0, E) is not dispatched: it is left out of the counts, its
// inv entry is -1 and no row is written for it (no out-of-range access).
#include "moe_internal.h"

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_SCATTER_U
#define MOE_SCATTER_U 4        // row vectors loaded per lane before their stores
#endif
#ifndef MOE_SCATTER_NT_LOAD
#define MOE_SCATTER_NT_LOAD 1  // non-temporal loads of x
#endif
#ifndef MOE_SCATTER_NT_STORE
#define MOE_SCATTER_NT_STORE 1 // non-temporal stores of x_perm (keeps them out of L2/MALL)
#endif

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_row(const u32x4* p) {
#if MOE_SCATTER_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ void st_row(u32x4* p, u32x4 v) {
#if MOE_SCATTER_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Exclusive scan of one int per thread over a 256-thread block.
// `lds` needs 4 ints.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) lds[wid] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = lds[w];
    if (w < wid) wbase += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

__global__ __launch_bounds__(64) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                           int64_t T, int K, int E, int num_sub,
                                                           int32_t* __restrict__ blockcnt) {
  __shared__ int h[kMaxExperts];
  const int tid = threadIdx.x;
  const int sub = blockIdx.x;
  for (int e = tid; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)sub * kDispatchTokens * K;
  int64_t s1 = s0 + (int64_t)kDispatchTokens * K;
  if (s1 > T) s1 = T;
  for (int64_t s = s0 + tid; s < s1; s += 64) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 64) blockcnt[(int64_t)e * num_sub + sub] = h[e];
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ blockcnt,
                                                            int num_sub,
                                                            int32_t* __restrict__ counts) {
  __shared__ int lds[4];
  int32_t* row = blockcnt + (int64_t)blockIdx.x * num_sub;
  const int per = (num_sub + 255) / 256;
  const int b0 = threadIdx.x * per;
  const int b1 = min(num_sub, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += row[b];
  int total;
  int run = block_exclusive_scan_256(local, lds, &total);
  for (int b = b0; b < b1; ++b) {
    const int c = row[b];
    row[b] = run;
    run += c;
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ blockcnt, int64_t N, int K, int E, int num_sub,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    const u32x4* __restrict__ x, u32x4* __restrict__ x_perm, int row_vecs) {
  extern __shared__ int dyn[];  // sid[S] then dst[S], S = kDispatchTokens*K
  __shared__ int off[kMaxExperts];
  __shared__ int scan_lds[4];
  const int tid = threadIdx.x;
  const int sub = blockIdx.x;

  // offsets = exclusive scan of counts (E <= 256: one expert per thread)
  {
    const int c = tid < E ? counts[tid] : 0;
    int total;
    const int ex = block_exclusive_scan_256(c, scan_lds, &total);
    if (tid < E) off[tid] = ex;
    if (sub == 0) {
      if (tid < E) offsets[tid] = ex;
      if (tid == 0) offsets[E] = total;
    }
  }

  const int64_t n0 = (int64_t)sub * kDispatchTokens;
  const int ntok = (int)min((int64_t)kDispatchTokens, N - n0);
  const int S = ntok * K;
  const int64_t s0 = n0 * K;
  int* sid = dyn;
  int* dst = dyn + kDispatchTokens * K;
  for (int j = tid; j < S; j += 256) sid[j] = ids[s0 + j];
  __syncthreads();  // also publishes off[]

  // stable rank inside the sub-chunk: earlier slots with the same expert
  for (int j = tid; j < S; j += 256) {
    const int e = sid[j];
    int d = -1;
    if ((unsigned)e < (unsigned)E) {
      int rank = 0;
      for (int q = 0; q < j; ++q) rank += (sid[q] == e);
      d = off[e] + blockcnt[(int64_t)e * num_sub + sub] + rank;
      perm[d] = (int32_t)(s0 + j);
    }
    inv[s0 + j] = d;
    dst[j] = d;
  }
  if (x_perm == nullptr) return;
  __syncthreads();

  // copy: flat index over (token, 16-byte column); each row is read once and
  // stored to its K dispatched rows.  U loads are issued before their stores.
  constexpr int U = MOE_SCATTER_U;
  const int total = ntok * row_vecs;
  const u32x4* xs = x + n0 * (int64_t)row_vecs;
  for (int base = tid; base < total; base += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(base + u * 256, total - 1);
      v[u] = ld_row(xs + idx);  // idx < ntok * row_vecs: token idx / row_vecs of this block
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256;
      if (idx < total) {
        const int tt = idx / row_vecs;
        const int c = idx - tt * row_vecs;
        const int* dd = dst + tt * K;
        for (int k = 0; k < K; ++k) {
          const int d = dd[k];
          if (d >= 0) st_row(x_perm + (int64_t)d * row_vecs + c, v[u]);
        }
      }
    }
  }
}

}  // namespace

int64_t dispatch_num_sub(int64_t N) { return (N + kDispatchTokens - 1) / kDispatchTokens; }

hipError_t launch_dispatch(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes, int E,
                           int K, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           void* x_perm, int32_t* blockcnt, hipStream_t s) {
  const int64_t T = N * K;
  const int num_sub = (int)dispatch_num_sub(N);
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(num_sub), dim3(64), 0, s, ids, T, K, E, num_sub,
                     blockcnt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(E), dim3(256), 0, s, blockcnt, num_sub, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t dyn = sizeof(int) * 2 * (size_t)kDispatchTokens * K;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(num_sub), dim3(256), dyn, s, ids, counts,
                     blockcnt, N, K, E, num_sub, offsets, perm, inv,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(x_perm),
                     (int)(row_bytes / 16));
  return hipGetLastError();
}

}  // namespace moe
