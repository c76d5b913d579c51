// Counting-sort MoE dispatch for gfx950: per-expert histogram, exclusive
// prefix sums, stable scatter of the N*K (token, expert) slots, and the copy
// of token rows into expert-contiguous order.
//
// Method: "Building a MoE training stack in 10k lines of Python", section 8.2
// "O(n) counting sort instead of O(n log n) argsort": an atomic-free parallel
// bincount over per-block private histograms, a reduction + prefix sum, and a
// counting-sort scatter producing the expand index -- replacing a chain of
// argsort / nonzero / searchsorted / repeat_interleave launches with fixed-size
// outputs.  The kernels here keep that three-kernel shape, on CDNA4:
//
//  count   (one workgroup per block of bt tokens)  stable rank of every slot
//          among the equal ids of its block (wave ballots on the id bits, then
//          per-wave counts in LDS), and the block's per-expert histogram
//          -> lrank[slot], bhist[e][block]
//  scan    (one workgroup per expert)  exclusive scan of bhist[e][:] across
//          blocks, in place; counts[e] = total
//  scatter (one workgroup per token)  offsets = exclusive scan of counts (each
//          workgroup redoes this E-wide scan in LDS; workgroup 0 stores it);
//          inv[slot] = offsets[e] + bhist[e][block] + lrank[slot]; perm; then
//          the token's row is read once with 16-byte loads (issued before the
//          index work) and written to its K rows with 16-byte stores.
//
// The block-prefix form (K <= 4 and at most 512 blocks; api.hip decides):
// the count kernel -- or, in moe_route_dispatch, the router's epilogue -- stores
// only each block's histogram and its exclusive prefix over the experts, and
// the scatter (MODE 3) finds each slot's position from those and from the
// earlier equal ids of its block: no ranking pass, no scan kernel.  Beyond
// those limits the count kernel (or the router's epilogue) ranks the slots
// and the scan kernel runs.  With a bhist of at most kSumAllMaxInts entries
// (small N and E) every scatter workgroup also sums whole histogram rows for
// the totals, so no scan kernel runs either.  Right after the router, the
// scatter takes its tokens in the router's XCD order, the router's last
// blocks first (see scatter_token), so its re-read of x finds the rows the
// memory-side cache received most recently.
//
// Atomics only ever produce counts; every position comes from a deterministic
// rank, so the output is bitwise reproducible and equal to a stable argsort.
// An id outside [0, E) is not dispatched: it is left out of the counts, its
// inv entry is -1 and no row is written for it (no out-of-range access).
#include "moe_internal.h"

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_SCATTER_NT_LOAD
#define MOE_SCATTER_NT_LOAD 1  // non-temporal loads of x
#endif
#ifndef MOE_SCATTER_NT_STORE
#define MOE_SCATTER_NT_STORE 1 // non-temporal stores of x_perm (keeps them out of L2/MALL)
#endif
#ifndef MOE_SCATTER_TOKENS
#define MOE_SCATTER_TOKENS 1   // tokens per scatter workgroup
#endif
#ifndef MOE_SCATTER_XCD
#define MOE_SCATTER_XCD 1      // scatter tokens in the router's XCD order, last blocks first
#endif
#ifndef MOE_SCATTER_U
#define MOE_SCATTER_U 2        // row vectors per lane loaded before their stores
#endif

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kScatterTokens = MOE_SCATTER_TOKENS;
#ifndef MOE_SCATTER_SUMALL_INTS
#define MOE_SCATTER_SUMALL_INTS 1024  // bhist up to this size: the scatter sums it itself
#endif
constexpr int kSumAllMaxInts = MOE_SCATTER_SUMALL_INTS;

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

// With bpre, also each block's exclusive prefix of its histogram over the
// experts (for the scan-free scatter, MODE 3).
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                             int64_t N, int K, int E, int bt,
                                                             int nb, int32_t* __restrict__ lrank,
                                                             int32_t* __restrict__ bhist,
                                                             int32_t* __restrict__ bpre) {
  extern __shared__ int sids[];  // [bt*K]
  __shared__ int hist[kMaxExperts];
  __shared__ int wcnt[4 * kMaxExperts];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * bt;
  const int ntok = (int)min((int64_t)bt, N - n0);
  const int S = ntok * K;
  const int64_t s0 = n0 * K;
  for (int j = tid; j < S; j += 256) sids[j] = ids[s0 + j];
  if (bpre) {  // the scatter ranks each slot itself: histogram and prefix only
    block_hist_prefix<256>(sids, S, E, hist, bhist, bpre, nb, blockIdx.x, wsum);
    return;
  }
  block_stable_rank<4>(sids, S, E, lrank + s0, hist, wcnt);
  for (int e = tid; e < E; e += 256) bhist[(int64_t)e * nb + blockIdx.x] = hist[e];
}

// rows below `split` total into counts[row], the others into counts2[row - split]
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ bhist,
                                                            int nb,
                                                            int32_t* __restrict__ counts,
                                                            int split,
                                                            int32_t* __restrict__ counts2) {
  __shared__ int lds[4];
  int32_t* row = bhist + (int64_t)blockIdx.x * nb;
  const int per = (nb + 255) / 256;
  const int b0 = threadIdx.x * per;
  const int b1 = min(nb, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += row[b];
  int total;
  int run = block_exclusive_scan_256(local, lds, &total);
  for (int b = b0; b < b1; ++b) {
    const int c = row[b];
    row[b] = run;
    run += c;
  }
  if (threadIdx.x == 0) {
    const int rr = (int)blockIdx.x;
    if (rr < split) counts[rr] = total;
    else counts2[rr - split] = total;
  }
}

// Token of scatter workgroup g.  With xbt > 0 (one token per workgroup, N a
// multiple of 8 * xbt): the router has just read x in blocks of xbt tokens,
// block j on XCD j % 8 (the dispatcher's round robin), so the last blocks'
// rows are the likeliest to still sit in the caches (the measured gain comes
// from the memory-side cache, which the L2 fetch counters cannot see).
// Workgroup g runs on XCD g % 8 and is given a token of a block of that XCD,
// the XCD's last blocks first.
// Otherwise tokens are taken in order.
__device__ __forceinline__ int64_t scatter_token(int64_t g, int64_t N, int xbt) {
  if (xbt == 0) return g * kScatterTokens;
  const int64_t x = g & 7, q = g >> 3;
  const int64_t per = N / (8 * (int64_t)xbt);  // blocks per XCD
  const int64_t i = per - 1 - q / xbt;
  return (int64_t)xbt * (x + 8 * i) + q % xbt;
}

// One workgroup per kScatterTokens tokens.  The rows' first loads are issued
// before the index work (they do not depend on it), so the E-wide offset
// scan and the index arithmetic overlap them.
// MODE 0: bhist holds the scanned block bases and counts the totals (the
// scan kernel ran).  MODE 2: bhist holds the raw per-block counts (small
// bhist only); each workgroup sums the blocks before its own for the experts
// of its slots (at most nb entries of one bhist row per slot) and whole bhist
// rows for the totals, workgroup 0 storing them to counts.
// MODE 3: bhist holds the raw per-block counts and bpre, per block, the
// exclusive prefix of the block's histogram over the experts; nothing else is
// needed (no in-block ranks).  A slot's position is sum_b bpre[e][b] (the
// slots of lower experts in every block, i.e. offsets[e]) + sum_{b < its
// block} bhist[e][b] + the number of earlier slots of its block with the
// same id: one wave per slot sums all three, so no counts have to be zeroed
// or added atomically beforehand, no E-wide scan runs and nobody ranks the
// blocks in advance.  The first workgroups also store counts and offsets.
template <int MODE>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    const int32_t* __restrict__ bhist, const int32_t* __restrict__ lrank, int64_t N, int K,
    int E, int nb, int bt, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, const u32x4* __restrict__ x, u32x4* __restrict__ x_perm,
    int row_vecs, int64_t dlim, int xbt, const int32_t* __restrict__ bpre) {
  extern __shared__ int dst[];  // [kScatterTokens*K], then (MODE >= 2) red[4][kScatterTokens*K]
  __shared__ int off[kMaxExperts];
  __shared__ int scan_lds[4];
  const int tid = threadIdx.x;
  const int64_t n0 = scatter_token(blockIdx.x, N, xbt);
  const int ntok = (int)min((int64_t)kScatterTokens, N - n0);
  int* red = dst + kScatterTokens * K;

  constexpr int U = MOE_SCATTER_U;
  const int total = ntok * row_vecs;
  const u32x4* xs = x + n0 * (int64_t)row_vecs;
  u32x4 v[U];
  if (x_perm != nullptr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(tid + u * 256, total - 1);
      v[u] = ld_row(xs + idx);
    }
  }

  const int S = ntok * K;
  const int64_t s0 = n0 * K;
  if constexpr (MODE == 3) {
    const int wv = tid >> 6, ln = tid & 63;
    for (int j = wv; j < S; j += 4) {
      const int64_t slot = s0 + j;
      const int e = ids[slot];
      int part = 0;
      if ((unsigned)e < (unsigned)E) {
        const int64_t b0 = (slot / K) / bt;
        const int32_t* pr = bpre + (int64_t)e * nb;
        const int32_t* hr = bhist + (int64_t)e * nb;
        for (int bb = ln; bb < nb; bb += 64) part += pr[bb] + (bb < b0 ? hr[bb] : 0);
        // its rank in its block: the block's earlier slots with the same id
        for (int64_t q = b0 * bt * K + ln; q < slot; q += 64) part += ids[q] == e ? 1 : 0;
      }
      part = wave_inclusive_sum(part);
      if (ln == 63) red[j] = part;
    }
    for (int g = blockIdx.x; g < E; g += gridDim.x) {  // uniform in the workgroup
      int c = 0, o = 0;
      for (int bb = tid; bb < nb; bb += 256) {
        c += bhist[(int64_t)g * nb + bb];
        o += bpre[(int64_t)g * nb + bb];
      }
      int ct, ot;
      block_exclusive_scan_256(c, scan_lds, &ct);
      block_exclusive_scan_256(o, scan_lds, &ot);
      if (tid == 0) {
        counts[g] = ct;
        offsets[g] = ot;
        if (g == E - 1) offsets[E] = ot + ct;
      }
    }
  } else if constexpr (MODE == 2) {
    // per slot: the counts of its expert in the blocks before its own (the
    // barriers of the offset scan below publish red)
    for (int j = 0; j < S; ++j) {
      const int64_t slot = s0 + j;
      const int e = ids[slot];
      const int64_t b = (slot / K) / bt;
      int part = 0;
      if ((unsigned)e < (unsigned)E)
        for (int64_t bb = tid; bb < b; bb += 256) part += bhist[(int64_t)e * nb + bb];
      part = __builtin_amdgcn_readlane(wave_inclusive_sum(part), 63);
      if ((tid & 63) == 0) red[(tid >> 6) * S + j] = part;
    }
  }

  // offsets = exclusive scan of counts (E <= 256: one expert per thread)
  if constexpr (MODE != 3) {
    int c = 0;
    if constexpr (MODE == 2) {
      if (tid < E) {
        const int32_t* row = bhist + (int64_t)tid * nb;
#pragma unroll 8
        for (int bb = 0; bb < nb; ++bb) c += row[bb];
        if (blockIdx.x == 0) counts[tid] = c;
      }
    } else {
      c = tid < E ? counts[tid] : 0;
    }
    int tot;
    const int ex = block_exclusive_scan_256(c, scan_lds, &tot);
    if (tid < E) off[tid] = ex;
    if (blockIdx.x == 0) {
      if (tid < E) offsets[tid] = ex;
      if (tid == 0) offsets[E] = tot;
    }
  }
  __syncthreads();

  for (int j = tid; j < S; j += 256) {
    const int64_t slot = s0 + j;
    const int e = ids[slot];
    int d = -1;
    if ((unsigned)e < (unsigned)E) {
      const int64_t b = (slot / K) / bt;
      int64_t dd;
      if constexpr (MODE == 3) {
        dd = (int64_t)red[j];
      } else {
        const int64_t base =
            MODE == 2 ? (int64_t)((red[j] + red[S + j]) + red[2 * S + j]) + red[3 * S + j]
                      : (int64_t)bhist[(int64_t)e * nb + b];
        dd = (int64_t)off[e] + base + lrank[slot];
      }
      if (dd >= 0 && dd < dlim) {  // always true for consistent inputs
        d = (int)dd;
        perm[d] = (int32_t)slot;
      }
    }
    inv[slot] = d;
    dst[j] = d;
  }
  if (x_perm == nullptr) return;
  __syncthreads();

  for (int base = 0; base < total; base += 256 * U) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = min(base + tid + u * 256, total - 1);
        v[u] = ld_row(xs + idx);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + tid + u * 256;
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

int64_t dispatch_num_blocks(int64_t N, int bt) { return (N + bt - 1) / bt; }

bool dispatch_needs_scan(int64_t nb, int E) { return nb * E > kSumAllMaxInts; }

hipError_t launch_dispatch_count(const int32_t* ids, int64_t N, int E, int K, int32_t* lrank,
                                 int32_t* bhist, hipStream_t s, int32_t* bpre) {
  const int bt = dispatch_count_tokens(K);
  const int nb = (int)dispatch_num_blocks(N, bt);
  const size_t dyn = sizeof(int) * (size_t)bt * K;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nb), dim3(256), dyn, s, ids, N, K, E, bt, nb,
                     lrank, bhist, bpre);
  return hipGetLastError();
}

hipError_t launch_dispatch_finish(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                                  int E, int K, int bt, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, void* x_perm,
                                  const int32_t* lrank, int32_t* bhist, hipStream_t s,
                                  int router_bt) {
  return launch_dispatch_finish(ids, x, N, row_bytes, E, K, bt, counts, offsets, perm, inv, x_perm,
                                lrank, bhist, N * K, s, router_bt);
}

// the token order of the scatter: XCD-matched to the router's blocks of
// router_bt tokens when that is a bijection, else in order
static int scatter_xbt(int64_t N, int router_bt) {
  if (MOE_SCATTER_XCD == 0 || router_bt <= 0 || kScatterTokens != 1) return 0;
  return N % (8 * (int64_t)router_bt) == 0 ? router_bt : 0;
}

hipError_t launch_dispatch_finish(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                                  int E, int K, int bt, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, void* x_perm,
                                  const int32_t* lrank, int32_t* bhist, int64_t dlim,
                                  hipStream_t s, int router_bt) {
  const int nb = (int)dispatch_num_blocks(N, bt);
  const int64_t blocks = (N + kScatterTokens - 1) / kScatterTokens;
  if ((int64_t)nb * E <= kSumAllMaxInts) {
    // a small bhist: every scatter workgroup sums it itself (no scan kernel;
    // measured slower from about 2048 entries on)
    const size_t dyn = sizeof(int) * 5 * (size_t)kScatterTokens * K;
    hipLaunchKernelGGL(dispatch_scatter_kernel<2>, dim3((unsigned)blocks), dim3(256), dyn, s, ids,
                       counts, bhist, lrank, N, K, E, nb, bt, offsets, perm, inv,
                       reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(x_perm),
                       (int)(row_bytes / 16), dlim, scatter_xbt(N, router_bt),
                       (const int32_t*)nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(E), dim3(256), 0, s, bhist, nb, counts, E,
                     (int32_t*)nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t dyn = sizeof(int) * (size_t)kScatterTokens * K;
  hipLaunchKernelGGL(dispatch_scatter_kernel<0>, dim3((unsigned)blocks), dim3(256), dyn, s, ids,
                     counts, bhist, lrank, N, K, E, nb, bt, offsets, perm, inv,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(x_perm),
                     (int)(row_bytes / 16), dlim, scatter_xbt(N, router_bt),
                     (const int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_dispatch_scatter_blockpre(const int32_t* ids, const void* x, int64_t N,
                                            int64_t row_bytes, int E, int K, int bt,
                                            int32_t* counts, int32_t* offsets, int32_t* perm,
                                            int32_t* inv, void* x_perm, const int32_t* lrank,
                                            const int32_t* bhist, const int32_t* bpre,
                                            hipStream_t s, int router_bt) {
  const int nb = (int)dispatch_num_blocks(N, bt);
  const int64_t blocks = (N + kScatterTokens - 1) / kScatterTokens;
  const size_t dyn = sizeof(int) * 5 * (size_t)kScatterTokens * K;
  hipLaunchKernelGGL(dispatch_scatter_kernel<3>, dim3((unsigned)blocks), dim3(256), dyn, s, ids,
                     counts, bhist, lrank, N, K, E, nb, bt, offsets, perm, inv,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(x_perm),
                     (int)(row_bytes / 16), N * K, scatter_xbt(N, router_bt < 0 ? bt : router_bt),
                     bpre);
  return hipGetLastError();
}

hipError_t launch_dispatch_scan(int32_t* bhist, int rows, int nb, int32_t* counts, int split,
                                int32_t* counts2, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(rows), dim3(256), 0, s, bhist, nb, counts, split,
                     counts2);
  return hipGetLastError();
}

}  // namespace moe
