// Expert-parallel send metadata on one GPU, with the ranks simulated as
// segments of one buffer.
//
// Method: "Building a MoE training stack in 10k lines of Python", section 8.2
// "O(n) counting sort instead of O(n log n) argsort": besides the per-expert
// counts, the dispatch counts tokens per expert-parallel rank, builds prefix
// sums and send metadata, and scatters each token once per destination rank
// (deduplication) with a counting sort, producing the index a receiver uses
// to expand its rows to its experts.
//
// Both levels run in the dispatch's three-kernel shape, side by side:
//  count   (one workgroup per block of bt tokens)  the stable rank of every
//          slot among the equal expert ids of its block, and among the equal
//          rank keys, where key[slot] = rank of its expert if the slot is the
//          first of its token on that rank, else -1 (not sent: deduplicated);
//          the block histograms of both -> bhist [E + R][blocks]
//  scan    (one workgroup per expert and per rank)  exclusive scan of each
//          bhist row in place; counts[e] and send_counts[r] = the totals
//  scatter (one workgroup per token)  offsets and send_offsets (E- and R-wide
//          scans in LDS; workgroup 0 stores them); the token's owner slots
//          get their send rows (send_tok); every slot gets its expert-level
//          position (perm, inv), its send row (its token's owner on that
//          rank) and, at its dispatched position, the receiver's expand index;
//          then the token's row is read once and written to its send rows.
// Every position comes from a deterministic rank: the output equals that of
// stable argsorts, bit for bit, run to run.
#include "moe_internal.h"

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kEpRowU = 2;  // row vectors per lane loaded before their stores

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ bool valid_id(int e, int E) { return (unsigned)e < (unsigned)E; }

// Slot k of a token whose K expert ids are tok[0..K): the rank of its expert
// if no earlier slot of the token is on that rank, else -1 (also for an id
// outside [0, E)).
__device__ __forceinline__ int ep_key(const int* tok, int k, int E, int per_rank) {
  const int e = tok[k];
  if (!valid_id(e, E)) return -1;
  const int r = e / per_rank;
  for (int k2 = 0; k2 < k; ++k2) {
    const int e2 = tok[k2];
    if (valid_id(e2, E) && e2 / per_rank == r) return -1;
  }
  return r;
}

__global__ __launch_bounds__(256) void ep_count_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                       int K, int E, int R, int bt, int nb,
                                                       int32_t* __restrict__ lrank_e,
                                                       int32_t* __restrict__ lrank_r,
                                                       int32_t* __restrict__ bhist) {
  extern __shared__ int sm[];  // ids [bt*K], then keys [bt*K]
  __shared__ int hist[kMaxExperts];
  __shared__ int wcnt[4 * kMaxExperts];
  int* sids = sm;
  int* skeys = sm + bt * K;
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * bt;
  const int ntok = (int)min((int64_t)bt, N - n0);
  const int S = ntok * K;
  const int64_t s0 = n0 * K;
  for (int j = tid; j < S; j += 256) sids[j] = ids[s0 + j];
  __syncthreads();
  const int per_rank = E / R;
  for (int j = tid; j < S; j += 256) {
    const int t = j / K;
    skeys[j] = ep_key(sids + t * K, j - t * K, E, per_rank);
  }
  // (the ranking's first barrier publishes the keys)
  block_stable_rank<4>(sids, S, E, lrank_e + s0, hist, wcnt);
  for (int e = tid; e < E; e += 256) bhist[(int64_t)e * nb + blockIdx.x] = hist[e];
  __syncthreads();  // hist is read above and cleared by the next ranking
  block_stable_rank<4>(skeys, S, R, lrank_r + s0, hist, wcnt);
  for (int r = tid; r < R; r += 256) bhist[(int64_t)(E + r) * nb + blockIdx.x] = hist[r];
}

__global__ __launch_bounds__(256) void ep_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ send_counts, const int32_t* __restrict__ bhist,
    const int32_t* __restrict__ lrank_e, const int32_t* __restrict__ lrank_r, int64_t N, int K,
    int E, int R, int nb, int bt, int64_t cap, int32_t* __restrict__ offsets,
    int32_t* __restrict__ send_offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ send_tok, int32_t* __restrict__ send_row,
    int32_t* __restrict__ expand_idx, const u32x4* __restrict__ x, u32x4* __restrict__ x_send,
    int row_vecs) {
  extern __shared__ int sm[];  // the token's ids [K], then its owner slots' send rows [K]
  __shared__ int off_e[kMaxExperts];
  __shared__ int off_r[kMaxExperts];
  __shared__ int scan_lds[4];
  int* tids = sm;
  int* own = sm + K;
  const int tid = threadIdx.x;
  const int64_t n = blockIdx.x;
  const int64_t s0 = n * K;
  const int64_t T = N * K;

  // the row's first loads do not depend on the index work: issue them first
  constexpr int U = kEpRowU;
  const u32x4* xs = x + n * (int64_t)row_vecs;
  u32x4 v[U];
  if (x_send != nullptr) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_nt(xs + min(tid + u * 256, row_vecs - 1));
  }
  for (int k = tid; k < K; k += 256) tids[k] = ids[s0 + k];

  int tot_e, tot_r;
  {
    const int c = tid < E ? counts[tid] : 0;
    const int ex = block_exclusive_scan_256(c, scan_lds, &tot_e);
    if (tid < E) off_e[tid] = ex;
    if (n == 0) {
      if (tid < E) offsets[tid] = ex;
      if (tid == 0) offsets[E] = tot_e;
    }
  }
  {
    const int c = tid < R ? send_counts[tid] : 0;
    const int ex = block_exclusive_scan_256(c, scan_lds, &tot_r);
    if (tid < R) off_r[tid] = ex;
    if (n == 0) {
      if (tid < R) send_offsets[tid] = ex;
      if (tid == 0) send_offsets[R] = tot_r;
    }
  }
  __syncthreads();  // tids, off_e, off_r

  const int per_rank = E / R;
  const int64_t b = n / bt;
  // owner slots: their send rows
  for (int k = tid; k < K; k += 256) {
    const int key = ep_key(tids, k, E, per_rank);
    int d = -1;
    if (key >= 0) {
      const int64_t dd =
          (int64_t)off_r[key] + bhist[(int64_t)(E + key) * nb + b] + lrank_r[s0 + k];
      if (dd >= 0 && dd < cap) {  // always true for consistent inputs
        d = (int)dd;
        send_tok[d] = (int32_t)n;
      }
    }
    own[k] = d;
  }
  __syncthreads();
  // every slot: its send row, its dispatched position, the expand index there
  for (int k = tid; k < K; k += 256) {
    const int e = tids[k];
    int srow = -1, pos = -1;
    if (valid_id(e, E)) {
      const int r = e / per_rank;
      int k0 = 0;  // the owner: the first slot of the token on rank r (k0 <= k)
      while (!(valid_id(tids[k0], E) && tids[k0] / per_rank == r)) ++k0;
      srow = own[k0];
      const int64_t dd = (int64_t)off_e[e] + bhist[(int64_t)e * nb + b] + lrank_e[s0 + k];
      if (dd >= 0 && dd < T) {  // always true for consistent inputs
        pos = (int)dd;
        perm[pos] = (int32_t)(s0 + k);
        expand_idx[pos] = srow >= 0 ? srow - off_r[r] : -1;
      }
    }
    send_row[s0 + k] = srow;
    inv[s0 + k] = pos;
    // rows past offsets[E] exist only for ids outside [0, E): nothing is
    // dispatched there
    if (s0 + k >= tot_e) expand_idx[s0 + k] = -1;
  }
  if (x_send == nullptr) return;

  for (int base = 0; base < row_vecs; base += 256 * U) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_nt(xs + min(base + tid + u * 256, row_vecs - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + tid + u * 256;
      if (idx < row_vecs) {
        for (int k = 0; k < K; ++k) {
          const int d = own[k];
          if (d >= 0) st_nt(x_send + (int64_t)d * row_vecs + idx, v[u]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_ep_dispatch(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                              int E, int K, int R, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, int32_t* send_counts,
                              int32_t* send_offsets, int32_t* send_tok, int32_t* send_row,
                              int32_t* expand_idx, void* x_send, int32_t* bhist,
                              int32_t* lrank_e, int32_t* lrank_r, hipStream_t s) {
  const int bt = dispatch_count_tokens(K);
  const int nb = (int)dispatch_num_blocks(N, bt);
  hipLaunchKernelGGL(ep_count_kernel, dim3(nb), dim3(256), sizeof(int) * 2 * (size_t)bt * K, s,
                     ids, N, K, E, R, bt, nb, lrank_e, lrank_r, bhist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_dispatch_scan(bhist, E + R, nb, counts, E, send_counts, s);
  if (err != hipSuccess) return err;
  const int64_t cap = N * (int64_t)(K < R ? K : R);
  hipLaunchKernelGGL(ep_scatter_kernel, dim3((unsigned)N), dim3(256), sizeof(int) * 2 * (size_t)K,
                     s, ids, counts, send_counts, bhist, lrank_e, lrank_r, N, K, E, R, nb, bt,
                     cap, offsets, send_offsets, perm, inv, send_tok, send_row, expand_idx,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(x_send),
                     (int)(row_bytes / 16));
  return hipGetLastError();
}

}  // namespace moe
