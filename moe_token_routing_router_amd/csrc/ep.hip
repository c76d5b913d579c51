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
// Here the rank-level pass reuses the dispatch's own kernels on derived keys:
//  keys    (one thread per token)  key[slot] = rank of its expert if the slot
//          is the first of its token on that rank, else -1 (not dispatched);
//  count / scan / scatter (dispatch.hip) on the keys with R "experts": the
//          send counts and offsets, the owner slots' send rows, the send slot
//          of each row, and the row copy x_send[row] = x[token];
//  finish  (one thread per slot)  send_tok = send slot / K; every slot's send
//          row (the owner's for slots sharing a rank); expand_idx for every
//          dispatched row of the expert-level pass.
#include "moe_internal.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void ep_keys_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                      int K, int E, int per_rank,
                                                      int32_t* __restrict__ keys) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int32_t* row = ids + n * K;
  for (int k = 0; k < K; ++k) {
    const int e = row[k];
    int key = -1;
    if ((unsigned)e < (unsigned)E) {
      const int r = e / per_rank;
      bool first = true;
      for (int k2 = 0; k2 < k; ++k2) {
        const int e2 = row[k2];
        first = first && !((unsigned)e2 < (unsigned)E && e2 / per_rank == r);
      }
      key = first ? r : -1;
    }
    keys[n * K + k] = key;
  }
}

// send row of token n for rank r: the row of its first slot on that rank
__device__ __forceinline__ int32_t owner_row_of(const int32_t* ids, const int32_t* owner_row,
                                                int64_t n, int K, int E, int per_rank, int r) {
  for (int k2 = 0; k2 < K; ++k2) {
    const int e2 = ids[n * K + k2];
    if ((unsigned)e2 < (unsigned)E && e2 / per_rank == r) return owner_row[n * K + k2];
  }
  return -1;
}

__global__ __launch_bounds__(256) void ep_finish_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ owner_row,
    const int32_t* __restrict__ send_offsets, int64_t N, int K, int E, int R,
    int32_t* __restrict__ send_tok, int32_t* __restrict__ send_row,
    int32_t* __restrict__ expand_idx) {
  const int64_t T = N * K;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= T) return;
  const int per_rank = E / R;
  // send row j: its slot -> its token
  if (j < send_offsets[R]) send_tok[j] = send_tok[j] / K;
  // slot j's send row
  {
    const int e = ids[j];
    send_row[j] = (unsigned)e < (unsigned)E
                      ? owner_row_of(ids, owner_row, j / K, K, E, per_rank, e / per_rank)
                      : -1;
  }
  // dispatched row j (expert-contiguous order) on the receiving rank
  {
    int32_t v = -1;
    if (j < offsets[E]) {
      const int64_t i = perm[j];
      const int r = ids[i] / per_rank;
      v = owner_row_of(ids, owner_row, i / K, K, E, per_rank, r) - send_offsets[r];
    }
    expand_idx[j] = v;
  }
}

}  // namespace

hipError_t launch_ep_keys(const int32_t* ids, int64_t N, int K, int E, int per_rank,
                          int32_t* keys, hipStream_t s) {
  hipLaunchKernelGGL(ep_keys_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, ids, N,
                     K, E, per_rank, keys);
  return hipGetLastError();
}

hipError_t launch_ep_finish(const int32_t* ids, const int32_t* perm, const int32_t* offsets,
                            const int32_t* owner_row, const int32_t* send_offsets, int64_t N,
                            int K, int E, int R, int32_t* send_tok, int32_t* send_row,
                            int32_t* expand_idx, hipStream_t s) {
  const int64_t T = N * K;
  hipLaunchKernelGGL(ep_finish_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, ids,
                     perm, offsets, owner_row, send_offsets, N, K, E, R, send_tok, send_row,
                     expand_idx);
  return hipGetLastError();
}

}  // namespace moe
