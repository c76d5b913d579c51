// Internal declarations shared by the HIP translation units of libmoe.so.
// Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

// ---- limits -------------------------------------------------------------
constexpr int kMaxExperts = 256;     // selection range of the fused router
constexpr int kMaxRouteK = 16;       // one 16-lane group keeps one pick per lane
// tokens per block of the standalone count kernel (at most 4096 slots, so
// its LDS copy of the ids stays at 16 KiB)
inline int dispatch_count_tokens(int K) { return K <= 64 ? 64 : 4096 / K; }

// ---- occupancy ------------------------------------------------------------
// Dynamic LDS reserved per workgroup so that at most w workgroups share a CU
// (160 KiB of LDS per CU on gfx950; 2 KiB below the exact share, which covers
// the kernel's own LDS and the allocation granularity, and still leaves no
// room for a (w+1)-th).
constexpr size_t kLdsPerCu = 160 * 1024;
inline size_t lds_for_workgroups_per_cu(int w) { return kLdsPerCu / w - 2048; }

// The per-token gathers (combine, aggregate, dispatch and combine backward)
// over large batches with large rows run faster with fewer workgroups in
// flight per CU than the wave slots allow: about `budget` bytes of rows
// moved per CU at once.  From 16384 tokens, 4 KiB rows and 24 KiB of rows
// per workgroup on, the dynamic LDS that caps a CU at budget / (rows *
// row_bytes) workgroups (at least 3); 0 (no cap) otherwise.  Smaller rows
// or batches need every slot (measured: 1-2 KiB rows at 16384 tokens run
// 8-60 % slower under a cap).
inline size_t gather_lds_cap(int64_t N, size_t row_bytes, size_t rows, size_t budget) {
  const size_t bytes_per_workgroup = rows * row_bytes;
  if (N < 16384 || row_bytes < 4096 || bytes_per_workgroup < 24 * 1024) return 0;
  const size_t w = budget / bytes_per_workgroup;
  if (w >= 8) return 0;
  return lds_for_workgroups_per_cu(w < 3 ? 3 : (int)w);
}

// ---- vector types -------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 (bf16 is the upper half of a binary32) ---------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- wave-wide inclusive prefix sum with DPP ------------------------------
// Hillis-Steele inside each 16-lane row (row_shr 1, 2, 4, 8: a lane without
// a source adds 0), then row_bcast:15 adds row 0's total to row 1 and row 2's
// to row 3, and row_bcast:31 adds lane 31's (rows 0-1) to rows 2 and 3.
// Register-to-register moves, no LDS round trips.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_add_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += dpp_add_src<0x111>(v);         // row_shr:1
  v += dpp_add_src<0x112>(v);         // row_shr:2
  v += dpp_add_src<0x114>(v);         // row_shr:4
  v += dpp_add_src<0x118>(v);         // row_shr:8
  v += dpp_add_src<0x142, 0xA>(v);    // row_bcast:15 into rows 1, 3
  v += dpp_add_src<0x143, 0xC>(v);    // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive scan of one int per thread over a 256-thread block.
// `lds` needs 4 ints.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int incl = wave_inclusive_sum(v);
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

// ---- wave-wide float sum, fixed order --------------------------------------
// Butterfly inside each 16-lane row (DPP quad_perm xor 1, xor 2,
// row_half_mirror, row_mirror: every lane ends with its row's sum), then the
// four row sums are added in row order.  The same order on every call.
template <int CTRL>
__device__ __forceinline__ float dpp_mov_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_mov_f32<0xB1>(v);   // quad_perm(1,0,3,2)
  v += dpp_mov_f32<0x4E>(v);   // quad_perm(2,3,0,1)
  v += dpp_mov_f32<0x141>(v);  // row_half_mirror
  v += dpp_mov_f32<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// The exactly rounded bf16 of a * b (fp32 a, b): the fp32 product p and its
// exact error e = a*b - p (one FMA) decide the one case where rounding p
// again could differ from rounding a*b directly -- p on a bf16 midpoint.
__device__ __forceinline__ uint32_t bf16_of_product(float a, float b) {
  const float p = __fmul_rn(a, b);
  const float e = __builtin_fmaf(a, b, -p);
  const uint32_t u = __float_as_uint(p);
  if ((u & 0xffffu) == 0x8000u && e != 0.f) {
    const bool away = (e > 0.f) == (p > 0.f);  // |a*b| above the midpoint
    return (u >> 16) + (away ? 1u : 0u);
  }
  return f32_to_bf16_rne(p);
}

// ---- block-level stable ranking ------------------------------------------
// For the S slot ids sids[0..S) of one block (in LDS, published by the
// caller's writes before the call), computes with NWAVES*64 threads:
//   out[j]  = #{ j' < j : sids[j'] == sids[j] }  for valid ids (0 <= id < E),
//             -1 for invalid ones (global memory);
//   hist[e] = #{ j : sids[j] == e }              (LDS, kMaxExperts ints).
// Slots are taken NWAVES*64 at a time.  Inside a wave, lanes holding the same
// id are found with one ballot per id bit (E <= 256: at most 8) and ranked by
// the count of matching lanes below them; per-wave counts in LDS (wcnt,
// NWAVES*kMaxExperts ints) give the offset of each wave, and hist carries the
// running count from round to round.  Every thread of the block must call it.
template <int NWAVES>
__device__ __forceinline__ void block_stable_rank(const int* sids, int S, int E, int32_t* out, int* hist,
                                  int* wcnt) {
  constexpr int NTH = NWAVES * 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int e = tid; e < E; e += NTH) hist[e] = 0;
  for (int i = tid; i < NWAVES * kMaxExperts; i += NTH) wcnt[i] = 0;
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int base = 0; base < S; base += NTH) {
    const int j = base + tid;
    const int e = (j < S) ? sids[j] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rw = __popcll(m & below);
    if (valid && rw == 0) wcnt[wid * kMaxExperts + e] = __popcll(m);
    __syncthreads();
    if (valid) {
      int rank = hist[e] + rw;
      for (int w = 0; w < wid; ++w) rank += wcnt[w * kMaxExperts + e];
      out[j] = rank;
    } else if (j < S) {
      out[j] = -1;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += NTH) {
      int sum = 0;
      for (int w = 0; w < NWAVES; ++w) {
        sum += wcnt[w * kMaxExperts + e2];
        wcnt[w * kMaxExperts + e2] = 0;
      }
      hist[e2] += sum;
    }
    __syncthreads();
  }
}

// bpre[e * nb + b] = sum over experts e' < e of rhist[e'], for e < E <= 256:
// the exclusive prefix of block b's histogram over the experts (the
// dispatch's scatter adds these up over the blocks to get the expert
// offsets).  The first four waves scan; every thread of the workgroup must
// call it; wsum needs 4 ints of LDS.
__device__ __forceinline__ void store_expert_prefix(const int* rhist, int E, int32_t* bpre, int nb,
                                                    int b, int* wsum) {
  const int tid = threadIdx.x;
  int v = 0, incl = 0;
  if (tid < 256) {
    v = tid < E ? rhist[tid] : 0;
    incl = wave_inclusive_sum(v);
    if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int base = 0;
    for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
    bpre[(int64_t)tid * nb + b] = base + incl - v;
  }
}

// The block's histogram of its S slot ids (E <= 256) in LDS by integer
// atomics (their order does not matter), then bhist[e * nb + b] and the
// block's exclusive prefix over the experts bpre[e * nb + b]: what the
// scatter needs when it ranks each slot itself.  Every thread of the
// workgroup (NTH of them) calls it after writing its sids; rhist holds E
// ints, wsum 4.
template <int NTH>
__device__ __forceinline__ void block_hist_prefix(const int* sids, int S, int E, int* rhist,
                                                  int32_t* bhist, int32_t* bpre, int nb, int b,
                                                  int* wsum) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NTH) rhist[e] = 0;
  __syncthreads();
  for (int j = tid; j < S; j += NTH) {
    const int e = sids[j];
    if ((unsigned)e < (unsigned)E) atomicAdd(&rhist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += NTH) bhist[(int64_t)e * nb + b] = rhist[e];
  store_expert_prefix(rhist, E, bpre, nb, b, wsum);
}

// ---- launchers (each validates nothing: the C ABI layer has done it) -----
// Router.  wgt is the fragment-major packed gate (bf16 path only).  When
// lrank is not null the router also ranks its own selections for the dispatch
// (blocks of route_tokens_per_block(E) tokens; see launch_dispatch_finish).
int route_padded_experts(int E);
int route_gate_rows(int H);  // H rounded up to whole 64-wide steps (packed gate)
int route_tokens_per_block(int E, int64_t N);  // tokens per router workgroup
// True when the bf16 router reads gate_w as it is (no packed copy, no
// packing kernel; wgt is then gate_w itself).
bool route_gate_raw(int E);
hipError_t launch_gate_transpose(const uint16_t* gate_w, int H, int E, uint16_t* wgt,
                                 int32_t* counts, hipStream_t s);
// bpre (fused path, optional): each block's exclusive prefix of its histogram
// over the experts, [E][blocks], for launch_dispatch_scatter_blockpre.
hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* wgt, const float* bias,
                             int64_t N, int H, int E, int K, int32_t* ids, float* w,
                             int32_t* counts, int32_t* lrank, int32_t* bhist, hipStream_t s,
                             int32_t* bpre = nullptr);
// The fp32 router works on blocks of kRouteF32Tokens tokens; with lrank it
// ranks its own picks per block like the bf16 router.
constexpr int kRouteF32Tokens = 16;
hipError_t launch_route_f32(const float* x, const float* gate_w, const float* bias, int64_t N,
                            int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                            int32_t* lrank, int32_t* bhist, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// Dispatch.  lrank [N*K] and bhist [E][dispatch_num_blocks(N, bt)] live in
// the workspace.  count: ranks + block histograms for bt = dispatch_count_tokens(K).
// finish: scan of bhist (in place) + counts, then scatter (offsets, inv,
// perm, rows).
int64_t dispatch_num_blocks(int64_t N, int bt);
// True when launch_dispatch_finish would run the scan kernel (the scatter
// sums a block histogram of nb blocks x E experts itself only when it is
// small).
bool dispatch_needs_scan(int64_t nb, int E);
// bpre (optional): each block's exclusive prefix over the experts, [E][nb].
hipError_t launch_dispatch_count(const int32_t* ids, int64_t N, int E, int K, int32_t* lrank,
                                 int32_t* bhist, hipStream_t s, int32_t* bpre = nullptr);
// router_bt > 0: x was just read by the router in blocks of that many
// tokens; the scatter then takes its tokens in the router's XCD order.
hipError_t launch_dispatch_finish(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                                  int E, int K, int bt, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, void* x_perm,
                                  const int32_t* lrank, int32_t* bhist, hipStream_t s,
                                  int router_bt = 0);
// ... with destinations limited to [0, dlim) (perm, x_perm capacity; N*K above)
hipError_t launch_dispatch_finish(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                                  int E, int K, int bt, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, void* x_perm,
                                  const int32_t* lrank, int32_t* bhist, int64_t dlim,
                                  hipStream_t s, int router_bt = 0);

// scatter only: bhist holds raw per-block counts (blocks of bt tokens) and
// bpre each block's exclusive prefix over the experts (from the router's
// epilogue or the count kernel); writes counts and offsets too.  Tokens in
// the XCD order of a router that read x in blocks of router_bt tokens (-1:
// bt).
hipError_t launch_dispatch_scatter_blockpre(const int32_t* ids, const void* x, int64_t N,
                                            int64_t row_bytes, int E, int K, int bt,
                                            int32_t* counts, int32_t* offsets, int32_t* perm,
                                            int32_t* inv, void* x_perm, const int32_t* lrank,
                                            const int32_t* bhist, const int32_t* bpre,
                                            hipStream_t s, int router_bt = -1);

// Scan of `rows` bhist rows of nb blocks (in place, exclusive); the totals
// of rows below `split` go to counts[row], the others to counts2[row - split].
hipError_t launch_dispatch_scan(int32_t* bhist, int rows, int nb, int32_t* counts, int split,
                                int32_t* counts2, hipStream_t s);

// Expert-parallel metadata (ep.hip): count, scan and scatter of both levels
// (experts and deduplicated ranks).  Scratch: bhist [E+R][dispatch_num_blocks(
// N, dispatch_count_tokens(K))], lrank_e and lrank_r [N*K].
hipError_t launch_ep_dispatch(const int32_t* ids, const void* x, int64_t N, int64_t row_bytes,
                              int E, int K, int R, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, int32_t* send_counts,
                              int32_t* send_offsets, int32_t* send_tok, int32_t* send_row,
                              int32_t* expand_idx, void* x_send, int32_t* bhist,
                              int32_t* lrank_e, int32_t* lrank_r, hipStream_t s);

// Combine (w may be null: unit weights, the dispatch backward; residual, if
// given, is added after the expert terms: forward_aggregate).
hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t N, int H,
                          int K, bool bf16, void* out, hipStream_t s,
                          const void* residual = nullptr);

// Grouped expert linear layer (grouped_gemm.hip): y rows p < offsets[E]
// (offsets clamped to [0, T]) of x_perm [T,H] times weight[e] [F,H]^T.
hipError_t launch_grouped_linear(const void* x_perm, const void* weight, const int32_t* offsets,
                                 int64_t T, int H, int E, int F, bool bf16, void* y,
                                 hipStream_t s);

// Backward (backward.hip).
hipError_t launch_combine_backward(const void* dout, const void* y, const int32_t* inv,
                                   const float* w, int64_t N, int H, int K, bool bf16, void* dy,
                                   float* dw, hipStream_t s);
// Router backward workspace: gate_t [E][H] (dtype), partials
// [route_bwd_max_chunks][H] fp32, bias partials [route_bwd_max_chunks] fp32
// -- laid out by the caller from these sizes.
int64_t route_bwd_max_chunks(int64_t T, int E);
hipError_t launch_route_backward(const void* x_perm, const void* gate_w, const int32_t* ids,
                                 const float* w, const float* dw, const int32_t* perm,
                                 const int32_t* offsets, const int32_t* inv, const void* dx_perm,
                                 int64_t N, int H, int E, int K, bool bf16, float* dgate_w,
                                 float* dbias, void* dx, void* gate_t, float* part, float* part_b,
                                 hipStream_t s);

}  // namespace moe
