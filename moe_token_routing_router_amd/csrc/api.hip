// extern "C" entry points of libmoe.so (declared in include/moe.h).
// Every argument is checked on the host before anything is enqueued; the
// launchers in route.hip / dispatch.hip / combine.hip assume valid input.
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr int64_t kMaxSlots = (int64_t)1 << 31;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int elem_bytes(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

inline bool valid_dtype(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// H elements of dtype form a whole number of 16-byte vectors
inline bool row_ok(int32_t H, moe_dtype_t dt) {
  return ((int64_t)H * elem_bytes(dt)) % 16 == 0;
}

inline moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

// Built-in workspace of moe_route_dispatch_noalloc.  Every GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code this name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress (noalloc_scratch below), and only
// that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device (with the device current) and kept.
moe_status_t noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Argument checks of moe_route other than the workspace's.
moe_status_t check_route(const void* x, const void* gate_w, const float* bias, int64_t N,
                         int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                         const int32_t* topk_ids, const float* topk_w, const int32_t* counts) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || E <= 0 || K < 1 || K > E)
    return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!x || !gate_w || !topk_ids || !topk_w)) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts || K > moe::kMaxRouteK || N * (int64_t)K >= kMaxSlots ||
      !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(gate_w, 16) || !aligned(bias, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(counts, 4))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// The launches of moe_route for N > 0.  bf16: the gate is re-laid out into
// the workspace first unless the router reads gate_w as it is (64 experts)
// or gate_w already is that layout (prepacked).
moe_status_t launch_route(const void* x, const void* gate_w, const float* bias, int64_t N,
                          int32_t H, int32_t E, int32_t K, moe_dtype_t dtype, int32_t* topk_ids,
                          float* topk_w, int32_t* counts, void* workspace, bool prepacked,
                          hipStream_t s) {
  if (dtype == MOE_BF16) {
    const uint16_t* wgt = reinterpret_cast<const uint16_t*>(gate_w);
    hipError_t e = hipSuccess;
    if (moe::route_gate_raw(E) || prepacked) {
      if (counts) e = moe::launch_fill_i32(counts, E, 0, s);
    } else {
      uint16_t* packed = reinterpret_cast<uint16_t*>(workspace);
      e = moe::launch_gate_transpose(wgt, H, E, packed, counts, s);
      wgt = packed;
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    return from_hip(moe::launch_route_bf16(reinterpret_cast<const uint16_t*>(x), wgt, bias, N, H,
                                           E, K, topk_ids, topk_w, counts, nullptr, nullptr, s));
  }
  if (counts) {
    hipError_t e = moe::launch_fill_i32(counts, E, 0, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return from_hip(moe::launch_route_f32(reinterpret_cast<const float*>(x),
                                        reinterpret_cast<const float*>(gate_w), bias, N, H, E, K,
                                        topk_ids, topk_w, counts, nullptr, nullptr, s));
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or shape";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t moe_route_workspace_size(int32_t H, int32_t E, moe_dtype_t dtype) {
  if (dtype != MOE_BF16 || H <= 0 || E <= 0 || E > moe::kMaxExperts) return 0;
  if (moe::route_gate_raw(E)) return 0;  // the router reads gate_w itself
  return round_up((size_t)moe::route_padded_experts(E) * (size_t)moe::route_gate_rows(H) * 2, 256);
}

moe_status_t moe_route(const void* x, const void* gate_w, const float* bias, int64_t N, int32_t H,
                       int32_t E, int32_t K, moe_dtype_t dtype, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t st = check_route(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w, counts);
  if (st != MOE_OK) return st;
  if (!aligned(workspace, 16)) return MOE_ERR_MISALIGNED;
  const size_t need = moe_route_workspace_size(H, E, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return counts ? from_hip(moe::launch_fill_i32(counts, E, 0, s)) : MOE_OK;
  return launch_route(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w, counts, workspace,
                      false, s);
}

moe_status_t moe_route_pack_gate(const void* gate_w, int32_t H, int32_t E, moe_dtype_t dtype,
                                 void* packed, size_t packed_bytes, void* stream) {
  if (!valid_dtype(dtype) || H <= 0 || E <= 0 || !gate_w) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts || !row_ok(H, dtype)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_route_workspace_size(H, E, dtype);
  if (need == 0) return MOE_OK;  // the router reads gate_w as it is
  if (!packed) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(gate_w, 16) || !aligned(packed, 16)) return MOE_ERR_MISALIGNED;
  if (packed_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(moe::launch_gate_transpose(reinterpret_cast<const uint16_t*>(gate_w), H, E,
                                             reinterpret_cast<uint16_t*>(packed), nullptr,
                                             reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_prepacked(const void* x, const void* packed_gate, size_t packed_bytes,
                                 const float* bias, int64_t N, int32_t H, int32_t E, int32_t K,
                                 moe_dtype_t dtype, int32_t* topk_ids, float* topk_w,
                                 int32_t* counts, void* stream) {
  moe_status_t st =
      check_route(x, packed_gate, bias, N, H, E, K, dtype, topk_ids, topk_w, counts);
  if (st != MOE_OK) return st;
  if (packed_bytes < moe_route_workspace_size(H, E, dtype)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return counts ? from_hip(moe::launch_fill_i32(counts, E, 0, s)) : MOE_OK;
  return launch_route(x, packed_gate, bias, N, H, E, K, dtype, topk_ids, topk_w, counts, nullptr,
                      true, s);
}

namespace {

// Fused bf16 route+dispatch: up to this many router blocks (and K), the
// scatter sums the per-block counts and expert prefixes itself instead of
// running the scan kernel.
#ifndef MOE_PREFIX_MAX_BLOCKS
#define MOE_PREFIX_MAX_BLOCKS 512
#endif
constexpr int64_t kPrefixMaxBlocks = MOE_PREFIX_MAX_BLOCKS;
#ifndef MOE_PREFIX_MAX_K
#define MOE_PREFIX_MAX_K 4
#endif
constexpr int kPrefixMaxK = MOE_PREFIX_MAX_K;
// In the fused call the blocks are the router's (128 tokens at 65..128
// experts from 32768 tokens), so each slot sums half the block entries it
// would over the standalone dispatch's 64-token count blocks: there K up to
// 8 (at K = 8 the standalone dispatch is slower in this form).
#ifndef MOE_PREFIX_MAX_K_FUSED
#define MOE_PREFIX_MAX_K_FUSED 8
#endif
constexpr int kPrefixMaxKFused = MOE_PREFIX_MAX_K_FUSED;

// dispatch scratch: bhist [E][blocks of bt tokens] then lrank [N*K]
size_t bhist_bytes(int64_t N, int32_t E, int bt) {
  return round_up((size_t)moe::dispatch_num_blocks(N, bt) * (size_t)E * sizeof(int32_t), 256);
}

size_t dispatch_scratch_bytes(int64_t N, int32_t E, int32_t K, int bt) {
  return bhist_bytes(N, E, bt) + round_up((size_t)N * (size_t)K * sizeof(int32_t), 256);
}

moe_status_t check_dispatch_outputs(int64_t N, int32_t H, int32_t E, int32_t K,
                                    moe_dtype_t dtype, const void* x, const int32_t* counts,
                                    const int32_t* offsets, const int32_t* perm,
                                    const int32_t* inv, const void* x_perm) {
  if (!counts || !offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!perm || !inv)) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && x_perm && !x) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv, 4) ||
      !aligned(x, 16) || !aligned(x_perm, 16))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status_t zero_counts_offsets(int32_t* counts, int32_t* offsets, int32_t E, hipStream_t s) {
  hipError_t e = moe::launch_fill_i32(counts, E, 0, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return from_hip(moe::launch_fill_i32(offsets, (int64_t)E + 1, 0, s));
}

}  // namespace

size_t moe_dispatch_workspace_size(int64_t N, int32_t E, int32_t K) {
  if (N < 0 || E <= 0 || E > moe::kMaxExperts || K < 1) return 0;
  // block histograms, in-block ranks, the blocks' expert prefixes
  const int bt = moe::dispatch_count_tokens(K);
  return dispatch_scratch_bytes(N, E, K, bt) + bhist_bytes(N, E, bt);
}

moe_status_t moe_dispatch(const int32_t* topk_ids, const void* x, int64_t N, int32_t H, int32_t E,
                          int32_t K, moe_dtype_t dtype, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, void* x_perm, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || E <= 0 || K < 1 || K > E)
    return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!topk_ids || !workspace)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_dispatch_outputs(N, H, E, K, dtype, x, counts, offsets, perm, inv, x_perm);
  if (st != MOE_OK) return st;
  if (!aligned(topk_ids, 4) || !aligned(workspace, 16)) return MOE_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return zero_counts_offsets(counts, offsets, E, s);
  if (workspace_bytes < moe_dispatch_workspace_size(N, E, K)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const int bt = moe::dispatch_count_tokens(K);
  int32_t* bhist = reinterpret_cast<int32_t*>(workspace);
  int32_t* lrank = reinterpret_cast<int32_t*>(
      reinterpret_cast<char*>(workspace) +
      round_up((size_t)moe::dispatch_num_blocks(N, bt) * E * sizeof(int32_t), 256));
  // the usual caller has just run the bf16 router over x: scatter in its
  // XCD order
  const int router_bt = dtype == MOE_BF16 ? moe::route_tokens_per_block(E, N) : 0;
  const int64_t row_bytes = (int64_t)H * elem_bytes(dtype);
  const int64_t nb = moe::dispatch_num_blocks(N, bt);
  if (moe::dispatch_needs_scan(nb, E) && nb <= kPrefixMaxBlocks && K <= kPrefixMaxK) {
    // instead of the scan kernel: the count kernel also stores each block's
    // prefix over the experts and the scatter sums what its slots need
    int32_t* bpre = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) +
                                               dispatch_scratch_bytes(N, E, K, bt));
    hipError_t e = moe::launch_dispatch_count(topk_ids, N, E, K, lrank, bhist, s, bpre);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return from_hip(moe::launch_dispatch_scatter_blockpre(topk_ids, x, N, row_bytes, E, K, bt,
                                                          counts, offsets, perm, inv, x_perm,
                                                          lrank, bhist, bpre, s, router_bt));
  }
  hipError_t e = moe::launch_dispatch_count(topk_ids, N, E, K, lrank, bhist, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return from_hip(moe::launch_dispatch_finish(topk_ids, x, N, row_bytes, E, K, bt, counts,
                                              offsets, perm, inv, x_perm, lrank, bhist, s,
                                              router_bt));
}

size_t moe_route_dispatch_workspace_size(int64_t N, int32_t H, int32_t E, int32_t K,
                                         moe_dtype_t dtype) {
  if (N < 0 || H <= 0 || E <= 0 || E > moe::kMaxExperts || K < 1 || !valid_dtype(dtype)) return 0;
  const int bt =
      dtype == MOE_BF16 ? moe::route_tokens_per_block(E, N) : moe::kRouteF32Tokens;
  // packed gate (if any), block histograms, in-block ranks, then (bf16) the
  // blocks' expert prefixes
  return moe_route_workspace_size(H, E, dtype) + dispatch_scratch_bytes(N, E, K, bt) +
         (dtype == MOE_BF16 ? bhist_bytes(N, E, bt) : 0);
}

namespace {

// Argument checks of moe_route_dispatch other than the workspace's.
moe_status_t check_route_dispatch(const void* x, const void* gate_w, const float* bias, int64_t N,
                                  int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                  const int32_t* topk_ids, const float* topk_w,
                                  const int32_t* counts, const int32_t* offsets,
                                  const int32_t* perm, const int32_t* inv, const void* x_perm) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || E <= 0 || K < 1 || K > E)
    return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!x || !gate_w || !topk_ids || !topk_w)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_dispatch_outputs(N, H, E, K, dtype, x, counts, offsets, perm, inv, x_perm);
  if (st != MOE_OK) return st;
  if (K > moe::kMaxRouteK) return MOE_ERR_UNSUPPORTED;
  if (!aligned(gate_w, 16) || !aligned(bias, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// The launches of moe_route_dispatch for N > 0 on a checked workspace.
moe_status_t launch_route_dispatch(const void* x, const void* gate_w, const float* bias, int64_t N,
                                   int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                   int32_t* topk_ids, float* topk_w, int32_t* counts,
                                   int32_t* offsets, int32_t* perm, int32_t* inv, void* x_perm,
                                   void* workspace, hipStream_t s, bool prepacked = false) {
  const size_t rws = moe_route_workspace_size(H, E, dtype);
  const int bt =
      dtype == MOE_BF16 ? moe::route_tokens_per_block(E, N) : moe::kRouteF32Tokens;
  char* base = reinterpret_cast<char*>(workspace);
  int32_t* bhist = reinterpret_cast<int32_t*>(base + rws);
  int32_t* lrank = reinterpret_cast<int32_t*>(
      base + rws + round_up((size_t)moe::dispatch_num_blocks(N, bt) * E * sizeof(int32_t), 256));
  hipError_t e;
  if (dtype == MOE_BF16) {
    // Few blocks (K <= 8): the router stores each block's histogram and its
    // exclusive prefix over the experts, and each scatter workgroup finds its
    // slots' positions itself, so neither a ranking pass, a scan kernel nor
    // zeroed counts are needed.  Otherwise the router ranks its picks and the
    // scan kernel runs.
    const bool prefix =
        moe::dispatch_num_blocks(N, bt) <= kPrefixMaxBlocks && K <= kPrefixMaxKFused;
    int32_t* bpre = reinterpret_cast<int32_t*>(
        base + rws + dispatch_scratch_bytes(N, E, K, bt));
    const uint16_t* wgt = reinterpret_cast<const uint16_t*>(gate_w);
    if (!moe::route_gate_raw(E) && !prepacked) {
      uint16_t* packed = reinterpret_cast<uint16_t*>(workspace);
      e = moe::launch_gate_transpose(wgt, H, E, packed, nullptr, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
      wgt = packed;
    }
    e = moe::launch_route_bf16(reinterpret_cast<const uint16_t*>(x), wgt, bias, N, H, E, K,
                               topk_ids, topk_w, nullptr, lrank, bhist, s,
                               prefix ? bpre : nullptr);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (prefix)
      return from_hip(moe::launch_dispatch_scatter_blockpre(
          topk_ids, x, N, (int64_t)H * elem_bytes(dtype), E, K, bt, counts, offsets, perm, inv,
          x_perm, lrank, bhist, bpre, s));
  } else {
    // the fp32 router ranks its own 16-token blocks: no count kernel
    e = moe::launch_route_f32(reinterpret_cast<const float*>(x),
                              reinterpret_cast<const float*>(gate_w), bias, N, H, E, K, topk_ids,
                              topk_w, nullptr, lrank, bhist, s);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  return from_hip(moe::launch_dispatch_finish(topk_ids, x, N, (int64_t)H * elem_bytes(dtype), E, K,
                                              bt, counts, offsets, perm, inv, x_perm, lrank,
                                              bhist, s, dtype == MOE_BF16 ? bt : 0));
}

}  // namespace

moe_status_t moe_route_dispatch(const void* x, const void* gate_w, const float* bias, int64_t N,
                                int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                int32_t* topk_ids, float* topk_w, int32_t* counts,
                                int32_t* offsets, int32_t* perm, int32_t* inv, void* x_perm,
                                void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t st = check_route_dispatch(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w,
                                         counts, offsets, perm, inv, x_perm);
  if (st != MOE_OK) return st;
  if (N > 0 && !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 16)) return MOE_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return zero_counts_offsets(counts, offsets, E, s);
  if (workspace_bytes < moe_route_dispatch_workspace_size(N, H, E, K, dtype))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return launch_route_dispatch(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w, counts,
                               offsets, perm, inv, x_perm, workspace, s);
}

moe_status_t moe_route_dispatch_prepacked(const void* x, const void* packed_gate,
                                          size_t packed_bytes, const float* bias, int64_t N,
                                          int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                          int32_t* topk_ids, float* topk_w, int32_t* counts,
                                          int32_t* offsets, int32_t* perm, int32_t* inv,
                                          void* x_perm, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  moe_status_t st = check_route_dispatch(x, packed_gate, bias, N, H, E, K, dtype, topk_ids,
                                         topk_w, counts, offsets, perm, inv, x_perm);
  if (st != MOE_OK) return st;
  if (packed_bytes < moe_route_workspace_size(H, E, dtype)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (N > 0 && !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 16)) return MOE_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return zero_counts_offsets(counts, offsets, E, s);
  if (workspace_bytes < moe_route_dispatch_workspace_size(N, H, E, K, dtype))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return launch_route_dispatch(x, packed_gate, bias, N, H, E, K, dtype, topk_ids, topk_w, counts,
                               offsets, perm, inv, x_perm, workspace, s, true);
}

moe_status_t moe_route_dispatch_noalloc(const void* x, const void* gate_w, const float* bias,
                                        int64_t N, int32_t H, int32_t E, int32_t K,
                                        moe_dtype_t dtype, int32_t* topk_ids, float* topk_w,
                                        int32_t* counts, int32_t* offsets, int32_t* perm,
                                        int32_t* inv, void* x_perm, void* stream) {
  moe_status_t st = check_route_dispatch(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w,
                                         counts, offsets, perm, inv, x_perm);
  if (st != MOE_OK) return st;
  if (moe_route_dispatch_workspace_size(N, H, E, K, dtype) > MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return zero_counts_offsets(counts, offsets, E, s);
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MOE_OK) return st;
  // every byte of the workspace the kernels read is written earlier in the
  // same call (packed gate, block histograms, in-block ranks), so nothing
  // left by an earlier call needs clearing
  return launch_route_dispatch(x, gate_w, bias, N, H, E, K, dtype, topk_ids, topk_w, counts,
                               offsets, perm, inv, x_perm, ws, s);
}

size_t moe_ep_dispatch_workspace_size(int64_t N, int32_t E, int32_t K, int32_t ep_size) {
  if (N < 0 || E <= 0 || E > moe::kMaxExperts || K < 1 || ep_size < 1 || E % ep_size != 0)
    return 0;
  // block histograms of both levels [E + R][blocks], then the slots' ranks
  // among equal experts and among equal rank keys [N*K] each
  return bhist_bytes(N, E + ep_size, moe::dispatch_count_tokens(K)) +
         2 * round_up((size_t)N * (size_t)K * sizeof(int32_t), 256);
}

moe_status_t moe_ep_dispatch(const int32_t* topk_ids, const void* x, int64_t N, int32_t H,
                             int32_t E, int32_t K, int32_t ep_size, moe_dtype_t dtype,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                             int32_t* send_counts, int32_t* send_offsets, int32_t* send_tok,
                             int32_t* send_row, int32_t* expand_idx, void* x_send,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || E <= 0 || K < 1 || K > E || ep_size < 1 ||
      E % ep_size != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!topk_ids || !workspace)) return MOE_ERR_INVALID_ARGUMENT;
  if (!send_counts || !send_offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!send_tok || !send_row || !expand_idx)) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && x_send && !x) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_dispatch_outputs(N, H, E, K, dtype, x, counts, offsets, perm, inv,
                                           nullptr);
  if (st != MOE_OK) return st;
  if (!aligned(topk_ids, 4) || !aligned(send_counts, 4) || !aligned(send_offsets, 4) ||
      !aligned(send_tok, 4) || !aligned(send_row, 4) || !aligned(expand_idx, 4) ||
      !aligned(x_send, 16) || !aligned(workspace, 16))
    return MOE_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) {
    st = zero_counts_offsets(counts, offsets, E, s);
    if (st != MOE_OK) return st;
    return zero_counts_offsets(send_counts, send_offsets, ep_size, s);
  }
  if (workspace_bytes < moe_ep_dispatch_workspace_size(N, E, K, ep_size))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const int64_t T = N * K;
  char* base = reinterpret_cast<char*>(workspace);
  const size_t hb = bhist_bytes(N, E + ep_size, moe::dispatch_count_tokens(K));
  int32_t* bhist = reinterpret_cast<int32_t*>(base);
  int32_t* lrank_e = reinterpret_cast<int32_t*>(base + hb);
  int32_t* lrank_r =
      reinterpret_cast<int32_t*>(base + hb + round_up((size_t)T * sizeof(int32_t), 256));
  return from_hip(moe::launch_ep_dispatch(
      topk_ids, x, N, (int64_t)H * elem_bytes(dtype), E, K, ep_size, counts, offsets, perm, inv,
      send_counts, send_offsets, send_tok, send_row, expand_idx, x_send, bhist, lrank_e, lrank_r,
      s));
}

moe_status_t moe_combine(const void* y, const int32_t* inv, const float* topk_w, int64_t N,
                         int32_t H, int32_t K, moe_dtype_t dtype, void* out, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!y || !inv || !topk_w || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (K > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(inv, 4) || !aligned(topk_w, 4))
    return MOE_ERR_MISALIGNED;
  if (N == 0) return MOE_OK;
  return from_hip(moe::launch_combine(y, inv, topk_w, N, H, K, dtype == MOE_BF16, out,
                                      reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_aggregate(const void* y, const int32_t* inv, const float* topk_w,
                           const void* residual, int64_t N, int32_t H, int32_t K,
                           moe_dtype_t dtype, void* out, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!y || !inv || !topk_w || !residual || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (K > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(residual, 16) || !aligned(inv, 4) ||
      !aligned(topk_w, 4))
    return MOE_ERR_MISALIGNED;
  if (N == 0) return MOE_OK;
  return from_hip(moe::launch_combine(y, inv, topk_w, N, H, K, dtype == MOE_BF16, out,
                                      reinterpret_cast<hipStream_t>(stream), residual));
}

moe_status_t moe_grouped_linear(const void* x_perm, const void* weight, const int32_t* offsets,
                                int64_t T, int32_t H, int32_t E, int32_t F, moe_dtype_t dtype,
                                void* y, void* stream) {
  if (!valid_dtype(dtype) || T < 0 || H <= 0 || E <= 0 || F <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!offsets || (T > 0 && (!x_perm || !weight || !y))) return MOE_ERR_INVALID_ARGUMENT;
  // one expert's weights and one 256-row tile of x_perm are indexed with
  // 32-bit offsets
  if (E > moe::kMaxExperts || T >= kMaxSlots || !row_ok(H, dtype) || !row_ok(F, dtype) ||
      (int64_t)F * H >= kMaxSlots || 256LL * H >= kMaxSlots)
    return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_F32 && (T * (int64_t)F + 255) / 256 >= kMaxSlots) return MOE_ERR_UNSUPPORTED;
  if (!aligned(x_perm, 16) || !aligned(weight, 16) || !aligned(y, 16) || !aligned(offsets, 4))
    return MOE_ERR_MISALIGNED;
  if (T == 0) return MOE_OK;
  return from_hip(moe::launch_grouped_linear(x_perm, weight, offsets, T, H, E, F,
                                             dtype == MOE_BF16, y,
                                             reinterpret_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- backward

moe_status_t moe_combine_backward(const void* dout, const void* y, const int32_t* inv,
                                  const float* topk_w, int64_t N, int32_t H, int32_t K,
                                  moe_dtype_t dtype, void* dy, float* dtopk_w, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!dout || !y || !inv || !topk_w || !dy || !dtopk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  if (K > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(dout, 16) || !aligned(y, 16) || !aligned(dy, 16) || !aligned(inv, 4) ||
      !aligned(topk_w, 4) || !aligned(dtopk_w, 4))
    return MOE_ERR_MISALIGNED;
  if (N == 0) return MOE_OK;
  return from_hip(moe::launch_combine_backward(dout, y, inv, topk_w, N, H, K, dtype == MOE_BF16,
                                               dy, dtopk_w,
                                               reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_backward(const void* dx_perm, const int32_t* inv, int64_t N, int32_t H,
                                   int32_t K, moe_dtype_t dtype, void* dx, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!dx_perm || !inv || !dx)) return MOE_ERR_INVALID_ARGUMENT;
  if (K > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(dx_perm, 16) || !aligned(dx, 16) || !aligned(inv, 4)) return MOE_ERR_MISALIGNED;
  if (N == 0) return MOE_OK;
  return from_hip(moe::launch_combine(dx_perm, inv, nullptr, N, H, K, dtype == MOE_BF16, dx,
                                      reinterpret_cast<hipStream_t>(stream)));
}

namespace {

struct RouteBwdLayout {
  size_t gate_t, part, part_b, total;
};

RouteBwdLayout route_bwd_layout(int64_t N, int32_t H, int32_t E, int32_t K, moe_dtype_t dtype) {
  const int64_t T = N * K;
  const int64_t chunks = moe::route_bwd_max_chunks(T, E);
  RouteBwdLayout l;
  l.gate_t = 0;
  l.part = l.gate_t + round_up((size_t)E * (size_t)H * elem_bytes(dtype), 256);
  l.part_b = l.part + round_up((size_t)chunks * (size_t)H * sizeof(float), 256);
  l.total = l.part_b + round_up((size_t)chunks * sizeof(float), 256);
  return l;
}

}  // namespace

size_t moe_route_backward_workspace_size(int64_t N, int32_t H, int32_t E, int32_t K,
                                         moe_dtype_t dtype) {
  if (N < 0 || H <= 0 || E <= 0 || E > moe::kMaxExperts || K < 1 || K > E || !valid_dtype(dtype) ||
      N * (int64_t)K >= kMaxSlots)
    return 0;
  return route_bwd_layout(N, H, E, K, dtype).total;
}

moe_status_t moe_route_backward(const void* x_perm, const void* gate_w, const int32_t* topk_ids,
                                const float* topk_w, const float* dtopk_w, const int32_t* perm,
                                const int32_t* offsets, const int32_t* inv, const void* dx_perm,
                                int64_t N, int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                float* dgate_w, float* dbias, void* dx, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || N < 0 || H <= 0 || E <= 0 || K < 1 || K > E)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!gate_w || !dgate_w) return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!x_perm || !topk_ids || !topk_w || !dtopk_w || !perm || !offsets || !dx ||
                !workspace))
    return MOE_ERR_INVALID_ARGUMENT;
  if (N > 0 && dx_perm && !inv) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts || N * (int64_t)K >= kMaxSlots || !row_ok(H, dtype))
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(x_perm, 16) || !aligned(gate_w, 16) || !aligned(dx_perm, 16) || !aligned(dx, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(dtopk_w, 4) || !aligned(perm, 4) ||
      !aligned(offsets, 4) || !aligned(inv, 4) || !aligned(dgate_w, 4) || !aligned(dbias, 4) ||
      !aligned(workspace, 16))
    return MOE_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) {
    // no tokens: the gate and bias gradients are zero
    hipError_t e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(dgate_w), (int64_t)H * E, 0, s);
    if (e != hipSuccess || !dbias) return from_hip(e);
    return from_hip(moe::launch_fill_i32(reinterpret_cast<int32_t*>(dbias), E, 0, s));
  }
  const RouteBwdLayout l = route_bwd_layout(N, H, E, K, dtype);
  if (workspace_bytes < l.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  char* base = reinterpret_cast<char*>(workspace);
  return from_hip(moe::launch_route_backward(
      x_perm, gate_w, topk_ids, topk_w, dtopk_w, perm, offsets, inv, dx_perm, N, H, E, K,
      dtype == MOE_BF16, dgate_w, dbias, dx, base + l.gate_t,
      reinterpret_cast<float*>(base + l.part), reinterpret_cast<float*>(base + l.part_b), s));
}

}  // extern "C"
