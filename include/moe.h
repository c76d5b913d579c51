/*
 * moe.h -- C ABI of libmoe.so, the MI355X (gfx950) MoE routing path:
 * route -> counting-sort dispatch -> weighted combine, on one GPU.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *    The library never allocates, frees or synchronises; it only enqueues
 *    kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream) and returns.  Outputs are valid once that stream reaches them.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and a status code is returned.  No entry point
 *    aborts or throws.
 *  - Results are bitwise reproducible run to run (integer atomics only, every
 *    floating-point sum in a fixed order).
 *  - Sizes: N tokens, H hidden size, E experts, K experts per token,
 *    T = N*K routed slots; slot i = n*K + k.
 *  - Limits (MOE_ERR_UNSUPPORTED otherwise): E <= 256, T < 2^31, a row of H
 *    elements is a multiple of 16 bytes (H % 8 == 0 for bf16, H % 4 == 0 for
 *    fp32); moe_route additionally needs K <= 16.
 *  - Alignment (MOE_ERR_MISALIGNED otherwise): x, gate_w, x_perm, y, out and
 *    the workspaces on 16 bytes; integer and fp32 side arrays on 4 bytes.
 *
 * Pages cited (by title and section):
 *  [R] "moe-engine: sparse MoE training infrastructure for 10k-GPU clusters",
 *      section "Fused Triton routing kernel" (核心组件深度解析 › 融合Triton路由内核)
 *      and section "Token conservation check" (Token守恒验证).
 *  [D] "Building a MoE training stack in 10k lines of Python", section 8.2
 *      "O(n) counting sort instead of O(n log n) argsort" (8.2 O(n) counting
 *      sort 替代 O(n log n) argsort).
 *  [A] same page, section 6.1 "Model protocol first" (6.1 模型协议先行),
 *      forward_aggregate.
 *  [P] same page, section 8.2, fused_dedup_prepare_dispatch: per-expert and
 *      per-rank counts, prefix sums and send metadata, deduplicated scatter
 *      with a counting sort and the receivers' expand index.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the two enums get int as their fixed underlying type, so any int a C
 * caller passes (e.g. an unknown status code) is a valid value of the type
 * rather than undefined behaviour; in C an enum is an int anyway. */
#ifdef __cplusplus
#define MOE_ENUM_BASE : int
#else
#define MOE_ENUM_BASE
#endif

typedef enum MOE_ENUM_BASE {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* NULL required pointer, bad size, K > E */
  MOE_ERR_UNSUPPORTED = 2,        /* outside the limits listed above */
  MOE_ERR_MISALIGNED = 3,         /* pointer not aligned as listed above */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4,/* workspace_bytes below the *_workspace_size */
  MOE_ERR_HIP = 5                 /* a kernel launch reported an error */
} moe_status_t;

typedef enum MOE_ENUM_BASE { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char *moe_status_string(moe_status_t status);

/*
 * Bytes of device workspace moe_route needs for (H, E, dtype); 0 if none.
 * (bf16: the gate matrix re-laid out in MFMA fragment order, padded to a
 * power-of-two multiple of 16 experts; none at exactly 64 experts, where the
 * router reads gate_w as it is.)
 */
size_t moe_route_workspace_size(int32_t H, int32_t E, moe_dtype_t dtype);

/*
 * moe_route -- the fused router of [R]: for each token
 *   logits[n,e] = sum_h x[n,h] * gate_w[h,e] + bias[e]
 *   ids[n,0..K-1] = the K experts of largest logit, in descending logit
 *                   order (equal logits: lower expert index first)
 *   w[n,k] = softmax over all E experts, restricted to the K chosen ones and
 *            renormalised to sum 1 (equal to the softmax over the K chosen
 *            logits)
 * in one pass over x.  The logits never leave the chip.
 *
 *   x        [N,H]  dtype    tokens
 *   gate_w   [H,E]  dtype    gate matrix (tokens @ gate_w)
 *   bias     [E]    fp32     per-expert logit bias, or NULL for none
 *   topk_ids [N,K]  int32    out
 *   topk_w   [N,K]  fp32     out
 *   counts   [E]    int32    out, optional (NULL to skip): tokens routed to
 *                            each expert (the dispatch count of [R]'s token
 *                            conservation check); overwritten, not added to
 *   workspace >= moe_route_workspace_size(H, E, dtype) bytes (may be NULL
 *            when that size is 0); contents are scratch
 * bf16 inputs are multiplied exactly and accumulated in fp32; fp32 inputs
 * use fp32 fused multiply-adds.  N == 0 is a valid no-op (counts zeroed).
 */
moe_status_t moe_route(const void *x, const void *gate_w, const float *bias,
                       int64_t N, int32_t H, int32_t E, int32_t K,
                       moe_dtype_t dtype, int32_t *topk_ids, float *topk_w,
                       int32_t *counts, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * moe_route_pack_gate -- the gate re-laid out once, for callers whose gate
 * does not change between router calls (inference; or a training step that
 * packs it once after each weight update, off the path of the forward
 * pass): the layout moe_route builds in its workspace on every call (bf16:
 * MFMA fragment order, padded to a power-of-two multiple of 16 experts).
 * moe_route_prepacked and moe_route_dispatch_prepacked take it instead of
 * gate_w and skip that re-layout (one kernel launch; about 4.5 us of the
 * router call at N = 32768, H = 2048, E = 128 and 6 us at N = 16384,
 * H = 4096, E = 128 on MI355X).
 *   gate_w [H,E] dtype; packed: moe_route_workspace_size(H, E, dtype) bytes,
 *   out, 16-byte aligned.  When that size is 0 (fp32, or bf16 at exactly 64
 *   experts, where the router reads gate_w as it is) nothing is written and
 *   the packed gate of the prepacked calls is gate_w itself.
 * The packed bytes depend on gate_w only; the caller owns them and repacks
 * after changing gate_w.
 */
moe_status_t moe_route_pack_gate(const void *gate_w, int32_t H, int32_t E, moe_dtype_t dtype,
                                 void *packed, size_t packed_bytes, void *stream);

/*
 * moe_route_prepacked -- moe_route with packed_gate = moe_route_pack_gate's
 * output for (gate_w, H, E, dtype) (gate_w itself when that size is 0) in
 * place of gate_w, and no workspace.  packed_bytes is the size of the
 * packed_gate buffer: MOE_ERR_WORKSPACE_TOO_SMALL when it is below
 * moe_route_workspace_size(H, E, dtype) (not checked when that size is 0).
 * Outputs, limits and status codes are otherwise those of moe_route, bit
 * for bit.  Packed bytes that are not moe_route_pack_gate's output for this
 * gate give wrong results, never an access outside the buffer.
 */
moe_status_t moe_route_prepacked(const void *x, const void *packed_gate, size_t packed_bytes,
                                 const float *bias, int64_t N, int32_t H, int32_t E, int32_t K,
                                 moe_dtype_t dtype, int32_t *topk_ids, float *topk_w,
                                 int32_t *counts, void *stream);

/*
 * Bytes of device workspace moe_dispatch needs for (N, E, K).
 */
size_t moe_dispatch_workspace_size(int64_t N, int32_t E, int32_t K);

/*
 * moe_dispatch -- the counting-sort dispatch of [D]: replaces an argsort of
 * the T expert ids by a histogram, an exclusive prefix sum and a stable
 * scatter, then copies token rows into expert-contiguous order.
 *   counts[e]   = #{i : ids[i] == e}                         (sum = N*K)
 *   offsets[e]  = sum_{e' < e} counts[e'],  offsets[E] = N*K
 *   inv[i]      = offsets[ids[i]] + #{j < i : ids[j] == ids[i]}
 *   perm[inv[i]] = i          (row -> slot; token = slot / K, k = slot % K)
 *   x_perm[inv[i], :] = x[i / K, :]   (bit copy)
 * No capacity limit: every slot is dispatched.  Inside an expert's segment
 * rows are in ascending slot order (stable).
 *
 *   topk_ids [N,K]   int32  expert ids; PRECONDITION 0 <= id < E and the K
 *                           ids of a token distinct (not checked)
 *   x        [N,H]   dtype  token rows (may be NULL iff x_perm is NULL)
 *   counts   [E]     int32  out
 *   offsets  [E+1]   int32  out
 *   perm     [N*K]   int32  out
 *   inv      [N*K]   int32  out
 *   x_perm   [N*K,H] dtype  out, or NULL to produce only the index arrays
 *   workspace >= moe_dispatch_workspace_size(N, E, K) bytes; scratch
 * N == 0 is a valid call: counts and offsets are zero-filled.
 */
moe_status_t moe_dispatch(const int32_t *topk_ids, const void *x, int64_t N,
                          int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                          int32_t *counts, int32_t *offsets, int32_t *perm,
                          int32_t *inv, void *x_perm, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace moe_route_dispatch needs for (N, H, E, K, dtype).
 */
size_t moe_route_dispatch_workspace_size(int64_t N, int32_t H, int32_t E, int32_t K,
                                         moe_dtype_t dtype);

/*
 * moe_route_dispatch -- moe_route followed by moe_dispatch of its ids, in
 * fewer launches: the router's own epilogue produces the per-block counts
 * and the stable in-block ranks the dispatch needs ([R]'s fused router feeds
 * [D]'s counting sort directly; the per-expert dispatch counts of [R]'s token
 * conservation check are `counts`).  Outputs are exactly those of the two
 * calls made in sequence (moe_route without its counts, then moe_dispatch):
 * topk_ids, topk_w [N,K]; counts [E]; offsets [E+1]; perm, inv [N*K];
 * x_perm [N*K,H] (or NULL for the index arrays only).  Limits and
 * preconditions are the union of the two calls' (notably K <= 16).
 *   workspace >= moe_route_dispatch_workspace_size(N, H, E, K, dtype) bytes;
 *              scratch
 * N == 0 is a valid call: counts and offsets are zero-filled.
 */
moe_status_t moe_route_dispatch(const void *x, const void *gate_w, const float *bias,
                                int64_t N, int32_t H, int32_t E, int32_t K,
                                moe_dtype_t dtype, int32_t *topk_ids, float *topk_w,
                                int32_t *counts, int32_t *offsets, int32_t *perm,
                                int32_t *inv, void *x_perm, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * moe_route_dispatch_prepacked -- moe_route_dispatch with the packed gate of
 * moe_route_pack_gate in place of gate_w (gate_w itself when the packed size
 * is 0; packed_bytes as for moe_route_prepacked).  Workspace as for
 * moe_route_dispatch (its packed-gate part is not used); outputs bit for bit
 * those of moe_route_dispatch.
 */
moe_status_t moe_route_dispatch_prepacked(const void *x, const void *packed_gate,
                                          size_t packed_bytes,
                                          const float *bias, int64_t N, int32_t H, int32_t E,
                                          int32_t K, moe_dtype_t dtype, int32_t *topk_ids,
                                          float *topk_w, int32_t *counts, int32_t *offsets,
                                          int32_t *perm, int32_t *inv, void *x_perm,
                                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of the built-in workspace of moe_route_dispatch_noalloc (one copy per
 * GPU, held by the library until the process ends).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * moe_route_dispatch_noalloc -- for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_route_dispatch with its
 * workspace taken from a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES
 * instead of a caller buffer.  Arguments, outputs, limits and status codes
 * are those of moe_route_dispatch without workspace/workspace_bytes; the
 * outputs are bit for bit those of moe_route_dispatch.
 *  - MOE_ERR_WORKSPACE_TOO_SMALL when moe_route_dispatch_workspace_size(N, H,
 *    E, K, dtype) exceeds MOE_NOALLOC_SCRATCH_BYTES (e.g. N = 16384, H = 4096,
 *    E = 64, K = 2 needs 0.7 MiB; N = 32768, H = 2048, E = 128, K = 8 needs
 *    1.8 MiB).
 *  - The device is the calling thread's current HIP device; `stream` must
 *    belong to it.  The first call on a device looks up that device's copy of
 *    the array (hipGetSymbolAddress, no allocation); MOE_ERR_HIP if that fails.
 *  - No hipMalloc, hipFree or memset is made, here or in any later call.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap
 *    on one GPU (different streams, or threads without ordering) RACE and
 *    must be serialised by the caller.  Nothing in the array needs clearing
 *    between calls (each call writes every byte it reads first).
 */
moe_status_t moe_route_dispatch_noalloc(const void *x, const void *gate_w, const float *bias,
                                        int64_t N, int32_t H, int32_t E, int32_t K,
                                        moe_dtype_t dtype, int32_t *topk_ids, float *topk_w,
                                        int32_t *counts, int32_t *offsets, int32_t *perm,
                                        int32_t *inv, void *x_perm, void *stream);

/*
 * Bytes of device workspace moe_ep_dispatch needs (0 for invalid sizes).
 */
size_t moe_ep_dispatch_workspace_size(int64_t N, int32_t E, int32_t K, int32_t ep_size);

/*
 * moe_ep_dispatch -- the expert-parallel send metadata of [P] on one GPU,
 * with ep_size = R ranks of E/R consecutive experts (expert e lives on rank
 * e / (E/R)) simulated as segments of one send buffer.  A token is sent once
 * to each distinct rank among its K experts; the send buffer is rank-major,
 * tokens ascending inside a rank.
 *   counts, offsets, perm, inv     exactly as moe_dispatch (expert level)
 *   send_counts [R]     int32 out  tokens sent to rank r (deduplicated)
 *   send_offsets [R+1]  int32 out  exclusive prefix sums; S = send_offsets[R]
 *   send_tok [N*min(K,R)] int32 out  token of send row j (j < S; the rest is
 *                                  not written)
 *   send_row [N*K]      int32 out  send row of token i/K for the rank of
 *                                  ids[i] (slots sharing a rank share it)
 *   expand_idx [N*K]    int32 out  for dispatched row p (expert-contiguous
 *                                  order): the row of the receiving rank's
 *                                  segment holding its token, counted from
 *                                  send_offsets[rank];  so
 *                                  x_perm[p] = x_send[send_offsets[r] + expand_idx[p]]
 *   x_send [N*min(K,R), H] dtype out, or NULL: x_send[j] = x[send_tok[j]]
 *   workspace >= moe_ep_dispatch_workspace_size(N, E, K, ep_size); scratch
 * INVALID_ARGUMENT also when ep_size < 1 or E % ep_size != 0.  Preconditions
 * and the treatment of ids outside [0,E) are those of moe_dispatch (such a
 * slot gets send_row = -1; expand_idx rows past offsets[E] are -1).
 * N == 0 is a valid call: the counts and offsets are zero-filled.
 */
moe_status_t moe_ep_dispatch(const int32_t *topk_ids, const void *x, int64_t N, int32_t H,
                             int32_t E, int32_t K, int32_t ep_size, moe_dtype_t dtype,
                             int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                             int32_t *send_counts, int32_t *send_offsets, int32_t *send_tok,
                             int32_t *send_row, int32_t *expand_idx, void *x_send,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_combine -- the weighted combine of [A] (forward_aggregate without the
 * residual): un-permutes the expert outputs and sums them per token
 *   out[n,:] = sum_{k=0..K-1} topk_w[n,k] * y[inv[n*K+k], :]
 * accumulated in fp32 with k ascending from 0, rounded once to dtype
 * (bf16: nearest, ties to even).
 *
 *   y      [N*K,H] dtype  expert outputs in dispatched (expert-contiguous) order
 *   inv    [N*K]   int32  slot -> row, as produced by moe_dispatch;
 *                         PRECONDITION 0 <= inv[i] < N*K (not checked)
 *   topk_w [N,K]   fp32   gate weights
 *   out    [N,H]   dtype  out
 * N == 0 is a valid no-op.
 */
moe_status_t moe_combine(const void *y, const int32_t *inv, const float *topk_w,
                         int64_t N, int32_t H, int32_t K, moe_dtype_t dtype,
                         void *out, void *stream);

/*
 * moe_aggregate -- forward_aggregate of [A]: the weighted expert output plus
 * the residual connection
 *   out[n,:] = sum_{k=0..K-1} topk_w[n,k] * y[inv[n*K+k], :]  +  residual[n,:]
 * accumulated in fp32 (k ascending from 0, then the residual), rounded once
 * to dtype.  Arguments as moe_combine; residual [N,H] dtype (may alias out).
 */
moe_status_t moe_aggregate(const void *y, const int32_t *inv, const float *topk_w,
                           const void *residual, int64_t N, int32_t H, int32_t K,
                           moe_dtype_t dtype, void *out, void *stream);

/*
 * moe_grouped_linear -- the expert layer between dispatch and combine ([A]
 * section 6.1, forward_mlp on the gathered tokens; the MoE GroupLinear of the
 * same page), one linear map per expert over its contiguous segment of the
 * dispatched rows:
 *   y[p, f] = sum_h x_perm[p, h] * weight[e][f][h]   for offsets[e] <= p < offsets[e+1]
 * bf16: products exact, fp32 accumulation on the matrix cores, one rounding;
 * fp32: fp32 FMAs with h ascending.
 *   x_perm [T,H] dtype   dispatched rows (moe_dispatch's x_perm)
 *   weight [E,F,H] dtype row f of expert e holds the weights of output f
 *   offsets [E+1] int32  moe_dispatch's offsets (PRECONDITION 0 = offsets[0]
 *                        <= ... <= offsets[E] <= T; values are clamped to
 *                        [0, T], so inconsistent offsets give wrong rows but
 *                        never an access outside the buffers)
 *   y [T,F] dtype        out; rows p >= offsets[E] are not written
 * F must make a row a multiple of 16 bytes, like H; F*H < 2^31 (one
 * expert's weights) and H < 2^23 (UNSUPPORTED otherwise).
 */
moe_status_t moe_grouped_linear(const void *x_perm, const void *weight, const int32_t *offsets,
                                int64_t T, int32_t H, int32_t E, int32_t F, moe_dtype_t dtype,
                                void *y, void *stream);

/* ---------------------------------------------------------------- backward
 * Training runs the path's stages backward ([A], section 6.2 "The five
 * stages").  Each call below is the exact gradient of the forward call named
 * in it, with the same layouts; floating-point sums run in fp32 in a fixed
 * order (bitwise reproducible), results are rounded once to their type.
 */

/*
 * moe_combine_backward -- gradient of moe_combine for an upstream gradient
 * dout [N,H] (dtype):
 *   dy[inv[n*K+k], :] = w[n,k] * dout[n, :]   rounded once, exactly (bf16:
 *                                             nearest, ties to even)
 *   dtopk_w[n,k]      = sum_h dout[n,h] * y[inv[n*K+k], h]    (fp32)
 *   y [N*K,H], dy [N*K,H] dtype, dispatched (expert-contiguous) row order;
 *   inv [N*K] int32 as from moe_dispatch; topk_w, dtopk_w [N,K] fp32.
 * Every row of dy is written once when inv is a permutation; a slot whose
 * inv is outside [0, N*K) writes no row and gets dtopk_w = 0.
 */
moe_status_t moe_combine_backward(const void *dout, const void *y, const int32_t *inv,
                                  const float *topk_w, int64_t N, int32_t H, int32_t K,
                                  moe_dtype_t dtype, void *dy, float *dtopk_w, void *stream);

/*
 * moe_dispatch_backward -- gradient of moe_dispatch's row copy:
 *   dx[n, :] = sum_k dx_perm[inv[n*K+k], :]   (fp32, k ascending, one rounding)
 *   dx_perm [N*K,H], dx [N,H] dtype; inv [N*K] int32.
 */
moe_status_t moe_dispatch_backward(const void *dx_perm, const int32_t *inv, int64_t N, int32_t H,
                                   int32_t K, moe_dtype_t dtype, void *dx, void *stream);

/*
 * Bytes of device workspace moe_route_backward needs (0 for invalid sizes).
 */
size_t moe_route_backward_workspace_size(int64_t N, int32_t H, int32_t E, int32_t K,
                                         moe_dtype_t dtype);

/*
 * moe_route_backward -- gradient of moe_route's weights (the selection ids
 * held fixed) for an upstream gradient dtopk_w [N,K], with respect to the
 * gate, the bias and the tokens, plus (optionally) the dispatch backward:
 *   dl[n,e] = w[n,k] * (dtopk_w[n,k] - sum_j w[n,j] dtopk_w[n,j]) if
 *             e = ids[n,k], else 0     (the gradient of the logits of [R]'s
 *             softmax -> top-K -> renorm chain: the full-softmax
 *             denominator cancels)
 *   dgate_w[h,e] = sum_n x[n,h] dl[n,e]           [H,E] fp32 out
 *   dbias[e]     = sum_n dl[n,e]                  [E] fp32 out, or NULL
 *   dx[n,:]      = sum_k dx_perm[inv[n*K+k],:]  +  sum_e dl[n,e] gate_w[:,e]
 *                  [N,H] dtype out, one rounding; the first sum is left out
 *                  when dx_perm is NULL
 * Inputs: x_perm [N*K,H] dtype, the forward's dispatched rows (x_perm[p] =
 * x[perm[p]/K]); gate_w [H,E] dtype; topk_ids [N,K] int32, topk_w [N,K]
 * fp32 (moe_route's outputs); perm [N*K], offsets [E+1] and inv [N*K]
 * int32 (moe_dispatch's outputs for those ids); dx_perm [N*K,H] dtype or
 * NULL.  Sums of dgate_w and dbias run over each expert's dispatched rows in
 * order, within fixed ranges of 8..256 dispatched rows (a function of N*K
 * only), then over the ranges in order: bitwise reproducible.
 *   workspace >= moe_route_backward_workspace_size(N, H, E, K, dtype); scratch
 * N == 0 is a valid call: dgate_w (and dbias) are zero-filled.
 */
moe_status_t moe_route_backward(const void *x_perm, const void *gate_w, const int32_t *topk_ids,
                                const float *topk_w, const float *dtopk_w, const int32_t *perm,
                                const int32_t *offsets, const int32_t *inv, const void *dx_perm,
                                int64_t N, int32_t H, int32_t E, int32_t K, moe_dtype_t dtype,
                                float *dgate_w, float *dbias, void *dx, void *workspace,
                                size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
