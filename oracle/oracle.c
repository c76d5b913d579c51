/*
 * Plain CPU oracle for the MoE routing path: router, counting-sort dispatch,
 * weighted combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * Every floating-point quantity is decoded from its storage bits to IEEE
 * double and computed in double with naive loops, in the order the method
 * states it.  Results are rounded once, at the end, to their storage type.
 * Build with strict IEEE semantics (no -ffast-math, -ffp-contract=off).
 *
 * Sources (the pages are cited by title and section):
 *  [R] "moe-engine: sparse MoE training infrastructure for 10k-GPU clusters"
 *      (zingnex.cn), section "Fused Triton routing kernel" (核心组件深度解析 ›
 *      融合Triton路由内核): the gate is tokens @ gate_w, then a softmax over
 *      the experts, then top-K, then renormalisation of the K kept weights.
 *      Section "Token conservation check" (Token守恒验证): the per-expert
 *      dispatch counts sum to N*K.
 *  [D] "Building a MoE training stack in 10k lines of Python" (yunpan.plus),
 *      section 8 "Expert-parallel dispatch" (八、专家并行 dispatch), 8.2
 *      "O(n) counting sort instead of O(n log n) argsort": per-expert
 *      bincount, prefix sum, then a counting-sort scatter that yields the
 *      expand index.
 *  [A] same page, section 6.1 "Model protocol first" (6.1 模型协议先行):
 *      forward_aggregate takes the expert outputs, the index that undoes the
 *      dispatch and the top-K weights, and forms the weighted expert output.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - the optional per-expert bias is part of the logits, added before the
 *    softmax;
 *  - experts are ranked by logit, descending; equal logits go to the lower
 *    expert index;
 *  - dispatch keeps no capacity limit and drops nothing; inside one expert's
 *    segment rows appear in ascending flat slot order n*K+k (stable);
 *  - combine sums k = 0..K-1 in ascending order and rounds once.
 *
 * Return codes: 0 on success, -1 on an argument this oracle does not accept.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ---- storage decode / encode (data handling, not the method) ---------- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == ORACLE_BF16) return bf16_to_double(((const uint16_t *)base)[idx]);
  return (double)((const float *)base)[idx];
}

/* Round a double to the nearest bf16, ties to even, in ONE rounding step.
 * bf16 keeps 8 significant bits (7 stored) and binary32's exponent range;
 * below 2^-126 its spacing is fixed at 2^-133.  v / q is an exact power-of-two
 * scaling, and rint() rounds half to even in the default rounding mode. */
static uint16_t double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  frexp(v, &e);           /* |v| = m * 2^e with m in [0.5, 1) */
  int unbiased = e - 1;   /* |v| = m' * 2^unbiased with m' in [1, 2) */
  double q = unbiased < -126 ? ldexp(1.0, -133) : ldexp(1.0, unbiased - 7);
  double r = rint(v / q) * q;
  if (fabs(r) >= ldexp(1.0, 128)) return signbit(v) ? 0xFF80 : 0x7F80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* Rounds v once to `dtype` and stores it at base[idx]. */
static void store_elem(void *base, int64_t idx, int dtype, double v) {
  if (dtype == ORACLE_BF16)
    ((uint16_t *)base)[idx] = double_to_bf16(v);
  else
    ((float *)base)[idx] = (float)v;
}

/* ---- threads (timing only) ------------------------------------------- */

/* Threads for the token loops of oracle_route and oracle_combine: 1 unless
 * a caller asks for more (the benchmark's CPU baseline does; the tests do
 * not).  Each token is computed the same way whatever the count, so results
 * are identical; without OpenMP the pragmas are ignored. */
static int g_threads = 1;

int oracle_set_threads(int32_t n) {
  g_threads = n < 1 ? 1 : n;
  return g_threads;
}

/* ---- [R] router -------------------------------------------------------- */

/*
 * oracle_route: for each token n
 *   logits[n,e] = sum_h x[n,h] * gate_w[h,e]  (+ bias[e])        (h ascending)
 *   order experts by (logit desc, index asc); ids[n,0..K-1] = first K
 *   p[n,e]  = exp(logit[n,e] - max_e logit) / sum_e exp(logit[n,e] - max)
 *   w[n,k]  = p[n,ids[n,k]] / sum_j p[n,ids[n,j]], rounded once to fp32
 *   margin[n] = logit of the K-th chosen expert minus the (K+1)-th, or
 *               +inf when K == E.
 * x [N,H] and gate_w [H,E] are row-major in `dtype`; bias [E] fp32 or NULL.
 * logits_out [N,E] (double) and margin [N] (double) may be NULL.
 */
/* One token of oracle_route (logit, p and order are E-entry scratch). */
static void route_token(const void *x, const void *gate_w, const float *bias, int64_t n,
                        int32_t H, int32_t E, int32_t K, int32_t dtype, int32_t *ids,
                        float *w, double *logits_out, double *margin, double *logit,
                        double *p, int32_t *order) {
  /* logits: a plain dot product per expert, h in ascending order */
  for (int32_t e = 0; e < E; ++e) logit[e] = 0.0;
  for (int32_t h = 0; h < H; ++h) {
    double xv = load_elem(x, n * (int64_t)H + h, dtype);
    for (int32_t e = 0; e < E; ++e)
      logit[e] += xv * load_elem(gate_w, (int64_t)h * E + e, dtype);
  }
  if (bias)
    for (int32_t e = 0; e < E; ++e) logit[e] += (double)bias[e];
  if (logits_out)
    for (int32_t e = 0; e < E; ++e) logits_out[n * (int64_t)E + e] = logit[e];

  /* full ordering of the experts by (logit desc, index asc):
   * insertion sort, which is stable, over indices 0..E-1 */
  for (int32_t e = 0; e < E; ++e) order[e] = e;
  for (int32_t i = 1; i < E; ++i) {
    int32_t cur = order[i];
    int32_t j = i - 1;
    while (j >= 0 && logit[order[j]] < logit[cur]) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = cur;
  }
  for (int32_t k = 0; k < K; ++k) ids[n * K + k] = order[k];
  if (margin)
    margin[n] = (K == E) ? INFINITY : logit[order[K - 1]] - logit[order[K]];

  /* softmax over all E experts */
  double mx = logit[0];
  for (int32_t e = 1; e < E; ++e)
    if (logit[e] > mx) mx = logit[e];
  double z = 0.0;
  for (int32_t e = 0; e < E; ++e) {
    p[e] = exp(logit[e] - mx);
    z += p[e];
  }
  for (int32_t e = 0; e < E; ++e) p[e] /= z;

  /* renormalise the K kept probabilities */
  double s = 0.0;
  for (int32_t k = 0; k < K; ++k) s += p[order[k]];
  for (int32_t k = 0; k < K; ++k) w[n * K + k] = (float)(p[order[k]] / s);
}

int oracle_route(const void *x, const void *gate_w, const float *bias, int64_t N,
                 int32_t H, int32_t E, int32_t K, int32_t dtype, int32_t *ids,
                 float *w, double *logits_out, double *margin) {
  if (N < 0 || H <= 0 || E <= 0 || K < 1 || K > E) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  int fail = 0;
  /* tokens are independent: each thread takes whole tokens with its own
   * scratch, so the result does not depend on the thread count */
#pragma omp parallel num_threads(g_threads)
  {
    double *logit = (double *)malloc(sizeof(double) * (size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    const int ok = logit && p && order;
    if (!ok) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n)
      if (ok)
        route_token(x, gate_w, bias, n, H, E, K, dtype, ids, w, logits_out, margin, logit, p,
                    order);
    free(logit);
    free(p);
    free(order);
  }
  return fail ? -1 : 0;
}

/* ---- [D] counting-sort dispatch --------------------------------------- */

/*
 * oracle_dispatch: ids [N,K] row-major, read as the flat slot list
 * i = n*K + k.
 *   counts[e]   = number of slots with ids[i] == e
 *   offsets[0]  = 0, offsets[e+1] = offsets[e] + counts[e]   (E+1 entries)
 *   counting sort, slots visited in ascending i:
 *       r = cursor[ids[i]]++ (cursor starts at offsets),  perm[r] = i,
 *       inv[i] = r.
 * Returns -1 if an id lies outside [0,E).
 */
int oracle_dispatch(const int32_t *ids, int64_t N, int32_t K, int32_t E,
                    int32_t *counts, int32_t *offsets, int32_t *perm,
                    int32_t *inv) {
  if (N < 0 || K < 1 || E <= 0) return -1;
  int64_t T = N * (int64_t)K;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T; ++i) {
    if (ids[i] < 0 || ids[i] >= E) return -1;
    counts[ids[i]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return -1;
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t i = 0; i < T; ++i) {
    int32_t r = cursor[ids[i]]++;
    perm[r] = (int32_t)i;
    inv[i] = r;
  }
  free(cursor);
  return 0;
}

/*
 * oracle_permute_rows: x_perm[r,:] = x[perm[r] / K, :] for r in [0, N*K),
 * a byte copy of rows of `row_bytes` bytes.
 */
int oracle_permute_rows(const void *x, int64_t N, int32_t K, int64_t row_bytes,
                        const int32_t *perm, void *x_perm) {
  if (N < 0 || K < 1 || row_bytes <= 0) return -1;
  int64_t T = N * (int64_t)K;
  const unsigned char *src = (const unsigned char *)x;
  unsigned char *dst = (unsigned char *)x_perm;
  for (int64_t r = 0; r < T; ++r) {
    int64_t n = perm[r] / K;
    if (n < 0 || n >= N) return -1;
    memcpy(dst + r * row_bytes, src + n * row_bytes, (size_t)row_bytes);
  }
  return 0;
}

/* ---- [D] expert-parallel dispatch metadata, deduplicated ---------------- */

/*
 * oracle_ep_dispatch: the metadata of [D] 8.2's fused_dedup_prepare_dispatch
 * for ep_size = R ranks holding E/R consecutive experts each (expert e lives
 * on rank e / (E/R)), with the ranks simulated as segments of one buffer.
 * Readings (the pages name the steps, not their outputs):
 *  - a token is sent once to each distinct rank among its K experts
 *    (deduplication); slot i = n*K+k "owns" the pair (n, rank of ids[i]) when
 *    no k' < k of the same token has an expert on that rank;
 *  - the send buffer is rank-major, tokens in ascending order inside a rank
 *    (a stable counting sort of the owner slots by rank);
 *  - expand_idx lists, for every dispatched row p of the expert-contiguous
 *    order of oracle_dispatch, the row of the receiving rank's segment that
 *    holds its token, counted from the start of that segment.
 * Outputs:
 *   send_counts[r]  = number of owner slots on rank r      (R entries)
 *   send_offsets[0] = 0, send_offsets[r+1] = send_offsets[r] + send_counts[r]
 *   send_tok[j]     = token of send row j, j < send_offsets[R]
 *   send_row[i]     = send row of token i/K for the rank of ids[i] (slots
 *                     sharing a rank share the row)
 *   expand_idx[p]   = send_row[perm[p]] - send_offsets[rank of ids[perm[p]]]
 * with perm from the counting-sort dispatch (computed here the same literal
 * way).  Returns -1 on a bad argument, E % R != 0, an id outside [0,E) or a
 * token with a repeated expert.
 */
int oracle_ep_dispatch(const int32_t *ids, int64_t N, int32_t K, int32_t E,
                       int32_t R, int32_t *send_counts, int32_t *send_offsets,
                       int32_t *send_tok, int32_t *send_row,
                       int32_t *expand_idx) {
  if (N < 0 || K < 1 || E <= 0 || R <= 0 || E % R != 0) return -1;
  const int32_t per_rank = E / R;
  const int64_t T = N * (int64_t)K;
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * ((size_t)E + 1));
  int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t *inv = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  unsigned char *owner = (unsigned char *)malloc((size_t)(T > 0 ? T : 1));
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int rc = -1;
  if (!counts || !offsets || !perm || !inv || !owner || !cursor) goto done;

  /* expert-level counting sort (the same definition as oracle_dispatch) */
  if (oracle_dispatch(ids, N, K, E, counts, offsets, perm, inv) != 0) goto done;

  /* which slots own a (token, rank) pair; per-rank counts of the owners */
  for (int32_t r = 0; r < R; ++r) send_counts[r] = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = ids[n * K + k];
      const int32_t r = e / per_rank;
      int first = 1;
      for (int32_t k2 = 0; k2 < k; ++k2) {
        if (ids[n * K + k2] == e) goto done; /* repeated expert */
        if (ids[n * K + k2] / per_rank == r) first = 0;
      }
      owner[n * K + k] = (unsigned char)first;
      if (first) send_counts[r] += 1;
    }
  }
  send_offsets[0] = 0;
  for (int32_t r = 0; r < R; ++r) send_offsets[r + 1] = send_offsets[r] + send_counts[r];

  /* stable counting sort of the owner slots by rank */
  for (int32_t r = 0; r < R; ++r) cursor[r] = send_offsets[r];
  for (int64_t i = 0; i < T; ++i) {
    if (!owner[i]) continue;
    const int32_t row = cursor[ids[i] / per_rank]++;
    send_tok[row] = (int32_t)(i / K);
    send_row[i] = row;
  }
  /* slots that share a rank with an earlier slot of their token */
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t k = 0; k < K; ++k) {
      if (owner[n * K + k]) continue;
      const int32_t r = ids[n * K + k] / per_rank;
      for (int32_t k2 = 0; k2 < k; ++k2) {
        if (owner[n * K + k2] && ids[n * K + k2] / per_rank == r) {
          send_row[n * K + k] = send_row[n * K + k2];
          break;
        }
      }
    }
  }
  /* receiver side: dispatched row p takes its token from its rank's segment */
  for (int64_t p = 0; p < T; ++p) {
    const int32_t i = perm[p];
    expand_idx[p] = send_row[i] - send_offsets[ids[i] / per_rank];
  }
  rc = 0;
done:
  free(counts);
  free(offsets);
  free(perm);
  free(inv);
  free(owner);
  free(cursor);
  return rc;
}

/* ---- [A] weighted combine --------------------------------------------- */

/*
 * oracle_combine: y [N*K, H] holds the expert outputs in dispatched
 * (expert-contiguous) row order, inv [N*K] maps slot n*K+k to its row, and
 * w [N,K] (fp32) are the renormalised gate weights.
 *   out[n,h] = round( sum_{k=0..K-1} (double)w[n,k] * y[inv[n*K+k], h] )
 * summed in double with k ascending from 0.0, rounded once to `dtype`
 * (bf16: nearest, ties to even; fp32: C's double->float conversion).
 */
int oracle_combine(const void *y, const int32_t *inv, const float *w, int64_t N,
                   int32_t H, int32_t K, int32_t dtype, void *out) {
  if (N < 0 || H <= 0 || K < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  int64_t T = N * (int64_t)K;
  int fail = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        int64_t row = inv[n * K + k];
        if (row < 0 || row >= T) {
#pragma omp atomic write
          fail = 1;
          continue;
        }
        acc += (double)w[n * K + k] * load_elem(y, row * H + h, dtype);
      }
      if (dtype == ORACLE_BF16)
        ((uint16_t *)out)[n * (int64_t)H + h] = double_to_bf16(acc);
      else
        ((float *)out)[n * (int64_t)H + h] = (float)acc;
    }
  }
  return fail ? -1 : 0;
}

/* ---- [A] forward_aggregate: weighted expert output + residual ------------ */

/*
 * oracle_aggregate: out[n,h] = round( sum_k w[n,k] * y[inv[n*K+k], h]
 *                                     + residual[n,h] )
 * the expert terms summed with k ascending from 0.0, then the residual
 * added, in double, rounded once to `dtype`.
 */
int oracle_aggregate(const void *y, const int32_t *inv, const float *w, const void *residual,
                     int64_t N, int32_t H, int32_t K, int32_t dtype, void *out) {
  if (N < 0 || H <= 0 || K < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t T = N * (int64_t)K;
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        const int64_t src = inv[n * K + k];
        if (src < 0 || src >= T) return -1;
        acc += (double)w[n * K + k] * load_elem(y, src * H + h, dtype);
      }
      acc += load_elem(residual, n * (int64_t)H + h, dtype);
      store_elem(out, n * (int64_t)H + h, dtype, acc);
    }
  }
  return 0;
}

/* ---- grouped expert linear layer over the dispatched rows --------------- */

/*
 * oracle_grouped_linear: the expert layer that runs between dispatch and
 * combine ([A] 6.1, forward_mlp on the gathered tokens; the MoE GroupLinear
 * of the same page's layer list), as one linear map per expert:
 *   y[p, f] = round( sum_h x_perm[p, h] * weight[e][f][h] )
 * for every dispatched row p of expert e (offsets[e] <= p < offsets[e+1]),
 * weight [E][F][H] (row f of expert e holds the weights of output f), the
 * sum in double with h ascending, rounded once to `dtype`.
 * rows (nrows entries) lists the rows to compute, y receiving them in that
 * order ([nrows][F]); rows == NULL computes every row p < offsets[E] into
 * y [offsets[E]][F].
 */
int oracle_grouped_linear(const void *x_perm, const void *weight, const int32_t *offsets,
                          int32_t E, int32_t H, int32_t F, int32_t dtype,
                          const int32_t *rows, int64_t nrows, void *y) {
  if (E <= 0 || H <= 0 || F <= 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  if (offsets[0] != 0) return -1;
  for (int32_t e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return -1;
  const int64_t total = offsets[E];
  const int64_t count = rows ? nrows : total;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t p = rows ? rows[i] : i;
    if (p < 0 || p >= total) return -1;
    int32_t e = 0;
    while (!(offsets[e] <= p && p < offsets[e + 1])) ++e; /* the segment holding p */
    for (int32_t f = 0; f < F; ++f) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += load_elem(x_perm, p * H + h, dtype) *
               load_elem(weight, ((int64_t)e * F + f) * H + h, dtype);
      store_elem(y, i * F + f, dtype, acc);
    }
  }
  return 0;
}

/* ---- backward of the path ([A] 6.2: the stages run backward in training) */

/*
 * oracle_combine_backward: the gradient of out[n,:] = sum_k w[n,k] *
 * y[inv[n*K+k],:] for an upstream gradient dout [N,H]:
 *   dy[inv[n*K+k], h] = round( w[n,k] * dout[n,h] )        (rows of y)
 *   dw[n,k]           = sum_h dout[n,h] * y[inv[n*K+k], h]  (h ascending, fp32)
 * Every row of dy is written once (inv is a permutation of [0, N*K)).
 */
int oracle_combine_backward(const void *dout, const void *y, const int32_t *inv,
                            const float *w, int64_t N, int32_t H, int32_t K,
                            int32_t dtype, void *dy, float *dw) {
  if (N < 0 || H <= 0 || K < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t T = N * (int64_t)K;
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t k = 0; k < K; ++k) {
      const int64_t rw = inv[n * K + k];
      if (rw < 0 || rw >= T) return -1;
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        const double g = load_elem(dout, n * (int64_t)H + h, dtype);
        acc += g * load_elem(y, rw * H + h, dtype);
        store_elem(dy, rw * H + h, dtype, (double)w[n * K + k] * g);
      }
      dw[n * K + k] = (float)acc;
    }
  }
  return 0;
}

/*
 * oracle_dispatch_backward: the gradient of x_perm[inv[n*K+k],:] = x[n,:]:
 *   dx[n,h] = round( sum_k dx_perm[inv[n*K+k], h] )   (k ascending)
 */
int oracle_dispatch_backward(const void *dx_perm, const int32_t *inv, int64_t N,
                             int32_t H, int32_t K, int32_t dtype, void *dx) {
  if (N < 0 || H <= 0 || K < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t T = N * (int64_t)K;
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        const int64_t rw = inv[n * K + k];
        if (rw < 0 || rw >= T) return -1;
        acc += load_elem(dx_perm, rw * H + h, dtype);
      }
      store_elem(dx, n * (int64_t)H + h, dtype, acc);
    }
  }
  return 0;
}

/*
 * oracle_route_backward: the gradient of the router's weights w [N,K] (for
 * the given selection ids) with respect to its inputs, for an upstream
 * gradient dw [N,K], by the chain rule through the two steps of [R]'s gate:
 *   p = softmax over all E experts of l = x @ gate_w (+ bias):
 *       dl[e] = p[e] * (dp[e] - sum_a dp[a] p[a])
 *   w[k] = p[ids[k]] / s, s = sum_j p[ids[j]]  (renormalisation):
 *       dp[a] = [a kept] dw[k(a)] / s - sum_k dw[k] p[ids[k]] / s^2
 * with l, p, s recomputed in double from x, gate_w and bias.  Then
 *   dgate_w[h,e] = sum_n x[n,h] dl[n,e]         (fp32 out)
 *   dbias[e]     = sum_n dl[n,e]                (fp32 out, may be NULL)
 *   dx[n,h]      = round( sum_k dx_perm[inv[n*K+k],h] + sum_e dl[n,e] gate_w[h,e] )
 * where the first term (the dispatch backward) is left out when dx_perm is
 * NULL.  dlogits [N,E] (double) may be NULL.
 */
int oracle_route_backward(const void *x, const void *gate_w, const float *bias,
                          const int32_t *ids, const float *dw, const void *dx_perm,
                          const int32_t *inv, int64_t N, int32_t H, int32_t E,
                          int32_t K, int32_t dtype, double *dlogits, float *dgate_w,
                          float *dbias, void *dx) {
  if (N < 0 || H <= 0 || E <= 0 || K < 1 || K > E) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t T = N * (int64_t)K;
  double *l = (double *)malloc(sizeof(double) * (size_t)E);
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  double *dp = (double *)malloc(sizeof(double) * (size_t)E);
  double *dl = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * (size_t)E);
  double *gacc = (double *)calloc((size_t)H * (size_t)E, sizeof(double));
  double *bacc = (double *)calloc((size_t)E, sizeof(double));
  int rc = -1;
  if (!l || !p || !dp || !dl || !gacc || !bacc) goto done;
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t e = 0; e < E; ++e) l[e] = 0.0;
    for (int32_t h = 0; h < H; ++h) {
      const double xv = load_elem(x, n * (int64_t)H + h, dtype);
      for (int32_t e = 0; e < E; ++e) l[e] += xv * load_elem(gate_w, h * (int64_t)E + e, dtype);
    }
    if (bias)
      for (int32_t e = 0; e < E; ++e) l[e] += (double)bias[e];
    double mx = l[0];
    for (int32_t e = 1; e < E; ++e)
      if (l[e] > mx) mx = l[e];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      p[e] = exp(l[e] - mx);
      z += p[e];
    }
    for (int32_t e = 0; e < E; ++e) p[e] /= z;
    double s = 0.0, t = 0.0;
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = ids[n * K + k];
      if (e < 0 || e >= E) goto done;
      s += p[e];
    }
    for (int32_t k = 0; k < K; ++k) t += (double)dw[n * K + k] * p[ids[n * K + k]];
    /* back through the renormalisation */
    for (int32_t e = 0; e < E; ++e) dp[e] = 0.0;
    for (int32_t k = 0; k < K; ++k) dp[ids[n * K + k]] = (double)dw[n * K + k] / s - t / (s * s);
    /* back through the softmax */
    double u = 0.0;
    for (int32_t a = 0; a < E; ++a) u += dp[a] * p[a];
    for (int32_t e = 0; e < E; ++e) dl[n * E + e] = p[e] * (dp[e] - u);
  }
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      const double xv = load_elem(x, n * (int64_t)H + h, dtype);
      for (int32_t e = 0; e < E; ++e) gacc[(int64_t)h * E + e] += xv * dl[n * E + e];
    }
    for (int32_t e = 0; e < E; ++e) bacc[e] += dl[n * E + e];
  }
  for (int64_t i = 0; i < (int64_t)H * E; ++i) dgate_w[i] = (float)gacc[i];
  if (dbias)
    for (int32_t e = 0; e < E; ++e) dbias[e] = (float)bacc[e];
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      if (dx_perm) {
        for (int32_t k = 0; k < K; ++k) {
          const int64_t rw = inv[n * K + k];
          if (rw < 0 || rw >= T) goto done;
          acc += load_elem(dx_perm, rw * (int64_t)H + h, dtype);
        }
      }
      for (int32_t e = 0; e < E; ++e)
        acc += dl[n * E + e] * load_elem(gate_w, h * (int64_t)E + e, dtype);
      store_elem(dx, n * (int64_t)H + h, dtype, acc);
    }
  }
  if (dlogits)
    for (int64_t i = 0; i < N * (int64_t)E; ++i) dlogits[i] = dl[i];
  rc = 0;
done:
  free(l);
  free(p);
  free(dp);
  free(dl);
  free(gacc);
  free(bacc);
  return rc;
}

/* Exposed for the encode/decode pins only. */
uint16_t oracle_round_bf16(double v) { return double_to_bf16(v); }
double oracle_decode_bf16(uint16_t b) { return bf16_to_double(b); }
