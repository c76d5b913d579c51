// Fused MoE router for gfx950: logits = x @ gate_w (+ bias), top-K by K
// rounds of selection, renormalised softmax weights -- one pass over x, the
// logits never leave the chip.
//
// Method: "moe-engine: sparse MoE training infrastructure for 10k-GPU
// clusters", section "Fused Triton routing kernel" (融合Triton路由内核): the
// gate chain tokens @ gate_w -> softmax -> top-K -> renorm is done in one
// memory pass, with K rounds of selection (not a bitonic sort) for small K and
// E <= 256.  The pages' kernel is a Triton kernel on 64x64 SRAM tiles; this one
// is laid out for CDNA4 instead:
//  * the contraction runs on v_mfma_f32_16x16x32_bf16 (bf16 products are exact
//    in fp32, accumulation in fp32);
//  * the gate is first re-laid out fragment-major (each MFMA B fragment one
//    contiguous 1 KiB block, padded to a multiple of 16 experts), so a wave
//    reads it from L2 with one 16-byte load per lane and fragment;
//  * token rows are read from HBM exactly once with coalesced 16-byte loads
//    and pass through the wave's own XOR-swizzled LDS tile into MFMA layout;
//  * a workgroup owns BM = 16*MT tokens; up to 64 experts its NW waves split H
//    and their fp32 partial logits are summed through LDS in a fixed order
//    (deterministic); for 65..128 experts, and 129..256 from 8192 tokens on,
//    the waves split the experts instead, share each step's token tile
//    through LDS and keep complete logits (route_bf16_esplit_kernel);
//  * softmax/top-K/renorm happen in registers: a token's logits live in one
//    16-lane row of the wave (lane r holds experts r, r+16, ...), and each of
//    the K rounds is a 16-lane max butterfly on order-preserving integer keys
//    followed by a min butterfly on the expert indices holding the maximum.
//
// Selection is on logits (softmax is monotone), ties go to the lower expert
// index, and since the renormalised weights equal a softmax over the K kept
// logits the full-E softmax denominator cancels and is not formed.
#include "moe_internal.h"

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_ROUTE_NW
#define MOE_ROUTE_NW 8       // waves per workgroup, splitting H (E <= 64)
#endif
#ifndef MOE_ROUTE_NW128
#define MOE_ROUTE_NW128 4    // ... for 64 < E <= 128
#endif
#ifndef MOE_ROUTE_MT64
#define MOE_ROUTE_MT64 4     // 16-token M-tiles per workgroup for E <= 64
#endif
#ifndef MOE_ROUTE_MT128
#define MOE_ROUTE_MT128 4    // ... for 64 < E <= 128 (4 waves per workgroup)
#endif
#ifndef MOE_ROUTE_ESPLIT_DEPTH
#define MOE_ROUTE_ESPLIT_DEPTH 2  // steps of register prefetch (1 or 2) in the experts-split
                                  // kernel at 65..128 experts (256 experts: always 1)
#endif
#ifndef MOE_ROUTE_ROTATE
#define MOE_ROUTE_ROTATE 1   // stagger each workgroup's first H step
#endif
#ifndef MOE_ROUTE_DEPTH
#define MOE_ROUTE_DEPTH 1    // steps of register prefetch (1 or 2) for E <= 64
#endif
#ifndef MOE_ROUTE_F32_SPLIT_H
#define MOE_ROUTE_F32_SPLIT_H 128  // fp32 router: H split four ways from this H on
#endif
#ifndef MOE_ROUTE_F32_UNROLL
#define MOE_ROUTE_F32_UNROLL 8  // fp32 router: h steps of 4 unrolled together
#endif
#ifndef MOE_ROUTE_RAW_GATE
#define MOE_ROUTE_RAW_GATE 1  // 64 experts: read the row-major gate through LDS, no packing kernel
#endif
#ifndef MOE_ROUTE_ESPLIT128
#define MOE_ROUTE_ESPLIT128 1  // 65..128 experts: waves split the experts instead of H
#endif
#ifndef MOE_ROUTE_ESPLIT256
#define MOE_ROUTE_ESPLIT256 1  // 129..256 experts: the same (from 8192 tokens on)
#endif

namespace moe {

namespace {

constexpr int kSentinel = 0x7fffffff;
constexpr int kRouteF32SplitH = MOE_ROUTE_F32_SPLIT_H;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Data movement inside a 16-lane row with DPP (a modifier on a VALU move, no
// LDS round trip).  quad_perm(1,0,3,2) and quad_perm(2,3,0,1) exchange lanes
// l^1 and l^2; row_half_mirror maps lane i to 7-i inside each half-row and
// row_mirror maps i to 15-i.  Combining a value with its image under these
// four, in that order, leaves every lane of the row with the combination of
// all 16 lanes.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

// K rounds of arg-max over the logits of U tokens, each held by this 16-lane
// group, then w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0) for the K picks.
// The U selections are independent and advance together, so their
// dependency chains interleave.  Lane r keeps round r's pick of token u and
// writes ids[t_u*K + r], w[t_u*K + r].
// v[u][q] is the logit of expert 16*q + r for token t[u] (already biased);
// experts >= E are never candidates.
//
// Each round is two 16-lane reductions on integer keys that order like the
// logits: the largest remaining key (a max butterfly), then the lowest expert
// index holding it (a min butterfly), so equal logits go to the lower index.
// key(x) flips the magnitude bits of negative values, so signed integer order
// equals float order; x + 0 first turns -0 into +0, so the two zeros are equal
// as they are for floats; a NaN logit (outside the finite-input precondition)
// is ranked as -inf.  A value that is no longer a candidate (already picked,
// or an expert index >= E) holds INT_MIN, below every key.  Integer max/min
// fold into one DPP instruction per butterfly step (a float max would also
// need the NaN-quieting of fmaxf).
__device__ __forceinline__ int order_key(float x) {
  x = (x == x) ? x + 0.0f : -__builtin_inff();
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}

template <int NT, int U>
__device__ __forceinline__ void select_topk_store(const float (&v)[U][NT], int r, int E, int K,
                                                  const int64_t (&t)[U], int64_t N,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ topw, int* hist,
                                                  int (&pick)[U]) {
  constexpr int kGone = (int)0x80000000;
  int c[U][NT];
  int my_key[U], top_key[U], my_id[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    my_key[u] = 0;
    top_key[u] = 0;
    my_id[u] = 0;
#pragma unroll
    for (int q = 0; q < NT; ++q) c[u][q] = (16 * q + r < E) ? order_key(v[u][q]) : kGone;
  }
  for (int k = 0; k < K; ++k) {
    int m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m[u] = c[u][0];
#pragma unroll
      for (int q = 1; q < NT; ++q) m[u] = max(m[u], c[u][q]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = max(m[u], dpp_i<kDppXor1>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = max(m[u], dpp_i<kDppXor2>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = max(m[u], dpp_i<kDppHalfMirror>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = max(m[u], dpp_i<kDppMirror>(m[u]));
    int ix[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ix[u] = kSentinel;
#pragma unroll
      for (int q = NT - 1; q >= 0; --q) ix[u] = (c[u][q] == m[u]) ? 16 * q + r : ix[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) ix[u] = min(ix[u], dpp_i<kDppXor1>(ix[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) ix[u] = min(ix[u], dpp_i<kDppXor2>(ix[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) ix[u] = min(ix[u], dpp_i<kDppHalfMirror>(ix[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) ix[u] = min(ix[u], dpp_i<kDppMirror>(ix[u]));
    const bool mine = (r == k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      top_key[u] = (k == 0) ? m[u] : top_key[u];
      my_key[u] = mine ? m[u] : my_key[u];
      my_id[u] = mine ? ix[u] : my_id[u];
#pragma unroll
      for (int q = 0; q < NT; ++q) c[u][q] = (16 * q + r == ix[u]) ? kGone : c[u][q];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    pick[u] = my_id[u];
    // the key transform is its own inverse
    const float my_val = __int_as_float(my_key[u] ^ ((my_key[u] >> 31) & 0x7fffffff));
    const float top = __int_as_float(top_key[u] ^ ((top_key[u] >> 31) & 0x7fffffff));
    const float ex = (r < K) ? expf(my_val - top) : 0.f;
    const float sum = sum16(ex);
    if ((t[u] < N) & (r < K)) {
      ids[t[u] * K + r] = my_id[u];
      topw[t[u] * K + r] = ex / sum;
      if (hist) atomicAdd(&hist[my_id[u]], 1);
    }
  }
}

// LDS token tiles: 16-byte chunk c of row r sits at chunk c ^ tile_swz(r).
// A 128-bit fragment read has 16 lanes on 16 consecutive rows, one logical
// chunk; with the row's low three bits alone, rows r and r + 8 land on the
// same banks when the LDS serves 16 lanes (256 bytes) at once; the fourth
// row bit flipping the low chunk bit separates them and keeps every aligned
// group of 8 rows on 8 distinct chunks.
__device__ __forceinline__ int tile_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// ---------------------------------------------------------------- bf16 MFMA
// Grid: ceil(N / BM) workgroups of NW waves, BM = 16*MT tokens each.  The NW
// waves split H into contiguous ranges of 64-wide steps; every wave computes
// fp32 partial logits of all BM tokens x EP experts over its range.
//
// A operand (token rows): per step, the wave's BM x 64 tile is read with
// coalesced 16-byte loads (8 lanes cover one 128-byte row segment), written
// to the wave's own LDS tile with an XOR swizzle (16-byte chunk c of row r is
// stored at chunk c ^ tile_swz(r)) and read back in MFMA layout; the swizzle
// makes both the writes and the fragment reads free of bank conflicts.
// B operand (gate): the gate has been packed fragment-major by
// gate_pack_kernel, so the B fragment of (step, expert tile q, half hf) is
// one contiguous 1 KiB block -- lane l loads bytes [16l, 16l+16).
//
// MFMA v_mfma_f32_16x16x32_bf16, lane l = 16g + r:
//   A[r][8g + j] = x[token 16m + r][h0 + 16g + 8hf + j]   (half hf = 0, 1)
//   B[8g + j][r] = gate[h0 + 16g + 8hf + j][expert 16q + r]
// both operands use the same (g, j) -> h map, so each MFMA pair sums h over
// [h0, h0 + 64) once.  Accumulator element i of lane l is D[4g + i][r]:
// token 16m + 4g + i, expert 16q + r.
//
// RAW (64 experts): the B operand comes straight from the row-major gate_w
// instead of the packed copy.  A step's 64 gate rows are one contiguous 8 KiB
// block; the wave copies it into its own LDS gate tile (row-major, 32-byte
// quarters of each row XOR-swizzled by (row & 3) ^ ((row >> 4) & 1), which
// keeps both the 16-byte writes and the transposing reads free of bank
// conflicts) and reads each B fragment with two ds_read_b64_tr_b16: in a
// 16-lane group, lane 4a + b points at row R + a, experts 16q + 4b .. +3, and
// the transpose hands lane r the four rows R .. R+3 of expert 16q + r.  No
// packing kernel runs.
template <int NT, int MT, int NW, int D, bool RAW>
__global__ __launch_bounds__(NW * 64) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ gfrag,
    const float* __restrict__ bias, int64_t N, int H, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ topw, int32_t* __restrict__ counts, int32_t* __restrict__ lrank,
    int32_t* __restrict__ bhist, int nb,
    int32_t* __restrict__ bpre) {
  constexpr int BM = 16 * MT;
  constexpr int EP = 16 * NT;
  constexpr int ROWP = EP + 4;
  constexpr int ALD = BM / 8;  // A load instructions per step (8 rows x 128 B each)
  constexpr int TILE = BM * 128;
  constexpr int GTILE = RAW ? 64 * EP * 2 : 0;  // the wave's gate rows of one step
  static_assert(!RAW || EP == 64, "the gate tile swizzle is laid out for 64 experts");
  constexpr int SMEM_A = NW * (TILE + GTILE);
  constexpr int SMEM_P = NW * BM * ROWP * 4;
  static_assert(BM % (4 * NW) == 0, "epilogue maps 4 tokens per wave per pass");
  static_assert((BM * kMaxRouteK + (NW + 1) * kMaxExperts) * 4 <= (SMEM_A > SMEM_P ? SMEM_A : SMEM_P),
                "dispatch ranking reuses the tile / partial-sum area");
  __shared__ __align__(16) char smem[SMEM_A > SMEM_P ? SMEM_A : SMEM_P];
  __shared__ int hist[EP];

  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BM;

  if (counts) {
    for (int e = tid; e < EP; e += NW * 64) hist[e] = 0;
  }

  // coalesced A loads: instruction j, lane -> (row 8j + lane/8, chunk lane%8)
  const int lrow = lane >> 3;
  const int lch = lane & 7;
  const uint16_t* aptr[ALD];
  int wofs[ALD];
#pragma unroll
  for (int j = 0; j < ALD; ++j) {
    const int row = 8 * j + lrow;
    int64_t t = t0 + row;
    if (t > N - 1) t = N - 1;  // tail rows recompute the last token; never stored
    aptr[j] = x + t * H + 8 * lch;
    wofs[j] = row * 128 + ((lch ^ tile_swz(row)) << 4);
  }
  // MFMA fragment reads: tile m, half hf -> (row 16m + r, chunk 2g + hf)
  int rofs[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 16 * m + r;
      rofs[m][hf] = row * 128 + (((2 * g + hf) ^ tile_swz(row)) << 4);
    }
  char* tile = smem + wid * (TILE + GTILE);
  char* gtile = tile + TILE;
  // RAW gate tile: chunk j of lane l is row 8j + l/8, 16-byte chunk l%8 of it;
  // its quarter (l%8)/2 moves to (l%8)/2 ^ ((l/8) & 3) ^ ((j/2) & 1)
  const int gw0 = (lane >> 3) * 128 + (((((lane & 7) >> 1) ^ ((lane >> 3) & 3)) << 5) | ((lane & 1) << 4));
  const int gw1 = (lane >> 3) * 128 + ((((((lane & 7) >> 1) ^ ((lane >> 3) & 3)) ^ 1) << 5) | ((lane & 1) << 4));
  // transposing reads: lane (g, r) of fragment (q, hf), half t4 reads row
  // 16g + 8hf + 4t4 + r/4, quarter q ^ ((r/4) & 3) ^ (g & 1), bytes 8(r%4)
  const int trb = (16 * g + (r >> 2)) * 128 + 8 * (r & 3);
  const int trs = ((r >> 2) & 3) ^ (g & 1);

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nss = (H + 63) >> 6;
  const int s_begin = (wid * nss) / NW;
  const int s_end = ((wid + 1) * nss) / NW;

  struct Buf {
    u32x4 a[ALD];
    u32x4 b[NT][2];
  };
  // Full steps: plain 16-byte loads that stay in flight until consumed.
  auto load = [&](Buf& bf, int s) {
#pragma unroll
    for (int j = 0; j < ALD; ++j) bf.a[j] = *reinterpret_cast<const u32x4*>(aptr[j] + s * 64);
    // packed: fragment (q, hf) of the step; RAW: 1 KiB chunk 2q + hf of the
    // step's 64 row-major gate rows
    const u32x4* gb = gfrag + (size_t)s * NT * 128 + lane;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      bf.b[q][0] = gb[(2 * q) * 64];
      bf.b[q][1] = gb[(2 * q + 1) * 64];
    }
  };
  // A ragged last step (H % 64 != 0): chunks beyond H read column 0 of
  // their row and are replaced by zeros (the packed gate is zero there).
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_masked = [&](Buf& bf, int s) {
    const bool ok = s * 64 + 8 * lch < H;  // H % 8 == 0: a chunk is all in or all out
    const int o = ok ? s * 64 : -8 * lch;
#pragma unroll
    for (int j = 0; j < ALD; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(aptr[j] + o);
      bf.a[j] = ok ? v : zero;
    }
    const u32x4* gb = gfrag + (size_t)s * NT * 128 + lane;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      if constexpr (RAW) {
        // rows at or beyond H are zero (chunk 2q + hf holds rows 16q + 8hf + lane/8)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bool in = s * 64 + 16 * q + 8 * hf + lrow < H;
          const u32x4 v = gb[in ? (2 * q + hf) * 64 : 0];
          bf.b[q][hf] = in ? v : zero;
        }
      } else {
        bf.b[q][0] = gb[(2 * q) * 64];
        bf.b[q][1] = gb[(2 * q + 1) * 64];
      }
    }
  };
  // A tile through the wave's LDS tile, then MT*NT*2 MFMAs; consecutive
  // MFMAs never depend on each other.  LDS operations of one wave complete in
  // issue order, so each read sees the writes before it and the next step's
  // writes follow this step's reads; the empty asm keeps the compiler from
  // reordering them.
  auto mma = [&](const Buf& bf) {
#pragma unroll
    for (int j = 0; j < ALD; ++j) *reinterpret_cast<u32x4*>(tile + wofs[j]) = bf.a[j];
    if constexpr (RAW) {
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j = 2 * q + hf;  // rows 8j .. 8j+7
          *reinterpret_cast<u32x4*>(gtile + 1024 * j + (((j >> 1) & 1) ? gw1 : gw0)) = bf.b[q][hf];
        }
    }
    asm volatile("" ::: "memory");
    u32x4 af[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        af[m][hf] = *reinterpret_cast<const u32x4*>(tile + rofs[m][hf]);
    bf16x8_t bfr[NT][2];
    if constexpr (RAW) {
      typedef short v4s __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          v4s h2[2];
#pragma unroll
          for (int t4 = 0; t4 < 2; ++t4)
            h2[t4] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(gtile + trb + (8 * hf + 4 * t4) * 128 +
                                                         ((q ^ trs) << 5)));
          bfr[q][hf] = __builtin_bit_cast(
              bf16x8_t, (short __attribute__((ext_vector_type(8)))){h2[0][0], h2[0][1], h2[0][2],
                                                                     h2[0][3], h2[1][0], h2[1][1],
                                                                     h2[1][2], h2[1][3]});
        }
    } else {
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) bfr[q][hf] = as_bf16x8(bf.b[q][hf]);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < NT; ++q)
          acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(af[m][hf]), bfr[q][hf], acc[m][q], 0, 0, 0);
  };

  // Each workgroup walks its range starting at a different step (rotated by
  // the workgroup index), so the resident workgroups read different column
  // windows of their rows at any moment.
  const int nfull = H >> 6;  // steps with all 64 columns inside H
  const int s_stop = s_end < nfull ? s_end : nfull;
  const int cnt = s_stop > s_begin ? s_stop - s_begin : 0;
  const int rot = (MOE_ROUTE_ROTATE && cnt > 0) ? (int)(blockIdx.x % (unsigned)cnt) : 0;
  auto step_of = [&](int i) {
    int s = s_begin + rot + i;
    return s >= s_stop ? s - cnt : s;
  };
  // Software pipeline over register buffers.  The loop bodies have no
  // branches (a branch there makes the compiler drain every outstanding load
  // at the loop head): the prefetch is always issued, clamped to the last
  // step, so the final iterations reload a step that is already cached.  A
  // scheduling barrier after each prefetch keeps its loads ahead of the
  // MFMAs, which then wait only for their own (older) loads.
  if (cnt > 0) {
    const int last = cnt - 1;
    if constexpr (D >= 2) {
      Buf p0, p1, p2;
      load(p0, step_of(0));
      load(p1, step_of(min(1, last)));
      int i = 0;
      for (; i + 3 <= cnt; i += 3) {
        load(p2, step_of(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        mma(p0);
        __builtin_amdgcn_sched_barrier(0);
        load(p0, step_of(min(i + 3, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(p1);
        __builtin_amdgcn_sched_barrier(0);
        load(p1, step_of(min(i + 4, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(p2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (cnt - i >= 1) mma(p0);
      if (cnt - i >= 2) mma(p1);
    } else {
      Buf p, q;
      load(p, step_of(0));
      int i = 0;
      for (; i + 2 <= cnt; i += 2) {
        load(q, step_of(i + 1));
        __builtin_amdgcn_sched_barrier(0);
        mma(p);
        __builtin_amdgcn_sched_barrier(0);
        load(p, step_of(min(i + 2, last)));
        __builtin_amdgcn_sched_barrier(0);
        mma(q);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i < cnt) mma(p);
    }
  }
  if (s_end > nfull && nfull >= s_begin) {  // the ragged last step, if this wave owns it
    Buf t;
    load_masked(t, nfull);
    mma(t);
  }

  // partial logits of all waves -> LDS (reusing the A tiles), summed in a
  // fixed order
  __syncthreads();
  float(*part)[BM][ROWP] = reinterpret_cast<float(*)[BM][ROWP]>(smem);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wid][16 * m + 4 * g + i][16 * q + r] = acc[m][q][i];
  __syncthreads();

  // each 16-lane group selects for the U tokens tl = wid*4 + g + u*NW*4
  constexpr int U = BM / (4 * NW);
  float v[U][NT];
  int64_t tt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tl = wid * 4 + g + u * NW * 4;
    tt[u] = t0 + tl;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      float sum = part[0][tl][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += part[w][tl][e];
      if (bias) sum += bias[e < E ? e : 0];  // e >= E is never a candidate
      v[u][q] = sum;
    }
  }
  int pick[U];
  // with lrank the dispatch histogram below also gives the counts
  select_topk_store<NT, U>(v, r, E, K, tt, N, ids, topw, (counts && !lrank) ? hist : nullptr,
                           pick);

  // For the fused dispatch (the dispatch count kernel's outputs for blocks of
  // BM tokens): the workgroup's per-expert histogram with, given bpre, its
  // exclusive prefix over the experts (the scatter ranks the slots), else the
  // stable rank of every selected slot among the equal ids of the block.
  int* sids = reinterpret_cast<int*>(smem);
  int* rhist = sids + BM * kMaxRouteK;
  if (lrank) {
    __syncthreads();  // every wave is done reading the partial sums
    int* wcnt = rhist + kMaxExperts;
    if (r < K) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tl = wid * 4 + g + u * NW * 4;
        sids[tl * K + r] = pick[u];
      }
    }
    const int ntok = (int)min((int64_t)BM, N - t0);
    if (bpre) {  // the scatter ranks each slot itself: histogram and prefix only
      block_hist_prefix<NW * 64>(sids, ntok * K, E, rhist, bhist, bpre, nb, blockIdx.x, hist);
    } else {
      block_stable_rank<NW>(sids, ntok * K, E, lrank + t0 * K, rhist, wcnt);
      for (int e = tid; e < E; e += NW * 64) bhist[(int64_t)e * nb + blockIdx.x] = rhist[e];
    }
  }

  if (counts) {
    __syncthreads();
    const int* h = lrank ? rhist : hist;
    for (int e = tid; e < E; e += NW * 64)
      if (h[e]) atomicAdd(&counts[e], h[e]);
  }
}

// ------------------------------------------------- bf16 MFMA, experts split
// The NW waves of a workgroup split the experts instead of H: wave w owns the
// 16-expert tiles [w*NTW, (w+1)*NTW) over all of H, so its accumulators hold
// complete logits (MT*NTW*4 registers) and no partial sums are exchanged.
// Each 64-wide step's token tile is loaded once per workgroup (every wave a
// share of its rows), double-buffered in LDS with the XOR swizzle above, and
// read by every wave: one barrier per step.  Up to 128 experts the registers
// hold two steps of prefetch (three buffers in rotation), 256 experts one.
// The small register and LDS footprint lets several workgroups share a CU,
// so one's selection overlaps the others' streaming.  Same MFMA operand layout as route_bf16_kernel.
template <int NT, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void route_bf16_esplit_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ gfrag,
    const float* __restrict__ bias, int64_t N, int H, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ topw, int32_t* __restrict__ counts, int32_t* __restrict__ lrank,
    int32_t* __restrict__ bhist, int nb,
    int32_t* __restrict__ bpre) {
  constexpr int BM = 16 * MT;
  constexpr int EP = 16 * NT;
  constexpr int NTW = NT / NW;   // expert tiles per wave
  constexpr int ROWP = EP + 4;
  constexpr int TILE = BM * 128;  // one step's token tile
  constexpr int ALD = BM / (8 * NW);  // token-tile loads per wave and step (8 rows each)
  static_assert(NT % NW == 0 && BM % (8 * NW) == 0, "whole expert tiles and row blocks per wave");
  static_assert(BM % (4 * NW) == 0, "epilogue maps 4 tokens per wave per pass");
  constexpr int SMEM_A = 2 * TILE;
  constexpr int SMEM_L = BM * ROWP * 4;
  constexpr int SMEM = SMEM_A > SMEM_L ? SMEM_A : SMEM_L;
  static_assert((BM * kMaxRouteK + (NW + 1) * kMaxExperts) * 4 <= SMEM,
                "dispatch ranking reuses the tile / logit area");
  __shared__ __align__(16) char smem[SMEM];
  __shared__ int hist[EP];

  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BM;
  const int q0 = wid * NTW;

  if (counts) {
    for (int e = tid; e < EP; e += NW * 64) hist[e] = 0;
  }

  // token-tile loads: wave w, load j -> row 8*(w*ALD + j) + lane/8, chunk lane%8
  const int lrow = lane >> 3;
  const int lch = lane & 7;
  const uint16_t* aptr[ALD];
  int wofs[ALD];
#pragma unroll
  for (int j = 0; j < ALD; ++j) {
    const int row = 8 * (wid * ALD + j) + lrow;
    int64_t t = t0 + row;
    if (t > N - 1) t = N - 1;  // tail rows recompute the last token; never stored
    aptr[j] = x + t * H + 8 * lch;
    wofs[j] = row * 128 + ((lch ^ tile_swz(row)) << 4);
  }
  int rofs[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 16 * m + r;
      rofs[m][hf] = row * 128 + (((2 * g + hf) ^ tile_swz(row)) << 4);
    }

  f32x4_t acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NTW; ++q) acc[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Buf {
    u32x4 a[ALD];
    u32x4 b[NTW][2];
  };
  auto load_gate = [&](Buf& bf, int s) {
    const u32x4* gb = gfrag + (size_t)s * NT * 128 + lane;
#pragma unroll
    for (int q = 0; q < NTW; ++q) {
      bf.b[q][0] = gb[(2 * (q0 + q)) * 64];
      bf.b[q][1] = gb[(2 * (q0 + q) + 1) * 64];
    }
  };
  auto load = [&](Buf& bf, int s) {
#pragma unroll
    for (int j = 0; j < ALD; ++j) bf.a[j] = *reinterpret_cast<const u32x4*>(aptr[j] + s * 64);
    load_gate(bf, s);
  };
  // the ragged last step (H % 64 != 0): chunks beyond H read column 0 of
  // their row and are replaced by zeros (the packed gate is zero there)
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_masked = [&](Buf& bf, int s) {
    const bool ok = s * 64 + 8 * lch < H;
    const int o = ok ? s * 64 : -8 * lch;
#pragma unroll
    for (int j = 0; j < ALD; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(aptr[j] + o);
      bf.a[j] = ok ? v : zero;
    }
    load_gate(bf, s);
  };
  // Step i uses LDS tile i % 2.  Its rows are written, then every wave's LDS
  // operations are waited for and the workgroup meets at a bare barrier (the
  // register prefetch of the next step stays in flight), then every wave reads
  // its fragments.  The tile written at step i was last read at step i - 2,
  // whose reads fed MFMAs issued before the barrier of step i - 1.
  auto mma = [&](const Buf& bf, int buf) {
    char* tile = smem + buf * TILE;
#pragma unroll
    for (int j = 0; j < ALD; ++j) *reinterpret_cast<u32x4*>(tile + wofs[j]) = bf.a[j];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    u32x4 af[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        af[m][hf] = *reinterpret_cast<const u32x4*>(tile + rofs[m][hf]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < NTW; ++q)
          acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(af[m][hf]), as_bf16x8(bf.b[q][hf]), acc[m][q], 0, 0, 0);
  };

  const int nfull = H >> 6;
  if (MOE_ROUTE_ESPLIT_DEPTH == 2 && NT <= 8 && nfull > 0) {
    // two steps of register prefetch: three buffers in rotation, the LDS
    // tile still alternating with the step (at 256 experts the extra 48
    // registers cost more than the deeper prefetch gains)
    const int last = nfull - 1;
    Buf p, q, o;
    load(p, 0);
    load(q, min(1, last));
    int i = 0;
    for (; i + 3 <= nfull; i += 3) {
      load(o, min(i + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      mma(p, i & 1);
      __builtin_amdgcn_sched_barrier(0);
      load(p, min(i + 3, last));
      __builtin_amdgcn_sched_barrier(0);
      mma(q, (i + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      load(q, min(i + 4, last));
      __builtin_amdgcn_sched_barrier(0);
      mma(o, (i + 2) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nfull) mma(p, i & 1);
    if (i + 1 < nfull) mma(q, (i + 1) & 1);
  } else if (nfull > 0) {
    const int last = nfull - 1;
    Buf p, q;
    load(p, 0);
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
      load(q, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(p, 0);
      __builtin_amdgcn_sched_barrier(0);
      load(p, min(i + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      mma(q, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nfull) mma(p, 0);
  }
  if (H & 63) {
    Buf t;
    load_masked(t, nfull);
    mma(t, nfull & 1);
  }

  // complete logits -> LDS (reusing the token tiles)
  __syncthreads();
  float(*lg)[ROWP] = reinterpret_cast<float(*)[ROWP]>(smem);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < NTW; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[16 * m + 4 * g + i][16 * (q0 + q) + r] = acc[m][q][i];
  __syncthreads();

  // each 16-lane group selects for the U tokens tl = wid*4 + g + u*NW*4
  constexpr int U = BM / (4 * NW);
  float v[U][NT];
  int64_t tt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tl = wid * 4 + g + u * NW * 4;
    tt[u] = t0 + tl;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      float sum = lg[tl][e];
      if (bias) sum += bias[e < E ? e : 0];  // e >= E is never a candidate
      v[u][q] = sum;
    }
  }
  int pick[U];
  select_topk_store<NT, U>(v, r, E, K, tt, N, ids, topw, (counts && !lrank) ? hist : nullptr,
                           pick);

  int* sids = reinterpret_cast<int*>(smem);
  int* rhist = sids + BM * kMaxRouteK;
  if (lrank) {
    __syncthreads();  // every wave is done reading the logits
    int* wcnt = rhist + kMaxExperts;
    if (r < K) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tl = wid * 4 + g + u * NW * 4;
        sids[tl * K + r] = pick[u];
      }
    }
    const int ntok = (int)min((int64_t)BM, N - t0);
    if (bpre) {  // the scatter ranks each slot itself: histogram and prefix only
      block_hist_prefix<NW * 64>(sids, ntok * K, E, rhist, bhist, bpre, nb, blockIdx.x, hist);
    } else {
      block_stable_rank<NW>(sids, ntok * K, E, lrank + t0 * K, rhist, wcnt);
      for (int e = tid; e < E; e += NW * 64) bhist[(int64_t)e * nb + blockIdx.x] = rhist[e];
    }
  }

  if (counts) {
    __syncthreads();
    const int* h = lrank ? rhist : hist;
    for (int e = tid; e < E; e += NW * 64)
      if (h[e]) atomicAdd(&counts[e], h[e]);
  }
}

// ---------------------------------------------------------------- fp32 VALU
// kRouteF32Tokens = 16 tokens per workgroup of 256 * HS threads: wave w
// (w % 4 = token group, w / 4 = quarter of H when HS = 4), lane group g owns
// token 16*blockIdx + 4(w % 4) + g; lane r accumulates experts r, r+16, ...
// with one fp32 FMA chain per expert and H part in ascending h; with HS = 4
// the four parts' sums are added in part order through LDS.  With lrank (the
// fused call) the workgroup ranks its picks for the dispatch like the bf16
// kernels.
template <int NT, int HS>
__global__ __launch_bounds__(256 * HS) void route_f32_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ gate_w,
                                                             const float* __restrict__ bias,
                                                             int64_t N, int H, int E, int K,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ topw,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ lrank,
                                                             int32_t* __restrict__ bhist,
                                                             int nb) {
  static_assert(kRouteF32Tokens == 16, "four tokens per wave, four token groups");
  static_assert(HS == 1 || HS == 4, "one or four parts of H");
  constexpr int EP = 16 * NT;
  __shared__ int hist[EP];
  __shared__ int sids[kRouteF32Tokens * kMaxRouteK];
  __shared__ int rhist[kMaxExperts];
  __shared__ int wcnt[4 * HS * kMaxExperts];
  __shared__ float part[HS > 1 ? (HS - 1) * kRouteF32Tokens * EP : 1];
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int tl = (wid & 3) * 4 + g;  // token within the workgroup
  const int hq = wid >> 2;           // part of H
  const int64_t t = (int64_t)blockIdx.x * 16 + tl;
  if (counts) {
    for (int e = tid; e < EP; e += 256 * HS) hist[e] = 0;
    __syncthreads();
  }
  const int64_t tc = t < N ? t : N - 1;
  const float* xr = x + tc * H;
  // this wave's part of H: whole 4-value steps
  const int nst = H >> 2;
  const int h_begin = 4 * ((hq * nst) / HS);
  const int h_end = 4 * (((hq + 1) * nst) / HS);
  float acc[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) acc[q] = 0.f;
  // (unrolled so that several steps' loads are in flight; the FMA order per
  // expert stays h ascending)
#pragma unroll MOE_ROUTE_F32_UNROLL
  for (int h = h_begin; h < h_end; h += 4) {
    const float4 xv = *reinterpret_cast<const float4*>(xr + h);
    const float* wr = gate_w + (int64_t)h * E;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + r;
      if (e < E) {
        acc[q] = fmaf(xv.x, wr[e], acc[q]);
        acc[q] = fmaf(xv.y, wr[E + e], acc[q]);
        acc[q] = fmaf(xv.z, wr[2 * E + e], acc[q]);
        acc[q] = fmaf(xv.w, wr[3 * E + e], acc[q]);
      }
    }
  }
  if constexpr (HS > 1) {
    if (hq > 0) {
#pragma unroll
      for (int q = 0; q < NT; ++q) part[((hq - 1) * kRouteF32Tokens + tl) * EP + 16 * q + r] = acc[q];
    }
    __syncthreads();
    if (hq == 0) {
#pragma unroll
      for (int p = 0; p < HS - 1; ++p)
#pragma unroll
        for (int q = 0; q < NT; ++q) acc[q] += part[(p * kRouteF32Tokens + tl) * EP + 16 * q + r];
    }
  }
  int pick[1] = {0};
  if (hq == 0) {
    if (bias) {
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const int e = 16 * q + r;
        acc[q] += bias[e < E ? e : 0];  // e >= E is never a candidate
      }
    }
    float v1[1][NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) v1[0][q] = acc[q];
    const int64_t t1[1] = {t};
    select_topk_store<NT, 1>(v1, r, E, K, t1, N, ids, topw, (counts && !lrank) ? hist : nullptr,
                             pick);
  }
  if (lrank) {
    const int64_t t0 = (int64_t)blockIdx.x * kRouteF32Tokens;
    if (hq == 0 && r < K) sids[tl * K + r] = pick[0];
    const int ntok = (int)min((int64_t)kRouteF32Tokens, N - t0);
    // (the ranking's first barrier publishes sids)
    block_stable_rank<4 * HS>(sids, ntok * K, E, lrank + t0 * K, rhist, wcnt);
    for (int e = tid; e < E; e += 256 * HS) bhist[(int64_t)e * nb + blockIdx.x] = rhist[e];
  }
  if (counts) {
    __syncthreads();
    const int* h = lrank ? rhist : hist;
    for (int e = tid; e < E; e += 256 * HS)
      if (h[e]) atomicAdd(&counts[e], h[e]);
  }
}

// ------------------------------------------------------- gate re-layout
// Packs gate_w [H,E] fragment-major for route_bf16_kernel: for step s (64
// values of h), expert tile q (16 experts) and half hf, a 1 KiB block whose
// 16 bytes at lane l = 16g + r hold gate[h0 .. h0+8][16q + r] with
// h0 = 64s + 16g + 8hf -- exactly one MFMA B fragment.  Values with h >= H or
// e >= E are zero, so the router needs no masking on this operand.
// Each thread builds one fragment entry: expert e, eight rows h0 .. h0+7
// (eight 2-byte loads -- the 64 lanes of a wave read 64 consecutive experts
// of a row, so each load instruction is one coalesced row segment -- and one
// 16-byte store).  One thread per entry keeps the launch wide (HP/8 * EP
// threads), which is what the latency of this small re-layout needs.
// Threads 0..E-1 also zero `counts` (the router then adds into it).
__global__ __launch_bounds__(64) void gate_pack_kernel(const uint16_t* __restrict__ gate_w, int H,
                                                       int E, int EP, int HP,
                                                       u32x4* __restrict__ gfrag,
                                                       int32_t* __restrict__ counts) {
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (counts && idx < E) counts[idx] = 0;
  const int nhb = HP / 8;  // 8-row blocks of h, including the zero padding up to HP
  if (idx >= (int64_t)nhb * EP) return;
  const int hb = (int)(idx / EP);
  const int e = (int)(idx - (int64_t)hb * EP);
  const int h0 = hb * 8;
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    t[i] = (e < E && h0 + i < H) ? (uint32_t)gate_w[(int64_t)(h0 + i) * E + e] : 0u;
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) o[p] = t[2 * p] | (t[2 * p + 1] << 16);
  const int s = h0 >> 6;
  const int g = (h0 >> 4) & 3;
  const int hf = (h0 >> 3) & 1;
  const int NTL = EP / 16;
  gfrag[((int64_t)(s * NTL + (e >> 4)) * 2 + hf) * 64 + 16 * g + (e & 15)] = o;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// the experts-split router: NW waves of NT / NW expert tiles each
template <int NT, int MT, int NW>
hipError_t launch_bf16_esplit(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                              int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                              int32_t* lrank, int32_t* bhist, int32_t* bpre, hipStream_t s) {
  const int64_t blocks = (N + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL((route_bf16_esplit_kernel<NT, MT, NW>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, s, x, reinterpret_cast<const u32x4*>(wgt), bias, N, H, E,
                     K, ids, w, counts, lrank, bhist, (int)blocks, bpre);
  return hipGetLastError();
}

template <int NT, int MT, int NW = (NT <= 4 ? MOE_ROUTE_NW : NT == 8 ? MOE_ROUTE_NW128 : 4),
          int D = (NT <= 4 ? MOE_ROUTE_DEPTH : 1)>
hipError_t launch_bf16_nt(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                          int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                          int32_t* lrank, int32_t* bhist, int32_t* bpre, hipStream_t s,
                          bool raw = false) {
  const int64_t blocks = (N + 16 * MT - 1) / (16 * MT);
  if constexpr (NT == 4) {
    if (raw) {
      hipLaunchKernelGGL((route_bf16_kernel<NT, MT, NW, D, true>), dim3((unsigned)blocks),
                         dim3(NW * 64), 0, s, x, reinterpret_cast<const u32x4*>(wgt), bias, N, H,
                         E, K, ids, w, counts, lrank, bhist, (int)blocks, bpre);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_bf16_kernel<NT, MT, NW, D, false>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, s, x, reinterpret_cast<const u32x4*>(wgt), bias, N, H, E, K,
                     ids, w, counts, lrank, bhist, (int)blocks, bpre);
  return hipGetLastError();
}

// tokens per workgroup of route_bf16_kernel for E experts (must match the
// MT chosen in launch_route_bf16)
constexpr int route_mt(int EP) {
  return EP <= 64 ? (EP <= 32 ? 4 : MOE_ROUTE_MT64) : EP == 128 ? MOE_ROUTE_MT128 : 1;
}

template <int NT>
hipError_t launch_f32_nt(const float* x, const float* gw, const float* bias, int64_t N, int H,
                         int E, int K, int32_t* ids, float* w, int32_t* counts, int32_t* lrank,
                         int32_t* bhist, hipStream_t s) {
  const int64_t blocks = (N + kRouteF32Tokens - 1) / kRouteF32Tokens;
  // four waves per token group over H once each part keeps a long chain
  if (H >= kRouteF32SplitH)
    hipLaunchKernelGGL((route_f32_kernel<NT, 4>), dim3((unsigned)blocks), dim3(1024), 0, s, x,
                       gw, bias, N, H, E, K, ids, w, counts, lrank, bhist, (int)blocks);
  else
    hipLaunchKernelGGL((route_f32_kernel<NT, 1>), dim3((unsigned)blocks), dim3(256), 0, s, x,
                       gw, bias, N, H, E, K, ids, w, counts, lrank, bhist, (int)blocks);
  return hipGetLastError();
}

}  // namespace

int route_padded_experts(int E) {
  int ep = 16;
  while (ep < E) ep *= 2;
  return ep;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n,
                     v);
  return hipGetLastError();
}

int route_gate_rows(int H) { return (H + 63) / 64 * 64; }

hipError_t launch_gate_transpose(const uint16_t* gate_w, int H, int E, uint16_t* wgt,
                                 int32_t* counts, hipStream_t s) {
  const int EP = route_padded_experts(E);
  const int HP = route_gate_rows(H);
  int64_t threads = (int64_t)(HP / 8) * EP;
  if (threads < E) threads = E;
  hipLaunchKernelGGL(gate_pack_kernel, dim3((unsigned)((threads + 63) / 64)), dim3(64), 0, s,
                     gate_w, H, E, EP, HP, reinterpret_cast<u32x4*>(wgt), counts);
  return hipGetLastError();
}

// For 32 < E <= 128 the workgroup takes 64 tokens only when that still gives
// every CU a workgroup (N >= 256 * 64); smaller N use 32-token workgroups,
// twice as many, so more CUs stream x (the gate is read once per workgroup).
// For 128 < E <= 256 the experts-split kernel takes 64 or 32 tokens the same
// way from 8192 tokens on; below that the H-split kernel with 16 tokens per
// workgroup is faster (more workgroups).
constexpr int64_t kRouteSmallN = 256 * 64;
constexpr int64_t kRoute256SplitN = 8192;
static bool route_small(int EP, int64_t N) { return (EP == 64 || EP == 128) && N < kRouteSmallN; }
// Up to 256 * 16 tokens, 33..64 experts take 16-token workgroups of 4 waves
// (one workgroup per CU at most, where 32-token workgroups of 8 waves would
// leave half the CUs idle); above that the 32-token ones are faster.
constexpr int64_t kRouteTinyN = 256 * 16;
static bool route_tiny64(int64_t N) { return N <= kRouteTinyN; }
static bool route_esplit256(int64_t N) { return MOE_ROUTE_ESPLIT256 && N >= kRoute256SplitN; }

#ifndef MOE_ROUTE_ESPLIT128_BIG
#define MOE_ROUTE_ESPLIT128_BIG 1  // 65..128 experts from 2*kRouteSmallN tokens: 128-token, 8-wave tiles
#endif
static bool route_esplit128_big(int64_t N) { return MOE_ROUTE_ESPLIT128_BIG && N >= 2 * kRouteSmallN; }

int route_tokens_per_block(int E, int64_t N) {
  const int EP = route_padded_experts(E);
  if (EP == 128 && MOE_ROUTE_ESPLIT128 && route_esplit128_big(N)) return 128;
  if (EP == 64 && route_tiny64(N)) return 16;
  if (EP == 256 && route_esplit256(N)) return N < kRouteSmallN ? 32 : 64;
  return route_small(EP, N) ? 32 : 16 * route_mt(EP);
}

bool route_gate_raw(int E) { return MOE_ROUTE_RAW_GATE && E == 64; }

hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* wgt, const float* bias, int64_t N,
                             int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                             int32_t* lrank, int32_t* bhist, hipStream_t s, int32_t* bpre) {
  const bool raw = route_gate_raw(E);
  switch (route_padded_experts(E)) {
    case 16:
      return launch_bf16_nt<1, route_mt(16)>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                             bhist, bpre, s);
    case 32:
      return launch_bf16_nt<2, route_mt(32)>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                             bhist, bpre, s);
    case 64:
      if (route_tiny64(N))
        return launch_bf16_nt<4, 1, 4, 1>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank, bhist, bpre, s,
                                          raw);
      if (route_small(64, N))
        return launch_bf16_nt<4, 2>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank, bhist, bpre, s, raw);
      return launch_bf16_nt<4, route_mt(64)>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                             bhist, bpre, s, raw);
    case 128:
      if (MOE_ROUTE_ESPLIT128) {
        if (route_esplit128_big(N))
          return launch_bf16_esplit<8, 8, 8>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                             bhist, bpre, s);
        if (route_small(128, N))
          return launch_bf16_esplit<8, 2, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                             bhist, bpre, s);
        return launch_bf16_esplit<8, route_mt(128), 4>(x, wgt, bias, N, H, E, K, ids, w, counts,
                                                       lrank, bhist, bpre, s);
      }
      if (route_small(128, N))
        return launch_bf16_nt<8, 2>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank, bhist, bpre, s);
      return launch_bf16_nt<8, route_mt(128)>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                              bhist, bpre, s);
    case 256:
      if (route_esplit256(N)) {
        if (N < kRouteSmallN)
          return launch_bf16_esplit<16, 2, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                              bhist, bpre, s);
        return launch_bf16_esplit<16, 4, 4>(x, wgt, bias, N, H, E, K, ids, w, counts, lrank,
                                            bhist, bpre, s);
      }
      return launch_bf16_nt<16, route_mt(256), 4>(x, wgt, bias, N, H, E, K, ids, w, counts,
                                                  lrank, bhist, bpre, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route_f32(const float* x, const float* gate_w, const float* bias, int64_t N,
                            int H, int E, int K, int32_t* ids, float* w, int32_t* counts,
                            int32_t* lrank, int32_t* bhist, hipStream_t s) {
  switch (route_padded_experts(E)) {
    case 16: return launch_f32_nt<1>(x, gate_w, bias, N, H, E, K, ids, w, counts, lrank, bhist, s);
    case 32: return launch_f32_nt<2>(x, gate_w, bias, N, H, E, K, ids, w, counts, lrank, bhist, s);
    case 64: return launch_f32_nt<4>(x, gate_w, bias, N, H, E, K, ids, w, counts, lrank, bhist, s);
    case 128: return launch_f32_nt<8>(x, gate_w, bias, N, H, E, K, ids, w, counts, lrank, bhist, s);
    case 256: return launch_f32_nt<16>(x, gate_w, bias, N, H, E, K, ids, w, counts, lrank, bhist, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
