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
//  * a workgroup computes a BM x 256 tile of one expert's output (BM = 256
//    once there are enough tiles to fill the chip, else 128); its m-tiles
//    are numbered expert by expert (the BM-row tiles of expert e start at
//    tile sum_{e'<e} ceil(count[e'] / BM)), so each expert's ragged last
//    tile stays inside its segment;
//  * tiles are ordered for the 8 XCDs: each XCD gets whole groups of two
//    consecutive m-tiles with all their n-tiles, so a group's token rows and
//    its expert's weight rows are fetched into that XCD's L2 once;
//  * both operands are K-contiguous rows (token rows of x_perm, weight rows
//    of one output each), copied global -> LDS with global_load_lds_dwordx4
//    into a ring of K steps ahead of the MFMAs: 64-wide steps (whole
//    128-byte lines of each row) in two 64 KiB slots for 256-row tiles when
//    H % 64 == 0, else 32-wide steps in four (three) slots, the 16-byte
//    chunks of each row XOR-swizzled;
//  * 8 waves (two per SIMD) in a 2 x 4 grid of (BM/2) x 64 blocks of
//    v_mfma_f32_16x16x32_bf16 tiles, fp32 accumulation, one rounding to bf16
//    at the end.
// When H % 32 != 0: 256 x 256 or 128 x 128 tiles of 4 waves with 64-wide K
// steps double-buffered through registers, chunk c of row r at c ^ (r & 7).
// fp32 inputs use an LDS-tiled fp32 FMA kernel (64 x 64 tiles).
#include "moe_internal.h"

#ifndef MOE_GEMM_SMALL_RING
#define MOE_GEMM_SMALL_RING 1     // small problems: 128 x 256 ring tiles (0: the 128 x 128 kernel)
#endif
#ifndef MOE_GEMM_RING128_SLOTS
#define MOE_GEMM_RING128_SLOTS 3  // ring slots of the 128-row ring tiles
#endif
#ifndef MOE_GEMM_HALF_SKIP
#define MOE_GEMM_HALF_SKIP 1      // ring tiles: waves whose half of a ragged tile is empty skip MFMAs
#endif

namespace moe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBK = 64;   // K step (h)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// LDS swizzle of a 128-byte tile row: 16-byte chunk c of row r is stored in
// slot c ^ swz(r)
__device__ __forceinline__ int swz(int r) { return r & 7; }

// s_waitcnt immediate for vmcnt(v) alone (expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int v) { return (v & 15) | 0x70 | 0xF00 | (((v >> 4) & 3) << 14); }

// This workgroup's expert and rows: tiles of BM rows are numbered expert by
// expert.  Offsets are clamped to [0, T] (inconsistent ones give wrong rows,
// never an access outside x_perm or y).  Returns false past the last tile.
// Works for any workgroup size: experts are taken one per thread by the first
// four waves (E <= 256); s_scan holds 4 ints.
template <int BM>
__device__ __forceinline__ bool tile_of(const int32_t* offsets, int E, int64_t T, int id,
                                        int* s_e, int64_t* s_m0, int* s_rows, int* s_scan) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t o0 = tid < E ? min(max((int64_t)offsets[tid], (int64_t)0), T) : 0;
  const int64_t o1 = tid < E ? min(max((int64_t)offsets[tid + 1], o0), T) : 0;
  const int nt = (int)((o1 - o0 + BM - 1) / BM);
  const int incl = wave_inclusive_sum(nt);
  if (lane == 63 && wid < 4) s_scan[wid] = incl;
  if (tid == 0) *s_e = -1;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) base += w < wid ? s_scan[w] : 0;
  const int cb = base + incl - nt;
  if (tid < E && id >= cb && id < cb + nt) {
    *s_e = tid;
    *s_m0 = o0 + (int64_t)(id - cb) * BM;
    *s_rows = (int)min((int64_t)BM, o1 - *s_m0);
  }
  __syncthreads();
  return *s_e >= 0;
}

// Tile order.  Workgroup b runs on XCD b % 8 (the dispatcher's round robin)
// and, on that XCD, in the order of b / 8.  Each XCD is given whole groups
// of kGroupM consecutive m-tiles (consecutive m-tiles are mostly one expert)
// with all their n-tiles, m-tile group j going to XCD j % 8: the group's
// token rows and its expert's weight rows are then fetched into that XCD's
// L2 once and reused by every n-tile, instead of every XCD streaming every
// operand.  Padding ids (past the last group) do nothing.
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 2   // consecutive m-tiles (with all their n-tiles) per XCD group
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;

__device__ __forceinline__ bool tile_coords(int ntn, int* mt, int* nt) {
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int slot = b >> 3;
  const int per_group = kGroupM * ntn;
  const int j = slot / per_group;          // this XCD's j-th group
  const int t = slot - j * per_group;
  *mt = (j * 8 + xcd) * kGroupM + t / ntn;
  *nt = t - (t / ntn) * ntn;
  return true;
}

// BM x BN output tile of one expert, 4 waves in a 2 x 2 grid, each wave a
// (BM/2) x (BN/2) block of 16 x 16 MFMA tiles.
template <int BM, int BN>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ offsets, int E, int64_t T, int H, int F, int ntn,
    uint16_t* __restrict__ y) {
  constexpr int MT = BM / 32;  // 16-row MFMA tiles per wave (rows)
  constexpr int NT = BN / 32;  // ... (outputs)
  constexpr int LA = BM / 32;  // 16-byte global loads per thread and step (A)
  constexpr int LB = BN / 32;  // ... (B)
  __shared__ __align__(16) char sA[2][BM * 128];
  __shared__ __align__(16) char sB[2][BN * 128];
  __shared__ int s_e, s_rows;
  __shared__ int64_t s_m0;
  __shared__ int s_scan[4];
  int mt, nt;
  if (!tile_coords(ntn, &mt, &nt)) return;
  if (!tile_of<BM>(offsets, E, T, mt, &s_e, &s_m0, &s_rows, s_scan)) return;
  const int e = s_e;
  const int64_t m0 = s_m0;
  const int rows = s_rows;
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int wm = wid & 1;
  const int wn = wid >> 1;

  // global -> LDS: 8 threads per 128-byte row segment of a 64-wide K step.
  // Rows past the tile's valid rows (outputs past F) reload the last valid
  // one; they are never stored.  Offsets are 32-bit from the tile's bases.
  // Thread t loads chunk lch = t % 8 of rows t/8 + 32*i, so its LDS slot of
  // load i is lof + 4096*i (the swizzle depends on the row mod 8 only).
  const uint16_t* xa = x + m0 * H;
  const uint16_t* wb = w + ((int64_t)e * F) * H;
  const int lch = tid & 7;
  const int rr0 = tid >> 3;
  const int lof = rr0 * 128 + ((lch ^ swz(rr0)) << 4);
  int aof[LA], bof[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) aof[i] = min(rr0 + 32 * i, rows - 1) * H + 8 * lch;
#pragma unroll
  for (int i = 0; i < LB; ++i) bof[i] = min(n0 + rr0 + 32 * i, F - 1) * H + 8 * lch;
  // fragment rows: A (BM/2)*wm + 16*t + r, B (BN/2)*wn + 16*t + r; chunk 4*kh + g
  auto frag_off = [&](int row, int kh) { return row * 128 + (((4 * kh + g) ^ swz(row)) << 4); };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](u32x4 (&ra)[LA], u32x4 (&rb)[LB], int kt) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(xa + aof[i] + kt * GBK);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(wb + bof[i] + kt * GBK);
  };
  // the ragged last K step (H % 64 != 0; H % 8 == 0): chunks with h >= H are
  // zero, their loads read column 0 of the row instead
  auto gload_masked = [&](u32x4 (&ra)[LA], u32x4 (&rb)[LB], int kt) {
    const bool ok = kt * GBK + 8 * lch < H;
    const int ko = ok ? kt * GBK : -8 * lch;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xa + aof[i] + ko);
      ra[i] = ok ? v : zero;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wb + bof[i] + ko);
      rb[i] = ok ? v : zero;
    }
  };
  auto lstore = [&](int buf, const u32x4 (&ra)[LA], const u32x4 (&rb)[LB]) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(sA[buf] + lof + 4096 * i) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4*>(sB[buf] + lof + 4096 * i) = rb[i];
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4 af[MT], bf[NT];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        af[t] = *reinterpret_cast<const u32x4*>(sA[buf] + frag_off((BM / 2) * wm + 16 * t + r, kh));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bf[t] = *reinterpret_cast<const u32x4*>(sB[buf] + frag_off((BN / 2) * wn + 16 * t + r, kh));
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
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
  u32x4 ra[LA], rb[LB];
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

  // lane (g, r), tile (mi, ni), element i: output row (BM/2)*wm + 16*mi +
  // 4*g + i, column n0 + (BN/2)*wn + 16*ni + r
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int col = n0 + (BN / 2) * wn + 16 * ni + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (BM / 2) * wm + 16 * mi + 4 * g + i;
        if (row < rows && col < F)
          y[(m0 + row) * F + col] = (uint16_t)f32_to_bf16_rne(acc[mi][ni][i]);
      }
    }
}

// Ring tiles (H % RK == 0): each K step's A and B tiles (BM and 256 rows of
// 2*RK bytes) are copied global -> LDS with global_load_lds (no registers)
// into a ring of slots, RING - 1 steps ahead of the MFMAs.
//  * RK = 64 (256-row tiles when H % 64 == 0): whole 128-byte lines per
//    row, 2 slots of 64 KiB; chunk c of row r at c ^ (r & 7).  All of a
//    step's fragments are read before its MFMAs, and the reads of its second
//    32-wide half are interleaved with the first half's MFMAs.
//  * RK = 32: 4 slots of 32 KiB (256-row tiles) or 3 of 24 KiB (128-row
//    tiles, two workgroups per CU); chunk c of row r at c ^ ((r >> 1) & 3).
// Either way the eight lanes of one LDS read phase (rows r..r+7 of one chunk
// column) hit eight different 16-byte bank groups.
// 8 waves (two per SIMD) in a 2 x 4 grid of (BM/2) x 64 blocks: 128
// accumulator registers per wave leave the register allocator room (a
// 4-wave 128 x 128 layout fills all 256 AGPRs and the compiler shuffles
// accumulators), and one wave's MFMAs cover the other's barrier and reads.
// Per step and wave: (BM + 256) / 8 rows of copies, counted by vmcnt in
// issue order; the ring keeps each wait count constant (the last steps
// re-copy the last step into slots nothing reads any more).
//
// The copies are issued from inline asm, so the compiler does not see them:
// it would otherwise treat every LDS read as possibly aliasing a copy still
// in flight and wait for all of them (vmcnt(0)) before each read.  The
// explicit vmcnt wait plus a bare workgroup barrier (no release fence, which
// would also wait for every copy) order each slot's copies before its reads.
// M0 holds the LDS destination of a copy; nothing else in this kernel uses it.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(src)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int RK>
__global__ __launch_bounds__(512) void grouped_gemm_ring_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ offsets, int E, int64_t T, int H, int F, int ntn,
    uint16_t* __restrict__ y) {
  static_assert(RK == 32 || RK == 64, "K step of 32 or 64");
  constexpr int BN = 256;
  constexpr int RB = 2 * RK;                  // bytes per row and step
  constexpr int CPR = RB / 16;                // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per copy instruction
  constexpr int SLOT = (BM + BN) * RB;        // A then B
  constexpr int RING = RK == 64 ? 2 : (BM == 256 ? 4 : MOE_GEMM_RING128_SLOTS);
  constexpr int MT = BM / 32, NT = 4;         // 16 x 16 tiles per wave (rows, outputs)
  constexpr int KH = RK / 32;                 // 32-wide MFMA steps per K step
  constexpr int LA = BM / 8 / RPI;            // copies per wave and step: A
  constexpr int LB = BN / 8 / RPI;            //                           B
  constexpr int OPS = LA + LB;
  __shared__ __align__(1024) char smem[RING * SLOT];
  __shared__ int s_e, s_rows;
  __shared__ int64_t s_m0;
  __shared__ int s_scan[4];
  int mt, nt;
  if (!tile_coords(ntn, &mt, &nt)) return;
  if (!tile_of<BM>(offsets, E, T, mt, &s_e, &s_m0, &s_rows, s_scan)) return;
  const int e = s_e;
  const int64_t m0 = s_m0;
  const int rows = s_rows;
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;   // 8 waves: a 2 x 4 grid of (BM/2) x 64 blocks
  const int g = lane >> 4;
  const int r = lane & 15;
  const int wm = wid & 1;
  const int wn = wid >> 1;
  // slot chunk of global chunk c in row rr (rows of one copy instruction
  // start at a multiple of RPI >= 8, so the swizzle depends on rr % RPI only)
  auto sw = [](int c, int rr) { return RK == 64 ? c ^ (rr & 7) : c ^ ((rr >> 1) & 3); };

  // copies: wave w fills A rows (BM/8)w + RPI*i .. +RPI (i < LA) and B rows
  // 32w + RPI*i .. +RPI (i < LB); lane l -> row +l/CPR, slot chunk l%CPR,
  // which holds global chunk sw(l%CPR, row).  Offsets are 32-bit from the
  // tile's bases.
  const uint16_t* xa = x + m0 * H;
  const uint16_t* wb = w + ((int64_t)e * F) * H;
  const int dr = lane / CPR;
  const int dch = sw(lane % CPR, dr);
  int aof[LA], bof[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) aof[i] = min((BM / 8) * wid + RPI * i + dr, rows - 1) * H + 8 * dch;
#pragma unroll
  for (int i = 0; i < LB; ++i) bof[i] = min(n0 + 32 * wid + RPI * i + dr, F - 1) * H + 8 * dch;
  const uint32_t base = lds_addr(smem);
  // (the LDS destination of a copy is wave-uniform: M0 takes a scalar)
  const uint32_t abase = __builtin_amdgcn_readfirstlane(base + (uint32_t)((BM / 8) * wid * RB));
  const uint32_t bbase =
      __builtin_amdgcn_readfirstlane(base + (uint32_t)(BM * RB + 32 * wid * RB));
  auto copy_step = [&](int slot, int kt) {
    const uint32_t so = (uint32_t)(slot * SLOT);
#pragma unroll
    for (int i = 0; i < LA; ++i)
      lds_copy16(xa + aof[i] + kt * RK, abase + so + (uint32_t)(RPI * RB * i));
#pragma unroll
    for (int i = 0; i < LB; ++i)
      lds_copy16(wb + bof[i] + kt * RK, bbase + so + (uint32_t)(RPI * RB * i));
  };
  // fragment reads of MFMA step h: A rows (BM/2)*wm + 16*t + r, B rows
  // 64*wn + 16*t + r, global chunk 4h + g
  int aoff[KH], boff[KH];
#pragma unroll
  for (int h = 0; h < KH; ++h) {
    aoff[h] = ((BM / 2) * wm + r) * RB + (sw(4 * h + g, r) << 4);
    boff[h] = BM * RB + (64 * wn + r) * RB + (sw(4 * h + g, r) << 4);
  }
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = H / RK;
  const int last = nk - 1;
#pragma unroll
  for (int j = 0; j < RING - 1; ++j) copy_step(j, min(j, last));
  // A ragged tile whose rows all lie in the first half: the waves of the
  // second half copy and meet every barrier but skip their reads and MFMAs,
  // which leaves the matrix units of each SIMD to the other wave.
  const bool live =
      !MOE_GEMM_HALF_SKIP || __builtin_amdgcn_readfirstlane((int)(wm == 0 || rows > BM / 2)) != 0;
  // step s: its copies landed (later steps may still be in flight) ->
  // barrier -> refill the slot of step s-1 with step s+RING-1 -> read step
  // s's fragments -> its MFMAs.  Two waves share each SIMD, so one's MFMAs
  // cover the other's wait, barrier and reads.
  for (int s = 0; s < nk; ++s) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((RING - 2) * OPS));
    wg_barrier();
    copy_step((s + RING - 1) % RING, min(s + RING - 1, last));
    if (!live) continue;
    const char* sl = smem + (s % RING) * SLOT;
    u32x4 af[KH][MT], bf[KH][NT];
#pragma unroll
    for (int h = 0; h < KH; ++h) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        af[h][t] = *reinterpret_cast<const u32x4*>(sl + aoff[h] + t * 16 * RB);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bf[h][t] = *reinterpret_cast<const u32x4*>(sl + boff[h] + t * 16 * RB);
    }
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(af[h][mi]), as_bf16x8(bf[h][ni]), acc[mi][ni], 0, 0, 0);
    if constexpr (KH == 2) {
      // the first half's reads, then each of the second half's reads after
      // one of the first half's MFMAs, then the remaining MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, MT + NT, 0);  // LDS reads
#pragma unroll
      for (int t = 0; t < MT + NT; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * MT * NT - (MT + NT), 0);
    }
  }
  // no copy may still be landing in LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int col = n0 + 64 * wn + 16 * ni + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (BM / 2) * wm + 16 * mi + 4 * g + i;
        if (row < rows && col < F)
          y[(m0 + row) * F + col] = (uint16_t)f32_to_bf16_rne(acc[mi][ni][i]);
      }
    }
}

// fp32: 64 x 64 output tiles of one expert (the tiles numbered expert by
// expert, as above), 256 threads with 4 x 4 outputs each; 16-wide K steps of
// both operands staged through LDS (transposed, so each thread reads its
// four rows' and four outputs' values as float4), fp32 FMAs with h
// ascending -- one sum per output in a fixed order.
constexpr int kF32Tile = 64;
constexpr int kF32K = 16;
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ offsets,
                                                               int E, int64_t T, int H, int F,
                                                               float* __restrict__ y) {
  __shared__ __align__(16) float xs[kF32K][kF32Tile];
  __shared__ __align__(16) float ws[kF32K][kF32Tile];
  __shared__ int s_e, s_rows;
  __shared__ int64_t s_m0;
  __shared__ int s_scan[4];
  if (!tile_of<kF32Tile>(offsets, E, T, (int)blockIdx.x, &s_e, &s_m0, &s_rows, s_scan)) return;
  const int e = s_e;
  const int64_t m0 = s_m0;
  const int rows = s_rows;
  const int n0 = (int)blockIdx.y * kF32Tile;
  const int tid = threadIdx.x;
  // staging: thread -> row (or output) tid / 4, h quarter tid % 4 of the step
  const int lr = tid >> 2, lq = (tid & 3) * 4;
  const float* xrow = x + (m0 + min(lr, rows - 1)) * (int64_t)H;
  const float* wrow = w + ((int64_t)e * F + min(n0 + lr, F - 1)) * (int64_t)H;
  // compute: thread -> rows 4ty..4ty+3, outputs 4tx..4tx+3
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < H; k0 += kF32K) {
    const int kn = min(kF32K, H - k0);  // the ragged last step: fewer FMAs, not zero ones
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int h = k0 + lq + q;
      xs[lq + q][lr] = h < H ? xrow[h] : 0.f;
      ws[lq + q][lr] = h < H ? wrow[h] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&xs[kk][4 * ty]);
      const float4 b = *reinterpret_cast<const float4*>(&ws[kk][4 * tx]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * ty + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = n0 + 4 * tx + j;
      if (f < F) y[(m0 + r) * F + f] = acc[i][j];
    }
  }
}

#ifndef MOE_GEMM_TILE
#define MOE_GEMM_TILE 256   // 256 x 256 output tiles (128 x 128 for small problems)
#endif
#ifndef MOE_GEMM_RING
#define MOE_GEMM_RING 1     // the 4-slot LDS ring kernel for 256 x 256 tiles (H % 32 == 0)
#endif
#ifndef MOE_GEMM_RK64
#define MOE_GEMM_RK64 1     // 256-row ring tiles with 64-wide K steps when H % 64 == 0
#endif
#ifndef MOE_GEMM_RING_BM
#define MOE_GEMM_RING_BM 256  // rows per tile of the ring kernel (256 or 128)
#endif

template <int BM, int BN>
hipError_t launch_gg(const void* x_perm, const void* weight, const int32_t* offsets, int64_t T,
                     int H, int E, int F, void* y, hipStream_t s) {
  // m-tiles: at most ceil(T / BM) + E (one ragged tile per expert); whole
  // groups of kGroupM on each of the 8 XCDs, every n-tile of each
  const int64_t mtiles = (T + BM - 1) / BM + E;
  const int ntn = (F + BN - 1) / BN;
  const int64_t groups = (mtiles + kGroupM - 1) / kGroupM;
  const int64_t blocks = ((groups + 7) / 8) * 8 * kGroupM * ntn;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN>),
                     dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(x_perm),
                     reinterpret_cast<const uint16_t*>(weight), offsets, E, T, H, F, ntn,
                     reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

template <int RBM, int RK>
hipError_t launch_ring(const void* x_perm, const void* weight, const int32_t* offsets, int64_t T,
                       int H, int E, int F, void* y, hipStream_t s) {
  const int64_t mtiles = (T + RBM - 1) / RBM + E;
  const int ntn = (F + 255) / 256;
  const int64_t groups = (mtiles + kGroupM - 1) / kGroupM;
  const int64_t blocks = ((groups + 7) / 8) * 8 * kGroupM * ntn;
  hipLaunchKernelGGL((grouped_gemm_ring_kernel<RBM, RK>), dim3((unsigned)blocks), dim3(512), 0, s,
                     reinterpret_cast<const uint16_t*>(x_perm),
                     reinterpret_cast<const uint16_t*>(weight), offsets, E, T, H, F, ntn,
                     reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_linear(const void* x_perm, const void* weight, const int32_t* offsets,
                                 int64_t T, int H, int E, int F, bool bf16, void* y,
                                 hipStream_t s) {
  if (bf16) {
    // large tiles once every CU gets several of them, small ones otherwise
    const int64_t big = ((T + 255) / 256) * ((F + 255) / 256);
    const bool ring = MOE_GEMM_RING && H % 32 == 0;
    if (MOE_GEMM_TILE == 256 && big >= 1024) {
      if (ring && MOE_GEMM_RK64 && H % 64 == 0)
        return launch_ring<MOE_GEMM_RING_BM, 64>(x_perm, weight, offsets, T, H, E, F, y, s);
      if (ring) return launch_ring<MOE_GEMM_RING_BM, 32>(x_perm, weight, offsets, T, H, E, F, y, s);
      return launch_gg<256, 256>(x_perm, weight, offsets, T, H, E, F, y, s);
    }
    if (ring && MOE_GEMM_SMALL_RING)
      return launch_ring<128, 32>(x_perm, weight, offsets, T, H, E, F, y, s);
    return launch_gg<128, 128>(x_perm, weight, offsets, T, H, E, F, y, s);
  } else {
    const int64_t mtiles = (T + kF32Tile - 1) / kF32Tile + E;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel,
                       dim3((unsigned)mtiles, (unsigned)((F + kF32Tile - 1) / kF32Tile)),
                       dim3(256), 0, s, reinterpret_cast<const float*>(x_perm),
                       reinterpret_cast<const float*>(weight), offsets, E, T, H, F,
                       reinterpret_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
