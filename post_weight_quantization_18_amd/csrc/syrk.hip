// Hessian accumulation H (+)= 2 X^T X on the gfx950 matrix cores.
//
// FDE Interviews breakdown of GPTQ, section 01: the layer-wise objective's
// curvature is H = 2XX^T from the calibration inputs.
//
// Design (MI355X):
//  * Output tiles of 256 (i) x 128 (j) cover the lower triangle only; a
//    workgroup of 8 waves (64 x 64 each, two per SIMD) owns one tile for one
//    token range (split-K when the tile count alone cannot fill 256 CUs).
//  * X is token-major fp16. Each 64-token stage of the tile's I and J feature
//    columns is copied into LDS by the gfx950 direct global->LDS DMA
//    (global_load_lds_dwordx4: lane l lands at bytes [16l, 16l+16) of its
//    wave's 1 KB), row-major with an XOR swizzle of the 16-byte chunks chosen
//    on the global side, into a 3-deep ring, so two stages are in flight while
//    the matrix cores work and no registers hold staged data.
//  * The MFMA operands (8 consecutive tokens per lane) come out of LDS with the
//    transpose read ds_read_b64_tr_b16; the swizzle keeps these reads free of
//    bank conflicts. v_mfma_f32_32x32x16_f16: fp16 x fp16 products are exact.
//  * Accuracy: every W tokens the fp32 accumulators are folded into a second
//    fp32 register (Fast2Sum) and the rounding error is put back into the MFMA
//    accumulator, so the running sum loses nothing to the fold: what remains
//    are the roundings of the W/16 matrix steps inside each window, whose sum
//    over a call of n tokens grows as W / sqrt(n) relative to H. W is chosen
//    per call as 1024 sqrt(n / 262144) rounded down to a power of two within
//    [256, 1024] (1024 from 262144 tokens, 512 from 65536, 256 below), which
//    keeps that error at the level of a 262144-token call with W = 1024 down to
//    16384 tokens. The final value is outer + acc in fp64, and split-K
//    partials are summed in a fixed order in fp64 (deterministic).
#include <mutex>
#include <type_traits>

#include "common.h"

// Scratch of gptq_accumulate_hessian_noalloc: the split-K partial tiles live in
// this file-scope device array instead of a caller workspace. Every GPU the
// library runs on holds its own copy until the process ends. In host code the
// name is only a stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device (see static_scratch).
static __device__ __align__(256) double scratch[gptq::kStaticScratchBytes / sizeof(double)];

namespace gptq {

namespace {

#ifndef GPTQ_SYRK_KS
#define GPTQ_SYRK_KS 64
#endif
#ifndef GPTQ_SYRK_NBUF
#define GPTQ_SYRK_NBUF 3
#endif
constexpr int TI = 256;            // tile rows (i features)
constexpr int TJ = 128;            // tile cols (j features)
constexpr int KS = GPTQ_SYRK_KS;   // tokens per LDS stage
constexpr int kFoldMinTokens = 256, kFoldMaxTokens = 1024;  // fold window W, tokens
#ifndef GPTQ_SYRK_WAVES
#define GPTQ_SYRK_WAVES 8
#endif
constexpr int NW = GPTQ_SYRK_WAVES;   // waves per workgroup: 2 columns of 64 x (NW/2) row bands
constexpr int NT = 64 * NW;           // threads per workgroup
constexpr int FI = TI / (NW / 2) / 32;  // 32-row subtiles per wave (2 or 4)
constexpr int RW = KS / NW;           // token rows each wave moves per stage
constexpr int EI = RW / 2;            // I-tile DMA instructions per wave per stage (2 rows each)
constexpr int EJ = RW / 4;            // J-tile DMA instructions per wave per stage (4 rows each)
constexpr int NBUF = GPTQ_SYRK_NBUF;  // LDS ring depth
static_assert(EI % (KS / 16) == 0 && (EJ % (KS / 16) == 0 || EJ < KS / 16), "DMA spread over the slices");


// Source of the DMA for rows past the token range or features past d: every
// lane issues the same number of loads per stage, so vmcnt waits stay exact.
__device__ const uint4 kZero16[1] = {{0u, 0u, 0u, 0u}};

// s_waitcnt vmcnt(PER * later) for a wave-uniform later in [0, MAXL]; the
// immediate must be a constant, so the count is chosen by a uniform switch.
template <int PER, int MAXL>
__device__ __forceinline__ void wait_vm_stages(int later) {
  static_assert(PER * MAXL < 64, "vmcnt holds at most 63");
  if constexpr (MAXL >= 0) {
    if (later >= MAXL) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((PER * MAXL) & 15) | (((PER * MAXL) >> 4) << 14));
      return;
    }
    if constexpr (MAXL > 0) wait_vm_stages<PER, MAXL - 1>(later);
  }
}

// Work split of one launch over the tile slots (t = 0 .. ntiles-1) and the
// launch's S stages of KS tokens:
//  * slots [0, dp_tiles) (whole rounds of 256): one workgroup per tile over
//    all S stages, written straight into H;
//  * the remaining slots (stream-K): nsk workgroups take equal ranges of W
//    consecutive (slot, stage) units in slot-major order. W < S, so a range
//    covers the end of one tile and at most the start of the next: two
//    segments, each written as an fp64 partial tile to part[(k * 2 + seg)],
//    which syrk_sk_reduce_kernel sums per tile in workgroup order.
// With fewer than 256 tiles the launch instead splits every tile's stages
// into nsplit equal ranges (nsplit * ntiles workgroups, partial tile per
// workgroup, summed by syrk_reduce_kernel): there the workgroups running
// together then stream the same token range, which shares X in the L2, where
// stream-K ranges would start at unrelated tokens.
struct SyrkArgs {
  const half_t* X;
  int64_t ldx, n, d;
  int ntiles, dp_tiles;
  int64_t S, W;     // stages per tile; stages per stream-K workgroup
  int nsplit;       // > 0: token-split mode (dp_tiles = 0)
  int64_t Ssp;      // stages per split
  double* part;     // partial tiles: stream-K [k][2][TI][TJ], split [split][tile][TI][TJ]
  void* H;
  int64_t ldh;
  int h_f64, accumulate;
  int fold_mask;    // W / KS - 1 (W / KS a power of two): fold after stages s with (s + 1) & fold_mask == 0
};

// Tile slot t -> (bi, bj), the same order in the SYRK and in the reductions.
// The tiles of I-block bi are bj = 0 .. 2 bi + 1. Slots run over bands of
// kBand I-blocks (band q: I-blocks r0 = q kBand .. r0 + n - 1, n = kBand but
// for the last band), the tiles before band q numbering r0 (r0 + 1). Inside a
// band the tiles go column by column: columns 0 .. 2 r0 + 1 hold all n rows,
// then come pairs of columns with n - 1, n - 2, .., 1 rows (row bi ends at
// column 2 bi + 1). The 32 workgroups that one XCD runs together (consecutive
// slots) then cover 4 I-blocks x 8 J-blocks, 2048 features of X per stage,
// instead of 1 x 32 (4352 features) in row order, so more of their DMA hits
// that XCD's L2. Tiles past d are empty.
constexpr int kBand = 4;
__device__ inline bool tile_coords(int t, int64_t d, int& bi, int& bj) {
  const int nb = (int)((d + TI - 1) / TI);
  int q = (int)(sqrtf((float)t) / kBand);
  while (q > 0 && (q * kBand) * (q * kBand + 1) > t) --q;
  while (((q + 1) * kBand) * ((q + 1) * kBand + 1) <= t && (q + 1) * kBand < nb) ++q;
  const int r0 = q * kBand, n = nb - r0 < kBand ? nb - r0 : kBand;
  int u = t - r0 * (r0 + 1);
  const int full = (2 * r0 + 2) * n;
  if (u < full) {
    bj = u / n;
    bi = r0 + u % n;
  } else {
    u -= full;
    int p = 0;
    while (u >= 2 * (n - 1 - p)) {
      u -= 2 * (n - 1 - p);
      ++p;
    }
    const int cnt = n - 1 - p;
    bj = 2 * r0 + 2 + 2 * p + u / cnt;
    bi = r0 + 1 + p + u % cnt;
  }
  return (int64_t)bj * TJ < d;
}

__device__ inline short4v tr_read(const half_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS short4v*)(p));
}

// 8 consecutive tokens of one feature per lane: two transpose reads 4 rows apart.
__device__ inline half8 frag(const half_t* p, int pitch) {
  short4v lo = tr_read(p);
  short4v hi = tr_read(p + 4 * pitch);
  short8v both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(half8, both);
}

// LDS chunk (16 B) position of feature chunk c in row r: c ^ 4 (r mod 4).
__device__ inline int swz(int row, int chunk) { return chunk ^ (4 * (row & 3)); }

// XT = false: X token-major [n][ldx] as the caller passes it; the operands
// come out of LDS with transpose reads. XT = true: a.X is the feature-major
// copy X^T [d][ldx] (ldx = a.n = the launch's tokens rounded up to KS, zeros
// past the last token) that syrk_transpose_kernel writes; each lane's 8
// tokens of one feature are 16 contiguous bytes in LDS, read with ds_read_b128.
template <bool XT>
__global__ __launch_bounds__(NT, 1) void syrk_kernel(SyrkArgs a) {
  // ring of NBUF stages; stage buffer b holds the I tile then the J tile
  __shared__ __attribute__((aligned(1024))) half_t ring[NBUF * KS * (TI + TJ)];

  // this workgroup's segments: (slot, first stage, end stage, partial slot or -1 for H)
  int seg_t[2], seg_p[2];
  int64_t seg_s0[2], seg_s1[2];
  int nseg = 0;
  if ((int)blockIdx.x < a.dp_tiles) {
    seg_t[0] = xcd_logical_block(blockIdx.x, a.dp_tiles);
    seg_s0[0] = 0;
    seg_s1[0] = a.S;
    seg_p[0] = -1;
    nseg = 1;
  } else if (a.nsplit > 0) {
    const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = logical / a.ntiles;
    seg_t[0] = logical - split * a.ntiles;
    seg_s0[0] = (int64_t)split * a.Ssp;
    seg_s1[0] = seg_s0[0] + a.Ssp < a.S ? seg_s0[0] + a.Ssp : a.S;
    seg_p[0] = logical;
    nseg = 1;
  } else {
    // consecutive ranges (neighbouring tiles) on one XCD, as for whole tiles
    // (dp_tiles is a multiple of 256, so the XCD of a block is its index mod 8)
    const int k = xcd_logical_block((int)blockIdx.x - a.dp_tiles, (int)gridDim.x - a.dp_tiles);
    const int64_t total = (int64_t)(a.ntiles - a.dp_tiles) * a.S;
    const int64_t b0 = (int64_t)k * a.W;
    const int64_t b1 = b0 + a.W < total ? b0 + a.W : total;
    if (b0 >= total) return;  // uniform
    const int64_t u = b0 / a.S;
    seg_t[0] = a.dp_tiles + (int)u;
    seg_s0[0] = b0 - u * a.S;
    seg_s1[0] = b1 - u * a.S < a.S ? b1 - u * a.S : a.S;
    seg_p[0] = 2 * k;
    nseg = 1;
    if (b1 > (u + 1) * a.S) {
      seg_t[1] = a.dp_tiles + (int)u + 1;
      seg_s0[1] = 0;
      seg_s1[1] = b1 - (u + 1) * a.S;
      seg_p[1] = 2 * k + 1;
      nseg = 2;
    }
  }
  for (int sg = 0; sg < nseg; ++sg) {
  if (sg > 0) __syncthreads();  // every wave is done with the ring
  const int t = seg_t[sg];
  int bi, bj;
  if (!tile_coords(t, a.d, bi, bj)) continue;  // empty slot (uniform)
  GPTQ_DASSERT(bj <= 2 * bi + 1 && (int64_t)bi * TI < a.d && t < a.ntiles);
  const int64_t I0 = (int64_t)bi * TI, J0 = (int64_t)bj * TJ;
  double* const part_out = seg_p[sg] < 0 ? nullptr : a.part + (int64_t)seg_p[sg] * TI * TJ;

  const int64_t tok0 = seg_s0[sg] * KS;
  int64_t tok1 = seg_s1[sg] * KS;
  if (tok1 > a.n) tok1 = a.n;
  const int nstages = tok1 > tok0 ? (int)((tok1 - tok0 + KS - 1) / KS) : 0;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w >> 1, wj = w & 1;  // wave tile: rows 32 FI wi .. + 32 FI - 1, cols 64 wj .. +63
  const bool j_in_i = (J0 >= I0) && (J0 < I0 + TI);

  // ---- DMA of one stage (tokens t0 .. t0+63) into ring buffer b ----
  // I tile: wave w, instruction e covers rows RW w + 2e + {0, 1} (1 KB); lane l
  // takes row RW w + 2e + l/32 and LDS chunk position l%32, holding feature
  // chunk (l%32) ^ 4 (row mod 4). The swizzle depends on e only through e&1.
  // J tile: instruction e covers rows RW w + 4e + {0..3}; lane l takes row
  // RW w + 4e + l/16 and position l%16 (swizzle independent of e).
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index, in an SGPR
  const int rI = lane >> 5, pI = lane & 31, rJ = lane >> 4, pJ = lane & 15;
  const int cI0 = pI ^ (4 * (rI & 3)), cI1 = pI ^ (4 * ((2 + rI) & 3));
  const int cJ = pJ ^ (4 * (rJ & 3));
  const bool okI0 = I0 + 8 * cI0 < a.d, okI1 = I0 + 8 * cI1 < a.d, okJ = J0 + 8 * cJ < a.d;
  const int64_t offI0 = (int64_t)(RW * w + rI) * a.ldx + I0 + 8 * cI0;
  const int64_t offI1 = (int64_t)(RW * w + rI) * a.ldx + I0 + 8 * cI1;
  const int64_t offJ = (int64_t)(RW * w + rJ) * a.ldx + J0 + 8 * cJ;
  const bool tile_inside = (I0 + TI <= a.d) && (J0 + TJ <= a.d);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GPTQ_LDS void*)ring);
  constexpr uint32_t STAGE_BYTES = KS * (TI + TJ) * 2;
  // instruction e (0 .. EI-1) of the I tile and (0 .. EJ-1) of the J tile for
  // the stage starting at token t0 into ring buffer b
  // XT layout: 16-byte slot s of a tile holds feature s / 8 and token chunk
  // (s % 8) ^ sw(s / 8), sw(i) = (i % 8) ^ ((i / 8) % 2): DMA instruction e of
  // wave w fills slots 64 (w E + e) + l, i.e. feature 8 (w E + e) + l / 8 and
  // chunk (l % 8) ^ (l / 8) ^ ((w E + e) % 2); the fragment reads of 16
  // consecutive features then touch 16 different 16-byte bank groups.
  const int xfeat = lane >> 3, xchunk = (lane & 7) ^ (lane >> 3);
  const int64_t xbaseI = (I0 + 8 * (wu * EI) + xfeat) * a.ldx;
  const int64_t xbaseJ = (J0 + 8 * (wu * EJ) + xfeat) * a.ldx;
  auto issue_I_xt = [&](int e, int64_t t0, int b) __attribute__((always_inline)) {
    const int64_t fi = I0 + 8 * (wu * EI + e) + xfeat;
    const int c = xchunk ^ ((wu * EI + e) & 1);
    const half_t* src = (tile_inside || fi < a.d) ? a.X + xbaseI + (int64_t)(8 * e) * a.ldx + t0 + 8 * c
                                                  : (const half_t*)kZero16;
    GPTQ_DASSERT(src == (const half_t*)kZero16 || (src >= a.X && src + 8 <= a.X + (a.d - 1) * a.ldx + a.n));
    dma16(src, ring_lds + b * STAGE_BYTES + (uint32_t)((wu * EI + e) * 1024));
  };
  auto issue_J_xt = [&](int e, int64_t t0, int b) __attribute__((always_inline)) {
    const int64_t fj = J0 + 8 * (wu * EJ + e) + xfeat;
    const int c = xchunk ^ ((wu * EJ + e) & 1);
    const half_t* src = (tile_inside || fj < a.d) ? a.X + xbaseJ + (int64_t)(8 * e) * a.ldx + t0 + 8 * c
                                                  : (const half_t*)kZero16;
    GPTQ_DASSERT(src == (const half_t*)kZero16 || (src >= a.X && src + 8 <= a.X + (a.d - 1) * a.ldx + a.n));
    dma16(src, ring_lds + b * STAGE_BYTES + KS * TI * 2 + (uint32_t)((wu * EJ + e) * 1024));
  };
  auto issue_I = [&](int e, int64_t t0, int b, bool full) __attribute__((always_inline)) {
    if constexpr (XT) {
      issue_I_xt(e, t0, b);
      return;
    }
    // row RW w + 2e + l/32; offI0 / offI1 carry row RW w + l/32 and the chunk
    // swizzle of the row's parity class (e even / odd)
    const half_t* src = a.X + t0 * a.ldx + (int64_t)(2 * e) * a.ldx + ((e & 1) ? offI1 : offI0);
    if (!full) {
      const int rows = (int)((tok1 - t0) < KS ? (tok1 - t0) : KS);
      const bool ok = ((e & 1) ? okI1 : okI0) && (RW * w + 2 * e + rI) < rows;
      if (!ok) src = (const half_t*)kZero16;
    }
    GPTQ_DASSERT(src == (const half_t*)kZero16 || (src >= a.X && src + 8 <= a.X + (a.n - 1) * a.ldx + a.d));
    dma16(src, ring_lds + b * STAGE_BYTES + (uint32_t)((RW * wu + 2 * e) * TI * 2));
  };
  auto issue_J = [&](int e, int64_t t0, int b, bool full) __attribute__((always_inline)) {
    if constexpr (XT) {
      issue_J_xt(e, t0, b);
      return;
    }
    const half_t* src = a.X + t0 * a.ldx + (int64_t)(4 * e) * a.ldx + offJ;
    if (!full) {
      const int rows = (int)((tok1 - t0) < KS ? (tok1 - t0) : KS);
      const bool ok = okJ && (RW * w + 4 * e + rJ) < rows;
      if (!ok) src = (const half_t*)kZero16;
    }
    GPTQ_DASSERT(src == (const half_t*)kZero16 || (src >= a.X && src + 8 <= a.X + (a.n - 1) * a.ldx + a.d));
    dma16(src, ring_lds + b * STAGE_BYTES + KS * TI * 2 + (uint32_t)((RW * wu + 4 * e) * TJ * 2));
  };
  auto issue = [&](int64_t t0, int b) __attribute__((always_inline)) {
    const bool full = tile_inside && t0 + KS <= tok1;
#pragma unroll
    for (int e = 0; e < EI; ++e) issue_I(e, t0, b, full);
    if (!j_in_i) {
#pragma unroll
      for (int e = 0; e < EJ; ++e) issue_J(e, t0, b, full);
    }
  };

  // ---- per-lane transpose-read offsets (halves) ----
  // lane: g = lane/16, e = (lane/4)%4, q = lane%4 reads token row 8(g/2) + e and
  // features base + 16(g%2) + 4q; the row's swizzle is 4e.
  const int g = lane >> 4, e4 = (lane >> 2) & 3, q = lane & 3;
  const int tokoff = 8 * (g >> 1) + e4;
  const int sub = 2 * (g & 1) + (q >> 1), halfsel = 4 * (q & 1);
  int offA[FI], offB[2];
#pragma unroll
  for (int f = 0; f < FI; ++f) offA[f] = tokoff * TI + (swz(tokoff, wi * 4 * FI + 4 * f + sub) << 3) + halfsel;
  const int bpitch = j_in_i ? TI : TJ;
  const int bchunk0 = j_in_i ? (int)((J0 - I0) / 8) : 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) offB[h] = tokoff * bpitch + (swz(tokoff, bchunk0 + wj * 8 + 4 * h + sub) << 3) + halfsel;
  // XT reads: row l % 32 of each 32-feature sub-tile (KS halves per feature),
  // chunk position (2 kk) ^ xv; B of a diagonal tile sits at feature J0 - I0 of the I tile
  const int xrow = (lane & 31) * KS;
  const int xv = (lane >> 5) ^ ((lane & 7) ^ ((lane >> 3) & 1));
  const int xboff = j_in_i ? (int)(J0 - I0) : 0;

  float16v acc[FI][2], outer[FI][2];
#pragma unroll
  for (int f = 0; f < FI; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[f][h][r] = 0.0f;
        outer[f][h][r] = 0.0f;
      }

  auto fold = [&]() __attribute__((always_inline)) {
    // Fast2Sum(outer, acc): outer <- fl(outer + acc), acc <- exact residual.
#pragma unroll
    for (int f = 0; f < FI; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float o = outer[f][h][r], c = acc[f][h][r];
          float sum = o + c;
          float z = sum - o;
          acc[f][h][r] = c - z;
          outer[f][h][r] = sum;
        }
        // one 32 x 32 sub-tile at a time keeps the temporaries to 16 registers
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  auto stage_i = [&](int b) __attribute__((always_inline)) { return ring + b * KS * (TI + TJ); };
  auto stage_j = [&](int b) __attribute__((always_inline)) { return ring + b * KS * (TI + TJ) + KS * TI; };

  // prologue: the first NBUF - 1 stages in flight
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nstages) issue(tok0 + (int64_t)p * KS, p);

  // Stage s uses ring buffer s mod NBUF and is cut into KS/16 slices of 16
  // tokens. Slice k issues its share of the DMA of stage s + NBUF - 1 (into the
  // buffer stage s - 1 used), then the fragment reads of slice k + 1, and only
  // then its own matrix-core work, so every read has a whole slice of MFMAs to
  // land. The last slice instead waits for stage s + 1's DMA, passes the
  // workgroup barrier and reads stage s + 1's first slice: the barrier and that
  // read are hidden behind the last slice's MFMAs, and once every wave is past
  // it no wave reads buffer s again, so stage s + 1 may refill it.
  // The stage loop is instantiated once per tile kind (diagonal tiles read B
  // from the I buffer): a branch inside the loop would make the compiler merge
  // the accumulators of the two paths with register copies on every stage.
  static_assert((KS / 16) % 2 == 0, "fragment slots alternate within a stage");
  auto stage_loop = [&](auto diag_tag) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    constexpr int PER = DIAG ? EI : EI + EJ;  // DMA instructions per wave per stage
    constexpr int bp = DIAG ? TI : TJ;
    auto buf_b = [&](int b) __attribute__((always_inline)) { return DIAG ? stage_i(b) : stage_j(b); };
    half8 af[2][FI], bf[2][2];
    auto read_slice = [&](int b, int kk, int slot) __attribute__((always_inline)) {
      if constexpr (XT) {
        // lane l: feature (sub-tile base) + l % 32, token chunk 2 kk + l / 32 at
        // position (2 kk + l / 32) ^ sw = (2 kk) ^ xv of the feature's 64 halves
        const int pos = 8 * ((2 * kk) ^ xv);
#pragma unroll
        for (int f = 0; f < FI; ++f)
          af[slot][f] = *(const GPTQ_LDS half8*)(stage_i(b) + (wi * 32 * FI + f * 32) * KS + xrow + pos);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          bf[slot][h] = *(const GPTQ_LDS half8*)(buf_b(b) + (xboff + wj * 64 + h * 32) * KS + xrow + pos);
      } else {
#pragma unroll
        for (int f = 0; f < FI; ++f) af[slot][f] = frag(stage_i(b) + offA[f] + kk * 16 * TI, TI);
#pragma unroll
        for (int h = 0; h < 2; ++h) bf[slot][h] = frag(buf_b(b) + offB[h] + kk * 16 * bp, bp);
      }
    };
    // stage s's DMA has landed for every wave once at most the later stages'
    // loads (up to NBUF - 2 stages of PER loads each) remain in flight
    auto wait_stage = [&](int st) __attribute__((always_inline)) {
      const int later = (nstages - 1 - st) < (NBUF - 2) ? (nstages - 1 - st) : (NBUF - 2);
      wait_vm_stages<PER, NBUF - 2>(later);
      lds_barrier();
    };
    if (nstages > 0) {
      wait_stage(0);
      read_slice(0, 0, 0);
    }
    int cur = 0;
    for (int s = 0; s < nstages; ++s) {
      const int nxt = cur == 0 ? NBUF - 1 : cur - 1;  // the buffer stage s - 1 used
      const int cnext = cur == NBUF - 1 ? 0 : cur + 1;
      const bool refill = s + NBUF - 1 < nstages;
      const int64_t t_next = tok0 + (int64_t)(s + NBUF - 1) * KS;
      const bool full = tile_inside && t_next + KS <= tok1;
#pragma unroll
      for (int kk = 0; kk < KS / 16; ++kk) {
        if (refill) {
          constexpr int PI = EI / (KS / 16), PJ = EJ >= KS / 16 ? EJ / (KS / 16) : 1;
#pragma unroll
          for (int e = 0; e < PI; ++e) issue_I(kk * PI + e, t_next, nxt, full);
          if (!DIAG && kk * PJ < EJ) {
#pragma unroll
            for (int e = 0; e < PJ; ++e) issue_J(kk * PJ + e, t_next, nxt, full);
          }
        }
        if (kk + 1 < KS / 16) {
          read_slice(cur, kk + 1, (kk + 1) & 1);
        } else {
          // after the last stage this waits for nothing and reads a buffer
          // that is never used; unconditional, so the read counters the
          // compiler tracks stay exact
          wait_stage(s + 1);
          read_slice(cnext, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int slot = kk & 1;
#pragma unroll
        for (int f = 0; f < FI; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[f][h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[slot][f], bf[slot][h], acc[f][h], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (((s + 1) & a.fold_mask) == 0) fold();
      cur = cnext;
    }
  };
  if (j_in_i)
    stage_loop(std::true_type{});
  else
    stage_loop(std::false_type{});

  // ---- epilogue ----
  // One 32 x 32 sub-tile at a time: all old H values of the sub-tile are read
  // before any is written, so the read-modify-write costs one memory round
  // trip per sub-tile instead of one per element.
  const int hl = lane >> 5, col = lane & 31;
#pragma unroll
  for (int f = 0; f < FI; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      double v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = 2.0 * ((double)outer[f][h][r] + (double)acc[f][h][r]);
      const int li0 = wi * 32 * FI + f * 32 + 4 * hl, lj = wj * 64 + h * 32 + col;
      if (part_out) {
#pragma unroll
        for (int r = 0; r < 16; ++r) part_out[(int64_t)(li0 + 8 * (r >> 2) + (r & 3)) * TJ + lj] = v[r];
        continue;
      }
      const int64_t j = J0 + lj;
      if (a.accumulate) {
        double old[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = I0 + li0 + 8 * (r >> 2) + (r & 3);
          const bool ok = i < a.d && j <= i;
          old[r] = !ok ? 0.0 : a.h_f64 ? ((const double*)a.H)[i * a.ldh + j]
                                        : (double)((const float*)a.H)[i * a.ldh + j];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += old[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = I0 + li0 + 8 * (r >> 2) + (r & 3);
        if (i < a.d && j <= i) {
          if (a.h_f64)
            ((double*)a.H)[i * a.ldh + j] = v[r];
          else
            ((float*)a.H)[i * a.ldh + j] = (float)v[r];
        }
      }
    }
  }  // segments
}

// X^T for the XT form: X token-major [nc][ldx] -> XT feature-major [d][T],
// T = nc rounded up to KS, zeros at tokens nc .. T-1. 64 x 64 tiles through
// LDS; 16-byte loads of 8 features of a token, 16-byte stores of 8 tokens of a
// feature.
__global__ __launch_bounds__(256) void syrk_transpose_kernel(const half_t* __restrict__ X, int64_t ldx, int64_t nc,
                                                             int64_t d, half_t* __restrict__ XT, int64_t T) {
  __shared__ half_t tile[64][64 + 8];
  const int64_t t0 = (int64_t)blockIdx.x * 64, f0 = (int64_t)blockIdx.y * 64;
  const int r = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t tok = t0 + r + 32 * pass, f = f0 + c8;
    half8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (tok < nc && f < d) v = *(const half8*)(X + tok * ldx + f);  // d % 32 == 0: f < d means f + 8 <= d
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[c8 + e][r + 32 * pass] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int fr = r + 32 * pass;
    const int64_t f = f0 + fr;
    if (f < d) {
      half8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[fr][c8 + e];
      GPTQ_DASSERT(t0 + c8 + 8 <= T);
      *(half8*)(XT + f * T + t0 + c8) = v;
    }
  }
}

// Token-split mode: H (+)= the sum of the tile's partials in split order.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const double* __restrict__ part, int nsplit,
                                                          int ntiles, void* Hout, int64_t d, int64_t ldh,
                                                          int h_f64, int accumulate) {
  const int64_t per_tile = (int64_t)TI * TJ;
  const int64_t total = (int64_t)ntiles * per_tile;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx / per_tile);
    const int64_t within = idx - (int64_t)t * per_tile;
    int bi, bj;
    if (!tile_coords(t, d, bi, bj)) continue;
    const int64_t i = (int64_t)bi * TI + within / TJ, j = (int64_t)bj * TJ + within % TJ;
    if (i >= d || j > i) continue;
    double s = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) s += part[((int64_t)sp * ntiles + t) * per_tile + within];
    if (h_f64) {
      double* H = (double*)Hout + i * ldh + j;
      *H = accumulate ? *H + s : s;
    } else {
      float* H = (float*)Hout + i * ldh + j;
      *H = (float)(accumulate ? (double)*H + s : s);
    }
  }
}

// Stream-K tiles: H (+)= the sum, in workgroup order, of the partial tiles of
// the workgroups whose ranges cover the tile (see SyrkArgs).
__global__ __launch_bounds__(256) void syrk_sk_reduce_kernel(const double* __restrict__ part, int dp_tiles,
                                                             int sk_tiles, int64_t S, int64_t W, int nsk,
                                                             void* Hout, int64_t d, int64_t ldh, int h_f64,
                                                             int accumulate) {
  const int64_t per_tile = (int64_t)TI * TJ;
  const int64_t total = (int64_t)sk_tiles * per_tile;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int u = (int)(idx / per_tile);
    const int64_t within = idx - (int64_t)u * per_tile;
    int bi, bj;
    if (!tile_coords(dp_tiles + u, d, bi, bj)) continue;
    const int64_t i = (int64_t)bi * TI + within / TJ, j = (int64_t)bj * TJ + within % TJ;
    if (i >= d || j > i) continue;
    const int64_t kf = ((int64_t)u * S) / W;
    int64_t kl = ((int64_t)(u + 1) * S - 1) / W;
    if (kl > nsk - 1) kl = nsk - 1;
    double s = 0.0;
    for (int64_t k = kf; k <= kl; ++k) {
      const int seg = (k * W) / S == u ? 0 : 1;  // the tile is k's first or second segment
      s += part[(k * 2 + seg) * per_tile + within];
    }
    if (h_f64) {
      double* H = (double*)Hout + i * ldh + j;
      *H = accumulate ? *H + s : s;
    } else {
      float* H = (float*)Hout + i * ldh + j;
      *H = (float)(accumulate ? (double)*H + s : s);
    }
  }
}

// Zeroes (or keeps) the lower triangle when there are no tokens.
__global__ void syrk_zero_kernel(void* H, int64_t d, int64_t ldh, int h_f64) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < d * d;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t i = idx / d, j = idx % d;
    if (j > i) continue;
    if (h_f64)
      ((double*)H)[i * ldh + j] = 0.0;
    else
      ((float*)H)[i * ldh + j] = 0.0f;
  }
}

int syrk_ntiles(int64_t d) {
  const int64_t T = ceil_div(d, TI);
  return (int)(T * (T + 1));
}

constexpr int64_t kLaunchTokens = 65536;
constexpr int64_t kXtMinD = 12288;     // the feature-major form from this width on
constexpr int kSkMax = 256;            // stream-K workgroups: one round
constexpr int64_t kSkMinStages = 16;   // at least 1024 tokens per stream-K range

// Tokens per launch: with whole rounds of tiles to run (ntiles >= 256) a long
// token range is cut into launches of kLaunchTokens, which bounds the
// feature-major copy in the workspace (d x 65536 fp16); otherwise one launch
// takes them all. Measured over 262144 tokens: at d = 49152 launches of 65536
// tokens take 1.4 % less than launches of 32768 (one launch of all 262144
// 1.8 % less, with a 25.8 GB copy); at d = 12288 they are even.
int64_t syrk_launch_tokens(int64_t d, int64_t n) {
  return (syrk_ntiles(d) >= kSkMax && n > 2 * kLaunchTokens) ? kLaunchTokens : n;
}

// Real (non-empty) tiles of the lower triangle at width d.
int syrk_real_tiles(int64_t d) {
  const int64_t ti = ceil_div(d, TI), tj = ceil_div(d, TJ);
  int64_t n = 0;
  for (int64_t bi = 0; bi < ti; ++bi) n += (2 * bi + 2 < tj ? 2 * bi + 2 : tj);
  return (int)n;
}

// Token split for fewer than 256 tiles: minimises an estimate of the call's
// time, ceil(tiles * s / 256) rounds x (stages per split + 4) stage times +
// the fp64 partial tiles written and read back; a split must win by 10%.
int syrk_choose_split(int64_t d, int64_t n) {
  const int64_t stages = ceil_div(n, KS);
  const int tiles = syrk_real_tiles(d);
  if (stages <= 1) return 1;
  const double stage_us = 0.45 * KS / 64.0;
  const double partial_us_per_tile = 2.0 * TI * TJ * 8 / 4.0e6;  // write + read at ~4 TB/s
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= 64 && s <= stages; ++s) {
    const int64_t rounds = ceil_div((int64_t)tiles * s, 256);
    const double t = (double)rounds * ((double)ceil_div(stages, s) + 4.0) * stage_us +
                     (s > 1 ? (double)s * tiles * partial_us_per_tile : 0.0);
    if (t < best_t * 0.90) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

struct SkPlan {
  int dp_tiles, sk_tiles, nsk;
  int64_t S, W;
  int nsplit;  // > 0: token-split mode
  int64_t Ssp;
};

SkPlan sk_plan(int64_t d, int64_t n_launch) {
  SkPlan p;
  const int nt = syrk_ntiles(d);
  p.S = ceil_div(n_launch, KS);
  p.nsplit = 0;
  p.Ssp = 0;
  if (nt < kSkMax) {
    const int s = syrk_choose_split(d, n_launch);
    p.dp_tiles = 0;
    p.sk_tiles = 0;
    p.nsk = 0;
    p.W = 0;
    if (s <= 1) {
      p.dp_tiles = nt;  // one workgroup per tile, straight into H
    } else {
      p.Ssp = ceil_div(p.S, s);
      p.nsplit = (int)ceil_div(p.S, p.Ssp);
    }
    return p;
  }
  p.dp_tiles = nt / kSkMax * kSkMax;
  p.sk_tiles = nt - p.dp_tiles;
  const int64_t units = (int64_t)p.sk_tiles * p.S;
  if (units == 0) {
    p.nsk = 0;
    p.W = 0;
    return p;
  }
  // W stages per workgroup: a share of one round, at least kSkMinStages, and
  // at most S, so that a range touches two tiles at most
  int64_t W = ceil_div(units, kSkMax);
  const int64_t lo = kSkMinStages < p.S ? kSkMinStages : p.S;
  if (W < lo) W = lo;
  if (W > p.S) W = p.S;
  p.W = W;
  p.nsk = (int)ceil_div(units, W);  // <= 256: units <= 255 S
  return p;
}

}  // namespace

namespace {
// Partial tiles of one launch of n_launch tokens (256-byte aligned).
size_t syrk_partial_bytes(const SkPlan& p, int64_t d) {
  const size_t b = p.nsplit > 0 ? (size_t)p.nsplit * syrk_ntiles(d) * TI * TJ * sizeof(double)
                                : (size_t)p.nsk * 2 * TI * TJ * sizeof(double);
  return (b + 255) / 256 * 256;
}
// The feature-major copy of one launch's tokens.
size_t syrk_xt_bytes(int64_t d, int64_t n_launch) { return (size_t)d * (size_t)ceil_div(n_launch, KS) * KS * 2; }
}  // namespace

size_t syrk_workspace_bytes(int64_t d, int64_t n) {
  if (n <= 0) return 0;
  const int64_t nl = syrk_launch_tokens(d, n);
  return syrk_partial_bytes(sk_plan(d, nl), d) + (d >= kXtMinD ? syrk_xt_bytes(d, nl) : 0);
}

size_t syrk_partials_workspace_bytes(int64_t d, int64_t n) {
  if (n <= 0) return 0;
  return syrk_partial_bytes(sk_plan(d, syrk_launch_tokens(d, n)), d);
}

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch` per device, 0 until first use
}  // namespace

gptq_status_t static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GPTQ_ERR_HIP;
  if (dev >= kScratchDevices) return GPTQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPTQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GPTQ_OK;
}

namespace {
// Fold window W of a call of n tokens (see the accuracy note at the top).
int syrk_fold_tokens(int64_t n) {
  int w = kFoldMaxTokens;
  while (w > kFoldMinTokens && (double)w * w * 262144.0 > (double)kFoldMaxTokens * kFoldMaxTokens * (double)n) w /= 2;
  return w;
}

gptq_status_t syrk_enqueue_launches(void* H, int h_f64, int64_t d, int64_t ldh, const half_t* X, int64_t n,
                                    int64_t ldx, int accumulate, void* ws, size_t ws_bytes, hipStream_t st,
                                    bool allow_xt, int fold_tokens) {
  const int nt = syrk_ntiles(d);
  if (n == 0) {
    if (!accumulate) {
      TraceScope tr(st, GPTQ_TRACE_SYRK_REDUCE);
      hipLaunchKernelGGL(syrk_zero_kernel, dim3(1024), dim3(256), 0, st, H, d, ldh, h_f64);
      GPTQ_CHECK_LAUNCH();
    }
    return GPTQ_OK;
  }
  const int64_t nl = syrk_launch_tokens(d, n);
  if (nl < n) {
    for (int64_t t0 = 0; t0 < n; t0 += nl) {
      const int64_t nc = n - t0 < nl ? n - t0 : nl;
      gptq_status_t s = syrk_enqueue_launches(H, h_f64, d, ldh, X + t0 * ldx, nc, ldx, accumulate || t0 > 0, ws,
                                              ws_bytes, st, allow_xt, fold_tokens);
      if (s != GPTQ_OK) return s;
    }
    return GPTQ_OK;
  }
  SkPlan p = sk_plan(d, n);
  const size_t need = syrk_partial_bytes(p, d);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    // no room for the partial tiles: every tile gets one workgroup
    p.dp_tiles = nt;
    p.sk_tiles = 0;
    p.nsk = 0;
    p.nsplit = 0;
  }
  const size_t part_bytes = syrk_partial_bytes(p, d);
  // the feature-major copy when the workspace holds it after the partials and
  // d is wide enough to repay the transpose (measured with the banded tile
  // order: 3.8 % faster at d = 12288; 13 % slower at d = 2560 in row order)
  const bool xt = allow_xt && d >= kXtMinD && ws != nullptr && ws_bytes >= part_bytes + syrk_xt_bytes(d, n);
  const int64_t Tpad = ceil_div(n, KS) * KS;
  half_t* XT = xt ? (half_t*)((char*)ws + part_bytes) : nullptr;
  if (xt) {
    TraceScope tr(st, GPTQ_TRACE_SYRK_TRANSPOSE);
    hipLaunchKernelGGL(syrk_transpose_kernel, dim3((unsigned)(Tpad / 64), (unsigned)ceil_div(d, 64)), dim3(256), 0,
                       st, X, ldx, n, d, XT, Tpad);
    GPTQ_CHECK_LAUNCH();
  }
  SyrkArgs a;
  a.X = xt ? XT : X;
  a.ldx = xt ? Tpad : ldx;
  a.n = xt ? Tpad : n;
  a.d = d;
  a.ntiles = nt;
  a.dp_tiles = p.dp_tiles;
  a.S = p.S;
  a.W = p.W;
  a.nsplit = p.nsplit;
  a.Ssp = p.Ssp;
  a.part = (double*)ws;
  a.H = H;
  a.ldh = ldh;
  a.h_f64 = h_f64;
  a.accumulate = accumulate;
  a.fold_mask = fold_tokens / KS - 1;
  {
    // executed: every non-empty tile over the launch's stages (diagonal tiles whole)
    const int64_t T = ceil_div(d, TI), Tj = ceil_div(d, TJ);
    int64_t live = 0;
    for (int64_t bi = 0; bi < T; ++bi) live += (2 * bi + 2 < Tj ? 2 * bi + 2 : Tj);
    TraceScope tr(st, GPTQ_TRACE_SYRK, 2.0 * TI * TJ * (double)(p.S * KS) * (double)live);
    const dim3 grid(p.nsplit > 0 ? p.nsplit * nt : p.dp_tiles + p.nsk);
    if (xt)
      hipLaunchKernelGGL(syrk_kernel<true>, grid, dim3(NT), 0, st, a);
    else
      hipLaunchKernelGGL(syrk_kernel<false>, grid, dim3(NT), 0, st, a);
    GPTQ_CHECK_LAUNCH();
  }
  TraceScope tr_reduce(st, GPTQ_TRACE_SYRK_REDUCE);
  if (p.nsplit > 0) {
    const int64_t total = (int64_t)nt * TI * TJ;
    int blocks = (int)ceil_div(total, 256 * 4);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(blocks), dim3(256), 0, st, (const double*)ws, p.nsplit, nt, H, d,
                       ldh, h_f64, accumulate);
    GPTQ_CHECK_LAUNCH();
  }
  if (p.nsk > 0) {
    const int64_t total = (int64_t)p.sk_tiles * TI * TJ;
    int blocks = (int)ceil_div(total, 256 * 4);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(syrk_sk_reduce_kernel, dim3(blocks), dim3(256), 0, st, (const double*)ws, p.dp_tiles,
                       p.sk_tiles, p.S, p.W, p.nsk, H, d, ldh, h_f64, accumulate);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}
}  // namespace

gptq_status_t syrk_enqueue(void* H, int h_f64, int64_t d, int64_t ldh, const half_t* X, int64_t n,
                           int64_t ldx, int accumulate, void* ws, size_t ws_bytes, hipStream_t st, bool allow_xt) {
  // the fold window follows the whole call's token count, not one launch's
  return syrk_enqueue_launches(H, h_f64, d, ldh, X, n, ldx, accumulate, ws, ws_bytes, st, allow_xt,
                               syrk_fold_tokens(n));
}

}  // namespace gptq
