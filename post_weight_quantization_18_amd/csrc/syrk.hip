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
//  * Accuracy: every 1024 tokens the fp32 accumulators are folded into a
//    second fp32 register (Fast2Sum) and the rounding error is put back into the
//    MFMA accumulator, so the partial sum is carried to ~2^-48 relative; the
//    final value is outer + acc in fp64, and split-K partials are summed in a
//    fixed order in fp64 (deterministic).
#include <type_traits>

#include "common.h"

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
constexpr int FOLD = 1024 / KS;    // stages between error folds (1024 tokens)
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

struct SyrkArgs {
  const half_t* X;
  int64_t ldx, n, d;
  int64_t tokens_per_split;
  int nsplit, ntiles;
  void* out;        // H (direct) or fp64 partial tiles
  int64_t ldh;
  int h_f64, accumulate, direct;
};

// Tile t -> (bi, bj): the tiles of I-block bi are bj = 0 .. 2 bi + 1, so t lies
// in [bi (bi + 1), (bi + 1)(bi + 2)). Consecutive tiles (which one XCD runs
// together) share their I columns. Tiles past d are empty.
__device__ inline bool tile_coords(int t, int64_t d, int& bi, int& bj) {
  int b = (int)((sqrtf(4.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((b + 1) * (b + 2) <= t) ++b;
  while (b * (b + 1) > t) --b;
  bi = b;
  bj = t - b * (b + 1);
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

__global__ __launch_bounds__(NT, 1) void syrk_kernel(SyrkArgs a) {
  // ring of NBUF stages; stage buffer b holds the I tile then the J tile
  __shared__ __attribute__((aligned(1024))) half_t ring[NBUF * KS * (TI + TJ)];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int split = logical / a.ntiles;
  const int t = logical - split * a.ntiles;
  int bi, bj;
  if (!tile_coords(t, a.d, bi, bj)) return;  // empty slot: the workgroup exits (uniform)
  const int64_t I0 = (int64_t)bi * TI, J0 = (int64_t)bj * TJ;

  const int64_t tok0 = (int64_t)split * a.tokens_per_split;
  int64_t tok1 = tok0 + a.tokens_per_split;
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
  auto issue_I = [&](int e, int64_t t0, int b, bool full) __attribute__((always_inline)) {
    // row RW w + 2e + l/32; offI0 / offI1 carry row RW w + l/32 and the chunk
    // swizzle of the row's parity class (e even / odd)
    const half_t* src = a.X + t0 * a.ldx + (int64_t)(2 * e) * a.ldx + ((e & 1) ? offI1 : offI0);
    if (!full) {
      const int rows = (int)((tok1 - t0) < KS ? (tok1 - t0) : KS);
      const bool ok = ((e & 1) ? okI1 : okI0) && (RW * w + 2 * e + rI) < rows;
      if (!ok) src = (const half_t*)kZero16;
    }
    dma16(src, ring_lds + b * STAGE_BYTES + (uint32_t)((RW * wu + 2 * e) * TI * 2));
  };
  auto issue_J = [&](int e, int64_t t0, int b, bool full) __attribute__((always_inline)) {
    const half_t* src = a.X + t0 * a.ldx + (int64_t)(4 * e) * a.ldx + offJ;
    if (!full) {
      const int rows = (int)((tok1 - t0) < KS ? (tok1 - t0) : KS);
      const bool ok = okJ && (RW * w + 4 * e + rJ) < rows;
      if (!ok) src = (const half_t*)kZero16;
    }
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
#pragma unroll
      for (int f = 0; f < FI; ++f) af[slot][f] = frag(stage_i(b) + offA[f] + kk * 16 * TI, TI);
#pragma unroll
      for (int h = 0; h < 2; ++h) bf[slot][h] = frag(buf_b(b) + offB[h] + kk * 16 * bp, bp);
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
      if ((s + 1) % FOLD == 0) fold();
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
      if (!a.direct) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ((double*)a.out)[((int64_t)logical * TI + li0 + 8 * (r >> 2) + (r & 3)) * TJ + lj] = v[r];
        continue;
      }
      const int64_t j = J0 + lj;
      if (a.accumulate) {
        double old[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = I0 + li0 + 8 * (r >> 2) + (r & 3);
          const bool ok = i < a.d && j <= i;
          old[r] = !ok ? 0.0 : a.h_f64 ? ((const double*)a.out)[i * a.ldh + j]
                                        : (double)((const float*)a.out)[i * a.ldh + j];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += old[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = I0 + li0 + 8 * (r >> 2) + (r & 3);
        if (i < a.d && j <= i) {
          if (a.h_f64)
            ((double*)a.out)[i * a.ldh + j] = v[r];
          else
            ((float*)a.out)[i * a.ldh + j] = (float)v[r];
        }
      }
    }
}

// Sums the split-K partial tiles in split order and adds them to H.
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

// Real (non-empty) tiles of the lower triangle at width d.
int syrk_real_tiles(int64_t d) {
  const int64_t ti = ceil_div(d, TI), tj = ceil_div(d, TJ);
  int64_t n = 0;
  for (int64_t bi = 0; bi < ti; ++bi) n += (2 * bi + 2 < tj ? 2 * bi + 2 : tj);
  return (int)n;
}

// Token split S: minimises an estimate of the call's time,
//   ceil(tiles * S / 256) rounds x (stages per split + 4) stage times
//   + the fp64 partial tiles written and read back (S > 1),
// with one workgroup per CU (the LDS ring takes most of a CU's LDS).
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
    if (t < best_t * 0.90) {  // a split must win clearly: partials cost more than modelled
      best_t = t;
      best = s;
    }
  }
  return best;
}

}  // namespace

size_t syrk_workspace_bytes(int64_t d, int64_t n) {
  const int nt = syrk_ntiles(d);
  const int s = syrk_choose_split(d, n);
  if (s <= 1) return 0;
  return (size_t)s * (size_t)nt * TI * TJ * sizeof(double);
}

constexpr int64_t kLaunchTokens = 32768;

gptq_status_t syrk_enqueue(void* H, int h_f64, int64_t d, int64_t ldh, const half_t* X, int64_t n,
                           int64_t ldx, int accumulate, void* ws, size_t ws_bytes, hipStream_t st) {
  const int nt = syrk_ntiles(d);
  if (n == 0) {
    if (!accumulate) {
      hipLaunchKernelGGL(syrk_zero_kernel, dim3(1024), dim3(256), 0, st, H, d, ldh, h_f64);
      GPTQ_CHECK_LAUNCH();
    }
    return GPTQ_OK;
  }
  int split = syrk_choose_split(d, n);
  const size_t per_split = (size_t)nt * TI * TJ * sizeof(double);
  if (split > 1 && (ws == nullptr || ws_bytes < (size_t)split * per_split)) {
    split = ws ? (int)(ws_bytes / per_split) : 1;
    if (split < 1) split = 1;
  }
  if (split == 1 && n > 2 * kLaunchTokens) {
    // without a token split the tiles already fill the GPU: cut the token
    // range into launches of kLaunchTokens (measured faster at d = 12288 than
    // one long launch), each adding into H
    for (int64_t t0 = 0; t0 < n; t0 += kLaunchTokens) {
      const int64_t nc = n - t0 < kLaunchTokens ? n - t0 : kLaunchTokens;
      gptq_status_t s = syrk_enqueue(H, h_f64, d, ldh, X + t0 * ldx, nc, ldx, accumulate || t0 > 0, ws, ws_bytes, st);
      if (s != GPTQ_OK) return s;
    }
    return GPTQ_OK;
  }
  int64_t tps = ceil_div(ceil_div(n, split), KS) * KS;
  split = (int)ceil_div(n, tps);

  SyrkArgs a;
  a.X = X;
  a.ldx = ldx;
  a.n = n;
  a.d = d;
  a.tokens_per_split = tps;
  a.nsplit = split;
  a.ntiles = nt;
  a.ldh = ldh;
  a.h_f64 = h_f64;
  a.accumulate = accumulate;
  a.direct = split == 1;
  a.out = split == 1 ? H : ws;
  hipLaunchKernelGGL(syrk_kernel, dim3(nt * split), dim3(NT), 0, st, a);
  GPTQ_CHECK_LAUNCH();
  if (split > 1) {
    const int64_t total = (int64_t)nt * TI * TJ;
    int blocks = (int)ceil_div(total, 256 * 4);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(blocks), dim3(256), 0, st, (const double*)ws, split, nt, H,
                       d, ldh, h_f64, accumulate);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace gptq
