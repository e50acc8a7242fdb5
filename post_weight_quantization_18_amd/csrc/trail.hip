// Trailing update of the lazy-block scheme on the gfx950 matrix cores:
//   W[:, far] -= E U[blocks, far]
// FDE Interviews breakdown of GPTQ, figure "Quantize a column, correct the
// rest", steps 3-4: the errors of a finished block of columns are pushed onto
// the columns not yet quantized as one matrix product.
//
// Precision: a single fp16 product moves the pre-round values by about 2^-11 of
// the update, which is more than the rounding-boundary band the codes must
// respect, so both operands are split into fp16 pairs (x = hi + lo, each with
// a power-of-two scale that puts the largest |x| just under 2^15) and the
// product is taken in three passes, hi*hi + hi*lo + lo*hi, accumulated in fp32
// (about 2^-22 relative; lo*lo is below fp32 rounding).
//
// Design (MI355X):
//  * 256 x 128 output tile per workgroup of 8 waves (64 x 64 each, two per
//    SIMD); v_mfma_f32_32x32x16_f16, 12 per wave per 16-deep K step.
//  * Both operands are stored K-tiled in slabs of 32 (a 32-deep slab of 16
//    rows is 1 KB of contiguous memory), so each 32-deep K stage is four
//    row-major LDS panels (A hi/lo 256 x 32, B hi/lo 128 x 32, 48 KB) filled by
//    fully coalesced direct global->LDS DMA into a 3-deep ring;
//    the 16-byte chunks of a row are XOR-swizzled by (row / 4) mod 4, chosen on
//    the global side, which makes the fragment reads (ds_read_b128, 32 rows x 2
//    chunks per wave) free of bank conflicts.
//  * Workgroups run in groups of 4 row tiles per column tile, and the groups
//    are laid out contiguously per XCD, so that the tiles resident on one XCD
//    share their A and B panels in its L2.
//  * Wide updates (the super-block GEMMs) take 256 x 256 tiles instead
//    (tgemm_wide_kernel below).
#include "common.h"

namespace gptq {

namespace {

constexpr int TM = 256, TN = 128, KS = 32, NT = 512, NBUF = 3;
constexpr int ROWB = KS * 2;                       // bytes per LDS panel row (32 halves)
constexpr uint32_t OFF_AH = 0, OFF_AL = TM * ROWB, OFF_BH = 2 * TM * ROWB, OFF_BL = 2 * TM * ROWB + TN * ROWB;
constexpr uint32_t STAGE_BYTES = (2 * TM + 2 * TN) * ROWB;  // 48 KB
constexpr int GROUP_M = 4;  // row tiles per column tile in the grouped order (the 32 workgroups of an XCD on 4 x 8 tiles)

__device__ const uint4 kZeroT[1] = {{0u, 0u, 0u, 0u}};

__device__ inline half8 lds_frag(const char* ring, uint32_t byte_off) {
  return *(const half8*)(ring + byte_off);
}

__global__ __launch_bounds__(NT, 1) void tgemm_kernel(TgemmArgs a, int ntm, int ntn) {
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * STAGE_BYTES];

  // grouped tile order inside each XCD's contiguous range of logical ids
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int per_group = GROUP_M * ntn;
  const int grp = logical / per_group, first_m = grp * GROUP_M;
  const int gm = (ntm - first_m) < GROUP_M ? (ntm - first_m) : GROUP_M;
  const int within = logical - grp * per_group;
  const int tm = first_m + within % gm, tn = within / gm;
  const int64_t I0 = (int64_t)tm * TM, J0 = (int64_t)tn * TN;
  GPTQ_DASSERT(tm < ntm && tn < ntn && I0 < a.M && J0 < a.N && a.K % KS == 0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int wi = w >> 1, wj = w & 1;
  const int nst = (int)(a.K / KS);

  // ---- DMA plan: wave w moves A rows 32w .. 32w+31 (hi and lo) and B rows
  // 16w .. 16w+15 (hi and lo): six 1 KB instructions per stage. Lane l covers
  // row (l / 4) of the instruction's 16 rows and LDS chunk position l % 4,
  // which holds global chunk (l % 4) ^ ((row / 4) % 4) = (l % 4) ^ ((l / 16) % 4).
  const int lrow = lane >> 2;
  const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
  int64_t srcA[2], srcB;
  bool okA[2], okB;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t r = I0 + 32 * w + 16 * e + lrow;
    okA[e] = r < a.M;
    srcA[e] = (okA[e] ? r : 0) * 32 + 8 * chunk;
  }
  {
    const int64_t c = J0 + 16 * w + lrow;
    okB = c < a.N;
    srcB = (okB ? c : 0) * 32 + 8 * chunk;
  }
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GPTQ_LDS void*)ring);
  // instruction e (0..5) of stage s into ring buffer b
  auto issue = [&](int e, int s, int b) {
    const int64_t k0 = (int64_t)s * KS;
    const void* src;
    uint32_t off;
    if (e < 4) {
      const int h = e & 1;  // which 16-row half of the wave's 32 A rows
      const half_t* base = (e < 2) ? a.Ah : a.Al;
      src = okA[h] ? (const void*)(base + (k0 >> 5) * a.a_kslab + srcA[h]) : (const void*)kZeroT;
      off = ((e < 2) ? OFF_AH : OFF_AL) + (uint32_t)((32 * wu + 16 * h) * ROWB);
    } else {
      const half_t* base = (e == 4) ? a.Bh : a.Bl;
      src = okB ? (const void*)(base + (k0 >> 7) * a.b_block + ((k0 & 127) >> 5) * a.b_kslab + srcB)
                : (const void*)kZeroT;
      off = ((e == 4) ? OFF_BH : OFF_BL) + (uint32_t)(16 * wu * ROWB);
    }
    dma16(src, ring_lds + (uint32_t)b * STAGE_BYTES + off);
  };

  // ---- fragment offsets: subtile row (l % 32), K chunk 2 kk + l / 32, stored
  // at position chunk ^ ((row / 4) % 4) = chunk ^ ((l / 4) % 4)
  const int frow = lane & 31, fsw = (lane >> 2) & 3, fhi = lane >> 5;
  uint32_t offA[2][2], offB[2][2];  // [subtile][kk]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t pos = (uint32_t)(((2 * kk + fhi) ^ fsw) * 16);
      offA[x][kk] = (uint32_t)((64 * wi + 32 * x + frow) * ROWB) + pos;
      offB[x][kk] = (uint32_t)((64 * wj + 32 * x + frow) * ROWB) + pos;
    }

  float16v acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

  auto compute = [&](int b, bool refill, int s_next, int b_next) {
    const char* st = ring + (size_t)b * STAGE_BYTES;
    half8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        ah[x] = lds_frag(st, OFF_AH + offA[x][kk]);
        al[x] = lds_frag(st, OFF_AL + offA[x][kk]);
        bh[x] = lds_frag(st, OFF_BH + offB[x][kk]);
        bl[x] = lds_frag(st, OFF_BL + offB[x][kk]);
      }
      if (refill) {
#pragma unroll
        for (int e = 3 * kk; e < 3 * kk + 3; ++e) issue(e, s_next, b_next);
      }
      // the three passes sweep all four sub-tiles in turn, so consecutive
      // MFMAs never accumulate into the same registers
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[x], bh[y], acc[x][y], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[x], bl[y], acc[x][y], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[x], bh[y], acc[x][y], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nst > 0) {
#pragma unroll
    for (int e = 0; e < 6; ++e) issue(e, 0, 0);
  }
  if (nst > 1) {
#pragma unroll
    for (int e = 0; e < 6; ++e) issue(e, 1, 1);
  }
  int cur = 0;
  for (int s = 0; s < nst; ++s) {
    // this stage's six loads are done once at most the next stage's six remain
    if (s + 1 >= nst)
      __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    else
      __builtin_amdgcn_s_waitcnt(WAIT_VM6);
    lds_barrier();
    const int nxt = cur == 0 ? NBUF - 1 : cur - 1;  // (cur + 2) mod 3: the buffer stage s-1 used
    compute(cur, s + 2 < nst, s + 2, nxt);
    cur = cur == NBUF - 1 ? 0 : cur + 1;
  }

  // ---- epilogue: C -= acc * rowscale[i] * cscale ----
  // All loads of a sub-tile row group are issued before any store, so the
  // read-modify-write costs one memory round trip per 16 rows instead of one
  // per element (the compiler cannot reorder loads across possibly aliasing
  // stores by itself).
  const float cs = *a.cscale;
  const int hl = lane >> 5, col = lane & 31;
  const bool full = (I0 + TM <= a.M) && (J0 + TN <= a.N);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int64_t ib = I0 + 64 * wi + 32 * x + 4 * hl;
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = ib + 8 * (r >> 2) + (r & 3);
      sc[r] = (i < a.M) ? a.rowscale[i] : 0.0f;
    }
    if (full) {
      float cv[2][16];
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cv[y][r] = a.C[(ib + 8 * (r >> 2) + (r & 3)) * a.ldc + J0 + 64 * wj + 32 * y + col];
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          a.C[(ib + 8 * (r >> 2) + (r & 3)) * a.ldc + J0 + 64 * wj + 32 * y + col] =
              fmaf(-acc[x][y][r], sc[r] * cs, cv[y][r]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = ib + 8 * (r >> 2) + (r & 3);
        if (i >= a.M) continue;
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int64_t j = J0 + 64 * wj + 32 * y + col;
          if (j < a.N) {
            float* c = a.C + i * a.ldc + j;
            *c = fmaf(-acc[x][y][r], sc[r] * cs, *c);
          }
        }
      }
    }
  }
}

// The same product on 256 x 256 output tiles, for wide updates (N of a few
// thousand columns and more): 8 waves of 64 x 128 (32 accumulator blocks of
// 32 x 32 per wave in 128 fp32 registers); each 32-deep K stage is 64 KB of
// operand panels (A hi/lo 256 x 32, B hi/lo 256 x 32) in a 2-deep ring, so the
// DMA moves a third fewer bytes per flop than on 256 x 128 tiles and the
// fragment reads a quarter fewer. Stage s + 1 is issued into the other buffer
// right after the barrier that ends stage s - 1's reads.
constexpr int TNW = 256, NBUFW = 2;
constexpr uint32_t W_OFF_AH = 0, W_OFF_AL = TM * ROWB, W_OFF_BH = 2 * TM * ROWB, W_OFF_BL = 2 * TM * ROWB + TNW * ROWB;
constexpr uint32_t W_STAGE_BYTES = (2 * TM + 2 * TNW) * ROWB;  // 64 KB

__global__ __launch_bounds__(NT, 1) void tgemm_wide_kernel(TgemmArgs a, int ntm, int ntn) {
  __shared__ __attribute__((aligned(1024))) char ring[NBUFW * W_STAGE_BYTES];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int per_group = GROUP_M * ntn;
  const int grp = logical / per_group, first_m = grp * GROUP_M;
  const int gm = (ntm - first_m) < GROUP_M ? (ntm - first_m) : GROUP_M;
  const int within = logical - grp * per_group;
  const int tm = first_m + within % gm, tn = within / gm;
  const int64_t I0 = (int64_t)tm * TM, J0 = (int64_t)tn * TNW;
  GPTQ_DASSERT(tm < ntm && tn < ntn && I0 < a.M && J0 < a.N && a.K % KS == 0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int wi = w >> 1, wj = w & 1;  // wave tile: rows 64 wi .., cols 128 wj ..
  const int nst = (int)(a.K / KS);

  // DMA plan: wave w moves A rows 32w .. 32w+31 and B rows (columns of the
  // update) 32w .. 32w+31, hi and lo: eight 1 KB instructions per stage, lane
  // l on row (l / 4) of the instruction's 16 rows at LDS chunk position l % 4
  // (global chunk (l % 4) ^ ((row / 4) % 4)), as in tgemm_kernel.
  const int lrow = lane >> 2;
  const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
  int64_t srcA[2], srcB[2];
  bool okA[2], okB[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t r = I0 + 32 * w + 16 * e + lrow;
    okA[e] = r < a.M;
    srcA[e] = (okA[e] ? r : 0) * 32 + 8 * chunk;
    const int64_t c = J0 + 32 * w + 16 * e + lrow;
    okB[e] = c < a.N;
    srcB[e] = (okB[e] ? c : 0) * 32 + 8 * chunk;
  }
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GPTQ_LDS void*)ring);
  // instruction e (0..7) of stage s into ring buffer b: e = 0..3 A (hi h0, hi
  // h1, lo h0, lo h1), e = 4..7 B likewise
  auto issue = [&](int e, int s, int b) {
    const int64_t k0 = (int64_t)s * KS;
    const int h = e & 1;
    const void* src;
    uint32_t off;
    if (e < 4) {
      const half_t* base = (e < 2) ? a.Ah : a.Al;
      src = okA[h] ? (const void*)(base + (k0 >> 5) * a.a_kslab + srcA[h]) : (const void*)kZeroT;
      off = ((e < 2) ? W_OFF_AH : W_OFF_AL) + (uint32_t)((32 * wu + 16 * h) * ROWB);
    } else {
      const half_t* base = (e < 6) ? a.Bh : a.Bl;
      src = okB[h] ? (const void*)(base + (k0 >> 7) * a.b_block + ((k0 & 127) >> 5) * a.b_kslab + srcB[h])
                   : (const void*)kZeroT;
      off = ((e < 6) ? W_OFF_BH : W_OFF_BL) + (uint32_t)((32 * wu + 16 * h) * ROWB);
    }
    dma16(src, ring_lds + (uint32_t)b * W_STAGE_BYTES + off);
  };

  const int frow = lane & 31, fsw = (lane >> 2) & 3, fhi = lane >> 5;
  uint32_t offA[2][2], offB[4][2];  // [subtile][kk]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint32_t pos = (uint32_t)(((2 * kk + fhi) ^ fsw) * 16);
#pragma unroll
    for (int x = 0; x < 2; ++x) offA[x][kk] = (uint32_t)((64 * wi + 32 * x + frow) * ROWB) + pos;
#pragma unroll
    for (int y = 0; y < 4; ++y) offB[y][kk] = (uint32_t)((128 * wj + 32 * y + frow) * ROWB) + pos;
  }

  float16v acc[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

  auto compute = [&](int b, bool refill, int s_next, int b_next) {
    const char* st = ring + (size_t)b * W_STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8 ah[2], al[2], bh[4], bl[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        ah[x] = lds_frag(st, W_OFF_AH + offA[x][kk]);
        al[x] = lds_frag(st, W_OFF_AL + offA[x][kk]);
      }
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        bh[y] = lds_frag(st, W_OFF_BH + offB[y][kk]);
        bl[y] = lds_frag(st, W_OFF_BL + offB[y][kk]);
      }
      if (refill) {
#pragma unroll
        for (int e = 4 * kk; e < 4 * kk + 4; ++e) issue(e, s_next, b_next);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[x], bh[y], acc[x][y], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[x], bl[y], acc[x][y], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[x], bh[y], acc[x][y], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nst > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) issue(e, 0, 0);
  }
  for (int s = 0; s < nst; ++s) {
    // stage s's eight loads are the only ones in flight; after the barrier no
    // wave reads the other buffer (stage s - 1) any more, so stage s + 1 may
    // land there while this one is computed
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    lds_barrier();
    compute(s & 1, s + 1 < nst, s + 1, (s + 1) & 1);
  }

  // ---- epilogue: C -= acc * rowscale[i] * cscale (loads of a 16-row group
  // before its stores, as in tgemm_kernel) ----
  const float cs = *a.cscale;
  const int hl = lane >> 5, col = lane & 31;
  const bool full = (I0 + TM <= a.M) && (J0 + TNW <= a.N);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int64_t ib = I0 + 64 * wi + 32 * x + 4 * hl;
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = ib + 8 * (r >> 2) + (r & 3);
      sc[r] = (i < a.M) ? a.rowscale[i] : 0.0f;
    }
#pragma unroll
    for (int yh = 0; yh < 2; ++yh) {  // two 32-column blocks at a time keep the staged values to 32 registers
      if (full) {
        float cv[2][16];
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cv[y][r] = a.C[(ib + 8 * (r >> 2) + (r & 3)) * a.ldc + J0 + 128 * wj + 32 * (2 * yh + y) + col];
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            a.C[(ib + 8 * (r >> 2) + (r & 3)) * a.ldc + J0 + 128 * wj + 32 * (2 * yh + y) + col] =
                fmaf(-acc[x][2 * yh + y][r], sc[r] * cs, cv[y][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = ib + 8 * (r >> 2) + (r & 3);
          if (i >= a.M) continue;
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            const int64_t j = J0 + 128 * wj + 32 * (2 * yh + y) + col;
            if (j < a.N) {
              float* c = a.C + i * a.ldc + j;
              *c = fmaf(-acc[x][2 * yh + y][r], sc[r] * cs, *c);
            }
          }
        }
      }
    }
  }
}

}  // namespace

gptq_status_t tgemm_enqueue(const TgemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return GPTQ_OK;
  if (a.K % KS) return GPTQ_ERR_INVALID_ARG;
  // 256 x 256 tiles for the super-block GEMMs; the narrow updates inside a
  // super-block keep twice as many 256 x 128 tiles
  const bool wide = a.N >= 4096;
  const int tn = wide ? TNW : TN;
  const int64_t ntm = ceil_div(a.M, TM), ntn = ceil_div(a.N, tn);
  if (ntm * ntn > 0x7fffffff) return GPTQ_ERR_UNSUPPORTED;
  // executed: three fp16 passes over the padded tiles
  TraceScope tr(st, GPTQ_TRACE_TGEMM, 3.0 * 2.0 * (double)(ntm * TM) * (double)(ntn * tn) * (double)a.K);
  if (wide)
    hipLaunchKernelGGL(tgemm_wide_kernel, dim3((unsigned)(ntm * ntn)), dim3(NT), 0, st, a, (int)ntm, (int)ntn);
  else
    hipLaunchKernelGGL(tgemm_kernel, dim3((unsigned)(ntm * ntn)), dim3(NT), 0, st, a, (int)ntm, (int)ntn);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
