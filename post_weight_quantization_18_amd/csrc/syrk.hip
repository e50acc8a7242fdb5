// Hessian accumulation H (+)= 2 X^T X on the gfx950 matrix cores.
//
// FDE Interviews breakdown of GPTQ, section 01: the layer-wise objective's
// curvature is H = 2XX^T from the calibration inputs.
//
// Design (MI355X):
//  * Output tiles of 256 (i) x 128 (j) cover the lower triangle only; a
//    workgroup of 4 waves owns one tile for one token range (split-K when the
//    tile count alone cannot fill 256 CUs).
//  * X is token-major fp16; each 64-token stage of the I- and J-feature columns
//    is copied row-major into LDS with 16-byte loads, and the MFMA operands
//    (8 consecutive tokens per lane) come out of LDS with the gfx950
//    transpose read ds_read_b64_tr_b16, so no transpose pass over X is needed.
//  * v_mfma_f32_32x32x16_f16: fp16 x fp16 products are exact in fp32.
//  * Accuracy: every 1024 tokens the fp32 accumulators are folded into a
//    second fp32 register (Fast2Sum) and the rounding error is put back into the
//    MFMA accumulator, so the partial sum is carried to ~2^-48 relative; the
//    final value is outer + acc in fp64, and split-K partials are summed in a
//    fixed order in fp64 (deterministic).
#include "common.h"

namespace gptq {

namespace {

constexpr int TI = 256;          // tile rows (i features)
constexpr int TJ = 128;          // tile cols (j features)
constexpr int KS = 64;           // tokens per LDS stage
constexpr int PI = TI + 32;      // LDS row pitch (halves) of the I tile: 576 B
constexpr int PJ = TJ + 32;      // LDS row pitch (halves) of the J tile: 320 B
constexpr int FOLD = 16;         // stages between error folds (1024 tokens)
constexpr int NT = 256;          // threads per workgroup
constexpr int STAGE_HALVES = KS * PI + KS * PJ;

struct SyrkArgs {
  const half_t* X;
  int64_t ldx, n, d;
  int64_t tokens_per_split;
  int nsplit, ntiles;
  void* out;        // H (direct) or fp64 partial tiles
  int64_t ldh;
  int h_f64, accumulate, direct;
};

__device__ inline void tile_coords(int t, int& bi, int& bj) {
  // tiles of I-block bi are bj = 0 .. 2*bi+1, so tile t lies in
  // [bi(bi+1), (bi+1)(bi+2)).
  int b = (int)((sqrtf(4.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((b + 1) * (b + 2) <= t) ++b;
  while (b * (b + 1) > t) --b;
  bi = b;
  bj = t - b * (b + 1);
}

__device__ inline short4v tr_read(const half_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS short4v*)(p));
}

__device__ inline half8 frag(const half_t* tile, int pitch, int lane_off) {
  // lane_off already holds (8*(g>>1) + e) * pitch + 16*(g&1) + 4*q; the second
  // read takes the next 4 tokens.
  short4v lo = tr_read(tile + lane_off);
  short4v hi = tr_read(tile + lane_off + 4 * pitch);
  // whole-vector reinterpretation: the two 64-bit results are the 8 halves
  short8v both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(half8, both);
}

__global__ __launch_bounds__(NT, 1) void syrk_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) half_t lds[2 * STAGE_HALVES];

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int split = logical / a.ntiles;
  const int t = logical - split * a.ntiles;
  int bi, bj;
  tile_coords(t, bi, bj);
  const int64_t I0 = (int64_t)bi * TI, J0 = (int64_t)bj * TJ;
  if (J0 >= a.d) return;  // whole workgroup exits together (uniform)

  const int64_t tok0 = (int64_t)split * a.tokens_per_split;
  int64_t tok1 = tok0 + a.tokens_per_split;
  if (tok1 > a.n) tok1 = a.n;
  const int nstages = tok1 > tok0 ? (int)((tok1 - tok0 + KS - 1) / KS) : 0;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w >> 1, wj = w & 1;
  const bool j_in_i = (J0 >= I0) && (J0 < I0 + TI);

  // ---- global -> register staging map ----
  // I tile: 64 rows x 32 chunks of 8 halves; thread: chunk tid%32, rows tid/32 + 8r.
  // J tile: 64 rows x 16 chunks; thread: chunk tid%16, rows tid/16 + 16r.
  const int ci = tid & 31, ri = tid >> 5;
  const int cj = tid & 15, rj = tid >> 4;
  const int64_t fi = I0 + 8 * ci, fj = J0 + 8 * cj;
  const bool fi_ok = fi < a.d, fj_ok = (!j_in_i) && (fj < a.d);

  uint4 pa[8], pb[4];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int64_t tok = k0 + ri + 8 * r;
      if (fi_ok && tok < tok1)
        pa[r] = *(const uint4*)(a.X + tok * a.ldx + fi);
      else
        pa[r] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int64_t tok = k0 + rj + 16 * r;
      if (fj_ok && tok < tok1)
        pb[r] = *(const uint4*)(a.X + tok * a.ldx + fj);
      else
        pb[r] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](half_t* buf) {
#pragma unroll
    for (int r = 0; r < 8; ++r) *(uint4*)(buf + (ri + 8 * r) * PI + 8 * ci) = pa[r];
    if (!j_in_i) {
      half_t* bj_buf = buf + KS * PI;
#pragma unroll
      for (int r = 0; r < 4; ++r) *(uint4*)(bj_buf + (rj + 16 * r) * PJ + 8 * cj) = pb[r];
    }
  };

  // ---- per-lane transpose-read offsets ----
  const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const int tokoff = 8 * (g >> 1) + e;
  const int featoff = 16 * (g & 1) + 4 * q;
  // A operand: I features wi*128 + f*32 ; B operand: J features wj*64 + f*32.
  const int a_off = tokoff * PI + wi * 128 + featoff;
  const int b_pitch = j_in_i ? PI : PJ;
  const int b_feat0 = j_in_i ? (int)(J0 - I0) : 0;
  const int b_off = tokoff * b_pitch + b_feat0 + wj * 64 + featoff;

  float16v acc[4][2], outer[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[f][h][r] = 0.0f;
        outer[f][h][r] = 0.0f;
      }

  if (nstages > 0) {
    load_stage(tok0);
    store_stage(lds);
  }
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;
    if (more) load_stage(tok0 + (int64_t)(s + 1) * KS);
    const half_t* buf = lds + (s & 1) * STAGE_HALVES;
    const half_t* bbuf = j_in_i ? buf : buf + KS * PI;
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      half8 af[4], bf[2];
#pragma unroll
      for (int f = 0; f < 4; ++f) af[f] = frag(buf, PI, a_off + kk * 16 * PI + f * 32);
#pragma unroll
      for (int h = 0; h < 2; ++h) bf[h] = frag(bbuf, b_pitch, b_off + kk * 16 * b_pitch + h * 32);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[f][h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f], bf[h], acc[f][h], 0, 0, 0);
    }
    if ((s + 1) % FOLD == 0) {
      // Fast2Sum(outer, acc): outer <- fl(outer + acc), acc <- exact residual.
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float o = outer[f][h][r], c = acc[f][h][r];
            float sum = o + c;
            float z = sum - o;
            acc[f][h][r] = c - z;
            outer[f][h][r] = sum;
          }
    }
    if (more) store_stage(lds + ((s + 1) & 1) * STAGE_HALVES);
    __syncthreads();
  }

  // ---- epilogue ----
  const int hl = lane >> 5, col = lane & 31;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int li = wi * 128 + f * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int lj = wj * 64 + h * 32 + col;
        const double v = 2.0 * ((double)outer[f][h][r] + (double)acc[f][h][r]);
        if (a.direct) {
          const int64_t i = I0 + li, j = J0 + lj;
          if (i < a.d && j <= i) {
            if (a.h_f64) {
              double* H = (double*)a.out + i * a.ldh + j;
              *H = a.accumulate ? *H + v : v;
            } else {
              float* H = (float*)a.out + i * a.ldh + j;
              *H = (float)(a.accumulate ? (double)*H + v : v);
            }
          }
        } else {
          double* P = (double*)a.out + ((int64_t)logical * TI + li) * TJ + lj;
          *P = v;
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
    tile_coords(t, bi, bj);
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
  int64_t T = ceil_div(d, TI);
  return (int)(T * (T + 1));
}

// Token split: enough workgroups to fill 256 CUs with a small tail, token
// ranges a multiple of the stage, bounded by the stages available.
int syrk_choose_split(int ntiles, int64_t n) {
  const int64_t stages = ceil_div(n, KS);
  if (stages <= 1 || ntiles >= 1024) return 1;
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= 64 && s <= stages; ++s) {
    const int64_t wgs = (int64_t)ntiles * s;
    const int64_t waves = ceil_div(wgs, 256);
    const double eff = (double)wgs / (double)(waves * 256);
    const double score = eff * (wgs >= 256 ? 1.0 : (double)wgs / 256.0);
    if (score > best_eff + 1e-9) {
      best_eff = score;
      best = s;
    }
    if (wgs >= 512 && eff >= 0.9) break;
  }
  return best;
}

}  // namespace

size_t syrk_workspace_bytes(int64_t d, int64_t n) {
  const int nt = syrk_ntiles(d);
  const int s = syrk_choose_split(nt, n);
  if (s <= 1) return 0;
  return (size_t)s * (size_t)nt * TI * TJ * sizeof(double);
}

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
  int split = syrk_choose_split(nt, n);
  const size_t per_split = (size_t)nt * TI * TJ * sizeof(double);
  if (split > 1 && (ws == nullptr || ws_bytes < (size_t)split * per_split)) {
    split = ws ? (int)(ws_bytes / per_split) : 1;
    if (split < 1) split = 1;
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
