// Definitions shared by the quantization driver (quant.hip) and the column-loop
// kernels (colloop_*.hip), which are compiled as separate translation units
// so that the build runs them in parallel (internal header).
#pragma once

#include "common.h"

namespace gptq {

constexpr int BLK = 128;          // lazy-update block (the figure's step 4)
constexpr int CL_THREADS = 256;   // column-loop workgroup: 64 rows x 4 lanes

struct GridFit {
  float s, z;
};

// Asymmetric min-max: lo = min(v, 0), hi = max(v, 0) (both 0 -> -1, 1),
// s = (hi - lo) / maxq, z = rint(-lo / s). Ternary: s = max|v| (0 -> 1), z = 1.
// Symmetric: a = max|v| (0 -> 1), s = 2a / maxq, z = (maxq + 1) / 2.
__device__ inline GridFit fit_grid(float vmin, float vmax, int gmode, float maxq) {
  float lo = fminf(vmin, 0.0f), hi = fmaxf(vmax, 0.0f);
  GridFit g;
  if (gmode == GPTQ_GRID_TERNARY) {
    float amax = fmaxf(-lo, hi);
    g.s = amax == 0.0f ? 1.0f : amax;
    g.z = 1.0f;
    return g;
  }
  if (gmode == GPTQ_GRID_SYM_MINMAX) {
    float amax = fmaxf(-lo, hi);
    if (amax == 0.0f) amax = 1.0f;
    g.s = 2.0f * amax / maxq;
    g.z = 0.5f * (maxq + 1.0f);
    return g;
  }
  if (lo == 0.0f && hi == 0.0f) {
    lo = -1.0f;
    hi = 1.0f;
  }
  g.s = (hi - lo) / maxq;
  g.z = rintf(-lo / g.s);
  return g;
}

struct ColArgs {
  float* Wk;
  const float* U;
  const float* rdiag;
  int64_t ldu, m, d, j0;
  int bw;          // block width (multiple of 32, <= 128)
  int gmode;
  float maxq;
  int group;       // runtime group size (used when G < 0)
  int ngroups;
  float* E;        // errors out: E[r * lde + ecol + k] for the block's columns k
  int64_t lde, ecol;
  half_t* Eh;      // when set, also the block's errors as scaled fp16 pairs (as esplit_kernel
  half_t* El;      // writes them, K-tiled with slab stride m * 32) and the row scales einv
  float* einv;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* err_sq;
  const int32_t* perm;  // quantization order (static groups: grids by natural group)
  int first;
  // R form: Wk holds the original weights (in the quantization order), Acc the
  // accumulator A of the pushes from earlier blocks, Ublk this block's U_bb
  // (the inverse of R's diagonal block, row pitch BLK)
  const float* Acc;
  const float* Ublk;
};

// The column loop over one block of a.bw columns starting at a.j0, for the
// group mode G: 0 = one grid per row (fitted before the loop); 16, 32, 64,
// 128 = a grid per group, refitted at every group start inside the block;
// -1 = every block lies inside one group that starts at a block start (groups
// that are multiples of 128 or that do not divide 128: the blocks are cut at
// group starts), refitted at the group's first block from the working weights;
// -2 = static groups (grids fitted before the loop, per natural group).
// RF: the factor is R (H_d = R R^T) instead of U = R^-1 (not with G = -1).
template <int G, bool RF>
gptq_status_t launch_colloop(const ColArgs& a, hipStream_t st);

}  // namespace gptq
