// The column loop of GPTQ on gfx950 (internal header, included once per group
// mode by colloop_*.hip).
//
// FDE Interviews breakdown of GPTQ, figure "Quantize a column, correct the
// rest", steps 1-3, for column i of the block: round w_i to the grid -> q_i;
// err = (w_i - q_i) / U_ii; the block's later columns -= err x U[i, ...].
// Rows are independent given U: four lanes (a DPP quad) own one row's 128
// block columns in registers; the block's U is in LDS and read as broadcasts.
//
// Two forms of the lazy updates between blocks:
//  * U form (RF = false): the factor is U = chol(H_d^-1). The working weights
//    W[:, later] carry every earlier push (-= e U[blk, later]); the block reads
//    its columns and runs steps 1-3 with the block's diagonal block of U.
//  * R form (RF = true): the factor is R with H_d = R R^T (R = U^-1, what the
//    Cholesky gives without any inverse). Since e = (w - q) R for the original
//    weights w, the pushes from earlier blocks sum to a term of the
//    accumulator A = sum_l (w_l - q_l) R[l, .]: the true state of the block's
//    columns at its start is w + A_blk U_bb with U_bb = (R_bb)^-1, the inverse
//    of R's diagonal block only. The block rebuilds that state in a first pass
//    over U_bb, runs the same steps 1-3, and hands (q - w) to the trailing GEMM
//    (A[:, later] -= (q - w)_blk R[blk, later]).
#pragma once

#include "quant_shared.h"

namespace gptq {

namespace {

// Layout of the column loop: four lanes (a DPP quad) share one row; lane
// group g = lane % 4 owns the block's columns [32g, 32g + 32) in registers.
// At step i the owner group o = i / 32 rounds column i and forms the error e,
// a quad broadcast hands e to the other three lanes, and every lane updates
// its 32 columns with the strictly upper part of row i of the block's U, read
// from LDS (zeros on and below the diagonal make the update branch-free).
constexpr int QL = 4;            // lanes per row
constexpr int CPL = BLK / QL;    // columns per lane (32)
constexpr int UGS = CPL + 4;     // LDS stride of a lane group's slice (floats):
                                 // the quad's four slices start in different banks
constexpr int UPITCH = QL * UGS; // LDS row pitch of the U block (floats)

struct LaneState {
  float w[CPL];         // the lane's 32 working weights, then its 32 errors (R form: q - w)
  float w0[CPL];        // R form: the original weights of its 32 columns
  uint32_t cw[CPL / 4]; // its 32 codes, one byte each
  float s, rs, zf, esum;
  float cs[CPL], crs[CPL], cz[CPL];  // static groups: the grid of each of its 32 columns
};

template <int O>
__device__ __forceinline__ float quad_bcast(float v) {
  // quad_perm(O, O, O, O)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), O | (O << 2) | (O << 4) | (O << 6),
                                                            0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor1(float v) {  // quad_perm(1, 0, 3, 2)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 1 | (0 << 2) | (3 << 4) | (2 << 6),
                                                            0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {  // quad_perm(2, 3, 0, 1)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 2 | (3 << 2) | (0 << 4) | (1 << 6),
                                                            0xF, 0xF, false));
}

template <int K, int END>
struct MinMax {  // running min/max over w[K .. END-1]
  __device__ __forceinline__ static void run(const LaneState& st, float& lo, float& hi) {
    lo = fminf(lo, st.w[K]);
    hi = fmaxf(hi, st.w[K]);
    MinMax<K + 1, END>::run(st, lo, hi);
  }
};
template <int END>
struct MinMax<END, END> {
  __device__ __forceinline__ static void run(const LaneState&, float&, float&) {}
};

// The lane's 32 entries of one row of the block's U and that row's 1 / U_ii,
// loaded one step ahead of their use.
struct URow {
  float4 u[CPL / 4];
  float rd;
};

__device__ __forceinline__ void load_urow(URow& ur, const float (*Us)[UPITCH], const float* rdiag, int i, int g) {
  const float4* u4 = (const float4*)(Us[i] + g * UGS);
#pragma unroll
  for (int k4 = 0; k4 < CPL / 4; ++k4) ur.u[k4] = u4[k4];
  ur.rd = rdiag[i];
}

template <int G, bool RF, int I>
__device__ __forceinline__ void col_step(LaneState& st, const ColArgs& a, int64_t r, int g, const URow& ur) {
  const float rd = ur.rd;
  constexpr int O = I / CPL, LI = I % CPL;
  if constexpr (G > 0 && I % (G > 0 ? G : 1) == 0) {
    // grid of the group [I, I + G): this lane's part, then across the lanes of the group
    float lo = st.w[LI], hi = st.w[LI];
    MinMax<LI + 1, (G < CPL ? LI + G : CPL)>::run(st, lo, hi);
    if constexpr (G >= 2 * CPL) {
      lo = fminf(lo, quad_xor1(lo));
      hi = fmaxf(hi, quad_xor1(hi));
    }
    if constexpr (G >= 4 * CPL) {
      lo = fminf(lo, quad_xor2(lo));
      hi = fmaxf(hi, quad_xor2(hi));
    }
    GridFit gf = fit_grid(lo, hi, a.gmode, a.maxq);
    if (g == O) {
      const int64_t gi = (a.j0 + I) / (G > 0 ? G : 1);
      a.scales[r * a.ngroups + gi] = gf.s;
      a.zeros[r * a.ngroups + gi] = (uint8_t)gf.z;
    }
    // groups of 32 or 64 start inside other lanes' ranges too: only the
    // lanes of this group adopt the new grid
    const bool mine = (G >= 4 * CPL) || (G == 2 * CPL ? (g >> 1) == (O >> 1) : g == O);
    if (mine) {
      st.s = gf.s;
      st.zf = gf.z;
      st.rs = 1.0f / gf.s;
    }
  }
  if constexpr (G == -2) {
    st.s = st.cs[LI];
    st.rs = st.crs[LI];
    st.zf = st.cz[LI];
  }
  const bool owner = (g == O);
  const float wv = st.w[LI];
  const float p = wv * st.rs + st.zf;
  const float c = fminf(fmaxf(rintf(p), 0.0f), a.maxq);
  const float qv = st.s * (c - st.zf);
  const float e_own = (wv - qv) * rd;
  if (owner) {
    st.esum += e_own * e_own;
    st.cw[LI >> 2] |= ((uint32_t)c) << (8 * (LI & 3));
    // the register now carries the error of column I (R form: q - w, the
    // trailing GEMM's operand; e itself only enters the OBS loss)
    if constexpr (RF)
      st.w[LI] = qv - st.w0[LI];
    else
      st.w[LI] = e_own;
  }
  const float e = quad_bcast<O>(e_own);
#pragma unroll
  for (int k4 = 0; k4 < CPL / 4; ++k4) {
    const float4 u = ur.u[k4];
    st.w[4 * k4] = fmaf(-e, u.x, st.w[4 * k4]);
    st.w[4 * k4 + 1] = fmaf(-e, u.y, st.w[4 * k4 + 1]);
    st.w[4 * k4 + 2] = fmaf(-e, u.z, st.w[4 * k4 + 2]);
    st.w[4 * k4 + 3] = fmaf(-e, u.w, st.w[4 * k4 + 3]);
  }
}

// Steps I .. BLK-1 of the block: row I + 1 of U is read from LDS before step I
// runs, so its latency hides behind the step's arithmetic.
template <int G, bool RF, int I>
struct Steps {
  __device__ __forceinline__ static void run(LaneState& st, const ColArgs& a, int64_t r, int g,
                                             const float (*Us)[UPITCH], const float* rdiag, int bw, const URow& cur) {
    if (I >= bw) return;
    URow nxt;
    if constexpr (I + 1 < BLK) load_urow(nxt, Us, rdiag, I + 1, g);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this step's work
    col_step<G, RF, I>(st, a, r, g, cur);
    if constexpr (I + 1 < BLK) Steps<G, RF, I + 1>::run(st, a, r, g, Us, rdiag, bw, nxt);
  }
};

// R form, first pass: w += A_blk U_bb (the lane's 32 columns; U_bb's strictly
// upper part from LDS, its diagonal 1 / R_ii from rdiag). The accumulator
// values are known up front, so the steps carry no dependency but the sums.
template <int I>
struct StateSteps {
  __device__ __forceinline__ static void run(LaneState& st, const float* acc, int g, const float (*Us)[UPITCH],
                                             const float* rdiag, int bw, const URow& cur) {
    if (I >= bw) return;
    constexpr int O = I / CPL, LI = I % CPL;
    URow nxt;
    if constexpr (I + 1 < BLK) load_urow(nxt, Us, rdiag, I + 1, g);
    const float av = quad_bcast<O>(acc[LI]);
#pragma unroll
    for (int k4 = 0; k4 < CPL / 4; ++k4) {
      const float4 u = cur.u[k4];
      st.w[4 * k4] = fmaf(av, u.x, st.w[4 * k4]);
      st.w[4 * k4 + 1] = fmaf(av, u.y, st.w[4 * k4 + 1]);
      st.w[4 * k4 + 2] = fmaf(av, u.z, st.w[4 * k4 + 2]);
      st.w[4 * k4 + 3] = fmaf(av, u.w, st.w[4 * k4 + 3]);
    }
    if (g == O) st.w[LI] += acc[LI] / cur.rd;
    if constexpr (I + 1 < BLK) StateSteps<I + 1>::run(st, acc, g, Us, rdiag, bw, nxt);
  }
};

// G = 0: one grid per row (already fitted); G = 32, 64, 128: refit at every
// group start inside the block; G = -1: groups span whole blocks, refit at the
// group's first block from the current working weights; G = -2: static groups,
// every column takes the grid of its natural group perm[j] / group (fitted
// before the loop).
template <int G, bool RF>
__global__ __launch_bounds__(CL_THREADS) void colloop_kernel(ColArgs a) {
  __shared__ __attribute__((aligned(16))) float Us[BLK][UPITCH];
  __shared__ float rdiag[BLK];
  static_assert(!RF || G != -1, "the R form fits groups within a block or from the original weights");
  const int tid = threadIdx.x;
  const int bw = a.bw;
  GPTQ_DASSERT(bw > 0 && bw <= BLK && bw % 32 == 0 && a.j0 >= 0 && a.j0 + bw <= a.d);
  // strictly upper part of the block's U (zeros on and below the diagonal);
  // R form: U_bb from the compact block inverses (row pitch BLK)
  for (int idx = tid; idx < BLK * BLK / 4; idx += CL_THREADS) {
    const int i = idx / (BLK / 4), k4 = (idx % (BLK / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < bw && k4 < bw)
      v = RF ? *(const float4*)(a.Ublk + i * BLK + k4) : *(const float4*)(a.U + (a.j0 + i) * a.ldu + a.j0 + k4);
    if (k4 + 0 <= i) v.x = 0.f;
    if (k4 + 1 <= i) v.y = 0.f;
    if (k4 + 2 <= i) v.z = 0.f;
    if (k4 + 3 <= i) v.w = 0.f;
    *(float4*)&Us[i][(k4 / CPL) * UGS + k4 % CPL] = v;
  }
  for (int i = tid; i < BLK; i += CL_THREADS) rdiag[i] = i < bw ? a.rdiag[a.j0 + i] : 0.0f;
  __syncthreads();

  const int g = tid % QL;
  const int64_t r = (int64_t)blockIdx.x * (CL_THREADS / QL) + tid / QL;
  const bool live = r < a.m;
  const int64_t rr = live ? r : a.m - 1;  // dead lanes mirror the last row and store nothing

  LaneState st;
  const float* wrow = a.Wk + rr * a.d + a.j0 + g * CPL;
  const bool cols_ok = g * CPL < bw;
#pragma unroll
  for (int k = 0; k < CPL; k += 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cols_ok) v = *(const float4*)(wrow + k);
    st.w[k] = v.x;
    st.w[k + 1] = v.y;
    st.w[k + 2] = v.z;
    st.w[k + 3] = v.w;
  }
  if constexpr (RF) {
    // the block's true state: original weights plus A_blk U_bb
    float acc[CPL];
    const float* arow = a.Acc + rr * a.d + a.j0 + g * CPL;
#pragma unroll
    for (int k = 0; k < CPL; k += 4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cols_ok) v = *(const float4*)(arow + k);
      acc[k] = v.x;
      acc[k + 1] = v.y;
      acc[k + 2] = v.z;
      acc[k + 3] = v.w;
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) st.w0[k] = st.w[k];
    URow first;
    load_urow(first, Us, rdiag, 0, g);
    StateSteps<0>::run(st, acc, g, Us, rdiag, bw, first);
  }
#pragma unroll
  for (int k = 0; k < CPL / 4; ++k) st.cw[k] = 0;
  st.esum = 0.0f;
  st.s = 1.0f;
  st.rs = 1.0f;
  st.zf = 0.0f;
  if (G == 0) {
    st.s = a.scales[rr];
    st.zf = (float)a.zeros[rr];
    st.rs = 1.0f / st.s;
  } else if (G == -1) {
    const int gi = (int)(a.j0 / a.group);
    if (a.j0 % a.group == 0) {
      // the group spans whole blocks: each lane scans a quarter of it
      float vmin = INFINITY, vmax = -INFINITY;
      const int part = a.group / QL;
      const float* grow = a.Wk + rr * a.d + a.j0 + g * part;
      for (int k = 0; k < part; k += 4) {
        float4 v = *(const float4*)(grow + k);
        vmin = fminf(fminf(fminf(vmin, v.x), fminf(v.y, v.z)), v.w);
        vmax = fmaxf(fmaxf(fmaxf(vmax, v.x), fmaxf(v.y, v.z)), v.w);
      }
      vmin = fminf(vmin, quad_xor1(vmin));
      vmax = fmaxf(vmax, quad_xor1(vmax));
      vmin = fminf(vmin, quad_xor2(vmin));
      vmax = fmaxf(vmax, quad_xor2(vmax));
      GridFit gf = fit_grid(vmin, vmax, a.gmode, a.maxq);
      if (g == 0 && live) {
        a.scales[r * a.ngroups + gi] = gf.s;
        a.zeros[r * a.ngroups + gi] = (uint8_t)gf.z;
      }
      st.s = gf.s;
      st.zf = gf.z;
    } else {
      st.s = a.scales[rr * a.ngroups + gi];
      st.zf = (float)a.zeros[rr * a.ngroups + gi];
    }
    st.rs = 1.0f / st.s;
  } else if (G == -2) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int64_t j = a.j0 + g * CPL + k;
      int64_t c = j < a.d ? a.perm[j] : 0;
      if (c < 0 || c >= a.d) c = 0;
      const int64_t gi = c / a.group;
      st.cs[k] = a.scales[rr * a.ngroups + gi];
      st.crs[k] = 1.0f / st.cs[k];
      st.cz[k] = (float)a.zeros[rr * a.ngroups + gi];
    }
  }

  if (live) {
    URow first;
    load_urow(first, Us, rdiag, 0, g);
    Steps<G, RF, 0>::run(st, a, r, g, Us, rdiag, bw, first);
  }

  if (a.Eh) {
    // the row's power-of-two scale over the block (quad max of |e|; columns
    // past bw hold 0), then the fp16 pair of every error: lane g's 32 columns
    // are K-slab g, 32 consecutive halves at g * m * 32 + r * 32
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) mx = fmaxf(mx, fabsf(st.w[k]));
    mx = fmaxf(mx, quad_xor1(mx));
    mx = fmaxf(mx, quad_xor2(mx));
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    const float sc = mx > 0.0f ? ldexpf(1.0f, 15 - ex) : 1.0f;
    if (live && cols_ok) {
      half_t h[CPL], l[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const float x = st.w[k] * sc;
        h[k] = (half_t)x;
        l[k] = (half_t)(x - (float)h[k]);
      }
      const int64_t o = (int64_t)g * a.m * 32 + r * 32;
#pragma unroll
      for (int k = 0; k < CPL; k += 8) {
        *(uint4*)(a.Eh + o + k) = *(const uint4*)(h + k);
        *(uint4*)(a.El + o + k) = *(const uint4*)(l + k);
      }
      if (g == 0) a.einv[r] = 1.0f / sc;
    }
  }
  if (live && cols_ok) {
    float* erow = a.E + r * a.lde + a.ecol + g * CPL;
#pragma unroll
    for (int k = 0; k < CPL; k += 4) *(float4*)(erow + k) = make_float4(st.w[k], st.w[k + 1], st.w[k + 2], st.w[k + 3]);
    uint8_t* crow = a.codes + r * a.d + a.j0 + g * CPL;
    *(uint4*)(crow) = make_uint4(st.cw[0], st.cw[1], st.cw[2], st.cw[3]);
    *(uint4*)(crow + 16) = make_uint4(st.cw[4], st.cw[5], st.cw[6], st.cw[7]);
  }
  // row sum of err^2 / 2 over the quad
  float es = st.esum;
  es += quad_xor1(es);
  es += quad_xor2(es);
  if (live && g == 0 && a.err_sq) a.err_sq[r] = (a.first ? 0.0f : a.err_sq[r]) + 0.5f * es;
}

}  // namespace

template <int G, bool RF>
gptq_status_t launch_colloop(const ColArgs& a, hipStream_t st) {
  TraceScope tr(st, GPTQ_TRACE_COLLOOP);
  hipLaunchKernelGGL((colloop_kernel<G, RF>), dim3((unsigned)ceil_div(a.m, CL_THREADS / 4)), dim3(CL_THREADS), 0, st, a);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
