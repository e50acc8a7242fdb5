// Column-by-column GPTQ quantization with lazy 128-column blocks on gfx950.
//
// FDE Interviews breakdown of GPTQ, figure "Quantize a column, correct the
// rest", for column i: (1) round w_i to the grid -> q_i; (2) err = (w_i - q_i) /
// U_ii; (3) W[:, i+1:] -= err x U[i, i+1:]; (4) apply the updates in blocks of
// 128 columns. Section 01: every row uses the same column order and the same U.
//
// Design (MI355X):
//  * Rows are independent given U, so one lane owns one row: its 128-column
//    tile of the fp32 working weights lives in registers and the block's U
//    (128 x 128 fp32) in LDS, read as wave-uniform broadcasts. Step 3 inside
//    the block is a chain of register FMAs; the group grid (min/max) is a
//    per-lane reduction over registers, no cross-lane traffic at all.
//  * The block's errors E [m, 128] go to the workspace. The columns not yet
//    quantized are updated on the matrix cores (trail.hip) in two levels, so
//    that the fp32 weights are not re-read and re-written once per 128-column
//    block: inside a super-block of S columns (a multiple of 128 near
//    sqrt(128 d)) every block updates the rest of its super-block; at the end
//    of a super-block one GEMM with K = S updates every later column. The sum
//    applied to each column is the same as with one update per block; only the
//    order in which its terms are added differs.
//  * Codes are kept one byte per weight in the workspace and packed (with the
//    dequantized W_hat) by a final kernel.
#include <utility>

#include "common.h"

namespace gptq {

namespace {

constexpr int BLK = 128;
constexpr int CL_THREADS = 256;  // 64 rows x 4 lanes

struct QuantWs {
  float* Wk;        // m x d working weights
  float* Esb;       // m x S errors of the current super-block
  half_t* Ehb;      // m x BLK errors of one block, scaled, fp16 high part (K-tiled by 32)
  half_t* Elb;      //                                    fp16 low part
  half_t* Ehs;      // m x S errors of one super-block, scaled, fp16 high part (K-tiled by 32)
  half_t* Els;      //                                          fp16 low part
  float* einv_b;    // m: inverse of the row scale of Ehb / Elb
  float* einv_s;    // m: inverse of the row scale of Ehs / Els
  uint8_t* codes;   // m x d
  float* rdiag;     // d: 1 / U_jj
  uint32_t* umax;   // [0]: bits of max |U| over the far part of every block row
  float* uinv;      // [0]: inverse of the power-of-two scale of U's fp16 pairs
  half_t* Uth;      // nblocks x d x BLK: U[blk, c] transposed, K-tiled by 32, scaled, fp16 high
  half_t* Utl;      //                                                         fp16 low
  float* U32;       // d x d (only when U is fp64)
  int32_t* inv;     // d: position of every natural column in the quantization order
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t nblocks_of(int64_t d) { return (d + BLK - 1) / BLK; }

// Super-block width: the multiple of 128 nearest sqrt(128 d), within [256, 2048]
// (balances the weight traffic of the in-super-block updates, ~ d S, against
// that of the super-block GEMMs, ~ d^2 / S). Groups wider than a block are
// fitted at their first block on the weights of the whole group, which must by
// then carry every earlier update: S is rounded up to a multiple of such a
// group, so that no group straddles two super-blocks.
int64_t sb_width(int64_t d, int group) {
  int64_t s = (int64_t)(sqrt(128.0 * (double)d) / BLK + 0.5) * BLK;
  if (s < 2 * BLK) s = 2 * BLK;
  if (s > 16 * BLK) s = 16 * BLK;
  if (group > BLK) s = ceil_div(s, group) * group;
  return s;
}

QuantWs quant_ws(void* ws, int64_t m, int64_t d, int group, int u_f64) {
  QuantWs w;
  char* p = (char*)ws;
  const int64_t nb = nblocks_of(d), S = sb_width(d, group);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += align256(bytes);
    return q;
  };
  w.Wk = (float*)take((size_t)m * d * sizeof(float));
  w.Esb = (float*)take((size_t)m * S * sizeof(float));
  w.Ehb = (half_t*)take((size_t)m * BLK * sizeof(half_t));
  w.Elb = (half_t*)take((size_t)m * BLK * sizeof(half_t));
  w.Ehs = (half_t*)take((size_t)m * S * sizeof(half_t));
  w.Els = (half_t*)take((size_t)m * S * sizeof(half_t));
  w.einv_b = (float*)take((size_t)m * sizeof(float));
  w.einv_s = (float*)take((size_t)m * sizeof(float));
  w.codes = (uint8_t*)take((size_t)m * d);
  w.rdiag = (float*)take((size_t)d * sizeof(float));
  w.umax = (uint32_t*)take(sizeof(uint32_t));
  w.uinv = (float*)take(sizeof(float));
  w.Uth = (half_t*)take((size_t)nb * d * BLK * sizeof(half_t));
  w.Utl = (half_t*)take((size_t)nb * d * BLK * sizeof(half_t));
  w.U32 = u_f64 ? (float*)take((size_t)d * d * sizeof(float)) : nullptr;
  w.inv = (int32_t*)take((size_t)d * sizeof(int32_t));
  return w;
}

size_t quant_ws_total(int64_t m, int64_t d, int group, int u_f64) {
  const int64_t nb = nblocks_of(d), S = sb_width(d, group);
  size_t b = align256((size_t)m * d * 4) + align256((size_t)m * S * 4) + 2 * align256((size_t)m * BLK * 2) +
             2 * align256((size_t)m * S * 2) + 2 * align256((size_t)m * 4) + align256((size_t)m * d) +
             align256((size_t)d * 4) + 2 * align256(4) + 2 * align256((size_t)nb * d * BLK * 2);
  if (u_f64) b += align256((size_t)d * d * 4);
  b += align256((size_t)d * 4);
  return b;
}

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

// W (fp16 | fp32) -> fp32 working copy; for one grid per row, fit it on the
// original row. One wave per row.
// With perm set, column j of the copy is column perm[j] of W (entries outside
// [0, d) read column 0).
__global__ __launch_bounds__(256) void prep_kernel(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw,
                                                   const int32_t* perm, float* Wk, int per_row, int gmode,
                                                   float maxq, float* scales, uint8_t* zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  float vmin = INFINITY, vmax = -INFINITY;
  const bool vec = !perm && !w_f32 && (ldw % 8) == 0 && (d % 8) == 0 && (((uintptr_t)W) & 15) == 0;
  if (vec) {
    // 8 weights per lane per pass: one 16-byte load, two 16-byte stores
    const half_t* wr = (const half_t*)W + r * ldw;
    float* kr = Wk + r * d;
    for (int64_t j = 8 * lane; j < d; j += 8 * 64) {
      const half8 h = *(const half8*)(wr + j);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = (float)h[e];
        vmin = fminf(vmin, v[e]);
        vmax = fmaxf(vmax, v[e]);
      }
      *(float4*)(kr + j) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(kr + j + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  } else {
    for (int64_t j = lane; j < d; j += 64) {
      int64_t c = j;
      if (perm) {
        c = perm[j];
        if (c < 0 || c >= d) c = 0;
      }
      float v = w_f32 ? ((const float*)W)[r * ldw + c] : (float)((const half_t*)W)[r * ldw + c];
      Wk[r * d + j] = v;
      vmin = fminf(vmin, v);
      vmax = fmaxf(vmax, v);
    }
  }
  if (!per_row) return;
  for (int off = 32; off > 0; off >>= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  if (lane == 0) {
    GridFit g = fit_grid(vmin, vmax, gmode, maxq);
    scales[r] = g.s;
    zeros[r] = (uint8_t)g.z;
  }
}

// The gathering copy for an order perm when a row of W fits in CAPB bytes of
// LDS (the smallest of 8, 16, 32 and 64 KB that holds it, so that small rows
// leave room for more workgroups): one workgroup per row reads the row
// coalesced into LDS (16-byte pieces when vec), then writes column j of the
// copy from LDS entry perm[j] (entries outside [0, d) read 0). For one grid
// per row it also fits that grid on the gathered values.
template <typename T, int CAPB>
__global__ __launch_bounds__(256) void prep_gather_kernel(const T* W, int64_t m, int64_t d, int64_t ldw,
                                                          const int32_t* perm, float* Wk, int per_row, int gmode,
                                                          float maxq, float* scales, uint8_t* zeros, int vec) {
  __shared__ __attribute__((aligned(16))) T row[CAPB / sizeof(T)];
  __shared__ float red[2][4];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  if (vec) {
    const uint4* src = (const uint4*)(W + r * ldw);
    for (int64_t k = tid; k < d * (int64_t)sizeof(T) / 16; k += 256) ((uint4*)row)[k] = src[k];
  } else {
    for (int64_t j = tid; j < d; j += 256) row[j] = W[r * ldw + j];
  }
  __syncthreads();
  float vmin = INFINITY, vmax = -INFINITY;
  for (int64_t j = tid; j < d; j += 256) {
    int64_t c = perm[j];
    if (c < 0 || c >= d) c = 0;
    const float v = (float)row[c];
    Wk[r * d + j] = v;
    vmin = fminf(vmin, v);
    vmax = fmaxf(vmax, v);
  }
  if (!per_row) return;
  for (int off = 32; off > 0; off >>= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = vmin;
    red[1][tid >> 6] = vmax;
  }
  __syncthreads();
  if (tid == 0) {
    vmin = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
    vmax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    GridFit g = fit_grid(vmin, vmax, gmode, maxq);
    scales[r] = g.s;
    zeros[r] = (uint8_t)g.z;
  }
}

// Static groups: the grid of every natural group of `group` columns, fitted on
// the original weights before the column loop. One wave per row.
__global__ __launch_bounds__(256) void static_fit_kernel(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw,
                                                         int group, int gmode, float maxq, float* scales,
                                                         uint8_t* zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  const int64_t ng = d / group;
  for (int64_t k = 0; k < ng; ++k) {
    float vmin = INFINITY, vmax = -INFINITY;
    for (int64_t t = lane; t < group; t += 64) {
      const int64_t c = k * group + t;
      const float v = w_f32 ? ((const float*)W)[r * ldw + c] : (float)((const half_t*)W)[r * ldw + c];
      vmin = fminf(vmin, v);
      vmax = fmaxf(vmax, v);
    }
    for (int off = 32; off > 0; off >>= 1) {
      vmin = fminf(vmin, __shfl_xor(vmin, off));
      vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
    if (lane == 0) {
      GridFit g = fit_grid(vmin, vmax, gmode, maxq);
      scales[r * ng + k] = g.s;
      zeros[r * ng + k] = (uint8_t)g.z;
    }
  }
}

// inv[perm[j]] = j, and the group number of every natural column: j / group
// in the order, c / group with static groups, 0 for one grid per row.
__global__ __launch_bounds__(256) void order_index_kernel(const int32_t* perm, int64_t d, int group, int static_groups,
                                                          int32_t* inv, int32_t* g_idx) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256) {
    int64_t c = perm[j];
    if (c < 0 || c >= d) c = 0;
    inv[c] = (int32_t)j;
    if (g_idx) g_idx[c] = group == 0 ? 0 : (int32_t)((static_groups ? c : j) / group);
  }
}

__global__ void f64_to_f32_kernel(const double* U, int64_t d, int64_t ldu, float* U32) {
  const int64_t i = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256)
    U32[i * d + j] = (float)U[i * ldu + j];
}

__global__ void rdiag_kernel(const float* U, int64_t d, int64_t ldu, float* rdiag) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < d; j += (int64_t)gridDim.x * blockDim.x)
    rdiag[j] = 1.0f / U[j * ldu + j];
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
};

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
  float w[CPL];         // the lane's 32 working weights, then its 32 errors
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

template <int G, int I>
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
    st.w[LI] = e_own;  // the register now carries the error of column I
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
template <int G, int I>
struct Steps {
  __device__ __forceinline__ static void run(LaneState& st, const ColArgs& a, int64_t r, int g,
                                             const float (*Us)[UPITCH], const float* rdiag, int bw, const URow& cur) {
    if (I >= bw) return;
    URow nxt;
    if constexpr (I + 1 < BLK) load_urow(nxt, Us, rdiag, I + 1, g);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this step's work
    col_step<G, I>(st, a, r, g, cur);
    if constexpr (I + 1 < BLK) Steps<G, I + 1>::run(st, a, r, g, Us, rdiag, bw, nxt);
  }
};

// G = 0: one grid per row (already fitted); G = 32, 64, 128: refit at every
// group start inside the block; G = -1: groups span whole blocks, refit at the
// group's first block from the current working weights; G = -2: static groups,
// every column takes the grid of its natural group perm[j] / group (fitted
// before the loop).
template <int G>
__global__ __launch_bounds__(CL_THREADS) void colloop_kernel(ColArgs a) {
  __shared__ __attribute__((aligned(16))) float Us[BLK][UPITCH];
  __shared__ float rdiag[BLK];
  const int tid = threadIdx.x;
  const int bw = a.bw;
  // strictly upper part of the block's U (zeros on and below the diagonal)
  for (int idx = tid; idx < BLK * BLK / 4; idx += CL_THREADS) {
    const int i = idx / (BLK / 4), k4 = (idx % (BLK / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < bw && k4 < bw) v = *(const float4*)(a.U + (a.j0 + i) * a.ldu + a.j0 + k4);
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
    Steps<G, 0>::run(st, a, r, g, Us, rdiag, bw, first);
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

// Errors E[r][0 .. kw) (fp32, leading dimension lde) -> fp16 pairs with one
// power-of-two scale per row that puts max |e| in [2^14, 2^15):
//   Eh = fp16(e * 2^k), El = fp16(e * 2^k - Eh), einv[r] = 2^-k,
// stored K-tiled for the trailing GEMM: (r, k) at (k / 32) * kslab + r * 32 + k % 32.
// One wave per row.
__global__ __launch_bounds__(256) void esplit_kernel(const float* E, int64_t lde, int64_t m, int kw, half_t* Eh,
                                                     half_t* El, int64_t kslab, float* einv) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  const float* erow = E + r * lde;
  float mx = 0.0f;
  for (int k = 4 * lane; k < kw; k += 256) {
    const float4 v = *(const float4*)(erow + k);
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  int ex = 0;
  if (mx > 0.0f) frexpf(mx, &ex);
  const float sc = mx > 0.0f ? ldexpf(1.0f, 15 - ex) : 1.0f;
  for (int k = 4 * lane; k < kw; k += 256) {
    const float4 v = *(const float4*)(erow + k);
    const float x[4] = {v.x * sc, v.y * sc, v.z * sc, v.w * sc};
    half_t h[4], l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h[t] = (half_t)x[t];
      l[t] = (half_t)(x[t] - (float)h[t]);
    }
    typedef half_t half4 __attribute__((ext_vector_type(4)));
    const int64_t o = (int64_t)(k >> 5) * kslab + r * 32 + (k & 31);
    *(half4*)(Eh + o) = half4{h[0], h[1], h[2], h[3]};
    *(half4*)(El + o) = half4{l[0], l[1], l[2], l[3]};
  }
  if (lane == 0) einv[r] = 1.0f / sc;
}

// max |U[j0 + k][c]| over k < BLK, c >= j0 + BLK, over every block but the
// last: float bits of non-negative values order like integers, so atomicMax on
// the bits is exact and order-independent.
__global__ __launch_bounds__(256) void umax_zero_kernel(uint32_t* umax) {
  if (threadIdx.x == 0) umax[0] = 0u;
}

__global__ __launch_bounds__(256) void umax_kernel(const float* U, int64_t ldu, int64_t d, uint32_t* umax) {
  const int64_t b = blockIdx.y, j0 = b * BLK, j1 = j0 + BLK;
  float mx = 0.0f;
  for (int64_t c = j1 + (int64_t)blockIdx.x * 256 + threadIdx.x; c < d; c += (int64_t)gridDim.x * 256)
    for (int k = 0; k < BLK; ++k) mx = fmaxf(mx, fabsf(U[(j0 + k) * ldu + c]));
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0 && mx > 0.0f) atomicMax(&umax[0], __float_as_uint(mx));
}

__device__ inline float u_scale(const uint32_t* umax) {
  const float mx = __uint_as_float(umax[0]);
  int ex = 0;
  if (mx > 0.0f) frexpf(mx, &ex);
  return mx > 0.0f ? ldexpf(1.0f, 15 - ex) : 1.0f;
}

// Transposed, scaled fp16 hi/lo panels of the far part of each block row of U,
// K-tiled in slabs of 32 for the trailing GEMM:
//   Ut{h,l}[b][k / 32][c][k % 32] = split(U[j0 + k][c] * 2^s),  c >= j0 + BLK, k < BLK,
// with 2^s the power of two that puts max |U| of all far parts in [2^14, 2^15)
// (uinv = 2^-s). One 64-column chunk per workgroup, transposed through LDS.
__global__ __launch_bounds__(256) void usplit_kernel(const float* U, int64_t ldu, int64_t d, const uint32_t* umax,
                                                     half_t* Uth, half_t* Utl, float* uinv) {
  __shared__ float tile[BLK][64 + 1];
  const int64_t b = blockIdx.y, j0 = b * BLK, j1 = j0 + BLK;
  const int64_t c0 = j1 + (int64_t)blockIdx.x * 64;
  const float sc = u_scale(umax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) uinv[0] = 1.0f / sc;
  if (c0 >= d) return;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < BLK * 64; idx += 256) {
    const int k = idx / 64, c = idx % 64;
    tile[k][c] = (c0 + c < d) ? U[(j0 + k) * ldu + c0 + c] * sc : 0.0f;
  }
  __syncthreads();
  // each thread writes 8 consecutive k of one column: 64 cols x 16 chunks
  for (int idx = tid; idx < 64 * (BLK / 8); idx += 256) {
    const int c = idx / (BLK / 8), k8 = (idx % (BLK / 8)) * 8;
    if (c0 + c >= d) continue;
    half8 hv, lv;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = tile[k8 + t][c];
      const half_t h = (half_t)v;
      hv[t] = h;
      lv[t] = (half_t)(v - (float)h);
    }
    const int64_t o = b * d * BLK + (int64_t)(k8 >> 5) * d * 32 + (c0 + c) * 32 + (k8 & 31);
    *(half8*)(Uth + o) = hv;
    *(half8*)(Utl + o) = lv;
  }
}

// Packs one row per workgroup into the LSB-first bitstream and, when W_hat is
// given, writes W_hat = s * (code - z). With inv set the codes are in the
// quantization order and natural column c is read from position inv[c]
// (entries outside [0, d) read position 0); its group is c / group with static
// groups, else inv[c] / group. STAGE > 0: the row of codes is first copied
// into STAGE bytes of LDS (d <= STAGE, d % 16 == 0, ldc % 16 == 0), so that
// the gathered reads come from LDS.
constexpr int PACK_STAGE_MAX = 49152;
template <int STAGE>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* codes, int64_t ldc, int64_t m, int64_t d,
                                                   int bits, uint32_t* out, float* W_hat, const float* scales,
                                                   const uint8_t* zeros, int group, int ngroups,
                                                   const int32_t* inv, int static_groups) {
  __shared__ __attribute__((aligned(16))) uint8_t cs[STAGE > 0 ? STAGE : 16];
  const int64_t r = blockIdx.x;
  if (r >= m) return;
  const uint8_t* crow = codes + r * ldc;
  if constexpr (STAGE > 0) {
    for (int64_t k = threadIdx.x; k < d / 16; k += 256) *(uint4*)(cs + 16 * k) = *(const uint4*)(crow + 16 * k);
    __syncthreads();
    crow = cs;
  }
  const int64_t nwords = d * bits / 32;
  for (int64_t wd = threadIdx.x; wd < nwords; wd += 256) {
    const int64_t b0 = wd * 32;
    int64_t j = b0 / bits;
    const int64_t jend = (b0 + 31) / bits;
    uint32_t word = 0;
    for (; j <= jend; ++j) {
      const int64_t shift = j * bits - b0;
      int64_t jp = j;
      if (inv) {
        jp = inv[j];
        if (jp < 0 || jp >= d) jp = 0;
      }
      const uint32_t c = crow[jp];
      word |= shift >= 0 ? (c << shift) : (c >> (-shift));
    }
    out[r * nwords + wd] = word;
  }
  if (W_hat && (inv || (((uintptr_t)W_hat) & 15) != 0)) {
    for (int64_t j = threadIdx.x; j < d; j += 256) {
      int64_t jp = j;
      if (inv) {
        jp = inv[j];
        if (jp < 0 || jp >= d) jp = 0;
      }
      const int64_t g = group ? (static_groups ? j : jp) / group : 0;
      const float s = scales[r * ngroups + g], z = (float)zeros[r * ngroups + g];
      W_hat[r * d + j] = s * ((float)crow[jp] - z);
    }
  } else if (W_hat) {
    // 4 weights per thread per pass (d and the groups are multiples of 32, so
    // the four share a group and the accesses are aligned)
    for (int64_t j = 4 * threadIdx.x; j < d; j += 4 * 256) {
      const int64_t g = group ? j / group : 0;
      const float s = scales[r * ngroups + g], z = (float)zeros[r * ngroups + g];
      const uchar4 c = *(const uchar4*)(crow + j);
      *(float4*)(W_hat + r * d + j) =
          make_float4(s * ((float)c.x - z), s * ((float)c.y - z), s * ((float)c.z - z), s * ((float)c.w - z));
    }
  }
}

template <int G>
gptq_status_t launch_colloop(const ColArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(colloop_kernel<G>, dim3((unsigned)ceil_div(a.m, CL_THREADS / 4)), dim3(CL_THREADS), 0, st, a);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace

size_t quant_workspace_bytes(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  return quant_ws_total(m, d, cfg.group_size, 0);
}

gptq_status_t quant_enqueue(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw, const void* U, int u_f64,
                            int64_t ldu, const gptq_qcfg_t& cfg, uint32_t* qcodes, float* scales, uint8_t* zeros,
                            float* W_hat, float* err_sq, void* ws, size_t ws_bytes, hipStream_t st,
                            const int32_t* perm, int static_groups, int32_t* g_idx) {
  const size_t need = quant_ws_total(m, d, cfg.group_size, u_f64);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  QuantWs w = quant_ws(ws, m, d, cfg.group_size, u_f64);
  const int gmode = cfg.grid;
  const float maxq = gmode == GPTQ_GRID_TERNARY ? 2.0f : (float)((1 << cfg.bits) - 1);
  const int group = cfg.group_size;
  const int ngroups = group ? (int)(d / group) : 1;
  const bool stat = perm && static_groups && group > 0;
  if (perm) {
    hipLaunchKernelGGL(order_index_kernel, dim3((unsigned)(ceil_div(d, 256) < 1024 ? ceil_div(d, 256) : 1024)),
                       dim3(256), 0, st, perm, d, group, stat ? 1 : 0, w.inv, g_idx);
    GPTQ_CHECK_LAUNCH();
  }
  if (stat) {
    hipLaunchKernelGGL(static_fit_kernel, dim3((unsigned)ceil_div(m, 4)), dim3(256), 0, st, W, w_f32, m, d, ldw,
                       group, gmode, maxq, scales, zeros);
    GPTQ_CHECK_LAUNCH();
  }

  const float* U32 = (const float*)U;
  int64_t ldu32 = ldu;
  if (u_f64) {
    hipLaunchKernelGGL(f64_to_f32_kernel, dim3((unsigned)(ceil_div(d, 256) < 64 ? ceil_div(d, 256) : 64), (unsigned)d),
                       dim3(256), 0, st, (const double*)U, d, ldu, w.U32);
    GPTQ_CHECK_LAUNCH();
    U32 = w.U32;
    ldu32 = d;
  }
  hipLaunchKernelGGL(rdiag_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st, U32, d, ldu32, w.rdiag);
  GPTQ_CHECK_LAUNCH();
  const int64_t nblk = nblocks_of(d);
  if (nblk > 1) {
    hipLaunchKernelGGL(umax_zero_kernel, dim3(1), dim3(64), 0, st, w.umax);
    GPTQ_CHECK_LAUNCH();
    const unsigned cgroups = (unsigned)(ceil_div(d, 256) < 16 ? ceil_div(d, 256) : 16);
    hipLaunchKernelGGL(umax_kernel, dim3(cgroups, (unsigned)(nblk - 1)), dim3(256), 0, st, U32, ldu32, d, w.umax);
    GPTQ_CHECK_LAUNCH();
    hipLaunchKernelGGL(usplit_kernel, dim3((unsigned)ceil_div(d, 64), (unsigned)(nblk - 1)), dim3(256), 0, st, U32,
                       ldu32, d, (const uint32_t*)w.umax, w.Uth, w.Utl, w.uinv);
    GPTQ_CHECK_LAUNCH();
  }
  const int64_t row_bytes = d * (w_f32 ? 4 : 2);
  if (perm && row_bytes <= 65536) {
    const int vec = (row_bytes % 16 == 0) && ((ldw * (w_f32 ? 4 : 2)) % 16 == 0) && (((uintptr_t)W) & 15) == 0;
    const int pr = group == 0 ? 1 : 0;
    const dim3 g((unsigned)m), b(256);
#define GPTQ_GATHER(T, CAPB) \
  hipLaunchKernelGGL((prep_gather_kernel<T, CAPB>), g, b, 0, st, (const T*)W, m, d, ldw, perm, w.Wk, pr, gmode, \
                     maxq, scales, zeros, vec)
    if (w_f32) {
      if (row_bytes <= 8192) GPTQ_GATHER(float, 8192);
      else if (row_bytes <= 16384) GPTQ_GATHER(float, 16384);
      else if (row_bytes <= 32768) GPTQ_GATHER(float, 32768);
      else GPTQ_GATHER(float, 65536);
    } else {
      if (row_bytes <= 8192) GPTQ_GATHER(half_t, 8192);
      else if (row_bytes <= 16384) GPTQ_GATHER(half_t, 16384);
      else if (row_bytes <= 32768) GPTQ_GATHER(half_t, 32768);
      else GPTQ_GATHER(half_t, 65536);
    }
#undef GPTQ_GATHER
  } else {
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)ceil_div(m, 4)), dim3(256), 0, st, W, w_f32, m, d, ldw, perm,
                       w.Wk, group == 0 ? 1 : 0, gmode, maxq, scales, zeros);
  }
  GPTQ_CHECK_LAUNCH();

  ColArgs a;
  a.Wk = w.Wk;
  a.U = U32;
  a.rdiag = w.rdiag;
  a.ldu = ldu32;
  a.m = m;
  a.d = d;
  a.gmode = gmode;
  a.maxq = maxq;
  a.group = group;
  a.ngroups = ngroups;
  a.codes = w.codes;
  a.scales = scales;
  a.zeros = zeros;
  a.err_sq = err_sq;
  a.perm = perm;
  const int64_t S = sb_width(d, group);
  a.E = w.Esb;
  a.lde = S;
  const int64_t nblocks = ceil_div(d, BLK);
  TgemmArgs t;
  t.C = nullptr;
  t.ldc = d;
  t.Bh = w.Uth;
  t.Bl = w.Utl;
  t.b_block = d * BLK;
  t.b_kslab = d * 32;
  t.a_kslab = m * 32;
  t.cscale = w.uinv;
  t.M = m;
  const unsigned egrid = (unsigned)ceil_div(m, 4);
  for (int64_t b = 0; b < nblocks; ++b) {
    a.j0 = b * BLK;
    a.bw = (int)((d - a.j0) < BLK ? (d - a.j0) : BLK);
    a.first = b == 0;
    const int64_t sb0 = (a.j0 / S) * S;
    const int64_t sb1 = (sb0 + S) < d ? (sb0 + S) : d;
    a.ecol = a.j0 - sb0;
    // an inner trailing update follows: the column loop splits its own errors
    const bool inner = a.j0 + a.bw < sb1;
    a.Eh = inner ? w.Ehb : nullptr;
    a.El = inner ? w.Elb : nullptr;
    a.einv = inner ? w.einv_b : nullptr;
    gptq_status_t s;
    if (stat)
      s = launch_colloop<-2>(a, st);
    else switch (group) {
      case 0: s = launch_colloop<0>(a, st); break;
      case 32: s = launch_colloop<32>(a, st); break;
      case 64: s = launch_colloop<64>(a, st); break;
      case 128: s = launch_colloop<128>(a, st); break;
      default: s = launch_colloop<-1>(a, st); break;
    }
    if (s != GPTQ_OK) return s;
    const int64_t j1 = a.j0 + a.bw;
    if (j1 < sb1) {
      // the rest of the super-block: K = this block (split by the column loop)
      t.C = w.Wk + j1;
      t.Ah = w.Ehb;
      t.Al = w.Elb;
      t.rowscale = w.einv_b;
      t.Bh = w.Uth + b * d * BLK + j1 * 32;
      t.Bl = w.Utl + b * d * BLK + j1 * 32;
      t.N = sb1 - j1;
      t.K = a.bw;
      if ((s = tgemm_enqueue(t, st)) != GPTQ_OK) return s;
    } else if (j1 == sb1 && sb1 < d) {
      // every later column: K = the whole super-block
      hipLaunchKernelGGL(esplit_kernel, dim3(egrid), dim3(256), 0, st, (const float*)w.Esb, S, m, (int)(sb1 - sb0),
                         w.Ehs, w.Els, m * 32, w.einv_s);
      GPTQ_CHECK_LAUNCH();
      t.C = w.Wk + sb1;
      t.Ah = w.Ehs;
      t.Al = w.Els;
      t.rowscale = w.einv_s;
      t.Bh = w.Uth + (sb0 / BLK) * d * BLK + sb1 * 32;
      t.Bl = w.Utl + (sb0 / BLK) * d * BLK + sb1 * 32;
      t.N = d - sb1;
      t.K = sb1 - sb0;
      if ((s = tgemm_enqueue(t, st)) != GPTQ_OK) return s;
    }
  }
#define GPTQ_PACK(STAGE, INV)                                                                                       \
  hipLaunchKernelGGL(pack_kernel<STAGE>, dim3((unsigned)m), dim3(256), 0, st, (const uint8_t*)w.codes, d, m, d,      \
                     cfg.bits, qcodes, W_hat, (const float*)scales, (const uint8_t*)zeros, group, ngroups, INV,       \
                     stat ? 1 : 0)
  if (perm && d <= PACK_STAGE_MAX && d % 16 == 0) {
    const int32_t* inv = w.inv;
    if (d <= 8192) GPTQ_PACK(8192, inv);
    else if (d <= 16384) GPTQ_PACK(16384, inv);
    else if (d <= 32768) GPTQ_PACK(32768, inv);
    else GPTQ_PACK(PACK_STAGE_MAX, inv);
  } else {
    const int32_t* inv = perm ? (const int32_t*)w.inv : (const int32_t*)nullptr;
    GPTQ_PACK(0, inv);
  }
#undef GPTQ_PACK
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status_t pack_enqueue(const uint8_t* codes, int64_t ldc, int64_t m, int64_t d, int bits, uint32_t* out,
                           hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel<0>, dim3((unsigned)m), dim3(256), 0, st, codes, ldc, m, d, bits, out,
                     (float*)nullptr,
                     (const float*)nullptr, (const uint8_t*)nullptr, 0, 1, (const int32_t*)nullptr, 0);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

size_t quant_workspace_bytes_u64(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  return quant_ws_total(m, d, cfg.group_size, 1);
}

}  // namespace gptq
