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

#include "quant_shared.h"

namespace gptq {

namespace {

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
  float* Acc;       // R form: m x d accumulator of the pushes from earlier blocks
  float* Ubb;       // R form: nblocks x BLK x BLK inverses of R's diagonal blocks
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
  if (group > 0 && BLK % group != 0) {
    // a group must never straddle two super-blocks: S a multiple of lcm(BLK, group)
    int64_t a = BLK, bb = group;
    while (bb) {
      const int64_t t = a % bb;
      a = bb;
      bb = t;
    }
    const int64_t l = BLK / a * group;
    s = ceil_div(s, l) * l;
  }
  return s;
}

QuantWs quant_ws(void* ws, int64_t m, int64_t d, int group, int u_f64, int rform) {
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
  w.Acc = rform ? (float*)take((size_t)m * d * sizeof(float)) : nullptr;
  w.Ubb = rform ? (float*)take((size_t)nb * BLK * BLK * sizeof(float)) : nullptr;
  return w;
}

size_t quant_ws_total(int64_t m, int64_t d, int group, int u_f64, int rform) {
  const int64_t nb = nblocks_of(d), S = sb_width(d, group);
  size_t b = align256((size_t)m * d * 4) + align256((size_t)m * S * 4) + 2 * align256((size_t)m * BLK * 2) +
             2 * align256((size_t)m * S * 2) + 2 * align256((size_t)m * 4) + align256((size_t)m * d) +
             align256((size_t)d * 4) + 2 * align256(4) + 2 * align256((size_t)nb * d * BLK * 2);
  if (u_f64) b += align256((size_t)d * d * 4);
  b += align256((size_t)d * 4);
  if (rform) b += align256((size_t)m * d * 4) + align256((size_t)nb * BLK * BLK * 4);
  return b;
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

// rdiag[j] = 1 / U_jj; in the R form U_jj = 1 / R_jj, so rdiag[j] = R_jj.
__global__ void rdiag_kernel(const float* U, int64_t d, int64_t ldu, int rform, float* rdiag) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < d; j += (int64_t)gridDim.x * blockDim.x)
    rdiag[j] = rform ? U[j * ldu + j] : 1.0f / U[j * ldu + j];
}

// x[0 .. n) = 0 (a kernel, not a memset: safe to capture in a graph).
__global__ void fill_zero_kernel(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n / 4; i += (int64_t)gridDim.x * blockDim.x)
    ((float4*)x)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) x[n - 1 - threadIdx.x] = 0.0f;
}

// R form: Ubb[b] = (R[b0:b1, b0:b1])^-1 for every 128-column block b (upper
// triangular; fp64 arithmetic from R as given, fp32 result, rows and columns
// past the block's width zero). One workgroup of 1024 threads per block; the
// inverse X is built row by row from the bottom, right-looking: once row k of
// X is final, every row i < k adds R_ik X_kc to its running sum S_ic, and row
// i is final as X_ic = (delta_ic - S_ic) / R_ii. Thread (g, c) keeps column c of
// rows 16 g .. 16 g + 15, so a step costs 16 independent FMAs per thread and
// three barriers (the sums S live in A until their row is final).
constexpr int RBI_THREADS = 1024;
__global__ __launch_bounds__(RBI_THREADS) void rblock_inverse_kernel(const void* R, int r_f64, int64_t d,
                                                                     int64_t ldr, float* Ubb) {
  __shared__ double A[BLK][BLK + 1];
  __shared__ double col[BLK];
  const int64_t b0 = (int64_t)blockIdx.x * BLK;
  const int bw = (int)((d - b0) < BLK ? (d - b0) : BLK);
  const int c = threadIdx.x & (BLK - 1), g = threadIdx.x / BLK;  // g = 0 .. 7
  constexpr int RPT = BLK / (RBI_THREADS / BLK);                  // rows per thread (16)
  auto rv = [&](int i, int k) -> double {
    const int64_t o = (b0 + i) * ldr + b0 + k;
    return r_f64 ? ((const double*)R)[o] : (double)((const float*)R)[o];
  };
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) A[g * RPT + rr][c] = 0.0;
  for (int i = bw - 1; i >= 0; --i) {
    // column i of R's block, rows 0 .. i
    if (threadIdx.x < BLK) col[threadIdx.x] = threadIdx.x <= i ? rv(threadIdx.x, i) : 0.0;
    __syncthreads();
    if (g == i / RPT && c < bw) A[i][c] = c == i ? 1.0 / col[i] : c > i ? -A[i][c] / col[i] : 0.0;
    __syncthreads();
    const double xi = A[i][c];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int r = g * RPT + rr;
      if (r < i) A[r][c] = fma(col[r], xi, A[r][c]);
    }
    __syncthreads();
  }
  float* out = Ubb + (int64_t)blockIdx.x * BLK * BLK;
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = g * RPT + rr;
    out[r * BLK + c] = (r < bw && c < bw && c >= r) ? (float)A[r][c] : 0.0f;
  }
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

// With cut set (lazy blocks also cut at group starts), the block's own strictly
// upper part is included: a sub-block [j0', j1') of the 128-block updates the
// columns [j1', ...) of its own block too.
__global__ __launch_bounds__(256) void umax_kernel(const float* U, int64_t ldu, int64_t d, int cut, uint32_t* umax) {
  const int64_t b = blockIdx.y, j0 = b * BLK, c_from = cut ? j0 : j0 + BLK;
  float mx = 0.0f;
  for (int64_t c = c_from + (int64_t)blockIdx.x * 256 + threadIdx.x; c < d; c += (int64_t)gridDim.x * 256)
    for (int k = 0; k < BLK && j0 + k < c; ++k) mx = fmaxf(mx, fabsf(U[(j0 + k) * ldu + c]));
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
//   Ut{h,l}[b][k / 32][c][k % 32] = split(U[j0 + k][c] * 2^s),  c >= j0 + BLK, k < BLK
// (with cut: c > j0 + k, the block's own strictly upper part too),
// with 2^s the power of two that puts max |U| of all far parts in [2^14, 2^15)
// (uinv = 2^-s). One 64-column chunk per workgroup, transposed through LDS.
__global__ __launch_bounds__(256) void usplit_kernel(const float* U, int64_t ldu, int64_t d, int cut,
                                                     const uint32_t* umax, half_t* Uth, half_t* Utl, float* uinv) {
  __shared__ float tile[BLK][64 + 1];
  const int64_t b = blockIdx.y, j0 = b * BLK;
  const int64_t c0 = (cut ? j0 : j0 + BLK) + (int64_t)blockIdx.x * 64;
  const float sc = u_scale(umax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) uinv[0] = 1.0f / sc;
  if (c0 >= d) return;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < BLK * 64; idx += 256) {
    const int k = idx / 64, c = idx % 64;
    tile[k][c] = (c0 + c < d && j0 + k < d && c0 + c > j0 + k) ? U[(j0 + k) * ldu + c0 + c] * sc : 0.0f;
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
  GPTQ_DASSERT(d % 32 == 0 && (d * bits) % 32 == 0 && (group == 0 || d % group == 0));
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


}  // namespace

size_t quant_workspace_bytes(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  return quant_ws_total(m, d, cfg.group_size, 0, cfg.factor == GPTQ_FACTOR_H_CHOL);
}

gptq_status_t quant_enqueue(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw, const void* U, int u_f64,
                            int64_t ldu, const gptq_qcfg_t& cfg, uint32_t* qcodes, float* scales, uint8_t* zeros,
                            float* W_hat, float* err_sq, void* ws, size_t ws_bytes, hipStream_t st,
                            const int32_t* perm, int static_groups, int32_t* g_idx) {
  const int rform = cfg.factor == GPTQ_FACTOR_H_CHOL;
  const size_t need = quant_ws_total(m, d, cfg.group_size, u_f64, rform);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  QuantWs w = quant_ws(ws, m, d, cfg.group_size, u_f64, rform);
  const int gmode = cfg.grid;
  const float maxq = gmode == GPTQ_GRID_TERNARY ? 2.0f : (float)((1 << cfg.bits) - 1);
  const int group = cfg.group_size;
  const int ngroups = group ? (int)(d / group) : 1;
  const bool stat = perm && static_groups && group > 0;
  // groups that neither divide the block nor are multiples of it (96, 160, ...):
  // the lazy blocks are also cut at group starts, so that every group starts at
  // a block start with all earlier updates applied, and is fitted there over
  // its whole width (the U form's wide-group path)
  const bool cut = !stat && group > 0 && BLK % group != 0 && group % BLK != 0;
  TraceScope tr_prep(st, GPTQ_TRACE_QUANT_PREP);
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
  hipLaunchKernelGGL(rdiag_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st, U32, d, ldu32, rform,
                     w.rdiag);
  GPTQ_CHECK_LAUNCH();
  const int64_t nblk = nblocks_of(d);
  if (rform) {
    // the inverses of R's diagonal blocks (from the factor as given, in fp64)
    // and a zero accumulator
    hipLaunchKernelGGL(rblock_inverse_kernel, dim3((unsigned)nblk), dim3(RBI_THREADS), 0, st, U, u_f64, d, ldu,
                       w.Ubb);
    GPTQ_CHECK_LAUNCH();
    const int64_t n = m * d;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(ceil_div(n / 4 + 1, 256) < 8192 ? ceil_div(n / 4 + 1, 256) : 8192)),
                       dim3(256), 0, st, w.Acc, n);
    GPTQ_CHECK_LAUNCH();
  }
  const int64_t nsplit_blk = cut ? nblk : nblk - 1;  // block rows whose far part the GEMMs read
  if (nsplit_blk > 0) {
    hipLaunchKernelGGL(umax_zero_kernel, dim3(1), dim3(64), 0, st, w.umax);
    GPTQ_CHECK_LAUNCH();
    const unsigned cgroups = (unsigned)(ceil_div(d, 256) < 16 ? ceil_div(d, 256) : 16);
    hipLaunchKernelGGL(umax_kernel, dim3(cgroups, (unsigned)nsplit_blk), dim3(256), 0, st, U32, ldu32, d, cut ? 1 : 0,
                       w.umax);
    GPTQ_CHECK_LAUNCH();
    hipLaunchKernelGGL(usplit_kernel, dim3((unsigned)ceil_div(d, 64), (unsigned)nsplit_blk), dim3(256), 0, st, U32,
                       ldu32, d, cut ? 1 : 0, (const uint32_t*)w.umax, w.Uth, w.Utl, w.uinv);
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
  tr_prep.end();

  ColArgs a;
  a.Wk = w.Wk;
  a.Acc = w.Acc;
  a.Ublk = nullptr;
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
  int first = 1;
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
  for (int64_t j0 = 0; j0 < d;) {
    // the next block: up to the next multiple of 128 (and, cut, of the group)
    int64_t jn = (j0 / BLK + 1) * BLK;
    if (cut && (j0 / group + 1) * group < jn) jn = (j0 / group + 1) * group;
    if (jn > d) jn = d;
    const int64_t b = j0 / BLK;                       // its 128-block
    const int64_t kslab0 = ((j0 % BLK) / 32) * d * 32;  // its first K-slab in the split panels of that block
    a.j0 = j0;
    a.bw = (int)(jn - j0);
    a.first = first;
    first = 0;
    j0 = jn;
    const int64_t sb0 = (a.j0 / S) * S;
    const int64_t sb1 = (sb0 + S) < d ? (sb0 + S) : d;
    a.ecol = a.j0 - sb0;
    // an inner trailing update follows: the column loop splits its own errors
    const bool inner = a.j0 + a.bw < sb1;
    a.Eh = inner ? w.Ehb : nullptr;
    a.El = inner ? w.Elb : nullptr;
    a.einv = inner ? w.einv_b : nullptr;
    gptq_status_t s;
    if (rform) {
      a.Ublk = w.Ubb + b * BLK * BLK;
      if (stat)
        s = launch_colloop<-2, true>(a, st);
      else switch (group) {
        case 0: s = launch_colloop<0, true>(a, st); break;
        case 16: s = launch_colloop<16, true>(a, st); break;
        case 32: s = launch_colloop<32, true>(a, st); break;
        case 64: s = launch_colloop<64, true>(a, st); break;
        case 128: s = launch_colloop<128, true>(a, st); break;
        default: return GPTQ_ERR_UNSUPPORTED;  // rejected by the entry point already
      }
    } else if (stat) {
      s = launch_colloop<-2, false>(a, st);
    } else switch (group) {
      case 0: s = launch_colloop<0, false>(a, st); break;
      case 16: s = launch_colloop<16, false>(a, st); break;
      case 32: s = launch_colloop<32, false>(a, st); break;
      case 64: s = launch_colloop<64, false>(a, st); break;
      case 128: s = launch_colloop<128, false>(a, st); break;
      default: s = launch_colloop<-1, false>(a, st); break;
    }
    if (s != GPTQ_OK) return s;
    // the trailing updates go to the working weights (U form) or to the
    // accumulator (R form, whose column loop hands over q - w)
    float* const tgt = rform ? w.Acc : w.Wk;
    const int64_t j1 = a.j0 + a.bw;
    if (j1 < sb1) {
      // the rest of the super-block: K = this block (split by the column loop)
      t.C = tgt + j1;
      t.Ah = w.Ehb;
      t.Al = w.Elb;
      t.rowscale = w.einv_b;
      t.Bh = w.Uth + b * d * BLK + kslab0 + j1 * 32;
      t.Bl = w.Utl + b * d * BLK + kslab0 + j1 * 32;
      t.N = sb1 - j1;
      t.K = a.bw;
      if ((s = tgemm_enqueue(t, st)) != GPTQ_OK) return s;
    } else if (j1 == sb1 && sb1 < d) {
      // every later column: K = the whole super-block
      {
        TraceScope tr(st, GPTQ_TRACE_ESPLIT);
        hipLaunchKernelGGL(esplit_kernel, dim3(egrid), dim3(256), 0, st, (const float*)w.Esb, S, m,
                           (int)(sb1 - sb0), w.Ehs, w.Els, m * 32, w.einv_s);
        GPTQ_CHECK_LAUNCH();
      }
      t.C = tgt + sb1;
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
  TraceScope tr_pack(st, GPTQ_TRACE_PACK);
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
  TraceScope tr(st, GPTQ_TRACE_PACK);
  hipLaunchKernelGGL(pack_kernel<0>, dim3((unsigned)m), dim3(256), 0, st, codes, ldc, m, d, bits, out,
                     (float*)nullptr,
                     (const float*)nullptr, (const uint8_t*)nullptr, 0, 1, (const int32_t*)nullptr, 0);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

size_t quant_workspace_bytes_u64(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  return quant_ws_total(m, d, cfg.group_size, 1, cfg.factor == GPTQ_FACTOR_H_CHOL);
}

}  // namespace gptq
