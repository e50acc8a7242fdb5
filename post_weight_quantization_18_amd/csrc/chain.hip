// Inverse-Hessian factor U = chol_upper((H + lambda I)^-1) in fp64 on gfx950.
//
// FDE Interviews breakdown of GPTQ, figure "Quantize a column, correct the
// rest", step 2 (U = chol(H^-1)) and section 01 (Cholesky for stability);
// nubint review, "Proposed method" (Cholesky reformulation and dampening).
//
// With J the reversal permutation and L L^T = J H_d J (lower Cholesky),
// H_d = (J L J)(J L J)^T with J L J upper, so H_d^-1 = U^T U for
// U = (J L J)^-1 = J L^-1 J: upper with a positive diagonal, hence THE factor.
// This costs a Cholesky and a triangular inverse (2 d^3 / 3 flops) instead of
// Cholesky, inverse and a second Cholesky.
//
// Work matrix A (fp64, d x d, row-major, lda = d) holds J H_d J (lower), then L,
// then L^-1, in place; its strictly upper triangle is kept at zero.
// Blocked right-looking Cholesky with 64-wide panels:
//   panel: the diagonal block is factored and inverted in LDS (the inverse
//          serves the panel solve and the inverse pass), and the panel rows
//          become A21 <- A21 L11^-T (fp64 MFMA), in one launch;
//   syrk:  A22 <- A22 - A21 A21^T on lower 64x64 tiles (v_mfma_f64_16x16x4).
// Triangular inverse by recursive doubling: the 64x64 diagonal blocks hold
// their inverses from the panel step; then for s = 64, 128, ... every pair of adjacent
// inverted s-blocks [[A, 0], [B, C]] is merged with
//   N21 = -C^-1 (B A^-1)
// as two batched fp64-MFMA launches per level (log2(d/64) levels), instead of
// a sequential sweep over the d/64 block columns.
#include <utility>

#include "common.h"

namespace gptq {

namespace {

constexpr int NB = 64;  // panel width

struct ChainWs {
  double* A;     // d x d
  double* Dinv;  // d x NB: inverse of each diagonal block (rows k0..k0+63)
  double* T;     // d x smax: B A^-1 of the pairs being merged
  double* lam;   // 1
};

// Outer panel width of the Cholesky: 8 NB panels (512 columns) per delayed
// trailing update.
int64_t chain_outer_panel(int64_t d) {
  (void)d;
  return 8 * NB;
}

// Largest merge size s (a power-of-two multiple of NB with s < d).
int64_t chain_smax(int64_t d) {
  int64_t s = NB;
  while (2 * s < d) s *= 2;
  return s;
}

ChainWs chain_ws(void* ws, int64_t d) {
  ChainWs w;
  char* p = (char*)ws;
  w.A = (double*)p;
  p += (size_t)d * d * sizeof(double);
  w.Dinv = (double*)p;
  p += (size_t)d * NB * sizeof(double);
  w.T = (double*)p;
  p += (size_t)d * chain_smax(d) * sizeof(double);
  w.lam = (double*)p;
  return w;
}

// lambda = damp * mean(diag H); also clears *info. One workgroup, fixed order.
__global__ __launch_bounds__(256) void damp_kernel(const void* H, int h_f64, int64_t d, int64_t ldh, double damp,
                                                   double* lam, double* lambda_out, int32_t* info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256)
    s += h_f64 ? ((const double*)H)[i * ldh + i] : (double)((const float*)H)[i * ldh + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double l = damp * red[0] / (double)d;
    *lam = l;
    if (lambda_out) *lambda_out = l;
    *info = 0;
  }
}

// A[i][j] = H_sym[d-1-i][d-1-j] (+ lambda on the diagonal) for i >= j, else 0.
// H holds its lower triangle, so H_sym[d-1-i][d-1-j] = H[d-1-j][d-1-i] there.
// 32x32 tiles through LDS keep both the read and the write coalesced.
__global__ __launch_bounds__(256) void load_reversed_kernel(const void* H, int h_f64, int64_t d, int64_t ldh,
                                                            const double* lam, double* A) {
  __shared__ double tile[32][33];
  const int64_t bi = blockIdx.y, bj = blockIdx.x;  // A tile (rows bi*32.., cols bj*32..)
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (bj > bi) {
    for (int r = ty; r < 32; r += 8) {
      int64_t i = bi * 32 + r, j = bj * 32 + tx;
      if (i < d && j < d) A[i * d + j] = 0.0;
    }
    return;
  }
  // A[i][j] with i in tile rows, j in tile cols reads H[d-1-j][d-1-i]:
  // H rows come from A's columns. Load H rows hr = d-1-(bj*32+r), cols hc = d-1-(bi*32+tx).
  for (int r = ty; r < 32; r += 8) {
    int64_t hr = d - 1 - (bj * 32 + r), hc = d - 1 - (bi * 32 + tx);
    double v = 0.0;
    if (hr >= 0 && hc >= 0 && hc <= hr)
      v = h_f64 ? ((const double*)H)[hr * ldh + hc] : (double)((const float*)H)[hr * ldh + hc];
    else if (hr >= 0 && hc >= 0)  // hc > hr only inside diagonal tiles: mirror
      v = h_f64 ? ((const double*)H)[hc * ldh + hr] : (double)((const float*)H)[hc * ldh + hr];
    tile[r][tx] = v;
  }
  __syncthreads();
  const double l = *lam;
  for (int r = ty; r < 32; r += 8) {
    int64_t i = bi * 32 + r, j = bj * 32 + tx;
    if (i >= d || j >= d) continue;
    double v = (j <= i) ? tile[tx][r] : 0.0;  // A[i][j] = H[d-1-j][d-1-i] = tile[j-row][i-col]
    if (i == j) v += l;
    A[i * d + j] = v;
  }
}

// One 64x64 fp64 MFMA tile step: acc[2][2] += As[rows][k..k+15] * Bs[k..k+15][cols]
// for a wave's 32x32 sub-tile. As is [64][KT+1] (row, k); Bs is [KT][64+1] (k, col).
// v_mfma_f64_16x16x4: A lane l holds A[l%16][l/16], B lane l holds B[l/16][l%16],
// D lane l, reg r holds D[l/16 + 4r][l%16].
template <int KT>
__device__ inline void mfma_f64_block(const double (*As)[KT + 1], const double (*Bs)[64 + 1], int wr, int wc,
                                      int lane, double4v (&acc)[2][2]) {
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int k = 0; k < KT; k += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) av[a] = As[wr + a * 16 + li][k + lk];
#pragma unroll
    for (int b = 0; b < 2; ++b) bv[b] = Bs[k + lk][wc + b * 16 + li];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
  }
}

// Delayed Cholesky update of one 64 x 64 tile (row tile ti, column tile tj
// from c0): A[i][j] -= sum_{k in [ka, ka + K)} A[i][k] A[j][k] for i < d,
// j < c1, j <= i (the strictly upper triangle stays zero). 4 waves of 32 x 32
// (fp64 MFMA 16x16x4); K is staged KT columns at a time through the caller's
// LDS (As [64][KT + 1], Bs [KT][64 + 1]) with the next slice prefetched into
// registers.
template <int KT>
__device__ __forceinline__ void update_tile(double* A, int64_t d, int64_t ka, int64_t K, int64_t c0, int64_t c1,
                                            int ti, int tj, double (*As)[KT + 1], double (*Bs)[64 + 1]) {
  const int64_t i0 = c0 + (int64_t)ti * 64, j0 = c0 + (int64_t)tj * 64;
  GPTQ_DASSERT(ti >= tj && i0 < d && j0 < c1 && ka >= 0 && ka + K <= d);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  double4v acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = (double4v){0.0, 0.0, 0.0, 0.0};
  const int64_t ke = ka + K;
  // each thread stages 8 elements of each 64 x KT panel, rows idx / KT, columns idx % KT
  double pa[8], pb[8];
  auto fetch = [&](int64_t k) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      const int r = idx / KT, c = idx % KT;
      const int64_t gk = k + c;
      pa[e] = (i0 + r < d && gk < ke) ? A[(i0 + r) * d + gk] : 0.0;
      pb[e] = (j0 + r < c1 && gk < ke) ? A[(j0 + r) * d + gk] : 0.0;
    }
  };
  fetch(ka);
  for (int64_t k = ka; k < ke; k += KT) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      As[idx / KT][idx % KT] = pa[e];
      Bs[idx % KT][idx / KT] = pb[e];
    }
    __syncthreads();
    if (k + KT < ke) fetch(k + KT);
    mfma_f64_block<KT>(As, Bs, wr, wc, lane, acc);
  }
  // all 16 old values are read before any is written: one memory round trip
  // for the read-modify-write instead of one per element
  double old[2][2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + x * 16 + (lane >> 4) + 4 * r;
        const int64_t j = j0 + wc + y * 16 + (lane & 15);
        old[x][y][r] = (i < d && j < c1 && j <= i) ? A[i * d + j] : 0.0;
      }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + x * 16 + (lane >> 4) + 4 * r;
        const int64_t j = j0 + wc + y * 16 + (lane & 15);
        if (i < d && j < c1 && j <= i) A[i * d + j] = old[x][y][r] - acc[x][y][r];
      }
}

// The update above over a grid of tiles.
// tri = 1: c1 = d and blockIdx.x enumerates the lower triangle of tiles;
// tri = 0: grid (column tiles, row tiles), tiles above the diagonal exit.
__global__ __launch_bounds__(256) void update_f64_kernel(double* A, int64_t d, int64_t ka, int64_t K, int64_t c0,
                                                         int64_t c1, int tri) {
  constexpr int KT = 32;
  __shared__ double As[64][KT + 1];
  __shared__ double Bs[KT][64 + 1];
  int ti, tj;
  if (tri) {
    const int t = blockIdx.x;
    ti = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    tj = t - ti * (ti + 1) / 2;
  } else {
    tj = blockIdx.x;
    ti = blockIdx.y;
    if (ti < tj) return;  // uniform per workgroup
  }
  update_tile<KT>(A, d, ka, K, c0, c1, ti, tj, As, Bs);
}

// The trailing update of an outer panel on wide tiles: A[i][j] -= sum over
// k in [ka, ka + K) of A[i][k] A[j][k] for i, j in [c0, d), j <= i, on TR x TC
// tiles of (TR / 32) x (TC / 32) waves of 32 x 32 (fp64 MFMA 16x16x4). K is
// staged KT columns at a time through LDS with the next slice prefetched into
// registers; DB = 1 keeps two LDS buffers (one barrier per slice), DB = 0 one
// buffer (two barriers). Tile t lies in row tile ti with M (ti + 1) column
// tiles, M = TR / TC, so the tiles before row ti number M ti (ti + 1) / 2.
// Measured against the 64 x 64 kernel on trailing blocks of 32256 / 8192 /
// 2048: 128 x 128 KT16 DB 70.4 / 62.7 / 34.5 % of the fp64 peak, 128 x 64 KT32
// 68.6 / 64.2 / 31.3 %, 64 x 64 62.5 / 60.3 / 37.8 %.
template <int TR, int TC, int KT, int DB>
__global__ __launch_bounds__(TR * TC / 16) void update_wide_kernel(double* A, int64_t d, int64_t ka, int64_t K,
                                                                   int64_t c0) {
  constexpr int NTH = TR * TC / 16;
  constexpr int NBUF = DB ? 2 : 1;
  constexpr int M = TR / TC;
  constexpr int WC = TC / 32;
  constexpr int PA = TR * KT / NTH, PB = TC * KT / NTH;
  static_assert(PA >= 1 && PB >= 1 && TR % TC == 0, "tile shape");
  __shared__ double As[NBUF][TR][KT + 1];
  __shared__ double Bs[NBUF][KT][TC + 1];
  const int t = blockIdx.x;
  int ti = (int)((sqrt(8.0 * t / M + 1.0) - 1.0) * 0.5);
  while ((int64_t)M * (ti + 1) * (ti + 2) / 2 <= t) ++ti;
  while ((int64_t)M * ti * (ti + 1) / 2 > t) --ti;
  const int tj = t - M * ti * (ti + 1) / 2;
  const int64_t i0 = c0 + (int64_t)ti * TR, j0 = c0 + (int64_t)tj * TC;
  GPTQ_DASSERT(tj < M * (ti + 1) && ka >= 0 && ka + K <= c0);
  if (i0 >= d) return;  // uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = (w / WC) * 32, wc = (w % WC) * 32;
  double4v acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = (double4v){0.0, 0.0, 0.0, 0.0};
  const int64_t ke = ka + K;
  double pa[PA], pb[PB];
  auto fetch = [&](int64_t k) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < PA; ++e) {
      const int idx = tid + NTH * e, r = idx / KT, c = idx % KT;
      const int64_t gk = k + c;
      pa[e] = (i0 + r < d && gk < ke) ? A[(i0 + r) * d + gk] : 0.0;
    }
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int idx = tid + NTH * e, r = idx / KT, c = idx % KT;
      const int64_t gk = k + c;
      pb[e] = (j0 + r < d && gk < ke) ? A[(j0 + r) * d + gk] : 0.0;
    }
  };
  auto store = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < PA; ++e) {
      const int idx = tid + NTH * e;
      As[b][idx / KT][idx % KT] = pa[e];
    }
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int idx = tid + NTH * e;
      Bs[b][idx % KT][idx / KT] = pb[e];
    }
  };
  // v_mfma_f64_16x16x4: A lane l holds A[l%16][l/16], B lane l holds B[l/16][l%16]
  const int li = lane & 15, lk = lane >> 4;
  auto compute = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KT; k += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) av[x] = As[b][wr + x * 16 + li][k + lk];
#pragma unroll
      for (int y = 0; y < 2; ++y) bv[y] = Bs[b][k + lk][wc + y * 16 + li];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
  };
  if constexpr (DB == 0) {
    fetch(ka);
    for (int64_t k = ka; k < ke; k += KT) {
      __syncthreads();
      store(0);
      __syncthreads();
      if (k + KT < ke) fetch(k + KT);
      compute(0);
    }
  } else {
    // slice k computes from buffer b while slice k + KT (already in registers)
    // goes into the other buffer, which every wave left at the last barrier
    fetch(ka);
    store(0);
    __syncthreads();
    if (ka + KT < ke) fetch(ka + KT);
    int b = 0;
    for (int64_t k = ka; k < ke; k += KT) {
      compute(b);
      if (k + KT < ke) {
        store(b ^ 1);
        if (k + 2 * KT < ke) fetch(k + 2 * KT);
      }
      __syncthreads();
      b ^= 1;
    }
  }
  // all 16 old values are read before any is written (one memory round trip)
  double old[2][2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + x * 16 + lk + 4 * r, j = j0 + wc + y * 16 + li;
        old[x][y][r] = (i < d && j <= i) ? A[i * d + j] : 0.0;
      }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + x * 16 + lk + 4 * r, j = j0 + wc + y * 16 + li;
        if (i < d && j <= i) A[i * d + j] = old[x][y][r] - acc[x][y][r];
      }
}

// Factor the 64 x 64 diagonal block at k0 (lower Cholesky) and invert the
// factor, in one workgroup of 4 waves, blocked by 16 columns so that only the
// 16-column leaves are serial. For each 16-block:
//   (1) wave 0 factors the 16 x 16 diagonal leaf and inverts it in the same
//       sweep, in registers: lanes 0-15 hold the leaf's rows, lanes 16-31 the
//       columns of its inverse (started from the identity). Step c takes the
//       pivot from lane c, its inverse square root (v_rsq_f64 + two Newton
//       steps), scales entry c of every lane, and subtracts entry c times
//       L[j][c] (read from lane j) from entry j > c: for a row lane that is the
//       Cholesky update, for an inverse lane it is forward substitution, so both
//       share one instruction stream and one set of lane reads;
//   (2) the rows below the leaf become A21 L11^-T (fp64 MFMA, a 16-row block
//       per wave);
//   (3) the lower 16 x 16 tiles of the rest take the rank-16 update
//       A22 - L21 L21^T (fp64 MFMA).
// The off-diagonal 16-blocks of L^-1 then follow block-row by block-row:
//   Li[I][J] = -Li[I][I] sum_{K=J}^{I-1} L[I][K] Li[K][J]  (fp64 MFMA).
// Then the rows below the block: workgroup b takes rows k0 + 64 (b + 1) ..
// + 63 and replaces A21 there by A21 L11^-T (fp64 MFMA). Every workgroup
// factors the block itself (it is small and latency-bound, so the copies cost
// no time) instead of waiting for one workgroup or a second launch; the
// workgroups' slab loads are issued before the factorisation and land during it.
// Workgroup 0 writes L11^-1 to Dinv and sets info (first failing order,
// k0 + c + 1). L11 itself is not written back: the triangular inverse puts
// L11^-1 in its place, and nothing reads it in between.
constexpr int LEAF = 16;
constexpr int LP = NB + 4;  // LDS pitch in doubles: the MFMA operand reads hit each bank pair at most twice

// 1 / sqrt(p) to fp64 accuracy for p > 0 (hardware estimate + two Newton steps).
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
  y = y * (1.5 - 0.5 * p * y * y);
  y = y * (1.5 - 0.5 * p * y * y);
  return y;
}

// x of lane l, as a wave-uniform value.
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// 16 x 16 blocks in LDS (pitch LP) with v_mfma_f64_16x16x4: lane l = 16 lk + li
// supplies A[li][k] and B[k][li] for k = lk of each 4-deep step, and holds
// D[lk + 4 r][li] in register r.
// acc + X Y for X 16 x 16 and Y 16 x 16.
__device__ __forceinline__ double4v mm16_nn(const double* X, const double* Y, double4v acc, int li, int lk) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(X[li * LP + 4 * s + lk], Y[(4 * s + lk) * LP + li], acc, 0, 0, 0);
  return acc;
}
// acc + sign X Z^T for X, Z 16 x 16.
template <bool NEG>
__device__ __forceinline__ double4v mm16_nt(const double* X, const double* Z, double4v acc, int li, int lk) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const double x = X[li * LP + 4 * s + lk];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(NEG ? -x : x, Z[li * LP + 4 * s + lk], acc, 0, 0, 0);
  }
  return acc;
}
__device__ __forceinline__ double4v load16(const double* P, int li, int lk) {
  double4v v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = P[(lk + 4 * r) * LP + li];
  return v;
}
__device__ __forceinline__ void store16(double* P, double4v v, int li, int lk) {
#pragma unroll
  for (int r = 0; r < 4; ++r) P[(lk + 4 * r) * LP + li] = v[r];
}

__global__ __launch_bounds__(256) void panel_kernel(double* A, int64_t d, int64_t k0, int64_t prev, int64_t pe,
                                                   int rb, double* Dinv, int32_t* info, double* Ldiag) {
  __shared__ double L[NB * LP];
  __shared__ double Li[NB * LP];
  __shared__ double Pd[NB * LP];  // panel prev's rows of the block: A[k0 + r][prev + c]
  __shared__ double Xs[NB * LP];  // panel prev's rows of the slab, then the slab itself
  __shared__ double col[64];      // leaf column broadcast
  if ((int)blockIdx.x >= rb) {
    // ---- the pending update of columns [k0 + NB, pe) by panel prev ----
    const int64_t c0 = k0 + NB;
    const int ncol = (int)((pe - c0 + 63) / 64);
    const int u = (int)blockIdx.x - rb, tj = u % ncol, ti = u / ncol;
    if (ti < tj) return;  // above the diagonal (uniform)
    update_tile<32>(A, d, prev, NB, c0, pe, ti, tj, (double(*)[33])L, (double(*)[65])Li);
    return;
  }
  const int nb = (int)((d - k0) < NB ? (d - k0) : NB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int li = lane & 15, lk = lane >> 4;
  const double* blk = A + k0 * d + k0;  // the block's (0, 0); always a valid address
  // this workgroup's slab of rows below the block (none when it is the last)
  const int64_t r0 = k0 + NB + (int64_t)blockIdx.x * NB;
  const bool has_slab = r0 < d;
  const bool upd = prev >= 0;
  // With a pending update (prev >= 0), wave 1 + v (v = 0, 1, 2) updates the
  // slab's 16-row bands v and v + 3 (so a band is read and rewritten by one
  // wave only); their old values come straight from memory in the MFMA result
  // layout: band p, column tile q, register r of lane (lk, li) holds slab row
  // 16 p + lk + 4 r, column 16 q + li.
  const bool band_wave = upd && has_slab && w > 0;
  double4v sold[2][4];
  if (band_wave) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int p = (w - 1) + 3 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = r0 + 16 * p + lk + 4 * r;
          sold[h][q][r] = (p < 4) ? A[(row < d ? row : r0) * d + k0 + 16 * q + li] : 0.0;
        }
    }
  }
  {
    // thread: column lane of rows w + 4q. The loads are unconditional (a
    // masked-off element reads a valid entry and is replaced) and all issued
    // before the first LDS write.
    double v[NB / 4], xs[NB / 4], pd[NB / 4], ps[NB / 4];
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      const int r = w + 4 * q;
      const int rr = r < nb ? r : 0, cc = lane < nb ? lane : 0;  // clamped into the block
      v[q] = blk[(int64_t)rr * d + cc];
      const int64_t sr = r0 + r < d ? r0 + r : k0;  // slab rows past d read row k0 (not stored)
      if (upd) {
        pd[q] = A[(k0 + rr) * d + prev + lane];
        if (has_slab) ps[q] = A[sr * d + prev + lane];
      } else if (has_slab) {
        xs[q] = A[sr * d + k0 + lane];
      }
    }
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      const int r = w + 4 * q;
      const bool in = r < nb && lane <= r;
      L[r * LP + lane] = in ? v[q] : (r == lane ? 1.0 : 0.0);  // identity padding past d
      Li[r * LP + lane] = 0.0;
      if (upd) {
        Pd[r * LP + lane] = r < nb ? pd[q] : 0.0;
        if (has_slab) Xs[r * LP + lane] = ps[q];  // panel prev's slab rows, replaced band by band
      } else if (has_slab) {
        Xs[r * LP + lane] = xs[q];
      }
    }
  }
  __syncthreads();
  if (upd) {
    // ---- block column k0 takes panel prev's update (the rest of its outer
    // panel is done by the extra workgroups): block -= Pd Pd^T, slab -= Ps Pd^T.
    // Wave 0 updates only the first 16 x 16 tile and goes on to factor it;
    // waves 1-3 update the other lower tiles of the block and the slab
    // meanwhile, and the barrier after the first leaf joins them. Every tile
    // and band is read and written by one wave. Rows of the block past d stay
    // identity (the Pd rows past nb are zero); the upper tiles are not needed
    // (the factorisation reads the lower triangle only). ----
    if (w == 0) {
      double4v t = load16(&L[0], li, lk);
#pragma unroll
      for (int kb = 0; kb < NB; kb += 16) t = mm16_nt<true>(&Pd[kb], &Pd[kb], t, li, lk);
      store16(&L[0], t, li, lk);
    } else {
      // the 9 lower tiles other than (0, 0): (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
      for (int tix = w - 1; tix < 9; tix += 3) {
        const int p = tix < 2 ? 1 : (tix < 5 ? 2 : 3);
        const int q = tix - (p == 1 ? 0 : (p == 2 ? 2 : 5));
        double* T = &L[16 * p * LP + 16 * q];
        double4v t = load16(T, li, lk);
#pragma unroll
        for (int kb = 0; kb < NB; kb += 16) t = mm16_nt<true>(&Pd[16 * p * LP + kb], &Pd[16 * q * LP + kb], t, li, lk);
        store16(T, t, li, lk);
      }
      if (band_wave) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int p = (w - 1) + 3 * h;
          if (p < 4) {
            double4v sb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              sb[q] = sold[h][q];
#pragma unroll
              for (int kb = 0; kb < NB; kb += 16)
                sb[q] = mm16_nt<true>(&Xs[16 * p * LP + kb], &Pd[16 * q * LP + kb], sb[q], li, lk);
            }
            // the wave's reads of its band precede these writes (one wave, in order)
#pragma unroll
            for (int q = 0; q < 4; ++q) store16(&Xs[16 * p * LP + 16 * q], sb[q], li, lk);
          }
        }
      }
    }
  }
  int first_bad = -1;  // first failing pivot of the block (wave 0)
  for (int b0 = 0; b0 < NB; b0 += LEAF) {
    // ---- (1) leaf factor and inverse (wave 0; lanes 32-63 repeat 0-31) ----
    if (w == 0) {
      const int t = li;
      const bool inv = (lane & 16) != 0;
      double g[LEAF];
#pragma unroll
      for (int j = 0; j < LEAF; ++j) {
        const double a = L[(b0 + t) * LP + b0 + j];
        g[j] = inv ? (j == t ? 1.0 : 0.0) : (j <= t ? a : 0.0);
      }
      // Step c updates entry c + 1 at once, with L[c + 1][c] read from lane
      // c + 1, and entries c + 2 .. 15 during step c + 1, where they overlap
      // that pivot's inverse square root; their L[j][c] come through LDS (one
      // write, broadcast reads issued in step c, a whole step before use).
      // The pivot chain is short: lane c + 1 holds L[c + 1][c] itself, so its
      // updated diagonal, the next pivot, needs no broadcast; a failing pivot
      // is replaced by 1 after the rsqrt, off the chain.
      double colv[LEAF];
      double vprev = 0.0;
      double p = readlane_f64(g[0], 0);
#pragma unroll
      for (int c = 0; c < LEAF; ++c) {
        double rs = rsqrt_f64(p);
        const bool bad = !(p > 0.0);  // not positive definite (or NaN): go on with 1
        rs = bad ? 1.0 : rs;
        first_bad = (bad && first_bad < 0) ? b0 + c : first_bad;
        if (c > 0) {
#pragma unroll
          for (int j = c + 1; j < LEAF; ++j) g[j] = fma(-vprev, colv[j], g[j]);
        }
        const double vc = g[c] * rs;  // L[t][c] (row lanes) or Li[c][t] (inverse lanes)
        g[c] = vc;
        if (c + 1 < LEAF) {
          // lane c + 1 holds L[c + 1][c] itself: its updated diagonal is the next pivot
          p = readlane_f64(fma(-vc, vc, g[c + 1]), c + 1);
          g[c + 1] = fma(-vc, readlane_f64(vc, c + 1), g[c + 1]);
        }
        if (c + 2 < LEAF) {
          col[lane] = vc;  // the wave's LDS accesses stay in order: the reads see this write
#pragma unroll
          for (int j = c + 2; j < LEAF; ++j) colv[j] = col[j];
        }
        vprev = vc;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (lane < LEAF) {
#pragma unroll
        for (int j = 0; j < LEAF; ++j) L[(b0 + t) * LP + b0 + j] = (j <= t) ? g[j] : 0.0;
      } else if (lane < 2 * LEAF) {
#pragma unroll
        for (int c = 0; c < LEAF; ++c) Li[(b0 + c) * LP + b0 + t] = (c >= t) ? g[c] : 0.0;
      }
    }
    __syncthreads();
    const int nrb = (NB - b0 - LEAF) / LEAF;  // 16-row blocks below the leaf
    if (nrb <= 0) break;
    // ---- (2) rows below: A21 <- A21 L11^-T, one 16-row block per wave ----
    if (w < nrb) {
      double* X = &L[(b0 + LEAF + LEAF * w) * LP + b0];
      const double4v z = {0.0, 0.0, 0.0, 0.0};
      const double4v x = mm16_nt<false>(X, &Li[b0 * LP + b0], z, li, lk);
      store16(X, x, li, lk);  // the wave read its whole block into the MFMAs first
    }
    __syncthreads();
    // ---- (3) rank-16 update of the lower tiles of the rest ----
    for (int tile = w; tile < nrb * (nrb + 1) / 2; tile += 4) {
      int p = 0;
      while ((p + 1) * (p + 2) / 2 <= tile) ++p;
      const int q = tile - p * (p + 1) / 2;
      double* T = &L[(b0 + LEAF + LEAF * p) * LP + b0 + LEAF + LEAF * q];
      double4v acc = load16(T, li, lk);
      acc = mm16_nt<true>(&L[(b0 + LEAF + LEAF * p) * LP + b0], &L[(b0 + LEAF + LEAF * q) * LP + b0], acc, li, lk);
      store16(T, acc, li, lk);
    }
    __syncthreads();
  }
  // ---- off-diagonal blocks of L^-1, block-row by block-row (wave J: block J) ----
  for (int I = 1; I < NB / LEAF; ++I) {
    if (w < I) {
      const int J = w;
      double4v tmp = {0.0, 0.0, 0.0, 0.0};
      for (int K = J; K < I; ++K)
        tmp = mm16_nn(&L[LEAF * I * LP + LEAF * K], &Li[LEAF * K * LP + LEAF * J], tmp, li, lk);
      // Li[I][J] = -Li[I][I] tmp, with tmp as the B operand straight from the
      // registers: step r pairs k = lk + 4 r of both operands
      const double* D = &Li[LEAF * I * LP + LEAF * I];
      double4v out = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out = __builtin_amdgcn_mfma_f64_16x16x4f64(-D[li * LP + lk + 4 * r], tmp[r], out, 0, 0, 0);
      store16(&Li[LEAF * I * LP + LEAF * J], out, li, lk);
    }
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    if (tid == 0 && first_bad >= 0 && first_bad < nb && *info == 0) *info = (int32_t)(k0 + first_bad + 1);
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      const int r = w + 4 * q, c = lane;
      if (r < nb) Dinv[(k0 + r) * NB + c] = (c < nb && c <= r) ? Li[r * LP + c] : 0.0;
      // the factored block itself (A's diagonal block is still being read by
      // the other workgroups of this launch, so it goes to the side)
      if (Ldiag && r < nb) Ldiag[(k0 + r) * NB + c] = (c < nb && c <= r) ? L[r * LP + c] : 0.0;
    }
  }
  if (!has_slab) return;  // uniform over the workgroup
  // ---- slab: X <- X L11^-T (X in Xs since the start) ----
  {
    // wave (wr, wc): 32 x 32 of the 64 x 64 result; out[i][j] = sum_k X[i][k] Li[j][k]
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
    double4v acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = (double4v){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < NB; k += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = Xs[(wr + 16 * a + li) * LP + k + lk];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Li[(wc + 16 * b + li) * LP + k + lk];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t i = r0 + wr + 16 * a + lk + 4 * r;
          if (i < d) A[i * d + k0 + wc + 16 * b + li] = acc[a][b][r];
        }
  }
}

// Every diagonal NB-block of A <- its inverse (lower, zero upper); with the
// factored blocks in place of the inverses, A becomes L itself.
__global__ __launch_bounds__(256) void put_diag_inverse_kernel(double* A, int64_t d, const double* Dinv) {
  const int64_t k0 = (int64_t)blockIdx.x * NB;
  const int nb = (int)((d - k0) < NB ? (d - k0) : NB);
  for (int idx = threadIdx.x; idx < nb * nb; idx += 256) {
    const int r = idx / nb, c = idx % nb;
    A[(k0 + r) * d + k0 + c] = Dinv[(k0 + r) * NB + c];
  }
}

// Merge step of the triangular inverse at block size s. Pair p covers
// rows/cols [a0, a0 + 2s): Ainv = A[a0:c0, a0:c0], Cinv = A[c0:c1, c0:c1] (both
// already inverted, lower), B = A[c0:c1, a0:c0] (still the factor L).
//   MODE 0: T[r][col - a0] = sum_{k in [col tile, c0)} B[r][k] Ainv[k][col]
//   MODE 1: A[r][col] = -sum_{k in [c0, r tile end)} Cinv[r][k] T[k][col - a0]
// grid: x = column tile in [a0, c0), y = row tile in [c0, c1), z = pair.
// KG groups of 4 waves split each tile's K range into equal KT-aligned parts
// (the last padded with zeros, so every group runs the same iterations) and
// the groups' tiles are summed in LDS in group order: at small d the longest
// K range, not the tile count, sets the launch's time.
template <int MODE, int KG>
__global__ __launch_bounds__(256 * KG) void merge_kernel(double* A, int64_t d, double* T, int64_t ldt, int64_t s) {
  constexpr int KT = 32;
  constexpr int AS = 64 * (KT + 1), BS = KT * (64 + 1);  // one group's A and B stages
  static_assert(KG == 1 || (KG - 1) * 64 * 64 <= KG * (AS + BS), "the partial tiles fit in the stages");
  __shared__ double smem[KG * (AS + BS)];
  const int64_t a0 = (int64_t)blockIdx.z * 2 * s, c0 = a0 + s;
  int64_t c1 = a0 + 2 * s;
  if (c1 > d) c1 = d;
  const int64_t r0 = c0 + (int64_t)blockIdx.y * 64;
  const int64_t col0 = a0 + (int64_t)blockIdx.x * 64;
  if (c0 >= d || r0 >= c1) return;  // uniform per workgroup
  int64_t kb, ke;
  if (MODE == 0) {
    kb = col0;
    ke = c0;
  } else {
    kb = c0;
    ke = r0 + 64 < c1 ? r0 + 64 : c1;
  }
  const int g = (int)(threadIdx.x >> 8);  // K group
  const int tid = threadIdx.x & 255, lane = tid & 63, w = tid >> 6;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  const int64_t part = (ke - kb + KG * KT - 1) / (KG * KT) * KT;  // K per group, a multiple of KT
  const int64_t gb = kb + g * part;
  const int64_t ge = gb + part < ke ? gb + part : ke;  // may be empty for the last groups
  double4v acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (double4v){0.0, 0.0, 0.0, 0.0};
  // each thread stages 8 elements of the A tile (64 x KT) and 8 of the B tile (KT x 64)
  double pa[8], pb[8];
  auto fetch = [&](int64_t k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      const int ar = idx / KT, ac = idx % KT;
      const int64_t gr = r0 + ar, gk = k + ac;
      pa[e] = (gr < c1 && gk < ge) ? A[gr * d + gk] : 0.0;
      const int br = idx / 64, bc = idx % 64;
      const int64_t bk = k + br, gc = col0 + bc;
      double v = 0.0;
      if (bk < ge && gc < c0) v = (MODE == 0) ? A[bk * d + gc] : T[bk * ldt + (gc - a0)];
      pb[e] = v;
    }
  };
  double (*As)[KT + 1] = (double(*)[KT + 1])(smem + g * AS);
  double (*Bs)[64 + 1] = (double(*)[64 + 1])(smem + KG * AS + g * BS);
  fetch(gb);
  for (int64_t k = 0; k < part; k += KT) {  // the same count in every group
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      As[idx / KT][idx % KT] = pa[e];
      Bs[idx / 64][idx % 64] = pb[e];
    }
    __syncthreads();
    if (k + KT < part) fetch(gb + k + KT);
    mfma_f64_block<KT>(As, Bs, wr, wc, lane, acc);
  }
  if constexpr (KG > 1) {
    // groups 1 .. KG-1 leave their 64 x 64 tiles in the (now free) stages;
    // group 0 adds them in group order and alone writes the result
    __syncthreads();
    if (g > 0) {
      double* mine = smem + (g - 1) * 64 * 64;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mine[(wr + a * 16 + (lane >> 4) + 4 * r) * 64 + wc + b * 16 + (lane & 15)] = acc[a][b][r];
    }
    __syncthreads();
    if (g > 0) return;
#pragma unroll
    for (int h = 0; h < KG - 1; ++h)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[a][b][r] += smem[h * 64 * 64 + (wr + a * 16 + (lane >> 4) + 4 * r) * 64 + wc + b * 16 + (lane & 15)];
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = r0 + wr + a * 16 + (lane >> 4) + 4 * r;
        const int64_t j = col0 + wc + b * 16 + (lane & 15);
        if (i < c1 && j < c0) {
          if (MODE == 0)
            T[i * ldt + (j - a0)] = acc[a][b][r];
          else
            A[i * d + j] = -acc[a][b][r];
        }
      }
}

// U[i][j] = A[d-1-i][d-1-j] for j >= i, else 0 (A lower holds L^-1; or L, which
// gives R = J L J instead).
__global__ __launch_bounds__(256) void store_u_kernel(const double* A, int64_t d, void* U, int u_f64, int64_t ldu) {
  const int64_t i = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256) {
    double v = (j >= i) ? A[(d - 1 - i) * d + (d - 1 - j)] : 0.0;
    if (u_f64)
      ((double*)U)[i * ldu + j] = v;
    else
      ((float*)U)[i * ldu + j] = (float)v;
  }
}

}  // namespace

size_t chain_workspace_bytes(int64_t d) {
  return (size_t)d * d * sizeof(double) + (size_t)d * NB * sizeof(double) +
         (size_t)d * chain_smax(d) * sizeof(double) + 256;
}

gptq_status_t chain_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, double damp, void* U, int u_f64,
                            int64_t ldu, int32_t* info, double* lambda_out, void* ws, size_t ws_bytes,
                            hipStream_t st, int inverse) {
  (void)ws_bytes;
  ChainWs w = chain_ws(ws, d);
  {
  TraceScope tr(st, GPTQ_TRACE_CHAIN_LOAD);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, H, h_f64, d, ldh, damp, w.lam, lambda_out, info);
  GPTQ_CHECK_LAUNCH();
  const int64_t nt32 = ceil_div(d, 32);
  hipLaunchKernelGGL(load_reversed_kernel, dim3((unsigned)nt32, (unsigned)nt32), dim3(256), 0, st, H, h_f64, d,
                     ldh, (const double*)w.lam, w.A);
  GPTQ_CHECK_LAUNCH();
  }
  // Blocked right-looking Cholesky in two levels: NB-wide panels are factored
  // (panel_kernel) inside outer panels of CP columns, each NB panel updating
  // only the rest of its outer panel; the trailing matrix receives one update
  // of depth CP per outer panel, so it is read and written d / CP times instead
  // of d / NB times.
  const int64_t nblk = ceil_div(d, NB);
  const int64_t CP = chain_outer_panel(d);
  for (int64_t p0 = 0; p0 < d; p0 += CP) {
    const int64_t pe = p0 + CP < d ? p0 + CP : d;
    for (int64_t k0 = p0; k0 < pe; k0 += NB) {
      // one launch per panel: rb workgroups factor block k0 (each first
      // applying panel k0 - NB's update to its part of block column k0) and
      // solve the rows below; the others apply panel k0 - NB's update to the
      // columns [k0 + NB, pe) of the outer panel
      const int64_t rest = d - k0 - NB;
      const int64_t rb = rest > 0 ? ceil_div(rest, 64) : 1;
      const int64_t prev = k0 > p0 ? k0 - NB : -1;
      const int64_t c0 = k0 + NB;
      const int64_t nupd = (prev >= 0 && c0 < pe) ? ceil_div(pe - c0, 64) * ceil_div(d - c0, 64) : 0;
      {
        TraceScope tr(st, GPTQ_TRACE_CHAIN_PANEL);
        hipLaunchKernelGGL(panel_kernel, dim3((unsigned)(rb + nupd)), dim3(256), 0, st, w.A, d, k0, prev, pe,
                           (int)rb, w.Dinv, info, inverse ? (double*)nullptr : w.T);
        GPTQ_CHECK_LAUNCH();
      }
      if (rest <= 0) break;
    }
    if (pe < d) {
      // the tile shape by the trailing block's size (measured on 32256 / 8192 / 2048)
      const int64_t nrest = d - pe;
      TraceScope tr(st, GPTQ_TRACE_CHAIN_UPDATE);
      if (nrest >= 16384) {
        const int64_t nr = ceil_div(nrest, 128);
        hipLaunchKernelGGL((update_wide_kernel<128, 128, 16, 1>), dim3((unsigned)(nr * (nr + 1) / 2)), dim3(1024), 0,
                           st, w.A, d, p0, pe - p0, pe);
      } else if (nrest >= 4096) {
        const int64_t nr = ceil_div(nrest, 128);
        hipLaunchKernelGGL((update_wide_kernel<128, 64, 32, 0>), dim3((unsigned)(nr * (nr + 1))), dim3(512), 0, st,
                           w.A, d, p0, pe - p0, pe);
      } else {
        const int64_t rb = ceil_div(nrest, 64);
        hipLaunchKernelGGL(update_f64_kernel, dim3((unsigned)(rb * (rb + 1) / 2)), dim3(256), 0, st, w.A, d, p0,
                           pe - p0, pe, d, 1);
      }
      GPTQ_CHECK_LAUNCH();
    }
  }
  if (!inverse) {
    // R = J L J: put the factored diagonal blocks (kept in T) into A
    TraceScope tr(st, GPTQ_TRACE_CHAIN_PANEL);
    hipLaunchKernelGGL(put_diag_inverse_kernel, dim3((unsigned)nblk), dim3(256), 0, st, w.A, d, (const double*)w.T);
    GPTQ_CHECK_LAUNCH();
  }
  // the triangular inverse (only for U): the diagonal blocks' inverses, then
  // recursive doubling
  if (inverse) {
    {
      TraceScope tr(st, GPTQ_TRACE_CHAIN_MERGE);
      hipLaunchKernelGGL(put_diag_inverse_kernel, dim3((unsigned)nblk), dim3(256), 0, st, w.A, d,
                         (const double*)w.Dinv);
      GPTQ_CHECK_LAUNCH();
    }
    const int64_t ldt = chain_smax(d);
    for (int64_t s = NB; s < d; s *= 2) {
      const int64_t pairs = ceil_div(d, 2 * s);
      dim3 grid((unsigned)(s / 64), (unsigned)(s / 64), (unsigned)pairs);
      // a grid that cannot fill the GPU splits each tile's K range over 2 wave
      // groups; counted are the tiles that have work (the last pair may be
      // partial or past d)
      int64_t active = 0;
      for (int64_t pr = 0; pr < pairs; ++pr) {
        const int64_t c0 = pr * 2 * s + s, c1 = pr * 2 * s + 2 * s < d ? pr * 2 * s + 2 * s : d;
        if (c0 < d) active += (s / 64) * ceil_div(c1 - c0, 64);
      }
      TraceScope tr(st, GPTQ_TRACE_CHAIN_MERGE);
      if (active < 512) {
        hipLaunchKernelGGL((merge_kernel<0, 2>), grid, dim3(512), 0, st, w.A, d, w.T, ldt, s);
        GPTQ_CHECK_LAUNCH();
        hipLaunchKernelGGL((merge_kernel<1, 2>), grid, dim3(512), 0, st, w.A, d, w.T, ldt, s);
        GPTQ_CHECK_LAUNCH();
      } else {
        hipLaunchKernelGGL((merge_kernel<0, 1>), grid, dim3(256), 0, st, w.A, d, w.T, ldt, s);
        GPTQ_CHECK_LAUNCH();
        hipLaunchKernelGGL((merge_kernel<1, 1>), grid, dim3(256), 0, st, w.A, d, w.T, ldt, s);
        GPTQ_CHECK_LAUNCH();
      }
    }
  }
  // U = J L^-1 J, or without the inverse pass R = J L J (upper, H_d = R R^T)
  TraceScope tr(st, GPTQ_TRACE_CHAIN_STORE);
  hipLaunchKernelGGL(store_u_kernel, dim3((unsigned)ceil_div(d, 256) < 64 ? (unsigned)ceil_div(d, 256) : 64u,
                                          (unsigned)d),
                     dim3(256), 0, st, (const double*)w.A, d, U, u_f64, ldu);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
