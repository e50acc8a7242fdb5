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
//   potf2: the diagonal block is factored in LDS by one workgroup, which also
//          inverts it (the inverse serves the panel solve and the inverse pass);
//   trsm:  panel rows A21 <- A21 L11^-T (row-local, fp64 FMA);
//   syrk:  A22 <- A22 - A21 A21^T on lower 64x64 tiles (v_mfma_f64_16x16x4).
// Blocked inverse from the last block column to the first:
//   A21 <- -(L22^-1 A21) L11^-1 (trmm on the matrix cores, then a row-local
//   product), A11 <- L11^-1.
#include "common.h"

namespace gptq {

namespace {

constexpr int NB = 64;  // panel width

struct ChainWs {
  double* A;     // d x d
  double* Dinv;  // d x NB: inverse of each diagonal block (rows k0..k0+63)
  double* T;     // d x NB scratch panel
  double* lam;   // 1
};

ChainWs chain_ws(void* ws, int64_t d) {
  ChainWs w;
  char* p = (char*)ws;
  w.A = (double*)p;
  p += (size_t)d * d * sizeof(double);
  w.Dinv = (double*)p;
  p += (size_t)d * NB * sizeof(double);
  w.T = (double*)p;
  p += (size_t)d * NB * sizeof(double);
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

// Factor the diagonal block at k0 in LDS (lower Cholesky), write L11 back with a
// zero upper triangle, and write L11^-1 to Dinv. info <- first failing order.
__global__ __launch_bounds__(256) void potf2_kernel(double* A, int64_t d, int64_t k0, double* Dinv,
                                                    int32_t* info) {
  __shared__ double L[NB][NB + 1];
  __shared__ double Li[NB][NB + 1];
  const int nb = (int)((d - k0) < NB ? (d - k0) : NB);
  const int tid = threadIdx.x;
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    double v = 0.0;
    if (r < nb && c < nb && c <= r) v = A[(k0 + r) * d + k0 + c];
    if (r >= nb && r == c) v = 1.0;  // identity padding beyond the matrix
    L[r][c] = v;
  }
  __syncthreads();
  __shared__ int bad;
  if (tid == 0) bad = 0;
  for (int c = 0; c < NB; ++c) {
    __syncthreads();
    if (tid == 0) {
      double p = L[c][c];
      if (!(p > 0.0)) {
        if (!bad && c < nb) {
          bad = 1;
          if (*info == 0) *info = (int32_t)(k0 + c + 1);
        }
        p = 1.0;
      }
      L[c][c] = sqrt(p);
    }
    __syncthreads();
    const double piv = L[c][c];
    for (int r = c + 1 + tid; r < NB; r += 256) L[r][c] /= piv;
    __syncthreads();
    // trailing update of the lower part: (r, cc) with c < cc <= r
    const int m = NB - c - 1;
    for (int idx = tid; idx < m * m; idx += 256) {
      int r = c + 1 + idx / m, cc = c + 1 + idx % m;
      if (cc <= r) L[r][cc] -= L[r][c] * L[cc][c];
    }
  }
  __syncthreads();
  // inverse of the lower-triangular L: column cc by forward substitution.
  if (tid < NB) {
    const int cc = tid;
    for (int r = 0; r < NB; ++r) Li[r][cc] = 0.0;
    Li[cc][cc] = 1.0 / L[cc][cc];
    for (int r = cc + 1; r < NB; ++r) {
      double s = 0.0;
      for (int k = cc; k < r; ++k) s += L[r][k] * Li[k][cc];
      Li[r][cc] = -s / L[r][r];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    if (r < nb && c < nb) A[(k0 + r) * d + k0 + c] = (c <= r) ? L[r][c] : 0.0;
    if (k0 + r < d) Dinv[(k0 + r) * NB + c] = (c <= r && r < nb && c < nb) ? Li[r][c] : 0.0;
  }
}

// Rows i >= k0+NB: A[i][k0:k0+NB] <- A[i][k0:k0+NB] * Linv^T, i.e.
// x'[c] = sum_{c' <= c} x[c'] Linv[c][c']. 64 rows per workgroup.
__global__ __launch_bounds__(256) void trsm_rows_kernel(double* A, int64_t d, int64_t k0, const double* Dinv) {
  __shared__ double Li[NB][NB + 1];
  __shared__ double X[NB][NB + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = k0 + NB + (int64_t)blockIdx.x * NB;
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    Li[r][c] = Dinv[(k0 + r) * NB + c];
    X[r][c] = (r0 + r < d) ? A[(r0 + r) * d + k0 + c] : 0.0;
  }
  __syncthreads();
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    double s = 0.0;
    for (int k = 0; k <= c; ++k) s += X[r][k] * Li[c][k];
    if (r0 + r < d) A[(r0 + r) * d + k0 + c] = s;
  }
}

// C[i][j] -= sum_k P[i][k] P[j][k] for the lower 64x64 tiles of the trailing
// matrix (rows/cols >= c0), P = A[:, k0:k0+NB]. fp64 MFMA 16x16x4.
// Diagonal tiles update only j <= i so the upper triangle stays zero.
__global__ __launch_bounds__(256) void syrk_f64_kernel(double* A, int64_t d, int64_t k0, int64_t c0) {
  __shared__ double Pi[64][NB + 1];
  __shared__ double Pj[64][NB + 1];
  // lower tile index -> (ti, tj), tj <= ti
  const int t = blockIdx.x;
  int ti = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
  while (ti * (ti + 1) / 2 > t) --ti;
  const int tj = t - ti * (ti + 1) / 2;
  const int64_t i0 = c0 + (int64_t)ti * 64, j0 = c0 + (int64_t)tj * 64;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    Pi[r][c] = (i0 + r < d) ? A[(i0 + r) * d + k0 + c] : 0.0;
    Pj[r][c] = (j0 + r < d) ? A[(j0 + r) * d + k0 + c] : 0.0;
  }
  __syncthreads();
  const int lane = tid & 63, w = tid >> 6;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;  // wave sub-tile
  double4v acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (double4v){0.0, 0.0, 0.0, 0.0};
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
  for (int k = 0; k < NB; k += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) av[a] = Pi[wr + a * 16 + li][k + lk];
#pragma unroll
    for (int b = 0; b < 2; ++b) bv[b] = Pj[wc + b * 16 + li][k + lk];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
  }
  // D[i][j]: i = lane/16 + 4*r, j = lane%16
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + a * 16 + (lane >> 4) + 4 * r;
        const int64_t j = j0 + wc + b * 16 + (lane & 15);
        if (i < d && j < d && j <= i) A[i * d + j] -= acc[a][b][r];
      }
}

// T[i][c] = sum_{c' in [c0, i]} A[i][c'] A[c'][k0 + c] for i >= c0 = k0 + NB:
// (L22^-1, already inverted in place and lower) x (the L21 panel).
// One 64-row tile per workgroup; fp64 MFMA with 64-wide K chunks via LDS.
__global__ __launch_bounds__(256) void trmm_kernel(const double* A, int64_t d, int64_t k0, double* T) {
  __shared__ double Ai[64][64 + 1];
  __shared__ double Bp[64][NB + 1];
  const int64_t c0 = k0 + NB;
  const int64_t i0 = c0 + (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  double4v acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (double4v){0.0, 0.0, 0.0, 0.0};
  const int li = lane & 15, lk = lane >> 4;
  int64_t kend = i0 + 64;
  if (kend > d) kend = d;
  for (int64_t kc = c0; kc < kend; kc += 64) {
    __syncthreads();
    for (int idx = tid; idx < 64 * 64; idx += 256) {
      int r = idx / 64, c = idx % 64;
      Ai[r][c] = (i0 + r < d && kc + c < d) ? A[(i0 + r) * d + kc + c] : 0.0;
      Bp[r][c] = (kc + r < d) ? A[(kc + r) * d + k0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < 64; k += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = Ai[wr + a * 16 + li][k + lk];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Bp[k + lk][wc + b * 16 + li];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + a * 16 + (lane >> 4) + 4 * r;
        const int c = wc + b * 16 + (lane & 15);
        if (i < d) T[i * NB + c] = acc[a][b][r];
      }
}

// Rows i >= k0+NB: A[i][k0+c] = -sum_{c' >= c} T[i][c'] Linv[c'][c].
__global__ __launch_bounds__(256) void trsm2_rows_kernel(double* A, int64_t d, int64_t k0, const double* T,
                                                         const double* Dinv) {
  __shared__ double Li[NB][NB + 1];
  __shared__ double X[NB][NB + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = k0 + NB + (int64_t)blockIdx.x * NB;
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    Li[r][c] = Dinv[(k0 + r) * NB + c];
    X[r][c] = (r0 + r < d) ? T[(r0 + r) * NB + c] : 0.0;
  }
  __syncthreads();
  for (int idx = tid; idx < NB * NB; idx += 256) {
    int r = idx / NB, c = idx % NB;
    double s = 0.0;
    for (int k = c; k < NB; ++k) s += X[r][k] * Li[k][c];
    if (r0 + r < d) A[(r0 + r) * d + k0 + c] = -s;
  }
}

// A11 <- L11^-1 (lower, zero upper).
__global__ __launch_bounds__(256) void put_diag_inverse_kernel(double* A, int64_t d, int64_t k0, const double* Dinv) {
  const int nb = (int)((d - k0) < NB ? (d - k0) : NB);
  for (int idx = threadIdx.x; idx < nb * nb; idx += 256) {
    int r = idx / nb, c = idx % nb;
    A[(k0 + r) * d + k0 + c] = Dinv[(k0 + r) * NB + c];
  }
}

// U[i][j] = A[d-1-i][d-1-j] for j >= i, else 0 (A lower holds L^-1).
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
  return (size_t)d * d * sizeof(double) + 2 * (size_t)d * NB * sizeof(double) + 256;
}

gptq_status_t chain_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, double damp, void* U, int u_f64,
                            int64_t ldu, int32_t* info, double* lambda_out, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  ChainWs w = chain_ws(ws, d);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, H, h_f64, d, ldh, damp, w.lam, lambda_out, info);
  GPTQ_CHECK_LAUNCH();
  const int64_t nt32 = ceil_div(d, 32);
  hipLaunchKernelGGL(load_reversed_kernel, dim3((unsigned)nt32, (unsigned)nt32), dim3(256), 0, st, H, h_f64, d,
                     ldh, (const double*)w.lam, w.A);
  GPTQ_CHECK_LAUNCH();
  const int64_t nblk = ceil_div(d, NB);
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t k0 = k * NB;
    hipLaunchKernelGGL(potf2_kernel, dim3(1), dim3(256), 0, st, w.A, d, k0, w.Dinv, info);
    GPTQ_CHECK_LAUNCH();
    const int64_t rest = d - k0 - NB;
    if (rest <= 0) break;
    const int64_t rb = ceil_div(rest, 64);
    hipLaunchKernelGGL(trsm_rows_kernel, dim3((unsigned)rb), dim3(256), 0, st, w.A, d, k0, (const double*)w.Dinv);
    GPTQ_CHECK_LAUNCH();
    hipLaunchKernelGGL(syrk_f64_kernel, dim3((unsigned)(rb * (rb + 1) / 2)), dim3(256), 0, st, w.A, d, k0,
                       k0 + NB);
    GPTQ_CHECK_LAUNCH();
  }
  for (int64_t k = nblk - 1; k >= 0; --k) {
    const int64_t k0 = k * NB;
    const int64_t rest = d - k0 - NB;
    if (rest > 0) {
      const int64_t rb = ceil_div(rest, 64);
      hipLaunchKernelGGL(trmm_kernel, dim3((unsigned)rb), dim3(256), 0, st, (const double*)w.A, d, k0, w.T);
      GPTQ_CHECK_LAUNCH();
      hipLaunchKernelGGL(trsm2_rows_kernel, dim3((unsigned)rb), dim3(256), 0, st, w.A, d, k0, (const double*)w.T,
                         (const double*)w.Dinv);
      GPTQ_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(put_diag_inverse_kernel, dim3(1), dim3(256), 0, st, w.A, d, k0, (const double*)w.Dinv);
    GPTQ_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(store_u_kernel, dim3((unsigned)ceil_div(d, 256) < 64 ? (unsigned)ceil_div(d, 256) : 64u,
                                          (unsigned)d),
                     dim3(256), 0, st, (const double*)w.A, d, U, u_f64, ldu);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
