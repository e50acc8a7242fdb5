// Act-order (desc_act): the column order of descending diag(H), and the
// Hessian gathered into that order.
//
// The pages name the option and no more: the zhiliyouxian blog passes desc_act
// ("实践指南", sort the columns by their activations, off by default; default
// listed in "超参数选择") and the CSDN page "GPTQ量化参数搜索工具" lists
// --desc_act and --static_groups in its parameter table. The library reads the
// size of column j's activations as H_jj = 2 sum_t x_tj^2 and orders the
// columns by it, largest first, ties in index order.
#include "common.h"

namespace gptq {
namespace {

// Sort key of a diagonal entry: an unsigned integer in the order of the value
// (+0 and -0 taken as equal, NaNs beyond the infinities), so that the order is
// a strict total order together with the index and the ranks form a
// permutation whatever H holds.
__device__ __forceinline__ uint64_t order_key(double v) {
  if (v == 0.0) v = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// rank(i) = the number of columns that come before column i: a larger key, or
// an equal key at a lower index; perm[rank(i)] = i. One workgroup per 64
// columns (one per lane); the keys are staged through LDS 2048 at a time, the
// four waves count over a quarter of each chunk, and the four partial counts
// are added in LDS.
template <typename T>
__global__ __launch_bounds__(256) void order_rank_kernel(const T* H, int64_t d, int64_t ldh, int32_t* perm) {
  constexpr int CH = 2048;
  __shared__ uint64_t keys[CH];
  __shared__ int32_t part[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  const uint64_t ki = order_key(i < d ? (double)H[i * ldh + i] : 0.0);
  int32_t rank = 0;
  for (int64_t t0 = 0; t0 < d; t0 += CH) {
    const int n = (int)(d - t0 < CH ? d - t0 : CH);
    __syncthreads();
    for (int k = threadIdx.x; k < n; k += 256) keys[k] = order_key((double)H[(t0 + k) * ldh + t0 + k]);
    __syncthreads();
    const int q = (n + 3) / 4;
    const int kb = wv * q, ke = kb + q < n ? kb + q : n;
    const int64_t il = i - t0;  // the tie-break compares chunk-local indices
#pragma unroll 8
    for (int k = kb; k < ke; ++k) {
      const uint64_t kv = keys[k];
      rank += (kv > ki) || (kv == ki && k < il);
    }
  }
  part[wv][lane] = rank;
  __syncthreads();
  if (wv == 0 && i < d) perm[part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane]] = (int32_t)i;
}

// Hp[i][j] = H[perm[i]][perm[j]] for j <= i, read from H's lower triangle.
// One workgroup per row (grid-stride over rows). perm entries outside [0, d)
// are read as 0, so that no access leaves H whatever perm holds.
template <typename T>
__global__ __launch_bounds__(256) void permute_h_kernel(const T* H, int64_t d, int64_t ldh, const int32_t* perm,
                                                        T* Hp, int64_t ldp) {
  for (int64_t i = blockIdx.x; i < d; i += gridDim.x) {
    int64_t pi = perm[i];
    if (pi < 0 || pi >= d) pi = 0;
    for (int64_t j = threadIdx.x; j <= i; j += 256) {
      int64_t pj = perm[j];
      if (pj < 0 || pj >= d) pj = 0;
      const int64_t a = pi > pj ? pi : pj, b = pi > pj ? pj : pi;
      Hp[i * ldp + j] = H[a * ldh + b];
    }
  }
}

}  // namespace

gptq_status_t act_order_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, int32_t* perm, hipStream_t st) {
  TraceScope tr(st, GPTQ_TRACE_ORDER);
  const dim3 grid((unsigned)ceil_div(d, 64));
  if (h_f64)
    hipLaunchKernelGGL(order_rank_kernel<double>, grid, dim3(256), 0, st, (const double*)H, d, ldh, perm);
  else
    hipLaunchKernelGGL(order_rank_kernel<float>, grid, dim3(256), 0, st, (const float*)H, d, ldh, perm);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status_t permute_hessian_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, const int32_t* perm,
                                      void* Hp, int64_t ldp, hipStream_t st) {
  const dim3 grid((unsigned)(d < 16384 ? d : 16384));
  TraceScope tr(st, GPTQ_TRACE_ORDER);
  if (h_f64)
    hipLaunchKernelGGL(permute_h_kernel<double>, grid, dim3(256), 0, st, (const double*)H, d, ldh, perm,
                       (double*)Hp, ldp);
  else
    hipLaunchKernelGGL(permute_h_kernel<float>, grid, dim3(256), 0, st, (const float*)H, d, ldh, perm, (float*)Hp,
                       ldp);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
