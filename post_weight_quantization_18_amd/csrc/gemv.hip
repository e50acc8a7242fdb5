// Generation with the packed weights: y = W_hat x for one token, the weights
// dequantized on the fly from the row bitstreams that the quantizer writes.
// FDE Interviews breakdown of GPTQ, section 01: the 3/4-bit weights are read
// by an inference kernel that dequantizes them on the fly; nubint review, "Key
// findings": 3-bit OPT-175B generation kernels run about 3.25x (A100) and 4.5x
// (A6000) faster than fp16. At batch 1 the product reads every weight once
// and does two flops with it: it is bound by HBM bandwidth.
#include "common.h"

namespace gptq {
namespace {

constexpr int GV_ROWS = 4;  // rows per wave, sharing each chunk of x

// Code j (0..31) of a 32-code chunk held in BITS words (bit j*BITS onward,
// low bits first, split across two words when it straddles them).
template <int BITS>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t (&w)[BITS], int j) {
  const int p = j * BITS, wd = p >> 5, off = p & 31;
  uint32_t v = w[wd] >> off;
  if (off + BITS > 32) v |= w[wd + 1] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

// One wave per GV_ROWS rows; lane l takes the 32-code chunks l, l + 64, ... of
// each row (chunk k = words [k BITS, (k + 1) BITS) of the row, which lie in one
// group because groups are multiples of 32 columns). Per chunk the lane forms
// cx = sum c_j x_j and sx = sum x_j in fp32 and adds s (cx - z sx); the lanes'
// sums are added across the wave. The codes, scales, zero points and x of the
// lane's next chunk are loaded before the current one is used, so that two
// chunks per row are in flight. The look-ahead load is unconditional (the last
// chunk loads itself again), so that the wait before each chunk's use counts
// only the older loads.
template <int BITS>
__global__ __launch_bounds__(256) void dq_gemv_kernel(const uint32_t* q, const float* scales, const uint8_t* zeros,
                                                      int64_t m, int64_t d, int group, int ngroups, const half_t* x,
                                                      float* y) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * GV_ROWS;
  if (r0 >= m) return;  // uniform per wave
  const int64_t nch = d / 32, wpr = d * BITS / 32;
  float acc[GV_ROWS];
#pragma unroll
  for (int rr = 0; rr < GV_ROWS; ++rr) acc[rr] = 0.0f;
  uint32_t wc[GV_ROWS][BITS];
  float sc[GV_ROWS];
  uint32_t zc[GV_ROWS];
  half8 xc[4];
  auto load = [&](int64_t k, uint32_t (&w)[GV_ROWS][BITS], float (&sv)[GV_ROWS], uint32_t (&zv)[GV_ROWS],
                  half8 (&xv)[4]) {
    const int64_t g = group ? (32 * k) / group : 0;
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
      const int64_t r = r0 + rr < m ? r0 + rr : m - 1;  // rows past m repeat the last row, unused
#pragma unroll
      for (int b = 0; b < BITS; ++b) w[rr][b] = q[r * wpr + k * BITS + b];
      sv[rr] = scales[r * ngroups + g];
      zv[rr] = zeros[r * ngroups + g];
    }
    const half8* xp = (const half8*)(x + 32 * k);
#pragma unroll
    for (int v = 0; v < 4; ++v) xv[v] = xp[v];
  };
  if (lane < nch) load(lane, wc, sc, zc, xc);
  for (int64_t k = lane; k < nch; k += 64) {
    uint32_t wn[GV_ROWS][BITS];
    float sn[GV_ROWS];
    uint32_t zn[GV_ROWS];
    half8 xn[4];
    load(k + 64 < nch ? k + 64 : k, wn, sn, zn, xn);
    asm volatile("" ::: "memory");  // the look-ahead loads stay ahead of this chunk's arithmetic
    float xf[32];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[8 * v + e] = (float)xc[v][e];
    float sx = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) sx += xf[j];
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
      float cx = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) cx = fmaf((float)chunk_code<BITS>(wc[rr], j), xf[j], cx);
      acc[rr] = fmaf(sc[rr], fmaf(-(float)zc[rr], sx, cx), acc[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
#pragma unroll
      for (int b = 0; b < BITS; ++b) wc[rr][b] = wn[rr][b];
      sc[rr] = sn[rr];
      zc[rr] = zn[rr];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) xc[v] = xn[v];
  }
#pragma unroll
  for (int rr = 0; rr < GV_ROWS; ++rr) {
    float v = acc[rr];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && r0 + rr < m) y[r0 + rr] = v;
  }
}

template <int BITS>
gptq_status_t launch_dq_gemv(const uint32_t* q, const float* scales, const uint8_t* zeros, int64_t m, int64_t d,
                             int group, const half_t* x, float* y, hipStream_t st) {
  const int ngroups = group ? (int)(d / group) : 1;
  const dim3 grid((unsigned)ceil_div(m, 4 * GV_ROWS));
  TraceScope tr(st, GPTQ_TRACE_GEMV);
  hipLaunchKernelGGL(dq_gemv_kernel<BITS>, grid, dim3(256), 0, st, q, scales, zeros, m, d, group, ngroups, x, y);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace

gptq_status_t dq_gemv_enqueue(const uint32_t* q, const float* scales, const uint8_t* zeros, int64_t m, int64_t d,
                              int bits, int group, const half_t* x, float* y, hipStream_t st) {
  switch (bits) {
    case 2: return launch_dq_gemv<2>(q, scales, zeros, m, d, group, x, y, st);
    case 3: return launch_dq_gemv<3>(q, scales, zeros, m, d, group, x, y, st);
    case 4: return launch_dq_gemv<4>(q, scales, zeros, m, d, group, x, y, st);
    case 8: return launch_dq_gemv<8>(q, scales, zeros, m, d, group, x, y, st);
    default: return GPTQ_ERR_UNSUPPORTED;
  }
}

}  // namespace gptq
