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
//  * The block's errors E [m, 128] go to the workspace; the far columns are
//    then updated by one GEMM W[:, end:] -= E U[blk, end:] on the matrix cores
//    (v_mfma_f32_32x32x2f32: fp32 operands, because single-pass fp16 operands
//    move the pre-round values by more than the 1e-3 grid-unit band).
//  * Codes are kept one byte per weight in the workspace and packed (with the
//    dequantized W_hat) by a final kernel.
#include <utility>

#include "common.h"

namespace gptq {

namespace {

constexpr int BLK = 128;
constexpr int CL_THREADS = 64;

struct QuantWs {
  float* Wk;       // m x d working weights
  float* E;        // m x BLK block errors
  uint8_t* codes;  // m x d
  float* U32;      // d x d (only when U is fp64)
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

QuantWs quant_ws(void* ws, int64_t m, int64_t d, int u_f64) {
  QuantWs w;
  char* p = (char*)ws;
  w.Wk = (float*)p;
  p += align256((size_t)m * d * sizeof(float));
  w.E = (float*)p;
  p += align256((size_t)m * BLK * sizeof(float));
  w.codes = (uint8_t*)p;
  p += align256((size_t)m * d);
  w.U32 = u_f64 ? (float*)p : nullptr;
  return w;
}

struct GridFit {
  float s, z;
};

// Asymmetric min-max: lo = min(v, 0), hi = max(v, 0) (both 0 -> -1, 1),
// s = (hi - lo) / maxq, z = rint(-lo / s). Ternary: s = max|v| (0 -> 1), z = 1.
__device__ inline GridFit fit_grid(float vmin, float vmax, int ternary, float maxq) {
  float lo = fminf(vmin, 0.0f), hi = fmaxf(vmax, 0.0f);
  GridFit g;
  if (ternary) {
    float amax = fmaxf(-lo, hi);
    g.s = amax == 0.0f ? 1.0f : amax;
    g.z = 1.0f;
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
__global__ __launch_bounds__(256) void prep_kernel(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw,
                                                   float* Wk, int per_row, int ternary, float maxq, float* scales,
                                                   uint8_t* zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  float vmin = INFINITY, vmax = -INFINITY;
  for (int64_t j = lane; j < d; j += 64) {
    float v = w_f32 ? ((const float*)W)[r * ldw + j] : (float)((const half_t*)W)[r * ldw + j];
    Wk[r * d + j] = v;
    vmin = fminf(vmin, v);
    vmax = fmaxf(vmax, v);
  }
  if (!per_row) return;
  for (int off = 32; off > 0; off >>= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  if (lane == 0) {
    GridFit g = fit_grid(vmin, vmax, ternary, maxq);
    scales[r] = g.s;
    zeros[r] = (uint8_t)g.z;
  }
}

__global__ void f64_to_f32_kernel(const double* U, int64_t d, int64_t ldu, float* U32) {
  const int64_t i = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256)
    U32[i * d + j] = (float)U[i * ldu + j];
}

struct ColArgs {
  float* Wk;
  const float* U;
  int64_t ldu, m, d, j0;
  int bw;          // block width (multiple of 32, <= 128)
  int ternary;
  float maxq;
  int group;       // runtime group size (used when G < 0)
  int ngroups;
  float* E;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* err_sq;
  int first;
};

// Per-lane state of the column loop: the row's 128-column tile, its grid and
// the packed codes. Every index below is a compile-time constant, so the
// arrays stay in registers.
struct RowState {
  float w[BLK];
  uint32_t cw[BLK / 4];
  float s, rs, zf, esum;
};

template <int I, int K>
struct Fma {  // w[k] -= e * U[I][k] for k = K .. BLK-1
  __device__ __forceinline__ static void run(RowState& st, float e, const float* urow) {
    st.w[K] = fmaf(-e, urow[K], st.w[K]);
    Fma<I, K + 1>::run(st, e, urow);
  }
};
template <int I>
struct Fma<I, BLK> {
  __device__ __forceinline__ static void run(RowState&, float, const float*) {}
};

template <int I, int K, int END>
struct MinMax {  // running min/max over w[K .. END-1]
  __device__ __forceinline__ static void run(const RowState& st, float& lo, float& hi) {
    lo = fminf(lo, st.w[K]);
    hi = fmaxf(hi, st.w[K]);
    MinMax<I, K + 1, END>::run(st, lo, hi);
  }
};
template <int I, int END>
struct MinMax<I, END, END> {
  __device__ __forceinline__ static void run(const RowState&, float&, float&) {}
};

template <int G, int I>
struct Step {
  __device__ __forceinline__ static void run(RowState& st, const ColArgs& a, int64_t r, const float (*Us)[BLK],
                                             const float* rdiag) {
    if (I < a.bw) {
      if constexpr (G > 0 && I % (G > 0 ? G : 1) == 0) {
        float lo = st.w[I], hi = st.w[I];
        MinMax<I, I + 1, I + (G > 0 ? G : 1)>::run(st, lo, hi);
        GridFit g = fit_grid(lo, hi, a.ternary, a.maxq);
        const int64_t gi = (a.j0 + I) / (G > 0 ? G : 1);
        a.scales[r * a.ngroups + gi] = g.s;
        a.zeros[r * a.ngroups + gi] = (uint8_t)g.z;
        st.s = g.s;
        st.zf = g.z;
        st.rs = 1.0f / g.s;
      }
      const float p = st.w[I] * st.rs + st.zf;
      const float c = fminf(fmaxf(rintf(p), 0.0f), a.maxq);
      const float qv = st.s * (c - st.zf);
      const float e = (st.w[I] - qv) * rdiag[I];
      st.esum += e * e;
      st.cw[I >> 2] |= ((uint32_t)c) << (8 * (I & 3));
      st.w[I] = e;  // the register now carries the error of column I
      Fma<I, I + 1>::run(st, e, Us[I]);
    }
  }
};

template <int G, int... Is>
__device__ __forceinline__ void run_steps(std::integer_sequence<int, Is...>, RowState& st, const ColArgs& a,
                                          int64_t r, const float (*Us)[BLK], const float* rdiag) {
  (Step<G, Is>::run(st, a, r, Us, rdiag), ...);
}

// G = 0: one grid per row (already fitted); G = 32, 64, 128: refit at every
// group start inside the block; G = -1: groups span whole blocks, refit at the
// group's first block from the current working weights.
template <int G>
__global__ __launch_bounds__(CL_THREADS) void colloop_kernel(ColArgs a) {
  __shared__ float Us[BLK][BLK];
  __shared__ float rdiag[BLK];
  const int tid = threadIdx.x;
  const int bw = a.bw;
  for (int idx = tid; idx < BLK * BLK / 4; idx += CL_THREADS) {
    const int i = idx / (BLK / 4), k4 = (idx % (BLK / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < bw && k4 < bw) v = *(const float4*)(a.U + (a.j0 + i) * a.ldu + a.j0 + k4);
    *(float4*)&Us[i][k4] = v;
  }
  __syncthreads();
  for (int i = tid; i < BLK; i += CL_THREADS) rdiag[i] = i < bw ? 1.0f / Us[i][i] : 0.0f;
  __syncthreads();

  const int64_t r = (int64_t)blockIdx.x * CL_THREADS + tid;
  if (r >= a.m) return;  // no barrier follows

  RowState st;
  const float* wrow = a.Wk + r * a.d + a.j0;
#pragma unroll
  for (int k = 0; k < BLK; k += 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < bw) v = *(const float4*)(wrow + k);
    st.w[k] = v.x;
    st.w[k + 1] = v.y;
    st.w[k + 2] = v.z;
    st.w[k + 3] = v.w;
  }
#pragma unroll
  for (int k = 0; k < BLK / 4; ++k) st.cw[k] = 0;
  st.esum = 0.0f;
  st.s = 1.0f;
  st.rs = 1.0f;
  st.zf = 0.0f;
  if (G == 0) {
    st.s = a.scales[r];
    st.zf = (float)a.zeros[r];
    st.rs = 1.0f / st.s;
  } else if (G < 0) {
    const int gi = (int)(a.j0 / a.group);
    if (a.j0 % a.group == 0) {
      float vmin = INFINITY, vmax = -INFINITY;
      const float* grow = a.Wk + r * a.d + a.j0;
      for (int k = 0; k < a.group; k += 4) {
        float4 v = *(const float4*)(grow + k);
        vmin = fminf(fminf(fminf(vmin, v.x), fminf(v.y, v.z)), v.w);
        vmax = fmaxf(fmaxf(fmaxf(vmax, v.x), fmaxf(v.y, v.z)), v.w);
      }
      GridFit g = fit_grid(vmin, vmax, a.ternary, a.maxq);
      a.scales[r * a.ngroups + gi] = g.s;
      a.zeros[r * a.ngroups + gi] = (uint8_t)g.z;
      st.s = g.s;
      st.zf = g.z;
    } else {
      st.s = a.scales[r * a.ngroups + gi];
      st.zf = (float)a.zeros[r * a.ngroups + gi];
    }
    st.rs = 1.0f / st.s;
  }

  run_steps<G>(std::make_integer_sequence<int, BLK>{}, st, a, r, Us, rdiag);

  float* erow = a.E + r * BLK;
#pragma unroll
  for (int k = 0; k < BLK; k += 4)
    if (k < bw) *(float4*)(erow + k) = make_float4(st.w[k], st.w[k + 1], st.w[k + 2], st.w[k + 3]);
  uint8_t* crow = a.codes + r * a.d + a.j0;
#pragma unroll
  for (int k = 0; k < BLK / 4; k += 4)
    if (4 * k < bw) *(uint4*)(crow + 4 * k) = make_uint4(st.cw[k], st.cw[k + 1], st.cw[k + 2], st.cw[k + 3]);
  if (a.err_sq) a.err_sq[r] = (a.first ? 0.0f : a.err_sq[r]) + 0.5f * st.esum;
}

// W[r][c] -= sum_{k < bw} E[r][k] U[j0 + k][c] for c >= j1.
// 128 x 128 output tile per workgroup, 4 waves of 64 x 64, fp32 MFMA 32x32x2.
__global__ __launch_bounds__(256) void trail_kernel(float* Wk, int64_t m, int64_t d, const float* E,
                                                    const float* U, int64_t ldu, int64_t j0, int bw, int64_t j1) {
  __shared__ float As[128][33];
  __shared__ float Bs[32][132];
  const int64_t row0 = (int64_t)blockIdx.y * 128, col0 = j1 + (int64_t)blockIdx.x * 128;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
  float16v acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;
  const int li = lane & 31, lk = lane >> 5;
  for (int kc = 0; kc < bw; kc += 32) {
    for (int idx = tid; idx < 128 * 8; idx += 256) {
      const int r = idx >> 3, c4 = (idx & 7) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + r < m) v = *(const float4*)(E + (row0 + r) * BLK + kc + c4);
      As[r][c4] = v.x;
      As[r][c4 + 1] = v.y;
      As[r][c4 + 2] = v.z;
      As[r][c4 + 3] = v.w;
    }
    for (int idx = tid; idx < 32 * 32; idx += 256) {
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (col0 + c4 < d) v = *(const float4*)(U + (j0 + kc + r) * ldu + col0 + c4);
      *(float4*)&Bs[r][c4] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      float av[2], bv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) av[x] = As[wr + x * 32 + li][k + lk];
#pragma unroll
      for (int y = 0; y < 2; ++y) bv[y] = Bs[k + lk][wc + y * 32 + li];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }
  const int hl = lane >> 5;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = row0 + wr + x * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int64_t j = col0 + wc + y * 32 + li;
        if (i < m && j < d) Wk[i * d + j] -= acc[x][y][r];
      }
}

// Packs one row per workgroup into the LSB-first bitstream and, when W_hat is
// given, writes W_hat = s * (code - z).
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* codes, int64_t ldc, int64_t m, int64_t d,
                                                   int bits, uint32_t* out, float* W_hat, const float* scales,
                                                   const uint8_t* zeros, int group, int ngroups) {
  const int64_t r = blockIdx.x;
  if (r >= m) return;
  const uint8_t* crow = codes + r * ldc;
  const int64_t nwords = d * bits / 32;
  for (int64_t wd = threadIdx.x; wd < nwords; wd += 256) {
    const int64_t b0 = wd * 32;
    int64_t j = b0 / bits;
    const int64_t jend = (b0 + 31) / bits;
    uint32_t word = 0;
    for (; j <= jend; ++j) {
      const int64_t shift = j * bits - b0;
      const uint32_t c = crow[j];
      word |= shift >= 0 ? (c << shift) : (c >> (-shift));
    }
    out[r * nwords + wd] = word;
  }
  if (W_hat) {
    for (int64_t j = threadIdx.x; j < d; j += 256) {
      const int64_t g = group ? j / group : 0;
      const float s = scales[r * ngroups + g], z = (float)zeros[r * ngroups + g];
      W_hat[r * d + j] = s * ((float)crow[j] - z);
    }
  }
}

template <int G>
gptq_status_t launch_colloop(const ColArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(colloop_kernel<G>, dim3((unsigned)ceil_div(a.m, CL_THREADS)), dim3(CL_THREADS), 0, st, a);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace

size_t quant_workspace_bytes(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  (void)cfg;
  size_t b = align256((size_t)m * d * sizeof(float)) + align256((size_t)m * BLK * sizeof(float)) +
             align256((size_t)m * d);
  return b;
}

static size_t quant_u32_bytes(int64_t d) { return align256((size_t)d * d * sizeof(float)); }

gptq_status_t quant_enqueue(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw, const void* U, int u_f64,
                            int64_t ldu, const gptq_qcfg_t& cfg, uint32_t* qcodes, float* scales, uint8_t* zeros,
                            float* W_hat, float* err_sq, void* ws, size_t ws_bytes, hipStream_t st) {
  const size_t need = quant_workspace_bytes(m, d, cfg) + (u_f64 ? quant_u32_bytes(d) : 0);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  QuantWs w = quant_ws(ws, m, d, u_f64);
  const int ternary = cfg.grid == GPTQ_GRID_TERNARY;
  const float maxq = ternary ? 2.0f : (float)((1 << cfg.bits) - 1);
  const int group = cfg.group_size;
  const int ngroups = group ? (int)(d / group) : 1;

  const float* U32 = (const float*)U;
  int64_t ldu32 = ldu;
  if (u_f64) {
    hipLaunchKernelGGL(f64_to_f32_kernel, dim3((unsigned)(ceil_div(d, 256) < 64 ? ceil_div(d, 256) : 64), (unsigned)d),
                       dim3(256), 0, st, (const double*)U, d, ldu, w.U32);
    GPTQ_CHECK_LAUNCH();
    U32 = w.U32;
    ldu32 = d;
  }
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)ceil_div(m, 4)), dim3(256), 0, st, W, w_f32, m, d, ldw, w.Wk,
                     group == 0 ? 1 : 0, ternary, maxq, scales, zeros);
  GPTQ_CHECK_LAUNCH();

  ColArgs a;
  a.Wk = w.Wk;
  a.U = U32;
  a.ldu = ldu32;
  a.m = m;
  a.d = d;
  a.ternary = ternary;
  a.maxq = maxq;
  a.group = group;
  a.ngroups = ngroups;
  a.E = w.E;
  a.codes = w.codes;
  a.scales = scales;
  a.zeros = zeros;
  a.err_sq = err_sq;
  const int64_t nblocks = ceil_div(d, BLK);
  for (int64_t b = 0; b < nblocks; ++b) {
    a.j0 = b * BLK;
    a.bw = (int)((d - a.j0) < BLK ? (d - a.j0) : BLK);
    a.first = b == 0;
    gptq_status_t s;
    switch (group) {
      case 0: s = launch_colloop<0>(a, st); break;
      case 32: s = launch_colloop<32>(a, st); break;
      case 64: s = launch_colloop<64>(a, st); break;
      case 128: s = launch_colloop<128>(a, st); break;
      default: s = launch_colloop<-1>(a, st); break;
    }
    if (s != GPTQ_OK) return s;
    const int64_t j1 = a.j0 + a.bw;
    if (j1 < d) {
      dim3 grid((unsigned)ceil_div(d - j1, 128), (unsigned)ceil_div(m, 128));
      hipLaunchKernelGGL(trail_kernel, grid, dim3(256), 0, st, w.Wk, m, d, (const float*)w.E, U32, ldu32, a.j0,
                         a.bw, j1);
      GPTQ_CHECK_LAUNCH();
    }
  }
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)m), dim3(256), 0, st, (const uint8_t*)w.codes, d, m, d, cfg.bits,
                     qcodes, W_hat, (const float*)scales, (const uint8_t*)zeros, group, ngroups);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status_t pack_enqueue(const uint8_t* codes, int64_t ldc, int64_t m, int64_t d, int bits, uint32_t* out,
                           hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)m), dim3(256), 0, st, codes, ldc, m, d, bits, out, (float*)nullptr,
                     (const float*)nullptr, (const uint8_t*)nullptr, 0, 1);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

size_t quant_workspace_bytes_u64(int64_t m, int64_t d, const gptq_qcfg_t& cfg) {
  return quant_workspace_bytes(m, d, cfg) + quant_u32_bytes(d);
}

}  // namespace gptq
