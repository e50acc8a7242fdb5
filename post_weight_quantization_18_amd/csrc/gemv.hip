// Generation with the packed weights: y = W_hat x for one token, the weights
// dequantized on the fly from the row bitstreams that the quantizer writes.
// FDE Interviews breakdown of GPTQ, section 01: the 3/4-bit weights are read
// by an inference kernel that dequantizes them on the fly; nubint review, "Key
// findings": 3-bit OPT-175B generation kernels run about 3.25x (A100) and 4.5x
// (A6000) faster than fp16. At batch 1 the product reads every weight once
// and does two flops with it: it is bound by HBM bandwidth.
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

// Rows per wave, sharing each chunk of x: 8 for tall layers (more code bytes
// per x chunk and per look-ahead), 4 otherwise (a 12288-row layer would fill
// only 384 workgroups with 8). Measured on the OPT-175B block: fc1 (49152 rows)
// 70.8 us with 8 against 74.9 us with 4; fc2 (12288 rows) 88.5 against 79.8 us.
constexpr int kTallRows = 32768;

typedef half_t half2v __attribute__((ext_vector_type(2)));

// The 32 codes of a chunk are consumed in pairs (a, b) whose fields lie 16 bits
// apart in one 32-bit word: masking such a word keeps both codes, OR-ing in
// 0x6400 per half makes each the fp16 number 1024 + code (the code sits in the
// low mantissa bits under the exponent of 2^10), and subtracting 1024 in both
// halves leaves the two codes exactly. One dot2 instruction then adds a x_a +
// b x_b to an fp32 sum (the fp16 x fp16 products are exact in fp32). Per pair
// that is a shift, an and-or, a packed subtract and the dot product: two
// vector instructions per code.
//
// Pairs of a chunk, by bit width (code index a, b):
//  2 bits: word k holds codes 16k .. 16k+15; pairs (16k + i, 16k + 8 + i), i < 8
//  4 bits: word k holds codes 8k .. 8k+7;    pairs (8k + i, 8k + 4 + i),   i < 4
//  8 bits: word k holds codes 4k .. 4k+3;    pairs (4k + i, 4k + 2 + i),   i < 2
//  3 bits: the chunk is 96 bits S with code j at bit 3j; codes 16 apart are 48
//          bits apart, so the words X = S[0,16) | S[48,64) << 16,
//          Y = S[16,32) | S[64,80) << 16 and Z = S[32,48) | S[80,96) << 16 hold
//          pairs (i, 16 + i) at bit 3i (i < 5), (6 + i, 22 + i) at 2 + 3i
//          (i < 4) and (11 + i, 27 + i) at 1 + 3i (i < 5); codes 5, 10, 21 and
//          26 straddle those halves and are taken one by one.
template <int BITS>
struct ChunkPairs {
  static constexpr int NP = 16;  // pairs
  static constexpr int NS = 0;   // single codes
  static constexpr int A(int p) { return (p / (16 / BITS)) * (32 / BITS) + p % (16 / BITS); }
  static constexpr int B(int p) { return A(p) + 16 / BITS; }
  static constexpr int S(int) { return 0; }
};
template <>
struct ChunkPairs<3> {
  static constexpr int NP = 14;
  static constexpr int NS = 4;
  static constexpr int A(int p) { return p < 5 ? p : p < 9 ? 6 + (p - 5) : 11 + (p - 9); }
  static constexpr int B(int p) { return A(p) + 16; }
  static constexpr int S(int q) { return q == 0 ? 5 : q == 1 ? 10 : q == 2 ? 21 : 26; }
};

// magic = 0x64006400 held in a register: with the mask in a scalar register
// the and-or is one v_and_or_b32 (a gfx9 vector instruction reads at most one
// scalar operand, and neither constant is an inline one).
template <int BITS>
__device__ __forceinline__ half2v code_pair(uint32_t t, int shift, uint32_t magic) {
  constexpr uint32_t mask = ((1u << BITS) - 1u) * 0x00010001u;
  const uint32_t v = ((t >> shift) & mask) | magic;
  return __builtin_bit_cast(half2v, v) - (half2v){(half_t)1024.0f, (half_t)1024.0f};
}

// sum_j c_j x_j over one chunk: xp[p] = (x_A(p), x_B(p)), xs[q] = x_S(q).
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint32_t (&w)[BITS], const half2v (&xp)[ChunkPairs<BITS>::NP],
                                           const float (&xs)[ChunkPairs<BITS>::NS > 0 ? ChunkPairs<BITS>::NS : 1],
                                           uint32_t magic) {
  float acc = 0.0f;
  if constexpr (BITS == 3) {
    const uint32_t X = (w[0] & 0xFFFFu) | (w[1] & 0xFFFF0000u);
    const uint32_t Y = __builtin_amdgcn_alignbit(w[2], w[0], 16);
    const uint32_t Z = (w[1] & 0xFFFFu) | (w[2] & 0xFFFF0000u);
#pragma unroll
    for (int i = 0; i < 5; ++i) acc = __builtin_amdgcn_fdot2(code_pair<3>(X, 3 * i, magic), xp[i], acc, false);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(code_pair<3>(Y, 2 + 3 * i, magic), xp[5 + i], acc, false);
#pragma unroll
    for (int i = 0; i < 5; ++i) acc = __builtin_amdgcn_fdot2(code_pair<3>(Z, 1 + 3 * i, magic), xp[9 + i], acc, false);
    const uint32_t c5 = (w[0] >> 15) & 7u;
    const uint32_t c10 = __builtin_amdgcn_alignbit(w[1], w[0], 30) & 7u;
    const uint32_t c21 = __builtin_amdgcn_alignbit(w[2], w[1], 31) & 7u;
    const uint32_t c26 = (w[2] >> 14) & 7u;
    acc = fmaf((float)c5, xs[0], acc);
    acc = fmaf((float)c10, xs[1], acc);
    acc = fmaf((float)c21, xs[2], acc);
    acc = fmaf((float)c26, xs[3], acc);
  } else {
    constexpr int PW = 16 / BITS;  // pairs per word
#pragma unroll
    for (int k = 0; k < BITS; ++k)
#pragma unroll
      for (int i = 0; i < PW; ++i)
        acc = __builtin_amdgcn_fdot2(code_pair<BITS>(w[k], BITS * i, magic), xp[k * PW + i], acc, false);
  }
  return acc;
}

// One wave per GV_ROWS rows; lane l takes the 32-code chunks l, l + 64, ... of
// each row (chunk k = words [k BITS, (k + 1) BITS) of the row, which lie in one
// group because groups are multiples of 32 columns). Per chunk the lane forms
// cx = sum c_j x_j (code pairs and dot2, above) and sx = sum x_j in fp32 and
// adds s (cx - z sx); the lanes' sums are added across the wave. The codes, scales, zero points and x of the
// lane's next chunk are loaded before the current one is used, so that two
// chunks per row are in flight. The look-ahead load is unconditional (the last
// chunk loads itself again), so that the wait before each chunk's use counts
// only the older loads.
template <int BITS, int GV_ROWS>
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
  uint32_t magic;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  uint32_t wc[GV_ROWS][BITS];
  float sc[GV_ROWS];
  uint32_t zc[GV_ROWS];
  half8 xc[4];
  auto load = [&](int64_t k, uint32_t (&w)[GV_ROWS][BITS], float (&sv)[GV_ROWS], uint32_t (&zv)[GV_ROWS],
                  half8 (&xv)[4]) {
    const int64_t g = group ? (32 * k) / group : 0;
    GPTQ_DASSERT(k >= 0 && k < nch && g < ngroups);
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
    using CP = ChunkPairs<BITS>;
    half_t xh[32];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) xh[8 * v + e] = xc[v][e];
    half2v xp[CP::NP];
    float xs[CP::NS > 0 ? CP::NS : 1];
    float sx = 0.0f;
#pragma unroll
    for (int p = 0; p < CP::NP; ++p) {
      xp[p] = (half2v){xh[CP::A(p)], xh[CP::B(p)]};
      sx = __builtin_amdgcn_fdot2(xp[p], (half2v){(half_t)1.0f, (half_t)1.0f}, sx, false);
    }
#pragma unroll
    for (int q = 0; q < CP::NS; ++q) {
      xs[q] = (float)xh[CP::S(q)];
      sx += xs[q];
    }
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
      const float cx = chunk_dot<BITS>(wc[rr], xp, xs, magic);
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
  TraceScope tr(st, GPTQ_TRACE_GEMV);
  if (m >= kTallRows)
    hipLaunchKernelGGL((dq_gemv_kernel<BITS, 8>), dim3((unsigned)ceil_div(m, 4 * 8)), dim3(256), 0, st, q, scales,
                       zeros, m, d, group, ngroups, x, y);
  else
    hipLaunchKernelGGL((dq_gemv_kernel<BITS, 4>), dim3((unsigned)ceil_div(m, 4 * 4)), dim3(256), 0, st, q, scales,
                       zeros, m, d, group, ngroups, x, y);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

// Act-order codes for the generation product. Without static groups the
// ordered quantizer keeps the codes in natural column order and names every
// column's group in g_idx; group k is the k-th run of group_size columns in the
// quantization order, so each group still holds group_size columns. Sorting
// the columns by group (ties by column index) makes the groups contiguous
// runs again: col_perm[k g + i] is the i-th column of group k. The codes are
// rewritten in that order once, and each product reads x in that order too.

// One thread per group: the group's columns in index order. info counts
// columns whose group is out of range and groups without exactly `group`
// columns (0: col_perm is a permutation).
__global__ __launch_bounds__(256) void group_order_kernel(const int32_t* g_idx, int64_t d, int group, int ngroups,
                                                          int32_t* col_perm, int32_t* info) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g == 0) {
    int bad = 0;
    for (int64_t j = 0; j < d; ++j) bad += (g_idx[j] < 0 || g_idx[j] >= ngroups);
    if (bad) atomicAdd(info, bad);
  }
  if (g >= ngroups) return;
  int cnt = 0;
  for (int64_t j = 0; j < d; ++j) {
    if (g_idx[j] == g) {
      if (cnt < group) col_perm[(int64_t)g * group + cnt] = (int32_t)j;
      ++cnt;
    }
  }
  // a short group leaves its last slots unset: fill them with a valid column
  for (int c = cnt; c < group; ++c) col_perm[(int64_t)g * group + c] = 0;
  if (cnt != group) atomicAdd(info, 1);
}

__global__ void zero_info_kernel(int32_t* info) { *info = 0; }

// Row r, output chunk c: the codes at natural columns col_perm[32 c .. 32 c + 31]
// packed into BITS words (low bits first).
template <int BITS>
__global__ __launch_bounds__(256) void reorder_codes_kernel(const uint32_t* q, const int32_t* col_perm, int64_t m,
                                                            int64_t d, uint32_t* out) {
  const int64_t nch = d / 32, wpr = d * BITS / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= m * nch) return;
  const int64_t r = t / nch, c = t - r * nch;
  GPTQ_DASSERT(r < m && c < nch);
  const uint32_t* row = q + r * wpr;
  uint32_t w[BITS];
#pragma unroll
  for (int b = 0; b < BITS; ++b) w[b] = 0u;
#pragma unroll 4
  for (int e = 0; e < 32; ++e) {
    int64_t j = col_perm[32 * c + e];
    if (j < 0 || j >= d) j = 0;
    const int64_t p = j * BITS;
    const int wd = (int)(p >> 5), off = (int)(p & 31);
    uint32_t v = row[wd] >> off;
    if (off + BITS > 32) v |= row[wd + 1] << (32 - off);
    v &= (1u << BITS) - 1u;
    const int po = e * BITS, pw = po >> 5, pb = po & 31;
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
      if (b == pw) w[b] |= v << pb;
      if (b == pw + 1 && pb + BITS > 32) w[b] |= v >> (32 - pb);
    }
  }
#pragma unroll
  for (int b = 0; b < BITS; ++b) out[r * wpr + c * BITS + b] = w[b];
}

// xp[p] = x[col_perm[p]] (entries outside [0, d) read x[0]).
__global__ __launch_bounds__(256) void gather_x_kernel(const half_t* x, const int32_t* col_perm, int64_t d,
                                                       half_t* xp) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= d) return;
  int64_t j = col_perm[p];
  if (j < 0 || j >= d) j = 0;
  xp[p] = x[j];
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

namespace gptq {

gptq_status_t gemv_act_order_prepare(const uint32_t* q, const int32_t* g_idx, int64_t m, int64_t d, int bits,
                                     int group, uint32_t* out, int32_t* col_perm, int32_t* info, hipStream_t st) {
  const int ngroups = (int)(d / group);
  TraceScope tr(st, GPTQ_TRACE_GEMV);
  hipLaunchKernelGGL(zero_info_kernel, dim3(1), dim3(1), 0, st, info);
  hipLaunchKernelGGL(group_order_kernel, dim3((unsigned)ceil_div(ngroups, 256)), dim3(256), 0, st, g_idx, d, group,
                     ngroups, col_perm, info);
  const dim3 grid((unsigned)ceil_div(m * (d / 32), 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL(reorder_codes_kernel<2>, grid, dim3(256), 0, st, q, col_perm, m, d, out); break;
    case 3: hipLaunchKernelGGL(reorder_codes_kernel<3>, grid, dim3(256), 0, st, q, col_perm, m, d, out); break;
    case 4: hipLaunchKernelGGL(reorder_codes_kernel<4>, grid, dim3(256), 0, st, q, col_perm, m, d, out); break;
    case 8: hipLaunchKernelGGL(reorder_codes_kernel<8>, grid, dim3(256), 0, st, q, col_perm, m, d, out); break;
    default: return GPTQ_ERR_UNSUPPORTED;
  }
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status_t gather_x_enqueue(const half_t* x, const int32_t* col_perm, int64_t d, half_t* xp, hipStream_t st) {
  TraceScope tr(st, GPTQ_TRACE_GEMV);
  hipLaunchKernelGGL(gather_x_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st, x, col_perm, d, xp);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
