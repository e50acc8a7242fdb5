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

// Rows per wave, sharing each chunk of x: 8 for tall layers (more code bytes
// per x chunk and per look-ahead), 4 otherwise (a 12288-row layer would fill
// only 384 workgroups with 8). Measured on the OPT-175B block (HIP events per
// call): fc1 (49152 rows) 58.4 us with 8 rows per wave, 58.5 / 59.3 / 61.1 /
// 63.3 us with 7 / 6 / 5 / 4; the 12288-row layers within 3 % of each other
// for 4 to 6 rows, slower with 2 or 3.
constexpr int kTallRows = 32768;

typedef half_t half2v __attribute__((ext_vector_type(2)));

// The 32 codes of a chunk are consumed in pairs (a, b) whose fields lie 16 bits
// apart in one 32-bit word, at the same bit p of the two halves. For p + BITS
// <= 10 the field sits inside an fp16 mantissa: masking the word to the two
// fields and OR-ing in the fp16 exponent of 2^(10 - p) in both halves makes
// each half the number 2^(10 - p) + code exactly (mantissa bit p weighs
// 2^(10 - p - 10 + p) = 1), and subtracting 2^(10 - p) in both halves leaves
// the two codes. Fields at p > 10 - BITS or p >= 8 are first brought down by
// 8 bits (one shift per word serves all of them). One dot2 instruction then adds
// a x_a + b x_b to an fp32 sum (the products are exact in fp32). Per pair that
// is an and-or, a packed subtract and the dot product.
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
//          26 straddle those halves and are paired as (5, 21) and (10, 26) in
//          words of their own.
template <int BITS>
struct ChunkPairs {
  static constexpr int NP = 16;  // pairs
  static constexpr int A(int p) { return (p / (16 / BITS)) * (32 / BITS) + p % (16 / BITS); }
  static constexpr int B(int p) { return A(p) + 16 / BITS; }
};
template <>
struct ChunkPairs<3> {
  static constexpr int NP = 16;  // 14 from X, Y, Z, then (5, 21) and (10, 26)
  static constexpr int A(int p) { return p < 5 ? p : p < 9 ? 6 + (p - 5) : p < 14 ? 11 + (p - 9) : p == 14 ? 5 : 10; }
  static constexpr int B(int p) { return A(p) + 16; }
};

// The OR constants (fp16 2^(10 - p) in both halves, p = 0 .. 7), held in
// registers: with the mask in a scalar register the and-or is one
// v_and_or_b32 (a gfx9 vector instruction reads at most one scalar operand,
// and neither constant is an inline one).
struct Magics {
  uint32_t m[8];
  __device__ __forceinline__ Magics() {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      uint32_t v = (uint32_t)(25 - p) << 10;
      v |= v << 16;
      asm volatile("" : "+v"(v));  // keep it in a vector register
      m[p] = v;
    }
  }
};

// The pair of fields at bit P of the halves of t (P + BITS <= 10), as fp16 codes.
template <int BITS, int P>
__device__ __forceinline__ half2v code_pair(uint32_t t, const Magics& mg) {
  static_assert(P + BITS <= 10 && P < 8, "field inside the fp16 mantissa, one of the eight OR constants");
  constexpr uint32_t mask = (((1u << BITS) - 1u) << P) * 0x00010001u;
  const uint32_t v = (t & mask) | mg.m[P];
  constexpr float off = (float)(1 << (10 - P));
  return __builtin_bit_cast(half2v, v) - (half2v){(half_t)off, (half_t)off};
}

// Pair at bit P of word t (any P <= 16 - BITS), t8 = t >> 8: in place for
// P < 8 and P + BITS <= 10, else from t8 (at P - 8 < 8, P - 8 + BITS <= 8).
template <int BITS, int P>
__device__ __forceinline__ half2v pair_at(uint32_t t, uint32_t t8, const Magics& mg) {
  if constexpr (P + BITS <= 10 && P < 8)
    return code_pair<BITS, P>(t, mg);
  else
    return code_pair<BITS, P - 8>(t8, mg);
}

template <int BITS, int K, int I>
__device__ __forceinline__ void word_pairs(uint32_t t, uint32_t t8, half2v* cp, const Magics& mg) {
  if constexpr (I < 16 / BITS) {
    cp[K * (16 / BITS) + I] = pair_at<BITS, BITS * I>(t, t8, mg);
    word_pairs<BITS, K, I + 1>(t, t8, cp, mg);
  }
}

template <int BITS, int K>
__device__ __forceinline__ void words(const uint32_t (&w)[BITS], half2v* cp, const Magics& mg) {
  if constexpr (K < BITS) {
    word_pairs<BITS, K, 0>(w[K], w[K] >> 8, cp, mg);
    words<BITS, K + 1>(w, cp, mg);
  }
}

// 3-bit: the pairs of word t whose fields start at bit P0 + 3 i, i < N, into
// cp[X0 + i].
template <int P0, int N, int X0, int I = 0>
__device__ __forceinline__ void word3(uint32_t t, uint32_t t8, half2v* cp, const Magics& mg) {
  if constexpr (I < N) {
    cp[X0 + I] = pair_at<3, P0 + 3 * I>(t, t8, mg);
    word3<P0, N, X0, I + 1>(t, t8, cp, mg);
  }
}

// sum_j c_j x_j over one chunk: xp[p] = (x_A(p), x_B(p)). All 16 code pairs are
// formed before the dot products, so that no dot waits on the subtract just
// before it.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint32_t (&w)[BITS], const half2v (&xp)[16], const Magics& mg) {
  half2v cp[16];
  if constexpr (BITS == 3) {
    const uint32_t X = __builtin_amdgcn_perm(w[1], w[0], 0x07060100u);  // w0 low half, w1 high half
    const uint32_t Y = __builtin_amdgcn_alignbit(w[2], w[0], 16);
    const uint32_t Z = __builtin_amdgcn_perm(w[2], w[1], 0x07060100u);  // w1 low half, w2 high half
    word3<0, 5, 0>(X, X >> 8, cp, mg);
    word3<2, 4, 5>(Y, Y >> 8, cp, mg);
    word3<1, 5, 9>(Z, Z >> 8, cp, mg);
    // code 5 = S[15,18) = w0 >> 15, code 21 = S[63,66) = (w2:w1) >> 31,
    // code 10 = S[30,33) = (w1:w0) >> 30, code 26 = S[78,81) = w2 >> 14:
    // each pair's low half-words joined into one word, fields at bit 0
    const uint32_t P = __builtin_amdgcn_perm(__builtin_amdgcn_alignbit(w[2], w[1], 31), w[0] >> 15, 0x05040100u);
    const uint32_t Q = __builtin_amdgcn_perm(w[2] >> 14, __builtin_amdgcn_alignbit(w[1], w[0], 30), 0x05040100u);
    cp[14] = code_pair<3, 0>(P, mg);
    cp[15] = code_pair<3, 0>(Q, mg);
  } else {
    words<BITS, 0>(w, cp, mg);
  }
  float acc = 0.0f;
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2(cp[p], xp[p], acc, false);
  return acc;
}

// One wave per GV_ROWS rows; lane l takes the 32-code chunks l, l + 64, ... of
// each row (chunk k = words [k BITS, (k + 1) BITS) of the row, which lie in one
// group because groups are multiples of 32 columns). Per chunk the lane forms
// cx = sum c_j x_j (code pairs and dot2, above) and sx = sum x_j in fp32 and
// adds s (cx - z sx); the lanes' sums are added across the wave. The codes,
// scales, zero points and x of the lane's next chunk are loaded before the
// current one is used, into the other of two register sets (two chunks per
// row in flight, and no copies between the sets). The look-ahead load is
// unconditional (the last chunk loads itself again), so that the wait before
// each chunk's use counts only the older loads. Row addresses are wave-uniform
// (rows past m repeat the last row, unused), lane offsets 32-bit.
template <int BITS, int GV_ROWS>
struct ChunkRegs {
  uint32_t w[GV_ROWS][BITS];
  float s[GV_ROWS];
  uint32_t z[GV_ROWS];
  half8 x[4];
};

template <int BITS, int GV_ROWS>
__global__ __launch_bounds__(256) void dq_gemv_kernel(const uint32_t* q, const float* scales, const uint8_t* zeros,
                                                      int64_t m, int64_t d, int group, int ngroups, const half_t* x,
                                                      float* y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform: row pointers in SGPRs
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * GV_ROWS;
  if (r0 >= m) return;  // uniform per wave
  const int nch = (int)(d / 32);
  const int64_t wpr = d * BITS / 32;
  const uint32_t* qrow[GV_ROWS];
  const float* srow[GV_ROWS];
  const uint8_t* zrow[GV_ROWS];
#pragma unroll
  for (int rr = 0; rr < GV_ROWS; ++rr) {
    const int64_t r = r0 + rr < m ? r0 + rr : m - 1;
    qrow[rr] = q + r * wpr;
    srow[rr] = scales + r * ngroups;
    zrow[rr] = zeros + r * ngroups;
  }
  float acc[GV_ROWS];
#pragma unroll
  for (int rr = 0; rr < GV_ROWS; ++rr) acc[rr] = 0.0f;
  const Magics mg;
  using Regs = ChunkRegs<BITS, GV_ROWS>;
  auto load = [&](int k, Regs& c) __attribute__((always_inline)) {
    // 32-bit byte offsets from wave-uniform bases (scalar-base addressing)
    const uint32_t g = group ? (uint32_t)(32 * k) / (uint32_t)group : 0u, kb = (uint32_t)k * (4 * BITS);
    GPTQ_DASSERT(k >= 0 && k < nch && (int)g < ngroups);
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
#pragma unroll
      for (int b = 0; b < BITS; ++b) c.w[rr][b] = ((const uint32_t*)((const char*)qrow[rr] + kb))[b];
      c.s[rr] = *(const float*)((const char*)srow[rr] + 4 * g);
      c.z[rr] = zrow[rr][g];
    }
    const half8* xp = (const half8*)((const char*)x + 64 * (uint32_t)k);
#pragma unroll
    for (int v = 0; v < 4; ++v) c.x[v] = xp[v];
  };
  auto compute = [&](const Regs& c) __attribute__((always_inline)) {
    using CP = ChunkPairs<BITS>;
    half_t xh[32];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) xh[8 * v + e] = c.x[v][e];
    half2v xp[16];
    float sx = 0.0f;
#pragma unroll
    for (int p = 0; p < CP::NP; ++p) {
      xp[p] = (half2v){xh[CP::A(p)], xh[CP::B(p)]};
      sx = __builtin_amdgcn_fdot2(xp[p], (half2v){(half_t)1.0f, (half_t)1.0f}, sx, false);
    }
#pragma unroll
    for (int rr = 0; rr < GV_ROWS; ++rr) {
      const float cx = chunk_dot<BITS>(c.w[rr], xp, mg);
      acc[rr] = fmaf(c.s[rr], fmaf(-(float)c.z[rr], sx, cx), acc[rr]);
    }
  };
  Regs ca, cb;
  if (lane < nch) load(lane, ca);
  for (int k = lane; k < nch; k += 128) {
    load(k + 64 < nch ? k + 64 : k, cb);
    asm volatile("" ::: "memory");  // the look-ahead loads stay ahead of this chunk's arithmetic
    compute(ca);
    if (k + 64 >= nch) break;
    load(k + 128 < nch ? k + 128 : k + 64, ca);
    asm volatile("" ::: "memory");
    compute(cb);
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
