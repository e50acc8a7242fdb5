// Shared device/host helpers of the gfx950 GPTQ library (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gptq.h"

namespace gptq {

typedef _Float16 half_t;
typedef half_t half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef double double4v __attribute__((ext_vector_type(4)));

#define GPTQ_LDS __attribute__((address_space(3)))
#define GPTQ_GLB __attribute__((address_space(1)))

// Device-side checks of the debug build (-DGPTQ_DEBUG, built by
// `python -m post_weight_quantization_18_amd.build --debug`): a failed check
// prints the condition with its file and line and stops the kernel, so the
// launch reports an error. The release build compiles them away.
#ifdef GPTQ_DEBUG
#define GPTQ_DASSERT(cond)                                                              \
  do {                                                                                  \
    if (!(cond)) {                                                                      \
      printf("gptq debug check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__);       \
      __builtin_trap();                                                                 \
    }                                                                                   \
  } while (0)
#else
#define GPTQ_DASSERT(cond) ((void)0)
#endif

// Returns GPTQ_ERR_HIP from the enclosing function when a launch failed.
#define GPTQ_CHECK_LAUNCH()                         \
  do {                                              \
    if (hipGetLastError() != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Logical block index that gives each of the 8 XCDs a contiguous range of
// logical ids (the dispatcher hands consecutive workgroups to XCDs round-robin),
// so that neighbouring tiles share one L2. A bijection for any grid size.
__device__ inline int xcd_logical_block(int id, int nblocks) {
  const int nx = 8;
  int x = id % nx, local = id / nx;
  int base = nblocks / nx, rem = nblocks % nx;
  return x * base + (x < rem ? x : rem) + local;
}

// gfx950 direct global -> LDS DMA of 16 bytes per lane: lane l writes LDS bytes
// [lds_off + 16 l, lds_off + 16 l + 16) (lds_off wave-uniform). Issued through
// asm so that the compiler does not insert its conservative "wait for every LDS
// access" (lgkmcnt(0)) around the DMA, which the compiler-managed builtin
// brings into the stage loops; callers wait on vmcnt themselves. The
// instruction takes its LDS base from M0 when it issues: the asm saves M0 in a
// scratch SGPR, sets it, issues the load and restores it, so M0 holds the
// compiler's value again when the asm ends.
__device__ inline void dma16(const void* src, uint32_t lds_off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_off), "v"(src)
      : "memory");
}

// Workgroup barrier after this wave's LDS accesses completed; the asm keeps the
// compiler from moving memory operations across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt immediates (gfx9 encoding): vmcnt(N), no wait on exp/lgkm.
constexpr int WAIT_VM0 = 0x0F70;
constexpr int WAIT_VM4 = 0x0F74;
constexpr int WAIT_VM6 = 0x0F76;

// Brackets the launches made in its scope with trace events when a trace is
// active on this thread (gptq_trace_start); `work` is the launch's executed
// matrix-core flops (0 when not counted).
// Turns the trace off on this thread for its lifetime (entry points that must
// not create events), restoring it afterwards.
class TracePause {
 public:
  TracePause();
  ~TracePause();

 private:
  bool was_on_;
};

class TraceScope {
 public:
  TraceScope(hipStream_t st, int family, double work = 0.0);
  ~TraceScope() { end(); }
  void end();  // records the closing event now (once)
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  hipStream_t st_;
  int idx_;
};

// Entry points of the individual kernel families (implemented in the .hip files).
gptq_status_t syrk_enqueue(void* H, int h_f64, int64_t d, int64_t ldh, const half_t* X, int64_t n,
                           int64_t ldx, int accumulate, void* ws, size_t ws_bytes, hipStream_t st,
                           bool allow_xt = true);
size_t syrk_workspace_bytes(int64_t d, int64_t n);
// The split-K partial tiles alone (what the token-major form needs; the
// feature-major copy of X is the rest of syrk_workspace_bytes).
size_t syrk_partials_workspace_bytes(int64_t d, int64_t n);

// Size of the SYRK's static scratch array (gptq_accumulate_hessian_noalloc):
// 768 fp64 partial tiles of 256 x 128 (192 MiB): the most a launch's split-K
// plan uses for any d <= 65536 over 262144 tokens (182 MiB at d = 3104..3328).
constexpr size_t kStaticScratchBytes = (size_t)768 * 256 * 128 * sizeof(double);
// The current device's address of that array (hipGetSymbolAddress, taken once
// per device and kept).
gptq_status_t static_scratch(void** ptr);

// inverse = 1: U = chol_upper(H_d^-1) = J L^-1 J; inverse = 0: R = J L J, the
// upper factor with H_d = R R^T (R = U^-1), without the triangular inverse.
gptq_status_t chain_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, double damp, void* U,
                            int u_f64, int64_t ldu, int32_t* info, double* lambda_out, void* ws,
                            size_t ws_bytes, hipStream_t st, int inverse = 1);
size_t chain_workspace_bytes(int64_t d);

// perm (optional): the quantization order, W and the outputs staying in natural
// column order; static_groups and g_idx as in gptq_quantize_layer_ordered.
gptq_status_t quant_enqueue(const void* W, int w_f32, int64_t m, int64_t d, int64_t ldw, const void* U,
                            int u_f64, int64_t ldu, const gptq_qcfg_t& cfg, uint32_t* qcodes,
                            float* scales, uint8_t* zeros, float* W_hat, float* err_sq, void* ws,
                            size_t ws_bytes, hipStream_t st, const int32_t* perm = nullptr,
                            int static_groups = 0, int32_t* g_idx = nullptr);
size_t quant_workspace_bytes(int64_t m, int64_t d, const gptq_qcfg_t& cfg);

// Act-order: perm[j] = the column with the j-th largest H_jj (ties in index
// order); Hp = H gathered into that order (lower triangles).
gptq_status_t act_order_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, int32_t* perm, hipStream_t st);
gptq_status_t permute_hessian_enqueue(const void* H, int h_f64, int64_t d, int64_t ldh, const int32_t* perm,
                                      void* Hp, int64_t ldp, hipStream_t st);

// C[i][j] -= rowscale[i] * cscale * sum_k A[i][k] B[k][j] for i < M, j < N, with
// A = Ah + Al and B = Bh + Bl given as fp16 pairs and the product taken as
// Ah Bh + Ah Bl + Al Bh on the fp16 matrix cores (fp32 accumulate).
// Both operands are stored K-tiled in slabs of 32 (so that one slab of 16 rows
// is 1 KB of contiguous memory):
//   A(i, k) at (k / 32) * a_kslab + i * 32 + k % 32   (a_kslab >= 32 * M)
//   B(k, j) at (k / 128) * b_block + ((k % 128) / 32) * b_kslab + j * 32 + k % 32
// K % 32 == 0.
struct TgemmArgs {
  float* C;
  int64_t ldc;
  const half_t* Ah;
  const half_t* Al;
  int64_t a_kslab;
  const float* rowscale;
  const half_t* Bh;
  const half_t* Bl;
  int64_t b_block, b_kslab;
  const float* cscale;  // device scalar (power of two), multiplies every row
  int64_t M, N, K;
};
gptq_status_t tgemm_enqueue(const TgemmArgs& a, hipStream_t st);

// y = W_hat x from the packed codes (one token); x fp16 [d] 16-byte aligned.
gptq_status_t dq_gemv_enqueue(const uint32_t* q, const float* scales, const uint8_t* zeros, int64_t m, int64_t d,
                              int bits, int group, const half_t* x, float* y, hipStream_t st);

// Act-order codes in group order (col_perm sorts the columns by g_idx) and
// x gathered in that order, for the generation product.
gptq_status_t gemv_act_order_prepare(const uint32_t* q, const int32_t* g_idx, int64_t m, int64_t d, int bits,
                                     int group, uint32_t* out, int32_t* col_perm, int32_t* info, hipStream_t st);
gptq_status_t gather_x_enqueue(const half_t* x, const int32_t* col_perm, int64_t d, half_t* xp, hipStream_t st);

gptq_status_t pack_enqueue(const uint8_t* codes, int64_t ldc, int64_t m, int64_t d, int bits,
                           uint32_t* out, hipStream_t st);

}  // namespace gptq
