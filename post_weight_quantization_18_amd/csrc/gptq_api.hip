// C ABI of the gfx950 GPTQ library: host-side validation, workspace sizing and
// stream-ordered dispatch to the kernel families. See include/gptq.h for the
// contract of each entry point.
#include <new>

#include "common.h"

namespace gptq {
size_t quant_workspace_bytes_u64(int64_t m, int64_t d, const gptq_qcfg_t& cfg);
}

using namespace gptq;

namespace {

bool valid_qcfg(const gptq_qcfg_t& c, int64_t d) {
  if (c.block_size != 128) return false;
  if (c.grid != GPTQ_GRID_ASYM_MINMAX && c.grid != GPTQ_GRID_TERNARY && c.grid != GPTQ_GRID_SYM_MINMAX) return false;
  if (c.grid == GPTQ_GRID_TERNARY && c.bits != 2) return false;
  if (c.bits != 2 && c.bits != 3 && c.bits != 4 && c.bits != 8) return false;
  const int g = c.group_size;
  if (g < 0) return false;
  if (g == 0) return true;
  if (d % g) return false;
  if (g == 32 || g == 64 || g == 128) return true;
  return g % 128 == 0 && d % 128 == 0;
}

gptq_qcfg_t default_qcfg() {
  gptq_qcfg_t c;
  c.bits = 4;
  c.grid = GPTQ_GRID_ASYM_MINMAX;
  c.group_size = 0;
  c.block_size = 128;
  return c;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

int32_t gptq_abi_version(void) { return 1; }

const char* gptq_status_string(int32_t s) {
  switch (s) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG: invalid argument";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE: workspace missing or too small";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP: a HIP launch failed";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED: unsupported option or device";
    default: return "unknown gptq status";
  }
}

size_t gptq_workspace_bytes(int32_t which, int64_t m, int64_t d, int64_t n, const gptq_qcfg_t* cfg) {
  if (d <= 0) return 0;
  switch (which) {
    case GPTQ_WS_ACCUMULATE_HESSIAN: return n > 0 ? syrk_workspace_bytes(d, n) : 0;
    case GPTQ_WS_PREPARE_HINV: return chain_workspace_bytes(d);
    case GPTQ_WS_QUANTIZE_LAYER: {
      if (m <= 0) return 0;
      gptq_qcfg_t c = cfg ? *cfg : default_qcfg();
      return quant_workspace_bytes_u64(m, d, c);  // enough for either U dtype
    }
    default: return 0;
  }
}

gptq_status_t gptq_accumulate_hessian(void* H, int32_t h_dtype, int64_t d, int64_t ldh, const void* X, int64_t n,
                                      int64_t ldx, int32_t accumulate, void* workspace, size_t ws_bytes,
                                      void* stream) {
  if (!H || d <= 0 || d % 32 || ldh < d || n < 0) return GPTQ_ERR_INVALID_ARG;
  if (h_dtype != GPTQ_F32 && h_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (n > 0 && (!X || ldx < d || ldx % 8 || !aligned(X, 16))) return GPTQ_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 256)) return GPTQ_ERR_INVALID_ARG;
  return syrk_enqueue(H, h_dtype == GPTQ_F64, d, ldh, (const half_t*)X, n, ldx, accumulate != 0, workspace,
                      ws_bytes, (hipStream_t)stream);
}

gptq_status_t gptq_prepare_hinv(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, double damp, void* U,
                                int32_t u_dtype, int64_t ldu, int32_t* info, double* lambda_out, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (!H || !U || !info || d <= 0 || ldh < d || ldu < d) return GPTQ_ERR_INVALID_ARG;
  if (!(damp >= 0.0)) return GPTQ_ERR_INVALID_ARG;
  if (h_dtype != GPTQ_F32 && h_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (u_dtype != GPTQ_F32 && u_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (H == U) return GPTQ_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < chain_workspace_bytes(d)) return GPTQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GPTQ_ERR_INVALID_ARG;
  return chain_enqueue(H, h_dtype == GPTQ_F64, d, ldh, damp, U, u_dtype == GPTQ_F64, ldu, info, lambda_out,
                       workspace, ws_bytes, (hipStream_t)stream);
}

gptq_status_t gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t m, int64_t d, int64_t ldw, const void* U,
                                  int32_t u_dtype, int64_t ldu, const gptq_qcfg_t* cfg, uint32_t* qcodes,
                                  float* scales, uint8_t* zeros, float* W_hat, float* err_sq, void* workspace,
                                  size_t ws_bytes, void* stream) {
  if (!W || !U || !cfg || !qcodes || !scales || !zeros) return GPTQ_ERR_INVALID_ARG;
  if (m <= 0 || d <= 0 || d % 32 || ldw < d || ldu < d) return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return GPTQ_ERR_INVALID_ARG;
  if (u_dtype != GPTQ_F32 && u_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (u_dtype == GPTQ_F32 && (ldu % 4 || !aligned(U, 16))) return GPTQ_ERR_INVALID_ARG;
  if (!valid_qcfg(*cfg, d)) return GPTQ_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256)) return GPTQ_ERR_WORKSPACE;
  return quant_enqueue(W, w_dtype == GPTQ_F32, m, d, ldw, U, u_dtype == GPTQ_F64, ldu, *cfg, qcodes, scales, zeros,
                       W_hat, err_sq, workspace, ws_bytes, (hipStream_t)stream);
}

gptq_status_t gptq_act_order(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, int32_t* perm, void* stream) {
  if (!H || !perm || d <= 0 || ldh < d) return GPTQ_ERR_INVALID_ARG;
  if (d > INT32_MAX) return GPTQ_ERR_INVALID_ARG;
  if (h_dtype != GPTQ_F32 && h_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  return act_order_enqueue(H, h_dtype == GPTQ_F64, d, ldh, perm, (hipStream_t)stream);
}

gptq_status_t gptq_permute_hessian(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, const int32_t* perm,
                                   void* Hp, int64_t ldhp, void* stream) {
  if (!H || !perm || !Hp || d <= 0 || ldh < d || ldhp < d) return GPTQ_ERR_INVALID_ARG;
  if (h_dtype != GPTQ_F32 && h_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (H == Hp) return GPTQ_ERR_INVALID_ARG;
  return permute_hessian_enqueue(H, h_dtype == GPTQ_F64, d, ldh, perm, Hp, ldhp, (hipStream_t)stream);
}

gptq_status_t gptq_quantize_layer_ordered(const void* W, int32_t w_dtype, int64_t m, int64_t d, int64_t ldw,
                                          const void* U, int32_t u_dtype, int64_t ldu, const gptq_qcfg_t* cfg,
                                          const int32_t* perm, int32_t static_groups, uint32_t* qcodes,
                                          float* scales, uint8_t* zeros, int32_t* g_idx, float* W_hat,
                                          float* err_sq, void* workspace, size_t ws_bytes, void* stream) {
  if (!W || !U || !cfg || !perm || !qcodes || !scales || !zeros) return GPTQ_ERR_INVALID_ARG;
  if (static_groups != 0 && static_groups != 1) return GPTQ_ERR_INVALID_ARG;
  if (m <= 0 || d <= 0 || d % 32 || d > INT32_MAX || ldw < d || ldu < d) return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return GPTQ_ERR_INVALID_ARG;
  if (u_dtype != GPTQ_F32 && u_dtype != GPTQ_F64) return GPTQ_ERR_INVALID_ARG;
  if (u_dtype == GPTQ_F32 && (ldu % 4 || !aligned(U, 16))) return GPTQ_ERR_INVALID_ARG;
  if (!valid_qcfg(*cfg, d)) return GPTQ_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256)) return GPTQ_ERR_WORKSPACE;
  return quant_enqueue(W, w_dtype == GPTQ_F32, m, d, ldw, U, u_dtype == GPTQ_F64, ldu, *cfg, qcodes, scales, zeros,
                       W_hat, err_sq, workspace, ws_bytes, (hipStream_t)stream, perm, static_groups, g_idx);
}

gptq_status_t gptq_dequant_gemv(const uint32_t* qcodes, const float* scales, const uint8_t* zeros, int64_t m,
                                int64_t d, int32_t bits, int32_t group_size, const void* x, float* y, void* stream) {
  if (!qcodes || !scales || !zeros || !x || !y || m <= 0 || d <= 0 || d % 32) return GPTQ_ERR_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_INVALID_ARG;
  if (group_size < 0 || (group_size && (group_size % 32 || d % group_size))) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(qcodes, 4)) return GPTQ_ERR_INVALID_ARG;
  return dq_gemv_enqueue(qcodes, scales, zeros, m, d, bits, group_size, (const half_t*)x, y, (hipStream_t)stream);
}

gptq_status_t gptq_pack_codes(const uint8_t* codes, int64_t m, int64_t d, int32_t bits, uint32_t* out,
                              void* stream) {
  if (!codes || !out || m <= 0 || d <= 0) return GPTQ_ERR_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_INVALID_ARG;
  if ((d * bits) % 32) return GPTQ_ERR_INVALID_ARG;
  return pack_enqueue(codes, d, m, d, bits, out, (hipStream_t)stream);
}

}  // extern "C"
