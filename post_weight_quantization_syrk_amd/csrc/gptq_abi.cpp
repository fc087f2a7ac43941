// C ABI front end: argument checks, workspace sizing and launch sequencing.
// Every entry point validates its arguments before enqueueing anything.
#include <hip/hip_runtime.h>

#include "../../include/gptq.h"
#include "kernels.h"

namespace {

inline bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_EHIP; }

bool valid_group(int64_t d_in, int group_size) {
  if (group_size == -1) return true;
  return group_size > 0 && d_in % group_size == 0;
}

bool supported_group(int group_size) {
  return group_size == -1 || group_size == 32 || group_size == 64 || group_size == 128;
}

}  // namespace

extern "C" {

int gptq_abi_version(void) { return 100; }

const char* gptq_strerror(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_EUNSUPPORTED: return "unsupported parameter";
    case GPTQ_EHIP: return "HIP runtime or launch failure";
    case GPTQ_ENOTSPD: return "Hessian not positive definite";
    default: return "unknown status";
  }
}

size_t gptq_hessian_workspace(int64_t d, int64_t n_tokens, int x_dtype) {
  if (d <= 0 || n_tokens < 0 || (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32)) return 0;
  if (n_tokens == 0) return 0;
  return gptq::syrk_plan(d, n_tokens, x_dtype).ws_bytes;
}

int gptq_hessian_accumulate(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tokens,
                            int64_t ldx, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (d <= 0 || d > (int64_t)1 << 20 || n_tokens < 0 || ldx < d) return GPTQ_EINVAL;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (!H) return GPTQ_EINVAL;
  if (n_tokens == 0) return GPTQ_OK;
  if (!X) return GPTQ_EINVAL;
  const gptq::SyrkPlan plan = gptq::syrk_plan(d, n_tokens, x_dtype);
  if (ws_bytes < plan.ws_bytes || (plan.ws_bytes && (!ws || !aligned256(ws)))) return GPTQ_EINVAL;
  return hip_status(
      gptq::syrk_launch(H, d, X, x_dtype, n_tokens, ldx, ws, plan, (hipStream_t)stream));
}

int gptq_hessian_accumulate_noalloc(float* H, int64_t d, const void* X, int x_dtype,
                                    int64_t n_tokens, int64_t ldx, gptq_stream stream) {
  if (d <= 0 || d > (int64_t)1 << 20 || n_tokens < 0 || ldx < d) return GPTQ_EINVAL;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (!H) return GPTQ_EINVAL;
  if (n_tokens == 0) return GPTQ_OK;
  if (!X) return GPTQ_EINVAL;
  const gptq::SyrkPlan plan =
      gptq::syrk_plan_capped(d, n_tokens, x_dtype, gptq::NOALLOC_SCRATCH_BYTES);
  if (plan.splits < 1) return GPTQ_EUNSUPPORTED;  // one split's partials exceed the array
  void* scratch = nullptr;
  const hipError_t e = gptq::syrk_scratch(&scratch);
  if (e != hipSuccess) return GPTQ_EHIP;
  return hip_status(
      gptq::syrk_launch(H, d, X, x_dtype, n_tokens, ldx, scratch, plan, (hipStream_t)stream));
}

size_t gptq_noalloc_scratch_bytes(void) { return gptq::NOALLOC_SCRATCH_BYTES; }

size_t gptq_prepare_workspace(int64_t d) {
  if (d <= 0) return 0;
  return gptq::prepare_workspace(d);
}

int gptq_prepare_hinv(float* H, int64_t d, double damp, float* U, uint8_t* dead,
                      int32_t* dev_status, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (d <= 0 || d > 65536 || !H || !U || !dev_status) return GPTQ_EINVAL;
  if (!(damp >= 0.0) || !(damp < 1e30)) return GPTQ_EINVAL;
  if (ws_bytes < gptq::prepare_workspace(d) || !ws || !aligned256(ws)) return GPTQ_EINVAL;
  return hip_status(
      gptq::prepare_launch(H, d, damp, U, dead, dev_status, ws, (hipStream_t)stream));
}

size_t gptq_quantize_workspace(int64_t d_out, int64_t d_in, int block) {
  if (d_out < 0 || d_in <= 0) return 0;
  return gptq::quantize_workspace(d_out, d_in, block);
}

int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U,
                        const uint8_t* dead, int bits, int group_size, int sym, int block,
                        uint8_t* codes, float* scales, float* zeros, float* loss_rows, void* ws,
                        size_t ws_bytes, gptq_stream stream) {
  if (d_out < 0 || d_in <= 0 || d_in > 65536) return GPTQ_EINVAL;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (bits != 2 && bits != 3 && bits != 4) return (bits == 8) ? GPTQ_EUNSUPPORTED : GPTQ_EINVAL;
  if (!valid_group(d_in, group_size)) return GPTQ_EINVAL;
  if (!supported_group(group_size)) return GPTQ_EUNSUPPORTED;
  if (sym != 0 && sym != 1) return GPTQ_EINVAL;
  if (block != 128) return GPTQ_EUNSUPPORTED;
  if (d_out == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros) return GPTQ_EINVAL;
  if (ws_bytes < gptq::quantize_workspace(d_out, d_in, block) || !ws || !aligned256(ws))
    return GPTQ_EINVAL;
  return hip_status(gptq::quantize_launch(W, w_dtype, d_out, d_in, U, dead, bits, group_size, sym,
                                          codes, scales, zeros, loss_rows, ws,
                                          (hipStream_t)stream));
}

int gptq_pack(const uint8_t* codes, const float* scales, const float* zeros, int64_t d_out,
              int64_t d_in, int bits, int group_size, int sym, uint32_t* qweight,
              uint16_t* scales_f16, uint16_t* zeros_f16, gptq_stream stream) {
  if (d_out < 0 || d_in <= 0) return GPTQ_EINVAL;
  if (bits != 2 && bits != 3 && bits != 4) return GPTQ_EINVAL;
  if (!valid_group(d_in, group_size)) return GPTQ_EINVAL;
  if (sym != 0 && sym != 1) return GPTQ_EINVAL;
  if (d_out == 0) return GPTQ_OK;
  if (!codes || !scales || !qweight || !scales_f16) return GPTQ_EINVAL;
  if (!sym && (!zeros || !zeros_f16)) return GPTQ_EINVAL;
  const int n_groups = (group_size == -1) ? 1 : (int)(d_in / group_size);
  return hip_status(gptq::pack_launch(codes, scales, zeros, d_out, d_in, bits, n_groups, sym,
                                      qweight, scales_f16, zeros_f16, (hipStream_t)stream));
}

size_t gptq_act_order_workspace(int64_t d, int64_t n_tokens) {
  return (d <= 0 || d > 65536 || n_tokens < 0) ? 0 : gptq::act_order_workspace(d, n_tokens);
}

int gptq_act_order(const void* X, int x_dtype, int64_t n_tokens, int64_t ldx, int64_t d,
                   int32_t* perm, double* act_sum, void* ws, size_t ws_bytes,
                   gptq_stream stream) {
  if (d <= 0 || d > 65536 || n_tokens < 0 || ldx < d) return GPTQ_EINVAL;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (!perm || (n_tokens > 0 && !X)) return GPTQ_EINVAL;
  if (ws_bytes < gptq::act_order_workspace(d, n_tokens) || !ws || !aligned256(ws))
    return GPTQ_EINVAL;
  return hip_status(gptq::act_order_launch(X, x_dtype, n_tokens, ldx, d, perm, act_sum, ws,
                                           (hipStream_t)stream));
}

int gptq_prepare_hinv_perm(float* H, int64_t d, double damp, const int32_t* perm, float* U,
                           uint8_t* dead, int32_t* dev_status, void* ws, size_t ws_bytes,
                           gptq_stream stream) {
  if (d <= 0 || d > 65536 || !H || !U || !dev_status) return GPTQ_EINVAL;
  if (!(damp >= 0.0) || !(damp < 1e30)) return GPTQ_EINVAL;
  if (ws_bytes < gptq::prepare_workspace(d) || !ws || !aligned256(ws)) return GPTQ_EINVAL;
  return hip_status(gptq::prepare_perm_launch(H, d, damp, perm, U, dead, dev_status, ws,
                                              (hipStream_t)stream));
}

size_t gptq_quantize_perm_workspace(int64_t d_out, int64_t d_in, int block) {
  if (d_out <= 0 || d_in <= 0) return 0;
  return gptq::quantize_perm_workspace(d_out, d_in, block);
}

int gptq_quantize_layer_perm(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                             const float* U, const uint8_t* dead, const int32_t* perm,
                             int static_groups, int bits, int group_size, int sym, int block,
                             uint8_t* codes, float* scales, float* zeros, int32_t* g_idx,
                             float* loss_rows, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (d_out < 0 || d_in <= 0 || d_in > 65536) return GPTQ_EINVAL;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (bits != 2 && bits != 3 && bits != 4) return (bits == 8) ? GPTQ_EUNSUPPORTED : GPTQ_EINVAL;
  if (!valid_group(d_in, group_size)) return GPTQ_EINVAL;
  if (!supported_group(group_size)) return GPTQ_EUNSUPPORTED;
  if (sym != 0 && sym != 1) return GPTQ_EINVAL;
  if (static_groups != 0 && static_groups != 1) return GPTQ_EINVAL;
  if (block != 128) return GPTQ_EUNSUPPORTED;
  if (d_out == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros) return GPTQ_EINVAL;
  if (ws_bytes < gptq::quantize_perm_workspace(d_out, d_in, block) || !ws || !aligned256(ws))
    return GPTQ_EINVAL;
  return hip_status(gptq::quantize_perm_launch(W, w_dtype, d_out, d_in, U, dead, perm,
                                               static_groups, bits, group_size, sym, codes,
                                               scales, zeros, g_idx, loss_rows, ws,
                                               (hipStream_t)stream));
}

int gptq_quantize_layers(const void* const* W_list, const int64_t* d_out_list, int count,
                         int w_dtype, int64_t d_in, const float* U, const uint8_t* dead, int bits,
                         int group_size, int sym, int block, uint8_t* codes, float* scales,
                         float* zeros, float* loss_rows, void* ws, size_t ws_bytes,
                         gptq_stream stream) {
  if (count < 1 || count > 64 || !W_list || !d_out_list) return GPTQ_EINVAL;
  if (d_in <= 0 || d_in > 65536) return GPTQ_EINVAL;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (bits != 2 && bits != 3 && bits != 4) return (bits == 8) ? GPTQ_EUNSUPPORTED : GPTQ_EINVAL;
  if (!valid_group(d_in, group_size)) return GPTQ_EINVAL;
  if (!supported_group(group_size)) return GPTQ_EUNSUPPORTED;
  if (sym != 0 && sym != 1) return GPTQ_EINVAL;
  if (block != 128) return GPTQ_EUNSUPPORTED;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    if (d_out_list[i] < 0) return GPTQ_EINVAL;
    if (d_out_list[i] > 0 && !W_list[i]) return GPTQ_EINVAL;
    rows += d_out_list[i];
  }
  if (rows == 0) return GPTQ_OK;
  if (rows > (int64_t)1 << 31) return GPTQ_EINVAL;
  if (!U || !codes || !scales || !zeros) return GPTQ_EINVAL;
  if (ws_bytes < gptq::quantize_workspace(rows, d_in, block) || !ws || !aligned256(ws))
    return GPTQ_EINVAL;
  return hip_status(gptq::quantize_multi_launch(W_list, d_out_list, count, w_dtype, d_in, U, dead,
                                                bits, group_size, sym, codes, scales, zeros,
                                                loss_rows, ws, (hipStream_t)stream));
}

int gptq_w4a16_matmul(const void* X, int64_t m, int64_t ldx, const uint32_t* qweight,
                      const uint16_t* scales_f16, const uint16_t* zeros_f16, int64_t d_out,
                      int64_t d_in, int group_size, int sym, float* Y, gptq_stream stream) {
  if (m < 0 || d_out <= 0 || d_in <= 0 || d_in > 65536 || d_out > (1 << 30)) return GPTQ_EINVAL;
  if (!valid_group(d_in, group_size)) return GPTQ_EINVAL;
  if (!supported_group(group_size)) return GPTQ_EUNSUPPORTED;
  if (sym != 0 && sym != 1) return GPTQ_EINVAL;
  if (d_in % 128 != 0) return GPTQ_EUNSUPPORTED;
  if (m == 0) return GPTQ_OK;
  if (m > (1 << 30) || ldx < d_in || ldx % 8 != 0) return GPTQ_EINVAL;
  if (!X || !qweight || !scales_f16 || !Y || (!sym && !zeros_f16)) return GPTQ_EINVAL;
  if ((uintptr_t)X % 16 != 0) return GPTQ_EINVAL;
  return hip_status(gptq::w4a16_launch(X, m, ldx, qweight, scales_f16, sym ? nullptr : zeros_f16,
                                       d_out, d_in, group_size, Y, (hipStream_t)stream));
}

size_t gptq2d_workspace(int64_t n) {
  return (n <= 0 || n > GPTQ2D_MAX_N) ? 0 : gptq::gptq2d_workspace(n);
}

int gptq2d_round(const double* Y, const double* left_basis, const double* right_basis, int64_t n,
                 double* Z, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (n < 0) return GPTQ_EINVAL;
  if (n > GPTQ2D_MAX_N) return GPTQ_EUNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  if (!Y || !left_basis || !right_basis || !Z || !ws) return GPTQ_EINVAL;
  if (ws_bytes < gptq::gptq2d_workspace(n) || !aligned256(ws)) return GPTQ_EINVAL;
  return hip_status(gptq::gptq2d_launch(Y, left_basis, right_basis, n, Z, ws,
                                        (hipStream_t)stream));
}

}  // extern "C"
