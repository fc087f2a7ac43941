// Host-only stand-ins for the launch layer (kernels.h), so the C ABI front
// end (gptq_abi.cpp) can be built and exercised under the address and
// undefined-behaviour sanitizers without a GPU.  Each stand-in checks what
// the front end promises before it launches (non-null buffers, positive
// sizes, a workspace at least the size the front end itself reported) and
// counts the calls; workspace sizes are small closed forms of the shapes.
#include <cstdio>
#include <cstdlib>

#include "kernels.h"

int g_launches = 0;

namespace {
void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: front end broke its promise: %s\n", what);
    std::abort();
  }
}
alignas(256) unsigned char g_scratch[4096];
}  // namespace

namespace gptq {

SyrkPlan syrk_plan(int64_t d, int64_t n, int x_dtype) {
  need(d > 0 && n > 0, "syrk_plan sizes");
  SyrkPlan p{};
  p.tile = x_dtype == 0 ? 256 : 64;
  p.ntile = (int)((d + p.tile - 1) / p.tile);
  p.ntri = p.ntile * (p.ntile + 1) / 2;
  p.splits = n > 1000 ? 3 : 1;
  p.kper = (n + p.splits - 1) / p.splits;
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * p.ntri * 1024 : 0;
  p.ws_bytes = p.partial_bytes;
  return p;
}
SyrkPlan syrk_plan_capped(int64_t d, int64_t n, int x_dtype, size_t max_bytes) {
  SyrkPlan p = syrk_plan(d, n, x_dtype);
  if (p.ws_bytes > max_bytes) p.splits = d > 100000 ? 0 : 1;  // huge d: not even one split
  return p;
}
hipError_t syrk_scratch(void** ptr) {
  need(ptr != nullptr, "syrk_scratch out pointer");
  *ptr = g_scratch;
  return hipSuccess;
}
hipError_t syrk_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n, int64_t ldx,
                       void* ws, const SyrkPlan& plan, hipStream_t) {
  need(H && X && d > 0 && n > 0 && ldx >= d && (x_dtype == 0 || x_dtype == 1), "syrk_launch");
  need(plan.splits >= 1 && (plan.ws_bytes == 0 || ws), "syrk_launch workspace");
  ++g_launches;
  return hipSuccess;
}
size_t prepare_workspace(int64_t d) { return 4096 + 16 * (size_t)d; }
hipError_t prepare_launch(float* H, int64_t d, double damp, float* U, uint8_t*, int32_t* st,
                          void* ws, hipStream_t) {
  need(H && U && st && ws && d > 0 && damp >= 0.0, "prepare_launch");
  ++g_launches;
  return hipSuccess;
}
hipError_t prepare_perm_launch(float* H, int64_t d, double damp, const int32_t*, float* U,
                               uint8_t*, int32_t* st, void* ws, hipStream_t) {
  need(H && U && st && ws && d > 0 && damp >= 0.0, "prepare_perm_launch");
  ++g_launches;
  return hipSuccess;
}
size_t quantize_workspace(int64_t d_out, int64_t d_in, int) {
  return 2048 + 8 * (size_t)(d_out + d_in);
}
hipError_t quantize_launch(const void* W, int, int64_t d_out, int64_t d_in, const float* U,
                           const uint8_t*, int bits, int, int, uint8_t* codes, float* scales,
                           float* zeros, float*, void* ws, hipStream_t) {
  need(W && U && codes && scales && zeros && ws && d_out > 0 && d_in > 0, "quantize_launch");
  need(bits >= 2 && bits <= 4, "quantize_launch bits");
  ++g_launches;
  return hipSuccess;
}
size_t quantize_perm_workspace(int64_t d_out, int64_t d_in, int) {
  return 3072 + 8 * (size_t)(d_out + d_in);
}
hipError_t quantize_perm_launch(const void* W, int, int64_t d_out, int64_t d_in, const float* U,
                                const uint8_t*, const int32_t*, int static_groups, int bits, int,
                                int, uint8_t* codes, float* scales, float* zeros, int32_t*,
                                float*, void* ws, hipStream_t) {
  need(W && U && codes && scales && zeros && ws && d_out > 0 && d_in > 0, "quantize_perm_launch");
  need(bits >= 2 && bits <= 4 && (static_groups == 0 || static_groups == 1), "perm flags");
  ++g_launches;
  return hipSuccess;
}
hipError_t quantize_multi_launch(const void* const* Ws, const int64_t* d_outs, int count, int,
                                 int64_t d_in, const float* U, const uint8_t*, int bits, int, int,
                                 uint8_t* codes, float* scales, float* zeros, float*, void* ws,
                                 hipStream_t) {
  need(Ws && d_outs && count >= 1 && d_in > 0 && U && codes && scales && zeros && ws,
       "quantize_multi_launch");
  for (int i = 0; i < count; ++i) need(d_outs[i] >= 0 && (d_outs[i] == 0 || Ws[i]), "list entry");
  need(bits >= 2 && bits <= 4, "quantize_multi_launch bits");
  ++g_launches;
  return hipSuccess;
}
size_t act_order_workspace(int64_t d, int64_t) { return 1024 + 8 * (size_t)d; }
hipError_t act_order_launch(const void* X, int, int64_t n, int64_t ldx, int64_t d,
                            int32_t* perm, double*, void* ws, hipStream_t) {
  need(perm && ws && d > 0 && ldx >= d && (n == 0 || X), "act_order_launch");
  ++g_launches;
  return hipSuccess;
}
hipError_t pack_launch(const uint8_t* codes, const float* scales, const float* zeros,
                       int64_t d_out, int64_t d_in, int bits, int n_groups, int sym,
                       uint32_t* qweight, uint16_t* scales_f16, uint16_t* zeros_f16,
                       hipStream_t) {
  need(codes && scales && qweight && scales_f16 && d_out > 0 && d_in > 0, "pack_launch");
  need(n_groups >= 1 && bits >= 2 && bits <= 4 && (sym || (zeros && zeros_f16)), "pack_launch");
  ++g_launches;
  return hipSuccess;
}
hipError_t w4a16_launch(const void* X, int64_t m, int64_t ldx, const uint32_t* qweight,
                        const uint16_t* scales_f16, const uint16_t*, int64_t d_out, int64_t d_in,
                        int, float* Y, hipStream_t) {
  need(X && qweight && scales_f16 && Y && m > 0 && d_out > 0 && d_in > 0 && ldx >= d_in,
       "w4a16_launch");
  ++g_launches;
  return hipSuccess;
}
size_t gptq2d_workspace(int64_t n) { return 512 + 16 * (size_t)n; }
hipError_t gptq2d_launch(const double* Y, const double* RL, const double* RR, int64_t n,
                         double* Z, void* ws, hipStream_t) {
  need(Y && RL && RR && Z && ws && n > 0, "gptq2d_launch");
  ++g_launches;
  return hipSuccess;
}

}  // namespace gptq
