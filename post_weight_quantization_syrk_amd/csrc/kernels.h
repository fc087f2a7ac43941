// Internal launchers behind the C ABI (include/gptq.h).  Each returns the
// hipError_t of its launches; argument validation happens in gptq_abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace gptq {

// ---- Hessian: H(lower) += 2 X^T X --------------------------------------
struct SyrkPlan {
  int tile;        // output tile edge (256 for bf16, 64 for fp32)
  int ntile;       // tiles per dimension
  int ntri;        // lower-triangle tiles
  int splits;      // token splits (split-K)
  int64_t kper;    // tokens per split
  size_t partial_bytes; // split-K partial tiles [splits][ntri][tile * tile] fp32
  size_t ws_bytes;      // = partial_bytes
};
SyrkPlan syrk_plan(int64_t d, int64_t n, int x_dtype);
// The allocation-free entry point: its split-K partials live in a fixed
// per-device array of NOALLOC_SCRATCH_BYTES; the split count is capped to fit
// (splits = 0: even one split does not fit).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int MAX_DEVICES = 64;
SyrkPlan syrk_plan_capped(int64_t d, int64_t n, int x_dtype, size_t max_bytes);
hipError_t syrk_scratch(void** ptr);  // this device's copy of the array
hipError_t syrk_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n, int64_t ldx,
                       void* ws, const SyrkPlan& plan, hipStream_t stream);

// ---- prepare: dead channels, damping, factorization, U ------------------
size_t prepare_workspace(int64_t d);
hipError_t prepare_launch(float* H, int64_t d, double damp, float* U, uint8_t* dead,
                          int32_t* dev_status, void* ws, hipStream_t stream);
// The same for H[perm][:, perm] (perm null: natural order); dead stays in
// natural order, U is the permuted problem's factor.
hipError_t prepare_perm_launch(float* H, int64_t d, double damp, const int32_t* perm, float* U,
                               uint8_t* dead, int32_t* dev_status, void* ws, hipStream_t stream);

// Several weight matrices that share U (one Hessian), stacked by rows in
// order; outputs stacked the same way.
hipError_t quantize_multi_launch(const void* const* Ws, const int64_t* d_outs, int count,
                                 int w_dtype, int64_t d_in, const float* U, const uint8_t* dead,
                                 int bits, int group_size, int sym, uint8_t* codes,
                                 float* scales, float* zeros, float* loss_rows, void* ws,
                                 hipStream_t stream);

// ---- activation order: perm = columns by ascending sum_t |x_t,c| ----------
size_t act_order_workspace(int64_t d, int64_t n_tokens);
hipError_t act_order_launch(const void* X, int x_dtype, int64_t n_tokens, int64_t ldx, int64_t d,
                            int32_t* perm, double* act_sum, void* ws, hipStream_t stream);

// ---- quantize ------------------------------------------------------------
size_t quantize_workspace(int64_t d_out, int64_t d_in, int block);
hipError_t quantize_launch(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                           const float* U, const uint8_t* dead, int bits, int group_size,
                           int sym, uint8_t* codes, float* scales, float* zeros,
                           float* loss_rows, void* ws, hipStream_t stream);
// Columns processed in the order perm (null: natural order), static or
// dynamic groups; codes come back in natural order, g_idx (may be null) maps
// each column to its group.
size_t quantize_perm_workspace(int64_t d_out, int64_t d_in, int block);
hipError_t quantize_perm_launch(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                                const float* U, const uint8_t* dead, const int32_t* perm,
                                int static_groups, int bits, int group_size, int sym,
                                uint8_t* codes, float* scales, float* zeros, int32_t* g_idx,
                                float* loss_rows, void* ws, hipStream_t stream);

// ---- pack ----------------------------------------------------------------
hipError_t pack_launch(const uint8_t* codes, const float* scales, const float* zeros,
                       int64_t d_out, int64_t d_in, int bits, int n_groups, int sym,
                       uint32_t* qweight, uint16_t* scales_f16, uint16_t* zeros_f16,
                       hipStream_t stream);

// ---- dequantized product with 4-bit packed weights ------------------------
hipError_t w4a16_launch(const void* X, int64_t m, int64_t ldx, const uint32_t* qweight,
                        const uint16_t* scales_f16, const uint16_t* zeros_f16, int64_t d_out,
                        int64_t d_in, int group_size, float* Y, hipStream_t stream);

// Polls a bounded wait between workgroups may take before it gives up
// (environment GPTQ_SYNC_SPIN_LIMIT, default 2^20), read once per process.
int64_t sync_spin_limit();

// ---- two-sided rounding (anti-diagonal schedule) ----------------------------
size_t gptq2d_workspace(int64_t n);
hipError_t gptq2d_launch(const double* Y, const double* RL, const double* RR, int64_t n,
                         double* Z, void* ws, hipStream_t stream);

}  // namespace gptq
