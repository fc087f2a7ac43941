// Column order for activation ordering ("GPTQ：基于近似二阶信息的大模型权重量化",
// GPTQ 的高级技巧, 激活排序（desc_act）): the columns are taken by the sum of
// the absolute values of their input activations, least influential first.
//
//   a_c = sum_t |X[t][c]|   (float64),   perm = columns by ascending a_c,
//                                          ties by column index.
//
// act_sum_kernel sums one token range per workgroup row (blockIdx.y), eight
// adjacent columns per thread when the layout allows 16-byte loads;
// act_reduce_kernel adds the ranges in a fixed order; act_rank_kernel gives
// column c the position #{c' : a_c' < a_c, or a_c' = a_c and c' < c}, so the
// result is deterministic and equals a stable ascending sort.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int AO_TOK = 1024;  // tokens per range
constexpr int AO_TILE = 2048; // columns of a per LDS tile in the rank kernel

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ __launch_bounds__(256) void act_sum_kernel(const void* __restrict__ X, int x_dtype,
                                                      int64_t n, int64_t ldx, int64_t d, int vec,
                                                      double* __restrict__ partial) {
  const int64_t t0 = (int64_t)blockIdx.y * AO_TOK, t1 = min<int64_t>(n, t0 + AO_TOK);
  double* out = partial + (int64_t)blockIdx.y * d;
  if (vec) {  // bf16, 8 columns per thread
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c0 >= d) return;
    double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* base = (const uint16_t*)X + c0;
    for (int64_t t = t0; t < t1; ++t) {
      const uint4 raw = *(const uint4*)(base + t * ldx);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += fabs((double)__uint_as_float(w[i] << 16));
        s[2 * i + 1] += fabs((double)__uint_as_float(w[i] & 0xffff0000u));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) out[c0 + i] = s[i];
    return;
  }
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double s = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    const float v = (x_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)X)[t * ldx + c])
                                   : ((const float*)X)[t * ldx + c];
    s += fabs((double)v);
  }
  out[c] = s;
}

__global__ __launch_bounds__(256) void act_reduce_kernel(const double* __restrict__ partial,
                                                         int64_t ranges, int64_t d,
                                                         double* __restrict__ a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double s = 0.0;
  for (int64_t r = 0; r < ranges; ++r) s += partial[r * d + c];
  a[c] = s;
}

__global__ __launch_bounds__(256) void act_rank_kernel(const double* __restrict__ a, int64_t d,
                                                       int32_t* __restrict__ perm) {
  __shared__ double tile[AO_TILE];
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const double ac = (c < d) ? a[c] : 0.0;
  int64_t rank = 0;
  for (int64_t b = 0; b < d; b += AO_TILE) {
    const int64_t nb = min<int64_t>(AO_TILE, d - b);
    __syncthreads();
    for (int64_t e = threadIdx.x; e < nb; e += 256) tile[e] = a[b + e];
    __syncthreads();
    for (int64_t e = 0; e < nb; ++e) {
      const double v = tile[e];
      rank += (v < ac || (v == ac && b + e < c)) ? 1 : 0;
    }
  }
  if (c < d && rank < d) perm[rank] = (int32_t)c;
}

}  // namespace

size_t act_order_workspace(int64_t d, int64_t n_tokens) {
  if (d <= 0) return 0;
  const int64_t ranges = std::max<int64_t>(1, ceil_div(n_tokens, AO_TOK));
  return align256((size_t)ranges * d * sizeof(double)) + align256((size_t)d * sizeof(double));
}

hipError_t act_order_launch(const void* X, int x_dtype, int64_t n, int64_t ldx, int64_t d,
                            int32_t* perm, double* act_sum, void* ws, hipStream_t stream) {
  const int64_t ranges = std::max<int64_t>(1, ceil_div(n, AO_TOK));
  double* partial = (double*)ws;
  double* a = act_sum ? act_sum
                      : (double*)((char*)ws + align256((size_t)ranges * d * sizeof(double)));
  if (n == 0) {
    // every column has influence 0: the natural order
    hipLaunchKernelGGL(act_reduce_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, stream,
                       (const double*)partial, (int64_t)0, d, a);
  } else {
    const int vec = (x_dtype == 0) && (d % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0);
    const dim3 grid((unsigned)ceil_div(vec ? d / 8 : d, 256), (unsigned)ranges);
    hipLaunchKernelGGL(act_sum_kernel, grid, dim3(256), 0, stream, X, x_dtype, n, ldx, d, vec,
                       partial);
    hipLaunchKernelGGL(act_reduce_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, stream,
                       (const double*)partial, ranges, d, a);
  }
  hipLaunchKernelGGL(act_rank_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, stream,
                     (const double*)a, d, perm);
  return hipGetLastError();
}

}  // namespace gptq
