// Column order for activation ordering ("GPTQ：基于近似二阶信息的大模型权重量化",
// GPTQ 的高级技巧, 激活排序（desc_act）): the columns are taken by the sum of
// the absolute values of their input activations, least influential first.
//
//   a_c = sum_t |X[t][c]|   (float64),   perm = columns by ascending a_c,
//                                          ties by column index.
//
// act_sum_kernel sums 256-token ranges (workgroup rows blockIdx.y, strided),
// eight adjacent columns per thread when the layout allows 16-byte loads;
// act_reduce_kernel adds the ranges in a fixed order; act_rank_kernel gives
// column c the position #{c' : a_c' < a_c, or a_c' = a_c and c' < c}, so the
// result is deterministic and equals a stable ascending sort.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int AO_TOK = 256;   // tokens per range

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ void act_sum_range(const void* __restrict__ X, int x_dtype, int64_t n,
                                              int64_t ldx, int64_t d, int vec, int64_t range,
                                              double* __restrict__ partial) {
  const int64_t t0 = range * AO_TOK, t1 = min<int64_t>(n, t0 + AO_TOK);
  double* out = partial + range * d;
  if (vec) {  // bf16, 8 columns per thread
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c0 >= d) return;
    double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* base = (const uint16_t*)X + c0;
    // 8 tokens' loads in flight (clamped to the range, masked after)
    for (int64_t tb = t0; tb < t1; tb += 8) {
      uint4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = *(const uint4*)(base + min(tb + u, t1 - 1) * ldx);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tb + u >= t1) break;
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[2 * i] += fabs((double)__uint_as_float(w[i] << 16));
          s[2 * i + 1] += fabs((double)__uint_as_float(w[i] & 0xffff0000u));
        }
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

// token ranges blockIdx.y, blockIdx.y + gridDim.y, ...
__global__ __launch_bounds__(256) void act_sum_kernel(const void* __restrict__ X, int x_dtype,
                                                      int64_t n, int64_t ldx, int64_t d, int vec,
                                                      int64_t ranges,
                                                      double* __restrict__ partial) {
  for (int64_t r = blockIdx.y; r < ranges; r += gridDim.y)
    act_sum_range(X, x_dtype, n, ldx, d, vec, r, partial);
}

// a_c = sum over ranges of partial[r][c], in a fixed order: thread (column
// cl, slice sl) of a workgroup of 32 columns adds ranges sl, sl + 8, ... (loads
// eight deep), then slice 0 adds the eight slice sums in order.
__global__ __launch_bounds__(256) void act_reduce_kernel(const double* __restrict__ partial,
                                                         int64_t ranges, int64_t d,
                                                         double* __restrict__ a) {
  __shared__ double part[8][32];
  const int cl = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int64_t c = (int64_t)blockIdx.x * 32 + cl;
  const int64_t cc = min<int64_t>(c, d - 1);
  double s = 0.0;
  for (int64_t r0 = sl; r0 < ranges; r0 += 8 * 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[min<int64_t>(r0 + 8 * u, ranges - 1) * d + cc];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (r0 + 8 * u < ranges) ? v[u] : 0.0;
  }
  part[sl][cl] = s;
  __syncthreads();
  if (sl == 0 && c < d) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += part[k][cl];
    a[c] = t;
  }
}

// One wave per column c (four per workgroup): lane l counts the columns
// c' = l, l + 64, ... that come before c (loads eight deep), and the counts
// are summed across the wave (integers: the order does not matter).
__global__ __launch_bounds__(256) void act_rank_kernel(const double* __restrict__ a, int64_t d,
                                                       int32_t* __restrict__ perm) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= d) return;
  const double ac = a[c];
  int cnt = 0;
  for (int64_t b0 = lane; b0 < d; b0 += 64 * 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a[min<int64_t>(b0 + 64 * u, d - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t e = b0 + 64 * u;
      cnt += (e < d && (v[u] < ac || (v[u] == ac && e < c))) ? 1 : 0;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, 64);
  if (lane == 0 && cnt < d) perm[cnt] = (int32_t)c;
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
    hipLaunchKernelGGL(act_reduce_kernel, dim3((unsigned)ceil_div(d, 32)), dim3(256), 0, stream,
                       (const double*)partial, (int64_t)0, d, a);
  } else {
    const int vec = (x_dtype == 0) && (d % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0);
    const dim3 grid((unsigned)ceil_div(vec ? d / 8 : d, 256),
                    (unsigned)std::min<int64_t>(ranges, 65535));
    hipLaunchKernelGGL(act_sum_kernel, grid, dim3(256), 0, stream, X, x_dtype, n, ldx, d, vec,
                       ranges, partial);
    hipLaunchKernelGGL(act_reduce_kernel, dim3((unsigned)ceil_div(d, 32)), dim3(256), 0, stream,
                       (const double*)partial, ranges, d, a);
  }
  hipLaunchKernelGGL(act_rank_kernel, dim3((unsigned)ceil_div(d, 4)), dim3(256), 0, stream,
                     (const double*)a, d, perm);
  return hipGetLastError();
}

}  // namespace gptq
