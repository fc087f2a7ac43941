// Two-sided adaptive rounding ("GPTQ-2D: 三次时间复杂度的双侧自适应舍入",
// 方法 steps 1-3 and 核心洞察): round a real n x n matrix Y to an integer
// matrix Z under the metric that puts a fixed nonsingular basis on each side,
//   || R_L (Y - Z) R_R^T ||_F^2,
// R_L and R_R upper triangular with positive diagonals.  Vectorized, the Gram
// is the Kronecker product R_R^T R_R (x) R_L^T R_L and its triangular factor is
// R_R (x) R_L; nearest-plane rounding on it, last coordinate first, needs
// entry (i, j) after every entry (k, l) with k >= i and l >= j, so the entries
// of one anti-diagonal i + j = s are independent and the anti-diagonals go
// from s = 2n - 2 down to 0.
//
// Errors e = Y - Z reach later entries through one running array
//   P[k][j] = sum over processed (k, l), l >= j, of e[k][l] R_R[j][l],
// so entry (i, j) needs
//   S = sum_{k >= i} R_L[i][k] P[k][j],   Z[i][j] = rint(Y[i][j] + S / (R_L[i][i] R_R[j][j])),
// and then adds e[i][j] R_R[0..j][j] to row i of P: O(n) per entry, O(n^3)
// in all.  On one anti-diagonal the rows are distinct and the column an entry
// reads lies right of every column a lower entry writes, so the entries run
// in parallel; kernel boundaries order the anti-diagonals.
//
// Layout: P row-major (the update of row i is a contiguous store); the read of
// column j strides by n, but the entries of one anti-diagonal read adjacent
// columns of the same rows, so neighbouring entries (the waves of a
// workgroup) share cache lines.  R_R is transposed once (RT[j][c] = R_R[c][j])
// so the update reads a contiguous row.  Everything is float64.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int G2_WAVES = 4;  // entries per workgroup, one wave each

// P = 0 and RT = R_R^T (upper triangle of R_R only; the rest of RT zero).
__global__ __launch_bounds__(256) void g2d_init_kernel(const double* __restrict__ RR,
                                                       double* __restrict__ RT,
                                                       double* __restrict__ P, int n) {
  const int64_t total = (int64_t)n * n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e / n), c = (int)(e % n);
    RT[e] = (c <= j) ? RR[(int64_t)c * n + j] : 0.0;
    P[e] = 0.0;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  // xor butterfly: every lane ends with the same value (each step adds the
  // same two operands on both partners)
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

constexpr int G2_B = 8;  // loads in flight per lane and operand

// Anti-diagonal s: entry i_lo + 4 blockIdx.x + wave.  Loads go in batches of
// G2_B from clamped (in-bounds) addresses, masked afterwards; the first batch
// of the update's operands does not depend on the error and is loaded with
// the feedback sum's.
__global__ __launch_bounds__(256) void g2d_diag_kernel(const double* __restrict__ Y,
                                                       const double* __restrict__ RL,
                                                       const double* __restrict__ RT,
                                                       double* __restrict__ P,
                                                       double* __restrict__ Z, int n, int s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i_lo = max(0, s - n + 1), i_hi = min(s, n - 1);
  const int i = i_lo + (int)blockIdx.x * G2_WAVES + wave;
  if (i > i_hi) return;
  const int j = s - i;
  const double* rl = RL + (int64_t)i * n;
  const double* rt = RT + (int64_t)j * n;
  double* prow = P + (int64_t)i * n;
  double pv[G2_B], tv[G2_B];
#pragma unroll
  for (int u = 0; u < G2_B; ++u) {
    const int c = min(lane + 64 * u, j);
    pv[u] = prow[c];
    tv[u] = rt[c];
  }
  double acc0 = 0.0, acc1 = 0.0;
  for (int k0 = i + lane; k0 < n + 63; k0 += 64 * G2_B) {
    double a[G2_B], b[G2_B];
#pragma unroll
    for (int u = 0; u < G2_B; ++u) {
      const int k = min(k0 + 64 * u, n - 1);
      a[u] = rl[k];
      b[u] = P[(int64_t)k * n + j];
    }
#pragma unroll
    for (int u = 0; u < G2_B; ++u) {
      const double x = (k0 + 64 * u < n) ? a[u] : 0.0;
      if (u & 1) acc1 = fma(x, b[u], acc1);
      else acc0 = fma(x, b[u], acc0);
    }
  }
  const double acc = wave_sum(acc0 + acc1);
  const double y = Y[(int64_t)i * n + j];
  const double z = rint(y + acc / (rl[i] * rt[j]));
  const double e = y - z;
  if (lane == 0) Z[(int64_t)i * n + j] = z;
#pragma unroll
  for (int u = 0; u < G2_B; ++u) {
    const int c = lane + 64 * u;
    if (c <= j) prow[c] = fma(e, tv[u], pv[u]);
  }
  for (int c0 = lane + 64 * G2_B; c0 <= j; c0 += 64 * G2_B) {
#pragma unroll
    for (int u = 0; u < G2_B; ++u) {
      const int c = min(c0 + 64 * u, j);
      pv[u] = prow[c];
      tv[u] = rt[c];
    }
#pragma unroll
    for (int u = 0; u < G2_B; ++u) {
      const int c = c0 + 64 * u;
      if (c <= j) prow[c] = fma(e, tv[u], pv[u]);
    }
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t gptq2d_workspace(int64_t n) {
  return n <= 0 ? 0 : 2 * align256((size_t)n * n * sizeof(double));
}

hipError_t gptq2d_launch(const double* Y, const double* RL, const double* RR, int64_t n64,
                         double* Z, void* ws, hipStream_t stream) {
  const int n = (int)n64;
  double* P = (double*)ws;
  double* RT = (double*)((char*)ws + align256((size_t)n * n * sizeof(double)));
  const int64_t total = (int64_t)n * n;
  const int grid = (int)std::min<int64_t>(ceil_div(total, 256), 16384);
  hipLaunchKernelGGL(g2d_init_kernel, dim3(grid), dim3(256), 0, stream, RR, RT, P, n);
  for (int s = 2 * n - 2; s >= 0; --s) {
    const int m = std::min(s, n - 1) - std::max(0, s - n + 1) + 1;
    hipLaunchKernelGGL(g2d_diag_kernel, dim3((unsigned)ceil_div(m, G2_WAVES)),
                       dim3(64 * G2_WAVES), 0, stream, Y, RL, (const double*)RT, P, Z, n, s);
  }
  return hipGetLastError();
}

}  // namespace gptq
