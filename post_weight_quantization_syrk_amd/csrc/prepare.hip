// Damping, Cholesky and the upper factor of the inverse Hessian
// ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段一: H ~ 2X^T X + lambda I and a
// Cholesky factorization whose triangular factor drives the error feedback).
//
// U is the upper triangular matrix with U^T U = H^{-1}.  Rather than inverting H
// and factorizing again, it is formed as U = V^{-1} with H = V V^T, V upper: in
// the index-reversed space A = J H J (J reverses the order) this is an ordinary
// Cholesky A = L L^T and a triangular inverse M = L^{-1}, and U = J M J.  Both
// run blocked (64 x 64 blocks) in float64, right-looking, fused per step:
//   diag   : L_kk = chol(A_kk) and its inverse in one workgroup;
//   panel  : L_ik = A_ik L_kk^{-T} (i > k) and M_kj = L_kk^{-1} B_kj (j < k);
//   update : A_ij -= L_ik L_jk^T (i >= j > k) and B_ij -= L_ik M_kj (i > k >= j),
// where B accumulates the right-hand side of L M = I.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int NB = 64;
constexpr int LDP = 65;  // LDS pitch for 64 x 64 float64 tiles

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrepWs {
  double* A;     // [d x d] reversed damped H, then L (lower)
  double* M;     // [d x d] right-hand side / L^{-1} (lower)
  double* Dinv;  // [NB x NB] inverse of the current diagonal block
  double* scal;  // [0] = lambda
};

PrepWs carve(void* ws, int64_t d) {
  char* p = (char*)ws;
  PrepWs w;
  const size_t mat = align256((size_t)d * d * sizeof(double));
  w.A = (double*)p;
  w.M = (double*)(p + mat);
  w.Dinv = (double*)(p + 2 * mat);
  w.scal = (double*)(p + 2 * mat + align256(NB * NB * sizeof(double)));
  return w;
}

__device__ __forceinline__ void tri_coords(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// dead[i] = (H_ii == 0); lambda = damp * mean(diag) with dead entries counted as 1.
__global__ __launch_bounds__(1024) void prep_stats_kernel(const float* __restrict__ H, int d,
                                                          double damp, uint8_t* dead,
                                                          double* scal, int32_t* status) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 1024) {
    const float h = H[(int64_t)i * d + i];
    const bool dd = (h == 0.0f);
    if (dead) dead[i] = dd ? 1 : 0;
    s += dd ? 1.0 : (double)h;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    scal[0] = damp * (red[0] / (double)d);
    *status = 0;
  }
}

// Mirror the lower triangle of H into the upper one, damp the diagonal, and
// build A = J H J (lower triangle, float64) and zero the lower triangle of M.
__global__ __launch_bounds__(256) void prep_build_kernel(float* __restrict__ H, int d,
                                                         const double* __restrict__ scal,
                                                         double* __restrict__ A,
                                                         double* __restrict__ M) {
  __shared__ float t[32][33];
  int ti, tj;
  tri_coords(blockIdx.x, ti, tj);
  const int i0 = ti * 32, j0 = tj * 32;
  const double lam = scal[0];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + tx;
    t[r][tx] = (i < d && j < d && j <= i) ? H[(int64_t)i * d + j] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int j = j0 + r, i = i0 + tx;  // element H[i][j], i >= j
    if (i >= d || j >= d || j > i) continue;
    const float v = t[tx][r];
    const int64_t ar = d - 1 - j, ac = d - 1 - i;
    if (i == j) {
      const double dv = (v == 0.0f ? 1.0 : (double)v) + lam;
      H[(int64_t)i * d + i] = (float)dv;
      A[ar * d + ac] = dv;
    } else {
      H[(int64_t)j * d + i] = v;
      A[ar * d + ac] = (double)v;
    }
    M[ar * d + ac] = 0.0;
  }
}

// ---- 64 x 64 float64 tile products through LDS ---------------------------
struct TileLds {
  double p[NB][LDP];  // p[t][r] = P[r][t]
  double q[NB][LDP];  // q[t][c] = Q[t][c]
};

// dst[t][x] = src[x][t]
__device__ __forceinline__ void load_T(double (*dst)[LDP], const double* src, int64_t ld, int rows,
                                       int cols) {
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int x = e >> 6, tt = e & 63;
    dst[tt][x] = (x < rows && tt < cols) ? src[(int64_t)x * ld + tt] : 0.0;
  }
}
// dst[t][x] = src[t][x]
__device__ __forceinline__ void load_N(double (*dst)[LDP], const double* src, int64_t ld, int rows,
                                       int cols) {
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int tt = e >> 6, x = e & 63;
    dst[tt][x] = (tt < rows && x < cols) ? src[(int64_t)tt * ld + x] : 0.0;
  }
}

__device__ __forceinline__ void tile_mma(const TileLds& s, double (&acc)[4][4]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll 4
  for (int t = 0; t < NB; ++t) {
    double pv[4], qv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) pv[a] = s.p[t][4 * ty + a];
#pragma unroll
    for (int b = 0; b < 4; ++b) qv[b] = s.q[t][4 * tx + b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(pv[a], qv[b], acc[a][b]);
  }
}

// C (rows x cols valid) = acc  or  C -= acc
template <bool SUB>
__device__ __forceinline__ void store_tile(double* C, int64_t ld, int rows, int cols,
                                           const double (&acc)[4][4]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = 4 * ty + a;
    if (r >= rows) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = 4 * tx + b;
      if (c >= cols) continue;
      double* p = C + (int64_t)r * ld + c;
      *p = SUB ? (*p - acc[a][b]) : acc[a][b];
    }
  }
}

// Diagonal block: L_kk = chol(A_kk) and Dinv = L_kk^{-1}, by 256 threads;
// thread (r = t % 64, q = t / 64) holds columns 16q..16q+15 of row r.
__global__ __launch_bounds__(256) void fac_diag_kernel(double* __restrict__ A,
                                                       double* __restrict__ M,
                                                       double* __restrict__ Dinv, int d, int k,
                                                       int32_t* status) {
  if (*status != 0) return;
  __shared__ double xs[NB];
  __shared__ double mrow[NB];
  __shared__ double piv_s;
  __shared__ double tile[NB][LDP];
  const int t = threadIdx.x, r = t & 63, q = t >> 6;
  const int k0 = k * NB;
  const int kb = min(NB, d - k0);
  for (int e = t; e < NB * NB; e += 256) {
    const int rr = e >> 6, cc = e & 63;
    double v;
    if (rr < kb && cc < kb)
      v = (cc <= rr) ? A[(int64_t)(k0 + rr) * d + k0 + cc] : 0.0;
    else
      v = (rr == cc) ? 1.0 : 0.0;
    tile[rr][cc] = v;
  }
  __syncthreads();
  double a[16], b[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = tile[r][16 * q + i];
    b[i] = (r == 16 * q + i) ? 1.0 : 0.0;
  }
  bool failed = false;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int qc = c >> 4, ic = c & 15;
    if (q == qc && r == c) piv_s = a[ic];
    __syncthreads();
    const double piv = piv_s;
    if (failed) continue;
    if (!(piv > 0.0) || !(piv < 1.0e300)) {  // non-positive, NaN or Inf pivot
      failed = true;
      if (t == 0) *status = d - (k0 + c);
      continue;
    }
    const double lc = sqrt(piv);
    const double inv = 1.0 / lc;
    if (q == qc) {
      const double x = (r > c) ? a[ic] * inv : (r == c ? lc : 0.0);
      a[ic] = x;
      xs[r] = x;
    }
    if (r == c) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        b[i] *= inv;
        mrow[16 * q + i] = b[i];
      }
    }
    __syncthreads();
    if (r > c) {
      const double xr = xs[r];
      if (q >= qc) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * q + i > c) a[i] = fma(-xr, xs[16 * q + i], a[i]);
      }
      if (q <= qc) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * q + i <= c) b[i] = fma(-xr, mrow[16 * q + i], b[i]);
      }
    }
  }
  if (failed) return;
  // write L_kk (lower), Dinv (full 64 x 64, zero above the diagonal) and M_kk
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 16 * q + i;
    const double lv = (c <= r) ? a[i] : 0.0;
    const double mv = (c <= r) ? b[i] : 0.0;
    Dinv[r * NB + c] = mv;
    if (r < kb && c < kb) {
      if (c <= r) A[(int64_t)(k0 + r) * d + k0 + c] = lv;
      M[(int64_t)(k0 + r) * d + k0 + c] = mv;  // zero above the diagonal
    }
  }
}

// Panel: L_ik = A_ik Dinv^T for row blocks i > k; M_kj = Dinv B_kj for column blocks j < k.
__global__ __launch_bounds__(256) void fac_panel_kernel(double* __restrict__ A,
                                                        double* __restrict__ M,
                                                        const double* __restrict__ Dinv, int d,
                                                        int k, int nrow, const int32_t* status) {
  if (*status != 0) return;
  __shared__ TileLds s;
  const int k0 = k * NB, kb = min(NB, d - k0);
  double acc[4][4] = {};
  const int wg = blockIdx.x;
  if (wg < nrow) {
    const int i0 = (k + 1 + wg) * NB, ib = min(NB, d - i0);
    double* Aik = A + (int64_t)i0 * d + k0;
    load_T(s.p, Aik, d, ib, kb);
    load_T(s.q, Dinv, NB, NB, NB);  // q[t][c] = Dinv[c][t]
    __syncthreads();
    tile_mma(s, acc);
    __syncthreads();
    store_tile<false>(Aik, d, ib, kb, acc);
  } else {
    const int j0 = (wg - nrow) * NB;  // full block, j < k
    double* Mkj = M + (int64_t)k0 * d + j0;
    load_T(s.p, Dinv, NB, NB, NB);  // p[t][r] = Dinv[r][t]
    load_N(s.q, Mkj, d, kb, NB);
    __syncthreads();
    tile_mma(s, acc);
    __syncthreads();
    store_tile<false>(Mkj, d, kb, NB, acc);
  }
}

// Trailing updates of both factorizations.
__global__ __launch_bounds__(256) void fac_update_kernel(double* __restrict__ A,
                                                         double* __restrict__ M, int d, int k,
                                                         int nb, const int32_t* status) {
  if (*status != 0) return;
  __shared__ TileLds s;
  const int k0 = k * NB, kb = min(NB, d - k0);
  const int T = nb - k - 1;
  const int ta = T * (T + 1) / 2;
  double acc[4][4] = {};
  const int wg = blockIdx.x;
  if (wg < ta) {
    int ii, jj;
    tri_coords(wg, ii, jj);
    const int i0 = (k + 1 + ii) * NB, j0 = (k + 1 + jj) * NB;
    const int ib = min(NB, d - i0), jb = min(NB, d - j0);
    load_T(s.p, A + (int64_t)i0 * d + k0, d, ib, kb);  // P = L_ik
    load_T(s.q, A + (int64_t)j0 * d + k0, d, jb, kb);  // q[t][c] = L_jk[c][t]
    __syncthreads();
    tile_mma(s, acc);
    store_tile<true>(A + (int64_t)i0 * d + j0, d, ib, jb, acc);
  } else {
    const int idx = wg - ta;
    const int ii = idx / (k + 1), j = idx % (k + 1);
    const int i0 = (k + 1 + ii) * NB, j0 = j * NB;
    const int ib = min(NB, d - i0), jb = min(NB, d - j0);
    load_T(s.p, A + (int64_t)i0 * d + k0, d, ib, kb);  // P = L_ik
    load_N(s.q, M + (int64_t)k0 * d + j0, d, kb, jb);  // Q = M_kj
    __syncthreads();
    tile_mma(s, acc);
    store_tile<true>(M + (int64_t)i0 * d + j0, d, ib, jb, acc);
  }
}

// U[i][j] = M[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const double* __restrict__ M,
                                                      float* __restrict__ U, int d) {
  const int64_t total = (int64_t)d * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / d), j = (int)(e % d);
    U[e] = (i <= j) ? (float)M[(int64_t)(d - 1 - i) * d + (d - 1 - j)] : 0.0f;
  }
}

}  // namespace

size_t prepare_workspace(int64_t d) {
  return 2 * align256((size_t)d * d * sizeof(double)) + align256(NB * NB * sizeof(double)) + 256;
}

hipError_t prepare_launch(float* H, int64_t d64, double damp, float* U, uint8_t* dead,
                          int32_t* dev_status, void* ws, hipStream_t stream) {
  const int d = (int)d64;
  PrepWs w = carve(ws, d64);
  hipLaunchKernelGGL(prep_stats_kernel, dim3(1), dim3(1024), 0, stream, H, d, damp, dead, w.scal,
                     dev_status);
  const int nt32 = (int)ceil_div(d, 32);
  hipLaunchKernelGGL(prep_build_kernel, dim3(nt32 * (nt32 + 1) / 2), dim3(256), 0, stream, H, d,
                     (const double*)w.scal, w.A, w.M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (int)ceil_div(d, NB);
  for (int k = 0; k < nb; ++k) {
    hipLaunchKernelGGL(fac_diag_kernel, dim3(1), dim3(256), 0, stream, w.A, w.M, w.Dinv, d, k,
                       dev_status);
    const int nrow = nb - k - 1;
    if (nrow + k > 0)
      hipLaunchKernelGGL(fac_panel_kernel, dim3(nrow + k), dim3(256), 0, stream, w.A, w.M,
                         (const double*)w.Dinv, d, k, nrow, (const int32_t*)dev_status);
    const int T = nb - k - 1;
    const int tiles = T * (T + 1) / 2 + T * (k + 1);
    if (tiles > 0)
      hipLaunchKernelGGL(fac_update_kernel, dim3(tiles), dim3(256), 0, stream, w.A, w.M, d, k, nb,
                         (const int32_t*)dev_status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = (int64_t)d * d;
  const int grid = (int)std::min<int64_t>(ceil_div(total, 256), 65536);
  hipLaunchKernelGGL(write_u_kernel, dim3(grid), dim3(256), 0, stream, (const double*)w.M, U, d);
  return hipGetLastError();
}

}  // namespace gptq
