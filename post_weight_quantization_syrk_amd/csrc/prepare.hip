// Damping, Cholesky and the upper factor of the inverse Hessian
// ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段一: H ~ 2X^T X + lambda I and a
// Cholesky factorization whose triangular factor drives the error feedback).
//
// U is the upper triangular matrix with U^T U = H^{-1}.  Rather than inverting H
// and factorizing again, it is formed as U = V^{-1} with H = V V^T, V upper: in
// the index-reversed space A = J H J (J reverses the order) this is an ordinary
// Cholesky A = L L^T and a triangular inverse M = L^{-1}, and U = J M J.  Both
// run blocked (64 x 64 blocks) in fp32, right-looking, fused per step:
//   diag   : L_kk = chol(A_kk) and its inverse, one workgroup;
//   panel  : L_ik = A_ik L_kk^{-T} (i > k) and M_kj = L_kk^{-1} B_kj (j < k);
//   update : A_ij -= L_ik L_jk^T (i >= j > k) and B_ij -= L_ik M_kj (i > k >= j),
// where B accumulates the right-hand side of L M = I.  Panel and update tiles
// are fp32 MFMA products (v_mfma_f32_32x32x2f32).
#include "common.h"
#include "kernels.h"
#include "mfma_f32.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int NB = 64;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrepWs {
  float* A;      // [d x d] reversed damped H, then L (lower)
  float* M;      // [d x d] right-hand side / L^{-1} (lower)
  float* Dinv;   // [NB x NB] inverse of the current diagonal block
  double* scal;  // [0] = lambda
};

PrepWs carve(void* ws, int64_t d) {
  char* p = (char*)ws;
  PrepWs w;
  const size_t mat = align256((size_t)d * d * sizeof(float));
  w.A = (float*)p;
  w.M = (float*)(p + mat);
  w.Dinv = (float*)(p + 2 * mat);
  w.scal = (double*)(p + 2 * mat + align256(NB * NB * sizeof(float)));
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

// Mirror the lower triangle of H into the upper one, damp the diagonal
// (lambda added in float64, stored rounded to fp32), and build A = J H J
// (lower triangle) and zero the lower triangle of M.
__global__ __launch_bounds__(256) void prep_build_kernel(float* __restrict__ H, int d,
                                                         const double* __restrict__ scal,
                                                         float* __restrict__ A,
                                                         float* __restrict__ M) {
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
      const float dv = (float)((v == 0.0f ? 1.0 : (double)v) + lam);
      H[(int64_t)i * d + i] = dv;
      A[ar * d + ac] = dv;
    } else {
      H[(int64_t)j * d + i] = v;
      A[ar * d + ac] = v;
    }
    M[ar * d + ac] = 0.0f;
  }
}

// Diagonal block: L_kk = chol(A_kk) and Dinv = L_kk^{-1} by 256 threads; thread
// (r = t % 64, wave q = t / 64) holds columns 16q..16q+15 of row r.  Column c of
// L below the diagonal and row c of L^{-1} are exchanged through LDS; all
// per-element conditions are folded into zeros so the loop has no divergent
// branches.
__global__ __launch_bounds__(256) void fac_diag_kernel(float* __restrict__ A,
                                                       float* __restrict__ M,
                                                       float* __restrict__ Dinv, int d, int k,
                                                       int32_t* status) {
  if (*status != 0) return;
  __shared__ float tile[NB][NB + 1];
  __shared__ float mtile[NB][NB + 1];
  // xs[c % 3]: column c of L strictly below the diagonal (zero elsewhere);
  // mrow[c % 2]: row c of L^{-1}; inv_s[c % 3]: 1 / L_cc.
  __shared__ __attribute__((aligned(16))) float xs[3][NB];
  __shared__ __attribute__((aligned(16))) float mrow[2][NB];
  __shared__ float inv_s[3];
  __shared__ int bad_s;
  const int t = threadIdx.x, r = t & 63;
  const int q = __builtin_amdgcn_readfirstlane(t >> 6);
  const int k0 = k * NB;
  const int kb = min(NB, d - k0);
  {
    // batched, unconditional loads (clamped addresses), masked afterwards
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + t, rr = e >> 6, cc = e & 63;
      const int r2 = rr < kb ? rr : kb - 1, c2 = cc < kb ? cc : kb - 1;
      v[u] = A[(int64_t)(k0 + r2) * d + k0 + c2];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + t, rr = e >> 6, cc = e & 63;
      tile[rr][cc] = (rr < kb && cc < kb) ? ((cc <= rr) ? v[u] : 0.0f) : (rr == cc ? 1.0f : 0.0f);
    }
  }
  __syncthreads();
  float a[16], b[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = tile[r][16 * q + i];
    b[i] = (r == 16 * q + i) ? 1.0f : 0.0f;
  }
  // Column c of L is formed by the wave that owns it, right after that wave has
  // applied step c-1's update, and published before the step's only barrier.
  // The update of L^{-1} by column c is applied one step late, just before the
  // row it completes is needed.
  auto make_col = [&](auto C) {
    constexpr int c = decltype(C)::value, ic = c & 15;
    float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[ic]), c));
    if (!(piv > 0.0f) || !(piv < 3.0e38f)) {  // non-positive, NaN or Inf pivot
      if (r == 0 && bad_s == 0) bad_s = c + 1;  // keep the first failure
      piv = 1.0f;
    }
    const float inv = __builtin_amdgcn_rsqf(piv);  // 1/sqrt, within 1 ulp
    const float lc = piv * inv;
    const float x = a[ic] * inv;
    xs[c % 3][r] = (r > c) ? x : 0.0f;
    a[ic] = (r > c) ? x : (r == c ? lc : 0.0f);
    if (r == 0) inv_s[c % 3] = inv;
  };
  if (t == 0) bad_s = 0;
  __syncthreads();
  if (q == 0) make_col(std::integral_constant<int, 0>{});
  __syncthreads();
  // A failed pivot is replaced by 1 so the loop runs on with finite values;
  // the first failure is reported after the loop.
  StaticFor<0, NB>::run([&](auto C) {
    constexpr int c = decltype(C)::value, qc = c >> 4;
    const float* xc = xs[c % 3];
    const float xr = xc[r];
    if (q >= qc) {
#pragma unroll
      for (int i = 0; i < 16; ++i) a[i] = fmaf(-xr, xc[16 * q + i], a[i]);
    }
    // Next column first: it is the only work on the step-to-step chain; the
    // inverse update below overlaps its LDS write and the barrier wait.
    if constexpr (c + 1 < NB) {
      if (q == ((c + 1) >> 4)) make_col(std::integral_constant<int, c + 1>{});
    }
    if constexpr (c > 0) {
      constexpr int qp = (c - 1) >> 4;
      const float xp = xs[(c - 1) % 3][r];
      const float* mp = mrow[(c - 1) % 2];
      if (q <= qp) {
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = fmaf(-xp, mp[16 * q + i], b[i]);
      }
    }
    if (r == c) {
      const float inv = inv_s[c % 3];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        b[i] *= inv;
        mrow[c % 2][16 * q + i] = b[i];
      }
    }
    __syncthreads();
  });
  if (bad_s != 0) {
    if (t == 0) *status = d - (k0 + bad_s - 1);
    return;
  }
  // Stage L and L^{-1} through LDS so the global stores are row-contiguous
  // (a thread's own 16 values all sit in one row: 64 rows per store
  // instruction otherwise).
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 16 * q + i;
    tile[r][c] = (c <= r) ? a[i] : 0.0f;
    mtile[r][c] = (c <= r) ? b[i] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rr = 16 * u + (t >> 4), c0 = 4 * (t & 15);
    float lv[4], mv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lv[e] = tile[rr][c0 + e];
      mv[e] = mtile[rr][c0 + e];
    }
    *(float4*)(Dinv + rr * NB + c0) = make_float4(mv[0], mv[1], mv[2], mv[3]);
    if (rr < kb) {
      float* arow = A + (int64_t)(k0 + rr) * d + k0;
      float* mrow_g = M + (int64_t)(k0 + rr) * d + k0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + e;
        if (c < kb) {
          if (c <= rr) arow[c] = lv[e];
          mrow_g[c] = mv[e];  // zero above the diagonal
        }
      }
    }
  }
}

using TileT = MfmaTile<NB, NB, NB, true>;   // C = P Q with Q given transposed
using TileN = MfmaTile<NB, NB, NB, false>;  // C = P Q with Q row-major
constexpr size_t TILE_LDS = (TileT::lds_floats > TileN::lds_floats ? TileT::lds_floats
                                                                     : TileN::lds_floats);

template <class Tile, bool SUB>
__device__ __forceinline__ void tile_store(float* C, int64_t ld, int rows, int cols,
                                           const f32x16 (&acc)[Tile::FM][Tile::FN]) {
  Tile::template store<SUB>(C, ld, rows, cols, acc);
}

// Panel: L_ik = A_ik Dinv^T for row blocks i > k; M_kj = Dinv B_kj for column blocks j < k.
__global__ __launch_bounds__(256) void fac_panel_kernel(float* __restrict__ A,
                                                        float* __restrict__ M,
                                                        const float* __restrict__ Dinv, int d,
                                                        int k, int nrow, const int32_t* status) {
  if (*status != 0) return;
  __shared__ __attribute__((aligned(16))) float lds[TILE_LDS];
  const int k0 = k * NB, kb = min(NB, d - k0);
  const int wg = blockIdx.x;
  if (wg < nrow) {
    const int i0 = (k + 1 + wg) * NB, ib = min(NB, d - i0);
    float* Aik = A + (int64_t)i0 * d + k0;
    f32x16 acc[TileT::FM][TileT::FN];
    TileT::zero(acc);
    TileT::load_p(lds, Aik, d, ib, kb);
    TileT::load_q(lds, Dinv, NB, NB, NB);  // Q^T = Dinv
    __syncthreads();
    TileT::mma(lds, acc);
    tile_store<TileT, false>(Aik, d, ib, kb, acc);
  } else {
    const int j0 = (wg - nrow) * NB;  // full block, j < k
    float* Mkj = M + (int64_t)k0 * d + j0;
    f32x16 acc[TileN::FM][TileN::FN];
    TileN::zero(acc);
    TileN::load_p(lds, Dinv, NB, NB, NB);
    TileN::load_q(lds, Mkj, d, kb, NB);
    __syncthreads();
    TileN::mma(lds, acc);
    __syncthreads();
    tile_store<TileN, false>(Mkj, d, kb, NB, acc);
  }
}

// Trailing updates of both factorizations.
__global__ __launch_bounds__(256) void fac_update_kernel(float* __restrict__ A,
                                                         float* __restrict__ M, int d, int k,
                                                         int nb, const int32_t* status) {
  if (*status != 0) return;
  __shared__ __attribute__((aligned(16))) float lds[TILE_LDS];
  const int k0 = k * NB, kb = min(NB, d - k0);
  const int T = nb - k - 1;
  const int ta = T * (T + 1) / 2;
  const int wg = blockIdx.x;
  if (wg < ta) {
    int ii, jj;
    tri_coords(wg, ii, jj);
    const int i0 = (k + 1 + ii) * NB, j0 = (k + 1 + jj) * NB;
    const int ib = min(NB, d - i0), jb = min(NB, d - j0);
    f32x16 acc[TileT::FM][TileT::FN];
    TileT::zero(acc);
    TileT::load_p(lds, A + (int64_t)i0 * d + k0, d, ib, kb);  // P = L_ik
    TileT::load_q(lds, A + (int64_t)j0 * d + k0, d, jb, kb);  // Q^T = L_jk
    __syncthreads();
    TileT::mma(lds, acc);
    tile_store<TileT, true>(A + (int64_t)i0 * d + j0, d, ib, jb, acc);
  } else {
    const int idx = wg - ta;
    const int ii = idx / (k + 1), j = idx % (k + 1);
    const int i0 = (k + 1 + ii) * NB, j0 = j * NB;
    const int ib = min(NB, d - i0), jb = min(NB, d - j0);
    f32x16 acc[TileN::FM][TileN::FN];
    TileN::zero(acc);
    TileN::load_p(lds, A + (int64_t)i0 * d + k0, d, ib, kb);  // P = L_ik
    TileN::load_q(lds, M + (int64_t)k0 * d + j0, d, kb, jb);  // Q = M_kj
    __syncthreads();
    TileN::mma(lds, acc);
    tile_store<TileN, true>(M + (int64_t)i0 * d + j0, d, ib, jb, acc);
  }
}

// U[i][j] = M[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const float* __restrict__ M,
                                                      float* __restrict__ U, int d) {
  const int64_t total = (int64_t)d * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / d), j = (int)(e % d);
    U[e] = (i <= j) ? M[(int64_t)(d - 1 - i) * d + (d - 1 - j)] : 0.0f;
  }
}

}  // namespace

size_t prepare_workspace(int64_t d) {
  return 2 * align256((size_t)d * d * sizeof(float)) + align256(NB * NB * sizeof(float)) + 256;
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
                         (const float*)w.Dinv, d, k, nrow, (const int32_t*)dev_status);
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
  hipLaunchKernelGGL(write_u_kernel, dim3(grid), dim3(256), 0, stream, (const float*)w.M, U, d);
  return hipGetLastError();
}

}  // namespace gptq
