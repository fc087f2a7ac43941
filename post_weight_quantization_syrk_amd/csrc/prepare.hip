// Damping, Cholesky and the upper factor of the inverse Hessian
// ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段一: H ~ 2X^T X + lambda I and a
// Cholesky factorization whose triangular factor drives the error feedback).
//
// U is the upper triangular matrix with U^T U = H^{-1}.  Rather than inverting H
// and factorizing again, it is formed as U = V^{-1} with H = V V^T, V upper: in
// the index-reversed space A = J H J (J reverses the order) this is an ordinary
// Cholesky A = L L^T and a triangular inverse M = L^{-1}, and U = J M J.  Both
// run blocked (64 x 64 blocks) in fp32, right-looking, per step k:
//   diag   : L_kk = chol(A_kk) and its inverse, one workgroup;
//   panel  : L_ik = A_ik L_kk^{-T} (i > k) and M_kj = L_kk^{-1} B_kj (j < k);
//   update : A_ij -= L_ik L_jk^T (i >= j > k) and B_ij -= L_ik M_kj (i > k >= j),
// where B accumulates the right-hand side of L M = I.  Steps go in groups of
// UG: inside a group only the next block column (and block row of B) is
// brought up to date before each step (fac_colupd_kernel, which also applies
// the previous step's panel), and after the group the trailing part receives
// the group's panels in two pieces: the band the next group's steps read
// (fac_update_kernel, whose workgroup on the next diagonal block factorizes it
// in the same launch), and the rest through extra workgroups of the next
// group's column-update launches, which by themselves leave most of the chip
// idle.
// Panel and update tiles are fp32 MFMA products (v_mfma_f32_32x32x2f32).
#include "common.h"
#include "kernels.h"
#include "mfma_f32.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int NB = 64;
constexpr int UG = 4;   // steps per delayed trailing update

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrepWs {
  float* A;      // [d x d] reversed damped H, then L (lower)
  float* M;      // [d x d] right-hand side / L^{-1} (lower)
  float* Dinv[2];  // [NB x NB] inverse of the diagonal block of step k, in Dinv[k % 2]
  double* scal;  // [0] = lambda
};

PrepWs carve(void* ws, int64_t d) {
  char* p = (char*)ws;
  PrepWs w;
  const size_t mat = align256((size_t)d * d * sizeof(float));
  w.A = (float*)p;
  w.M = (float*)(p + mat);
  w.Dinv[0] = (float*)(p + 2 * mat);
  w.Dinv[1] = (float*)(p + 2 * mat + align256(NB * NB * sizeof(float)));
  w.scal = (double*)(p + 2 * mat + 2 * align256(NB * NB * sizeof(float)));
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

// Column order ([P1] GPTQ 的高级技巧, 激活排序): the factorization is of the
// permuted matrix H[perm][:, perm], i.e. A[a][b] = H[perm[d-1-a]][perm[d-1-b]]
// on A's lower triangle, gathered from H after prep_build_kernel has mirrored
// and damped it (so the values are the ones the natural order would use).
// perm entries are clamped to [0, d).
__global__ __launch_bounds__(256) void prep_perm_kernel(const float* __restrict__ H, int d,
                                                        const int32_t* __restrict__ perm,
                                                        float* __restrict__ A) {
  // grid: x over columns b, y over rows a (strided)
  const int b = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (b >= d) return;
  const int q = min(max(perm[d - 1 - b], 0), d - 1);
  const int G = (int)gridDim.y;
  int a0 = (int)blockIdx.y;  // rows a0, a0 + G, ...: the first one >= b
  if (a0 < b) a0 += ((b - a0 + G - 1) / G) * G;
  for (int a = a0; a < d; a += G) {
    const int p = min(max(perm[d - 1 - a], 0), d - 1);
    A[(int64_t)a * d + b] = H[(int64_t)p * d + q];
  }
}

// Diagonal block: L_kk = chol(A_kk) and Dinv = L_kk^{-1}, by 256 threads in
// four 16-column sub-steps S = [s0, s0 + 16), s0 = 16 s:
//   A: wave 0 factors the 16 x 16 block A_SS in registers and inverts it.
//      Lane (g, r) (16-lane row g, lane r of the row) holds row r of the
//      symmetric Schur complement and columns 4g .. 4g+3 of row r of the
//      inverse; pivot and column values are broadcast with DPP row
//      broadcasts, so the 16 dependent pivot steps need no barrier and no
//      scalar registers.  The four row groups repeat the factorization and
//      share the inverse.
//      Meanwhile waves 1-3 form R = L_{S,0:s0} M_{0:s0,0:s0}, which the rows
//      of L^{-1} below need;
//   B: the panel L_{i,S} = A_{i,S} M_SS^T for rows i below S, and the row
//      block M_{S,0:s0} = -M_SS R of L^{-1};
//   C: the rank-16 update A_{i,j} -= L_{i,S} L_{j,S}^T of the rows below S.
// The upper triangles of the LDS copies of L and L^{-1} hold zeros, so the
// triangular products run over full index ranges without per-lane branches.
// A pivot that is not positive and finite turns its diagonal entry of L into
// NaN or 0 and every later pivot into NaN; the first diagonal entry of L that
// is not positive and finite is the first failed pivot, and is reported.
constexpr int SB = 16;
constexpr int PP16 = 20;  // LDS pitch (floats) of the 16-wide panel copy: 16-byte rows

struct DiagLds {
  float tile[NB][NB + 1];   // A_kk, becomes L_kk (lower)
  float mtile[NB][NB + 1];  // L_kk^{-1} (lower)
  float rbuf[SB][NB + 1];   // R of the current sub-step
  alignas(16) float pan[NB][PP16];  // panel copy L_{i,S}
};
constexpr size_t DIAG_LDS_FLOATS = (sizeof(DiagLds) + 3) / 4;

// LDS copy of the diagonal block entry (rr, cc) from its value v: lower
// triangle, identity past the matrix edge (kb = valid rows/columns).
__device__ __forceinline__ float diag_entry(int rr, int cc, int kb, float v) {
  return (rr < kb && cc < kb) ? ((cc <= rr) ? v : 0.0f) : (rr == cc ? 1.0f : 0.0f);
}

// A_kk from global memory into the LDS copies (batched, unconditional loads
// from clamped addresses, masked afterwards); L^{-1} starts at zero.
__device__ __forceinline__ void diag_load(DiagLds& L, const float* __restrict__ A, int d, int k) {
  const int t = threadIdx.x;
  const int k0 = k * NB;
  const int kb = min(NB, d - k0);
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
    L.tile[rr][cc] = diag_entry(rr, cc, kb, v[u]);
    L.mtile[rr][cc] = 0.0f;
  }
}

// The factorization proper, from the LDS copies (filled and published by a
// barrier); writes L_kk and L_kk^{-1} to A and M and L_kk^{-1} to Dinv.
__device__ __forceinline__ void diag_factor(DiagLds& L, float* __restrict__ A,
                                            float* __restrict__ M, float* __restrict__ Dinv,
                                            int d, int k, int32_t* status) {
  auto& tile = L.tile;
  auto& mtile = L.mtile;
  auto& rbuf = L.rbuf;
  auto& pan = L.pan;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int k0 = k * NB;
  const int kb = min(NB, d - k0);
  // Per-lane masks of the in-register factorization (row r = lane % 16):
  // ngt[c] = -1 below pivot c, else 0; eqf[c] = 1 on the pivot row.
  const int r = lane & (SB - 1), grp = lane >> 4;
  float ngt[SB], eqf[SB];
#pragma unroll
  for (int c = 0; c < SB; ++c) {
    ngt[c] = (r > c) ? -1.0f : 0.0f;
    eqf[c] = (r == c) ? 1.0f : 0.0f;
  }

  StaticFor<0, NB / SB>::run([&](auto Sv) {
    constexpr int s = decltype(Sv)::value, s0 = SB * s;
    constexpr int rows = NB - s0 - SB;  // rows below the sub-block
    // ---------------- A
    if (wave == 0) {
      // a[j]: row r of the symmetric Schur complement of A_SS (both halves,
      // so no lane ever holds values that are not bounded by the matrix's).
      // mv[q]: row r of the partially eliminated identity, columns 4 grp + q;
      // row c of L_SS^{-1} is mv of lane c times 1 / L_cc.
      float a[SB], mv[4];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        a[j] = (j <= r) ? tile[s0 + r][s0 + j] : tile[s0 + j][s0 + r];
#pragma unroll
      for (int q = 0; q < 4; ++q) mv[q] = eqf[4 * grp + q];
      float myinv = 0.0f;
      StaticFor<0, SB>::run([&](auto Cv) {
        constexpr int c = decltype(Cv)::value;
        const float inv = __builtin_amdgcn_rsqf(row_bcast<c>(a[c]));  // 1/sqrt, within 1 ulp
        const float l = a[c] * inv;  // L[r][c] below the pivot, L[c][c] on it
        a[c] = l;
        const float nl = l * ngt[c];  // -L[r][c] below the pivot, 0 elsewhere
        StaticFor<c + 1, SB>::run([&](auto Jv) {
          constexpr int j = decltype(Jv)::value;
          a[j] = fmaf(row_bcast<j>(l), nl, a[j]);
        });
        const float nlm = nl * inv;  // -L[r][c] / L[c][c]
#pragma unroll
        for (int q = 0; q < 4; ++q) mv[q] = fmaf(row_bcast<c>(mv[q]), nlm, mv[q]);
        myinv = fmaf(inv, eqf[c], myinv);
      });
      if (grp == 0) {
#pragma unroll
        for (int j = 0; j < SB; ++j) tile[s0 + r][s0 + j] = (j <= r) ? a[j] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) mtile[s0 + r][s0 + 4 * grp + q] = mv[q] * myinv;
    } else if constexpr (s > 0) {
      // R[r][c] = sum_{m<s0} L[s0+r][m] M[m][c] (M[m][c] = 0 for m < c):
      // thread (c, 4 rows)
      const int e = t - 64;
      if (e < 4 * s0) {
        const int c = e % s0, r0 = 4 * (e / s0);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mm = 0; mm < s0; ++mm) {
          const float mvv = mtile[mm][c];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(tile[s0 + r0 + i][mm], mvv, acc[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) rbuf[r0 + i][c] = acc[i];
      }
      // The deferred part of the previous sub-step's rank-16 update: rows
      // i >= s0 + 16, columns s0 <= j <= i (its block-s part ran before this
      // sub-step).  pan still holds the previous sub-step's panel.  Nothing
      // here touches block s, which wave 0 is factoring.
      constexpr int drows = NB - s0 - SB, dcols = NB - s0;
      if constexpr (drows > 0) {
        for (int q = e; q < drows * dcols; q += 192) {
          const int i = s0 + SB + q / dcols, jj = s0 + q % dcols;
          if (jj <= i) {
            const float4* pi = (const float4*)pan[i];
            const float4* pj = (const float4*)pan[jj];
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < SB / 4; ++u) {
              const float4 x = pi[u], y = pj[u];
              acc = fmaf(x.x, y.x, acc);
              acc = fmaf(x.y, y.y, acc);
              acc = fmaf(x.z, y.z, acc);
              acc = fmaf(x.w, y.w, acc);
            }
            tile[i][jj] -= acc;
          }
        }
      }
    }
    __syncthreads();
    // ---------------- B
    // Threads [0, 4 rows): panel row i, columns 4jg..4jg+3:
    //   L[i][s0+j] = sum_q A[i][s0+q] M_SS[j][q]   (M_SS[j][q] = 0 for q > j).
    // Threads [4 rows, 4 rows + 4 s0): row block of L^{-1}, column c, rows
    //   4g..4g+3:  M[s0+r][c] = -sum_p M_SS[r][p] R[p][c]   (M_SS[r][p] = 0 for p > r).
    // A panel row is read and written only by its own four threads, which
    // are lanes of one wave (their reads all precede their writes), and the
    // L^{-1} row block writes columns < s0, which nobody reads here: one
    // barrier at the end suffices.
    if (t < 4 * rows) {
      const int i = s0 + SB + (t >> 2), j0 = 4 * (t & 3);
      float pv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const float av = tile[i][s0 + q];
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = fmaf(av, mtile[s0 + j0 + u][s0 + q], pv[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        tile[i][s0 + j0 + u] = pv[u];
        pan[i][j0 + u] = pv[u];
      }
    }
    if constexpr (s > 0) {
      if (t >= 4 * rows && t < 4 * rows + 4 * s0) {
        const int e = t - 4 * rows;
        const int c = e % s0, g0 = 4 * (e / s0);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < SB; ++p) {
          const float rv = rbuf[p][c];
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = fmaf(mtile[s0 + g0 + u][s0 + p], rv, acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) mtile[s0 + g0 + u][c] = -acc[u];
      }
    }
    __syncthreads();
    // ---------------- C
    // The rank-16 update A_{i,j} -= L_{i,S} L_{j,S}^T on the next diagonal
    // block only (rows and columns s0+16 .. s0+31, one element per thread):
    // that is all the next sub-step's pivots need.  The rest of the update
    // (rows below it) runs on waves 1-3 while wave 0 factors that block.
    if constexpr (rows > 0) {
      {
        const int e = t;
        const int i = s0 + SB + (e >> 4), jj = s0 + SB + (e & 15);
        if (jj <= i) {
          const float4* pi = (const float4*)pan[i];
          const float4* pj = (const float4*)pan[jj];
          float acc = 0.0f;
#pragma unroll
          for (int q = 0; q < SB / 4; ++q) {
            const float4 x = pi[q], y = pj[q];
            acc = fmaf(x.x, y.x, acc);
            acc = fmaf(x.y, y.y, acc);
            acc = fmaf(x.z, y.z, acc);
            acc = fmaf(x.w, y.w, acc);
          }
          tile[i][jj] -= acc;
        }
      }
      __syncthreads();
    }
  });
  {
    // First failed pivot: the first diagonal entry of L that is not positive
    // and finite (every wave takes the same decision).
    const float dg = tile[lane][lane];
    const uint64_t badm = __ballot(!(dg > 0.0f && dg < INFINITY));
    if (badm != 0) {
      if (t == 0) *status = d - (k0 + __ffsll((unsigned long long)badm) - 1);
      return;
    }
  }
  // Global stores, row-contiguous (16 threads per 64-float row).  The upper
  // triangles of both LDS copies are zero, so whole rows are written.
  const bool vec = (kb == NB) && (d % 4 == 0);
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
    float* arow = A + (int64_t)(k0 + rr) * d + k0;
    float* mrow_g = M + (int64_t)(k0 + rr) * d + k0;
    if (vec) {
      *(float4*)(arow + c0) = make_float4(lv[0], lv[1], lv[2], lv[3]);
      *(float4*)(mrow_g + c0) = make_float4(mv[0], mv[1], mv[2], mv[3]);
    } else if (rr < kb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + e;
        if (c < kb) {
          arow[c] = lv[e];
          mrow_g[c] = mv[e];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void fac_diag_kernel(float* __restrict__ A,
                                                       float* __restrict__ M,
                                                       float* __restrict__ Dinv, int d, int k,
                                                       int32_t* status) {
  if (*status != 0) return;
  __shared__ DiagLds L;
  diag_load(L, A, d, k);
  __syncthreads();
  diag_factor(L, A, M, Dinv, d, k, status);
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

// After a group of steps [mlo, mhi) (delayed, grouped updates: the trailing
// matrix is read and written once per group of steps instead of once per
// step), both factorizations receive the group's panels:
//   L tiles  A_ij -= sum_m L_im L_jm^T   (i >= j >= mhi)
//   M tiles  B_ij -= sum_m L_im M_mj     (i >= mhi, j < mhi; only m >= j
//                                         contributes: M is lower)
// Each step m is one K = 64 chunk through LDS, accumulated in registers.
// One output tile (block bi, bj) per call; with diag (tile (mhi, mhi) only)
// the updated block goes from its accumulators straight into the diagonal
// factorization's LDS copies and is factorized into Dinv instead of stored.
__device__ __forceinline__ void update_tile(float* __restrict__ A, float* __restrict__ M,
                                            float* __restrict__ Dinv, float* lds, int d,
                                            int mlo, int mhi, bool ltile, int bi, int bj,
                                            bool diag, int32_t* status) {
  const int i0 = bi * NB, j0 = bj * NB;
  const int ib = min(NB, d - i0), jb = min(NB, d - j0);
  // The output tile is loaded into the accumulators and the products
  // accumulate onto it with P negated on its way into LDS; step m+1's
  // operands are loaded while step m multiplies.
  if (ltile) {
    float* C = A + (int64_t)i0 * d + j0;
    f32x16 acc[TileT::FM][TileT::FN];
    TileT::set_each(acc, [&](int row, int col) {
      return C[(int64_t)(row < ib ? row : ib - 1) * d + (col < jb ? col : jb - 1)];
    });
    TileT::PQRegs v;
    auto fetch = [&](int m) __attribute__((always_inline)) {
      const int m0 = m * NB, mb = min(NB, d - m0);
      TileT::fetch_pq(v, A + (int64_t)i0 * d + m0, d, ib, mb,   // P = L_im
                      A + (int64_t)j0 * d + m0, d, jb, mb);     // Q^T = L_jm
    };
    fetch(mlo);
    for (int m = mlo; m < mhi; ++m) {
      const int mb = min(NB, d - m * NB);
      if (m > mlo) __syncthreads();
      TileT::stage_pq<true>(lds, v, ib, mb, jb, mb);
      __syncthreads();
      if (m + 1 < mhi) fetch(m + 1);
      TileT::mma(lds, acc);
    }
    if (diag) {
      DiagLds& L = *reinterpret_cast<DiagLds*>(lds);
      __syncthreads();  // every wave is done with the product's LDS operands
      TileT::for_each(acc, [&](int row, int col, float val) {
        L.tile[row][col] = diag_entry(row, col, ib, val);
      });
      for (int e = threadIdx.x; e < NB * (NB + 1); e += 256) (&L.mtile[0][0])[e] = 0.0f;
      __syncthreads();
      diag_factor(L, A, M, Dinv, d, bi, status);
      return;
    }
    tile_store<TileT, false>(C, d, ib, jb, acc);
  } else {
    const int ms = max(mlo, bj);
    if (ms >= mhi) return;
    float* C = M + (int64_t)i0 * d + j0;
    f32x16 acc[TileN::FM][TileN::FN];
    TileN::set_each(acc, [&](int row, int col) {
      return C[(int64_t)(row < ib ? row : ib - 1) * d + (col < jb ? col : jb - 1)];
    });
    TileN::PQRegs v;
    auto fetch = [&](int m) __attribute__((always_inline)) {
      const int m0 = m * NB, mb = min(NB, d - m0);
      TileN::fetch_pq(v, A + (int64_t)i0 * d + m0, d, ib, mb,   // P = L_im
                      M + (int64_t)m0 * d + j0, d, mb, jb);     // Q = M_mj
    };
    fetch(ms);
    for (int m = ms; m < mhi; ++m) {
      const int mb = min(NB, d - m * NB);
      if (m > ms) __syncthreads();
      TileN::stage_pq<true>(lds, v, ib, mb, mb, jb);
      __syncthreads();
      if (m + 1 < mhi) fetch(m + 1);
      TileN::mma(lds, acc);
    }
    tile_store<TileN, false>(C, d, ib, jb, acc);
  }
}

// The tiles a group's update touches split in two.  The band -- L block
// columns [mhi, mhi + UG) and B block rows [mhi, mhi + UG), what the next
// group's steps read -- is updated right after the group (fac_update_kernel).
// The rest -- L block columns and B block rows from mhi + UG on -- is read by
// nothing until the next group's own update, and is updated meanwhile by
// extra workgroups of the next group's column-update launches, on the compute
// units those latency-bound launches leave idle.  The two sets are disjoint
// from each other and from everything the next group's column updates and
// panel read or write.
__host__ __device__ inline int band_ltiles(int nb, int c0, int c1) {
  return (c1 - c0) * nb - (c0 + c1 - 1) * (c1 - c0) / 2;
}
__host__ __device__ inline int band_tiles(int nb, int mhi) {
  const int c1 = min(nb, mhi + UG);
  return band_ltiles(nb, mhi, c1) + (c1 - mhi) * mhi;
}
__host__ __device__ inline int rest_tiles(int nb, int mhi) {
  const int T = nb - (mhi + UG);
  return T > 0 ? T * (T + 1) / 2 + T * mhi : 0;
}

// Band tile t: L tiles column by column from (mhi, mhi) down, then the B
// tiles row by row.  Workgroup 0 (tile (mhi, mhi)) also factorizes the next
// diagonal block into Dinv: it touches only block (mhi, mhi) of A and M and
// Dinv, which no other tile of this launch reads.
__global__ __launch_bounds__(256) void fac_update_kernel(float* __restrict__ A,
                                                         float* __restrict__ M,
                                                         float* __restrict__ Dinv, int d, int nb,
                                                         int mlo, int mhi, int32_t* status) {
  if (*status != 0) return;
  constexpr size_t LDS_FLOATS = TILE_LDS > DIAG_LDS_FLOATS ? TILE_LDS : DIAG_LDS_FLOATS;
  __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
  const int c1 = min(nb, mhi + UG);
  int t = blockIdx.x;
  const int nl = band_ltiles(nb, mhi, c1);
  if (t < nl) {
    int bj = mhi;
    while (t >= nb - bj) {
      t -= nb - bj;
      ++bj;
    }
    update_tile(A, M, Dinv, lds, d, mlo, mhi, true, bj + t, bj, blockIdx.x == 0, status);
  } else {
    t -= nl;
    update_tile(A, M, Dinv, lds, d, mlo, mhi, false, mhi + t / mhi, t % mhi, false, status);
  }
}

// Rest tile t of the group [mhi - UG, mhi): the L triangle from block mhi + UG
// row by row, then the B tiles row by row.
__device__ __forceinline__ void rest_tile(float* __restrict__ A, float* __restrict__ M,
                                          float* lds, int d, int nb, int mhi, int t,
                                          int32_t* status) {
  const int c0 = mhi + UG, T = nb - c0, ta = T * (T + 1) / 2;
  if (t < ta) {
    int ii, jj;
    tri_coords(t, ii, jj);
    update_tile(A, M, nullptr, lds, d, mhi - UG, mhi, true, c0 + ii, c0 + jj, false, status);
  } else {
    t -= ta;
    update_tile(A, M, nullptr, lds, d, mhi - UG, mhi, false, c0 + t / mhi, t % mhi, false,
                status);
  }
}

// Part 1 of step kc (g0 < kc < group end) with step p = kc - 1's panel folded
// in, so no panel launch sits between the two diagonal factorizations:
//   L tile (i, kc), i >= kc:  P_i = A_ip Dinv_p^T (stored: the panel block
//     L_ip) and P_k = A_kc,p Dinv_p^T (recomputed by every workgroup), then
//     A_i,kc -= sum_{m in [g0, p)} L_im L_kc,m^T + P_i P_k^T;
//   B tile (kc, j), j < kc:   for j < p, M_pj = Dinv_p B_pj (stored: the
//     panel's block of L^{-1}); M_pp = Dinv_p; then
//     B_kc,j -= sum_{m in [max(g0, j), p)} L_kc,m M_mj + P_k M_pj.
// The output tile is preloaded into the accumulators and the products
// accumulate onto it with P negated.  Workgroup 0 (tile (kc, kc)) then
// factorizes the diagonal block, as in fac_update_kernel, into Dinv_out (the
// other buffer: the others read Dinv_p throughout).  Block p is never the
// last block, so it is a full one.
__global__ __launch_bounds__(256, 2) void fac_colupd_kernel(float* __restrict__ A,
                                                         float* __restrict__ M,
                                                         const float* __restrict__ Dinv,
                                                         float* __restrict__ Dinv_out, int d,
                                                         int nb, int g0, int kc, int rest_lo,
                                                         int32_t* status) {
  if (*status != 0) return;
  constexpr size_t LDS_FLOATS = TILE_LDS > DIAG_LDS_FLOATS ? TILE_LDS : DIAG_LDS_FLOATS;
  __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
  if ((int)blockIdx.x >= nb) {  // the previous group's rest tiles
    rest_tile(A, M, lds, d, nb, g0, rest_lo + (int)blockIdx.x - nb, status);
    return;
  }
  const int p = kc - 1, p0 = p * NB, kc0 = kc * NB;
  const int kcb = min(NB, d - kc0);
  const int wg = blockIdx.x, T = nb - kc;
  const float* Akp = A + (int64_t)kc0 * d + p0;
  // acc = (rows x 64 block at src) * Dinv_p^T
  auto panel_t = [&](f32x16 (&acc)[TileT::FM][TileT::FN], const float* src, int rows)
      __attribute__((always_inline)) {
    TileT::zero(acc);
    TileT::load_p(lds, src, d, rows, NB);
    TileT::load_q(lds, Dinv, NB, NB, NB);  // Q^T = Dinv_p
    __syncthreads();
    TileT::mma(lds, acc);
    __syncthreads();  // LDS free again
  };
  if (wg < T) {
    const int i = kc + wg, i0 = i * NB, ib = min(NB, d - i0);
    f32x16 pi[TileT::FM][TileT::FN], pk[TileT::FM][TileT::FN];
    panel_t(pi, A + (int64_t)i0 * d + p0, ib);
    if (wg == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pk[0][0][r] = pi[0][0][r];
    } else {
      panel_t(pk, Akp, kcb);
    }
    // L_ip, for the rows below kc (row kc's is used only here, and every
    // workgroup reads row kc's A_kc,p, so it stays as it is)
    if (wg != 0) tile_store<TileT, false>(A + (int64_t)i0 * d + p0, d, ib, NB, pi);
    float* C = A + (int64_t)i0 * d + kc0;
    f32x16 acc[TileT::FM][TileT::FN];
    TileT::set_each(acc, [&](int row, int col) {
      return C[(int64_t)(row < ib ? row : ib - 1) * d + (col < kcb ? col : kcb - 1)];
    });
    TileT::PQRegs v;
    auto fetch = [&](int m) __attribute__((always_inline)) {
      TileT::fetch_pq(v, A + (int64_t)i0 * d + m * NB, d, ib, NB,   // P = L_im
                      A + (int64_t)kc0 * d + m * NB, d, kcb, NB);   // Q^T = L_kc,m
    };
    if (g0 < p) fetch(g0);
    for (int m = g0; m < p; ++m) {
      if (m > g0) __syncthreads();
      TileT::stage_pq<true>(lds, v, ib, NB, kcb, NB);
      __syncthreads();
      if (m + 1 < p) fetch(m + 1);
      TileT::mma(lds, acc);
    }
    // step p from registers: P = -P_i, Q^T = P_k
    __syncthreads();
    TileT::for_each(pi, [&](int row, int col, float x) { lds[row * TileT::PP + col] = -x; });
    TileT::for_each(pk, [&](int row, int col, float x) {
      lds[TileT::lds_q_offset + row * TileT::QPITCH + col] = x;
    });
    __syncthreads();
    TileT::mma(lds, acc);
    if (wg == 0) {
      DiagLds& L = *reinterpret_cast<DiagLds*>(lds);
      __syncthreads();  // every wave is done with the product's LDS operands
      TileT::for_each(acc, [&](int row, int col, float val) {
        L.tile[row][col] = diag_entry(row, col, ib, val);
      });
      for (int e = threadIdx.x; e < NB * (NB + 1); e += 256) (&L.mtile[0][0])[e] = 0.0f;
      __syncthreads();
      diag_factor(L, A, M, Dinv_out, d, kc, status);
      return;
    }
    tile_store<TileT, false>(C, d, ib, kcb, acc);
  } else {
    const int j = wg - T, j0 = j * NB;  // full block, j < kc
    f32x16 mpj[TileN::FM][TileN::FN];
    if (j < p) {
      TileN::zero(mpj);
      TileN::load_p(lds, Dinv, NB, NB, NB);
      TileN::load_q(lds, M + (int64_t)p0 * d + j0, d, NB, NB);  // B_pj
      __syncthreads();
      TileN::mma(lds, mpj);
      __syncthreads();
      tile_store<TileN, false>(M + (int64_t)p0 * d + j0, d, NB, NB, mpj);  // M_pj
    }
    f32x16 pk[TileT::FM][TileT::FN];
    panel_t(pk, Akp, kcb);
    float* C = M + (int64_t)kc0 * d + j0;
    f32x16 acc[TileN::FM][TileN::FN];
    TileN::set_each(acc, [&](int row, int col) {
      return C[(int64_t)(row < kcb ? row : kcb - 1) * d + col];
    });
    const int ms = max(g0, j);
    TileN::PQRegs v;
    auto fetch = [&](int m) __attribute__((always_inline)) {
      TileN::fetch_pq(v, A + (int64_t)kc0 * d + m * NB, d, kcb, NB,   // P = L_kc,m
                      M + (int64_t)m * NB * d + j0, d, NB, NB);       // Q = M_mj
    };
    if (ms < p) fetch(ms);
    for (int m = ms; m < p; ++m) {
      if (m > ms) __syncthreads();
      TileN::stage_pq<true>(lds, v, kcb, NB, NB, NB);
      __syncthreads();
      if (m + 1 < p) fetch(m + 1);
      TileN::mma(lds, acc);
    }
    // step p: P = -P_k, Q = M_pj (Dinv_p itself when j = p)
    __syncthreads();
    TileT::for_each(pk, [&](int row, int col, float x) { lds[row * TileN::PP + col] = -x; });
    if (j < p) {
      TileN::for_each(mpj, [&](int row, int col, float x) {
        lds[TileN::lds_q_offset + row * TileN::QPITCH + col] = x;
      });
    } else {
      for (int e = threadIdx.x; e < NB * NB; e += 256)
        lds[TileN::lds_q_offset + (e / NB) * TileN::QPITCH + e % NB] = Dinv[e];
    }
    __syncthreads();
    TileN::mma(lds, acc);
    tile_store<TileN, false>(C, d, kcb, NB, acc);
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
  return 2 * align256((size_t)d * d * sizeof(float)) + 2 * align256(NB * NB * sizeof(float)) + 256;
}

hipError_t prepare_launch(float* H, int64_t d64, double damp, float* U, uint8_t* dead,
                          int32_t* dev_status, void* ws, hipStream_t stream) {
  return prepare_perm_launch(H, d64, damp, nullptr, U, dead, dev_status, ws, stream);
}

hipError_t prepare_perm_launch(float* H, int64_t d64, double damp, const int32_t* perm, float* U,
                               uint8_t* dead, int32_t* dev_status, void* ws, hipStream_t stream) {
  const int d = (int)d64;
  PrepWs w = carve(ws, d64);
  hipLaunchKernelGGL(prep_stats_kernel, dim3(1), dim3(1024), 0, stream, H, d, damp, dead, w.scal,
                     dev_status);
  const int nt32 = (int)ceil_div(d, 32);
  hipLaunchKernelGGL(prep_build_kernel, dim3(nt32 * (nt32 + 1) / 2), dim3(256), 0, stream, H, d,
                     (const double*)w.scal, w.A, w.M);
  if (perm)
    hipLaunchKernelGGL(prep_perm_kernel,
                       dim3((unsigned)ceil_div(d, 256), (unsigned)std::min(d, 1024)), dim3(256), 0,
                       stream, (const float*)H, d, perm, w.A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Steps in groups of UG: before each step of a group, its block column
  // (and block row of B) receives the group's earlier panels; after the
  // group, everything further right receives all of the group's panels at
  // once (K = 64 UG).
  const int nb = (int)ceil_div(d, NB);
  for (int g0 = 0; g0 < nb; g0 += UG) {
    const int gend = std::min(nb, g0 + UG);
    // the previous group's rest tiles, spread evenly over this group's column
    // updates (there are UG - 1 of them whenever the rest is not empty)
    const int rest = g0 > 0 ? rest_tiles(nb, g0) : 0;
    const int share = (int)ceil_div(rest, UG - 1);
    for (int k = g0; k < gend; ++k) {
      // the diagonal block of step k is factorized by the update launch that
      // brings it up to date (this group's part 1, or the previous group's
      // part 2); only step 0 needs a launch of its own.  Part 1 also applies
      // the previous step's panel, so only a group's last step has a panel
      // launch.
      if (k > g0) {
        const int lo = std::min(rest, (k - g0 - 1) * share);
        const int n = std::min(rest, lo + share) - lo;
        hipLaunchKernelGGL(fac_colupd_kernel, dim3(nb + n), dim3(256), 0, stream, w.A, w.M,
                           (const float*)w.Dinv[(k - 1) & 1], w.Dinv[k & 1], d, nb, g0, k, lo,
                           dev_status);
      } else if (k == 0) {
        hipLaunchKernelGGL(fac_diag_kernel, dim3(1), dim3(256), 0, stream, w.A, w.M, w.Dinv[0], d,
                           k, dev_status);
      }
      if (k + 1 < gend) continue;
      const int nrow = nb - k - 1;
      if (nrow + k > 0)
        hipLaunchKernelGGL(fac_panel_kernel, dim3(nrow + k), dim3(256), 0, stream, w.A, w.M,
                           (const float*)w.Dinv[k & 1], d, k, nrow, (const int32_t*)dev_status);
    }
    if (gend < nb)
      hipLaunchKernelGGL(fac_update_kernel, dim3(band_tiles(nb, gend)), dim3(256), 0, stream,
                         w.A, w.M, w.Dinv[gend & 1], d, nb, g0, gend, dev_status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = (int64_t)d * d;
  const int grid = (int)std::min<int64_t>(ceil_div(total, 256), 65536);
  hipLaunchKernelGGL(write_u_kernel, dim3(grid), dim3(256), 0, stream, (const float*)w.M, U, d);
  return hipGetLastError();
}

}  // namespace gptq
