// Damping, Cholesky and the upper factor of the inverse Hessian
// ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段一: H ~ 2X^T X + lambda I and a
// Cholesky factorization whose triangular factor drives the error feedback).
//
// U is the upper triangular matrix with U^T U = H^{-1}.  Rather than inverting H
// and factorizing again, it is formed as U = V^{-1} with H = V V^T, V upper: in
// the index-reversed space A = J H J (J reverses the order) this is an ordinary
// Cholesky A = L L^T and a triangular inverse M = L^{-1}, and U = J M J.  Both
// run in fp32 with IEEE fused multiply-adds (the fp32 matrix cores round like a
// chain of FMAs):
//   Cholesky, two-level and right-looking.  Panels of PW = 256 columns; each
//     is factorized by one persistent launch (chol_panel_kernel) in four
//     64-column steps: the 64 x 64 diagonal block is factorized and inverted
//     by one workgroup, every row block below multiplies its block by that
//     inverse (L_rj = A_rj L_jj^{-T}) and updates its later panel columns,
//     workgroups handing results to each other through release/acquire flags
//     with bounded waits.  Each workgroup keeps its row block's panel columns
//     in registers for the whole panel.  After the panel, the trailing matrix
//     receives the panel at once (K = 256): the next panel's columns right
//     away (chol_band_kernel), the rest by extra workgroups of the next
//     panel's launch.
//   Inverse, by recursive doubling: with the diagonal blocks' inverses from the
//     panels, blocks of size s pair up into blocks of 2s,
//       inv([L11 0; L21 L22]) = [X11 0; -X22 L21 X11  X22],
//     two matrix-product launches per level (inv_t_kernel: T = L21 X11,
//     inv_x_kernel: X21 = -X22 T), log2(d / 64) levels.
// Every product is an fp32 MFMA tile (v_mfma_f32_32x32x2f32).  This ordering
// keeps the rounding error of a textbook blocked factorization: U comes out
// within a few times sqrt(d) u sqrt(kappa(H)) of the exact factor.
#include "common.h"
#include "kernels.h"
#include "mfma_f32.h"
#include "inv_plan.h"

#include <algorithm>
#include <cstdlib>
#include <vector>

namespace gptq {

namespace {

constexpr int NB = 64;
constexpr int NJ = 4;                        // 64-column steps per panel
constexpr int PW = NB * NJ;                  // panel width
static_assert(NB == INV_NB && PW == INV_PW, "the inverse plan counts these tiles and panels");
constexpr int FLAGS_PER_PANEL = NJ + NJ * NJ;  // diagonal-block flags, then block-column flags
constexpr int SYNC_TIMEOUT = -1;             // dev_status when a bounded wait expires

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrepWs {
  float* A;      // [d x d] reversed damped H, then L (lower)
  float* M;      // [d x d] L^{-1} (lower)
  float* T;      // [d x d] the inverse's products T = L21 X11 (lower blocks)
  float* Dinv;   // [nb][NB x NB] inverses of the diagonal blocks
  int* flags;    // [panels][FLAGS_PER_PANEL]
  double* scal;  // [0] = lambda
};

inline int64_t n_panels(int64_t d) { return (d + PW - 1) / PW; }

PrepWs carve(void* ws, int64_t d) {
  char* p = (char*)ws;
  PrepWs w;
  const size_t mat = align256((size_t)d * d * sizeof(float));
  const size_t dinv = align256((size_t)((d + NB - 1) / NB) * NB * NB * sizeof(float));
  const size_t flg = align256((size_t)n_panels(d) * FLAGS_PER_PANEL * sizeof(int));
  w.A = (float*)p;
  w.M = (float*)(p + mat);
  w.T = (float*)(p + 2 * mat);
  w.Dinv = (float*)(p + 3 * mat);
  w.flags = (int*)(p + 3 * mat + dinv);
  w.scal = (double*)(p + 3 * mat + dinv + flg);
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
                                                          double* scal, int32_t* status,
                                                          int* __restrict__ flags,
                                                          int64_t nflags) {
  __shared__ double red[1024];
  // the factorization's hand-off flags start at zero
  for (int64_t i = threadIdx.x; i < nflags; i += 1024) flags[i] = 0;
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
// (lower triangle).
__global__ __launch_bounds__(256) void prep_build_kernel(float* __restrict__ H, int d,
                                                         const double* __restrict__ scal,
                                                         float* __restrict__ A) {
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

// DPP row broadcasts fused into the multiply-add that consumes them.  The
// compiler keeps a v_mov_b32_dpp apart from its v_fmac_f32 (and reuses one
// temporary for all of them, which serialises the pairs), so the fused form
// v_fmac_f32_dpp is written out:  acc += (lane SRC of b's 16-lane row) * m.
// A DPP read of a VGPR needs two wait states after the VALU instruction that
// wrote it; the inline assembly is opaque to the compiler's hazard checks,
// so those states are inserted explicitly: dpp_source_ready after the sources
// of a run of fmac_bcast are computed, and bcast_after_write for a value
// that an fmac_bcast has just written.
template <int SRC>
__device__ __forceinline__ void fmac_bcast(float& acc, float b, float m) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(b), "v"(m), "n"(SRC));
}
__device__ __forceinline__ void dpp_source_ready(float b, float m) {
  asm volatile("s_nop 1" ::"v"(b), "v"(m));
}
template <int SRC>
__device__ __forceinline__ float bcast_after_write(float v) {
  float r;
  asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
               : "=v"(r)
               : "v"(v), "n"(SRC));
  return r;
}

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
        const float inv = __builtin_amdgcn_rsqf(bcast_after_write<c>(a[c]));  // 1/sqrt, within 1 ulp
        const float l = a[c] * inv;  // L[r][c] below the pivot, L[c][c] on it
        a[c] = l;
        const float nl = l * ngt[c];  // -L[r][c] below the pivot, 0 elsewhere
        dpp_source_ready(l, nl);
        StaticFor<c + 1, SB>::run([&](auto Jv) {
          constexpr int j = decltype(Jv)::value;
          fmac_bcast<j>(a[j], l, nl);  // a[j] += L[j][c] nl
        });
        const float nlm = nl * inv;  // -L[r][c] / L[c][c]
        dpp_source_ready(mv[0], mv[1]);  // (their first values come from plain code)
        dpp_source_ready(mv[2], mv[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) fmac_bcast<c>(mv[q], mv[q], nlm);
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


// ---- synchronisation between the workgroups of one panel launch ----------
// Everything one workgroup hands to another inside a launch -- the diagonal
// block's inverse, the panel's blocks of L, the flags, a failure status -- is
// written and read with system-coherent accesses, which bypass the per-XCD L2
// caches.  With ordinary accesses and device-scope release/acquire fences, a
// reader on another XCD was measured to see stale data (wrong factors that
// varied from call to call); with coherent accesses the results are
// bit-reproducible.  A producer waits for its own stores to complete, the
// workgroup meets at a barrier, then one thread sets the flag (no cache-wide
// writeback).  A consumer's thread 0 polls the flag, then every thread takes
// an acquire fence, which drops stale copies from its XCD's L2 (measured:
// without it a reader could still see data from before the producer's
// write).  Every wait is bounded: it also stops when the factorization has
// failed (dev_status set by another workgroup) or after `spin` polls, which
// sets dev_status to SYNC_TIMEOUT; either way the workgroup leaves, so the
// launch always drains.  Flags live in the workspace and are cleared before
// the panels start (by prep_stats_kernel, the first launch of the step).

__device__ __forceinline__ void xstore2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float2 xload2(const float* p) {
  const uint64_t v =
      __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

__device__ __forceinline__ void publish(int* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool wait_flag(const int* flag, int32_t* status, int64_t spin,
                                          int* ok_lds) {
  if (threadIdx.x == 0) {
    int ok = 1;
    for (int64_t it = 0;; ++it) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) break;
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) {
        ok = 0;
        break;
      }
      if (it >= spin) {
        atomicCAS((int*)status, 0, SYNC_TIMEOUT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok && __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) ok = 0;
    *ok_lds = ok;
  }
  __syncthreads();
  // Coherent stores bypass the L2 without invalidating a copy that an earlier
  // ordinary load left in this XCD's L2; an acquire at device scope drops
  // such copies before the reads.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const bool ok = *ok_lds != 0;
  __syncthreads();  // everyone has read ok_lds before it is written again
  return ok;
}

// One panel of the Cholesky factorization: columns [c0, c0 + pw), pw =
// min(PW, d - c0), rows c0 .. d-1, everything left of c0 already applied.
// Workgroup r owns row block r (rows c0 + 64 r ..), and holds its blocks of
// the panel's column blocks j = 0 .. min(r, nj - 1) in accumulator registers
// (one 32 x 32 MFMA tile per wave and block).  Step j:
//   workgroup j      : factorizes and inverts its diagonal block (into A, M
//                      and Dinv), publishes flag diag[j] and is done;
//   workgroups r > j : wait for diag[j]; L_rj = A_rj Dinv_j^T; the panel's
//                      row blocks (r < nj) publish L_rj (flag col[j][r]);
//                      then A_{r,jj} -= L_rj L_{jj,j}^T for j < jj <= min(r,
//                      nj - 1), waiting for col[j][jj] (jj != r); the
//                      product is summed from zero and subtracted once.
// Every workgroup waits only on workgroups 0 .. nj-1, which never wait on a
// later one, so the launch completes whatever the residency.
using TileT = MfmaTile<NB, NB, NB, true>;   // C = P Q with Q given transposed
static_assert(TileT::FM == 1 && TileT::FN == 1, "one MFMA tile per wave and block");

template <class F>
__device__ __forceinline__ void acc_each(const f32x16& a, F&& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    f(wm * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3), wn * 32 + (lane & 31), q);
}

// Stage a register block as the P operand (rows x cols valid, zero outside),
// negated when NEG.
template <bool NEG>
__device__ __forceinline__ void stage_p_regs(float* lds, const f32x16& a, int rows, int cols) {
  acc_each(a, [&](int row, int col, int q) {
    const float x = a[q];
    lds[row * TileT::PP + col] = (row < rows && col < cols) ? (NEG ? -x : x) : 0.0f;
  });
}
// Stage a register block as the Q^T operand (rows = n, cols = k valid).
__device__ __forceinline__ void stage_q_regs(float* lds, const f32x16& a, int rows, int cols) {
  acc_each(a, [&](int row, int col, int q) {
    lds[TileT::lds_q_offset + row * TileT::QPITCH + col] =
        (row < rows && col < cols) ? a[q] : 0.0f;
  });
}

__device__ __forceinline__ void xstore1(float* p, float a) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float xload1(const float* p) {
  return __uint_as_float(
      __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
}

// Q^T operand (rows x cols valid, zero outside) from another workgroup's
// block, read coherently: in 8-byte pairs when the rows are 8-byte aligned
// (even leading dimension and base), else one element at a time.
__device__ __forceinline__ void load_q_xchg(float* lds, const float* src, int64_t ld, int rows,
                                            int cols) {
  float* q0 = lds + TileT::lds_q_offset;
  if ((ld & 1) == 0 && ((uintptr_t)src & 7) == 0) {
    float2 v[NB * NB / 512];
#pragma unroll
    for (int u = 0; u < NB * NB / 512; ++u) {
      const int e = u * 256 + threadIdx.x, r = e / (NB / 2), c = 2 * (e % (NB / 2));
      v[u] = xload2(src + (int64_t)min(r, rows - 1) * ld + min(c, (cols - 1) & ~1));
    }
#pragma unroll
    for (int u = 0; u < NB * NB / 512; ++u) {
      const int e = u * 256 + threadIdx.x, r = e / (NB / 2), c = 2 * (e % (NB / 2));
      q0[r * TileT::QPITCH + c] = (r < rows && c < cols) ? v[u].x : 0.0f;
      q0[r * TileT::QPITCH + c + 1] = (r < rows && c + 1 < cols) ? v[u].y : 0.0f;
    }
    return;
  }
  float v[NB * NB / 256];
#pragma unroll
  for (int u = 0; u < NB * NB / 256; ++u) {
    const int e = u * 256 + threadIdx.x, r = e / NB, c = e % NB;
    v[u] = xload1(src + (int64_t)min(r, rows - 1) * ld + min(c, cols - 1));
  }
#pragma unroll
  for (int u = 0; u < NB * NB / 256; ++u) {
    const int e = u * 256 + threadIdx.x, r = e / NB, c = e % NB;
    q0[r * TileT::QPITCH + c] = (r < rows && c < cols) ? v[u] : 0.0f;
  }
}

__device__ __forceinline__ void mma1(const float* lds, f32x16& acc) {
  TileT::mma(lds, *reinterpret_cast<f32x16(*)[1][1]>(&acc));
}

template <int TS>
__device__ __forceinline__ void syrk_tile(float* __restrict__ A, int d, int c0, int c1, int i0,
                                          int j0, float* lds);

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// ---- the inverse L^{-1} by recursive doubling --------------------------
// Level s (a power of two times 64): pairs (a, b = a + s, e = min(b + s, d)),
// a = 0, 2s, 4s, ..., b < d, with
//   inv([L11 0; L21 L22]) = [X11 0; -X22 L21 X11  X22]
// in two steps over 64 x 64 tiles (sb = s / 64, sb^2 tiles per pair):
//   T step: T[b:e, a:b] = L[b:e, a:b] M[a:b, a:b]   (M lower: k >= 64 ct)
//   X step: M[b:e, a:b] = -M[b:e, b:e] T[b:e, a:b]  (M lower: k < 64 rt + 64)
// starting from the diagonal blocks' inverses, which the factorization writes
// into M.  A step's tiles are numbered g = pair * sb^2 + local, the local
// order longest tile first (ct ascending for T, rt descending for X).  A T
// tile needs L's columns a .. b final and M[a:b, a:b] complete; an X tile
// needs its pair's T tiles and M[b:e, b:e].  The host hands each launch the
// tiles whose operands are complete when it starts: the factorization's
// launches carry the ones that are ready before it ends (on the CUs its
// latency-bound chain leaves idle), inv_items_kernel the rest.  The T regions
// (and the X regions of M) of different pairs and levels are disjoint, and
// every tile does the same arithmetic whichever launch runs it.
using InvTile = MfmaTile<NB, NB, 32, false>;  // C = P Q with Q row-major

template <bool XSTEP>
__device__ __forceinline__ void inv_tile(const float* __restrict__ L, float* __restrict__ M,
                                         float* __restrict__ Tb, int d, int s, int g, float* lds) {
  using Tile = InvTile;
  const int sb = s / NB;
  const int p = g / (sb * sb), lt = g % (sb * sb);
  const int major = lt / sb, minor = lt % sb;
  const int rt = XSTEP ? sb - 1 - major : minor, ct = XSTEP ? minor : major;
  const int a = 2 * s * p, b = a + s;
  const int i0 = b + NB * rt, j0 = a + NB * ct;
  if (i0 >= d) return;
  const int ib = min(NB, d - i0);
  const int k_lo = XSTEP ? 0 : NB * ct, k_hi = XSTEP ? min(NB * rt + NB, d - b) : s;
  const float* Pb = XSTEP ? M + (int64_t)i0 * d + b : L + (int64_t)i0 * d + a;
  const float* Qb = XSTEP ? Tb + (int64_t)b * d + j0 : M + (int64_t)a * d + j0;
  f32x16 acc[Tile::FM][Tile::FN];
  Tile::zero(acc);
  typename Tile::PQRegs v;
  auto fetch = [&](int k) __attribute__((always_inline)) {
    const int kn = min(32, k_hi - k);
    Tile::fetch_pq(v, Pb + k, d, ib, kn, Qb + (int64_t)k * d, d, kn, NB);
  };
  fetch(k_lo);
  for (int k = k_lo; k < k_hi; k += 32) {
    const int kn = min(32, k_hi - k);
    if (k > k_lo) __syncthreads();
    Tile::template stage_pq<XSTEP>(lds, v, ib, kn, kn, NB);
    __syncthreads();
    if (k + 32 < k_hi) fetch(k + 32);
    Tile::mma(lds, acc);
  }
  float* C = (XSTEP ? M : Tb) + (int64_t)i0 * d + j0;
  Tile::template store<false>(C, d, ib, NB, acc);
}

// Tile k of a launch's items (k < the sum of cnt).
__device__ __forceinline__ void inv_item_tile(const InvItems& it, int k, const float* L, float* M,
                                              float* Tb, int d, float* lds) {
  int s = 0, x = 0, g = -1;
#pragma unroll
  for (int i = 0; i < INV_ITEMS; ++i) {
    if (g < 0 && i < it.n) {
      if (k < it.cnt[i]) {
        s = it.s[i];
        x = it.x[i];
        g = it.g0[i] + k;
      } else {
        k -= it.cnt[i];
      }
    }
  }
  if (g < 0) return;
  if (x)
    inv_tile<true>(L, M, Tb, d, s, g, lds);
  else
    inv_tile<false>(L, M, Tb, d, s, g, lds);
}

// Workgroups past the panel's row blocks (blockIdx.x >= rows) are passengers:
// the first `rest` apply the previous panel [pc0, c0) to the trailing tiles
// from c0 + PW on (128 x 128 lower tiles of that region), which this panel does
// not touch; the others are tiles of the inverse whose operands were complete
// when the launch started (inv_tile: they read L's columns before c0 and M, T,
// which nothing else in the launch writes).
__global__ __launch_bounds__(256) void chol_panel_kernel(float* __restrict__ A,
                                                         float* __restrict__ M,
                                                         float* __restrict__ Dinv,
                                                         int* __restrict__ flags, int d, int c0,
                                                         int rows, int pc0, int rest,
                                                         float* __restrict__ Tb, InvItems inv,
                                                         int32_t* status, int64_t spin) {
  if (*status != 0) return;
  constexpr size_t LDS_FLOATS =
      cmax(cmax(cmax(TileT::lds_floats, DIAG_LDS_FLOATS), MfmaTile<128, 128, 32, true>::lds_floats),
           InvTile::lds_floats);
  __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
  __shared__ int ok_lds;
  if ((int)blockIdx.x >= rows + rest) {
    inv_item_tile(inv, (int)blockIdx.x - rows - rest, A, M, Tb, d, lds);
    return;
  }
  if ((int)blockIdx.x >= rows) {
    int ti, tj;
    tri_coords((int)blockIdx.x - rows, ti, tj);
    const int r0 = c0 + PW;
    syrk_tile<128>(A, d, pc0, c0, r0 + 128 * ti, r0 + 128 * tj, lds);
    return;
  }
  const int r = blockIdx.x;
  const int pw = min(PW, d - c0), nj = (pw + NB - 1) / NB;
  const int i0 = c0 + NB * r, ib = min(NB, d - i0);
  int* fdiag = flags + (int64_t)(c0 / PW) * FLAGS_PER_PANEL;
  int* fcol = fdiag + NJ;
  const int jmax = min(r, nj - 1);
  // this row block's panel blocks (unconditional loads from clamped
  // addresses; blocks past jmax are never used)
  f32x16 acc[NJ];
  StaticFor<0, NJ>::run([&](auto J) {
    constexpr int j = decltype(J)::value;
    const int k0 = min(c0 + NB * j, d - 1), kb = max(1, min(NB, d - k0));
    acc_each(acc[j], [&](int row, int col, int q) {
      acc[j][q] = A[(int64_t)(i0 + min(row, ib - 1)) * d + k0 + min(col, kb - 1)];
    });
  });
  bool done = false;
  StaticFor<0, NJ>::run([&](auto J) {
    constexpr int j = decltype(J)::value;
    if (done || j > jmax) return;
    const int k0 = c0 + NB * j, kb = min(NB, d - k0), kg = k0 / NB;
    if (j == r) {
      // the diagonal block, brought up to date in registers, straight into the
      // factorization's LDS copy
      DiagLds& L = *reinterpret_cast<DiagLds*>(lds);
      __syncthreads();
      acc_each(acc[j], [&](int row, int col, int q) {
        L.tile[row][col] = diag_entry(row, col, kb, acc[j][q]);
      });
      for (int e = threadIdx.x; e < NB * (NB + 1); e += 256) (&L.mtile[0][0])[e] = 0.0f;
      __syncthreads();
      diag_factor(L, A, M, Dinv + (size_t)kg * NB * NB, d, kg, status);
      // the inverse again, for the other workgroups, from its LDS copy, and
      // a failure made visible to them
      for (int e = threadIdx.x; e < NB * NB / 2; e += 256) {
        const int rr = e / (NB / 2), cc = 2 * (e % (NB / 2));
        xstore2(Dinv + (size_t)kg * NB * NB + rr * NB + cc, L.mtile[rr][cc], L.mtile[rr][cc + 1]);
      }
      if (threadIdx.x == 0 && *status != 0)
        __hip_atomic_store(status, *status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      publish(fdiag + j);
      done = true;
      return;
    }
    if (!wait_flag(fdiag + j, status, spin, &ok_lds)) {
      done = true;
      return;
    }
    // L_rj = A_rj Dinv_j^T
    stage_p_regs<false>(lds, acc[j], ib, kb);
    load_q_xchg(lds, Dinv + (size_t)kg * NB * NB, NB, NB, NB);
    __syncthreads();
    TileT::zero(*reinterpret_cast<f32x16(*)[1][1]>(&acc[j]));
    mma1(lds, acc[j]);
    __syncthreads();
    float* Arj = A + (int64_t)i0 * d + k0;
    if (r < nj) {
      // through LDS (the P slot, free after the product) into coherent pairs
      acc_each(acc[j], [&](int row, int col, int q) { lds[row * TileT::PP + col] = acc[j][q]; });
      __syncthreads();
      if ((d & 1) == 0) {  // rows 8-byte aligned: coherent pairs
        for (int e = threadIdx.x; e < NB * NB / 2; e += 256) {
          const int rr = e / (NB / 2), cc = 2 * (e % (NB / 2));
          if (rr < ib && cc + 1 < kb)
            xstore2(Arj + (int64_t)rr * d + cc, lds[rr * TileT::PP + cc],
                    lds[rr * TileT::PP + cc + 1]);
          else if (rr < ib && cc < kb)
            xstore1(Arj + (int64_t)rr * d + cc, lds[rr * TileT::PP + cc]);
        }
      } else {
        for (int e = threadIdx.x; e < NB * NB; e += 256) {
          const int rr = e / NB, cc = e % NB;
          if (rr < ib && cc < kb) xstore1(Arj + (int64_t)rr * d + cc, lds[rr * TileT::PP + cc]);
        }
      }
      __syncthreads();
    } else {
      acc_each(acc[j], [&](int row, int col, int q) {
        if (row < ib && col < kb) Arj[(int64_t)row * d + col] = acc[j][q];
      });
    }
    // (a panel row block publishes L_rj after its own update below: the
    // stores complete meanwhile, and the workgroups that wait for it need it
    // only after the next diagonal block, so the wait for them stays off the
    // chain of diagonal blocks)
    // later panel columns of this row block: A_{r,jj} -= L_rj L_{jj,j}^T
    StaticFor<j + 1, NJ>::run([&](auto JJ) {
      constexpr int jj = decltype(JJ)::value;
      if (done || jj > jmax) return;
      const int kk0 = c0 + NB * jj, kkb = min(NB, d - kk0);
      if (jj != r) {
        if (!wait_flag(fcol + j * NJ + jj, status, spin, &ok_lds)) {
          done = true;
          return;
        }
        load_q_xchg(lds, A + (int64_t)kk0 * d + k0, d, kkb, kb);    // Q^T = L_{jj,j}
      } else {
        stage_q_regs(lds, acc[j], ib, kb);                          // Q^T = L_rj itself
      }
      stage_p_regs<false>(lds, acc[j], ib, kb);
      __syncthreads();
      f32x16 prod;
      TileT::zero(*reinterpret_cast<f32x16(*)[1][1]>(&prod));
      mma1(lds, prod);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[jj][q] -= prod[q];
    });
    if (!done && r < nj) publish(fcol + j * NJ + r);
  });
}

// Trailing update after a panel [c0, c1): A[c1:, c1:] (lower) -= P P^T with
// P = L[c1:, c0:c1] (K = c1 - c0 <= 256), in TS x TS tiles, K in chunks of 32,
// the next chunk's operands loaded while the current one multiplies.  The
// products are summed from zero and subtracted from A once: summed onto a
// preloaded A, every one of the K roundings would be at A's magnitude, which
// on the large diagonal entries grows the factor's error like sqrt(d) u |A|.
// Diagonal tiles are computed whole (their upper halves land in A's unused
// upper triangle).  The update is split in two: the band -- the next panel's
// columns [c1, c1 + PW), all rows below -- runs right after the panel
// (chol_band_kernel, 64 x 64 tiles); the rest -- rows and columns from
// c1 + PW on, which nothing reads before the panel after next -- runs as
// extra workgroups of the next panel's launch (128 x 128 tiles), on the
// compute units its latency-bound chain leaves idle.
template <int TS>
__device__ __forceinline__ void syrk_tile(float* __restrict__ A, int d, int c0, int c1, int i0,
                                          int j0, float* lds) {
  using TileS = MfmaTile<TS, TS, 32, true>;
  const int ib = min(TS, d - i0), jb = min(TS, d - j0);
  const int kw = c1 - c0;
  float* C = A + (int64_t)i0 * d + j0;
  f32x16 acc[TileS::FM][TileS::FN];
  TileS::zero(acc);
  typename TileS::PQRegs v;
  auto fetch = [&](int kc) __attribute__((always_inline)) {
    const int kn = min(32, kw - kc);
    TileS::fetch_pq(v, A + (int64_t)i0 * d + c0 + kc, d, ib, kn,
                    A + (int64_t)j0 * d + c0 + kc, d, jb, kn);
  };
  fetch(0);
  for (int kc = 0; kc < kw; kc += 32) {
    const int kn = min(32, kw - kc);
    if (kc > 0) __syncthreads();
    TileS::template stage_pq<false>(lds, v, ib, kn, jb, kn);
    __syncthreads();
    if (kc + 32 < kw) fetch(kc + 32);
    TileS::mma(lds, acc);
  }
  TileS::template store<true>(C, d, ib, jb, acc);
}

// The band after panel [c0, c1): tiles (rows c1 + 64 i, columns c1 + 64 j) of
// the next panel's columns, lower ones only; workgroups past the band's
// ntiles are short tiles of the inverse (inv_tile) that were ready when the
// launch started.
__global__ __launch_bounds__(256) void chol_band_kernel(float* __restrict__ A, int d, int c0,
                                                        int c1, int nbc, int ntiles,
                                                        float* __restrict__ M,
                                                        float* __restrict__ Tb, InvItems inv,
                                                        const int32_t* status) {
  if (*status != 0) return;
  __shared__ __attribute__((aligned(16))) float
      lds[cmax(MfmaTile<64, 64, 32, true>::lds_floats, InvTile::lds_floats)];
  if ((int)blockIdx.x >= ntiles) {
    inv_item_tile(inv, (int)blockIdx.x - ntiles, A, M, Tb, d, lds);
    return;
  }
  const int i = blockIdx.x / nbc, j = blockIdx.x % nbc;
  if (j > i) return;
  syrk_tile<64>(A, d, c0, c1, c1 + 64 * i, c1 + 64 * j, lds);
}

// The inverse's tiles that were not carried by the factorization's launches:
// one launch per round of tiles whose operands are complete (inv_tile).
// When the whole grid is resident at once (up to four workgroups per CU),
// nothing is handed out as CUs free up, so the longest-first order would give
// the first CUs all the long tiles: workgroups t, t + 256, t + 512, t + 768
// share a CU, and a snake over blocks of 256 (odd blocks reversed) gives every
// CU a mix of long and short tiles with about the same total.
__global__ __launch_bounds__(256) void inv_items_kernel(const float* __restrict__ L,
                                                        float* __restrict__ M,
                                                        float* __restrict__ Tb, int d,
                                                        InvItems items, const int32_t* status) {
  if (*status != 0) return;
  __shared__ __attribute__((aligned(16))) float lds[InvTile::lds_floats];
  int t = blockIdx.x;
  if (gridDim.x <= 4 * 256) {
    const int blk = t >> 8, r = t & 255;
    t = (blk & 1) ? (blk << 8) + min(255, (int)gridDim.x - 1 - (blk << 8)) - r : t;
  }
  inv_item_tile(items, t, L, M, Tb, d, lds);
}

// U[i][j] = M[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const float* __restrict__ M,
                                                      float* __restrict__ U, int d, int vec) {
  const int64_t total = (int64_t)d * d;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (vec) {
    // four entries of a row per thread (d a multiple of 4, U 16-byte
    // aligned): U[i][j .. j + 3] come from M[d - 1 - i][d - 4 - j .. d - 1 - j],
    // one aligned float4 read backwards
    for (int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x; e4 < total / 4; e4 += stride) {
      const int64_t e = 4 * e4;
      const int i = (int)(e / d), j = (int)(e % d);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j + 3 >= i) {
        const float4 m = *(const float4*)(M + (int64_t)(d - 1 - i) * d + (d - 4 - j));
        o.x = (i <= j) ? m.w : 0.0f;
        o.y = (i <= j + 1) ? m.z : 0.0f;
        o.z = (i <= j + 2) ? m.y : 0.0f;
        o.w = m.x;
      }
      *(float4*)(U + e) = o;
    }
    return;
  }
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += stride) {
    const int i = (int)(e / d), j = (int)(e % d);
    U[e] = (i <= j) ? M[(int64_t)(d - 1 - i) * d + (d - 1 - j)] : 0.0f;
  }
}


// Polls of a bounded wait before it gives up (GPTQ_SYNC_SPIN_LIMIT overrides;
// a tiny value forces the timeout path, for tests of it).
}  // namespace

int64_t sync_spin_limit() {
  static const int64_t v = [] {
    const char* e = std::getenv("GPTQ_SYNC_SPIN_LIMIT");
    return e ? std::max<int64_t>(0, std::atoll(e)) : ((int64_t)1 << 20);
  }();
  return v;
}

size_t prepare_workspace(int64_t d) {
  const size_t mat = align256((size_t)d * d * sizeof(float));
  return 3 * mat + align256((size_t)((d + NB - 1) / NB) * NB * NB * sizeof(float)) +
         align256((size_t)n_panels(d) * FLAGS_PER_PANEL * sizeof(int)) + 256;
}

hipError_t prepare_launch(float* H, int64_t d64, double damp, float* U, uint8_t* dead,
                          int32_t* dev_status, void* ws, hipStream_t stream) {
  return prepare_perm_launch(H, d64, damp, nullptr, U, dead, dev_status, ws, stream);
}

hipError_t prepare_perm_launch(float* H, int64_t d64, double damp, const int32_t* perm, float* U,
                               uint8_t* dead, int32_t* dev_status, void* ws, hipStream_t stream) {
  const int d = (int)d64;
  PrepWs w = carve(ws, d64);
  const int64_t nflags = n_panels(d) * FLAGS_PER_PANEL;
  hipLaunchKernelGGL(prep_stats_kernel, dim3(1), dim3(1024), 0, stream, H, d, damp, dead, w.scal,
                     dev_status, w.flags, nflags);
  const int nt32 = (int)ceil_div(d, 32);
  hipLaunchKernelGGL(prep_build_kernel, dim3(nt32 * (nt32 + 1) / 2), dim3(256), 0, stream, H, d,
                     (const double*)w.scal, w.A);
  if (perm)
    hipLaunchKernelGGL(prep_perm_kernel,
                       dim3((unsigned)ceil_div(d, 256), (unsigned)std::min(d, 1024)), dim3(256), 0,
                       stream, (const float*)H, d, perm, w.A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t spin = sync_spin_limit();
  InvPlan inv(d);
  for (int c0 = 0; c0 < d; c0 += PW) {
    const int rows = (int)ceil_div(d - c0, NB);
    // passengers: the previous panel's update of the region from c0 + PW on,
    // then the inverse's tiles that are ready, within what is left of the
    // launch's passenger budget
    int rest = 0;
    if (c0 > 0 && c0 + PW < d) {
      const int nt = (int)ceil_div(d - c0 - PW, 128);
      rest = nt * (nt + 1) / 2;
    }
    const InvItems items = inv_panel_items(inv, c0, rest);
    hipLaunchKernelGGL(chol_panel_kernel, dim3(rows + rest + InvPlan::count(items)), dim3(256), 0,
                       stream, w.A, w.M, w.Dinv, w.flags, d, c0, rows, c0 - PW, rest, w.T, items,
                       dev_status, spin);
    const int c1 = std::min(d, c0 + PW);
    if (c1 < d) {  // the band: the next panel's columns
      const int nr = (int)ceil_div(d - c1, 64);
      const int nbc = (int)ceil_div(std::min(d, c1 + PW) - c1, 64);
      const InvItems bitems = inv_band_items(inv, c1);
      hipLaunchKernelGGL(chol_band_kernel, dim3(nr * nbc + InvPlan::count(bitems)), dim3(256), 0,
                         stream, w.A, d, c0, c1, nbc, nr * nbc, w.M, w.T, bitems,
                         (const int32_t*)dev_status);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the rest of the inverse, a launch per round of ready tiles
  while (!inv.finished()) {
    const InvItems items = inv.take(d, -1.0);
    const int n = InvPlan::count(items);
    if (n == 0) return hipErrorUnknown;  // unreachable: with every column final a step is ready
    hipLaunchKernelGGL(inv_items_kernel, dim3(n), dim3(256), 0, stream, (const float*)w.A, w.M,
                       w.T, d, items, (const int32_t*)dev_status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = (int64_t)d * d;
  const int vec = (d % 4 == 0) && ((uintptr_t)U % 16 == 0);
  const int grid = (int)std::min<int64_t>(ceil_div(vec ? total / 4 : total, 256), 65536);
  hipLaunchKernelGGL(write_u_kernel, dim3(grid), dim3(256), 0, stream, (const float*)w.M, U, d,
                     vec);
  return hipGetLastError();
}

}  // namespace gptq
