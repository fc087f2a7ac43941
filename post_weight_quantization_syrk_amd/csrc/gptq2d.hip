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
// Two schedules, the same arithmetic per entry:
//   n <= 1024, one persistent launch (g2d_rows_kernel).  Each wave owns one
//     row i and walks it from j = n - 1 down to 0, holding row i of P (and of
//     R_L) in registers.  P[k][j] receives its last term when row k handles
//     entry (k, j), and entry (i, j) reads P[k][j] only for k > i, so it
//     suffices that row i + 1 has finished column j (row i + 1 waited in turn
//     for row i + 2, and so on).  After entry (i, j) the wave publishes the
//     final P[i][j] into a write-once array F[j][i] (transposed: the reads of
//     one entry are a contiguous run); F starts filled with a signalling NaN,
//     which no float64 operation produces, so each value is its own "ready"
//     flag.  F goes through memory with system-coherent accesses (the rows
//     run on every XCD); the rows of one workgroup also hand their values to
//     each other through LDS.  Every wait is bounded: a wait that gives up
//     takes NaN for the value, which spreads to every entry that depends on
//     it, so the launch always drains and Z shows the failure.  Rows go to
//     waves in descending order, so a workgroup waits only on itself and on
//     earlier workgroups.
//   n > 1024, one launch per anti-diagonal (g2d_diag_kernel): P row-major in
//     memory (the update of row i is a contiguous store); the read of column
//     j strides by n, but the entries of one anti-diagonal read adjacent
//     columns of the same rows, so neighbouring entries (the waves of a
//     workgroup) share cache lines.
// R_R is transposed once (RT[j][c] = R_R[c][j]) so the update reads a
// contiguous row.  Everything is float64.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int G2_WAVES = 4;  // entries per workgroup, one wave each

// A signalling NaN: arithmetic only ever produces quiet NaNs, so no computed
// value of P has these bits.
constexpr uint64_t G2_EMPTY = 0x7FF4DEADBEEF0001ull;
constexpr int G2_ROWS_MAX_NU = 16;  // register-resident rows: n <= 64 * 16

__device__ __forceinline__ uint64_t sys_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void sys_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// RT = R_R^T (upper triangle of R_R only; the rest of RT zero) and the
// running array: P = 0 (one launch per anti-diagonal) or F = empty (the
// persistent launch, stored coherently like every later access to it).
__global__ __launch_bounds__(256) void g2d_init_kernel(const double* __restrict__ RR,
                                                       double* __restrict__ RT,
                                                       uint64_t* __restrict__ P, int n,
                                                       int persistent) {
  const int64_t total = (int64_t)n * n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e / n), c = (int)(e % n);
    RT[e] = (c <= j) ? RR[(int64_t)c * n + j] : 0.0;
    if (persistent) sys_store(P + e, G2_EMPTY);
    else P[e] = 0;  // the bits of +0.0
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

__device__ __forceinline__ double lane_value(double x, int src) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), src);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), src);
  return __hiloint2double(hi, lo);
}

// Poll one entry of F until it holds a value or the wave's poll budget is
// spent (then NaN, and the budget stays spent); b is a first read of it.
__device__ __forceinline__ double wait_value(const uint64_t* p, uint64_t b, int64_t& budget) {
  while (b == G2_EMPTY && budget > 0) {
    __builtin_amdgcn_s_sleep(1);
    b = sys_load(p);
    --budget;
  }
  return b == G2_EMPTY ? __builtin_nan("") : __longlong_as_double((long long)b);
}

// The sum of v over the wave, the same in every lane: DPP exchanges inside
// each 16-lane row (pairs, quads, mirrored halves, mirrored rows: each step
// adds two operands that its partner lane adds in the other order), then
// the four row sums in lane order.  Nothing here waits on the LDS counter.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  double s = lane_value(v, 0);
  s += lane_value(v, 16);
  s += lane_value(v, 32);
  s += lane_value(v, 48);
  return s;
}

// The same for a value another wave of this workgroup puts into LDS.
__device__ __forceinline__ uint64_t lds_get(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ double lds_wait(const uint64_t* p, uint64_t b, int64_t& budget) {
  while (b == G2_EMPTY && budget > 0) {
    __builtin_amdgcn_s_sleep(1);
    b = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    --budget;
  }
  return b == G2_EMPTY ? __builtin_nan("") : __longlong_as_double((long long)b);
}
__device__ __forceinline__ void lds_put(uint64_t* p, double v) {
  __hip_atomic_store(p, (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Rows (waves) per workgroup of the persistent launch: eight, or four where a
// wave needs more than the 256 registers two waves per SIMD leave it.
template <int NU>
constexpr int g2_rows_per_wg() { return NU >= 16 ? 4 : 8; }

// The persistent schedule.  Workgroup b holds rows i0, i0 - 1, ..., i0 - RW + 1
// (i0 = n - 1 - RW b), wave w row i = i0 - w; lane l holds columns c = l + 64 u,
// u < NU.  Entry (i, j) sums R_L[i][k] P[k][j] over three kinds of rows k:
//   far   k >= i0 + 3   read from F one entry ahead (with the next row of
//                       R_R^T): those rows finished column j at least two
//                       anti-diagonals before this entry starts;
//   near  k = i0 + 1, i0 + 2 (the two rows below the workgroup): wave 0 reads
//                       them from F, waiting for i0 + 1, and puts both into
//                       LDS for the other waves;
//         i < k <= i0   the workgroup's own rows, each published into LDS by
//                       its wave; wave w waits for wave w - 1 (row i + 1);
//   own   k = i         P[i][j] from registers;
// then Z, the published value P[i][j] + e R_R[j][j] (the same fused
// multiply-add as the row update's) into LDS and F, and the row update.  The
// far sum is taken before the wait, so after it only the near terms, the
// division and the rounding remain: most hand-offs stay inside a compute
// unit, and one in RW goes through memory.  Every read value is checked
// against the empty pattern and read again if needed.
template <int NU, int RW>
__global__ __launch_bounds__(64 * RW) void g2d_rows_kernel(const double* __restrict__ Y,
                                                           const double* __restrict__ RL,
                                                           const double* __restrict__ RT,
                                                           uint64_t* __restrict__ F,
                                                           double* __restrict__ Z, int n,
                                                           int64_t spin) {
  static_assert((RW & (RW - 1)) == 0, "rows per workgroup: a power of two");
  constexpr int NC = 64 * NU;
  __shared__ uint64_t lv[RW][NC];  // the workgroup's rows: lv[w][j] = P[i0 - w][j]
  __shared__ uint64_t ext[2][NC];  // ext[t][j] = P[i0 + 1 + t][j]
  for (int e = threadIdx.x; e < RW * NC; e += 64 * RW) (&lv[0][0])[e] = G2_EMPTY;
  for (int e = threadIdx.x; e < 2 * NC; e += 64 * RW) (&ext[0][0])[e] = G2_EMPTY;
  __syncthreads();  // the only barrier: from here on the waves run apart
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i0 = n - 1 - RW * (int)blockIdx.x;
  const int i = i0 - w;
  if (i < 0) return;  // past row 0: no wave waits for these
  const double* rlrow = RL + (int64_t)i * n;
  const int kf = i0 + 3;  // first far row
  double rl[NU], p[NU], yv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = lane + 64 * u;
    rl[u] = (c >= kf && c < n) ? rlrow[c] : 0.0;
    yv[u] = (c < n) ? Y[(int64_t)i * n + c] : 0.0;
    p[u] = 0.0;
  }
  // near coefficients cn[t] = R_L[i][i + t], t = 1 .. w + 2 (0 past the matrix)
  double cn[RW + 2];
#pragma unroll
  for (int t = 0; t < RW + 2; ++t)
    cn[t] = (t >= 1 && t <= w + 2 && i + t < n) ? rlrow[i + t] : 0.0;
  const double rl_ii = rlrow[i];
  int64_t budget = spin;
  // Operands of entry j, read one entry ahead: the row of R_R^T, the far
  // values of F and (wave 0) the two rows below the workgroup.  Two sets used
  // in turn (the loop body is written out twice), so no copy waits for a
  // read in flight.  No scalar loads inside the loop: their results come
  // back out of order, so any wait for LDS would wait for them too.
  struct Ops {
    double rt[NU];
    uint64_t fb[NU];
    uint64_t b1, b2;
  };
  // Every load is unconditional, from an address clamped into the matrix,
  // and masked afterwards: with no branch around them the compiler can count
  // them, and the wait for this entry's operands leaves the next entry's in
  // flight.  (jj = -1, past the last entry, reads row 0 and is never used.)
  auto fetch = [&](int jj, Ops& o) __attribute__((always_inline)) {
    const int jc = max(jj, 0);
    const double* rtrow = RT + (int64_t)jc * n;
    const uint64_t* frow = F + (int64_t)jc * n;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = lane + 64 * u;
      const double r = rtrow[min(c, jc)];
      const uint64_t f = sys_load(frow + min(max(c, kf), n - 1));
      o.rt[u] = (c <= jc) ? r : 0.0;
      o.fb[u] = (c >= kf && c < n) ? f : 0;  // 0: the bits of +0.0
    }
    const uint64_t f2 = sys_load(frow + min(i0 + 2, n - 1));
    const uint64_t f1 = sys_load(frow + min(i0 + 1, n - 1));
    o.b2 = (w == 0 && i0 + 2 < n) ? f2 : 0;
    o.b1 = (w == 0 && i0 + 1 < n) ? f1 : 0;
  };
  // entry j's element of a register row (lane j % 64, slot j / 64), in every lane
  auto at_col = [&](const double (&v)[NU], int j) __attribute__((always_inline)) {
    double x = 0.0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (u == (j >> 6)) x = v[u];
    return lane_value(x, j & 63);
  };
  auto entry = [&](int j, const Ops& o) __attribute__((always_inline)) {
    // far rows
    double acc0 = 0.0, acc1 = 0.0;
    int64_t lb = budget;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      double f = __longlong_as_double((long long)o.fb[u]);
      if (o.fb[u] == G2_EMPTY) f = wait_value(F + (int64_t)j * n + lane + 64 * u, o.fb[u], lb);
      if (u & 1) acc1 = fma(rl[u], f, acc1);
      else acc0 = fma(rl[u], f, acc0);
    }
    if (__any(lb <= 0)) budget = 0;
    double S = wave_sum_dpp(acc0 + acc1);
    const double pj = at_col(p, j);
    const double y = at_col(yv, j);
    const double rr = at_col(o.rt, j);
    const double den = rl_ii * rr;
    // near rows, farthest first; all first reads issued together
    if (w == 0) {
      const uint64_t* frow = F + (int64_t)j * n;
      const double v2 = wait_value(frow + i0 + 2, o.b2, budget);
      const double v1 = wait_value(frow + i0 + 1, o.b1, budget);
      if (lane == 0) {
        lds_put(&ext[1][j], v2);
        lds_put(&ext[0][j], v1);
      }
      S = fma(cn[2], v2, S);
      S = fma(cn[1], v1, S);
    } else {
      const uint64_t* src[RW + 2];
      uint64_t nb[RW + 2];
#pragma unroll
      for (int t = 1; t < RW + 2; ++t) {
        src[t] = (t == w + 2) ? &ext[1][j] : (t == w + 1) ? &ext[0][j] : &lv[(w - t) & (RW - 1)][j];
        nb[t] = (t <= w + 2) ? lds_get(src[t]) : 0;
      }
#pragma unroll
      for (int t = RW + 1; t >= 1; --t)
        if (t <= w + 2) S = fma(cn[t], lds_wait(src[t], nb[t], budget), S);
    }
    S = fma(rl_ii, pj, S);
    const double z = rint(y + S / den);
    const double e = y - z;
    const double fv = fma(e, rr, pj);
    if (lane == 0) {
      lds_put(&lv[w][j], fv);
      sys_store(F + (int64_t)j * n + i, (uint64_t)__double_as_longlong(fv));
      Z[(int64_t)i * n + j] = z;
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) p[u] = fma(e, o.rt[u], p[u]);
  };
  Ops oa, ob;
  fetch(n - 1, oa);
  for (int j = n - 1; j >= 0; j -= 2) {
    fetch(j - 1, ob);
    entry(j, oa);
    if (j == 0) break;
    fetch(j - 2, oa);
    entry(j - 1, ob);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int NU>
void launch_rows(const double* Y, const double* RL, const double* RT, uint64_t* F, double* Z,
                 int n, hipStream_t stream) {
  constexpr int RW = g2_rows_per_wg<NU>();
  hipLaunchKernelGGL((g2d_rows_kernel<NU, RW>), dim3((unsigned)ceil_div(n, RW)), dim3(64 * RW), 0,
                     stream, Y, RL, RT, F, Z, n, sync_spin_limit());
}

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
  const int nu = (int)ceil_div(n, 64);
  const int persistent = nu <= G2_ROWS_MAX_NU;
  hipLaunchKernelGGL(g2d_init_kernel, dim3(grid), dim3(256), 0, stream, RR, RT, (uint64_t*)P, n,
                     persistent);
  if (persistent) {
    const double* RTc = RT;
    uint64_t* F = (uint64_t*)P;
    if (nu <= 1) launch_rows<1>(Y, RL, RTc, F, Z, n, stream);
    else if (nu <= 2) launch_rows<2>(Y, RL, RTc, F, Z, n, stream);
    else if (nu <= 4) launch_rows<4>(Y, RL, RTc, F, Z, n, stream);
    else if (nu <= 8) launch_rows<8>(Y, RL, RTc, F, Z, n, stream);
    else launch_rows<16>(Y, RL, RTc, F, Z, n, stream);
    return hipGetLastError();
  }
  for (int s = 2 * n - 2; s >= 0; --s) {
    const int m = std::min(s, n - 1) - std::max(0, s - n + 1) + 1;
    hipLaunchKernelGGL(g2d_diag_kernel, dim3((unsigned)ceil_div(m, G2_WAVES)),
                       dim3(64 * G2_WAVES), 0, stream, Y, RL, (const double*)RT, P, Z, n, s);
  }
  return hipGetLastError();
}

}  // namespace gptq
