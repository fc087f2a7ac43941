// Hessian accumulation H += 2 X^T X  ("GPTQ：基于近似二阶信息的大模型权重量化",
// 阶段一: the layer Hessian is 2 X^T X over the calibration tokens).
//
// bf16 inputs: an MFMA SYRK on gfx950.  Each workgroup (4 waves) owns one
// 256 x 256 lower-triangle tile of H and one contiguous token range (split-K);
// X tiles are staged through LDS in their natural token-major layout and fed
// to v_mfma_f32_32x32x16_bf16 through LDS transpose reads
// (ds_read_b64_tr_b16), which deliver each lane 8 consecutive tokens of one
// column.  bf16 x bf16 products are exact in fp32; sums are fp32.
// Workgroup -> (tile, split) is XCD-aware: consecutive workgroup ids land on
// different XCDs, so split s is pinned to XCD s % 8 and every tile of one split
// streams the same token rows through that XCD's L2 at about the same time.
// Partial tiles go to a workspace; the last workgroup to finish a tile adds its
// partials to H in a fixed order, so results are deterministic.
//
// fp32 inputs: a plain LDS-tiled fp32 FMA kernel (64 x 64 tiles) with the same
// split-K / reduction structure.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>

namespace gptq {

namespace {

constexpr int TB = 256;          // bf16 output tile edge
constexpr int BK = 64;           // tokens per pipeline stage
constexpr int PITCH = 288;       // LDS row pitch in bf16 elements (256 + 32)
constexpr int NTHR = 256;        // 4 waves
constexpr int BUF = BK * PITCH;  // elements per operand buffer

constexpr int TF = 64;           // fp32 output tile edge
constexpr int BKF = 32;          // fp32 tokens per stage

__device__ __forceinline__ void tri_coords(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

struct SyrkArgs {
  const uint16_t* X;
  int64_t ldx;
  int64_t n;
  int d;
  int ntri;
  int splits;
  int64_t kper;
  float* partial;
  unsigned int* counters;  // one per tile, zero on entry, left zero on exit
  float* H;
};

// Split-K epilogue shared by both kernels.  Every workgroup has written its
// partial tile; the last one to arrive for a tile (device-scope counter) adds
// the partials to H in the fixed order s = 0..S-1, so the result does not
// depend on which workgroup finishes last.
template <int TILE, int NT>
__device__ __forceinline__ void splitk_finish(float* __restrict__ H, int d,
                                              const float* __restrict__ partial, int ntri,
                                              int splits, unsigned int* counters, int tile,
                                              int ti, int tj) {
  __shared__ unsigned int last_s;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int old = atomicAdd(&counters[tile], 1u);
    last_s = (old == (unsigned int)(splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  constexpr int64_t TSZ = (int64_t)TILE * TILE;
  const float4* base = (const float4*)(partial + (size_t)tile * TSZ);
  const size_t sstride = (size_t)ntri * (TSZ / 4);
  for (int e4 = threadIdx.x; e4 < TSZ / 4; e4 += NT) {
    const int r = (4 * e4) / TILE, c0 = (4 * e4) % TILE;
    const int gi = ti * TILE + r, gj0 = tj * TILE + c0;
    if (gi >= d || gj0 >= d || gj0 > gi) continue;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; ++k) {
      const float4 v = base[(size_t)k * sstride + e4];
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    float* h = H + (int64_t)gi * d + gj0;
    const float vals[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (gj0 + q < d && gj0 + q <= gi) h[q] = h[q] + 2.0f * vals[q];
  }
  if (threadIdx.x == 0) counters[tile] = 0u;
}

__global__ void clear_counters_kernel(unsigned int* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0u;
}

template <bool VEC>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ X, int64_t ldx, int64_t k0,
                                          int64_t kend, int c0, int d, int tid, uint4 (&reg)[8]) {
  const int col = c0 + (tid & 31) * 8;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t row = k0 + r * 8 + (tid >> 5);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < kend) {
      const uint16_t* src = X + row * ldx + col;
      if (VEC && col + 8 <= d) {
        v = *(const uint4*)src;
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8; ++e)
          if (col + e < d) w[e >> 1] |= ((uint32_t)src[e]) << (16 * (e & 1));
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    reg[r] = v;
  }
}

__device__ __forceinline__ void store_rows(uint16_t* buf, int tid, const uint4 (&reg)[8]) {
  const int vec = tid & 31;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = r * 8 + (tid >> 5);
    *(uint4*)(buf + row * PITCH + vec * 8) = reg[r];
  }
}

__device__ __forceinline__ bf16x8 frag(const uint16_t* p) {
  s16x4 lo = lds_read_tr16(p);
  s16x4 hi = lds_read_tr16(p + 4 * PITCH);
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <bool VEC>
__global__ __launch_bounds__(NTHR, 1) void syrk_bf16_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * BUF];

  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j = b >> 3;
  const int tile = j % a.ntri;
  const int split = (j / a.ntri) * 8 + xcd;
  int ti, tj;
  tri_coords(tile, ti, tj);
  const bool diag = (ti == tj);
  const int ci = ti * TB, cj = tj * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, i16 = lane & 15;
  const int lane_off = (8 * (g >> 1) + (i16 >> 2)) * PITCH + 16 * (g & 1) + 4 * (i16 & 3);

  const int64_t kb = (int64_t)split * a.kper;
  const int64_t ke = min(a.n, kb + a.kper);
  const int nst = (ke > kb) ? (int)ceil_div(ke - kb, BK) : 0;

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  uint4 ra[8], rb[8];
  if (nst > 0) {
    load_rows<VEC>(a.X, a.ldx, kb, ke, ci, a.d, tid, ra);
    if (!diag) load_rows<VEC>(a.X, a.ldx, kb, ke, cj, a.d, tid, rb);
    store_rows(lds, tid, ra);
    if (!diag) store_rows(lds + BUF, tid, rb);
    __syncthreads();
  }
  for (int s = 0; s < nst; ++s) {
    const bool more = (s + 1 < nst);
    if (more) {
      const int64_t k1 = kb + (int64_t)(s + 1) * BK;
      load_rows<VEC>(a.X, a.ldx, k1, ke, ci, a.d, tid, ra);
      if (!diag) load_rows<VEC>(a.X, a.ldx, k1, ke, cj, a.d, tid, rb);
    }
    const uint16_t* bufA = lds + (s & 1) * 2 * BUF;
    const uint16_t* bufB = diag ? bufA : bufA + BUF;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        fa[mi] = frag(bufA + lane_off + kk * 16 * PITCH + 128 * wm + 32 * mi);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        fb[ni] = frag(bufB + lane_off + kk * 16 * PITCH + 128 * wn + 32 * ni);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) {
      uint16_t* nb = lds + ((s + 1) & 1) * 2 * BUF;
      store_rows(nb, tid, ra);
      if (!diag) store_rows(nb + BUF, tid, rb);
    }
    __syncthreads();
  }

  float* out = a.partial + ((size_t)split * a.ntri + tile) * (size_t)(TB * TB);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 128 * wn + 32 * ni + (lane & 31);
        out[row * TB + col] = acc[mi][ni][r];
      }
  splitk_finish<TB, NTHR>(a.H, a.d, a.partial, a.ntri, a.splits, a.counters, tile, ti, tj);
}

// fp32 inputs: 64 x 64 tile per workgroup, 256 threads x (4 x 4) outputs.
struct SyrkF32Args {
  const float* X;
  int64_t ldx;
  int64_t n;
  int d;
  int ntri;
  int splits;
  int64_t kper;
  float* partial;
  unsigned int* counters;
  float* H;
};

__global__ __launch_bounds__(256) void syrk_f32_kernel(SyrkF32Args a) {
  __shared__ float sa[BKF][TF + 4];
  __shared__ float sb[BKF][TF + 4];
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j = b >> 3;
  const int tile = j % a.ntri;
  const int split = (j / a.ntri) * 8 + xcd;
  int ti, tj;
  tri_coords(tile, ti, tj);
  const int ci = ti * TF, cj = tj * TF;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t kb = (int64_t)split * a.kper;
  const int64_t ke = min(a.n, kb + a.kper);
  float acc[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += BKF) {
    // 32 x 64 elements per operand, 8 per thread
    for (int e = tid; e < BKF * TF; e += 256) {
      const int kr = e / TF, c = e % TF;
      const int64_t row = k0 + kr;
      float va = 0.f, vb = 0.f;
      if (row < ke) {
        if (ci + c < a.d) va = a.X[row * a.ldx + ci + c];
        if (cj + c < a.d) vb = a.X[row * a.ldx + cj + c];
      }
      sa[kr][c] = va;
      sb[kr][c] = vb;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < BKF; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = sa[k][ty * 4 + q];
        bv[q] = sb[k][tx * 4 + q];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(av[p], bv[q], acc[p][q]);
    }
    __syncthreads();
  }
  float* out = a.partial + ((size_t)split * a.ntri + tile) * (size_t)(TF * TF);
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) out[(ty * 4 + p) * TF + tx * 4 + q] = acc[p][q];
  splitk_finish<TF, 256>(a.H, a.d, a.partial, a.ntri, a.splits, a.counters, tile, ti, tj);
}

}  // namespace

SyrkPlan syrk_plan(int64_t d, int64_t n, int x_dtype) {
  SyrkPlan p{};
  p.tile = (x_dtype == 0) ? TB : TF;
  p.ntile = (int)ceil_div(d, p.tile);
  p.ntri = p.ntile * (p.ntile + 1) / 2;
  const int bk = (x_dtype == 0) ? BK : BKF;
  // Split the tokens so that the grid covers the 256 CUs several times over,
  // but keep each split at least 4 pipeline stages long.
  int splits = 8;
  const char* env = getenv("GPTQ_SYRK_SPLITS");
  if (env && atoi(env) > 0) {
    splits = std::max(8, (atoi(env) + 7) / 8 * 8);
  } else {
    while (splits < 64 && (int64_t)p.ntri * splits < 4 * 256 &&
           n / (2 * splits) >= 4 * bk)
      splits *= 2;
  }
  p.splits = splits;
  p.kper = std::max<int64_t>(bk, ceil_div(ceil_div(std::max<int64_t>(n, 1), splits), bk) * bk);
  p.partial_bytes = ((size_t)p.splits * p.ntri * (size_t)p.tile * p.tile * sizeof(float) + 255) &
                    ~(size_t)255;
  p.ws_bytes = p.partial_bytes + (((size_t)p.ntri * sizeof(unsigned int) + 255) & ~(size_t)255);
  return p;
}

hipError_t syrk_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n, int64_t ldx,
                       void* ws, const SyrkPlan& plan, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  float* partial = (float*)ws;
  unsigned int* counters = (unsigned int*)((char*)ws + plan.partial_bytes);
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)ceil_div(plan.ntri, 256)), dim3(256), 0,
                     stream, counters, plan.ntri);
  const int grid = plan.ntri * plan.splits;
  if (x_dtype == 0) {
    SyrkArgs a{(const uint16_t*)X, ldx, n, (int)d, plan.ntri, plan.splits, plan.kper, partial,
               counters, H};
    const bool vec = ((uintptr_t)X % 16 == 0) && (ldx % 8 == 0);
    if (vec)
      hipLaunchKernelGGL(syrk_bf16_kernel<true>, dim3(grid), dim3(NTHR), 0, stream, a);
    else
      hipLaunchKernelGGL(syrk_bf16_kernel<false>, dim3(grid), dim3(NTHR), 0, stream, a);
  } else {
    SyrkF32Args a{(const float*)X, ldx, n, (int)d, plan.ntri, plan.splits, plan.kper, partial,
                  counters, H};
    hipLaunchKernelGGL(syrk_f32_kernel, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gptq
