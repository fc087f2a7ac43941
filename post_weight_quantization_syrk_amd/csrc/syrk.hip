// Hessian accumulation H += 2 X^T X  ("GPTQ：基于近似二阶信息的大模型权重量化",
// 阶段一: the layer Hessian is 2 X^T X over the calibration tokens).
//
// bf16 inputs: an MFMA SYRK on gfx950.  Each workgroup (4 waves) owns one
// 256 x 256 lower-triangle tile of H and one contiguous token range (split-K);
// X tiles are staged through LDS in their natural token-major layout and fed
// to v_mfma_f32_32x32x16_bf16 through LDS transpose reads
// (ds_read_b64_tr_b16), which deliver each lane 8 consecutive tokens of one
// column.  bf16 x bf16 products are exact in fp32; sums are fp32.
// Each token range (split) is pinned to one XCD: its X rows are fetched by that
// XCD only and shared through its L2 by the tiles resident there.
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
  constexpr int PER = 4;  // float4 chunks per thread per pass, loads issued together
  for (int e0 = threadIdx.x; e0 < TSZ / 4; e0 += NT * PER) {
    float4 sum[PER];
    float hv[PER][4];
    int gi[PER], gj0[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e4 = e0 + u * NT;
      const int r = (4 * e4) / TILE, c0 = (4 * e4) % TILE;
      gi[u] = ti * TILE + r;
      gj0[u] = tj * TILE + c0;
      sum[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      const bool live = e4 < TSZ / 4 && gi[u] < d && gj0[u] < d && gj0[u] <= gi[u];
      if (!live) gi[u] = -1;
    }
    for (int k = 0; k < splits; ++k) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        if (gi[u] < 0) continue;
        const float4 v = base[(size_t)k * sstride + e0 + u * NT];
        sum[u].x += v.x;
        sum[u].y += v.y;
        sum[u].z += v.z;
        sum[u].w += v.w;
      }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (gi[u] < 0) continue;
      const float* h = H + (int64_t)gi[u] * d + gj0[u];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        hv[u][q] = (gj0[u] + q < d && gj0[u] + q <= gi[u]) ? h[q] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (gi[u] < 0) continue;
      float* h = H + (int64_t)gi[u] * d + gj0[u];
      const float vals[4] = {sum[u].x, sum[u].y, sum[u].z, sum[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (gj0[u] + q < d && gj0[u] + q <= gi[u]) h[q] = hv[u][q] + 2.0f * vals[q];
    }
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
  if (VEC && k0 + BK <= kend && c0 + TB <= d) {
    // Whole stage inside the matrix (the common case): eight unconditional
    // 16-byte loads, all in flight together.
    const uint16_t* src = X + (k0 + (tid >> 5)) * ldx + col;
#pragma unroll
    for (int r = 0; r < 8; ++r) reg[r] = *(const uint4*)(src + (int64_t)r * 8 * ldx);
    return;
  }
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

  // Workgroups are handed to the 8 XCDs round-robin, so consecutive ids are on
  // different XCDs.  Token range `split` is pinned to XCD split % 8: every X
  // row is fetched by one XCD only, and the tiles resident on that XCD stream
  // the same rows through its L2 at about the same time.
  const int xcd = blockIdx.x & 7;
  const int jj = blockIdx.x >> 3;
  const int tile = jj % a.ntri;
  const int split = (jj / a.ntri) * 8 + xcd;
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

  // One register stage in flight: stage s+1 is fetched into registers while
  // stage s is multiplied out of LDS, then written to the other LDS buffer.
  // (A second register stage does not fit beside the 256 accumulator
  // registers without spilling.)
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

// ---------------------------------------------------------------------------
// Pipelined variant: X stages go straight from global memory into LDS
// (global_load_lds, 16 bytes per lane) with no staging registers, four LDS
// stages of 32 tokens, loads issued four stages ahead; each wave keeps one
// stage of MFMA fragments in registers and reads the next stage's fragments
// while it multiplies.  Rows are stored
// unpadded (512 B) with their 16-byte units XOR-swizzled by 4*(row % 4) so the
// transpose reads of four consecutive rows fall in four different bank
// groups.  Tiles that overhang the matrix and a partial last stage take a
// masked register path that writes the same layout.
// ---------------------------------------------------------------------------
constexpr int ABK = 32;                  // tokens per stage
constexpr int ANS = 4;                   // LDS stages
constexpr int AROW = TB * 2;             // bytes per LDS row (256 bf16)
constexpr int AOP = ABK * AROW;          // bytes per operand per stage (16 KiB)
constexpr int ASTAGE = 2 * AOP;          // bytes per stage (A and B)

__device__ __forceinline__ int swz_unit(int row, int unit) { return unit ^ (4 * (row & 3)); }

// Byte offset in an operand buffer of the 8-byte chunk (row, col..col+3).
__device__ __forceinline__ int aoff(int row, int col) {
  return row * AROW + swz_unit(row, col >> 3) * 16 + (col & 7) * 2;
}

__device__ __forceinline__ bf16x8 afrag(const char* buf, int row, int col) {
  s16x4 lo = lds_read_tr16(buf + aoff(row, col));
  s16x4 hi = lds_read_tr16(buf + aoff(row + 4, col));
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds + 16 l (M0 holds the wave-uniform LDS base).  Written in asm rather
// than with the compiler builtin: the compiler tracks builtin LDS-DMA writes
// with one conservative counter and would wait for every load in flight
// (vmcnt(0)) before any LDS read, which serialises the stage pipeline.  The
// asm has no output registers; completion is awaited explicitly (wait_vm)
// before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* src, char* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "s"(base)
                   : "memory", "m0");
}

// One operand of one stage.  Wave w fills rows 8w..8w+7 (two rows per 1 KiB
// wave load); lane l covers row r0 + l/32, physical unit l%32.
__device__ __forceinline__ void async_fill(char* buf, const uint16_t* __restrict__ X, int64_t ldx,
                                           int64_t k0, int c0, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = 8 * wave + 2 * q;
    const int row = r0 + (lane >> 5);
    const int unit = swz_unit(row, lane & 31);
    const uint16_t* src = X + (k0 + row) * ldx + c0 + 8 * unit;
    dma16(src, buf + r0 * AROW);
  }
}

// Masked path (tile overhanging the matrix, or a partial stage): same layout.
__device__ __forceinline__ void masked_fill(char* buf, const uint16_t* __restrict__ X, int64_t ldx,
                                            int64_t k0, int64_t kend, int c0, int d, int wave,
                                            int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = 8 * wave + 2 * q;
    const int row = r0 + (lane >> 5);
    const int unit = swz_unit(row, lane & 31);
    const int col = c0 + 8 * unit;
    const int64_t grow = k0 + row;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (grow < kend) {
      const uint16_t* src = X + grow * ldx + col;
      for (int e = 0; e < 8; ++e)
        if (col + e < d) w[e >> 1] |= ((uint32_t)src[e]) << (16 * (e & 1));
    }
    *(uint4*)(buf + r0 * AROW + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ void wait_vm(int n) {
  // Wait until at most n of this wave's direct loads are outstanding (n is
  // wave-uniform; rounded down to the next supported count, which only waits
  // longer).
  if (n >= 24)
    __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (n >= 16)
    __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 12)
    __asm__ volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n >= 8)
    __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 4)
    __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Fragments of one stage (two 16-token MFMA steps) for one wave.
struct StageFrags {
  bf16x8 a[ABK / 16][4];
  bf16x8 b[ABK / 16][4];
};

__global__ __launch_bounds__(NTHR, 1) void syrk_bf16_async_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[ANS * ASTAGE];

  const int xcd = blockIdx.x & 7;
  const int jj = blockIdx.x >> 3;
  const int tile = jj % a.ntri;
  const int split = (jj / a.ntri) * 8 + xcd;
  int ti, tj;
  tri_coords(tile, ti, tj);
  const bool diag = (ti == tj);
  const int ci = ti * TB, cj = tj * TB;
  const bool full_tile = (ci + TB <= a.d) && (cj + TB <= a.d);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, i16 = lane & 15;
  const int frow = 8 * (g >> 1) + (i16 >> 2);      // fragment row within a 16-token step
  const int fcol = 16 * (g & 1) + 4 * (i16 & 3);   // fragment column offset

  const int64_t kb = (int64_t)split * a.kper;
  const int64_t ke = min(a.n, kb + a.kper);
  const int nst = (ke > kb) ? (int)ceil_div(ke - kb, ABK) : 0;
  const int per_stage = diag ? 4 : 8;  // direct loads per wave per full stage

  auto stage_async = [&](int t) { return full_tile && kb + (int64_t)(t + 1) * ABK <= ke; };
  auto issue = [&](int t) {
    char* buf = lds + (t % ANS) * ASTAGE;
    const int64_t k0 = kb + (int64_t)t * ABK;
    if (stage_async(t)) {
      async_fill(buf, a.X, a.ldx, k0, ci, wave, lane);
      if (!diag) async_fill(buf + AOP, a.X, a.ldx, k0, cj, wave, lane);
    } else {
      masked_fill(buf, a.X, a.ldx, k0, ke, ci, a.d, wave, lane);
      if (!diag) masked_fill(buf + AOP, a.X, a.ldx, k0, ke, cj, a.d, wave, lane);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto loads_of = [&](int t) { return (t < nst && stage_async(t)) ? per_stage : 0; };
  auto read_stage = [&](int t, StageFrags& f) __attribute__((always_inline)) {
    const char* bufA = lds + (t % ANS) * ASTAGE;
    const char* bufB = diag ? bufA : bufA + AOP;
#pragma unroll
    for (int kk = 0; kk < ABK / 16; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        f.a[kk][mi] = afrag(bufA, kk * 16 + frow, 128 * wm + 32 * mi + fcol);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        f.b[kk][ni] = afrag(bufB, kk * 16 + frow, 128 * wn + 32 * ni + fcol);
    }
  };
  // One stage: publish stage s+1, start loading stage s+ANS into the buffer
  // stage s occupied (its fragments are already in registers), then run the
  // 32 MFMAs of stage s interleaved one-to-one with the 32 LDS reads that
  // fetch stage s+1's fragments.
  auto step = [&](int s, const StageFrags& cur, StageFrags& nxt) __attribute__((always_inline)) {
    wait_vm(loads_of(s + 2) + loads_of(s + 3));  // own part of stage s+1 landed
    __syncthreads();  // everyone's part landed; every read of stage s's buffer done
    if (s + ANS < nst) issue(s + ANS);
    read_stage(min(s + 1, nst - 1), nxt);
#pragma unroll
    for (int kk = 0; kk < ABK / 16; ++kk)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[kk][mi], cur.b[kk][ni],
                                                               acc[mi][ni], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * (ABK / 16) * 16; i += 2) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  for (int t = 0; t < ANS && t < nst; ++t) issue(t);
  StageFrags f0, f1;
  if (nst > 0) {
    wait_vm(loads_of(1) + loads_of(2) + loads_of(3));
    __syncthreads();
    read_stage(0, f0);
  }
  int s = 0;
  for (; s + 1 < nst; s += 2) {
    step(s, f0, f1);
    step(s + 1, f1, f0);
  }
  if (s < nst) step(s, f0, f1);

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
  // Workgroups are handed to the 8 XCDs round-robin, so consecutive ids are on
  // different XCDs.  Token range `split` is pinned to XCD split % 8: every X
  // row is fetched by one XCD only, and the tiles resident on that XCD stream
  // the same rows through its L2 at about the same time.
  const int xcd = blockIdx.x & 7;
  const int jj = blockIdx.x >> 3;
  const int tile = jj % a.ntri;
  const int split = (jj / a.ntri) * 8 + xcd;
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
  // Split the tokens so that the grid covers the 256 CUs about 4 times over
  // (one workgroup per CU; a fractional last wave then costs little), but
  // keep each split at least 4 pipeline stages long.  More splits cost more
  // partial-tile traffic than they gain in balance (measured at d = 4096).
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
    const char* kenv = getenv("GPTQ_SYRK_KERNEL");  // "staged": register-staged variant
    const bool staged = kenv && kenv[0] == 's';
    if (vec && !staged)
      hipLaunchKernelGGL(syrk_bf16_async_kernel, dim3(grid), dim3(NTHR), 0, stream, a);
    else if (vec)
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
