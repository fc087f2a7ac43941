// Hessian accumulation H += 2 X^T X  ("GPTQ：基于近似二阶信息的大模型权重量化",
// 阶段一: the layer Hessian is 2 X^T X over the calibration tokens).
//
// bf16 inputs: an MFMA SYRK on gfx950.  Each workgroup (4 waves) owns one
// 256 x 256 lower-triangle tile of H and one contiguous token range (split-K).
// X stages go straight from global memory into LDS (global_load_lds, 16 bytes
// per lane, no staging registers) in their natural token-major layout and are
// fed to v_mfma_f32_32x32x16_bf16 through LDS transpose reads
// (ds_read_b64_tr_b16), which deliver each lane 8 consecutive tokens of one
// column.  bf16 x bf16 products are exact in fp32; sums are fp32.
// Every workgroup writes its partial tile to a workspace; a second kernel adds
// the partials of each tile to H in split order, so results are deterministic
// and no workgroup waits on another.
//
// fp32 inputs: 64 x 64 tiles on the fp32 matrix cores (v_mfma_f32_32x32x2f32)
// with the same split-K / reduction structure.
#include "common.h"
#include "kernels.h"
#include "mfma_f32.h"

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <cmath>
#include <cstdlib>

namespace gptq {

namespace {

constexpr int TB = 256;          // bf16 output tile edge
constexpr int NTHR = 256;        // 4 waves

constexpr int TF = 64;           // fp32 output tile edge
constexpr int BKF = 32;          // fp32 tokens per stage

__device__ __forceinline__ void tri_coords(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Lower-triangle tile of workgroup slot t (0 <= t < ntp, ntp a multiple of
// 8).  Slots t = 8 i + x go to XCD x; XCD x takes ranks x ntp/8 .. + ntp/8 - 1
// of an order that walks 4 x 4 blocks of tiles (row-major over the lower
// triangle of blocks, row-major inside a block), so consecutive ranks share
// panels.  Returns false for ranks past the last tile.
__device__ __forceinline__ bool tile_of_id(int t, int ntp, int ntri, int& ti, int& tj) {
  constexpr int SBK = 4;
  const int r = (t & 7) * (ntp >> 3) + (t >> 3);
  if (r >= ntri) return false;
  const int ntile = (int)((sqrtf(8.0f * (float)ntri + 1.0f) - 1.0f) * 0.5f + 0.5f);
  const int nblk = (ntile + SBK - 1) / SBK;
  int rr = r;
  for (int bi = 0; bi < nblk; ++bi) {
    const int h = min(SBK, ntile - bi * SBK);
    for (int bj = 0; bj <= bi; ++bj) {
      const int w = min(SBK, ntile - bj * SBK);
      const int sz = (bi == bj) ? h * (h + 1) / 2 : h * w;
      if (rr < sz) {
        if (bi != bj) {
          ti = bi * SBK + rr / w;
          tj = bj * SBK + rr % w;
        } else {
          int k = 0;
          while ((k + 1) * (k + 2) / 2 <= rr) ++k;
          ti = bi * SBK + k;
          tj = bj * SBK + rr - k * (k + 1) / 2;
        }
        return true;
      }
      rr -= sz;
    }
  }
  return false;
}

struct SyrkArgs {
  const uint16_t* X;
  int64_t ldx;
  int64_t n;
  int d;
  int ntri;
  int splits;
  int vec;          // X rows 16-byte aligned (direct loads allowed)
  int64_t kper;
  float* partial;   // [splits][ntri][TB * TB]
};

// H(lower) += 2 * sum over splits of the partial tiles, in split order.
// One workgroup covers 1024 float4 of one tile; each thread keeps 4 float4
// sums and issues the loads of 4 splits (16 loads) before it adds.
template <int TILE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(float* __restrict__ H, int d,
                                                            const float* __restrict__ partial,
                                                            int ntri, int splits) {
  constexpr int F4 = TILE * TILE / 4;   // float4 per tile
  constexpr int PER_BLOCK = 1024;       // float4 per workgroup
  constexpr int BLOCKS = F4 / PER_BLOCK;
  static_assert(F4 % PER_BLOCK == 0, "tile size");
  const int tile = blockIdx.x / BLOCKS;
  const int part = blockIdx.x % BLOCKS;
  int ti, tj;
  tri_coords(tile, ti, tj);
  const float4* base = (const float4*)partial + (size_t)tile * F4 + part * PER_BLOCK + threadIdx.x;
  const size_t sstride = (size_t)ntri * F4;
  float4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  int k = 0;
  for (; k + 4 <= splits; k += 4) {
    float4 v[4][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[kk][u] = base[(size_t)(k + kk) * sstride + u * 256];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sum[u].x += v[kk][u].x;
        sum[u].y += v[kk][u].y;
        sum[u].z += v[kk][u].z;
        sum[u].w += v[kk][u].w;
      }
  }
  for (; k < splits; ++k) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = base[(size_t)k * sstride + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sum[u].x += v[u].x;
      sum[u].y += v[u].y;
      sum[u].z += v[u].z;
      sum[u].w += v[u].w;
    }
  }
  float hv[4][4];
  int gi[4], gj0[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e4 = part * PER_BLOCK + u * 256 + threadIdx.x;
    gi[u] = ti * TILE + (4 * e4) / TILE;
    gj0[u] = tj * TILE + (4 * e4) % TILE;
    const float* h = H + (int64_t)gi[u] * d + gj0[u];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      hv[u][q] = (gi[u] < d && gj0[u] + q < d && gj0[u] + q <= gi[u]) ? h[q] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float* h = H + (int64_t)gi[u] * d + gj0[u];
    const float vals[4] = {sum[u].x, sum[u].y, sum[u].z, sum[u].w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (gi[u] < d && gj0[u] + q < d && gj0[u] + q <= gi[u]) h[q] = hv[u][q] + 2.0f * vals[q];
  }
}

// ---------------------------------------------------------------------------
// bf16 SYRK main loop: three LDS stages of 48 tokens, loads issued three
// stages ahead; each wave keeps one stage of MFMA fragments in registers and
// reads the next stage's fragments while it multiplies.  Rows are stored unpadded
// (512 B) with their 16-byte units XOR-swizzled by 4*(row % 4) so the
// transpose reads of four consecutive rows fall in four different bank
// groups.  Tiles that overhang the matrix, unaligned X and a partial last
// stage take a masked register path that writes the same layout.
// ---------------------------------------------------------------------------
constexpr int ABK = 48;                  // tokens per stage
constexpr int ANS = 3;                   // LDS stages (3 x 48 KiB)
constexpr int RPW = ABK / 4;             // rows per wave per operand
constexpr int NQ = RPW / 2;              // direct loads per wave per operand
constexpr int AROW = TB * 2;             // bytes per LDS row (256 bf16)
constexpr int AOP = ABK * AROW;          // bytes per operand per stage (24 KiB)
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
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_off) {
  // base and the LDS offset are wave-uniform by construction; readfirstlane
  // lets the compiler keep them in SGPRs for the "s" operands
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const void* sbase = (const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo);
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_off);
  __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(voff), "s"(sbase), "s"(lbase)
                   : "memory", "m0");
}

// One operand of one stage.  Wave w fills rows RPW*w .. RPW*w + RPW-1 with
// wave loads of two rows each (q = 0 .. NQ-1); lane l covers row r0 + l/32,
// physical unit l%32.  The row pair's start is a wave-uniform base; the
// per-lane byte offset within the pair depends only on the swizzle phase
// (q % 2), so two offsets per operand serve every load.
struct DmaOff {
  uint32_t v[2];
};
__device__ __forceinline__ DmaOff dma_offsets(int64_t ldx, int c0, int lane) {
  DmaOff o;
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
    const int rl = lane >> 5;
    const int unit = swz_unit(2 * ph + rl, lane & 31);
    o.v[ph] = (uint32_t)(((int64_t)rl * ldx + c0 + 8 * unit) * 2);
  }
  return o;
}
// buf: LDS byte offset of the operand buffer.
__device__ __forceinline__ void async_rows(uint32_t buf, const uint16_t* __restrict__ X,
                                           int64_t ldx, int64_t k0, const DmaOff& off, int wave,
                                           int q) {
  const int r0 = RPW * wave + 2 * q;
  dma16(X + (k0 + r0) * ldx, off.v[q & 1], buf + (uint32_t)(r0 * AROW));
}
__device__ __forceinline__ void async_fill(uint32_t buf, const uint16_t* __restrict__ X,
                                           int64_t ldx, int64_t k0, const DmaOff& off, int wave) {
#pragma unroll
  for (int q = 0; q < NQ; ++q) async_rows(buf, X, ldx, k0, off, wave, q);
}

// Masked path (tile overhanging the matrix, or a partial stage): same layout.
__device__ __forceinline__ void masked_fill(char* buf, const uint16_t* __restrict__ X, int64_t ldx,
                                            int64_t k0, int64_t kend, int c0, int d, int wave,
                                            int lane) {
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r0 = RPW * wave + 2 * q;
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
  else if (n >= 6)
    __asm__ volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n >= 4)
    __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// LDS transpose read at an LDS byte address (the constant part of the
// address folds into the instruction's offset field).
__device__ __forceinline__ s16x4 lds_tr_at(uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)off);
}
__device__ __forceinline__ bf16x8 afrag_at(uint32_t off) {
  s16x4 lo = lds_tr_at(off);
  s16x4 hi = lds_tr_at(off + 4 * AROW);
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
// Direct load with M0 = lds_base + IMM (IMM a compile-time constant).
template <uint32_t IMM>
__device__ __forceinline__ void dma16_imm(const void* sbase, uint32_t voff, uint32_t lds_base) {
  __asm__ volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(voff), "s"(sbase), "s"(lds_base), "i"(IMM)
                   : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Fragments of one stage (two 16-token MFMA steps) for one wave.
struct StageFrags {
  bf16x8 a[ABK / 16][4];
  bf16x8 b[ABK / 16][4];
};

__global__ __launch_bounds__(NTHR, 1) void syrk_bf16_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[ANS * ASTAGE];
  const uint32_t lds_off = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

  // Split-major order: the workgroups resident at any time (about one per
  // CU) cover all tiles of one or two token ranges, so the XCDs stream the
  // same X rows at about the same time.  Within a range, workgroup ids are
  // handed to the 8 XCDs round-robin; tile_of_id gives each XCD a compact
  // block of tiles, so its L2 serves one fetch of a panel's rows to several
  // of its tiles.  Ids past the last tile (padding to a multiple of 8) exit.
  const int ntp = (a.ntri + 7) & ~7;
  const int split = blockIdx.x / ntp;
  int ti, tj;
  if (!tile_of_id(blockIdx.x % ntp, ntp, a.ntri, ti, tj)) return;
  const int tile = ti * (ti + 1) / 2 + tj;
  const bool diag = (ti == tj);
  const int ci = ti * TB, cj = tj * TB;
  const bool full_tile = a.vec && (ci + TB <= a.d) && (cj + TB <= a.d);

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
  const int per_stage = diag ? NQ : 2 * NQ;  // direct loads per wave per full stage
  const DmaOff offA = dma_offsets(a.ldx, ci, lane), offB = dma_offsets(a.ldx, cj, lane);

  auto stage_async = [&](int t) __attribute__((always_inline)) { return full_tile && kb + (int64_t)(t + 1) * ABK <= ke; };
  auto issue = [&](int t) __attribute__((always_inline)) {
    char* buf = lds + (t % ANS) * ASTAGE;
    const int64_t k0 = kb + (int64_t)t * ABK;
    if (stage_async(t)) {
      const uint32_t bo = lds_off + (uint32_t)((t % ANS) * ASTAGE);
      async_fill(bo, a.X, a.ldx, k0, offA, wave);
      if (!diag) async_fill(bo + AOP, a.X, a.ldx, k0, offB, wave);
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

  auto loads_of = [&](int t) __attribute__((always_inline)) { return (t < nst && stage_async(t)) ? per_stage : 0; };
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
  // One stage: publish stage s+1, then run the 48 MFMAs of stage s in six
  // groups of 8.  Each group is interleaved one-to-one with 8 of the LDS
  // reads that fetch stage s+1's fragments, and is preceded by one of the
  // six direct loads (per operand) of stage s+ANS, into the buffer stage s
  // occupied (its fragments are already in registers).  Spreading the loads
  // keeps the in-order issue of each wave from stalling on a burst of memory
  // instructions while the matrix cores sit idle.
  auto step = [&](int s, const StageFrags& cur, StageFrags& nxt) __attribute__((always_inline)) {
    { int later = 0;
#pragma unroll
      for (int t = 2; t < ANS; ++t) later += loads_of(s + t);
      wait_vm(later); }
    __syncthreads();  // everyone's part landed; every read of stage s's buffer done
    const int tn = s + ANS;
    const bool dma = tn < nst && stage_async(tn);
    if (tn < nst && !dma) issue(tn);  // masked register path
    const int64_t nk0 = kb + (int64_t)tn * ABK;
    const char* rA = lds + (min(s + 1, nst - 1) % ANS) * ASTAGE;
    const char* rB = diag ? rA : rA + AOP;
    StaticFor<0, 2 * (ABK / 16)>::run([&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value;
      constexpr int kk = g >> 1;
      if (dma) {
        const uint32_t nbo = lds_off + (uint32_t)((tn % ANS) * ASTAGE);
        async_rows(nbo, a.X, a.ldx, nk0, offA, wave, g);
        if (!diag) async_rows(nbo + AOP, a.X, a.ldx, nk0, offB, wave, g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr ((g & 1) == 0)
          nxt.a[kk][i] = afrag(rA, kk * 16 + frow, 128 * wm + 32 * i + fcol);
        else
          nxt.b[kk][i] = afrag(rB, kk * 16 + frow, 128 * wn + 32 * i + fcol);
      }
#pragma unroll
      for (int mi = 2 * (g & 1); mi < 2 * (g & 1) + 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[kk][mi], cur.b[kk][ni],
                                                               acc[mi][ni], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  for (int t = 0; t < ANS && t < nst; ++t) issue(t);
  StageFrags f0, f1;
  if (nst > 0) {
    { int later = 0;
#pragma unroll
      for (int t = 1; t < ANS; ++t) later += loads_of(t);
      wait_vm(later); }
    __syncthreads();
    read_stage(0, f0);
  }
  int s = 0;
  // Steady state of a full tile: every stage in flight is a full direct-load
  // stage.  Six steps per iteration, so the LDS slot (s % 3) and the fragment
  // set (s % 2) are compile-time constants; load addresses advance by one
  // scalar add per step, and LDS read and load destination offsets are
  // immediates on precomputed per-lane bases.
  const int nfull = full_tile ? (int)((ke - kb) / ABK) : 0;
  const bool fast = full_tile && (int64_t)(ABK * a.ldx + a.d) * 2 < ((int64_t)1 << 31);
  auto fast_loop = [&](auto DiagC, auto ModeC) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(DiagC)::value;
    // Which of the wave's 32 x 32 blocks it multiplies: 0 every block; in a
    // diagonal tile, 1 for the two quadrants on the diagonal (blocks with
    // ni <= mi, the rest lie above it) and 2 for the quadrant above the
    // diagonal (none: the wave only loads and keeps the barriers).  The
    // blocks left out lie strictly above the diagonal, which the reduction
    // never reads; under sustained matrix-core load the engine clock is
    // power-limited, so products saved there speed up the rest.
    constexpr int MODE = decltype(ModeC)::value;
    constexpr uint32_t OPB = DIAG ? 0u : (uint32_t)AOP;
    // per-lane LDS read bases of slot 1 (stage 1 is read during step 0);
    // moved to the next slot after every step
    uint32_t rdA[4], rdB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rdA[i] = lds_off + ASTAGE + aoff(frow, 128 * wm + 32 * i + fcol);
      rdB[i] = lds_off + ASTAGE + OPB + aoff(frow, 128 * wn + 32 * i + fcol);
    }
    const uint32_t rowoff = __builtin_amdgcn_readfirstlane((uint32_t)(RPW * wave * a.ldx * 2));
    const uint32_t rowstep = (uint32_t)(4 * a.ldx);  // two rows, bytes
    const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds_off + RPW * wave * AROW);
    const uint16_t* xs = a.X + (kb + (int64_t)ANS * ABK) * a.ldx;  // stage s + 3
    const int64_t xstep = (int64_t)ABK * a.ldx;
    for (; s + 6 + ANS <= nfull; s += 6) {
      StaticFor<0, 6>::run([&](auto St) __attribute__((always_inline)) {
        constexpr int st = decltype(St)::value;
        constexpr int SLOT = st % ANS, NSLOT = (st + 1) % ANS;
        static_assert(ANS == 3, "slot rotation");
        StageFrags& cur = (st % 2 == 0) ? f0 : f1;
        StageFrags& nxt = (st % 2 == 0) ? f1 : f0;
        wait_vm_n<DIAG ? NQ : 2 * NQ>();
        __syncthreads();
        const uint64_t xb = (uint64_t)(uintptr_t)xs;
        const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)xb);
        const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(xb >> 32));
        const void* sb = (const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo);
        StaticFor<0, 2 * (ABK / 16)>::run([&](auto G) __attribute__((always_inline)) {
          constexpr int g = decltype(G)::value;
          constexpr int kk = g >> 1;
          // row-pair offset of this load, kept inside the loop (hoisting the
          // twelve per-lane offsets out of it would spill them)
          uint32_t ro = rowoff + (uint32_t)g * rowstep;
          __asm__ volatile("" : "+s"(ro));
          dma16_imm<(uint32_t)(SLOT * ASTAGE + 2 * g * AROW)>(sb, offA.v[g & 1] + ro, ldsw);
          if constexpr (!DIAG)
            dma16_imm<(uint32_t)(SLOT * ASTAGE + AOP + 2 * g * AROW)>(sb, offB.v[g & 1] + ro,
                                                                       ldsw);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (MODE != 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr ((g & 1) == 0)
              nxt.a[kk][i] = afrag_at(rdA[i] + kk * 16 * AROW);
            else
              nxt.b[kk][i] = afrag_at(rdB[i] + kk * 16 * AROW);
          }
#pragma unroll
          for (int mi = 2 * (g & 1); mi < 2 * (g & 1) + 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
              if (MODE == 0 || ni <= mi)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[kk][mi], cur.b[kk][ni],
                                                                     acc[mi][ni], 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        xs += xstep;
        // next step reads slot (st + 2) % 3
        constexpr int DS = (NSLOT == ANS - 1) ? -(ANS - 1) * ASTAGE : ASTAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rdA[i] += (uint32_t)DS;
          rdB[i] += (uint32_t)DS;
          // opaque to the compiler: folding the slot rotation into the read
          // offsets would exceed the 16-bit offset field
          __asm__ volatile("" : "+v"(rdA[i]), "+v"(rdB[i]));
        }
      });
    }
  };
  if (fast && nst > 0) {
    if (!diag)
      fast_loop(std::false_type{}, std::integral_constant<int, 0>{});
    else if (wm == wn)
      fast_loop(std::true_type{}, std::integral_constant<int, 1>{});
    else if (wm < wn)
      fast_loop(std::true_type{}, std::integral_constant<int, 2>{});
    else
      fast_loop(std::true_type{}, std::integral_constant<int, 0>{});
  }
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
        __builtin_nontemporal_store(acc[mi][ni][r], out + row * TB + col);
      }
}

// fp32 inputs: 64 x 64 tile per workgroup on the fp32 matrix cores.  Each
// wave owns a 32 x 32 quadrant and accumulates v_mfma_f32_32x32x2f32 over the
// tokens two at a time: lane l supplies X[k0 + l / 32][column l % 32] of its
// row and column quadrants, straight from the LDS stage.  The row pitch of 96
// floats puts the two tokens' reads in opposite bank halves.
constexpr int PF = TF + 32;

struct SyrkF32Args {
  const float* X;
  int64_t ldx;
  int64_t n;
  int d;
  int ntri;
  int splits;
  int64_t kper;
  float* partial;
};

__global__ __launch_bounds__(256) void syrk_f32_kernel(SyrkF32Args a) {
  __shared__ float sa[BKF][PF];
  __shared__ float sb[BKF][PF];
  const int tile = blockIdx.x % a.ntri;  // split-major, as for bf16
  const int split = blockIdx.x / a.ntri;
  int ti, tj;
  tri_coords(tile, ti, tj);
  const int ci = ti * TF, cj = tj * TF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int kl = lane >> 5, cl = lane & 31;
  const int64_t kb = (int64_t)split * a.kper;
  const int64_t ke = min(a.n, kb + a.kper);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
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
#pragma unroll
    for (int k = 0; k < BKF; k += 2) {
      const float av = sa[k + kl][32 * wm + cl];
      const float bv = sb[k + kl][32 * wn + cl];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  float* out = a.partial + ((size_t)split * a.ntri + tile) * (size_t)(TF * TF);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wm + 8 * (r >> 2) + 4 * kl + (r & 3);
    const int col = 32 * wn + cl;
    out[row * TF + col] = acc[r];
  }
}


}  // namespace

// Split count: the grid is splits x ntri workgroups, about one resident per
// CU (144 KiB of LDS each), so it runs in ceil(splits * ntri / 256) rounds of
// ceil(n / splits / 48) stages.  Pick the split count that minimises rounds x
// stages plus the cost of writing and re-reading one partial tile per
// workgroup (about 0.1 stage times each, from the measured stage time and
// HBM rate), keeping every split at least four stages long.
static int pick_splits(int64_t n, int ntri, int stage, double partial_cost) {
  const int64_t max_s = std::max<int64_t>(1, std::min<int64_t>(64, n / (4 * stage)));
  int best = 1;
  double best_cost = 0.0;
  for (int s = 1; s <= max_s; ++s) {
    const double rounds = (double)ceil_div((int64_t)((ntri + 7) & ~7) * s, 256);
    const double stages = (double)ceil_div(ceil_div(n, (int64_t)s), (int64_t)stage);
    const double cost = rounds * stages + partial_cost * s * ntri;
    if (s == 1 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// ---- the allocation-free entry point's scratch ------------------------------
// A fixed array in the code object: each GPU the library runs on holds its own
// copy from the library's load until the process ends.  In host code the
// name is only a stand-in; the device address comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept here.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t syrk_scratch(void** ptr) {
  static std::mutex mu;
  static void* cached[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cached[dev] = p;
  }
  *ptr = cached[dev];
  return hipSuccess;
}

SyrkPlan syrk_plan_capped(int64_t d, int64_t n, int x_dtype, size_t max_bytes) {
  SyrkPlan p = syrk_plan(d, n, x_dtype);
  const size_t per_split = (size_t)p.ntri * (size_t)p.tile * p.tile * sizeof(float);
  const int64_t fit = (int64_t)(max_bytes / per_split);
  if (fit < 1) {
    p.splits = 0;  // does not fit even one split
    return p;
  }
  if (p.splits > fit) {
    const int bk = (x_dtype == 0) ? ABK : BKF;
    p.splits = (int)fit;
    p.kper = std::max<int64_t>(bk, ceil_div(ceil_div(std::max<int64_t>(n, 1), p.splits), bk) * bk);
    p.partial_bytes = (p.splits * per_split + 255) & ~(size_t)255;
    p.ws_bytes = p.partial_bytes;
  }
  return p;
}

SyrkPlan syrk_plan(int64_t d, int64_t n, int x_dtype) {
  SyrkPlan p{};
  p.tile = (x_dtype == 0) ? TB : TF;
  p.ntile = (int)ceil_div(d, p.tile);
  p.ntri = p.ntile * (p.ntile + 1) / 2;
  const int bk = (x_dtype == 0) ? ABK : BKF;
  // fp32 tiles are small (many workgroups per CU): weigh partials lightly.
  p.splits = pick_splits(std::max<int64_t>(n, 1), p.ntri, bk, (x_dtype == 0) ? 0.1 : 0.01);
  p.kper = std::max<int64_t>(bk, ceil_div(ceil_div(std::max<int64_t>(n, 1), p.splits), bk) * bk);
  p.partial_bytes = ((size_t)p.splits * p.ntri * (size_t)p.tile * p.tile * sizeof(float) + 255) &
                    ~(size_t)255;
  p.ws_bytes = p.partial_bytes;
  return p;
}

hipError_t syrk_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n, int64_t ldx,
                       void* ws, const SyrkPlan& plan, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  float* partial = (float*)ws;
  const int grid = plan.ntri * plan.splits;
  if (x_dtype == 0) {
    // direct loads: 16-byte aligned rows, and per-lane byte offsets within a
    // row pair (< 2 ldx + d elements) that fit the 32-bit offset operand
    const int vec = ((uintptr_t)X % 16 == 0) && (ldx % 8 == 0) &&
                    (2 * ldx + d) * 2 < ((int64_t)1 << 31);
    SyrkArgs a{(const uint16_t*)X, ldx, n, (int)d, plan.ntri, plan.splits, vec, plan.kper, partial};
    const int ntp = (plan.ntri + 7) & ~7;
    hipLaunchKernelGGL(syrk_bf16_kernel, dim3(ntp * plan.splits), dim3(NTHR), 0, stream, a);
    hipLaunchKernelGGL(splitk_reduce_kernel<TB>, dim3(plan.ntri * (TB * TB / 4 / 1024)), dim3(256),
                       0, stream, H, (int)d, partial, plan.ntri, plan.splits);
  } else {
    SyrkF32Args a{(const float*)X, ldx, n, (int)d, plan.ntri, plan.splits, plan.kper, partial};
    hipLaunchKernelGGL(syrk_f32_kernel, dim3(grid), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(splitk_reduce_kernel<TF>, dim3(plan.ntri * (TF * TF / 4 / 1024)), dim3(256),
                       0, stream, H, (int)d, partial, plan.ntri, plan.splits);
  }
  return hipGetLastError();
}

}  // namespace gptq
