// Dequantized product with the packed 4-bit weights (W4A16):
//   Y[m][n] = sum_k X[m][k] W_hat[n][k],  W_hat[n][k] = s[n][k/g] (q[n][k] - z[n][k/g])
// ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段三: inference uses the integer
// codes with per-group scale and zero; "GPTQ/AWQ量化中Group Size的精确含义与计算",
// 存储代价: 16-bit scale and zero per group of g columns).  X is bf16, Y fp32.
//
// v_mfma_f32_32x32x16_bf16 takes, per lane l, 8 consecutive k of one row
// (l % 32) of each operand (k = 8 (l / 32) ...): for X that is 16 bytes of a
// row, and for W it is exactly one uint32 word of the packed row (8 codes,
// little-endian nibbles), so neither operand goes through LDS.  The word is
// turned into the 8 integers q - z as bf16, which are exact (|q - z| <= 15),
// so every product x (q - z) is exact in fp32; a group's products accumulate
// on their own and are then scaled, tot += s * acc_g, with s the lane's
// column's binary16 scale.  Only fp32 accumulation rounds.
//
// Tile: 128 (M) x 128 (N) per workgroup; wave w owns columns 32 w .. 32 w + 31
// of it and all 128 rows, as four 32 x 32 blocks, so each dequantized word
// feeds four MFMAs.  K runs in chunks of 4 steps of 16, the next chunk's
// operands loaded while the current one multiplies.
#include "common.h"
#include "kernels.h"

#include <hip/hip_fp16.h>
#include <algorithm>

namespace gptq {

namespace {

constexpr int WA_M = 128, WA_N = 128;
constexpr int WA_KC = 4;  // k-steps (of 16) per chunk

__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// the 8 codes of a word minus the zero, as exact bf16 integers, k order kept
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w, float z) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (float)((w >> (8 * j)) & 15u) - z;
    const float hi = (float)((w >> (8 * j + 4)) & 15u) - z;
    o[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  bf16x8 r;
  __builtin_memcpy(&r, o, sizeof(r));
  return r;
}

__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                    int M, int N, int K,
                                                    const uint32_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ S16,
                                                    const uint16_t* __restrict__ Z16, int G,
                                                    float* __restrict__ Y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * WA_M, n0 = blockIdx.x * WA_N + 32 * wave;
  const int wpr = K / 8, ng = K / G, gsteps = G / 16, nsteps = K / 16;
  const int n = min(n0 + l32, N - 1);
  const uint32_t* qrow = Q + (int64_t)n * wpr + h;
  const uint16_t* xrow[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    xrow[mi] = X + (int64_t)min(m0 + 32 * mi + l32, M - 1) * ldx + 8 * h;
  f32x16 tot[4], acc[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tot[mi][i] = 0.0f;
      acc[mi][i] = 0.0f;
    }
  struct Ops {
    bf16x8 a[WA_KC][4];
    uint32_t b[WA_KC];
  };
  auto load = [&](Ops& o, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < WA_KC; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) o.a[kk][mi] = *(const bf16x8*)(xrow[mi] + 16 * (ks + kk));
      o.b[kk] = qrow[2 * (ks + kk)];
    }
  };
  // the lane's column's scale and zero, one group ahead
  const uint16_t* srow = S16 + (int64_t)n * ng;
  const uint16_t* zrow = Z16 ? Z16 + (int64_t)n * ng : nullptr;
  uint16_t s_b = srow[0], z_b = zrow ? zrow[0] : 0;
  uint16_t s_nb = srow[min(1, ng - 1)], z_nb = zrow ? zrow[min(1, ng - 1)] : 0;
  float s = 0.0f, z = 8.0f;  // symmetric 4-bit: z = (maxq + 1) / 2
  // one chunk: multiply c (steps ks ..), having started the loads of the
  // next chunk into nx
  auto chunk = [&](Ops& c, Ops& nx, int ks) __attribute__((always_inline)) {
    if (ks + WA_KC < nsteps) load(nx, ks + WA_KC);
#pragma unroll
    for (int kk = 0; kk < WA_KC; ++kk) {
      const int step = ks + kk;
      if (step % gsteps == 0) {  // a group starts: take its parameters, fetch a later one's
        const int g = step / gsteps;
        s = f16_bits_to_float(s_b);
        if (zrow) z = f16_bits_to_float(z_b);
        s_b = s_nb;
        z_b = z_nb;
        const int gn = min(g + 2, ng - 1);
        s_nb = srow[gn];
        if (zrow) z_nb = zrow[gn];
      }
      const bf16x8 bv = dequant_word(c.b[kk], z);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.a[kk][mi], bv, acc[mi], 0, 0, 0);
      if ((step + 1) % gsteps == 0) {  // the group ends: scale it into the total
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            tot[mi][i] = fmaf(s, acc[mi][i], tot[mi][i]);
            acc[mi][i] = 0.0f;
          }
      }
    }
  };
  Ops o0, o1;
  load(o0, 0);
  for (int ks = 0; ks < nsteps; ks += 2 * WA_KC) {
    chunk(o0, o1, ks);
    if (ks + WA_KC < nsteps) chunk(o1, o0, ks + WA_KC);
  }
  const int col = n0 + l32;
  if (col >= N) return;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + 32 * mi + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < M) Y[(int64_t)row * N + col] = tot[mi][i];
    }
}

}  // namespace

hipError_t w4a16_launch(const void* X, int64_t m, int64_t ldx, const uint32_t* qweight,
                        const uint16_t* scales_f16, const uint16_t* zeros_f16, int64_t d_out,
                        int64_t d_in, int group_size, float* Y, hipStream_t stream) {
  const int G = group_size == -1 ? (int)d_in : group_size;
  const dim3 grid((unsigned)ceil_div(d_out, WA_N), (unsigned)ceil_div(m, WA_M));
  hipLaunchKernelGGL(w4a16_kernel, grid, dim3(256), 0, stream, (const uint16_t*)X, ldx, (int)m,
                     (int)d_out, (int)d_in, qweight, scales_f16, zeros_f16, G, Y);
  return hipGetLastError();
}

}  // namespace gptq
