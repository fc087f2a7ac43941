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
// feeds four MFMAs.  K runs in chunks of 64: the chunk's X tile (128 rows x
// 128 bytes) and packed words (128 rows x 32 bytes) are loaded with coalesced
// 16-byte loads into double-buffered LDS (the next chunk's loads in flight
// while the current one multiplies; one barrier per chunk).  Within a chunk,
// MFMA kk and lane half h take k = 32 (kk / 2) + 16 h + 8 (kk % 2) + 0..7, so
// each MFMA stays inside a group of 32 and a lane's two words for MFMAs 2j,
// 2j + 1 are adjacent (one 8-byte LDS read).  Row pitches of 144 bytes (X)
// and 40 bytes (words) keep the LDS reads free of bank conflicts.
#include "common.h"
#include "kernels.h"

#include <hip/hip_fp16.h>
#include <algorithm>

namespace gptq {

namespace {

constexpr int WA_M = 128, WA_N = 128;

__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// the 8 codes of a word minus the zero, as exact bf16 integers, k order kept:
// the even codes go to the bytes of one register and the odd ones to the
// bytes of another, so each code converts to float straight from its byte
// (the empty asm keeps the masks from being folded into per-code bit-field
// extracts, so the conversions select the byte themselves), and each pair's
// two upper halves (exact: small integers) are joined with one byte permute
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w, float z) {
  uint32_t ev = w & 0x0f0f0f0fu, od = (w >> 4) & 0x0f0f0f0fu;
  asm("" : "+v"(ev), "+v"(od));
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (float)((ev >> (8 * j)) & 0xffu) - z;
    const float hi = (float)((od >> (8 * j)) & 0xffu) - z;
    // bytes 2, 3 of lo, then bytes 2, 3 of hi
    o[j] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  bf16x8 r;
  __builtin_memcpy(&r, o, sizeof(r));
  return r;
}

constexpr int WA_KCH = 64;         // k per chunk
constexpr int XP = WA_KCH + 8;     // X tile pitch (bf16 elements): 144 bytes
constexpr int WP = 10;             // word tile pitch (uint32): 8 words + 2

__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                    int M, int N, int K,
                                                    const uint32_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ S16,
                                                    const uint16_t* __restrict__ Z16, int G,
                                                    float* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][WA_M * XP];
  __shared__ __attribute__((aligned(16))) uint32_t ws[2][WA_N * WP];
  __shared__ float psz[2][WA_N][2][2];  // per column: (scale, zero) of the chunk's groups
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * WA_M, nb = blockIdx.x * WA_N, n0 = nb + 32 * wave;
  const int wpr = K / 8, ng = K / G, nch = K / WA_KCH;
  // global -> LDS: X rows tid/8 + 32 i (16 bytes at 8 (tid % 8)), word rows
  // tid/2 (16 bytes at 4 (tid % 2))
  const uint16_t* xg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xg[i] = X + (int64_t)min(m0 + (tid >> 3) + 32 * i, M - 1) * ldx + 8 * (tid & 7);
  const uint32_t* qg = Q + (int64_t)min(nb + (tid >> 1), N - 1) * wpr + 4 * (tid & 1);
  // group parameters: thread t stages column t/2, slot t%2 (the chunk's first
  // group and the next; one group per chunk unless g = 32)
  const int pcol = min(nb + (tid >> 1), N - 1), pslot = tid & 1;
  uint4 xr[4], qr;
  uint16_t sr, zr;
  auto gload = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = *(const uint4*)(xg[i] + (int64_t)c * WA_KCH);
    qr = *(const uint4*)(qg + (int64_t)c * (WA_KCH / 8));
    const int g = min(c * WA_KCH / G + pslot, ng - 1);
    sr = S16[(int64_t)pcol * ng + g];
    zr = Z16 ? Z16[(int64_t)pcol * ng + g] : (uint16_t)0;
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4*)(&xs[buf][((tid >> 3) + 32 * i) * XP + 8 * (tid & 7)]) = xr[i];
    // 8-byte stores: rows are 40 bytes apart, so 8-byte aligned
    uint2* wdst = (uint2*)(&ws[buf][(tid >> 1) * WP + 4 * (tid & 1)]);
    wdst[0] = make_uint2(qr.x, qr.y);
    wdst[1] = make_uint2(qr.z, qr.w);
    psz[buf][tid >> 1][pslot][0] = f16_bits_to_float(sr);
    psz[buf][tid >> 1][pslot][1] = Z16 ? f16_bits_to_float(zr) : 8.0f;  // sym 4-bit: 8
  };
  f32x16 tot[4], acc[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tot[mi][i] = 0.0f;
      acc[mi][i] = 0.0f;
    }
  float s = 0.0f, z = 8.0f;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) gload(c + 1);
    const uint16_t* xb = xs[buf];
    const uint32_t* wb = ws[buf] + (32 * wave + l32) * WP + 2 * h;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int k0 = c * WA_KCH + 32 * (kk >> 1) + 16 * (kk & 1);  // first k of this MFMA
      if (k0 % G == 0) {  // a group starts: its parameters, staged with the chunk
        const int slot = (k0 - c * WA_KCH) / G;
        s = psz[buf][32 * wave + l32][slot][0];
        z = psz[buf][32 * wave + l32][slot][1];
      }
      const uint32_t word = wb[4 * (kk >> 1) + (kk & 1)];
      const bf16x8 bv = dequant_word(word, z);
      const int koff = 32 * (kk >> 1) + 16 * h + 8 * (kk & 1);
      bf16x8 av[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) av[mi] = *(const bf16x8*)(xb + (32 * mi + l32) * XP + koff);
      if (k0 % G == 0) {  // a group's first products start from zero
        const f32x16 zero = {};
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mi], bv, zero, 0, 0, 0);
      } else {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mi], bv, acc[mi], 0, 0, 0);
      }
      if ((k0 + 16) % G == 0) {  // the group ends: scale it into the total
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) tot[mi][i] = fmaf(s, acc[mi][i], tot[mi][i]);
      }
    }
    if (c + 1 < nch) {
      // keep the stores of the next chunk after this chunk's products, so its
      // loads have the whole chunk to arrive
#pragma unroll
      for (int i = 0; i < 4; ++i)
        asm volatile("" : "+v"(xr[i].x), "+v"(xr[i].y), "+v"(xr[i].z), "+v"(xr[i].w));
      asm volatile("" : "+v"(qr.x), "+v"(qr.y), "+v"(qr.z), "+v"(qr.w));
      lstore(buf ^ 1);
    }
    __syncthreads();
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
