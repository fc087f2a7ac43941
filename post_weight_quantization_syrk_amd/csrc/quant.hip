// Greedy column-by-column quantization with error feedback and lazy batched
// trailing updates ("GPTQ：基于近似二阶信息的大模型权重量化", 阶段二 and
// 量化误差与补偿; group-wise scales and zero points after 对称与仿射量化 and
// "GPTQ/AWQ量化中Group Size的精确含义与计算", 存储代价 / 小 group 买到了什么).
//
// Per block of 128 columns:
//   colloop  : 16 lanes share one row, each lane holding 8 consecutive columns
//              of the row in registers; the 128 x 128 block of U sits in LDS.
//              Column j's value is broadcast inside the 16-lane row group
//              (DPP row broadcast), every lane takes the same rounding decision,
//              and each lane applies the feedback to its own 8 columns.  Group
//              min/max come from a 16-lane butterfly at the group's first column.
//   trailing : W[:, next blocks] -= Err_blk U[blk, next blocks], an fp32 MFMA
//              GEMM (v_mfma_f32_32x32x2f32), K = 128.
#include "common.h"
#include "kernels.h"

#include <hip/hip_fp16.h>
#include <algorithm>

namespace gptq {

namespace {

constexpr int QB = 128;      // block width (columns)
constexpr int UPITCH = 132;  // LDS pitch (floats) of the U block in the column loop

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct QuantWs {
  float* Wc;   // [d_out x d_in] working copy
  float* Err;  // [d_out x d_in] scaled errors delta
};

QuantWs carve(void* ws, int64_t d_out, int64_t d_in) {
  QuantWs w;
  const size_t m = align256((size_t)d_out * d_in * sizeof(float));
  w.Wc = (float*)ws;
  w.Err = (float*)((char*)ws + m);
  return w;
}

// One rounding of a positive float64 to binary16, nearest-even.  Returns the
// binary16 value as a float64 (0 when it underflows, +inf on overflow).
__device__ __forceinline__ double f64_to_f16_value(double x) {
  if (!(x > 0.0)) return 0.0;
  int e;
  (void)frexp(x, &e);            // x = m * 2^e, m in [0.5, 1)
  int ulp_exp = (e - 1) - 10;    // binary16 ulp exponent for normal numbers
  if (ulp_exp < -24) ulp_exp = -24;  // subnormal range: ulp = 2^-24
  const double q = ldexp(x, -ulp_exp);
  const double r = rint(q);
  const double v = ldexp(r, ulp_exp);
  return (v >= 65520.0) ? __builtin_inf() : v;
}

__global__ __launch_bounds__(256) void qinit_kernel(const void* __restrict__ W, int w_dtype,
                                                    int64_t d_out, int64_t d_in,
                                                    const uint8_t* __restrict__ dead,
                                                    float* __restrict__ Wc) {
  const int64_t total = d_out * d_in;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t c = e % d_in;
    float v = (w_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)W)[e]) : ((const float*)W)[e];
    if (dead && dead[c]) v = 0.0f;
    Wc[e] = v;
  }
}

struct GroupParams {
  float s, inv_s, hs, z;
};

template <int BITS, bool SYM>
__device__ __forceinline__ GroupParams make_params(float lo_or_amax, float hi) {
  constexpr int maxq = (1 << BITS) - 1;
  GroupParams p;
  double s;
  float z;
  if (SYM) {
    const double amax = (double)lo_or_amax;
    s = f64_to_f16_value(2.0 * amax / (double)maxq);
    z = (float)((maxq + 1) / 2);
    if (!(amax > 0.0) || !(s > 0.0)) s = 1.0;
  } else {
    const double lo = (double)lo_or_amax, h = (double)hi;
    s = f64_to_f16_value((h - lo) / (double)maxq);
    if (h > lo && s > 0.0) {
      double zz = rint(-lo / s);
      zz = zz < 0.0 ? 0.0 : (zz > (double)maxq ? (double)maxq : zz);
      z = (float)zz;
    } else {
      s = 1.0;
      z = 0.0f;
    }
  }
  p.s = (float)s;
  p.inv_s = 1.0f / p.s;
  p.hs = 0.5f * p.s;
  p.z = z;
  return p;
}

// Nearest integer to the exact quotient x/s, ties to even, then code clamp.
template <int BITS>
__device__ __forceinline__ float quantize_code(float x, const GroupParams& p) {
  constexpr float maxq = (float)((1 << BITS) - 1);
  float q0 = rintf(x * p.inv_s);
  q0 = fminf(fmaxf(q0, -2047.0f), 2047.0f);
  const float up = fmaf(q0, p.s, p.hs);    // (q0 + 1/2) s, exact
  const float dn = fmaf(q0, p.s, -p.hs);   // (q0 - 1/2) s, exact
  const bool odd = (((int)q0) & 1) != 0;
  if (x > up || (x == up && odd))
    q0 += 1.0f;
  else if (x < dn || (x == dn && odd))
    q0 -= 1.0f;
  return fminf(fmaxf(q0 + p.z, 0.0f), maxq);
}

// g = -1: one group per row from the whole (current = original) row.
template <int BITS, bool SYM>
__global__ __launch_bounds__(256) void rowparams_kernel(const float* __restrict__ Wc,
                                                        int64_t d_out, int64_t d_in,
                                                        float* __restrict__ scales,
                                                        float* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const float* w = Wc + row * d_in;
  float mn = 0.0f, mx = 0.0f;  // the range always contains 0
  for (int64_t c = lane; c < d_in; c += 64) {
    const float v = w[c];
    if (SYM) {
      mx = fmaxf(mx, fabsf(v));
    } else {
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (lane == 0) {
    const GroupParams p = SYM ? make_params<BITS, true>(mx, 0.0f) : make_params<BITS, false>(mn, mx);
    scales[row] = p.s;
    zeros[row] = p.z;
  }
}

// Broadcast lane `src` (0..15) of each 16-lane row to the whole row.
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + SRC, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_min(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fminf(v, __shfl_xor(v, m, 16));
  return v;
}
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 16));
  return v;
}

template <int J>
struct BcastAt {
  static __device__ __forceinline__ float get(const float (&w)[8]) {
    return row_bcast<J / 8>(w[J % 8]);
  }
};

// G = 0 means one group per row with parameters precomputed by rowparams_kernel.
template <int BITS, int G, bool SYM>
__global__ __launch_bounds__(256) void colloop_kernel(
    float* __restrict__ Wc, float* __restrict__ Err, const float* __restrict__ U,
    int64_t d_out, int64_t d_in, int64_t b0, uint8_t* __restrict__ codes,
    float* __restrict__ scales, float* __restrict__ zeros, float* __restrict__ loss_rows,
    int n_groups) {
  __shared__ __attribute__((aligned(16))) float us[QB * UPITCH];
  __shared__ float invd[QB];
  const int tid = threadIdx.x;
  const int bw = (int)min<int64_t>(QB, d_in - b0);
  // U block: upper triangle only, identity padding past the matrix edge.
  for (int e = tid; e < QB * QB; e += 256) {
    const int r = e >> 7, c = e & 127;
    float v;
    if (r < bw && c < bw)
      v = (c >= r) ? U[(b0 + r) * d_in + b0 + c] : 0.0f;
    else
      v = (r == c) ? 1.0f : 0.0f;
    us[r * UPITCH + c] = v;
  }
  __syncthreads();
  if (tid < QB) invd[tid] = 1.0f / us[tid * UPITCH + tid];
  __syncthreads();

  const int c = tid & 15;                  // lane within the row group
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool live = row < d_out;
  const int64_t rr = live ? row : 0;
  float w[8];
  {
    const float* src = Wc + rr * d_in + b0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (8 * c + i < bw && live) ? src[i] : 0.0f;
  }
  GroupParams gp;
  if (G == 0) {
    gp = make_params<BITS, SYM>(0.0f, 0.0f);
    gp.s = scales[rr];
    gp.inv_s = 1.0f / gp.s;
    gp.hs = 0.5f * gp.s;
    gp.z = zeros[rr];
  }
  float cr[8], er[8];
  float loss = 0.0f;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (j >= bw) continue;
    if (G > 0 && (j % (G > 0 ? G : 1)) == 0) {
      const bool mine = (8 * c >= j) && (8 * c < j + G);
      float mn = 0.0f, mx = 0.0f;
      if (mine) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (SYM) {
            mx = fmaxf(mx, fabsf(w[i]));
          } else {
            mn = fminf(mn, w[i]);
            mx = fmaxf(mx, w[i]);
          }
        }
      }
      mx = row_max(mx);
      if (!SYM) mn = row_min(mn);
      gp = SYM ? make_params<BITS, true>(mx, 0.0f) : make_params<BITS, false>(mn, mx);
      if (c == (j >> 3) && live) {
        const int64_t gi = rr * n_groups + (b0 + j) / G;
        scales[gi] = gp.s;
        zeros[gi] = gp.z;
      }
    }
    float x;
    switch (j >> 3) {
      case 0: x = row_bcast<0>(w[j & 7]); break;
      case 1: x = row_bcast<1>(w[j & 7]); break;
      case 2: x = row_bcast<2>(w[j & 7]); break;
      case 3: x = row_bcast<3>(w[j & 7]); break;
      case 4: x = row_bcast<4>(w[j & 7]); break;
      case 5: x = row_bcast<5>(w[j & 7]); break;
      case 6: x = row_bcast<6>(w[j & 7]); break;
      case 7: x = row_bcast<7>(w[j & 7]); break;
      case 8: x = row_bcast<8>(w[j & 7]); break;
      case 9: x = row_bcast<9>(w[j & 7]); break;
      case 10: x = row_bcast<10>(w[j & 7]); break;
      case 11: x = row_bcast<11>(w[j & 7]); break;
      case 12: x = row_bcast<12>(w[j & 7]); break;
      case 13: x = row_bcast<13>(w[j & 7]); break;
      case 14: x = row_bcast<14>(w[j & 7]); break;
      default: x = row_bcast<15>(w[j & 7]); break;
    }
    const float code = quantize_code<BITS>(x, gp);
    const float what = gp.s * (code - gp.z);
    const float delta = (x - what) * invd[j];
    loss = fmaf(delta, delta, loss);
    if (c == (j >> 3)) {
      cr[j & 7] = code;
      er[j & 7] = delta;
    }
    const float* urow = us + j * UPITCH + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = fmaf(-delta, urow[i], w[i]);
  }
  if (!live) return;
  // codes and scaled errors of this lane's 8 columns
  uint8_t* cdst = codes + rr * d_in + b0 + 8 * c;
  float* edst = Err + rr * d_in + b0 + 8 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (8 * c + i < bw) {
      cdst[i] = (uint8_t)cr[i];
      edst[i] = er[i];
    }
  }
  if (loss_rows && c == 0) loss_rows[rr] = (b0 == 0 ? 0.0f : loss_rows[rr]) + loss;
}

// Wc[:, n0:] -= Err[:, b0:b0+kb] * U[b0:b0+kb, n0:]   (fp32 MFMA, 128 x 128 tiles)
__global__ __launch_bounds__(256) void trailing_kernel(float* __restrict__ Wc,
                                                       const float* __restrict__ Err,
                                                       const float* __restrict__ U,
                                                       int64_t d_out, int64_t d_in, int64_t b0,
                                                       int kb, int64_t n0) {
  constexpr int T = 128;
  // sa[k][m] = Err[m0+m][b0+k], sb[k][n] = U[b0+k][n0t+n]; odd k rows are stored
  // with column index ^ 32 so the two 32-lane halves of an MFMA operand read
  // (rows k and k+1) fall in different LDS banks.
  __shared__ float sa[QB][T];
  __shared__ float sb[QB][T];
  const int64_t ncols = d_in - n0;
  const int ntn = (int)ceil_div(ncols, T);
  const int64_t m0 = (int64_t)(blockIdx.x / ntn) * T;
  const int64_t n0t = n0 + (int64_t)(blockIdx.x % ntn) * T;
  const int tid = threadIdx.x;
  for (int e = tid; e < T * QB; e += 256) {
    const int m = e >> 7, k = e & 127;  // consecutive threads: consecutive k
    const int64_t gm = m0 + m;
    sa[k][m ^ ((k & 1) << 5)] = (gm < d_out && k < kb) ? Err[gm * d_in + b0 + k] : 0.0f;
  }
  for (int e = tid; e < QB * T; e += 256) {
    const int k = e >> 7, n = e & 127;
    const int64_t gn = n0t + n;
    sb[k][n ^ ((k & 1) << 5)] = (k < kb && gn < d_in) ? U[(b0 + k) * d_in + gn] : 0.0f;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  const int kl = lane >> 5, ml = lane & 31;
#pragma unroll 4
  for (int k = 0; k < QB; k += 2) {
    float av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) av[a] = sa[k + kl][(64 * wm + 32 * a + ml) ^ (kl << 5)];
#pragma unroll
    for (int b = 0; b < 2; ++b) bv[b] = sb[k + kl][(64 * wn + 32 * b + ml) ^ (kl << 5)];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t gn = n0t + 64 * wn + 32 * b + (lane & 31);
        if (gm < d_out && gn < d_in) {
          float* p = Wc + gm * d_in + gn;
          *p = *p - acc[a][b][r];
        }
      }
}

template <int BITS, int G, bool SYM>
hipError_t run_quant(float* Wc, float* Err, const float* U, int64_t d_out, int64_t d_in,
                     uint8_t* codes, float* scales, float* zeros, float* loss_rows,
                     int n_groups, hipStream_t stream) {
  if (G == 0)
    hipLaunchKernelGGL((rowparams_kernel<BITS, SYM>), dim3((unsigned)ceil_div(d_out, 4)),
                       dim3(256), 0, stream, (const float*)Wc, d_out, d_in, scales, zeros);
  const unsigned rgrid = (unsigned)ceil_div(d_out, 16);
  for (int64_t b0 = 0; b0 < d_in; b0 += QB) {
    hipLaunchKernelGGL((colloop_kernel<BITS, G, SYM>), dim3(rgrid), dim3(256), 0, stream, Wc, Err,
                       U, d_out, d_in, b0, codes, scales, zeros, loss_rows, n_groups);
    const int kb = (int)std::min<int64_t>(QB, d_in - b0);
    const int64_t n0 = b0 + kb;
    if (n0 < d_in) {
      const int64_t tiles = ceil_div(d_out, 128) * ceil_div(d_in - n0, 128);
      hipLaunchKernelGGL(trailing_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, Wc,
                         (const float*)Err, U, d_out, d_in, b0, kb, n0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, bool SYM>
hipError_t dispatch_g(int group_size, float* Wc, float* Err, const float* U, int64_t d_out,
                      int64_t d_in, uint8_t* codes, float* scales, float* zeros,
                      float* loss_rows, int n_groups, hipStream_t s) {
  switch (group_size) {
    case 32: return run_quant<BITS, 32, SYM>(Wc, Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, s);
    case 64: return run_quant<BITS, 64, SYM>(Wc, Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, s);
    case 128: return run_quant<BITS, 128, SYM>(Wc, Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, s);
    default: return run_quant<BITS, 0, SYM>(Wc, Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, s);
  }
}

// ---- pack -------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t d_out, int64_t d_in, int bits,
                                                         int64_t words, uint32_t* __restrict__ qw) {
  const int64_t total = d_out * words;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / words, wi = e % words;
    const int64_t bit0 = wi * 32;
    int64_t j = bit0 / bits;
    const int64_t jend = std::min<int64_t>(d_in, (bit0 + 32 + bits - 1) / bits);
    const uint8_t* src = codes + r * d_in;
    uint64_t acc = 0;
    for (; j < jend; ++j) {
      const int64_t sh = (int64_t)bits * j - bit0;  // may be negative for a straddling code
      const uint64_t v = (uint64_t)(src[j] & ((1u << bits) - 1));
      acc |= (sh >= 0) ? (v << sh) : (v >> (-sh));
    }
    qw[e] = (uint32_t)acc;
  }
}

__global__ __launch_bounds__(256) void pack_meta_kernel(const float* __restrict__ scales,
                                                        const float* __restrict__ zeros,
                                                        int64_t n, uint16_t* __restrict__ s16,
                                                        uint16_t* __restrict__ z16) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    s16[e] = __half_as_ushort(__float2half_rn(scales[e]));
    if (z16) z16[e] = __half_as_ushort(__float2half_rn(zeros[e]));
  }
}

}  // namespace

size_t quantize_workspace(int64_t d_out, int64_t d_in, int /*block*/) {
  return 2 * align256((size_t)d_out * d_in * sizeof(float));
}

hipError_t quantize_launch(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                           const float* U, const uint8_t* dead, int bits, int group_size, int sym,
                           uint8_t* codes, float* scales, float* zeros, float* loss_rows,
                           void* ws, hipStream_t stream) {
  QuantWs w = carve(ws, d_out, d_in);
  const int64_t total = d_out * d_in;
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(total, 256), 65536);
  hipLaunchKernelGGL(qinit_kernel, dim3(grid), dim3(256), 0, stream, W, w_dtype, d_out, d_in,
                     dead, w.Wc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_groups = (group_size == -1) ? 1 : (int)(d_in / group_size);
  const int g = (group_size == -1) ? 0 : group_size;
  if (sym) {
    switch (bits) {
      case 2: return dispatch_g<2, true>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
      case 3: return dispatch_g<3, true>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
      default: return dispatch_g<4, true>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
    }
  }
  switch (bits) {
    case 2: return dispatch_g<2, false>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
    case 3: return dispatch_g<3, false>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
    default: return dispatch_g<4, false>(g, w.Wc, w.Err, U, d_out, d_in, codes, scales, zeros, loss_rows, n_groups, stream);
  }
}

hipError_t pack_launch(const uint8_t* codes, const float* scales, const float* zeros,
                       int64_t d_out, int64_t d_in, int bits, int n_groups, int sym,
                       uint32_t* qweight, uint16_t* scales_f16, uint16_t* zeros_f16,
                       hipStream_t stream) {
  const int64_t words = ceil_div(d_in * bits, 32);
  const int64_t total = d_out * words;
  if (total > 0)
    hipLaunchKernelGGL(pack_codes_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(total, 256), 65536)), dim3(256),
                       0, stream, codes, d_out, d_in, bits, words, qweight);
  const int64_t nm = d_out * n_groups;
  if (nm > 0)
    hipLaunchKernelGGL(pack_meta_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(nm, 256), 65536)), dim3(256), 0,
                       stream, scales, zeros, nm, scales_f16, sym ? (uint16_t*)nullptr : zeros_f16);
  return hipGetLastError();
}

}  // namespace gptq
