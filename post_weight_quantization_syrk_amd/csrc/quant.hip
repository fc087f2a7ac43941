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
//   trailing : W[:, later columns] -= Err U on the bf16 matrix cores, the
//              fp32 operands split into bf16 hi + lo and the product formed
//              in three passes (trailing3_kernel).  Blocks go in groups of four: after
//              each block, its errors update the rest of its group (K = 128);
//              after the group, all four blocks' errors update every column
//              after it at once (K = 512), so the bulk of W is read and
//              written once per group.
#include "common.h"
#include "kernels.h"
#include "mfma_f32.h"  // StaticFor

#include <hip/hip_fp16.h>
#include <algorithm>

namespace gptq {

namespace {

constexpr int QB = 128;      // block width (columns)
constexpr int UPITCH = 132;  // LDS pitch (floats) of the U block in the column loop
constexpr int QG = 4;        // blocks per far trailing update

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

// Quantizer shape, uniform over the launch.
struct QSpec {
  int maxq;     // 2^bits - 1
  int sym;      // 0 asymmetric, 1 symmetric
  int gsize;    // group size (power of two, <= 128), 0 = one group per row
  int gshift;   // log2(gsize)
  int n_groups;
};

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

// Wc = W as fp32, dead columns zeroed.  With vec (d_in % 8 == 0 and W
// 16-byte aligned) each thread converts 8 consecutive elements of a row:
// one 16-byte load of bf16 (or two of fp32) and two 16-byte stores.
__global__ __launch_bounds__(256) void qinit_kernel(const void* __restrict__ W, int w_dtype,
                                                    int64_t d_out, int64_t d_in,
                                                    const uint8_t* __restrict__ dead,
                                                    float* __restrict__ Wc, int vec) {
  const int64_t total = d_out * d_in;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (vec) {
    for (int64_t e8 = (int64_t)blockIdx.x * 256 + threadIdx.x; e8 < total / 8; e8 += stride) {
      const int64_t c = (e8 * 8) % d_in;
      float v[8];
      if (w_dtype == 0) {
        const uint4 raw = ((const uint4*)W)[e8];
        const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(wds[i] << 16);
          v[2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
        }
      } else {
        const float4 a = ((const float4*)W)[2 * e8], b = ((const float4*)W)[2 * e8 + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
      if (dead) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = dead[c + i] ? 0.0f : v[i];
      }
      float4* dst = (float4*)Wc + 2 * e8;
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    return;
  }
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += stride) {
    const int64_t c = e % d_in;
    float v = (w_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)W)[e]) : ((const float*)W)[e];
    if (dead && dead[c]) v = 0.0f;
    Wc[e] = v;
  }
}

// Column order ([P1] GPTQ 的高级技巧, 激活排序): Wc[:, k] = W[:, perm[k]] as fp32,
// dead columns zeroed.  perm entries are clamped to [0, d_in) (a caller that
// passes no permutation gets garbage, never an out-of-bounds access).
__global__ __launch_bounds__(256) void qinit_perm_kernel(const void* __restrict__ W, int w_dtype,
                                                         int64_t d_out, int64_t d_in,
                                                         const uint8_t* __restrict__ dead,
                                                         const int32_t* __restrict__ perm,
                                                         float* __restrict__ Wc) {
  // grid: x over columns, y over rows (strided)
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= d_in) return;
  const int64_t c = min<int64_t>(max(perm[k], 0), d_in - 1);
  const bool dc = dead && dead[c];
  for (int64_t r = blockIdx.y; r < d_out; r += gridDim.y) {
    const int64_t src = r * d_in + c;
    const float v = (w_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)W)[src])
                                   : ((const float*)W)[src];
    Wc[r * d_in + k] = dc ? 0.0f : v;
  }
}

// codes[:, perm[k]] = codes_p[:, k]
__global__ __launch_bounds__(256) void unpermute_codes_kernel(const uint8_t* __restrict__ cp,
                                                              const int32_t* __restrict__ perm,
                                                              int64_t d_out, int64_t d_in,
                                                              uint8_t* __restrict__ codes) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= d_in) return;
  const int64_t c = min<int64_t>(max(perm[k], 0), d_in - 1);
  for (int64_t r = blockIdx.y; r < d_out; r += gridDim.y) codes[r * d_in + c] = cp[r * d_in + k];
}

// Group of each natural column: static groups c >> gshift; dynamic groups
// follow the processing order, g_idx[perm[k]] = k >> gshift; one group per
// row gives 0.
__global__ __launch_bounds__(256) void gidx_kernel(const int32_t* __restrict__ perm, int64_t d_in,
                                                   int gsize, int gshift, int static_groups,
                                                   int32_t* __restrict__ g_idx) {
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < d_in;
       k += (int64_t)gridDim.x * 256) {
    if (gsize == 0) {
      g_idx[k] = 0;
    } else if (static_groups || !perm) {
      g_idx[k] = (int32_t)(k >> gshift);
    } else {
      const int64_t c = min<int64_t>(max(perm[k], 0), d_in - 1);
      g_idx[c] = (int32_t)(k >> gshift);
    }
  }
}

struct GroupParams {
  float s, inv_s, hs, z;
  float hs_lo;  // the largest float below hs (s/2)
};

// Scale and zero from the group's min/max (asymmetric) or max |v| (symmetric).
// The step is formed in float64 and rounded once to binary16.
__device__ __forceinline__ GroupParams make_params(float lo_or_amax, float hi, int maxq, int sym) {
  GroupParams p;
  double s;
  float z;
  if (sym) {
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
  p.hs_lo = __int_as_float(__float_as_int(p.hs) - 1);  // hs >= 2^-25: a normal float
  p.z = z;
  return p;
}

// Nearest integer to the exact quotient x/s, ties to even, then code clamp.
// q0 = rint(x * (1/s)) is within 1 of it.  r = x - q0 s is exact (q0 s has
// at most 22 significant bits, and |r| <= s keeps the difference within
// x's precision), so comparing r with +-s/2 settles the last unit; a tie
// (|r| = s/2) moves an odd q0 to its even neighbour, which is the same as
// comparing against the float just below s/2 when q0 is odd.  Selects only:
// this sits on the column loop's dependency chain.
__device__ __forceinline__ float quantize_code(float x, const GroupParams& p, float maxq) {
  const float q0 = __builtin_amdgcn_fmed3f(rintf(x * p.inv_s), -2047.0f, 2047.0f);
  const float t = (((int)q0) & 1) ? p.hs_lo : p.hs;
  const float r = fmaf(-q0, p.s, x);
  const float adj = (r > t) ? 1.0f : ((r < -t) ? -1.0f : 0.0f);
  return __builtin_amdgcn_fmed3f(q0 + adj + p.z, 0.0f, maxq);
}

// One group per row: parameters from the whole (current = original) row.
__global__ __launch_bounds__(256) void rowparams_kernel(const float* __restrict__ Wc,
                                                        int64_t d_out, int64_t d_in, QSpec q,
                                                        float* __restrict__ scales,
                                                        float* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const float* w = Wc + row * d_in;
  float mn = 0.0f, mx = 0.0f;  // the range always contains 0
  for (int64_t c = lane; c < d_in; c += 64) {
    const float v = w[c];
    mn = fminf(mn, v);
    mx = fmaxf(mx, q.sym ? fabsf(v) : v);
  }
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (lane == 0) {
    const GroupParams p = q.sym ? make_params(mx, 0.0f, q.maxq, 1) : make_params(mn, mx, q.maxq, 0);
    scales[row] = p.s;
    zeros[row] = p.z;
  }
}


// Static groups ([P1] GPTQ 的高级技巧, 静态与动态分组): every natural group's
// scale and zero from the original weights (dead columns zeroed), before any
// error feedback.  One wave per (row, group); the group's columns are read
// 64 at a time.
__global__ __launch_bounds__(256) void static_params_kernel(const void* __restrict__ W,
                                                            int w_dtype, int64_t d_out,
                                                            int64_t d_in,
                                                            const uint8_t* __restrict__ dead,
                                                            QSpec q, float* __restrict__ scales,
                                                            float* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= d_out * q.n_groups) return;
  const int64_t row = item / q.n_groups, g = item % q.n_groups;
  float mn = 0.0f, mx = 0.0f;  // the range always contains 0
  for (int64_t c = g * q.gsize + lane; c < (g + 1) * q.gsize; c += 64) {
    const int64_t e = row * d_in + c;
    float v = (w_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)W)[e]) : ((const float*)W)[e];
    if (dead && dead[c]) v = 0.0f;
    mn = fminf(mn, v);
    mx = fmaxf(mx, q.sym ? fabsf(v) : v);
  }
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (lane == 0) {
    const GroupParams p = q.sym ? make_params(mx, 0.0f, q.maxq, 1) : make_params(mn, mx, q.maxq, 0);
    scales[item] = p.s;
    zeros[item] = p.z;
  }
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
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m, 16);
  return v;
}

// STATIC: the group parameters are given (static groups, natural groups of
// the original weights, in scales/zeros) and column k of the block uses those
// of group perm[b0 + k] >> gshift (perm may be null: natural order); they are
// staged in LDS per row and column at the start.  Otherwise each group's
// parameters are set at its first column from the current values and
// written to scales/zeros.
template <bool STATIC>
__global__ __launch_bounds__(256) void colloop_kernel(
    float* __restrict__ Wc, float* __restrict__ Err, const float* __restrict__ U,
    int64_t d_out, int64_t d_in, int64_t b0, QSpec q, uint8_t* __restrict__ codes,
    float* __restrict__ scales, float* __restrict__ zeros, float* __restrict__ loss_rows,
    const int32_t* __restrict__ perm) {
  __shared__ __attribute__((aligned(16))) float us[QB * UPITCH];
  __shared__ float invd[QB];
  __shared__ float sps[STATIC ? 16 * QB : 1], spi[STATIC ? 16 * QB : 1], spz[STATIC ? 16 * QB : 1];
  const int tid = threadIdx.x;
  const int bw = (int)min<int64_t>(QB, d_in - b0);
  const int c = tid & 15;  // lane within the row group
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool live = row < d_out;
  const int64_t rr = live ? row : 0;
  const float maxq = (float)q.maxq;
  float w[8];
  {
    // this lane's 8 columns of the row (unconditional loads, masked after)
    const float* src = Wc + rr * d_in + b0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = src[min(8 * c + i, bw - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (8 * c + i < bw) ? w[i] : 0.0f;
  }
  // U block: upper triangle only, identity padding past the matrix edge.
  // 64 elements per thread, all loads in flight at once (clamped addresses).
  {
    float v[QB * QB / 256];
#pragma unroll
    for (int u = 0; u < QB * QB / 256; ++u) {
      const int e = u * 256 + tid, r = e >> 7, cc = e & 127;
      v[u] = U[(b0 + min(r, bw - 1)) * d_in + b0 + min(cc, bw - 1)];
    }
#pragma unroll
    for (int u = 0; u < QB * QB / 256; ++u) {
      const int e = u * 256 + tid, r = e >> 7, cc = e & 127;
      us[r * UPITCH + cc] = (r < bw && cc < bw) ? (cc >= r ? v[u] : 0.0f) : (r == cc ? 1.0f : 0.0f);
    }
  }
  if constexpr (STATIC) {
    for (int e = tid; e < 16 * QB; e += 256) {
      const int rl = e / QB, k = e % QB;
      const int64_t r = min<int64_t>((int64_t)blockIdx.x * 16 + rl, d_out - 1);
      const int64_t col = b0 + min(k, bw - 1);
      const int64_t pc = perm ? min<int64_t>(max(perm[col], 0), d_in - 1) : col;
      const int64_t gi = r * q.n_groups + (pc >> q.gshift);
      const float sv = scales[gi];
      sps[e] = sv;
      spi[e] = 1.0f / sv;
      spz[e] = zeros[gi];
    }
  }
  __syncthreads();
  if (tid < QB) invd[tid] = 1.0f / us[tid * UPITCH + tid];
  __syncthreads();
  // Row j of the block scaled by 1 / U_jj: column j's feedback is then its
  // unscaled error x - what times the scaled row, and neither the division
  // nor its LDS read sits on the chain from one column to the next.  Thread
  // t scales half t % 2 of row t / 2 (16-byte LDS accesses).
  {
    const float sc = invd[tid >> 1];
    float4* rw = (float4*)(us + (tid >> 1) * UPITCH + 64 * (tid & 1));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float4 v = rw[i];
      v.x *= sc;
      v.y *= sc;
      v.z *= sc;
      v.w *= sc;
      rw[i] = v;
    }
  }
  __syncthreads();

  GroupParams gp;
  if (q.gsize == 0) {
    gp.s = scales[rr];
    gp.inv_s = 1.0f / gp.s;
    gp.hs = 0.5f * gp.s;
    gp.hs_lo = __int_as_float(__float_as_int(gp.hs) - 1);
    gp.z = zeros[rr];
  }
  const int gmask = q.gsize - 1;
  // STATIC: the next column's parameters, read one column ahead
  float ns = 0.0f, ni = 0.0f, nz = 0.0f;
  if constexpr (STATIC) {
    const int e = (tid >> 4) * QB;
    ns = sps[e];
    ni = spi[e];
    nz = spz[e];
  }
  float cr[8], er[8];
  // U row of the next column, read one column ahead so the LDS latency is off
  // the dependency chain.
  float4 un0 = ((const float4*)(us + 8 * c))[0], un1 = ((const float4*)(us + 8 * c))[1];
  // Fully unrolled over the 128 columns: register indices and the DPP source
  // lane are compile-time constants.  Columns past the matrix edge (j >= bw)
  // run too, on zero weights against identity rows of U: their delta is 0,
  // so they change nothing, and keeping every column branch-free lets the
  // LDS reads of later columns be hoisted off the dependency chain.
  StaticFor<0, QB>::run([&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (STATIC) {
      gp.s = ns;
      gp.inv_s = ni;
      gp.z = nz;
      gp.hs = 0.5f * gp.s;
      gp.hs_lo = __int_as_float(__float_as_int(gp.hs) - 1);
      if constexpr (j + 1 < QB) {
        const int e = (tid >> 4) * QB + j + 1;
        ns = sps[e];
        ni = spi[e];
        nz = spz[e];
      }
    } else if constexpr (j % 32 == 0) {  // every supported group size is a multiple of 32
      if (q.gsize != 0 && (j & gmask) == 0) {
        const bool mine = (8 * c >= j) && (8 * c < j + q.gsize);
        float mn = 0.0f, mx = 0.0f;
        if (mine) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            mn = fminf(mn, w[i]);
            mx = fmaxf(mx, q.sym ? fabsf(w[i]) : w[i]);
          }
        }
        mx = row_max(mx);
        mn = row_min(mn);
        gp = q.sym ? make_params(mx, 0.0f, q.maxq, 1) : make_params(mn, mx, q.maxq, 0);
        if (c == (j >> 3) && live && j < bw) {
          const int64_t gi = rr * q.n_groups + ((b0 + j) >> q.gshift);
          scales[gi] = gp.s;
          zeros[gi] = gp.z;
        }
      }
    }
    const float x = row_bcast<(j >> 3)>(w[j & 7]);
    const float code = quantize_code(x, gp, maxq);
    const float what = gp.s * (code - gp.z);
    const float e = x - what;
    if (c == (j >> 3)) {
      cr[j & 7] = code;
      er[j & 7] = e;
    }
    const float4 u0 = un0, u1 = un1;
    if constexpr (j + 1 < QB) {
      const float4* urow = (const float4*)(us + (j + 1) * UPITCH + 8 * c);
      un0 = urow[0];
      un1 = urow[1];
    }
    w[0] = fmaf(-e, u0.x, w[0]);
    w[1] = fmaf(-e, u0.y, w[1]);
    w[2] = fmaf(-e, u0.z, w[2]);
    w[3] = fmaf(-e, u0.w, w[3]);
    w[4] = fmaf(-e, u1.x, w[4]);
    w[5] = fmaf(-e, u1.y, w[5]);
    w[6] = fmaf(-e, u1.z, w[6]);
    w[7] = fmaf(-e, u1.w, w[7]);
  });
  // the scaled errors delta = (x - what) / U_jj of this lane's 8 columns
  // (columns past the edge have x - what = 0), and the row's loss sum_j
  // delta_j^2: this lane's 8 terms, then the row's 16 lanes
  float loss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    er[i] *= invd[8 * c + i];
    loss = fmaf(er[i], er[i], loss);
  }
  loss = row_sum(loss);
  if (!live) return;
  // codes and scaled errors of this lane's 8 columns (the errors as two
  // 16-byte stores when the lane's columns are all inside and 16-byte aligned:
  // d_in a multiple of 4, b0 a multiple of 128)
  // (the codes as one 8-byte store when d_in is a multiple of 8 and codes is
  // 8-byte aligned)
  uint8_t* cdst = codes + rr * d_in + b0 + 8 * c;
  float* edst = Err + rr * d_in + b0 + 8 * c;
  if ((d_in & 7) == 0 && ((uintptr_t)codes & 7) == 0 && 8 * c + 8 <= bw) {
    uint32_t cw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      cw[t] = (uint32_t)cr[4 * t] | ((uint32_t)cr[4 * t + 1] << 8) |
              ((uint32_t)cr[4 * t + 2] << 16) | ((uint32_t)cr[4 * t + 3] << 24);
    *(uint2*)cdst = make_uint2(cw[0], cw[1]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (8 * c + i < bw) cdst[i] = (uint8_t)cr[i];
  }
  if ((d_in & 3) == 0 && 8 * c + 8 <= bw) {
    ((float4*)edst)[0] = make_float4(er[0], er[1], er[2], er[3]);
    ((float4*)edst)[1] = make_float4(er[4], er[5], er[6], er[7]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (8 * c + i < bw) edst[i] = er[i];
  }
  if (loss_rows && c == 0) loss_rows[rr] = (b0 == 0 ? 0.0f : loss_rows[rr]) + loss;
}

// Wc[:, n0:n1] -= Err[:, b0:b0+kb] * U[b0:b0+kb, n0:n1] on the bf16 matrix
// cores: each fp32 operand is split into bf16 hi + lo (hi the nearest bf16,
// lo the nearest bf16 of the exact remainder) and the product is formed as
// lo*hi + hi*lo + hi*hi with v_mfma_f32_32x32x16_bf16 into fp32 accumulators,
// which keeps about 16 significant bits of every product (the dropped lo*lo
// term and the rounding of lo are below 2^-16 relative); the errors it leaves
// in the feedback are far below a quantization step.  TM x 64 tiles, K in
// chunks of 32 (two MFMA steps of 16).  The error tile is stored row-major
// (k contiguous), the U tile transposed (n-major, k contiguous), so every lane
// reads its 8 consecutive k as 16 bytes; row pitches of 80 bytes keep those
// reads free of bank conflicts.  The accumulators start at -Wc and collect
// Err U, and the tile is stored back negated: negation commutes with every
// rounding, so this is Wc - Err U as accumulated the other way round, with no
// negation per staged element.
constexpr int T3K = 32;           // k per chunk
constexpr int T3P = T3K + 8;      // LDS row pitch (bf16 elements): 80 bytes

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
// The same split for a pair, with the hardware's nearest-even conversion of
// two floats at once: hi parts packed low-first, lo parts likewise into lo.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t split_pair(float x0, float x1, uint32_t& lo) {
  const f32x2v x = {x0, x1};
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
  const f32x2v hf = {__uint_as_float(hb << 16), __uint_as_float(hb & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hf, bf16x2v));
  return hb;
}

// VEC (d_in a multiple of 4, U 16-byte aligned; the launches give kb a
// multiple of 32 and b0, n0 multiples of 64): each thread loads 4 consecutive
// k of an error row and 2 k rows x 4 columns of U as 16-byte vectors, and
// splits and stores them in pairs of k.
template <int TM, bool VEC>
__global__ __launch_bounds__(256) void trailing3_kernel(float* __restrict__ Wc,
                                                        const float* __restrict__ Err,
                                                        const float* __restrict__ U,
                                                        int64_t d_out, int64_t d_in, int64_t b0,
                                                        int kb, int64_t n0, int64_t n1) {
  constexpr int TN = 64;
  constexpr int NBLK = (TM / 32) * (TN / 32) / 4;  // 32 x 32 blocks per wave
  constexpr int NP = TM * T3K / 256, NQ = T3K * TN / 256;
  __shared__ __attribute__((aligned(16))) uint16_t ah[TM * T3P], al[TM * T3P];
  __shared__ __attribute__((aligned(16))) uint16_t bh[TN * T3P], bl[TN * T3P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t ncols = n1 - n0;
  const int ntn = (int)ceil_div(ncols, TN);
  const int64_t m0 = (int64_t)(blockIdx.x / ntn) * TM;
  const int64_t n0t = n0 + (int64_t)(blockIdx.x % ntn) * TN;
  const int rows = (int)min<int64_t>(TM, d_out - m0);
  const int cols = (int)min<int64_t>(TN, n1 - n0t);
  // this wave's blocks: (bm, bn) with bm = row block, bn = column block
  int bm[NBLK], bn[NBLK];
#pragma unroll
  for (int q = 0; q < NBLK; ++q) {
    const int blk = wave * NBLK + q;  // row-block major over (TM / 32) x 2
    bm[q] = blk >> 1;
    bn[q] = blk & 1;
  }
  float* C = Wc + m0 * d_in + n0t;
  f32x16 acc[NBLK];
#pragma unroll
  for (int q = 0; q < NBLK; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * bm[q] + 8 * (i >> 2) + 4 * h + (i & 3);
      const int c = 32 * bn[q] + l32;
      acc[q][i] = -C[(int64_t)(r < rows ? r : rows - 1) * d_in + (c < cols ? c : cols - 1)];
    }
  const float* P = Err + m0 * d_in + b0;
  const float* Q = U + b0 * d_in + n0t;
  float vp[NP], vq[NQ];
  static_assert(NQ == 8 && NP % 4 == 0, "vector staging takes 2 x 4 U values per thread");
  const int vn = 4 * (tid & 15), vk = 2 * (tid >> 4);  // VEC: this thread's U columns, k pair
  auto gload = [&](int kc) __attribute__((always_inline)) {
    const int kn = min(T3K, kb - kc);
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < NP / 4; ++j) {
        const int e = 4 * (j * 256 + tid), r = e / T3K, c = e % T3K;
        const float4 v =
            *(const float4*)(P + (int64_t)(r < rows ? r : rows - 1) * d_in + kc + c);
        vp[4 * j] = v.x; vp[4 * j + 1] = v.y; vp[4 * j + 2] = v.z; vp[4 * j + 3] = v.w;
      }
      const int nc = vn < cols ? vn : 0;
      const float4 v0 = *(const float4*)(Q + (int64_t)(kc + vk) * d_in + nc);
      const float4 v1 = *(const float4*)(Q + (int64_t)(kc + vk + 1) * d_in + nc);
      vq[0] = v0.x; vq[1] = v0.y; vq[2] = v0.z; vq[3] = v0.w;
      vq[4] = v1.x; vq[5] = v1.y; vq[6] = v1.z; vq[7] = v1.w;
      return;
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = u * 256 + tid, r = e / T3K, c = e % T3K;
      vp[u] = P[(int64_t)(r < rows ? r : rows - 1) * d_in + kc + (c < kn ? c : kn - 1)];
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = u * 256 + tid, r = e / TN, c = e % TN;
      vq[u] = Q[(int64_t)(kc + (r < kn ? r : kn - 1)) * d_in + (c < cols ? c : cols - 1)];
    }
  };
  auto lstore = [&](int kc) __attribute__((always_inline)) {
    const int kn = min(T3K, kb - kc);
    if constexpr (VEC) {
      // no masks: every k is inside the block, and rows past d_out or columns
      // past n1 (clamped copies of finite values) only reach accumulator rows
      // or columns that are never stored
#pragma unroll
      for (int j = 0; j < NP / 4; ++j) {
        const int e = 4 * (j * 256 + tid), r = e / T3K, c = e % T3K;
        uint32_t l0, l1;
        const uint32_t h0 = split_pair(vp[4 * j], vp[4 * j + 1], l0);
        const uint32_t h1 = split_pair(vp[4 * j + 2], vp[4 * j + 3], l1);
        *(uint2*)(ah + r * T3P + c) = make_uint2(h0, h1);
        *(uint2*)(al + r * T3P + c) = make_uint2(l0, l1);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t l;
        const uint32_t hw = split_pair(vq[t], vq[4 + t], l);
        *(uint32_t*)(bh + (vn + t) * T3P + vk) = hw;
        *(uint32_t*)(bl + (vn + t) * T3P + vk) = l;
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = u * 256 + tid, r = e / T3K, c = e % T3K;
      const float x = (r < rows && c < kn) ? vp[u] : 0.0f;
      const uint16_t hi = bf16_rne_bits(x);
      ah[r * T3P + c] = hi;
      al[r * T3P + c] = bf16_rne_bits(x - bf16_bits_to_f32(hi));
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = u * 256 + tid, r = e / TN, c = e % TN;  // r = k, c = n
      const float x = (r < kn && c < cols) ? vq[u] : 0.0f;
      const uint16_t hi = bf16_rne_bits(x);
      bh[c * T3P + r] = hi;
      bl[c * T3P + r] = bf16_rne_bits(x - bf16_bits_to_f32(hi));
    }
  };
  gload(0);
  for (int kc = 0; kc < kb; kc += T3K) {
    if (kc > 0) __syncthreads();  // the previous chunk's products are done with LDS
    lstore(kc);
    __syncthreads();
    if (kc + T3K < kb) gload(kc + T3K);
#pragma unroll
    for (int ks = 0; ks < T3K / 16; ++ks) {
      const int ko = 16 * ks + 8 * h;
#pragma unroll
      for (int q = 0; q < NBLK; ++q) {
        const int ar = (32 * bm[q] + l32) * T3P + ko, br = (32 * bn[q] + l32) * T3P + ko;
        const bf16x8 a_h = *(const bf16x8*)(ah + ar), a_l = *(const bf16x8*)(al + ar);
        const bf16x8 b_h = *(const bf16x8*)(bh + br), b_l = *(const bf16x8*)(bl + br);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_l, b_h, acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_h, b_l, acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_h, b_h, acc[q], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NBLK; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * bm[q] + 8 * (i >> 2) + 4 * h + (i & 3);
      const int c = 32 * bn[q] + l32;
      if (r < rows && c < cols) C[(int64_t)r * d_in + c] = -acc[q][i];
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

size_t quantize_perm_workspace(int64_t d_out, int64_t d_in, int block) {
  return quantize_workspace(d_out, d_in, block) + align256((size_t)d_out * d_in);
}

hipError_t quantize_launch(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                           const float* U, const uint8_t* dead, int bits, int group_size, int sym,
                           uint8_t* codes, float* scales, float* zeros, float* loss_rows,
                           void* ws, hipStream_t stream) {
  return quantize_perm_launch(W, w_dtype, d_out, d_in, U, dead, nullptr, 0, bits, group_size,
                              sym, codes, scales, zeros, nullptr, loss_rows, ws, stream);
}

namespace {

// Rows of the working copy come from one or more weight matrices (stacked in
// order); with several, the columns are in natural order and groups dynamic.
struct WSource {
  const void* const* ptrs;
  const int64_t* rows;
  int count;
};

hipError_t quantize_core(const WSource& src, int w_dtype, int64_t d_out, int64_t d_in,
                         const float* U, const uint8_t* dead, const int32_t* perm,
                         int static_groups, int bits, int group_size, int sym, uint8_t* codes,
                         float* scales, float* zeros, int32_t* g_idx, float* loss_rows, void* ws,
                         hipStream_t stream) {
  QuantWs w = carve(ws, d_out, d_in);
  const void* W = src.ptrs[0];
  // with a permutation the column loop writes codes in processing order to
  // the workspace; they are put back in natural order at the end
  uint8_t* codes_k = perm ? (uint8_t*)ws + quantize_workspace(d_out, d_in, QB) : codes;
  const dim3 pgrid((unsigned)ceil_div(d_in, 256), (unsigned)std::min<int64_t>(d_out, 1024));
  if (perm) {
    hipLaunchKernelGGL(qinit_perm_kernel, pgrid, dim3(256), 0, stream, W, w_dtype, d_out, d_in,
                       dead, perm, w.Wc);
  } else {
    int64_t r0 = 0;
    for (int i = 0; i < src.count; ++i) {
      const int64_t rows = src.rows[i];
      if (rows == 0) continue;
      const int64_t total = rows * d_in;
      const int vec = (d_in % 8 == 0) && ((uintptr_t)src.ptrs[i] % 16 == 0);
      const unsigned grid =
          (unsigned)std::min<int64_t>(ceil_div(vec ? total / 8 : total, 256), 65536);
      hipLaunchKernelGGL(qinit_kernel, dim3(grid), dim3(256), 0, stream, src.ptrs[i], w_dtype,
                         rows, d_in, dead, w.Wc + r0 * d_in, vec);
      r0 += rows;
    }
  }
  QSpec q;
  q.maxq = (1 << bits) - 1;
  q.sym = sym ? 1 : 0;
  q.gsize = (group_size == -1) ? 0 : group_size;
  q.gshift = 0;
  while (q.gsize && (1 << q.gshift) < q.gsize) ++q.gshift;
  q.n_groups = (group_size == -1) ? 1 : (int)(d_in / group_size);
  if (q.gsize == 0)
    hipLaunchKernelGGL(rowparams_kernel, dim3((unsigned)ceil_div(d_out, 4)), dim3(256), 0, stream,
                       (const float*)w.Wc, d_out, d_in, q, scales, zeros);
  // one group per row: static and dynamic coincide (the whole original row)
  const bool stat = static_groups && q.gsize != 0;
  if (stat)
    hipLaunchKernelGGL(static_params_kernel,
                       dim3((unsigned)ceil_div(d_out * q.n_groups, 4)), dim3(256), 0, stream, W,
                       w_dtype, d_out, d_in, dead, q, scales, zeros);
  // Blocks in groups of QG: after each block's column loop its errors go to
  // the rest of its group only (near update, K = 128); after the group, all
  // of the group's errors go to the columns after it at once (far update,
  // K = 128 QG), so the bulk of W is read and written once per group.
  const unsigned rgrid = (unsigned)ceil_div(d_out, 16);
  static_assert(QB % T3K == 0, "trailing updates take whole chunks");
  const bool tvec = (d_in % 4 == 0) && ((uintptr_t)U % 16 == 0);
  const int64_t nb = ceil_div(d_in, QB);
  for (int64_t g0 = 0; g0 < nb; g0 += QG) {
    const int64_t gend = std::min<int64_t>(nb, g0 + QG);
    const int64_t gcol = std::min<int64_t>(d_in, gend * QB);  // first column after the group
    for (int64_t b = g0; b < gend; ++b) {
      const int64_t b0 = b * QB;
      if (stat)
        hipLaunchKernelGGL(colloop_kernel<true>, dim3(rgrid), dim3(256), 0, stream, w.Wc, w.Err,
                           U, d_out, d_in, b0, q, codes_k, scales, zeros, loss_rows, perm);
      else
        hipLaunchKernelGGL(colloop_kernel<false>, dim3(rgrid), dim3(256), 0, stream, w.Wc, w.Err,
                           U, d_out, d_in, b0, q, codes_k, scales, zeros, loss_rows, perm);
      const int64_t n0 = b0 + QB;
      if (b + 1 < gend) {  // blocks before the group's last are full
        const int64_t tiles = ceil_div(d_out, 64) * ceil_div(gcol - n0, 64);
        if (tvec)
          hipLaunchKernelGGL((trailing3_kernel<64, true>), dim3((unsigned)tiles), dim3(256), 0,
                             stream, w.Wc, (const float*)w.Err, U, d_out, d_in, b0, QB, n0, gcol);
        else
          hipLaunchKernelGGL((trailing3_kernel<64, false>), dim3((unsigned)tiles), dim3(256), 0,
                             stream, w.Wc, (const float*)w.Err, U, d_out, d_in, b0, QB, n0, gcol);
      }
    }
    if (gcol < d_in) {  // every block of the group is full
      const int64_t tiles = ceil_div(d_out, 128) * ceil_div(d_in - gcol, 64);
      const int kb = (int)(gcol - g0 * QB);
      if (tvec)
        hipLaunchKernelGGL((trailing3_kernel<128, true>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, w.Wc, (const float*)w.Err, U, d_out, d_in, g0 * QB, kb, gcol,
                           d_in);
      else
        hipLaunchKernelGGL((trailing3_kernel<128, false>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, w.Wc, (const float*)w.Err, U, d_out, d_in, g0 * QB, kb, gcol,
                           d_in);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (perm)
    hipLaunchKernelGGL(unpermute_codes_kernel, pgrid, dim3(256), 0, stream,
                       (const uint8_t*)codes_k, perm, d_out, d_in, codes);
  if (g_idx)
    hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(d_in, 256), 1024)),
                       dim3(256), 0, stream, perm, d_in, q.gsize, q.gshift, static_groups ? 1 : 0,
                       g_idx);
  return hipGetLastError();
}

}  // namespace

hipError_t quantize_perm_launch(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                                const float* U, const uint8_t* dead, const int32_t* perm,
                                int static_groups, int bits, int group_size, int sym,
                                uint8_t* codes, float* scales, float* zeros, int32_t* g_idx,
                                float* loss_rows, void* ws, hipStream_t stream) {
  const WSource src{&W, &d_out, 1};
  return quantize_core(src, w_dtype, d_out, d_in, U, dead, perm, static_groups, bits, group_size,
                       sym, codes, scales, zeros, g_idx, loss_rows, ws, stream);
}

hipError_t quantize_multi_launch(const void* const* Ws, const int64_t* d_outs, int count,
                                 int w_dtype, int64_t d_in, const float* U, const uint8_t* dead,
                                 int bits, int group_size, int sym, uint8_t* codes,
                                 float* scales, float* zeros, float* loss_rows, void* ws,
                                 hipStream_t stream) {
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += d_outs[i];
  const WSource src{Ws, d_outs, count};
  return quantize_core(src, w_dtype, rows, d_in, U, dead, nullptr, 0, bits, group_size, sym,
                       codes, scales, zeros, nullptr, loss_rows, ws, stream);
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
