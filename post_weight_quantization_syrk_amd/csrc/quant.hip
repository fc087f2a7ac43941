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
//              fp32 operands split exactly into three bf16 parts and the
//              product formed from the six leading part products
//              (trailing3_kernel), as accurate as an fp32 product.  Blocks go in groups of four: after
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
constexpr int CL_LPR = 16;   // lanes per row in the column loop
constexpr int64_t FAR_BIG_MIN = 2048;  // 128 x 128 far tiles from this many on

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: the fp32 working copy, then the trailing update's operands
// split into three bf16 parts (h, m, l): the scaled errors delta and U
// transposed (row n holds column n of U), both k-chunk major,
//   E3 [k / 32][part][d_out rows][32],   Ut3 [k / 32][part][d_in rows][32],
// so the 32 k of one chunk and part are 64 contiguous bytes per row and the
// rows of a tile follow each other: one tile operand per chunk and part is
// one contiguous run.
constexpr int KC = 32;  // k per chunk of the split operands

// Then the column loop's diagonal blocks of U: block b's rows scaled by
// 1 / U_jj (Ub, [blocks][QB][QB]) and the 1 / U_jj themselves (Uinv).
struct QuantWs {
  float* Wc;      // [d_out x d_in] working copy
  uint16_t* E3;   // parts of the scaled errors delta
  uint16_t* Ut3;  // parts of U^T (entries with k < n are used)
  float* Ub;      // scaled diagonal blocks of U
  float* Uinv;    // 1 / U_jj
  int64_t se, su; // elements per (chunk, part): d_out * KC and d_in * KC
};

inline int64_t n_chunks(int64_t d_in) { return (d_in + KC - 1) / KC; }
inline int64_t n_blocks(int64_t d_in) { return (d_in + QB - 1) / QB; }

QuantWs carve(void* ws, int64_t d_out, int64_t d_in) {
  QuantWs w;
  const size_t m = align256((size_t)d_out * d_in * sizeof(float));
  w.se = d_out * KC;
  w.su = d_in * KC;
  w.Wc = (float*)ws;
  w.E3 = (uint16_t*)((char*)ws + m);
  w.Ut3 = (uint16_t*)((char*)w.E3 + align256((size_t)n_chunks(d_in) * 3 * w.se * 2));
  w.Ub = (float*)((char*)w.Ut3 + align256((size_t)n_chunks(d_in) * 3 * w.su * 2));
  w.Uinv = w.Ub + n_blocks(d_in) * QB * QB;
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
// (Workgroup bid of nbid doing this part of a launch.)
__device__ __forceinline__ void qinit_part(const void* __restrict__ W, int w_dtype, int64_t d_out,
                                           int64_t d_in, const uint8_t* __restrict__ dead,
                                           float* __restrict__ Wc, int vec, int bid, int nbid) {
  const int64_t total = d_out * d_in;
  const int64_t stride = (int64_t)nbid * 256;
  if (vec) {
    for (int64_t e8 = (int64_t)bid * 256 + threadIdx.x; e8 < total / 8; e8 += stride) {
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
  for (int64_t e = (int64_t)bid * 256 + threadIdx.x; e < total; e += stride) {
    const int64_t c = e % d_in;
    float v = (w_dtype == 0) ? bf16_bits_to_float(((const uint16_t*)W)[e]) : ((const float*)W)[e];
    if (dead && dead[c]) v = 0.0f;
    Wc[e] = v;
  }
}
__global__ __launch_bounds__(256) void qinit_kernel(const void* __restrict__ W, int w_dtype,
                                                    int64_t d_out, int64_t d_in,
                                                    const uint8_t* __restrict__ dead,
                                                    float* __restrict__ Wc, int vec) {
  qinit_part(W, w_dtype, d_out, d_in, dead, Wc, vec, (int)blockIdx.x, (int)gridDim.x);
}
inline unsigned qinit_grid(int64_t rows, int64_t d_in, int vec) {
  const int64_t total = rows * d_in;
  return (unsigned)std::min<int64_t>(ceil_div(vec ? total / 8 : total, 256), 65536);
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
  float s, inv_s, hs, z;  // hs = s/2 (a normal float: s >= 2^-24)
  float zlo, zhi;  // -z and maxq - z: the range of code - z
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
  p.z = z;
  p.zlo = -z;
  p.zhi = (float)maxq - z;
  return p;
}

// Nearest integer to the exact quotient x/s, ties to even, then code clamp.
// q0, the nearest integer to y = x * (1/s), is within 1 of it: adding 1.5 *
// 2^23 to y rounds y half-to-even into the sum's last mantissa bit (for |y| <
// 2^22, where that sum has unit spacing), which then holds q0's parity, and
// subtracting it again gives q0 exactly.  r = x - q0 s is exact (q0 s has at
// most 22 significant bits while |q0| <= 2^11, and |r| <= s keeps the
// difference within x's precision), so comparing |r| with s/2 settles the
// last unit: q0 moves one step towards r's sign when |r| > s/2; a tie (|r| =
// s/2) moves an odd q0 to its even neighbour, which is the same as comparing
// against the float just below s/2 (its bit pattern minus one) when q0 is
// odd.  Larger |y| (where r may be inexact) clamp to 0 or maxq whatever the
// last unit.  The clamp is applied to code - z (to [-z, maxq - z], exact on
// these small integers), and the error x - s (code - z) is formed with one
// rounding.  Selects and integer arithmetic only, with a single decision on
// |r|: this sits on the column loop's dependency chain.  Returns the error;
// the code goes to *code.
__device__ __forceinline__ float quantize_step(float x, const GroupParams& p, float* code) {
  constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
  const float m = fmaf(x, p.inv_s, MAGIC);
  const float q0 = m - MAGIC;
  const float t = __int_as_float(__float_as_int(p.hs) - (int)(__float_as_uint(m) & 1u));
  const float r = fmaf(-q0, p.s, x);
  const float v = (fabsf(r) > t) ? q0 + copysignf(1.0f, r) : q0;
  const float cz = __builtin_amdgcn_fmed3f(v, p.zlo, p.zhi);
  *code = cz + p.z;
  return fmaf(-p.s, cz, x);
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

// Reductions over the LPR lanes that share one row.
template <int LPR>
__device__ __forceinline__ float row_min(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v = fminf(v, __shfl_xor(v, m, LPR));
  return v;
}
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, LPR));
  return v;
}
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, LPR);
  return v;
}
// Lane SRC's v to every lane of its LPR-lane row group (LPR = 16: one DPP
// row broadcast; LPR = 32: the broadcast inside each 16-lane row, then
// v_permlane16_swap, which hands each odd row the even row's value and each
// even row the odd row's, so that both halves of the group see the owner's).
template <int LPR, int SRC>
__device__ __forceinline__ float group_bcast(float v) {
  const float r = row_bcast<(SRC & 15)>(v);
  if constexpr (LPR == 16) {
    return r;
  } else {
    static_assert(LPR == 32, "16 or 32 lanes per row");
    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(r), __float_as_uint(r),
                                                     false, false);
    return __uint_as_float(SRC < 16 ? pr[0] : pr[1]);
  }
}

// Exact three-part bf16 split of fp32 values for the trailing update: x = h
// + m + l with h the nearest bf16 of x, m that of x - h and l that of the
// remainder, which has at most 8 significant bits left and so is exact.
__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
// The three-part split of one float (element-wise staging).
__device__ __forceinline__ uint16_t split3(float x, uint16_t& mid, uint16_t& lo) {
  const uint16_t hi = bf16_rne_bits(x);
  const float r = x - bf16_bits_to_f32(hi);
  mid = bf16_rne_bits(r);
  lo = bf16_rne_bits(r - bf16_bits_to_f32(mid));
  return hi;
}
// The same split for a pair, with the hardware's nearest-even conversion of
// two floats at once: each part packed low-first into one word.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2v bf16x2_widen(uint32_t b) {
  const f32x2v v = {__uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u)};
  return v;
}
__device__ __forceinline__ uint32_t split_pair(float x0, float x1, uint32_t& mid, uint32_t& lo) {
  const f32x2v x = {x0, x1};
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
  const f32x2v r = x - bf16x2_widen(hb);
  mid = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2v));
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r - bf16x2_widen(mid), bf16x2v));
  return hb;
}

// The column loop's diagonal blocks of U, once per call: block b (columns
// b0 = QB b ..) as its upper triangle with identity padding past the matrix
// edge, row j scaled by 1 / U_jj, and the 1 / U_jj.  Column j's feedback is
// then its unscaled error x - what times the scaled row, and neither the
// division nor its read sits on the chain from one column to the next.  One
// workgroup per block; thread t does half t % 2 of row t / 2.
__device__ __forceinline__ void ublock_block(const float* __restrict__ U, int64_t d_in,
                                             float* __restrict__ Ub, float* __restrict__ Uinv,
                                             int blk) {
  const int64_t b0 = (int64_t)blk * QB;
  const int bw = (int)min<int64_t>(QB, d_in - b0);
  const int tid = threadIdx.x, r = tid >> 1, h = tid & 1;
  const float diag = (r < bw) ? U[(b0 + r) * d_in + b0 + r] : 1.0f;
  const float sc = 1.0f / diag;
  if (h == 0) Uinv[b0 + r] = sc;
  float* dst = Ub + (int64_t)blk * QB * QB + r * QB + 64 * h;
  const float* src = U + (b0 + min(r, bw - 1)) * d_in + b0;
#pragma unroll 4
  for (int i = 0; i < 64; ++i) {
    const int cc = 64 * h + i;
    const float x = src[min(cc, bw - 1)];  // clamped address, masked below
    const float v = (r < bw && cc < bw) ? (cc >= r ? x : 0.0f) : (r == cc ? 1.0f : 0.0f);
    dst[i] = v * sc;
  }
}

// STATIC: the group parameters are given (static groups, natural groups of
// the original weights, in scales/zeros) and column k of the block uses those
// of group perm[b0 + k] >> gshift (perm may be null: natural order); they are
// staged in LDS per row and column at the start.  Otherwise each group's
// parameters are set at its first column from the current values and
// written to scales/zeros.
//
// One launch takes a group of nblk blocks from column g0 on.  The rows of a
// workgroup are its own for the whole group, so after each block's column
// loop it applies that block's scaled errors to the group's later blocks
// itself (the near update W[rows, later] -= delta U[block, later], the
// operands and products of the trailing update: the errors' three bf16 parts
// staged in LDS, U^T's parts read from memory, six part products per product
// on the matrix cores, summed from zero and subtracted once), and its next
// block starts from those values: no launch per block and none for the near
// updates.
constexpr int EAP = QB + 8;  // LDS pitch (bf16) of the staged error parts
template <bool STATIC, int LPR>
__global__ __launch_bounds__(256) void colloop_kernel(
    float* __restrict__ Wc, uint16_t* __restrict__ E3, int64_t se, const float* __restrict__ Ub,
    const float* __restrict__ Uinv, const uint16_t* __restrict__ Ut3, int64_t su, int64_t d_out,
    int64_t d_in, int64_t g0, int nblk, QSpec q, uint8_t* __restrict__ codes,
    float* __restrict__ scales, float* __restrict__ zeros, float* __restrict__ loss_rows,
    const int32_t* __restrict__ perm) {
  constexpr int CPL = QB / LPR;   // columns per lane
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  static_assert(CPL == 8 && RPB == 16, "16 lanes per row, 16 rows per workgroup");
  __shared__ __attribute__((aligned(16))) float us[QB * UPITCH];
  __shared__ float invd[QB];
  __shared__ __attribute__((aligned(16))) uint16_t ea[3][RPB * EAP];  // the block's error parts
  __shared__ float sps[STATIC ? RPB * QB : 1], spi[STATIC ? RPB * QB : 1],
      spz[STATIC ? RPB * QB : 1];
  const int tid = threadIdx.x;
  const int c = tid & (LPR - 1);  // lane within the row group
  const int rl = tid / LPR;       // row within the workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + rl;
  const bool live = row < d_out;
  const int64_t rr = live ? row : 0;
  const float maxq = (float)q.maxq;
  for (int jb = 0; jb < nblk; ++jb) {
  const int64_t b0 = g0 + (int64_t)jb * QB;
  const int bw = (int)min<int64_t>(QB, d_in - b0);
  if (jb > 0) __syncthreads();  // the previous block's near updates are in Wc, us is free
  float w[CPL];
  {
    // this lane's CPL columns of the row (unconditional loads, masked after)
    const float* src = Wc + rr * d_in + b0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) w[i] = src[min(CPL * c + i, bw - 1)];
#pragma unroll
    for (int i = 0; i < CPL; ++i) w[i] = (CPL * c + i < bw) ? w[i] : 0.0f;
  }
  // this block's diagonal block of U, rows scaled by 1 / U_jj (prepared once
  // per call), and the 1 / U_jj: 16 float4 per thread
  {
    const float4* ub = (const float4*)(Ub + (b0 / QB) * QB * QB);
    float4 v[QB * QB / 4 / 256];
#pragma unroll
    for (int u = 0; u < QB * QB / 4 / 256; ++u) v[u] = ub[u * 256 + tid];
#pragma unroll
    for (int u = 0; u < QB * QB / 4 / 256; ++u) {
      const int e = u * 256 + tid, r = e / (QB / 4), c4 = e % (QB / 4);
      *(float4*)(us + r * UPITCH + 4 * c4) = v[u];
    }
    if (tid < QB) invd[tid] = Uinv[b0 + tid];
  }
  if constexpr (STATIC) {
    for (int e = tid; e < RPB * QB; e += 256) {
      const int rl = e / QB, k = e % QB;
      const int64_t r = min<int64_t>((int64_t)blockIdx.x * RPB + rl, d_out - 1);
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

  GroupParams gp;
  if (q.gsize == 0) {
    gp.s = scales[rr];
    gp.inv_s = 1.0f / gp.s;
    gp.hs = 0.5f * gp.s;
    gp.z = zeros[rr];
    gp.zlo = -gp.z;
    gp.zhi = maxq - gp.z;
  }
  const int gmask = q.gsize - 1;
  // STATIC: the next column's parameters, read one column ahead
  float ns = 0.0f, ni = 0.0f, nz = 0.0f;
  if constexpr (STATIC) {
    const int e = (tid / LPR) * QB;
    ns = sps[e];
    ni = spi[e];
    nz = spz[e];
  }
  float cr[CPL], er[CPL];
  // U row of the next column (this lane's CPL entries), read one column
  // ahead so the LDS latency is off the dependency chain.
  float un[CPL];
  auto read_urow = [&](int jn) __attribute__((always_inline)) {
    const float4* urow = (const float4*)(us + jn * UPITCH + CPL * c);
#pragma unroll
    for (int h = 0; h < CPL / 4; ++h) {
      const float4 v = urow[h];
      un[4 * h] = v.x;
      un[4 * h + 1] = v.y;
      un[4 * h + 2] = v.z;
      un[4 * h + 3] = v.w;
    }
  };
  read_urow(0);
  float xv = w[0];
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
      gp.zlo = -nz;
      gp.zhi = maxq - nz;
      gp.hs = 0.5f * gp.s;
      if constexpr (j + 1 < QB) {
        const int e = (tid / LPR) * QB + j + 1;
        ns = sps[e];
        ni = spi[e];
        nz = spz[e];
      }
    } else if constexpr (j % 32 == 0) {  // every supported group size is a multiple of 32
      if (q.gsize != 0 && (j & gmask) == 0) {
        const bool mine = (CPL * c >= j) && (CPL * c < j + q.gsize);
        float mn = 0.0f, mx = 0.0f;
        if (mine) {
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
            mn = fminf(mn, w[i]);
            mx = fmaxf(mx, q.sym ? fabsf(w[i]) : w[i]);
          }
        }
        mx = row_max<LPR>(mx);
        mn = row_min<LPR>(mn);
        gp = q.sym ? make_params(mx, 0.0f, q.maxq, 1) : make_params(mn, mx, q.maxq, 0);
        if (c == j / CPL && live && j < bw) {
          const int64_t gi = rr * q.n_groups + ((b0 + j) >> q.gshift);
          scales[gi] = gp.s;
          zeros[gi] = gp.z;
        }
      }
    }
    // xv: column j's current value on its owner lane (lane j / CPL).  The
    // owner quantizes it, updates its own next column with its own error, and
    // so carries the chain from column to column without a broadcast as long
    // as the next column is its own; the error reaches the other lanes by a
    // DPP broadcast that only their later columns wait for.
    float code;
    const float e = quantize_step(xv, gp, &code);
    if (c == j / CPL) {
      cr[j % CPL] = code;
      er[j % CPL] = e;
    }
    float uu[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) uu[i] = un[i];
    if constexpr (j + 1 < QB) read_urow(j + 1);
    constexpr int nx = (j + 1) % CPL;
    if constexpr (j + 1 < QB && nx != 0) xv = fmaf(-e, uu[nx], w[nx]);
    // every lane's columns, with the owner's error (the owner's own
    // broadcast is its e, so its next column gets the value xv holds)
    const float eb = group_bcast<LPR, j / CPL>(e);
#pragma unroll
    for (int i = 0; i < CPL; ++i) w[i] = fmaf(-eb, uu[i], w[i]);
    if constexpr (j + 1 < QB && nx == 0) xv = w[0];  // the next lane's first column
  });
  // the scaled errors delta = (x - what) / U_jj of this lane's columns
  // (columns past the edge have x - what = 0), and the row's loss sum_j
  // delta_j^2: this lane's terms, then the row's lanes
  float loss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    er[i] *= invd[CPL * c + i];
    loss = fmaf(er[i], er[i], loss);
  }
  loss = row_sum<LPR>(loss);
  // codes and scaled errors of this lane's columns: the codes as one store
  // of CPL bytes when d_in is a multiple of CPL and codes is aligned to it;
  // the errors split into their three bf16 parts, one store of CPL values per
  // part (they lie in one k chunk: b0 and CPL c are multiples of CPL)
  if (live) {
  uint8_t* cdst = codes + rr * d_in + b0 + CPL * c;
  const int64_t kabs = b0 + CPL * c;
  uint16_t* edst = E3 + (kabs / KC) * 3 * se + rr * KC + kabs % KC;
  if ((d_in % CPL) == 0 && ((uintptr_t)codes % CPL) == 0 && CPL * c + CPL <= bw) {
    uint32_t cw[CPL / 4];
#pragma unroll
    for (int t = 0; t < CPL / 4; ++t)
      cw[t] = (uint32_t)cr[4 * t] | ((uint32_t)cr[4 * t + 1] << 8) |
              ((uint32_t)cr[4 * t + 2] << 16) | ((uint32_t)cr[4 * t + 3] << 24);
    if constexpr (CPL == 8)
      *(uint2*)cdst = make_uint2(cw[0], cw[1]);
    else
      *(uint32_t*)cdst = cw[0];
  } else {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (CPL * c + i < bw) cdst[i] = (uint8_t)cr[i];
  }
  if (CPL * c + CPL <= bw) {
    uint32_t hw[CPL / 2], mw[CPL / 2], lw[CPL / 2];
#pragma unroll
    for (int t = 0; t < CPL / 2; ++t) hw[t] = split_pair(er[2 * t], er[2 * t + 1], mw[t], lw[t]);
    if (jb + 1 < nblk) {  // the parts again, for this workgroup's near updates
      *(uint4*)(&ea[0][rl * EAP + CPL * c]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *(uint4*)(&ea[1][rl * EAP + CPL * c]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      *(uint4*)(&ea[2][rl * EAP + CPL * c]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    if constexpr (CPL == 8) {
      *(uint4*)edst = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *(uint4*)(edst + se) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      *(uint4*)(edst + 2 * se) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
      *(uint2*)edst = make_uint2(hw[0], hw[1]);
      *(uint2*)(edst + se) = make_uint2(mw[0], mw[1]);
      *(uint2*)(edst + 2 * se) = make_uint2(lw[0], lw[1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (CPL * c + i < bw) {
        uint16_t mi, lo;
        edst[i] = split3(er[i], mi, lo);
        edst[se + i] = mi;
        edst[2 * se + i] = lo;
      }
  }
  }  // live
  if (loss_rows && c == 0 && live) loss_rows[rr] = (b0 == 0 ? 0.0f : loss_rows[rr]) + loss;
  if (jb + 1 < nblk) {
    // Rows past d_out hold whatever LDS held: a product keeps rows apart
    // and those rows are never stored.  Every block but the matrix's last is
    // full, so the staged parts cover all 128 columns.
    const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const bool arow = l32 < RPB;  // MFMA rows 16..31 are zero padding
    // U^T parts of target block jt, 32-k chunk kc: this lane's column and k
    auto bload = [&](uint4 (&bb)[2][3], int jt, int kc) __attribute__((always_inline)) {
      const int64_t bt = g0 + (int64_t)jt * QB;
      const int64_t ncol = bt + min(32 * wave + l32, (int)min<int64_t>(QB, d_in - bt) - 1);
      const uint16_t* pb = Ut3 + ((b0 + kc) / KC) * 3 * su + ncol * KC + 8 * h;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) bb[ks][pt] = *(const uint4*)(pb + pt * su + 16 * ks);
    };
    uint4 bq[2][2][3];  // [buffer][16-k step][part]
    // the first target's first two chunks (every later target's come at the
    // end of the one before, so each target starts with them in flight)
    bload(bq[0], jb + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    bload(bq[1], jb + 1, 32);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // ea complete
    for (int jt = jb + 1; jt < nblk; ++jt) {
      const int64_t bt = g0 + (int64_t)jt * QB;
      const int btw = (int)min<int64_t>(QB, d_in - bt);
      const int jn = min(jt + 1, nblk - 1);  // the next target (the last loads itself again)
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
      auto prod = [&](const uint4 (&bb)[2][3], int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int ko = kc + 16 * ks + 8 * h;
          uint4 av[3];
#pragma unroll
          for (int pt = 0; pt < 3; ++pt)
            av[pt] = arow ? *(const uint4*)(&ea[pt][l32 * EAP + ko]) : make_uint4(0, 0, 0, 0);
          const bf16x8 ah = __builtin_bit_cast(bf16x8, av[0]);
          const bf16x8 am = __builtin_bit_cast(bf16x8, av[1]);
          const bf16x8 al = __builtin_bit_cast(bf16x8, av[2]);
          const bf16x8 bh = __builtin_bit_cast(bf16x8, bb[ks][0]);
          const bf16x8 bm = __builtin_bit_cast(bf16x8, bb[ks][1]);
          const bf16x8 bl = __builtin_bit_cast(bf16x8, bb[ks][2]);
          // the six part products, smallest first: l h, h l, m m, m h, h m, h h
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bm, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
        }
      };
      // the target's current values (registers 0..7 of the product hold the
      // 16 real rows, 8 (r / 4) + 4 h + r % 4), read before the products
      const int cl = 32 * wave + l32;
      float* col = Wc + bt + min(cl, btw - 1);
      float old[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t gr = (int64_t)blockIdx.x * RPB + 8 * (r >> 2) + 4 * h + (r & 3);
        old[r] = col[min(gr, d_out - 1) * d_in];
      }
      __builtin_amdgcn_sched_barrier(0);
      // four 32-k chunks, each next one's U^T parts loaded during the products,
      // then the next target's first two
      prod(bq[0], 0);
      bload(bq[0], jt, 64);
      __builtin_amdgcn_sched_barrier(0);
      prod(bq[1], 32);
      bload(bq[1], jt, 96);
      __builtin_amdgcn_sched_barrier(0);
      prod(bq[0], 64);
      bload(bq[0], jn, 0);
      __builtin_amdgcn_sched_barrier(0);
      prod(bq[1], 96);
      bload(bq[1], jn, 32);
      __builtin_amdgcn_sched_barrier(0);
      if (cl < btw) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int64_t gr = (int64_t)blockIdx.x * RPB + 8 * (r >> 2) + 4 * h + (r & 3);
          if (gr < d_out) col[gr * d_in] = old[r] - acc[r];
        }
      }
    }
  }
  }  // blocks of the group
}

// Wc[:, n0:n1] -= delta[:, b0:b0+kb] * U[b0:b0+kb, n0:n1] on the bf16 matrix
// cores.  Both operands come already split into their three bf16 parts (the
// column loop splits the errors it writes, uprep_kernel splits U^T once
// per call), and the product is formed from the six part products that
// matter,
//   l*h + h*l + m*m + m*h + h*m + h*h,
// with v_mfma_f32_32x32x16_bf16 into fp32 accumulators, smallest first.  The
// dropped terms (m*l, l*m, l*l) come to at most about 2^-23 of the product
// (|m| <= 2^-8 |x|, |l| <= 2^-16 |x|), so each product carries an error of
// about one fp32 rounding, as with fp32 FMAs; the feedback is then as exact
// as fp32 working weights allow.  TM x 64 tiles, K in chunks of 32 (two MFMA
// steps of 16): a chunk of one part is one contiguous run of the k-chunk
// major operands, loaded 16 bytes per lane.  The LDS tile of U^T holds
// k-contiguous rows, so every lane reads its 8 consecutive k as 16 bytes; a
// row pitch of 80 bytes keeps those reads free of bank conflicts.  The accumulators start at zero and collect delta U, and Wc
// - acc is stored: summed onto a preloaded Wc instead, every one of the K
// roundings would be at the weights' magnitude rather than the products'.
constexpr int T3K = KC;           // k per chunk
constexpr int T3P = T3K + 8;      // LDS row pitch (bf16 elements): 80 bytes

// U^T split into parts: part p of U[k][n] goes to Ut3 at chunk k / 32, part
// p, row n, position k % 32, for the 64 x 64 tiles (k block kt, n block nt)
// with kt <= nt (the update reads k < n only).  The tile goes through LDS so
// that the loads of U's rows and the stores of U^T's rows are contiguous.
__device__ __forceinline__ void split_ut_tile(const float* __restrict__ U, int64_t d_in,
                                              uint16_t* __restrict__ Ut3, int64_t su, int tile) {
  __shared__ float t[64][65];
  int nt = (int)((sqrtf(8.0f * (float)tile + 1.0f) - 1.0f) * 0.5f);
  while ((nt + 1) * (nt + 2) / 2 <= tile) ++nt;
  while (nt * (nt + 1) / 2 > tile) --nt;
  const int kt = tile - nt * (nt + 1) / 2;
  const int64_t k0 = 64 * (int64_t)kt, n0 = 64 * (int64_t)nt;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;  // r = k, c = n
    const int64_t k = k0 + r, n = n0 + c;
    t[r][c] = (k < d_in && n < d_in) ? U[k * d_in + n] : 0.0f;
  }
  __syncthreads();
  // thread: row n = tid % 64 of U^T, 16 consecutive k from 16 (tid / 64)
  // (a wave's stores of one part are 64 rows x 32 bytes of one chunk)
  const int nl = tid & 63, kl = 16 * (tid >> 6);
  const int64_t n = n0 + nl;
  if (n >= d_in || k0 + kl >= d_in) return;
  uint16_t* dst = Ut3 + ((k0 + kl) / KC) * 3 * su + n * KC + (k0 + kl) % KC;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t hw[4], mw[4], lw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      hw[q] = split_pair(t[kl + 8 * h + 2 * q][nl], t[kl + 8 * h + 2 * q + 1][nl], mw[q], lw[q]);
    *(uint4*)(dst + 8 * h) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *(uint4*)(dst + su + 8 * h) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
    *(uint4*)(dst + 2 * su + 8 * h) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// Once per call, in one launch: the column loop's scaled diagonal blocks of
// U (workgroups 0 .. nblk - 1, first, as they take longest), U^T's bf16 parts
// for the trailing updates (the next nsplit), and, when nq > 0, the working
// copy Wc of W (the last nq: qinit_part).
__global__ __launch_bounds__(256) void uprep_kernel(const float* __restrict__ U, int64_t d_in,
                                                    float* __restrict__ Ub,
                                                    float* __restrict__ Uinv,
                                                    uint16_t* __restrict__ Ut3, int64_t su,
                                                    int nblk, int nsplit, const void* W,
                                                    int w_dtype, int64_t d_out,
                                                    const uint8_t* __restrict__ dead,
                                                    float* __restrict__ Wc, int vec, int nq) {
  const int b = (int)blockIdx.x;
  if (b < nblk)
    ublock_block(U, d_in, Ub, Uinv, b);
  else if (b < nblk + nsplit)
    split_ut_tile(U, d_in, Ut3, su, b - nblk);
  else
    qinit_part(W, w_dtype, d_out, d_in, dead, Wc, vec, b - nblk - nsplit, nq);
}

// The launches give b0 and kb multiples of 32 (whole chunks) and n0 a
// multiple of 64; rows past d_out and columns past n1 are loaded as clamped
// copies of finite values, which only reach accumulator rows or columns that
// are never stored.
//
// Operand paths: each wave's error rows are its own (no other wave of the
// workgroup reads them), so a lane loads its MFMA fragments of them straight
// from memory into registers, 16 bytes per part and 16-k step, one chunk
// ahead of the products; only the rows of U^T, which every wave of a column
// of the wave grid reads, go through LDS.  Against staging both operands in
// LDS this takes the error tile's LDS stores and reads off the LDS port,
// which bound the kernel.
template <int TM, int TN>
__global__ __launch_bounds__(256, (TM * TN >= 128 * 128) ? 2 : 1) void trailing3_kernel(
                                                        float* __restrict__ Wc,
                                                        const uint16_t* __restrict__ E3, int64_t se,
                                                        const uint16_t* __restrict__ Ut3,
                                                        int64_t su, int64_t d_out, int64_t d_in,
                                                        int64_t b0, int kb, int64_t n0,
                                                        int64_t n1) {
  // each wave owns RB x CB of the tile's 32 x 32 blocks: the waves form a
  // WR x WC grid over the tile's (TM / 32) x (TN / 32) blocks
  constexpr int NBLK = (TM / 32) * (TN / 32) / 4;  // 32 x 32 blocks per wave
  static_assert(NBLK == 1 || NBLK == 2 || NBLK == 4, "tile shape");
  constexpr int RB = NBLK == 4 ? 2 : 1, CB = NBLK / RB;
  constexpr int WC = (TN / 32) / CB;
  static_assert(WC >= 1 && 4 % WC == 0 && (TM / 32) == (4 / WC) * RB, "wave grid");
  constexpr int VQ = TN * T3K / 8 / 256;  // 16-byte pieces per thread and part (U^T)
  static_assert(VQ >= 1, "whole pieces");
  constexpr int KS = T3K / 16;            // 16-k MFMA steps per chunk
  __shared__ __attribute__((aligned(16))) uint16_t bh[TN * T3P], bmid[TN * T3P], bl[TN * T3P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wr = wave / WC, wc = wave % WC;
  const int64_t ncols = n1 - n0;
  const int ntn = (int)ceil_div(ncols, TN);
  const int ntm = (int)ceil_div(d_out, TM);
  // XCD-aware tile order.  Workgroup ids go to the eight XCDs round-robin,
  // and each XCD's L2 is its own, so id t = 8 i + x takes rank x T8 + i (T8 =
  // ranks per XCD) of an order in which consecutive ranks are close: row
  // bands of a quarter of the row tiles, and inside a band column after
  // column.  Each XCD then holds a quarter of the rows by half of the
  // columns, and fetches a quarter of the errors and half of U^T instead of
  // all the errors.  The grid is rounded up to a multiple of eight; the
  // padding ranks exit.
  const int ntiles = ntm * ntn;
  const int t8 = (int)ceil_div(ntiles, 8);
  const int rank = ((int)blockIdx.x % 8) * t8 + (int)blockIdx.x / 8;
  if (rank >= ntiles) return;
  const int hb = (int)ceil_div(ntm, 4);
  const int band = rank / (hb * ntn), within = rank % (hb * ntn);
  const int bh_rows = min(hb, ntm - band * hb);
  const int64_t m0 = (int64_t)(band * hb + within % bh_rows) * TM;
  const int64_t n0t = n0 + (int64_t)(within / bh_rows) * TN;
  const int rows = (int)min<int64_t>(TM, d_out - m0);
  const int cols = (int)min<int64_t>(TN, n1 - n0t);
  float* C = Wc + m0 * d_in + n0t;
  f32x16 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // this lane's error rows (clamped) and k offset inside a 16-k step
  int64_t offa[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int r = 32 * (wr * RB + i) + l32;
    offa[i] = (m0 + (r < rows ? r : rows - 1)) * KC + 8 * h;
  }
  // this thread's pieces of the U^T tile: tile row (clamped), k offset 8 (e % 4)
  int64_t offq[VQ];
#pragma unroll
  for (int j = 0; j < VQ; ++j) {
    const int e = j * 256 + tid, r = e >> 2;
    offq[j] = (n0t + (r < cols ? r : cols - 1)) * KC + 8 * (e & 3);
  }
  // staged U^T chunk, as 32-bit words (arrays of scalars stay in registers)
  uint32_t xq[3 * VQ * 4];
  auto gload = [&](int kc) __attribute__((always_inline)) {
    const uint16_t* pb = Ut3 + ((b0 + kc) / KC) * 3 * su;
#pragma unroll
    for (int pt = 0; pt < 3; ++pt)
#pragma unroll
      for (int j = 0; j < VQ; ++j) {
        const uint4 v = *(const uint4*)(pb + pt * su + offq[j]);
        const int x = 4 * (3 * j + pt);
        xq[x] = v.x;
        xq[x + 1] = v.y;
        xq[x + 2] = v.z;
        xq[x + 3] = v.w;
      }
  };
  auto lstore = [&]() __attribute__((always_inline)) {
    uint16_t* const pb[3] = {bh, bmid, bl};
#pragma unroll
    for (int pt = 0; pt < 3; ++pt)
#pragma unroll
      for (int j = 0; j < VQ; ++j) {
        const int e = j * 256 + tid, r = e >> 2, c = 8 * (e & 3);
        const int x = 4 * (3 * j + pt);
        *(uint4*)(pb[pt] + r * T3P + c) = make_uint4(xq[x], xq[x + 1], xq[x + 2], xq[x + 3]);
      }
  };
  // the error fragments of one chunk: [row block][16-k step][part]
  typedef uint4 AFrag[RB][KS][3];
  auto aload = [&](AFrag& a, int kc) __attribute__((always_inline)) {
    const uint16_t* pa = E3 + ((b0 + kc) / KC) * 3 * se;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pt = 0; pt < 3; ++pt)
          a[i][ks][pt] = *(const uint4*)(pa + pt * se + offa[i] + 16 * ks);
  };
  auto products = [&](const AFrag& a) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ko = 16 * ks + 8 * h;
      bf16x8 b3[CB][3];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int br = (32 * (wc * CB + j) + l32) * T3P + ko;
        b3[j][0] = *(const bf16x8*)(bh + br);
        b3[j][1] = *(const bf16x8*)(bmid + br);
        b3[j][2] = *(const bf16x8*)(bl + br);
      }
      // the six part products, smallest first: l h, h l, m m, m h, h m, h h
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const bf16x8 ah = __builtin_bit_cast(bf16x8, a[i][ks][0]);
        const bf16x8 am = __builtin_bit_cast(bf16x8, a[i][ks][1]);
        const bf16x8 al = __builtin_bit_cast(bf16x8, a[i][ks][2]);
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          f32x16 c = acc[i][j];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b3[j][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b3[j][2], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, b3[j][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, b3[j][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b3[j][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b3[j][0], c, 0, 0, 0);
          acc[i][j] = c;
        }
      }
    }
  };
  // one chunk: publish its U^T rows in LDS, start the loads of chunk kn,
  // multiply with this chunk's error fragments (a); chunk kn's go to an.
  // The loads are unconditional (the last chunk loads itself again), so
  // every path has the same loads in flight and the wait before the
  // products only covers the fragments they use; a branch around them made
  // the compiler wait for every load there.
  auto chunk = [&](const AFrag& a, AFrag& an, int kc, int kn) __attribute__((always_inline)) {
    if (kc > 0) __syncthreads();  // the previous chunk's products are done with LDS
    lstore();
    __syncthreads();
    gload(kn);
    __builtin_amdgcn_sched_barrier(0);
    aload(an, kn);
    // keep the loads ahead of the products and in the same order on every
    // path (the scheduler would otherwise sink them next to their first use,
    // a chunk later in program order but not in time)
    __builtin_amdgcn_sched_barrier(0);
    products(a);
  };
  // the launches give kb a multiple of 4 chunks (whole 128-column blocks)
  AFrag a0, a1;
  gload(0);
  __builtin_amdgcn_sched_barrier(0);
  aload(a0, 0);
  __builtin_amdgcn_sched_barrier(0);
  const int klast = kb - T3K;
  for (int kc = 0; kc < kb; kc += 2 * T3K) {
    chunk(a0, a1, kc, min(kc + T3K, klast));
    chunk(a1, a0, kc + T3K, min(kc + 2 * T3K, klast));
  }
  // per block: its old values, the 16 loads in flight together (clamped
  // addresses), then Wc - acc
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      float old[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 32 * (wr * RB + i) + 8 * (q >> 2) + 4 * h + (q & 3);
        const int c = 32 * (wc * CB + j) + l32;
        old[q] = C[(int64_t)(r < rows ? r : rows - 1) * d_in + (c < cols ? c : cols - 1)];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 32 * (wr * RB + i) + 8 * (q >> 2) + 4 * h + (q & 3);
        const int c = 32 * (wc * CB + j) + l32;
        if (r < rows && c < cols) C[(int64_t)r * d_in + c] = old[q] - acc[i][j][q];
      }
    }
}

// ---- pack -------------------------------------------------------------------
// CPW > 0: bits divides 32, a row is a whole number of words (CPW = 32 /
// bits codes each) and codes is aligned to CPW bytes, so word e holds codes
// e CPW .. e CPW + CPW - 1 of the row-major matrix, read as one load.
template <int CPW>
__device__ __forceinline__ uint32_t pack_word(const uint8_t* __restrict__ codes, int64_t e) {
  constexpr int B = 32 / CPW;
  constexpr uint32_t MASK = (1u << B) - 1;
  uint32_t b[CPW / 4];
  if constexpr (CPW == 16) {
    const uint4 v = *(const uint4*)(codes + 16 * e);
    b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
  } else if constexpr (CPW == 8) {
    const uint2 v = *(const uint2*)(codes + 8 * e);
    b[0] = v.x; b[1] = v.y;
  } else {
    b[0] = *(const uint32_t*)(codes + 4 * e);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < CPW; ++k) acc |= ((b[k / 4] >> (8 * (k % 4))) & MASK) << (B * k);
  return acc;
}

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t d_out, int64_t d_in, int bits,
                                                         int64_t words, uint32_t* __restrict__ qw,
                                                         int cpw) {
  const int64_t total = d_out * words;
  if (cpw) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256)
      qw[e] = (cpw == 16) ? pack_word<16>(codes, e)
              : (cpw == 8) ? pack_word<8>(codes, e) : pack_word<4>(codes, e);
    return;
  }
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
  const size_t per_chunk = 3 * KC * sizeof(uint16_t);  // three parts of 32 k
  return align256((size_t)d_out * d_in * sizeof(float)) +
         align256((size_t)n_chunks(d_in) * per_chunk * d_out) +
         align256((size_t)n_chunks(d_in) * per_chunk * d_in) +
         align256((size_t)n_blocks(d_in) * QB * (QB + 1) * sizeof(float));
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
  // One matrix in natural order: its working copy is made in the same launch
  // as U's preparation (below); otherwise here.
  const bool q_merged = !perm && src.count == 1 && d_out > 0;
  const int q_vec = (d_in % 8 == 0) && ((uintptr_t)W % 16 == 0);
  if (perm) {
    hipLaunchKernelGGL(qinit_perm_kernel, pgrid, dim3(256), 0, stream, W, w_dtype, d_out, d_in,
                       dead, perm, w.Wc);
  } else if (!q_merged) {
    int64_t r0 = 0;
    for (int i = 0; i < src.count; ++i) {
      const int64_t rows = src.rows[i];
      if (rows == 0) continue;
      const int vec = (d_in % 8 == 0) && ((uintptr_t)src.ptrs[i] % 16 == 0);
      hipLaunchKernelGGL(qinit_kernel, dim3(qinit_grid(rows, d_in, vec)), dim3(256), 0, stream,
                         src.ptrs[i], w_dtype, rows, d_in, dead, w.Wc + r0 * d_in, vec);
      r0 += rows;
    }
  }
  // the scaled diagonal blocks of U, and U^T in parts for every trailing
  // update of this call (only the 64 x 64 tiles on or above U's diagonal)
  {
    const int64_t nt = ceil_div(d_in, 64);
    const int nsplit = (d_in > QB) ? (int)(nt * (nt + 1) / 2) : 0;
    const int nblk_u = (int)n_blocks(d_in);
    const int nq = q_merged ? (int)qinit_grid(d_out, d_in, q_vec) : 0;
    hipLaunchKernelGGL(uprep_kernel, dim3((unsigned)(nblk_u + nsplit + nq)), dim3(256), 0, stream,
                       U, d_in, w.Ub, w.Uinv, w.Ut3, w.su, nblk_u, nsplit, W, w_dtype, d_out,
                       dead, w.Wc, q_vec, nq);
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
  const unsigned rgrid = (unsigned)ceil_div(d_out, 256 / CL_LPR);
  static_assert(QB % T3K == 0, "trailing updates take whole chunks");

  const int64_t nb = ceil_div(d_in, QB);
  for (int64_t g0 = 0; g0 < nb; g0 += QG) {
    const int64_t gend = std::min<int64_t>(nb, g0 + QG);
    const int64_t gcol = std::min<int64_t>(d_in, gend * QB);  // first column after the group
    // the group's column loops and their near updates, one launch
    const int nblk = (int)(gend - g0);
    if (stat)
      hipLaunchKernelGGL((colloop_kernel<true, CL_LPR>), dim3(rgrid), dim3(256), 0, stream, w.Wc,
                         w.E3, w.se, w.Ub, w.Uinv, (const uint16_t*)w.Ut3, w.su, d_out, d_in,
                         g0 * QB, nblk, q, codes_k, scales, zeros, loss_rows, perm);
    else
      hipLaunchKernelGGL((colloop_kernel<false, CL_LPR>), dim3(rgrid), dim3(256), 0, stream, w.Wc,
                         w.E3, w.se, w.Ub, w.Uinv, (const uint16_t*)w.Ut3, w.su, d_out, d_in,
                         g0 * QB, nblk, q, codes_k, scales, zeros, loss_rows, perm);
    if (gcol < d_in) {  // every block of the group is full
      // 128 x 128 tiles (half the LDS bytes per product, two waves per SIMD)
      // when the launch still has enough of them to fill the chip several
      // times over, else 128 x 64 (three waves per SIMD)
      const int kb = (int)(gcol - g0 * QB);
      const int64_t big = ceil_div(d_out, 128) * ceil_div(d_in - gcol, 128);
      const int64_t small = ceil_div(d_out, 128) * ceil_div(d_in - gcol, 64);
      if (big >= FAR_BIG_MIN)
        hipLaunchKernelGGL((trailing3_kernel<128, 128>), dim3((unsigned)(8 * ceil_div(big, 8))),
                           dim3(256), 0, stream, w.Wc, (const uint16_t*)w.E3, w.se,
                           (const uint16_t*)w.Ut3, w.su, d_out, d_in, g0 * QB, kb, gcol, d_in);
      else
        hipLaunchKernelGGL((trailing3_kernel<128, 64>), dim3((unsigned)(8 * ceil_div(small, 8))),
                           dim3(256), 0, stream, w.Wc, (const uint16_t*)w.E3, w.se,
                           (const uint16_t*)w.Ut3, w.su, d_out, d_in, g0 * QB, kb, gcol, d_in);
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
  const int cpw = (32 % bits == 0) ? 32 / bits : 0;
  const int fast = (cpw >= 4 && cpw <= 16 && d_in % cpw == 0 && (uintptr_t)codes % cpw == 0)
                       ? cpw : 0;
  if (total > 0)
    hipLaunchKernelGGL(pack_codes_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(total, 256), 65536)), dim3(256),
                       0, stream, codes, d_out, d_in, bits, words, qweight, fast);
  const int64_t nm = d_out * n_groups;
  if (nm > 0)
    hipLaunchKernelGGL(pack_meta_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(nm, 256), 65536)), dim3(256), 0,
                       stream, scales, zeros, nm, scales_f16, sym ? (uint16_t*)nullptr : zeros_f16);
  return hipGetLastError();
}

}  // namespace gptq
