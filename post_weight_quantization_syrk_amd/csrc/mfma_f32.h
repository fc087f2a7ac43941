// fp32 MFMA tile product through LDS (v_mfma_f32_32x32x2f32), used by the
// factorization updates and by the trailing update of the column loop.
//
//   C[TM x TN] (+)= P[TM x K] * Q[K x TN]
//
// 256 threads = 4 waves in a 2 x 2 grid; each wave owns a (TM/2) x (TN/2)
// sub-tile made of 32 x 32 MFMA tiles.  Operand lane layout (32x32x2 f32):
// A: lane l holds A[m = l%32][k = l/32]; B: lane l holds B[k = l/32][n = l%32];
// C: register r of lane l is C[8(r/4) + 4(l/32) + r%4][l%32].
//
// LDS layouts (fp32 words; 64 banks of 4 bytes):
//   P is kept row-major [m][k] with a row pitch p == 2 (mod 32): the 32 lanes
//   of an A read hit rows r = 0..31 at one column, banks (p r) mod 64 =
//   2 ((p/2) r mod 32) with p/2 odd -> 32 distinct even banks, and the other
//   32 lanes (column k+1) -> odd banks.  No conflicts.  Q given transposed (Q^T
//   row-major [n][k]) uses the same layout; Q given row-major [k][n] uses a row
//   pitch == 32 (mod 64) so the two half-waves (rows k and k+1) fall in
//   disjoint bank halves.
#pragma once

#include "common.h"

#include <type_traits>

namespace gptq {

template <int TM, int TN, int K, bool QT>
struct MfmaTile {
  static constexpr int PP = K + 2 + ((K % 32) ? 32 - (K % 32) : 0);  // == 2 (mod 32)
  static constexpr int PQN = TN + 32 + ((TN % 64) ? 64 - (TN % 64) : 0);  // == 32 (mod 64)
  static constexpr int QROWS = QT ? TN : K;
  static constexpr int QPITCH = QT ? PP : PQN;
  static constexpr int WM = TM / 2, WN = TN / 2;  // per-wave sub-tile
  static constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && K % 2 == 0, "tile shape");
  static constexpr size_t lds_floats = (size_t)TM * PP + (size_t)QROWS * QPITCH;
  static constexpr int lds_q_offset = TM * PP;  // where the Q operand starts in LDS

  // Copy an R x C block (rows x cols valid, zero-padded) from row-major global
  // memory into LDS with the given pitch.  Loads are unconditional (addresses
  // clamped into the valid block, values masked afterwards) and issued in
  // batches of 16 per thread, so they are all in flight together instead of
  // one guarded load per memory round trip.  Needs rows, cols >= 1.
  template <int R, int C, int PITCH>
  __device__ static void load_block(float* dst, const float* __restrict__ src, int64_t ld,
                                    int rows, int cols) {
    constexpr int N = R * C / 256;
    static_assert(R * C % 256 == 0, "block size");
    constexpr int BATCH = N < 16 ? N : 16;
#pragma unroll
    for (int b0 = 0; b0 < N; b0 += BATCH) {
      float v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int e = (b0 + u) * 256 + threadIdx.x;
        const int r = e / C, c = e % C;
        const int rc = r < rows ? r : rows - 1, cc = c < cols ? c : cols - 1;
        v[u] = src[(int64_t)rc * ld + cc];
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int e = (b0 + u) * 256 + threadIdx.x;
        const int r = e / C, c = e % C;
        dst[r * PITCH + c] = (r < rows && c < cols) ? v[u] : 0.0f;
      }
    }
  }
  // Load P (rows x K valid; zero-padded) from row-major global memory.
  __device__ static void load_p(float* lds, const float* __restrict__ src, int64_t ld, int rows,
                                int cols) {
    load_block<TM, K, PP>(lds, src, ld, rows, cols);
  }
  // Load Q: if QT, src is Q^T row-major [TN][K] (rows = valid n, cols = valid k);
  // else src is Q row-major [K][TN] (rows = valid k, cols = valid n).
  __device__ static void load_q(float* lds, const float* __restrict__ src, int64_t ld, int rows,
                                int cols) {
    constexpr int R = QT ? TN : K, C = QT ? K : TN;
    load_block<R, C, QPITCH>(lds + TM * PP, src, ld, rows, cols);
  }
  // Operands of one chunk held in registers between their loads and their
  // stores to LDS, so the next chunk's loads can be in flight while the
  // current one multiplies.
  static constexpr int NPR = TM * K / 256;
  static constexpr int NQR = (QT ? TN * K : K * TN) / 256;
  struct PQRegs {
    float p[NPR];
    float q[NQR];
  };
  // Unconditional loads from clamped addresses (rows, cols >= 1).
  __device__ static void fetch_pq(PQRegs& v, const float* __restrict__ ps, int64_t pld,
                                  int prows, int pcols, const float* __restrict__ qs,
                                  int64_t qld, int qrows, int qcols) {
    constexpr int QR = QT ? TN : K, QC = QT ? K : TN;
#pragma unroll
    for (int u = 0; u < NPR; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / K, c = e % K;
      const int rc = r < prows ? r : prows - 1, cc = c < pcols ? c : pcols - 1;
      v.p[u] = ps[(int64_t)rc * pld + cc];
    }
#pragma unroll
    for (int u = 0; u < NQR; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / QC, c = e % QC;
      const int rc = r < qrows ? r : qrows - 1, cc = c < qcols ? c : qcols - 1;
      v.q[u] = qs[(int64_t)rc * qld + cc];
    }
    (void)QR;
  }
  // Into LDS, zero outside the valid block; NEG negates P (so products
  // accumulate with a minus sign onto preloaded accumulators).
  template <bool NEG>
  __device__ static void stage_pq(float* lds, const PQRegs& v, int prows, int pcols, int qrows,
                                  int qcols) {
    constexpr int QC = QT ? K : TN;
#pragma unroll
    for (int u = 0; u < NPR; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / K, c = e % K;
      lds[r * PP + c] = (r < prows && c < pcols) ? (NEG ? -v.p[u] : v.p[u]) : 0.0f;
    }
    float* lq = lds + TM * PP;
#pragma unroll
    for (int u = 0; u < NQR; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / QC, c = e % QC;
      lq[r * QPITCH + c] = (r < qrows && c < qcols) ? v.q[u] : 0.0f;
    }
  }

  // P and Q together with every load of both in flight at once (one memory
  // round trip; needs (TM*K + K*TN)/256 staging registers per thread).
  __device__ static void load_pq(float* lds, const float* __restrict__ ps, int64_t pld, int prows,
                                 int pcols, const float* __restrict__ qs, int64_t qld, int qrows,
                                 int qcols) {
    constexpr int NP = TM * K / 256;
    constexpr int QR = QT ? TN : K, QC = QT ? K : TN;
    constexpr int NQ = QR * QC / 256;
    static_assert(TM * K % 256 == 0 && QR * QC % 256 == 0, "block size");
    float vp[NP], vq[NQ];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / K, c = e % K;
      const int rc = r < prows ? r : prows - 1, cc = c < pcols ? c : pcols - 1;
      vp[u] = ps[(int64_t)rc * pld + cc];
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / QC, c = e % QC;
      const int rc = r < qrows ? r : qrows - 1, cc = c < qcols ? c : qcols - 1;
      vq[u] = qs[(int64_t)rc * qld + cc];
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / K, c = e % K;
      lds[r * PP + c] = (r < prows && c < pcols) ? vp[u] : 0.0f;
    }
    float* lq = lds + TM * PP;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int r = e / QC, c = e % QC;
      lq[r * QPITCH + c] = (r < qrows && c < qcols) ? vq[u] : 0.0f;
    }
  }

  __device__ static void zero(f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  }

  __device__ static void mma(const float* lds, f32x16 (&acc)[FM][FN]) {
    const float* p = lds;
    const float* q = lds + TM * PP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int kl = lane >> 5, ml = lane & 31;
#pragma unroll 4
    for (int k = 0; k < K; k += 2) {
      float av[FM], bv[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) av[a] = p[(wm * WM + 32 * a + ml) * PP + k + kl];
#pragma unroll
      for (int b = 0; b < FN; ++b)
        bv[b] = QT ? q[(wn * WN + 32 * b + ml) * QPITCH + k + kl]
                   : q[(k + kl) * QPITCH + wn * WN + 32 * b + ml];
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }

  // C[row][col] -= acc (or = acc) for rows < rows, cols < cols (both >= 1).
  // All loads of C are issued before any store so the read-modify-write is
  // not serialised on possible aliasing between the stores and later loads.
  template <bool SUB>
  __device__ static void store(float* C, int64_t ld, int rows, int cols,
                               const f32x16 (&acc)[FM][FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    // One row of MFMA tiles at a time: its loads all in flight, then its
    // stores (bounds the registers held for the old values).
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      float old[FN][16];
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WM + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * WN + 32 * b + (lane & 31);
          // unconditional load from a clamped address: guarded loads would each
          // wait for their own memory round trip
          const int rr = row < rows ? row : rows - 1, cc = col < cols ? col : cols - 1;
          old[b][r] = SUB ? C[(int64_t)rr * ld + cc] : 0.0f;
        }
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WM + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * WN + 32 * b + (lane & 31);
          if (row < rows && col < cols)
            C[(int64_t)row * ld + col] = SUB ? old[b][r] - acc[a][b][r] : acc[a][b][r];
        }
    }
  }

  // Set every accumulator element to f(row, col) of its place in the tile.
  template <class F>
  __device__ static void set_each(f32x16 (&acc)[FM][FN], F&& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WM + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * WN + 32 * b + (lane & 31);
          acc[a][b][r] = f(row, col);
        }
  }

  // Visit every accumulator element with its (row, col) inside the tile.
  template <class F>
  __device__ static void for_each(const f32x16 (&acc)[FM][FN], F&& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WM + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * WN + 32 * b + (lane & 31);
          f(row, col, acc[a][b][r]);
        }
  }
};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, B>{});
    StaticFor<B + 1, E>::run(f);
  }
};
template <int E>
struct StaticFor<E, E> {
  template <class F>
  __device__ __forceinline__ static void run(F&&) {}
};

}  // namespace gptq
