// Drives every entry point of include/gptq.h through its argument checks,
// against the stand-in launchers of stub_launchers.cpp: the status each call
// must return, and that a rejected call launches nothing.  Built and run
// under the address and undefined-behaviour sanitizers by the tests; buffers
// are host memory the stand-ins never touch, and per-call arrays (the layer
// lists) are heap blocks of exactly the given length, so a read past them is
// reported.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "gptq.h"

extern int g_launches;

namespace {
int g_fails = 0, g_checks = 0;

void check(int got, int want, int launches_before, const char* what, int line) {
  ++g_checks;
  const int launched = g_launches - launches_before;
  if (got != want) {
    std::printf("FAIL line %d: %s returned %d, want %d\n", line, what, got, want);
    ++g_fails;
  }
  if (want != GPTQ_OK && launched != 0) {
    std::printf("FAIL line %d: %s was rejected but launched %d kernels\n", line, what, launched);
    ++g_fails;
  }
}
#define EXPECT(call, want)                        \
  do {                                            \
    const int lb_ = g_launches;                   \
    check((call), (want), lb_, #call, __LINE__);  \
  } while (0)
#define EXPECT_TRUE(cond)                                          \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(cond)) {                                                 \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);          \
      ++g_fails;                                                   \
    }                                                              \
  } while (0)

void* aligned_block(size_t bytes) {
  void* p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
  std::memset(p, 0, (bytes + 255) / 256 * 256);
  return p;
}
}  // namespace

int main() {
  const gptq_stream s0 = nullptr;
  void* ws = aligned_block(1 << 20);
  void* ws_mis = (char*)ws + 64;  // not 256-byte aligned
  float* H = (float*)aligned_block(4096);
  float* U = (float*)aligned_block(4096);
  uint8_t* dead = (uint8_t*)aligned_block(256);
  int32_t* st = (int32_t*)aligned_block(256);
  void* X = aligned_block(4096);
  uint8_t* codes = (uint8_t*)aligned_block(4096);
  float* sc = (float*)aligned_block(4096);
  float* zr = (float*)aligned_block(4096);
  uint32_t* qw = (uint32_t*)aligned_block(4096);
  uint16_t* s16 = (uint16_t*)aligned_block(4096);
  uint16_t* z16 = (uint16_t*)aligned_block(4096);
  int32_t* perm = (int32_t*)aligned_block(4096);
  double* dv = (double*)aligned_block(4096);

  // ---- version and messages
  EXPECT_TRUE(gptq_abi_version() == 100);
  for (int c = -8; c < 8; ++c) EXPECT_TRUE(gptq_strerror(c) != nullptr);

  // ---- Hessian
  const size_t hw = gptq_hessian_workspace(300, 5000, GPTQ_BF16);
  EXPECT_TRUE(hw > 0 && hw <= (1 << 20));
  EXPECT_TRUE(gptq_hessian_workspace(0, 10, GPTQ_BF16) == 0);
  EXPECT_TRUE(gptq_hessian_workspace(10, -1, GPTQ_BF16) == 0);
  EXPECT_TRUE(gptq_hessian_workspace(10, 10, 7) == 0);
  EXPECT_TRUE(gptq_hessian_workspace(10, 0, GPTQ_F32) == 0);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 5000, 300, ws, hw, s0), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_F32, 10, 320, nullptr, 0, s0), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 0, 300, nullptr, 0, s0), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate(H, 0, X, GPTQ_BF16, 10, 300, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, ((int64_t)1 << 20) + 1, X, GPTQ_BF16, 10, ((int64_t)1 << 21), ws,
                                 hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, -1, 300, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 10, 299, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, 5, 10, 300, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(nullptr, 300, X, GPTQ_BF16, 10, 300, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, nullptr, GPTQ_BF16, 10, 300, ws, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 5000, 300, ws, hw - 1, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 5000, 300, ws_mis, hw, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(H, 300, X, GPTQ_BF16, 5000, 300, nullptr, hw, s0), GPTQ_EINVAL);
  // without allocation
  EXPECT_TRUE(gptq_noalloc_scratch_bytes() == ((size_t)64 << 20));
  EXPECT(gptq_hessian_accumulate_noalloc(H, 300, X, GPTQ_BF16, 5000, 300, s0), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate_noalloc(H, 300, X, GPTQ_BF16, 0, 300, s0), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate_noalloc(H, 300, nullptr, GPTQ_BF16, 10, 300, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate_noalloc(H, 300, X, GPTQ_BF16, 10, 10, s0), GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate_noalloc(H, 900000, X, GPTQ_BF16, 100000000, 900000, s0),
         GPTQ_EUNSUPPORTED);

  // ---- damping, factorization, U
  const size_t pw = gptq_prepare_workspace(300);
  EXPECT_TRUE(pw > 0 && gptq_prepare_workspace(0) == 0 && gptq_prepare_workspace(-5) == 0);
  EXPECT(gptq_prepare_hinv(H, 300, 0.01, U, dead, st, ws, pw, s0), GPTQ_OK);
  EXPECT(gptq_prepare_hinv(H, 300, 0.0, U, nullptr, st, ws, pw, s0), GPTQ_OK);
  EXPECT(gptq_prepare_hinv(H, 65537, 0.01, U, dead, st, ws, 1 << 20, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, -0.01, U, dead, st, ws, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, std::nan(""), U, dead, st, ws, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, INFINITY, U, dead, st, ws, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, 0.01, nullptr, dead, st, ws, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, 0.01, U, dead, nullptr, ws, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, 0.01, U, dead, st, ws, pw - 1, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(H, 300, 0.01, U, dead, st, ws_mis, pw, s0), GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv_perm(H, 300, 0.01, perm, U, dead, st, ws, pw, s0), GPTQ_OK);
  EXPECT(gptq_prepare_hinv_perm(H, 300, 0.01, nullptr, U, dead, st, ws, pw, s0), GPTQ_OK);
  EXPECT(gptq_prepare_hinv_perm(nullptr, 300, 0.01, perm, U, dead, st, ws, pw, s0), GPTQ_EINVAL);

  // ---- quantizer
  const size_t qwb = gptq_quantize_workspace(64, 512, 128);
  EXPECT_TRUE(qwb > 0 && gptq_quantize_workspace(-1, 512, 128) == 0 &&
              gptq_quantize_workspace(4, 0, 128) == 0);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 128, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_OK);
  EXPECT(gptq_quantize_layer(X, GPTQ_F32, 64, 512, U, nullptr, 2, -1, 1, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_OK);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 0, 512, U, dead, 4, 128, 0, 128, nullptr, nullptr,
                             nullptr, nullptr, nullptr, 0, s0), GPTQ_OK);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 8, 128, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EUNSUPPORTED);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 5, 128, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 500, U, dead, 4, 128, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EINVAL);  // 128 does not divide 500
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 256, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EUNSUPPORTED);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 128, 2, 128, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 128, 0, 64, codes, sc, zr,
                             nullptr, ws, qwb, s0), GPTQ_EUNSUPPORTED);
  EXPECT(gptq_quantize_layer(X, 9, 64, 512, U, dead, 4, 128, 0, 128, codes, sc, zr, nullptr, ws,
                             qwb, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 65537, U, dead, 4, -1, 0, 128, codes, sc, zr,
                             nullptr, ws, 1 << 20, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(nullptr, GPTQ_BF16, 64, 512, U, dead, 4, 128, 0, 128, codes, sc,
                             zr, nullptr, ws, qwb, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 128, 0, 128, codes, sc, zr,
                             nullptr, ws, qwb - 1, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(X, GPTQ_BF16, 64, 512, U, dead, 4, 128, 0, 128, codes, sc, zr,
                             nullptr, ws_mis, qwb, s0), GPTQ_EINVAL);

  // ---- with a column order
  const size_t qpw = gptq_quantize_perm_workspace(64, 512, 128);
  EXPECT_TRUE(qpw > 0 && gptq_quantize_perm_workspace(0, 512, 128) == 0);
  EXPECT(gptq_quantize_layer_perm(X, GPTQ_BF16, 64, 512, U, dead, perm, 1, 4, 128, 0, 128, codes,
                                  sc, zr, perm, nullptr, ws, qpw, s0), GPTQ_OK);
  EXPECT(gptq_quantize_layer_perm(X, GPTQ_BF16, 64, 512, U, dead, perm, 2, 4, 128, 0, 128, codes,
                                  sc, zr, perm, nullptr, ws, qpw, s0), GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer_perm(X, GPTQ_BF16, 64, 512, U, dead, perm, 0, 4, 128, 0, 128, codes,
                                  sc, zr, perm, nullptr, ws, qpw - 1, s0), GPTQ_EINVAL);
  const size_t aw = gptq_act_order_workspace(300, 5000);
  EXPECT_TRUE(aw > 0 && gptq_act_order_workspace(0, 5) == 0 &&
              gptq_act_order_workspace(70000, 5) == 0);
  EXPECT(gptq_act_order(X, GPTQ_BF16, 5000, 300, 300, perm, dv, ws, aw, s0), GPTQ_OK);
  EXPECT(gptq_act_order(nullptr, GPTQ_BF16, 0, 300, 300, perm, dv, ws, aw, s0), GPTQ_OK);
  EXPECT(gptq_act_order(nullptr, GPTQ_BF16, 5, 300, 300, perm, dv, ws, aw, s0), GPTQ_EINVAL);
  EXPECT(gptq_act_order(X, GPTQ_BF16, 5000, 300, 300, nullptr, dv, ws, aw, s0), GPTQ_EINVAL);
  EXPECT(gptq_act_order(X, GPTQ_BF16, 5000, 299, 300, perm, dv, ws, aw, s0), GPTQ_EINVAL);
  EXPECT(gptq_act_order(X, GPTQ_BF16, 5000, 300, 300, perm, dv, ws_mis, aw, s0), GPTQ_EINVAL);

  // ---- several matrices sharing one Hessian: the lists are exact-length heap blocks
  {
    const int count = 3;
    const void** wl = (const void**)std::malloc(count * sizeof(void*));
    int64_t* dl = (int64_t*)std::malloc(count * sizeof(int64_t));
    wl[0] = X; wl[1] = X; wl[2] = X;
    dl[0] = 40; dl[1] = 0; dl[2] = 24;
    const size_t lw = gptq_quantize_workspace(64, 512, 128);
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, lw, s0), GPTQ_OK);
    wl[1] = nullptr;  // a zero-row entry may be null
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, lw, s0), GPTQ_OK);
    wl[2] = nullptr;  // a non-empty one may not
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, lw, s0), GPTQ_EINVAL);
    wl[2] = X;
    dl[1] = -1;
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, lw, s0), GPTQ_EINVAL);
    dl[0] = 0; dl[1] = 0; dl[2] = 0;
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, nullptr,
                                nullptr, nullptr, nullptr, nullptr, 0, s0), GPTQ_OK);
    dl[0] = (int64_t)1 << 30; dl[1] = (int64_t)1 << 30; dl[2] = 1;
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, 1 << 20, s0), GPTQ_EINVAL);
    dl[0] = 40; dl[1] = 0; dl[2] = 24;
    EXPECT(gptq_quantize_layers(wl, dl, 0, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc, zr,
                                nullptr, ws, lw, s0), GPTQ_EINVAL);
    EXPECT(gptq_quantize_layers(wl, dl, 65, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc, zr,
                                nullptr, ws, lw, s0), GPTQ_EINVAL);
    EXPECT(gptq_quantize_layers(wl, dl, count, GPTQ_BF16, 512, U, dead, 3, 64, 1, 128, codes, sc,
                                zr, nullptr, ws, lw - 1, s0), GPTQ_EINVAL);
    std::free(wl);
    std::free(dl);
  }

  // ---- packing
  EXPECT(gptq_pack(codes, sc, zr, 64, 512, 4, 128, 0, qw, s16, z16, s0), GPTQ_OK);
  EXPECT(gptq_pack(codes, sc, nullptr, 64, 512, 3, -1, 1, qw, s16, nullptr, s0), GPTQ_OK);
  EXPECT(gptq_pack(codes, sc, nullptr, 64, 512, 4, 128, 0, qw, s16, z16, s0), GPTQ_EINVAL);
  EXPECT(gptq_pack(codes, sc, zr, 64, 512, 5, 128, 0, qw, s16, z16, s0), GPTQ_EINVAL);
  EXPECT(gptq_pack(codes, sc, zr, 64, 500, 4, 128, 0, qw, s16, z16, s0), GPTQ_EINVAL);
  EXPECT(gptq_pack(codes, sc, zr, 0, 512, 4, 128, 0, nullptr, nullptr, nullptr, s0), GPTQ_OK);
  EXPECT(gptq_pack(codes, sc, zr, 64, 512, 4, 128, 0, nullptr, s16, z16, s0), GPTQ_EINVAL);

  // ---- dequantized product
  EXPECT(gptq_w4a16_matmul(X, 16, 512, qw, s16, z16, 64, 512, 128, 0, sc, s0), GPTQ_OK);
  EXPECT(gptq_w4a16_matmul(X, 16, 512, qw, s16, nullptr, 64, 512, 128, 1, sc, s0), GPTQ_OK);
  EXPECT(gptq_w4a16_matmul(X, 0, 512, qw, s16, z16, 64, 512, 128, 0, sc, s0), GPTQ_OK);
  EXPECT(gptq_w4a16_matmul(X, 16, 512, qw, s16, nullptr, 64, 512, 128, 0, sc, s0), GPTQ_EINVAL);
  EXPECT(gptq_w4a16_matmul(X, 16, 192, qw, s16, z16, 64, 192, 32, 0, sc, s0), GPTQ_EUNSUPPORTED);
  EXPECT(gptq_w4a16_matmul(X, 16, 516, qw, s16, z16, 64, 512, 128, 0, sc, s0), GPTQ_EINVAL);
  EXPECT(gptq_w4a16_matmul((char*)X + 2, 16, 512, qw, s16, z16, 64, 512, 128, 0, sc, s0),
         GPTQ_EINVAL);
  EXPECT(gptq_w4a16_matmul(X, -1, 512, qw, s16, z16, 64, 512, 128, 0, sc, s0), GPTQ_EINVAL);

  // ---- two-sided rounding
  const size_t gw = gptq2d_workspace(100);
  EXPECT_TRUE(gw > 0 && gptq2d_workspace(0) == 0 && gptq2d_workspace(GPTQ2D_MAX_N + 1) == 0);
  EXPECT(gptq2d_round(dv, dv, dv, 100, dv, ws, gw, s0), GPTQ_OK);
  EXPECT(gptq2d_round(dv, dv, dv, 0, dv, nullptr, 0, s0), GPTQ_OK);
  EXPECT(gptq2d_round(dv, dv, dv, -1, dv, ws, gw, s0), GPTQ_EINVAL);
  EXPECT(gptq2d_round(dv, dv, dv, GPTQ2D_MAX_N + 1, dv, ws, gw, s0), GPTQ_EUNSUPPORTED);
  EXPECT(gptq2d_round(dv, nullptr, dv, 100, dv, ws, gw, s0), GPTQ_EINVAL);
  EXPECT(gptq2d_round(dv, dv, dv, 100, dv, ws, gw - 1, s0), GPTQ_EINVAL);
  EXPECT(gptq2d_round(dv, dv, dv, 100, dv, ws_mis, gw, s0), GPTQ_EINVAL);

  std::free(ws); std::free(H); std::free(U); std::free(dead); std::free(st); std::free(X);
  std::free(codes); std::free(sc); std::free(zr); std::free(qw); std::free(s16); std::free(z16);
  std::free(perm); std::free(dv);
  std::printf("%d checks, %d failed, %d launches\n", g_checks, g_fails, g_launches);
  return g_fails == 0 ? 0 : 1;
}
