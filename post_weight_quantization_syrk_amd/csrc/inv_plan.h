// Host plan of the triangular inverse's tiles (L^{-1} by recursive doubling,
// the last part of the prepare step: dead channels and damping, Cholesky, the
// inverse, then U; "GPTQ：基于近似二阶信息的大模型权重量化", 阶段一).
//
// Level s (a power of two times 64) pairs the blocks [a, b) and [b, e), a =
// 0, 2s, 4s, ..., b = a + s < d, e = min(b + s, d), and forms the lower-left
// block of the pair's inverse in two steps over 64 x 64 tiles:
//   T step: T[b:e, a:b] = L[b:e, a:b] M[a:b, a:b]
//   X step: M[b:e, a:b] = -M[b:e, b:e] T[b:e, a:b]
// (M = L^{-1}; the diagonal 64 x 64 blocks of M come with the factorization).
// A step's tiles are numbered g = pair * sb^2 + local (sb = s / 64), the local
// order longest tile first (ct ascending for T, rt descending for X).
//
// The plan hands each launch the tiles whose operands are complete when it
// starts: a T tile needs L's columns before b final and every lower level
// done inside [0, b); an X tile needs its pair's T tiles, L's columns before e
// final and every lower level done inside [0, e).  The factorization's panel
// and band launches carry the tiles that are ready before the chain ends,
// within a flop budget; the rest runs in rounds afterwards.  Host code only:
// the device side (InvItems read by inv_tile) shares just the struct.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <climits>
#include <vector>

namespace gptq {

constexpr int INV_NB = 64;      // tile width
constexpr int INV_PW = 256;     // factorization panel width
constexpr int INV_ITEMS = 16;   // steps one launch can carry

// Tiles g0[i] .. g0[i] + cnt[i] - 1 of step (s[i], x[i]) (x = 1: the X step),
// in order; a launch's extra workgroup k takes the k-th of them.
struct InvItems {
  int n;
  int s[INV_ITEMS], x[INV_ITEMS], g0[INV_ITEMS], cnt[INV_ITEMS];
};

// Flops of inverse tiles a panel launch takes on beyond its own
// trailing-update passengers: about what the CUs its latency-bound chain
// leaves idle do in one panel's time.  Band launches (about 11 us at d =
// 4096) take a small budget of short tiles only: one tile runs on one CU,
// and a long one would hold up a short launch.
constexpr double INV_PANEL_FLOPS = 4.0e9;
constexpr double INV_BAND_FLOPS = 0.5e9;
constexpr int64_t INV_BAND_KMAX = 256;

class InvPlan {
 public:
  explicit InvPlan(int d) : d_(d) {
    for (int64_t s = INV_NB; s < d; s *= 2) {
      const int64_t pairs = cdiv(d - s, 2 * s), sb = s / INV_NB;
      S_.push_back((int)s);
      P_.push_back(pairs);
      G_.push_back(pairs * sb * sb);
    }
    done_[0].assign(S_.size(), 0);
    done_[1].assign(S_.size(), 0);
  }
  bool finished() const {
    for (size_t li = 0; li < S_.size(); ++li)
      if (done_[1][li] < G_[li]) return false;
    return true;
  }
  // The tiles whose operands are complete when a launch starts with L's
  // columns before cfin final, steps in level order (T before X), up to
  // `budget` flops (all of them for a negative budget), tiles with K above
  // kmax left out, and INV_ITEMS steps.  Tiles taken now count as done for
  // later launches only.
  InvItems take(int cfin, double budget, int64_t kmax = INT32_MAX) {
    InvItems it{};
    double used = 0.0;
    std::vector<int64_t> add[2] = {std::vector<int64_t>(S_.size(), 0),
                                   std::vector<int64_t>(S_.size(), 0)};
    for (size_t li = 0; li < S_.size() && it.n < INV_ITEMS; ++li) {
      for (int x = 0; x < 2 && it.n < INV_ITEMS; ++x) {
        const int64_t g0 = done_[x][li];
        int64_t c = 0;
        while (g0 + c < G_[li] && ready((int)li, x, g0 + c, cfin)) {
          const double f = tile_flops((int)li, x, g0 + c);
          if (budget >= 0.0 &&
              (used + f > budget || f > 2.0 * INV_NB * INV_NB * (double)kmax))
            break;
          used += f;
          ++c;
        }
        if (c > 0) {
          it.s[it.n] = S_[li];
          it.x[it.n] = x;
          it.g0[it.n] = (int)g0;
          it.cnt[it.n] = (int)c;
          ++it.n;
          add[x][li] = c;
        }
      }
    }
    for (int x = 0; x < 2; ++x)
      for (size_t li = 0; li < S_.size(); ++li) done_[x][li] += add[x][li];
    return it;
  }
  static int count(const InvItems& it) {
    int n = 0;
    for (int i = 0; i < it.n; ++i) n += it.cnt[i];
    return n;
  }

 private:
  static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
  bool ready(int li, int x, int64_t g, int cfin) const {
    const int64_t s = S_[li], sb = s / INV_NB;
    const int64_t p = g / (sb * sb);
    const int64_t a = 2 * s * p, b = a + s, e = std::min<int64_t>(b + s, d_);
    const int64_t need = x ? e : b;
    if (need > cfin) return false;
    if (x && done_[0][li] < (p + 1) * sb * sb) return false;
    for (int lj = 0; lj < li; ++lj) {
      const int64_t sj = S_[lj], sbj = sj / INV_NB;
      const int64_t pairs = std::min<int64_t>(P_[lj], cdiv(need, 2 * sj));
      if (done_[1][lj] < pairs * sbj * sbj) return false;
    }
    return true;
  }
  double tile_flops(int li, int x, int64_t g) const {
    const int64_t s = S_[li], sb = s / INV_NB;
    const int64_t p = g / (sb * sb), lt = g % (sb * sb), major = lt / sb;
    const int64_t b = 2 * s * p + s, e = std::min<int64_t>(b + s, d_);
    const int64_t k =
        x ? std::min<int64_t>(INV_NB * (sb - 1 - major) + INV_NB, e - b) : s - INV_NB * major;
    return 2.0 * INV_NB * INV_NB * (double)std::max<int64_t>(k, 0);
  }
  int d_;
  std::vector<int> S_;
  std::vector<int64_t> P_, G_;
  std::vector<int64_t> done_[2];
};

// The items of the panel launch at column c0 (rest = its trailing-update
// passenger tiles, 128 x 128 with K = INV_PW) and of the band launch after
// the panel (c1 = its first column after the panel).
inline InvItems inv_panel_items(InvPlan& plan, int c0, int rest) {
  const double trail = 2.0 * 128 * 128 * INV_PW * (double)rest;
  return plan.take(c0, std::max(0.0, INV_PANEL_FLOPS - trail));
}
inline InvItems inv_band_items(InvPlan& plan, int c1) {
  return plan.take(c1, INV_BAND_FLOPS, INV_BAND_KMAX);
}

}  // namespace gptq
