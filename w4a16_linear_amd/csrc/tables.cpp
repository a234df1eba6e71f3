// Host-side tables of the OPQ quantizer (model card "OPQ INT4 Z-Image",
// section "OPQ 原理"): the decision points of q = round(15 u^alpha) and the
// reconstruction levels (q/15)^(1/alpha) of section "推理解码".
//
// Decision points are found in 113-bit binary128 arithmetic (libquadmath), so a
// binary32 candidate t is classified exactly unless 15 t^alpha lies within about
// 1e-30 of a half-integer; the only exact half is alpha = 1, t = 1/2, which is
// evaluated exactly below.
//
// Both tables depend on alpha alone and cost tens of microseconds of binary128
// arithmetic, so the last few alphas' tables are memoised (under a mutex; the
// memo is the library's only global state and holds pure function values).
#include <quadmath.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "opq_internal.hpp"

namespace opq {

namespace {

// Does the code of u = t reach k, i.e. 15 t^alpha >= k - 1/2 ?
bool reaches(float t, float alpha, int k) {
  if (!(t > 0.0f)) return false;
  const __float128 fifteen = 15, half_k = (__float128)k - (__float128)0.5;
  if (alpha == 1.0f) return fifteen * (__float128)t >= half_k;  // exact
  return fifteen * powq((__float128)t, (__float128)alpha) >= half_k;
}

bool compute_decision_points(float alpha, float out[kLevels]) {
  for (int k = 1; k <= kLevels; ++k) {
    const __float128 b = powq((__float128)(2 * k - 1) / (__float128)30, 1 / (__float128)alpha);
    float t = (float)b;
    while (!reaches(t, alpha, k)) t = std::nextafter(t, 2.0f);
    while (t > 0.0f && reaches(std::nextafter(t, 0.0f), alpha, k)) t = std::nextafter(t, 0.0f);
    out[k - 1] = t;
  }
  return true;
}

// G_q in binary128, then rounded to double: within half an ulp of the real value.
void compute_levels(float alpha, double out[kLevels + 1]) {
  const __float128 inv = 1 / (__float128)alpha;
  out[0] = 0.0;
  for (int q = 1; q < kLevels; ++q) out[q] = (double)powq((__float128)q / (__float128)kLevels, inv);
  out[kLevels] = 1.0;
}

struct Entry {
  uint32_t alpha_bits = 0;
  bool used = false;
  float t[kLevels];
  double g[kLevels + 1];
};

constexpr int kMemo = 8;
std::mutex g_memo_mutex;
Entry g_memo[kMemo];
int g_memo_next = 0;

// Fills the entry for alpha (finite, > 0), from the memo or computed.
Entry lookup(float alpha) {
  uint32_t bits;
  std::memcpy(&bits, &alpha, sizeof bits);
  {
    std::lock_guard<std::mutex> lock(g_memo_mutex);
    for (const Entry& e : g_memo)
      if (e.used && e.alpha_bits == bits) return e;
  }
  Entry e;
  e.alpha_bits = bits;
  e.used = true;
  compute_decision_points(alpha, e.t);
  compute_levels(alpha, e.g);
  std::lock_guard<std::mutex> lock(g_memo_mutex);
  g_memo[g_memo_next] = e;
  g_memo_next = (g_memo_next + 1) % kMemo;
  return e;
}

}  // namespace

bool decision_points(float alpha, float out[kLevels]) {
  if (!std::isfinite(alpha) || !(alpha > 0.0f)) return false;
  const Entry e = lookup(alpha);
  std::memcpy(out, e.t, sizeof e.t);
  return true;
}

void levels(float alpha, double out[kLevels + 1]) {
  const Entry e = lookup(alpha);
  std::memcpy(out, e.g, sizeof e.g);
}

}  // namespace opq
