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

// Does the code of u = t reach k, i.e. L t^alpha >= k - 1/2 (L = 15 for 4 bits)?
bool reaches(float t, float alpha, int k, int L) {
  if (!(t > 0.0f)) return false;
  const __float128 lv = L, half_k = (__float128)k - (__float128)0.5;
  if (alpha == 1.0f) return lv * (__float128)t >= half_k;  // exact
  return lv * powq((__float128)t, (__float128)alpha) >= half_k;
}

bool compute_decision_points(float alpha, int L, float* out) {
  for (int k = 1; k <= L; ++k) {
    const __float128 b = powq((__float128)(2 * k - 1) / (__float128)(2 * L), 1 / (__float128)alpha);
    float t = (float)b;
    while (!reaches(t, alpha, k, L)) t = std::nextafter(t, 2.0f);
    while (t > 0.0f && reaches(std::nextafter(t, 0.0f), alpha, k, L)) t = std::nextafter(t, 0.0f);
    out[k - 1] = t;
  }
  return true;
}

// G_q in binary128, then rounded to double: within half an ulp of the real value.
void compute_levels(float alpha, int L, double* out) {
  const __float128 inv = 1 / (__float128)alpha;
  out[0] = 0.0;
  for (int q = 1; q < L; ++q) out[q] = (double)powq((__float128)q / (__float128)L, inv);
  out[L] = 1.0;
}

struct Entry {
  uint32_t alpha_bits = 0;
  int L = 0;
  bool used = false;
  float t[kMaxLevels];
  double g[kMaxLevels + 1];
};

constexpr int kMemo = 12;
std::mutex g_memo_mutex;
Entry g_memo[kMemo];
int g_memo_next = 0;

// Fills the entry for (alpha, L), alpha finite and > 0, from the memo or computed.
Entry lookup(float alpha, int L) {
  uint32_t bits;
  std::memcpy(&bits, &alpha, sizeof bits);
  {
    std::lock_guard<std::mutex> lock(g_memo_mutex);
    for (const Entry& e : g_memo)
      if (e.used && e.alpha_bits == bits && e.L == L) return e;
  }
  Entry e;
  e.alpha_bits = bits;
  e.L = L;
  e.used = true;
  compute_decision_points(alpha, L, e.t);
  compute_levels(alpha, L, e.g);
  std::lock_guard<std::mutex> lock(g_memo_mutex);
  g_memo[g_memo_next] = e;
  g_memo_next = (g_memo_next + 1) % kMemo;
  return e;
}

}  // namespace

bool decision_points(float alpha, float out[kLevels]) {
  if (!std::isfinite(alpha) || !(alpha > 0.0f)) return false;
  const Entry e = lookup(alpha, kLevels);
  std::memcpy(out, e.t, kLevels * sizeof(float));
  return true;
}

void levels(float alpha, double out[kLevels + 1]) {
  const Entry e = lookup(alpha, kLevels);
  std::memcpy(out, e.g, (kLevels + 1) * sizeof(double));
}

bool decision_points_n(float alpha, int L, float* out) {
  if (!std::isfinite(alpha) || !(alpha > 0.0f) || L < 1 || L > kMaxLevels) return false;
  const Entry e = lookup(alpha, L);
  std::memcpy(out, e.t, L * sizeof(float));
  return true;
}

void levels_n(float alpha, int L, double* out) {
  const Entry e = lookup(alpha, L);
  std::memcpy(out, e.g, (L + 1) * sizeof(double));
}

}  // namespace opq
