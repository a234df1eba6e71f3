// Host-only driver for the sanitizer test: the decision points and levels of
// every code width over a spread of alphas, from four threads at once (the
// per-alpha memo is shared), with monotonicity and end-point checks.
#include <cstdio>
#include <thread>
#include <vector>

#include "opq_internal.hpp"

int main() {
  int bad = 0;
  auto work = [&bad](int seed) {
    int local = 0;
    for (int i = 0; i < 400; ++i) {
      const float alpha = 0.02f + 0.15f * (float)((i * 7 + seed) % 400);
      float t[opq::kMaxLevels];
      double g[opq::kMaxLevels + 1];
      for (int L : {7, 15, 31, 63}) {
        if (opq::decision_points_n(alpha, L, t))
          for (int k = 1; k < L; ++k) local += !(t[k] >= t[k - 1]);
        opq::levels_n(alpha, L, g);
        local += g[0] != 0.0 || g[L] != 1.0;
      }
      float t15[opq::kLevels];
      double g16[opq::kLevels + 1];
      if (opq::decision_points(alpha, t15))
        for (int k = 1; k < opq::kLevels; ++k) local += !(t15[k] >= t15[k - 1]);
      opq::levels(alpha, g16);
      local += g16[0] != 0.0 || g16[opq::kLevels] != 1.0;
    }
    __atomic_add_fetch(&bad, local, __ATOMIC_RELAXED);
  };
  std::vector<std::thread> th;
  for (int s = 0; s < 4; ++s) th.emplace_back(work, s);
  for (auto& x : th) x.join();
  std::printf("bad=%d\n", bad);
  return bad != 0;
}
