// The library's host C++ (table builder and trainer) driven under
// AddressSanitizer and UndefinedBehaviorSanitizer: training on 128- and
// 64-value samples with 64 and 16 patterns, the trained blob read back and
// rebuilt byte for byte, and degenerate samples (all zero, constant, a size
// that is not a whole number of groups).  Exits non-zero on any failure; the
// sanitizers abort on the first report.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "ecco.h"

namespace {

// Float to FP16 bits by truncation, tiny values to zero: test data only.
uint16_t to_half(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const int e = (int)((x >> 23) & 0xffu) - 127 + 15;
  if (e <= 0) return (uint16_t)sign;
  if (e >= 31) return (uint16_t)(sign | 0x7bffu);
  return (uint16_t)(sign | ((uint32_t)e << 10) | ((x & 0x7fffffu) >> 13));
}

}  // namespace

int main() {
  std::mt19937 rng(5);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (uint32_t group : {128u, 64u}) {
    for (uint32_t np : {64u, 16u}) {
      std::vector<uint16_t> s(1 << 17);
      for (auto& v : s) {
        float x = nd(rng) * std::exp(0.5f * nd(rng));
        if (rng() % 2000 == 0) x *= 20.f;
        v = to_half(x * 0.02f);
      }
      ecco_train_opts_t o;
      std::memset(&o, 0, sizeof(o));
      o.kmeans_iters = 8;
      o.huff_iters = 4;
      o.threads = 4;
      o.n_patterns = np;
      o.group = group;
      std::vector<uint8_t> blob(ecco_tables_size());
      if (ecco_train_patterns(s.data(), s.size(), &o, blob.data()) != ECCO_OK) return 1;
      if (ecco_tables_validate(blob.data()) != ECCO_OK) return 2;
      std::vector<float> c(ECCO_N_PATTERNS * ECCO_N_CENTROIDS);
      std::vector<uint8_t> l(ECCO_N_PATTERNS * ECCO_N_CODEBOOKS * ECCO_N_SYMBOLS);
      if (ecco_tables_get(blob.data(), c.data(), l.data()) != ECCO_OK) return 3;
      std::vector<uint8_t> again(ecco_tables_size());
      if (ecco_tables_build(c.data(), l.data(), again.data()) != ECCO_OK) return 4;
      if (std::memcmp(blob.data(), again.data(), blob.size()) != 0) return 5;
    }
  }
  std::vector<uint16_t> z(128 * 64, 0);
  std::vector<uint8_t> blob(ecco_tables_size());
  if (ecco_train_patterns(z.data(), z.size(), nullptr, blob.data()) != ECCO_OK) return 6;
  for (auto& v : z) v = to_half(0.5f);
  if (ecco_train_patterns(z.data(), z.size(), nullptr, blob.data()) != ECCO_OK) return 7;
  if (ecco_train_patterns(z.data(), 100, nullptr, blob.data()) != ECCO_ESIZE) return 8;
  std::printf("ok\n");
  return 0;
}
