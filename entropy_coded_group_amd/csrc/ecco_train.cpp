// Offline learning of the shared patterns and codebooks (host only).
//
// The pages: patterns and codebooks are learned once, offline, on a
// calibration set (Ecco review, "Load-bearing premise"; "Assumptions & free
// parameters": 64 patterns of 15 centroids, 4 codebooks per pattern).  The
// paper's "activation-aware" weighting is undefined (referee report, minor 4),
// so plain k-means is used.  Steps:
//   1. normalise each group as the encoder does (scale element, FP8 group
//      scale, a = |S|) and keep its other 127 values divided by a;
//   2. exact 1-D k-means of each group into 15 clusters (dynamic programme
//      over the sorted values);
//   3. Lloyd k-means of the sorted 15-vectors into 64 patterns (k-means++
//      start; an empty cluster takes the farthest point); round to FP16,
//      sort, clamp to [-1, 1];
//   4. assign every group with the encoder's min/max rule and quantiser and
//      count its symbols;
//   5. per pattern, 4 codebooks by Lloyd iterations on code length: start
//      from entropy quartiles, give each codebook the optimal 2..8-bit
//      lengths for its counts plus one (knapsack over Kraft capacity), move
//      each group to its shortest codebook, repeat until stable.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <thread>
#include <vector>

#include "ecco_internal.h"

namespace ecco {
namespace {

float half_to_float(uint16_t h) {
  uint32_t s = uint32_t(h & 0x8000u) << 16, e = (h >> 10) & 31u, m = h & 1023u, u;
  if (e == 0) {
    if (m == 0) {
      u = s;
    } else {  // subnormal: normalise
      int sh = 0;
      while (!(m & 1024u)) { m <<= 1; ++sh; }
      m &= 1023u;
      u = s | (uint32_t(127 - 15 - sh + 1) << 23) | (m << 13);
    }
  } else if (e == 31) {
    u = s | 0x7f800000u | (m << 13);
  } else {
    u = s | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t float_to_half_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t s = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return uint16_t(s | (a > 0x7f800000u ? 0x7e00u : 0x7c00u));
  if (a >= 0x477ff000u) return uint16_t(s | 0x7c00u);          // rounds to >= 65536: inf
  if (a < 0x38800000u) {                                         // below 2^-14: subnormal half
    if (a < 0x33000000u) return uint16_t(s);                    // below 2^-25: rounds to 0
    uint32_t e = a >> 23, m = (a & 0x7fffffu) | 0x800000u;
    uint32_t sh = 126 - e;                                       // 14..24 +
    uint32_t q = m >> sh, rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return uint16_t(s | q);
  }
  uint32_t r = a - (112u << 23);
  r += 0xfffu + ((r >> 13) & 1u);
  return uint16_t(s | (r >> 13));
}

uint32_t fp8_encode(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;                     // >= 448: saturate
  if (a < 0x3c800000u) {                                         // < 2^-6: subnormal grid 2^-9
    float m;
    std::memcpy(&m, &a, 4);
    return sign | uint32_t(std::nearbyint(m * 512.0f));
  }
  uint32_t r = a - (120u << 23);
  r += 0x7ffffu + ((r >> 20) & 1u);
  return sign | (r >> 20);
}

float fp8_value(uint32_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  float mag = e == 0 ? std::ldexp(float(m), -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
  return s ? -mag : mag;
}

struct Rng {  // splitmix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  double uniform() { return (next() >> 11) * (1.0 / 9007199254740992.0); }
};

template <class F>
void parallel_for(size_t n, unsigned threads, F f) {
  if (threads <= 1 || n < 64) {
    for (size_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<size_t> next(0);
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (size_t i; (i = next.fetch_add(16)) < n;)
        for (size_t j = i; j < std::min(n, i + 16); ++j) f(j);
    });
  for (auto& th : pool) th.join();
}

// Exact 1-D k-means of sorted v[0..n) into k runs; writes the k run means.
void kmeans_1d(const double* v, int n, int k, double* means, std::vector<double>& work) {
  work.resize(size_t(2 * (n + 1) + 2 * (k + 1) * (n + 1)));
  double* ps = work.data();
  double* ps2 = ps + (n + 1);
  double* dp = ps2 + (n + 1);
  int32_t* arg = reinterpret_cast<int32_t*>(dp + (k + 1) * (n + 1));
  ps[0] = ps2[0] = 0;
  for (int i = 0; i < n; ++i) {
    ps[i + 1] = ps[i] + v[i];
    ps2[i + 1] = ps2[i] + v[i] * v[i];
  }
  const double inf = std::numeric_limits<double>::infinity();
  for (int i = 0; i <= n; ++i) dp[i] = inf;
  dp[0] = 0;
  for (int c = 1; c <= k; ++c) {
    double* cur = dp + c * (n + 1);
    const double* prev = dp + (c - 1) * (n + 1);
    int32_t* a = arg + c * (n + 1);
    for (int i = 0; i <= n; ++i) cur[i] = inf;
    for (int i = c; i <= n - (k - c); ++i) {
      double best = inf;
      int bj = c - 1;
      for (int j = c - 1; j < i; ++j) {
        double cnt = i - j, s = ps[i] - ps[j], s2 = ps2[i] - ps2[j];
        double cost = std::max(s2 - s * s / cnt, 0.0) + prev[j];
        if (cost < best) { best = cost; bj = j; }
      }
      cur[i] = best;
      a[i] = bj;
    }
  }
  int i = n;
  for (int c = k; c >= 1; --c) {
    int j = arg[c * (n + 1) + i];
    means[c - 1] = (ps[i] - ps[j]) / (i - j);
    i = j;
  }
}

// Optimal code lengths in [2, 8] for the given counts under Kraft <= 1:
// knapsack over capacity units of 2^-8 (exact minimum of sum count * length).
void limited_lengths(const uint64_t* cnt, uint8_t* out) {
  constexpr int CAP = 256;
  const uint64_t INF = std::numeric_limits<uint64_t>::max() / 4;
  static thread_local uint64_t dp[A + 1][CAP + 1];
  static thread_local uint8_t ch[A + 1][CAP + 1];
  for (int u = 0; u <= CAP; ++u) dp[0][u] = INF;
  dp[0][0] = 0;
  for (int i = 0; i < A; ++i) {
    for (int u = 0; u <= CAP; ++u) dp[i + 1][u] = INF;
    for (int u = 0; u <= CAP; ++u) {
      if (dp[i][u] == INF) continue;
      for (int l = ECCO_LEN_MIN; l <= ECCO_LEN_MAX; ++l) {
        int nu = u + (1 << (8 - l));
        if (nu > CAP) continue;
        uint64_t c = dp[i][u] + cnt[i] * uint64_t(l);
        if (c < dp[i + 1][nu]) { dp[i + 1][nu] = c; ch[i + 1][nu] = uint8_t(l); }
      }
    }
  }
  // counts are all >= 1, so the optimum uses the full capacity (complete code)
  int u = CAP;
  for (int i = A; i >= 1; --i) {
    out[i - 1] = ch[i][u];
    u -= 1 << (8 - ch[i][u]);
  }
}

}  // namespace
}  // namespace ecco

using namespace ecco;

extern "C" int ecco_train_patterns(const uint16_t* sample, uint64_t n_values, const ecco_train_opts_t* opts,
                                   void* tables_host) {
  if (!sample || !tables_host) return ECCO_EINVAL;
  ecco_train_opts_t o = {25, 10, 0, 0, 0, 0, 0};
  if (opts) o = *opts;
  if (o.group == 0) o.group = G;
  if (o.group != 64 && o.group != (uint32_t)G) return ECCO_EINVAL;
  const int gs = int(o.group);                 // values per group: 128, or 64 for the activation format
  if (n_values == 0 || n_values % gs != 0) return ECCO_ESIZE;
  if (o.n_patterns == 0) o.n_patterns = S;
  if (o.n_patterns != 16 && o.n_patterns != 32 && o.n_patterns != (uint32_t)S) return ECCO_EINVAL;
  const int D = int(o.n_patterns);
  if (o.kmeans_iters == 0) o.kmeans_iters = 25;
  if (o.huff_iters == 0) o.huff_iters = 10;
  unsigned threads = o.threads ? o.threads : std::max(1u, std::thread::hardware_concurrency());
  size_t ng = n_values / gs;
  if (o.max_groups && ng > o.max_groups) ng = o.max_groups;

  // 1. per-tensor scale and group normalisation
  float amax = 0;
  for (size_t i = 0; i < ng * gs; ++i) {
    float v = std::fabs(half_to_float(sample[i]));
    if (v > amax) amax = v;
  }
  float t = ecco_tensor_scale_from_amax(amax);
  volatile float inv_t_v = 1.0f / t;
  float inv_t = inv_t_v;
  std::vector<float> xs(ng * gs), a(ng);
  std::vector<int> istar(ng);
  for (size_t g = 0; g < ng; ++g) {
    float* x = &xs[g * gs];
    int is = 0;
    for (int j = 0; j < gs; ++j) {
      x[j] = half_to_float(sample[g * gs + j]);
      if (std::fabs(x[j]) > std::fabs(x[is])) is = j;
    }
    istar[g] = is;
    volatile float prod = x[is] * inv_t;
    volatile float S = fp8_value(fp8_encode(prod)) * t;
    a[g] = std::fabs(S);
  }
  std::vector<size_t> used;
  for (size_t g = 0; g < ng; ++g)
    if (a[g] > 0 && std::isfinite(a[g])) used.push_back(g);

  // 2. exact 1-D k-means per group
  std::vector<double> vec(used.size() * C);
  parallel_for(used.size(), threads, [&](size_t u) {
    thread_local std::vector<double> work;
    size_t g = used[u];
    double v[G];
    int n = 0;
    for (int j = 0; j < gs; ++j)
      if (j != istar[g]) v[n++] = double(xs[g * gs + j]) / double(a[g]);
    std::sort(v, v + n);
    kmeans_1d(v, n, C, &vec[u * C], work);
  });

  // 3. Lloyd k-means of the 15-vectors into S patterns
  std::vector<double> cent(S * C, 0.0);
  size_t N = used.size();
  if (N == 0) {
    for (int p = 0; p < S; ++p)
      for (int k = 0; k < C; ++k) cent[p * C + k] = -1.0 + 2.0 * k / (C - 1);
  } else {
    Rng rng{o.seed * 0x2545F4914F6CDD1Dull + 1};
    std::vector<double> d2(N, std::numeric_limits<double>::infinity());
    auto dist = [&](size_t i, const double* c) {
      double s = 0;
      for (int k = 0; k < C; ++k) { double d = vec[i * C + k] - c[k]; s += d * d; }
      return s;
    };
    int K = int(std::min<size_t>(D, N));
    size_t first = rng.next() % N;
    std::copy(&vec[first * C], &vec[first * C] + C, &cent[0]);
    for (int c = 1; c < K; ++c) {
      double tot = 0;
      for (size_t i = 0; i < N; ++i) { d2[i] = std::min(d2[i], dist(i, &cent[(c - 1) * C])); tot += d2[i]; }
      size_t pick = rng.next() % N;
      if (tot > 0) {
        double r = rng.uniform() * tot, acc = 0;
        for (size_t i = 0; i < N; ++i) { acc += d2[i]; if (acc >= r) { pick = i; break; } }
      }
      std::copy(&vec[pick * C], &vec[pick * C] + C, &cent[c * C]);
    }
    for (int c = K; c < D; ++c) std::copy(&cent[(K - 1) * C], &cent[(K - 1) * C] + C, &cent[c * C]);
    std::vector<int> asg(N, -1);
    for (uint32_t it = 0; it < o.kmeans_iters; ++it) {
      std::atomic<size_t> moved(0);
      parallel_for(N, threads, [&](size_t i) {
        int best = 0;
        double bd = dist(i, &cent[0]);
        for (int c = 1; c < K; ++c) { double d = dist(i, &cent[c * C]); if (d < bd) { bd = d; best = c; } }
        if (asg[i] != best) { asg[i] = best; moved.fetch_add(1); }
      });
      if (it > 0 && moved.load() == 0) break;
      std::vector<double> sum(K * C, 0.0);
      std::vector<size_t> cnt(K, 0);
      for (size_t i = 0; i < N; ++i) {
        cnt[asg[i]]++;
        for (int k = 0; k < C; ++k) sum[asg[i] * C + k] += vec[i * C + k];
      }
      for (int c = 0; c < K; ++c)
        if (cnt[c])
          for (int k = 0; k < C; ++k) cent[c * C + k] = sum[c * C + k] / cnt[c];
      for (int c = 0; c < K; ++c) {
        if (cnt[c]) continue;
        size_t far = 0;
        double fd = -1;
        for (size_t i = 0; i < N; ++i) { double d = dist(i, &cent[asg[i] * C]); if (d > fd) { fd = d; far = i; } }
        std::copy(&vec[far * C], &vec[far * C] + C, &cent[c * C]);
        asg[far] = c;
      }
    }
  }
  // slots D..63 repeat the D learned patterns
  for (int p = D; p < S; ++p) std::copy(&cent[(p % D) * C], &cent[(p % D) * C] + C, &cent[p * C]);
  std::vector<float> c32(S * C);
  for (int p = 0; p < S; ++p) {
    float row[C];
    for (int k = 0; k < C; ++k) {
      double v = std::min(1.0, std::max(-1.0, cent[p * C + k]));
      row[k] = half_to_float(float_to_half_rne(float(v)));
    }
    std::sort(row, row + C);
    for (int k = 0; k < C; ++k) c32[p * C + k] = row[k];
  }

  // 4. assign groups with the encoder's rules and count symbols
  std::vector<int> pat(ng, 0);
  std::vector<uint64_t> counts(ng * A, 0);
  std::vector<float> mid(S * 14);
  for (int p = 0; p < S; ++p)
    for (int k = 0; k < 14; ++k) {
      volatile float s = c32[p * C + k] + c32[p * C + k + 1];
      mid[p * 14 + k] = s * 0.5f;
    }
  parallel_for(ng, threads, [&](size_t g) {
    const float* x = &xs[g * gs];
    float aa = a[g];
    float gmin = std::numeric_limits<float>::infinity(), gmax = -gmin;
    for (int j = 0; j < gs; ++j)
      if (j != istar[g]) { gmin = std::min(gmin, x[j]); gmax = std::max(gmax, x[j]); }
    int bp = 0;
    float bf = std::numeric_limits<float>::infinity();
    for (int p = 0; p < S; ++p) {
      volatile float c0a = c32[p * C] * aa, c14a = c32[p * C + C - 1] * aa;
      volatile float d1 = gmin - c0a, d2 = gmax - c14a;
      volatile float q1 = d1 * d1, q2 = d2 * d2;
      float f = q1 + q2;
      if (f < bf || p == 0) { bf = f; bp = p; }
    }
    pat[g] = bp;
    for (int j = 0; j < gs; ++j) {
      int s = 15;
      if (j != istar[g]) {
        s = 0;
        for (int k = 0; k < 14; ++k) {
          volatile float th = mid[bp * 14 + k] * aa;
          if (x[j] > th) ++s;
        }
      }
      counts[g * A + s]++;
    }
  });

  // 5. codebooks per pattern
  std::vector<uint8_t> lens(S * H * A, 4);
  std::vector<std::vector<size_t>> members(S);
  for (size_t g = 0; g < ng; ++g) members[pat[g]].push_back(g);
  parallel_for(S, threads, [&](size_t p) {
    const auto& mem = members[p];
    uint8_t* L = &lens[p * H * A];
    if (mem.empty()) return;
    size_t M = mem.size();
    std::vector<double> ent(M);
    for (size_t i = 0; i < M; ++i) {
      const uint64_t* c = &counts[mem[i] * A];
      double e = 0;
      for (int s = 0; s < A; ++s)
        if (c[s]) { double q = c[s] / double(gs); e -= q * std::log2(q); }
      ent[i] = e;
    }
    std::vector<size_t> order(M);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return ent[x] < ent[y]; });
    std::vector<int> asg(M);
    for (size_t r = 0; r < M; ++r) asg[order[r]] = int(r * H / M);
    for (uint32_t it = 0; it < o.huff_iters; ++it) {
      for (int h = 0; h < H; ++h) {
        uint64_t tot[A];
        for (int s = 0; s < A; ++s) tot[s] = 1;
        for (size_t i = 0; i < M; ++i)
          if (asg[i] == h)
            for (int s = 0; s < A; ++s) tot[s] += counts[mem[i] * A + s];
        limited_lengths(tot, L + h * A);
      }
      bool moved = false;
      for (size_t i = 0; i < M; ++i) {
        int bh = 0;
        uint64_t bl = ~0ull;
        for (int h = 0; h < H; ++h) {
          uint64_t l = 0;
          for (int s = 0; s < A; ++s) l += counts[mem[i] * A + s] * L[h * A + s];
          if (l < bl) { bl = l; bh = h; }
        }
        if (bh != asg[i]) { asg[i] = bh; moved = true; }
      }
      if (!moved) break;
    }
  });
  return ecco_tables_build(c32.data(), lens.data(), tables_host);
}
