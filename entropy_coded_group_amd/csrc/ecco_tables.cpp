// Host side of the table blob: build, validate, extract.
//
// The blob holds the caller's centroids and code lengths plus what the
// kernels derive from them: canonical codewords in stream order, an 8-bit
// window decode table, midpoints, packed code lengths and the exact value of
// every FP8 E4M3FN code.  Codes are canonical in the DEFLATE sense (RFC 1951
// section 3.2.2); code lengths are limited to 2..8 bits as the pages' parallel
// decoder requires (Ecco review, referee report major comment 1).
#include <cmath>
#include <cstring>
#include <limits>

#include "ecco_internal.h"

namespace ecco {

// Least n in {16, 32, 64} such that every pattern p >= n has the first and
// last centroid of pattern p mod n: patterns past n then never win the
// min/max search (equal fitness, lower index first).
uint32_t search_width(const Tables* t) {
  for (uint32_t n = 16; n < (uint32_t)S; n *= 2) {
    bool rep = true;
    for (uint32_t p = n; p < (uint32_t)S && rep; ++p)
      rep = t->c0c14[p][0] == t->c0c14[p % n][0] && t->c0c14[p][1] == t->c0c14[p % n][1];
    if (rep) return n;
  }
  return S;
}

uint32_t checksum_of(const Tables* t) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(t) + offsetof(Tables, centroids);
  const uint8_t* e = reinterpret_cast<const uint8_t*>(t) + sizeof(Tables);
  uint32_t h = 2166136261u;
  for (; p < e; ++p) {
    h ^= *p;
    h *= 16777619u;
  }
  return h;
}

namespace {

bool fp16_exact(float v) {
  // A float is exactly representable in binary16 iff converting to half and
  // back is the identity; done with integer bit arithmetic to avoid relying on
  // a host half type.
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint32_t mag = u & 0x7fffffffu;
  if (mag == 0) return true;
  int e = int(mag >> 23) - 127;
  uint32_t m = mag & 0x7fffffu;
  if (e > 15) return false;
  if (e >= -14) return (m & 0x1fffu) == 0;                 // normal half: 10 mantissa bits
  if (e < -24) return false;                                // below the smallest subnormal
  // subnormal half: value must be a multiple of 2^-24
  int drop = 13 + (-14 - e);                                // mantissa bits beyond the grid
  uint32_t full = m | 0x800000u;
  return drop <= 24 && (full & ((1u << drop) - 1u)) == 0;
}

float fp8_code_value(int b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return std::numeric_limits<float>::quiet_NaN();
  float mag = e == 0 ? std::ldexp(float(m), -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
  return s ? -mag : mag;
}

int check_inputs(const float* c, const uint8_t* len) {
  for (int p = 0; p < S; ++p) {
    for (int k = 0; k < C; ++k) {
      float v = c[p * C + k];
      if (!std::isfinite(v) || v < -1.0f || v > 1.0f || !fp16_exact(v)) return ECCO_ETABLES;
      if (k > 0 && v < c[p * C + k - 1]) return ECCO_ETABLES;
    }
    for (int h = 0; h < H; ++h) {
      uint32_t kraft = 0;   // in units of 2^-8
      for (int s = 0; s < A; ++s) {
        int l = len[(p * H + h) * A + s];
        if (l < ECCO_LEN_MIN || l > ECCO_LEN_MAX) return ECCO_ETABLES;
        kraft += 1u << (8 - l);
      }
      if (kraft != 256u) return ECCO_ETABLES;   // complete prefix code
    }
  }
  return ECCO_OK;
}

// Canonical codewords of one codebook: symbols taken in (length, symbol)
// order receive consecutive code values, shifted left whenever the length
// grows.  Returned in stream order: the code's most significant bit is the
// first stream bit, so the value is bit-reversed into the low bits.
void canonical_stream_codes(const uint8_t* len, uint32_t* rev) {
  uint32_t code = 0;
  int prev = 0;
  bool first = true;
  for (int l = ECCO_LEN_MIN; l <= ECCO_LEN_MAX; ++l) {
    for (int s = 0; s < A; ++s) {
      if (len[s] != l) continue;
      if (first) {
        code = 0;
        first = false;
      } else {
        code = (code + 1) << (l - prev);
      }
      prev = l;
      uint32_t r = 0;
      for (int i = 0; i < l; ++i) r |= ((code >> (l - 1 - i)) & 1u) << i;
      rev[s] = r;
    }
  }
}

}  // namespace

}  // namespace ecco

using namespace ecco;

extern "C" size_t ecco_tables_size(void) { return sizeof(Tables); }

extern "C" int ecco_tables_build(const float* centroids, const uint8_t* code_len, void* out) {
  if (!centroids || !code_len || !out) return ECCO_EINVAL;
  int rc = check_inputs(centroids, code_len);
  if (rc) return rc;
  Tables* t = static_cast<Tables*>(out);
  std::memset(t, 0, sizeof(Tables));
  t->magic = kMagic;
  t->version = kVersion;
  t->size = sizeof(Tables);
  const float inf = std::numeric_limits<float>::infinity();
  for (int p = 0; p < S; ++p) {
    for (int k = 0; k < C; ++k) t->centroids[p][k] = centroids[p * C + k];
    for (int k = 0; k + 1 < C; ++k) {
      volatile float sum = t->centroids[p][k] + t->centroids[p][k + 1];   // one float add, then one float multiply
      t->midpoints[p][k] = sum * 0.5f;
    }
    t->midpoints[p][14] = inf;
    t->midpoints[p][15] = inf;
    t->c0c14[p][0] = t->centroids[p][0];
    t->c0c14[p][1] = t->centroids[p][C - 1];
    for (int h = 0; h < H; ++h) {
      const uint8_t* L = code_len + (p * H + h) * A;
      uint32_t rev[A];
      canonical_stream_codes(L, rev);
      for (int s = 0; s < A; ++s) {
        t->code_len[p][h][s] = L[s];
        t->enc[p][h][s] = uint16_t(rev[s] | (uint32_t(L[s]) << 8));
        for (int w = int(rev[s]); w < 256; w += 1 << L[s]) t->lut[p][h][w] = lut_entry(s, L[s]);
      }
    }
    for (int s = 0; s < A; ++s) {
      uint32_t v = 0;
      for (int h = 0; h < H; ++h) v |= uint32_t(t->code_len[p][h][s]) << (8 * h);
      t->len4[p][s] = v;
    }
  }
  for (int b = 0; b < 256; ++b) t->fp8_value[b] = fp8_code_value(b);
  t->n_search = search_width(t);
  t->checksum = checksum_of(t);
  return ECCO_OK;
}

extern "C" int ecco_tables_validate(const void* blob) {
  if (!blob) return ECCO_EINVAL;
  const Tables* t = static_cast<const Tables*>(blob);
  if (t->magic != kMagic || t->version != kVersion || t->size != sizeof(Tables)) return ECCO_ETABLES;
  if (t->checksum != checksum_of(t)) return ECCO_ETABLES;
  if (t->n_search != search_width(t)) return ECCO_ETABLES;
  float c[S * C];
  uint8_t l[S * H * A];
  for (int p = 0; p < S; ++p)
    for (int k = 0; k < C; ++k) c[p * C + k] = t->centroids[p][k];
  std::memcpy(l, t->code_len, sizeof(l));
  return check_inputs(c, l);
}

extern "C" int ecco_tables_get(const void* blob, float* centroids, uint8_t* code_len) {
  if (!blob || !centroids || !code_len) return ECCO_EINVAL;
  int rc = ecco_tables_validate(blob);
  if (rc) return rc;
  const Tables* t = static_cast<const Tables*>(blob);
  for (int p = 0; p < S; ++p)
    for (int k = 0; k < C; ++k) centroids[p * C + k] = t->centroids[p][k];
  std::memcpy(code_len, t->code_len, sizeof(t->code_len));
  return ECCO_OK;
}

extern "C" float ecco_tensor_scale_from_amax(float amax) {
  if (!(amax > 0.0f) || !std::isfinite(amax)) return 1.0f;
  volatile float t = amax / 448.0f;
  return t;
}

extern "C" const char* ecco_strerror(int code) {
  switch (code) {
    case ECCO_OK: return "ok";
    case ECCO_EINVAL: return "invalid argument (null pointer or bad option)";
    case ECCO_EALIGN: return "misaligned pointer or stride";
    case ECCO_ESIZE: return "size out of range";
    case ECCO_ETABLES: return "invalid tables";
    case ECCO_EHIP: return "HIP runtime error";
    case ECCO_EDEVICE: return "device is not gfx950";
    default: return "unknown error";
  }
}

extern "C" const char* ecco_version(void) { return "ecco 1.0 (format v1, gfx950)"; }
