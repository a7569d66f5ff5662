// Host side of the table blob: build, validate, extract.
//
// The blob holds the caller's centroids and code lengths plus what the
// kernels derive from them: canonical codewords in stream order, an 8-bit
// window decode table, midpoints, the encoder's quantiser bins and pattern
// candidates, packed code lengths and the exact value of every FP8 E4M3FN
// code.  Codes are canonical in the DEFLATE sense (RFC 1951
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

// Bins B, C of each pattern over [m_0 - 2 margin, m_13 + 2 margin], and per
// bin the midpoints surely below it; checks that at most one midpoint is
// within the margin of any bin (the last bin: none, all 14 below it).  The
// bin edges are taken from the binary32 B and C the kernel uses.
uint32_t build_quantiser_bins(const float (*mid)[16], uint8_t (*qbin)[kQBins], float (*qaxis)[2]) {
  const double d = kQBinMargin, inf = std::numeric_limits<double>::infinity();
  bool ok = true;
  for (int p = 0; p < S; ++p) {
    double m[14];
    for (int k = 0; k < 14; ++k) m[k] = mid[p][k];
    const double lo_all = m[0] - 2.0 * d, hi_all = m[13] + 2.0 * d;
    const float B = (float)((kQBins - 1) / (hi_all - lo_all));
    const float Cq = (float)(-lo_all * (double)B);
    qaxis[p][0] = B;
    qaxis[p][1] = Cq;
    for (int j = 0; j < kQBins; ++j) {
      const double lo = j == 0 ? -inf : (j - (double)Cq) / (double)B;
      const double hi = j == kQBins - 1 ? inf : (j + 1 - (double)Cq) / (double)B;
      int below = 0, unsure = 0;
      for (int k = 0; k < 14; ++k) {
        if (m[k] < lo - d)
          ++below;
        else if (m[k] <= hi + d)
          ++unsure;
      }
      if (j == kQBins - 1 ? below != 14 : unsure > 1) ok = false;
      qbin[p][j] = (uint8_t)below;
    }
  }
  return ok ? 1u : 0u;
}

// Cell by cell: start from the widened cell's rectangle and, for pattern q,
// cut it by every half-plane F_q - F_p <= margin (F_q - F_p is affine in
// (x, y): the squares cancel); q is a candidate if anything is left.  A
// quick test first drops the patterns whose nearest point of the cell is
// farther than the farthest point from the pattern nearest the centre.
void build_pattern_candidates(const float (*c0c14)[2], uint8_t (*pcand)[kPCand], float* pgrid) {
  const double cm = kPCellMargin, fm = kPFitMargin;
  double ax[S], by[S];
  bool dup[S];
  double xlo = 1e9, xhi = -1e9, ylo = 1e9, yhi = -1e9;
  for (int p = 0; p < S; ++p) {
    ax[p] = c0c14[p][0];
    by[p] = c0c14[p][1];
    xlo = std::fmin(xlo, ax[p]);
    xhi = std::fmax(xhi, ax[p]);
    ylo = std::fmin(ylo, by[p]);
    yhi = std::fmax(yhi, by[p]);
    dup[p] = false;
    for (int r = 0; r < p && !dup[p]; ++r) dup[p] = c0c14[r][0] == c0c14[p][0] && c0c14[r][1] == c0c14[p][1];
  }
  // the grid: the centroids' range and an eighth of it on each side (at
  // least 1/16), with binary32 scales; cells are placed as the kernel
  // places them, from the stored floats
  const double ex = std::fmax(0.125 * (xhi - xlo), 0.0625), ey = std::fmax(0.125 * (yhi - ylo), 0.0625);
  const float sx = (float)(kPGrid / (xhi - xlo + 2 * ex)), sy = (float)(kPGrid / (yhi - ylo + 2 * ey));
  const float ox = (float)(-(xlo - ex) * (double)sx), oy = (float)(-(ylo - ey) * (double)sy);
  pgrid[0] = sx;
  pgrid[1] = ox;
  pgrid[2] = sy;
  pgrid[3] = oy;
  struct Pt {
    double x, y;
  };
  for (int cy = 0; cy < kPGrid; ++cy) {
    for (int cx = 0; cx < kPGrid; ++cx) {
      const double x0 = (cx - (double)ox) / sx - cm, x1 = (cx + 1 - (double)ox) / sx + cm;
      const double y0 = (cy - (double)oy) / sy - cm, y1 = (cy + 1 - (double)oy) / sy + cm;
      const double xc = 0.5 * (x0 + x1), yc = 0.5 * (y0 + y1);
      // the farthest-point distance of the pattern nearest the centre
      int pn = 0;
      double dn = 1e300;
      for (int p = 0; p < S; ++p) {
        const double d = (xc - ax[p]) * (xc - ax[p]) + (yc - by[p]) * (yc - by[p]);
        if (d < dn) { dn = d; pn = p; }
      }
      const double fx = std::fmax(std::fabs(x0 - ax[pn]), std::fabs(x1 - ax[pn]));
      const double fy = std::fmax(std::fabs(y0 - by[pn]), std::fabs(y1 - by[pn]));
      const double far = fx * fx + fy * fy;
      uint8_t* out = pcand[cy * kPGrid + cx];
      int n = 0;
      bool many = false;
      for (int q = 0; q < S && !many; ++q) {
        if (dup[q]) continue;
        const double nx = std::fmax(0.0, std::fmax(x0 - ax[q], ax[q] - x1));
        const double ny = std::fmax(0.0, std::fmax(y0 - by[q], by[q] - y1));
        if (nx * nx + ny * ny > far + fm) continue;
        Pt poly[4 + S], next[4 + S];
        int np = 4;
        poly[0] = {x0, y0}; poly[1] = {x1, y0}; poly[2] = {x1, y1}; poly[3] = {x0, y1};
        for (int p = 0; p < S && np > 0; ++p) {
          if (p == q || dup[p]) continue;
          // F_q - F_p = gx * x + gy * y + g0 <= fm
          const double gx = -2.0 * (ax[q] - ax[p]), gy = -2.0 * (by[q] - by[p]);
          const double g0 = ax[q] * ax[q] + by[q] * by[q] - ax[p] * ax[p] - by[p] * by[p] - fm;
          int nn = 0;
          for (int i = 0; i < np; ++i) {
            const Pt a = poly[i], b = poly[(i + 1) % np];
            const double va = gx * a.x + gy * a.y + g0, vb = gx * b.x + gy * b.y + g0;
            if (va <= 0.0) next[nn++] = a;
            if ((va <= 0.0) != (vb <= 0.0)) {
              const double t = va / (va - vb);
              next[nn++] = {a.x + t * (b.x - a.x), a.y + t * (b.y - a.y)};
            }
          }
          np = nn;
          for (int i = 0; i < np; ++i) poly[i] = next[i];
        }
        if (np == 0) continue;
        if (n == kPCand) {
          many = true;
        } else {
          out[n++] = (uint8_t)q;
        }
      }
      for (int i = n; i < kPCand; ++i) out[i] = kPCandNone;
      if (many) out[0] = kPCandMany;
    }
  }
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
      if (kraft > 256u) return ECCO_ETABLES;    // a prefix code exists (complete or not)
    }
  }
  return ECCO_OK;
}

// 1 if every codebook's Kraft sum is 1 (lengths already checked).
uint32_t all_complete(const uint8_t* len) {
  for (int b = 0; b < S * H; ++b) {
    uint32_t kraft = 0;
    for (int s = 0; s < A; ++s) kraft += 1u << (8 - len[b * A + s]);
    if (kraft != 256u) return 0u;
  }
  return 1u;
}

// Canonical codewords of one codebook: symbols taken in (length, symbol)
// order receive consecutive code values, shifted left whenever the length
// grows.  value[s] is the codeword as a number (most significant code bit
// first); rev[s] is it in stream order: the code's most significant bit is
// the first stream bit, so the value is bit-reversed into the low bits.
void canonical_stream_codes(const uint8_t* len, uint32_t* value, uint32_t* rev) {
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
      value[s] = code;
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
      uint32_t code[A], rev[A];
      canonical_stream_codes(L, code, rev);
      std::memset(t->lut[p][h], kLutNoCode, 256);   // windows no codeword prefixes
      for (int s = 0; s < A; ++s) {
        t->code_len[p][h][s] = L[s];
        t->enc[p][h][s] = (code[s] << (32 - L[s])) | uint32_t(32 - L[s]);
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
  t->qbins_ok = build_quantiser_bins(t->midpoints, t->qbin, t->qaxis);
  build_pattern_candidates(t->c0c14, t->pcand, t->pgrid);
  t->n_search = search_width(t);
  t->complete = all_complete(code_len);
  t->checksum = checksum_of(t);
  return ECCO_OK;
}

extern "C" int ecco_tables_validate(const void* blob) {
  if (!blob) return ECCO_EINVAL;
  const Tables* t = static_cast<const Tables*>(blob);
  if (t->magic != kMagic || t->version != kVersion || t->size != sizeof(Tables)) return ECCO_ETABLES;
  if (t->checksum != checksum_of(t)) return ECCO_ETABLES;
  if (t->n_search != search_width(t)) return ECCO_ETABLES;
  {
    // the quantiser bins are derived from the midpoints: rebuild and compare
    uint8_t qbin[S][kQBins];
    float qaxis[S][2];
    const uint32_t ok = build_quantiser_bins(t->midpoints, qbin, qaxis);
    if (ok != t->qbins_ok || std::memcmp(qbin, t->qbin, sizeof(qbin)) || std::memcmp(qaxis, t->qaxis, sizeof(qaxis)))
      return ECCO_ETABLES;
    uint8_t pcand[kPGrid * kPGrid][kPCand];
    float pgrid[4];
    build_pattern_candidates(t->c0c14, pcand, pgrid);
    if (std::memcmp(pcand, t->pcand, sizeof(pcand)) || std::memcmp(pgrid, t->pgrid, sizeof(pgrid))) return ECCO_ETABLES;
  }
  float c[S * C];
  uint8_t l[S * H * A];
  for (int p = 0; p < S; ++p)
    for (int k = 0; k < C; ++k) c[p * C + k] = t->centroids[p][k];
  std::memcpy(l, t->code_len, sizeof(l));
  const int rc = check_inputs(c, l);
  if (rc) return rc;
  return t->complete == all_complete(l) ? ECCO_OK : ECCO_ETABLES;
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
