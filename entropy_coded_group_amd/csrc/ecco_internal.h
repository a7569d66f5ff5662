// Internal layout of the table blob and shared constants of libecco.
//
// The blob carries the caller's inputs (centroids, code lengths) and the
// tables the kernels derive from them.  It is plain data with no pointers, so
// the caller can copy it byte for byte to device memory.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ecco.h"

namespace ecco {

constexpr uint32_t kMagic = 0x31434345u;   // "ECC1"
constexpr uint32_t kVersion = 4;
constexpr int G = ECCO_GROUP;
constexpr int S = ECCO_N_PATTERNS;
constexpr int C = ECCO_N_CENTROIDS;
constexpr int H = ECCO_N_CODEBOOKS;
constexpr int A = ECCO_N_SYMBOLS;

// Quantiser bins of a pattern (see Tables::qbin): kQBins - 1 equal bins over
// the normalised range of its midpoints, then one bin for everything above it.
constexpr int kQBins = 128;
// Margin, in units of the group scale a, by which a bin's edges are widened
// when it is decided which midpoints a value in it may fall on either side
// of.  It covers the rounding of the bin position x * (B / a) + C in binary32
// (B / a from an approximate reciprocal, within 2^-22) and of the thresholds
// m_k * a: below 1e-6 for values near the midpoints' range, |x / a| <= 1 +
// 3 * margin (a value far outside it lands in the first or last bin anyway).
constexpr double kQBinMargin = 1e-5;

// Pattern candidates (see Tables::pcand): a kPGrid x kPGrid grid, in units
// of the group scale a, over (min, max) of a group's other values, spanning
// the patterns' first and last centroids and an eighth of their spread on
// each side; per cell the patterns that can have the least min/max fitness
// somewhere in it.
constexpr int kPGrid = 32;
constexpr int kPCand = 8;                  // candidates a cell can list
constexpr uint8_t kPCandNone = 0xff;       // an empty slot
constexpr uint8_t kPCandMany = 0xfe;       // in slot 0: more than kPCand candidates
// Margins in units of a (and a^2 for fitness): a cell is widened by
// kPCellMargin on every side, and a pattern is a candidate where its fitness
// is within kPFitMargin of the least.  They cover the rounding of the cell
// position and of the binary32 fitness (d1^2 + d2^2 with d = min - c0 * a,
// each within 2^-23 (|c| + |d / a|) a of exact): below 1e-6 in the grid.
constexpr double kPCellMargin = 1e-5;
constexpr double kPFitMargin = 1e-5;

// Decode look-up table entry for an 8-bit window of stream bits read LSB
// first: bits 0..4 = symbol (0..15), bits 5..7 = code length - 1.  A window
// that no codeword prefixes (an incomplete codebook: Kraft sum below 1) holds
// kLutNoCode, the only entry with bit 4 set besides the clipped-stream
// table's symbol 16: the decoder stops the stream there.
constexpr uint8_t lut_entry(int sym, int len) { return (uint8_t)(sym | ((len - 1) << 5)); }
constexpr uint8_t kLutNoCode = lut_entry(17, 1);

struct alignas(256) Tables {
  // header
  uint32_t magic;
  uint32_t version;
  uint32_t size;
  uint32_t checksum;        // FNV-1a over every byte after the header
  uint32_t n_search;        // patterns the encoder searches (16, 32 or 64), derived from the centroids
  uint32_t complete;        // 1 if every codebook is complete (Kraft sum 1): no window lacks a codeword
  uint32_t reserved[58];
  // inputs
  float centroids[S][16];       // [p][0..14] centroid, [15] = 0
  uint8_t code_len[S][H][A];    // 2..8
  // derived
  float midpoints[S][16];       // [p][0..13] (c_k + c_k+1) * 0.5f, [14], [15] = +inf
  float c0c14[S][2];            // first and last centroid of each pattern
  uint32_t len4[S][A];          // byte h = code_len[p][h][s]
  uint32_t enc[S][H][A];        // canonical codeword left-aligned (bits 32 - len .. 31, most significant
                                // code bit at bit 31), 32 - len in bits 0..4
  float fp8_value[256];         // exact value of every E4M3FN code (NaN for 0x7F, 0xFF)
  uint8_t lut[S][H][256];       // decode look-up table
  // Quantiser bins (used when qbins_ok): for pattern p, a value x of a group
  // with scale a > 0 falls in bin j = min(floor(x * (qaxis[p][0] / a) +
  // qaxis[p][1]), kQBins - 1) (j = 0 below the range, kQBins - 1 above it and
  // for NaN); qbin[p][j] midpoints lie surely below every x of the bin, and
  // at most one more (midpoint qbin[p][j]) may lie on either side, so that
  // #{k : x > m_k a} = qbin[p][j] + (x > m_qbin a).  The last bin has all
  // 14 below it and compares with the largest finite float instead.
  uint8_t qbin[S][kQBins];
  float qaxis[S][2];            // [p][0] = B, bins per unit of x / a; [p][1] = C = -L * B
  uint32_t qbins_ok;            // 1 if every pattern's bins meet the rule above
  // Pattern candidates of each grid cell, lowest first (kPCandNone after the
  // last; kPCandMany in slot 0 if more than kPCand): every pattern whose
  // fitness (x - c0)^2 + (y - c14)^2, at some (x, y) of the widened cell, is
  // within kPFitMargin of the least there, less any pattern whose end
  // centroids repeat a lower one's.
  alignas(16) uint8_t pcand[kPGrid * kPGrid][kPCand];
  // The grid: cell (i, j) holds x = min / a in [x0 + i / sx, x0 + (i + 1) / sx)
  // and y = max / a likewise; {sx, -x0 * sx, sy, -y0 * sy}, so a cell index
  // is floor(min * (sx / a) + [1]).
  float pgrid[4];
};

static_assert(sizeof(Tables) % 256 == 0, "blob size");
static_assert(offsetof(Tables, lut) % 256 == 0, "lut alignment");
static_assert(offsetof(Tables, centroids) % 16 == 0, "centroid alignment");
static_assert(offsetof(Tables, qbin) % 16 == 0 && offsetof(Tables, pcand) % 16 == 0, "16-byte staging");

uint32_t checksum_of(const Tables* t);
uint32_t search_width(const Tables* t);
// The quantiser bins (Tables::qbin, qaxis) of the midpoints; returns qbins_ok.
uint32_t build_quantiser_bins(const float (*mid)[16], uint8_t (*qbin)[kQBins], float (*qaxis)[2]);
// The pattern candidates (Tables::pcand) and grid (Tables::pgrid) of the end
// centroids.
void build_pattern_candidates(const float (*c0c14)[2], uint8_t (*pcand)[kPCand], float* pgrid);

// Device checks used by every device entry point (defined with the kernels):
// ECCO_OK and the current device's compute-unit count if it is a gfx950.
int check_gfx950(int* cus);
inline bool host_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Number of groups of an n_rows x groups_per_row job.  False unless both
// factors are in 1 .. 2^32 - 1 and so is their product; the factors are
// bounded first, so the 64-bit product cannot wrap.
inline bool group_count(uint64_t n_rows, uint64_t gpr, uint64_t* total) {
  if (n_rows == 0 || gpr == 0 || n_rows >= (1ull << 32) || gpr >= (1ull << 32)) return false;
  *total = n_rows * gpr;
  return *total < (1ull << 32);
}

}  // namespace ecco
