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
constexpr uint32_t kVersion = 1;
constexpr int G = ECCO_GROUP;
constexpr int S = ECCO_N_PATTERNS;
constexpr int C = ECCO_N_CENTROIDS;
constexpr int H = ECCO_N_CODEBOOKS;
constexpr int A = ECCO_N_SYMBOLS;

// Decode look-up table entry for an 8-bit window of stream bits read LSB
// first: bits 0..4 = symbol (0..15), bits 5..7 = code length - 1.  Every
// window decodes because codebooks are complete prefix codes.
constexpr uint8_t lut_entry(int sym, int len) { return (uint8_t)(sym | ((len - 1) << 5)); }

struct alignas(256) Tables {
  // header
  uint32_t magic;
  uint32_t version;
  uint32_t size;
  uint32_t checksum;        // FNV-1a over every byte after the header
  uint32_t n_search;        // patterns the encoder searches (16, 32 or 64), derived from the centroids
  uint32_t reserved[59];
  // inputs
  float centroids[S][16];       // [p][0..14] centroid, [15] = 0
  uint8_t code_len[S][H][A];    // 2..8
  // derived
  float midpoints[S][16];       // [p][0..13] (c_k + c_k+1) * 0.5f, [14], [15] = +inf
  float c0c14[S][2];            // first and last centroid of each pattern
  uint32_t len4[S][A];          // byte h = code_len[p][h][s]
  uint16_t enc[S][H][A];        // bits 0..7 codeword in stream order (bit-reversed), bits 8..11 length
  float fp8_value[256];         // exact value of every E4M3FN code (NaN for 0x7F, 0xFF)
  uint8_t lut[S][H][256];       // decode look-up table
};

static_assert(sizeof(Tables) % 256 == 0, "blob size");
static_assert(offsetof(Tables, lut) % 256 == 0, "lut alignment");
static_assert(offsetof(Tables, centroids) % 16 == 0, "centroid alignment");

uint32_t checksum_of(const Tables* t);
uint32_t search_width(const Tables* t);

// Device checks used by every device entry point (defined with the kernels):
// ECCO_OK and the current device's compute-unit count if it is a gfx950.
int check_gfx950(int* cus);
inline bool host_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace ecco
