// HIP kernels of libecco for gfx950 (MI355X) and the device entry points of
// the C ABI.
//
// Method: the Ecco block codec (pith.science review of arXiv 2505.06901).
// A group of 128 FP16 values becomes one self-contained 512-bit block: FP8
// group scale, pattern id chosen by min/max comparison, codebook id, canonical
// Huffman codewords of the 128 centroid indices, clipped at the block end or
// followed by zero fill and 15-bit outlier records ("What carries the
// argument"; "Core claim"; Fig. 4 caption; referee report major comment 1).
// The activation format codes groups of 64 values the same way, with 14-bit
// records ("free parameters": activation group size; Fig. 9 caption); the
// encode and decode kernels are templates on the group size.
//
// Kernel design (the pages' decoder is a 64-way hardware unit; on a GPU the
// parallelism comes from decoding many independent blocks at once):
//   decode  one wavefront owns a batch of 64 blocks.  The batch is loaded with
//           coalesced 16-byte loads into LDS; each lane then decodes one
//           block's codeword stream through an 8-bit-window look-up table
//           staged in LDS (all 256 codebooks, 64 KiB), four codewords per
//           64-bit bit-window refill.  Symbols are written back to LDS and the
//           wave turns around: eight values per lane (sixteen lanes per
//           128-value block) are looked up in a per-block 32-entry FP16 table
//           (15 centroids * a, the scale, outliers) and written with 128-bit
//           stores, whole rows per store instruction.
//   encode  sixteen values per lane, so eight lanes (half a DPP row) per
//           128-value group and eight groups per wave (4 lanes and 16 groups
//           for 64-value groups): segment-wide max/min/argmin/sum/scan
//           through DPP, LDS-resident thresholds for a branch-free binary
//           search, codewords merged into the block with LDS atomic OR.
//   amax    grid-stride max of |x| over up to 16 tensors in one launch.
// All floating-point steps that decide a bit of the output are single IEEE
// binary32 operations (the library is built with -ffp-contract=off).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "ecco_device.h"

namespace ecco {

// -------------------------------------------------------------------- decode

// One tensor of a decode launch, and the contiguous range of workgroups that
// decode it.
struct DecodeJob {
  const uint8_t* blocks;
  uint16_t* y;
  const Tables* tab;
  uint64_t blk_stride;   // blocks per row
  uint64_t y_stride;     // elements per row
  DivMagic gpr;          // groups per row
  uint32_t n_groups;
  uint32_t n_batches;
  float t;
  uint32_t contiguous;
  uint32_t wg_first, wg_count;
};

constexpr int kMaxJobs = ECCO_DECODE_MAX_JOBS;
static_assert(ECCO_AMAX_MAX_JOBS == kMaxJobs && kMaxJobs <= 64, "amax jobs: one array size, outputs zeroed by one wave");

struct DecodeArgs {
  DecodeJob job[kMaxJobs];
  uint32_t n_jobs;
};

// Decode of workgroup lw's share of one job: a contiguous range of the
// job's batches, interleaved over the waves.  GS values per group.
template <int GS, bool CONTIG>
__device__ __forceinline__ void decode_job(DecodeSmem<kDecWaves>& sm, const DecodeJob& a, uint32_t lw) {
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t b_end = (uint32_t)((uint64_t)a.n_batches * (lw + 1) / a.wg_count);
  uint32_t batch = (uint32_t)((uint64_t)a.n_batches * lw / a.wg_count) + wave;
  auto src_of = [&](uint32_t gidx) -> const uint8_t* {
    if (CONTIG) return a.blocks + (uint64_t)gidx * 64u;
    const uint32_t r = div_magic(gidx, a.gpr), g = gidx - r * a.gpr.d;
    return a.blocks + ((uint64_t)r * a.blk_stride + g) * 64u;
  };
  // A prefetch past the wave's last batch reads the (cached) table blob
  // instead: the loads stay unconditional without re-reading blocks.
  const uint8_t* idle = reinterpret_cast<const uint8_t*>(a.tab);
  auto fetch = [&](uint32_t b, bool live) {
    const uint32_t g0 = b * 64u;
    return fetch_batch(lane, min(64u, a.n_groups - g0), [&](uint32_t i, uint32_t q) {
      return load_stream((live ? src_of(g0 + i) : idle + 64u * (i & 63u)) + 16u * q);
    });
  };
  if (batch >= b_end) return;
  BatchRegs cur = fetch(batch, true);
  for (; batch < b_end; batch += kDecWaves) {
    const uint32_t nb = batch + kDecWaves;
    const bool more = nb < b_end;
    const BatchRegs nxt = fetch(more ? nb : batch, more);
    const uint32_t g0 = batch * 64u;
    auto sink = [&](uint32_t b, uint32_t j0, uint4 v, uint32_t, uint32_t) {
      const uint32_t gidx = g0 + b;
      uint64_t yoff;
      if (CONTIG) {
        yoff = (uint64_t)gidx * GS;
      } else {
        const uint32_t r = div_magic(gidx, a.gpr), g = gidx - r * a.gpr.d;
        yoff = (uint64_t)r * a.y_stride + (uint64_t)g * GS;
      }
      store_stream(a.y + yoff + j0, v);
    };
    const uint32_t n_valid = min(64u, a.n_groups - g0);
    if (n_valid == 64u)
      decode_batch<true, kDecWaves, GS, true>(sm, wave, lane, 64u, a.t, cur, sink);
    else
      decode_batch<false, kDecWaves, GS, true>(sm, wave, lane, n_valid, a.t, cur, sink);
    cur = nxt;
  }
}

// Each workgroup decodes one tensor, so the look-up tables it stages in LDS
// serve every block it sees.
template <int GS>
__global__ __launch_bounds__(kDecWaves * 64) void decode_kernel(DecodeArgs args) {
  __shared__ DecodeSmem<kDecWaves> sm;
  uint32_t j = 0;
  while (j + 1 < args.n_jobs && blockIdx.x >= args.job[j + 1].wg_first) ++j;
  const DecodeJob a = args.job[j];          // one copy, kept in scalar registers
  stage_decode_tables(sm, a.tab);
  __syncthreads();
  const uint32_t lw = blockIdx.x - a.wg_first;
  if (a.contiguous)
    decode_job<GS, true>(sm, a, lw);
  else
    decode_job<GS, false>(sm, a, lw);
}

// -------------------------------------------------------------------- encode

// One tensor of an encode launch, and the contiguous range of workgroups
// that encode it.
struct EncodeJob {
  const uint16_t* x;
  uint8_t* blocks;
  const Tables* tab;
  ecco_stats_t* stats;
  uint64_t x_stride;     // elements per row
  uint64_t blk_stride;   // blocks per row
  DivMagic gpr;
  uint32_t n_groups;
  uint32_t n_units;      // groups / (groups per wave), rounded up
  float t, inv_t;
  uint32_t wg_first, wg_count;
};

struct EncodeArgs {
  EncodeJob job[kMaxJobs];
  uint32_t n_jobs;
};

constexpr int kEncWaves = 4;
constexpr uint32_t kOutlierSortRounds = 3;   // more outlier rounds than this: sort each lane's keys first

// Sorts 8 keys into descending order (an optimal 19-comparator network).
__device__ __forceinline__ void sort8_desc(uint32_t (&k)[8]) {
  auto ce = [&](int i, int j) {
    const uint32_t a = max(k[i], k[j]), b = min(k[i], k[j]);
    k[i] = a;
    k[j] = b;
  };
  ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
  ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
  ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
  ce(2, 4); ce(3, 5);
  ce(1, 4); ce(3, 6);
  ce(1, 2); ce(3, 4); ce(5, 6);
}

struct EncodeSmem {
  float mid[S * 16];
  float c0c14[S * 2];
  uint32_t len4[S * A];
  uint16_t enc[S * H * A];
  float thr[kEncWaves][16][16];      // threshold tree of each group of a wave
  uint32_t out[kEncWaves][16][16];    // block words of each group of a wave
};

// Encoder lane layout: 16 values per lane, so a group takes LPG = GS / 16
// lanes (8 for 128-value groups, 4 for 64) and a wave encodes GPW = 64 / LPG
// groups at a time.  Work that every lane of a group repeats (scale,
// reductions, outlier rounds) costs less per group the fewer lanes share it.
template <int GS>
struct EncGeom {
  static constexpr int NV = 16;                   // values per lane
  static constexpr int NL = NV / 8;               // 16-byte loads (8 values) per lane
  static constexpr int LPG = GS / NV;             // lanes per group
  static constexpr int GPW = 64 / LPG;            // groups per wave
};

// (At least four waves per SIMD: the compiler is held to 128 VGPRs, which the
// kernel fits without spilling; left to itself it takes 135 and three waves.)
template <int GS>
__global__ __launch_bounds__(kEncWaves * 64, 4) void encode_kernel(EncodeArgs args) {
  uint32_t jj = 0;
  while (jj + 1 < args.n_jobs && blockIdx.x >= args.job[jj + 1].wg_first) ++jj;
  const EncodeJob a = args.job[jj];         // one copy, kept in scalar registers
  const uint32_t lw = blockIdx.x - a.wg_first;
  using Geo = GroupGeom<GS>;
  using EG = EncGeom<GS>;
  constexpr int NV = EG::NV, NL = EG::NL, LPG = EG::LPG, GPW = EG::GPW;
  static_assert((LPG == 8 || LPG == 4) && GPW <= 16, "EncodeSmem holds 16 groups per wave");
  constexpr uint32_t RB = Geo::kRecBits;
  constexpr int NSLOT = 16 / LPG;           // outlier records (and thresholds) per lane
  __shared__ EncodeSmem sm;
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < S * 16; i += blockDim.x) sm.mid[i] = (&a.tab->midpoints[0][0])[i];
  for (uint32_t i = tid; i < S * 2; i += blockDim.x) sm.c0c14[i] = (&a.tab->c0c14[0][0])[i];
  for (uint32_t i = tid; i < S * A; i += blockDim.x) sm.len4[i] = (&a.tab->len4[0][0])[i];
  for (uint32_t i = tid; i < S * H * A; i += blockDim.x) sm.enc[i] = (&a.tab->enc[0][0][0])[i];
  __syncthreads();

  const uint32_t lane = lane_id(), wave = tid >> 6;
  const uint32_t q = lane / LPG, tl = lane % LPG;
  const float t = a.t, inv_t = a.inv_t;
  const int n_search_lane = (int)(a.tab->n_search / LPG);
  float* thr = sm.thr[wave][q];
  // tree node of threshold k (k < 15): with v = k + 1 = odd * 2^z, the node
  // sits on level 3 - z at index 2^(3 - z) + (v >> (z + 1))
  auto enode = [](uint32_t k) { return (8u >> __builtin_ctz(k + 1u)) + ((k + 1u) >> (__builtin_ctz(k + 1u) + 1u)); };
  uint32_t* out = sm.out[wave][q];
  // per-lane statistics (kept by lane tl == 0 of each group)
  uint64_t st_groups = 0, st_clip = 0, st_clipv = 0, st_pad = 0, st_fill = 0, st_nonfin = 0;

  // the NV values of group g (clamped to the last group) that lane tl holds
  struct Raw {
    uint4 v[NL];
  };
  auto load_group = [&](uint32_t g) -> Raw {
    g = min(g, a.n_groups - 1u);
    const uint32_t row = div_magic(g, a.gpr), col = g - row * a.gpr.d;
    const uint16_t* src = a.x + (uint64_t)row * a.x_stride + (uint64_t)col * GS + NV * tl;
    Raw r;
#pragma unroll
    for (int c = 0; c < NL; ++c) r.v[c] = load_stream(src + 8 * c);
    return r;
  };
  const uint32_t ustride = a.wg_count * kEncWaves;
  uint32_t unit = lw * kEncWaves + wave;
  Raw raw = load_group(unit * GPW + q);
  for (; unit < a.n_units; unit += ustride) {
    const uint32_t gidx = unit * GPW + q;
    const bool valid = gidx < a.n_groups;
    // the next unit's input is loaded before this one is worked on
    const Raw nraw = load_group((unit + ustride) * GPW + q);
    uint32_t row = 0, col = 0;
    if (valid) {
      row = div_magic(gidx, a.gpr);
      col = gidx - row * a.gpr.d;
    }
    uint32_t hb[NV];
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const uint4 w = raw.v[c];
      hb[8 * c + 0] = w.x & 0xffffu;
      hb[8 * c + 1] = w.x >> 16;
      hb[8 * c + 2] = w.y & 0xffffu;
      hb[8 * c + 3] = w.y >> 16;
      hb[8 * c + 4] = w.z & 0xffffu;
      hb[8 * c + 5] = w.z >> 16;
      hb[8 * c + 6] = w.w & 0xffffu;
      hb[8 * c + 7] = w.w >> 16;
    }
    float xf[NV];
    uint32_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      xf[i] = f16_value(hb[i]);
      const uint32_t j = NV * tl + i;
      key[i] = ((hb[i] & 0x7fffu) << 8) | ((127u - j) << 1) | (hb[i] >> 15);
    }
    // 1. scale element: largest |x|, lowest index on ties
    uint32_t km = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) km = max(km, key[i]);
    km = seg_max_u32<LPG>(km);
    const float xs = f16_value((km >> 8) | ((km & 1u) << 15));
    const uint32_t s8 = fp8_encode(xs * inv_t);
    const float S = fp8_decode<0>(s8) * t;
    const float aa = fabsf(S);
    // 2. min / max of the other GS - 1 values (the scale element, whose key
    //    is km, counts as +inf for the min and -inf for the max)
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool s = key[i] == km;
      mn = fminf(mn, s ? __builtin_inff() : xf[i]);
      mx = fmaxf(mx, s ? -__builtin_inff() : xf[i]);
    }
    mn = seg_min_f32<LPG>(mn);
    mx = seg_max_f32<LPG>(mx);
    // 3. pattern: min/max squared error, lowest p on ties.  Each lane keeps its
    //    best of 64 / LPG (p rising, so a strict < keeps the lowest); the
    //    segment then takes the least fitness (non-negative, so its bits
    //    order like it) and the least p among the lanes that reach it.
    float bf = __builtin_inff();
    uint32_t bp = tl;
#pragma unroll
    for (int k = 0; k < 64 / LPG; ++k) {
      if (k >= n_search_lane) break;    // later patterns repeat earlier ones' end centroids
      const uint32_t p = tl + LPG * k;
      const float d1 = mn - sm.c0c14[2 * p] * aa;
      const float d2 = mx - sm.c0c14[2 * p + 1] * aa;
      const float f = d1 * d1 + d2 * d2;
      if (f < bf) {
        bf = f;
        bp = p;
      }
    }
    const uint32_t fmin = seg_min_u32<LPG>(__float_as_uint(bf));
    const uint32_t pstar = seg_min_u32<LPG>(__float_as_uint(bf) == fmin ? bp : 63u) & 63u;
    // 4. quantise: sym = #{k : x > m_pk * a}.  The 15 thresholds (m_p14 * a
    //    taken as +inf) sit in LDS as an implicit binary tree, node 1 the
    //    root and node u's children 2u and 2u + 1 (lane tl writes thresholds
    //    tl, tl + LPG, ... to their nodes); four compares walk it, the root
    //    one against a register copy.
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const uint32_t k = tl + LPG * sl;
      if (k < 15u) thr[enode(k)] = k < 14u ? sm.mid[pstar * 16u + k] * aa : __builtin_inff();
    }
    wave_sync();
    const float root = thr[1];
    uint32_t sym[NV];
    uint32_t l4 = 0;                       // four byte counters (codebooks 0..3): at most 16 x 8
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      uint32_t u = xf[i] > root ? 3u : 2u;
      u = u + u + (xf[i] > thr[u] ? 1u : 0u);
      u = u + u + (xf[i] > thr[u] ? 1u : 0u);
      u = u + u + (xf[i] > thr[u] ? 1u : 0u);
      sym[i] = key[i] == km ? 15u : u - 16u;
      l4 += sm.len4[pstar * 16u + sym[i]];
    }
    // 5. codebook with the shortest stream, lowest h on ties
    uint32_t l02 = seg_add_u32<LPG>(l4 & 0x00ff00ffu), l13 = seg_add_u32<LPG>((l4 >> 8) & 0x00ff00ffu);
    uint32_t Lh[4] = {l02 & 0xffffu, l13 & 0xffffu, l02 >> 16, l13 >> 16};
    uint32_t hstar = 0, L = Lh[0];
#pragma unroll
    for (int h = 1; h < 4; ++h)
      if (Lh[h] < L) { L = Lh[h]; hstar = h; }
    // 6. codewords: lane-local concatenation (each 8 values at most 64 bits),
    //    segment scan for positions, OR into the block
    uint64_t acc[NL];
    uint32_t offs[NL];
    const uint32_t eb = (pstar * 4u + hstar) * 16u;
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      acc[c] = 0;
      offs[c] = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t e = sm.enc[eb + sym[8 * c + i]];
        acc[c] |= (uint64_t)(e & 0xffu) << offs[c];
        offs[c] += e >> 8;
      }
    }
    uint32_t off = 0;
#pragma unroll
    for (int c = 0; c < NL; ++c) off += offs[c];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) out[tl + LPG * sl] = 0;
    const uint32_t incl = seg_scan_add<LPG>(off, tl);
    const uint32_t pos = 16u + incl - off;
    wave_sync();
    {
      // each part's <= 64 bits land in words w, w + 1, w + 2; words past 15
      // are beyond bit 512 and dropped, which is exactly the clipping rule
      uint32_t pp = pos;
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        const uint32_t w = pp >> 5, sh = pp & 31u;
        const uint64_t low = acc[c] << sh;
        const uint32_t top = sh ? (uint32_t)(acc[c] >> (64u - sh)) : 0u;
        if (w < 16u && (uint32_t)low) atomicOr(&out[w], (uint32_t)low);
        if (w + 1u < 16u && (uint32_t)(low >> 32)) atomicOr(&out[w + 1u], (uint32_t)(low >> 32));
        if (w + 2u < 16u && top) atomicOr(&out[w + 2u], top);
        pp += offs[c];
      }
    }
    const bool clipped = 16u + L > 512u;
    const uint32_t n = clipped ? 0u : min(16u, (496u - L) / RB);
    // 7. outliers: n largest |x| (j != i*), lower j first on ties.  Keys are
    //    unique and the scale element holds the group's largest (km), so the
    //    outliers are the next n keys: after removing km, each round takes
    //    the group's largest remaining key (lane rr % LPG keeps round rr's in
    //    slot rr / LPG) and removes it, until no group of the wave needs
    //    another round.  For a few rounds the lane's keys are searched and
    //    cleared in place; for more, the lane first sorts each 8 of its keys
    //    (descending, 19 compare-exchanges) so that a round only compares the
    //    lists' heads and the owner of the largest shifts its list.
    uint32_t mykey[NSLOT];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) mykey[sl] = 0;
    if (__any(n > kOutlierSortRounds)) {
      uint32_t k8[NL][8];
#pragma unroll
      for (int c = 0; c < NL; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) k8[c][i] = key[8 * c + i];
        sort8_desc(k8[c]);
      }
      auto pop = [&](uint32_t m) {
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const bool own = k8[c][0] == m;
#pragma unroll
          for (int i = 0; i < 7; ++i) k8[c][i] = own ? k8[c][i + 1] : k8[c][i];
          k8[c][7] = own ? 0u : k8[c][7];
        }
      };
      pop(km);                             // the scale element heads one list
      for (uint32_t rr = 0;; ++rr) {
        uint32_t head = k8[0][0];
#pragma unroll
        for (int c = 1; c < NL; ++c) head = max(head, k8[c][0]);
        const uint32_t m = seg_max_u32<LPG>(head);
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) mykey[sl] = rr == tl + LPG * sl ? m : mykey[sl];
        if (!__any(rr + 1u < n)) break;
        pop(m);
      }
    } else if (__any(n > 0u)) {
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] = key[i] == km ? 0u : key[i];
      for (uint32_t rr = 0;; ++rr) {
        uint32_t m = key[0];
#pragma unroll
        for (int i = 1; i < NV; ++i) m = max(m, key[i]);
        m = seg_max_u32<LPG>(m);
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) mykey[sl] = rr == tl + LPG * sl ? m : mykey[sl];
        if (!__any(rr + 1u < n)) break;
#pragma unroll
        for (int i = 0; i < NV; ++i) key[i] = key[i] == m ? 0u : key[i];
      }
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const uint32_t r = tl + LPG * sl;
      if (r < n) {
        const uint32_t j = 127u - ((mykey[sl] >> 1) & 127u);
        const float xv = f16_value((mykey[sl] >> 8) | ((mykey[sl] & 1u) << 15));
        const uint32_t myrec = j | (fp8_encode(xv * inv_t) << Geo::kPosBits);
        const uint32_t rp = 512u - RB * (r + 1u);
        const uint32_t w = rp >> 5, sh = rp & 31u;
        atomicOr(&out[w], myrec << sh);
        if (sh + RB > 32u) atomicOr(&out[w + 1u], myrec >> (32u - sh));
      }
    }
    if (tl == 0) atomicOr(&out[0], pstar | (hstar << 6) | (s8 << 8));
    wave_sync();
    if (valid) {
      // 16 words over LPG lanes: 16 / LPG each
      uint8_t* dst = a.blocks + ((uint64_t)row * a.blk_stride + col) * 64u;
      if constexpr (LPG == 8) {
        reinterpret_cast<uint2*>(dst)[tl] = make_uint2(out[2u * tl], out[2u * tl + 1u]);
      } else {
        reinterpret_cast<uint4*>(dst)[tl] =
            make_uint4(out[4u * tl], out[4u * tl + 1u], out[4u * tl + 2u], out[4u * tl + 3u]);
      }
    }
    if (a.stats) {
      // whole codewords inside the block (k of a clipped group)
      uint32_t e = pos, ends = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        e += sm.enc[eb + sym[i]] >> 8;
        ends += e <= 512u ? 1u : 0u;
      }
      const uint32_t k = seg_add_u32<LPG>(ends);
      bool nonfin = false;
#pragma unroll
      for (int i = 0; i < NV; ++i) nonfin |= (hb[i] & 0x7c00u) == 0x7c00u;
      const uint32_t nf = seg_max_u32<LPG>(nonfin ? 1u : 0u);
      if (valid && tl == 0) {
        st_groups += 1;
        st_clip += clipped;
        st_clipv += GS - k;
        st_pad += n;
        st_fill += clipped ? 0u : (496u - L - RB * n);
        st_nonfin += nf;
      }
    }
    raw = nraw;
    wave_sync();
  }
  if (a.stats && tl == 0 && st_groups) {
    atomicAdd(&a.stats->groups, (unsigned long long)st_groups);
    atomicAdd(&a.stats->clipped_groups, (unsigned long long)st_clip);
    atomicAdd(&a.stats->clipped_values, (unsigned long long)st_clipv);
    atomicAdd(&a.stats->padded_outliers, (unsigned long long)st_pad);
    atomicAdd(&a.stats->pad_bits, (unsigned long long)(RB * st_pad));
    atomicAdd(&a.stats->fill_bits, (unsigned long long)st_fill);
    atomicAdd(&a.stats->nonfinite_groups, (unsigned long long)st_nonfin);
  }
}

// ---------------------------------------------------------------------- amax

// One tensor of a launch; its workgroups are wg_first .. wg_first + wg_count - 1.
struct AmaxJob {
  const uint16_t* x;
  uint64_t n;
  float* out;
  uint32_t wg_first, wg_count;
};

struct AmaxArgs {
  AmaxJob job[kMaxJobs];
  uint32_t n_jobs;
};

__global__ void amax_init_kernel(AmaxArgs a) {
  if (threadIdx.x < a.n_jobs) *a.job[threadIdx.x].out = 0.0f;
}

constexpr int kAmaxUnroll = 16;      // 16-byte loads in flight per thread
constexpr uint32_t kAmaxThreads = 256;
constexpr uint32_t kAmaxWgPerCu = 2;

__device__ __forceinline__ uint32_t abs_max_bits(uint32_t m, uint32_t w) {
  uint32_t a0 = w & 0x7fffu, a1 = (w >> 16) & 0x7fffu;
  a0 = a0 > 0x7c00u ? 0u : a0;
  a1 = a1 > 0x7c00u ? 0u : a1;
  return max(m, max(a0, a1));
}

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(AmaxArgs args) {
  uint32_t jj = 0;
  while (jj + 1 < args.n_jobs && blockIdx.x >= args.job[jj + 1].wg_first) ++jj;
  const AmaxJob a = args.job[jj];
  // |x| bit patterns of finite FP16 values order like the values (NaN ignored)
  __shared__ uint32_t red[kAmaxThreads / 64];
  uint32_t m = 0;
  const uint4* x4 = reinterpret_cast<const uint4*>(a.x);
  const uint64_t n8 = a.n / 8;
  const uint64_t stride = (uint64_t)a.wg_count * kAmaxThreads;
  const uint64_t first = (uint64_t)(blockIdx.x - a.wg_first) * kAmaxThreads + threadIdx.x;
  uint64_t i = first;
  // several independent loads per thread before any is used
  for (; i + (kAmaxUnroll - 1) * stride < n8; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = load_stream(x4 + i + u * stride);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      m = abs_max_bits(m, v[u].x);
      m = abs_max_bits(m, v[u].y);
      m = abs_max_bits(m, v[u].z);
      m = abs_max_bits(m, v[u].w);
    }
  }
  for (; i < n8; i += stride) {
    const uint4 v = load_stream(x4 + i);
    m = abs_max_bits(abs_max_bits(m, v.x), v.y);
    m = abs_max_bits(abs_max_bits(m, v.z), v.w);
  }
  for (uint64_t k = n8 * 8 + first; k < a.n; k += stride) m = abs_max_bits(m, a.x[k]);
  // wave, then workgroup reduction: one atomic per workgroup
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (lane_id() == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    // the result only grows, so a workgroup whose maximum does not exceed a
    // value already read from it has nothing to add (saves most atomics)
    unsigned int* o = reinterpret_cast<unsigned int*>(a.out);
    const uint32_t mb = __float_as_uint(f16_value(m));
    if (m && mb > __hip_atomic_load(o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(o, mb);
  }
}

}  // namespace ecco

// ------------------------------------------------------------ entry points

using namespace ecco;

namespace {
struct DeviceInfo {
  int ok = 0;        // 1 gfx950, -1 other
  int cus = 0;
};
std::mutex g_mu;
DeviceInfo g_dev[64];
int launch_status() { return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP; }
}  // namespace

namespace ecco {
int check_gfx950(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ECCO_EHIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ECCO_EHIP;
    d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    d.cus = prop.multiProcessorCount;
  }
  if (d.ok != 1) return ECCO_EDEVICE;
  *cus = d.cus;
  return ECCO_OK;
}
}  // namespace ecco

namespace {

// Checks one amax job and fills its descriptor (all but the workgroup range).
int make_amax_job(const uint16_t* x, uint64_t n, float* amax, AmaxJob* out) {
  if (!x || !amax) return ECCO_EINVAL;
  if (n == 0) return ECCO_ESIZE;
  if (!host_aligned(x, 16) || !host_aligned(amax, 4)) return ECCO_EALIGN;
  out->x = x;
  out->n = n;
  out->out = amax;
  return ECCO_OK;
}

// Zeroes the outputs, then reads every job in one launch: kAmaxWgPerCu
// workgroups per CU shared out in proportion to the jobs' sizes (at least one
// each, and no more than a job has 16-byte loads for).
int launch_amax(AmaxArgs& args, int cus, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t total = 0;
  for (uint32_t k = 0; k < args.n_jobs; ++k) total += args.job[k].n;
  const uint64_t budget = (uint64_t)cus * kAmaxWgPerCu;
  uint32_t first = 0;
  for (uint32_t k = 0; k < args.n_jobs; ++k) {
    AmaxJob& j = args.job[k];
    const uint64_t want = std::max<uint64_t>(1, (j.n / 8 + kAmaxThreads - 1) / kAmaxThreads);
    // budget * n / total without overflow (budget < 2^20, n < 2^64)
    const uint64_t share = (uint64_t)((unsigned __int128)budget * j.n / total);
    j.wg_first = first;
    j.wg_count = (uint32_t)std::min<uint64_t>(want, std::max<uint64_t>(1, share));
    first += j.wg_count;
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(64), 0, s, args);
  hipLaunchKernelGGL(amax_kernel, dim3(first), dim3(kAmaxThreads), 0, s, args);
  return launch_status();
}

}  // namespace

extern "C" int ecco_amax(const uint16_t* x, uint64_t n, float* amax, void* stream) {
  AmaxArgs args{};
  args.n_jobs = 1;
  int rc = make_amax_job(x, n, amax, &args.job[0]);
  if (rc) return rc;
  int cus = 0;
  rc = check_gfx950(&cus);
  if (rc) return rc;
  return launch_amax(args, cus, stream);
}

extern "C" int ecco_amax_many(const ecco_amax_job_t* jobs, uint32_t n_jobs, void* stream) {
  if (!jobs) return ECCO_EINVAL;
  if (n_jobs == 0 || n_jobs > (uint32_t)kMaxJobs) return ECCO_ESIZE;
  AmaxArgs args{};
  args.n_jobs = n_jobs;
  for (uint32_t k = 0; k < n_jobs; ++k) {
    const int rc = make_amax_job(jobs[k].x_dev, jobs[k].n_values, jobs[k].amax_dev, &args.job[k]);
    if (rc) return rc;
  }
  int cus = 0;
  const int rc = check_gfx950(&cus);
  if (rc) return rc;
  return launch_amax(args, cus, stream);
}

namespace {

// Checks one encode job of GS-value groups and fills its kernel descriptor
// (all but the workgroup range).
template <int GS>
int make_encode_job(const uint16_t* x, uint64_t n_rows, uint64_t gpr, uint64_t x_stride, uint64_t blk_stride,
                    const void* tables, float tensor_scale, void* blocks, ecco_stats_t* stats, EncodeJob* out) {
  if (!x || !tables || !blocks) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  const uint64_t total = n_rows * gpr;
  if (n_rows == 0 || gpr == 0 || total >= (1ull << 32) || gpr >= (1ull << 32)) return ECCO_ESIZE;
  if (n_rows > 1 && (x_stride < gpr * GS || blk_stride < gpr)) return ECCO_ESIZE;
  if (!host_aligned(x, 16) || (x_stride % 8) != 0 || !host_aligned(blocks, 64) || !host_aligned(tables, 256) ||
      (stats && !host_aligned(stats, 8)))
    return ECCO_EALIGN;
  EncodeJob& a = *out;
  a.x = x;
  a.blocks = static_cast<uint8_t*>(blocks);
  a.tab = static_cast<const Tables*>(tables);
  a.stats = stats;
  a.x_stride = x_stride;
  a.blk_stride = blk_stride;
  a.gpr = make_magic((uint32_t)gpr);
  a.n_groups = (uint32_t)total;
  constexpr uint32_t kGroupsPerWave = EncGeom<GS>::GPW;
  a.n_units = (uint32_t)((total + kGroupsPerWave - 1) / kGroupsPerWave);
  a.t = tensor_scale;
  volatile float inv = 1.0f / tensor_scale;
  a.inv_t = inv;
  a.wg_first = a.wg_count = 0;
  return ECCO_OK;
}

// Up to 16 workgroups of kEncWaves waves per CU (four are resident at a time;
// the later ones even out the tail), no more than a job has units for: each
// job gets its share of the grid in proportion to its units (at least one
// workgroup), and the few workgroups the rounding leaves go one by one to the
// job whose workgroups carry the most units.
void assign_encode_workgroups(EncodeArgs& args, uint32_t cus) {
  uint64_t want[kMaxJobs], total = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) {
    want[j] = (args.job[j].n_units + kEncWaves - 1) / kEncWaves;
    total += want[j];
  }
  const uint64_t grid = std::max<uint64_t>(args.n_jobs, std::min<uint64_t>(total, (uint64_t)cus * 16));
  uint64_t used = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) {
    const uint64_t share = (uint64_t)((unsigned __int128)grid * want[j] / total);
    args.job[j].wg_count = (uint32_t)std::min<uint64_t>(want[j], std::max<uint64_t>(1, share));
    used += args.job[j].wg_count;
  }
  for (; used < grid; ++used) {
    uint32_t best = 0;
    uint64_t best_load = 0;
    for (uint32_t j = 0; j < args.n_jobs; ++j) {
      const EncodeJob& a = args.job[j];
      if (a.wg_count >= want[j]) continue;
      const uint64_t load = (a.n_units + a.wg_count - 1) / a.wg_count;
      if (load > best_load) best_load = load, best = j;
    }
    if (best_load == 0) break;
    args.job[best].wg_count++;
  }
  uint32_t first = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) {
    args.job[j].wg_first = first;
    first += args.job[j].wg_count;
  }
}

template <int GS>
int launch_encode(EncodeArgs& args, void* stream) {
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  assign_encode_workgroups(args, (uint32_t)cus);
  const EncodeJob& last = args.job[args.n_jobs - 1];
  const uint32_t grid = last.wg_first + last.wg_count;
  (void)hipGetLastError();
  hipLaunchKernelGGL(encode_kernel<GS>, dim3(grid), dim3(kEncWaves * 64), 0, static_cast<hipStream_t>(stream), args);
  return launch_status();
}

template <int GS>
int encode_one(const uint16_t* x, uint64_t n_rows, uint64_t gpr, uint64_t x_stride, uint64_t blk_stride,
               const void* tables, float tensor_scale, void* blocks, ecco_stats_t* stats, void* stream) {
  EncodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = 1;
  int rc = make_encode_job<GS>(x, n_rows, gpr, x_stride, blk_stride, tables, tensor_scale, blocks, stats,
                               &args.job[0]);
  if (rc) return rc;
  return launch_encode<GS>(args, stream);
}

}  // namespace

extern "C" int ecco_encode(const uint16_t* x, uint64_t n_rows, uint64_t gpr, uint64_t x_stride,
                           uint64_t blk_stride, const void* tables, float tensor_scale, void* blocks,
                           ecco_stats_t* stats, void* stream) {
  return encode_one<128>(x, n_rows, gpr, x_stride, blk_stride, tables, tensor_scale, blocks, stats, stream);
}

extern "C" int ecco_encode_many(const ecco_encode_job_t* jobs, uint32_t n_jobs, void* stream) {
  if (!jobs) return ECCO_EINVAL;
  if (n_jobs == 0 || n_jobs > (uint32_t)kMaxJobs) return ECCO_ESIZE;
  EncodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = n_jobs;
  for (uint32_t j = 0; j < n_jobs; ++j) {
    const ecco_encode_job_t& q = jobs[j];
    if (q.reserved != 0) return ECCO_EINVAL;
    int rc = make_encode_job<128>(q.x_dev, q.n_rows, q.groups_per_row, q.x_row_stride_elems, q.blk_row_stride_blocks,
                                  q.tables_dev, q.tensor_scale, q.blocks_dev, q.stats_dev, &args.job[j]);
    if (rc) return rc;
  }
  return launch_encode<128>(args, stream);
}

extern "C" int ecco_encode_act(const uint16_t* x, uint64_t n_rows, uint64_t gpr, uint64_t x_stride,
                               uint64_t blk_stride, const void* tables, float tensor_scale, void* blocks,
                               ecco_stats_t* stats, void* stream) {
  return encode_one<64>(x, n_rows, gpr, x_stride, blk_stride, tables, tensor_scale, blocks, stats, stream);
}

namespace {

// Checks one decode job of GS-value groups and fills its kernel descriptor
// (all but the workgroup range).
int make_decode_job(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride, uint64_t y_stride,
                    const void* tables, float tensor_scale, uint16_t* y, DecodeJob* out, uint32_t GS = 128) {
  if (!blocks || !tables || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  const uint64_t total = n_rows * gpr;
  if (n_rows == 0 || gpr == 0 || total >= (1ull << 32) || gpr >= (1ull << 32)) return ECCO_ESIZE;
  if (n_rows > 1 && (y_stride < gpr * GS || blk_stride < gpr)) return ECCO_ESIZE;
  if (!host_aligned(y, 16) || (y_stride % 8) != 0 || !host_aligned(blocks, 64) || !host_aligned(tables, 256)) return ECCO_EALIGN;
  DecodeJob& a = *out;
  a.blocks = static_cast<const uint8_t*>(blocks);
  a.y = y;
  a.tab = static_cast<const Tables*>(tables);
  a.blk_stride = blk_stride;
  a.y_stride = y_stride;
  a.gpr = make_magic((uint32_t)gpr);
  a.n_groups = (uint32_t)total;
  a.n_batches = (uint32_t)((total + 63) / 64);
  a.t = tensor_scale;
  a.contiguous = (n_rows == 1 || (blk_stride == gpr && y_stride == gpr * GS)) ? 1u : 0u;
  a.wg_first = a.wg_count = 0;
  return ECCO_OK;
}

// Splits the workgroups (at most one per CU, as many as there are batches)
// among the jobs: one each, then each further workgroup to the job whose
// workgroups carry the most batches.
void assign_workgroups(DecodeArgs& args, uint32_t cus) {
  uint64_t total = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) total += args.job[j].n_batches;
  const uint32_t grid = (uint32_t)std::max<uint64_t>(args.n_jobs, std::min<uint64_t>(total, cus));
  for (uint32_t j = 0; j < args.n_jobs; ++j) args.job[j].wg_count = 1;
  for (uint32_t k = args.n_jobs; k < grid; ++k) {
    uint32_t best = 0;
    uint64_t best_load = 0;
    for (uint32_t j = 0; j < args.n_jobs; ++j) {
      const DecodeJob& a = args.job[j];
      if (a.wg_count >= a.n_batches) continue;
      const uint64_t load = (a.n_batches + a.wg_count - 1) / a.wg_count;
      if (load > best_load) best_load = load, best = j;
    }
    if (best_load == 0) break;
    args.job[best].wg_count++;
  }
  uint32_t first = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) {
    args.job[j].wg_first = first;
    first += args.job[j].wg_count;
  }
}

template <int GS>
int launch_decode(DecodeArgs& args, void* stream) {
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  assign_workgroups(args, (uint32_t)cus);
  const DecodeJob& last = args.job[args.n_jobs - 1];
  const uint32_t grid = last.wg_first + last.wg_count;
  (void)hipGetLastError();
  hipLaunchKernelGGL(decode_kernel<GS>, dim3(grid), dim3(kDecWaves * 64), 0, static_cast<hipStream_t>(stream), args);
  return launch_status();
}

}  // namespace

extern "C" int ecco_decode(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride,
                           uint64_t y_stride, const void* tables, float tensor_scale, uint16_t* y, void* stream) {
  DecodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = 1;
  int rc = make_decode_job(blocks, n_rows, gpr, blk_stride, y_stride, tables, tensor_scale, y, &args.job[0]);
  if (rc) return rc;
  return launch_decode<128>(args, stream);
}

extern "C" int ecco_decode_act(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride,
                               uint64_t y_stride, const void* tables, float tensor_scale, uint16_t* y, void* stream) {
  DecodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = 1;
  int rc = make_decode_job(blocks, n_rows, gpr, blk_stride, y_stride, tables, tensor_scale, y, &args.job[0], 64);
  if (rc) return rc;
  return launch_decode<64>(args, stream);
}

extern "C" int ecco_decode_many(const ecco_decode_job_t* jobs, uint32_t n_jobs, void* stream) {
  if (!jobs) return ECCO_EINVAL;
  if (n_jobs == 0 || n_jobs > (uint32_t)kMaxJobs) return ECCO_ESIZE;
  DecodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = n_jobs;
  for (uint32_t j = 0; j < n_jobs; ++j) {
    const ecco_decode_job_t& q = jobs[j];
    if (q.reserved != 0) return ECCO_EINVAL;
    int rc = make_decode_job(q.blocks_dev, q.n_rows, q.groups_per_row, q.blk_row_stride_blocks,
                             q.y_row_stride_elems, q.tables_dev, q.tensor_scale, q.y_dev, &args.job[j]);
    if (rc) return rc;
  }
  return launch_decode<128>(args, stream);
}
