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
// job's batches, interleaved over the waves.  GS values per group; STOP for
// tables with an incomplete codebook.
template <int GS, bool CONTIG, bool STOP>
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
      decode_batch<true, kDecWaves, GS, true, STOP>(sm, wave, lane, 64u, a.t, cur, sink);
    else
      decode_batch<false, kDecWaves, GS, true, STOP>(sm, wave, lane, n_valid, a.t, cur, sink);
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
  if (!a.tab->complete)
    decode_job<GS, false, true>(sm, a, lw);        // (strided addressing serves contiguous tensors too)
  else if (a.contiguous)
    decode_job<GS, true, false>(sm, a, lw);
  else
    decode_job<GS, false, false>(sm, a, lw);
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

constexpr int kEncWaves = 8;        // waves per workgroup (two workgroups resident per CU)
constexpr uint32_t kOutlierSortRounds = 3;   // more outlier rounds than this: sort each lane's keys first
// Words per group in the encoder's block staging: the block's 16, then a sink
// for the bits of a clipped stream past bit 511 (a group's codewords end by
// bit 16 + 128 * 8, word 32; the sink takes them, so the packing needs no
// bounds test), rounded up to a multiple of 4 for the 16-byte reads.
constexpr int kOutWords = 36;

// N 16-byte pieces of a table, copied from global memory to LDS by NT
// threads: every thread's loads first (index clamped to the last piece, so
// each load is unconditional and the pieces stay in registers), then its
// LDS writes.
template <uint32_t N, uint32_t NT>
struct Stage16 {
  static constexpr uint32_t K = (N + NT - 1) / NT;
  uint4 v[K];
  __device__ __forceinline__ void load(const void* src, uint32_t tid) {
    const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) v[k] = p[min(tid + k * NT, N - 1u)];
  }
  __device__ __forceinline__ void store(void* dst, uint32_t tid) const {
    uint4* p = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (uint32_t k = 0; k < K; ++k)
      if (tid + k * NT < N) p[tid + k * NT] = v[k];
  }
};

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
  alignas(16) float mid[S * 16];
  alignas(16) float c0c14[S * 2];    // pattern p's first and last centroid at 2p, 2p + 1
  alignas(16) uint32_t len4[16 + S * A];     // entry (p, s) at 16 + 16 p + s: index 16 p + u for tree leaf u = 16 + s
  alignas(16) uint32_t enc[16 + S * H * A];  // entry (p, h, s) at 16 + 16 (4 p + h) + s, likewise
  float thr[kEncWaves][16][16];      // threshold tree of each group of a wave
  uint32_t out[kEncWaves][16][kOutWords];   // block words of each group of a wave (then a sink)
  alignas(16) uint8_t qbin[S * kQBins];      // quantiser bins of each pattern
  alignas(16) float qaxis[S * 2];            // their B and C
  alignas(16) uint8_t pcand[kPGrid * kPGrid * kPCand];   // pattern candidates of each grid cell
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

// One step down the quantiser's threshold tree: u' = 2 u + !(x <= t), which
// is x > t for every x but NaN, and 1 for NaN.  The compare writes VCC and
// the add-with-carry reads it, two instructions where a compare, a select
// and a shift-or would take three.
__device__ __forceinline__ uint32_t tree_step(uint32_t u, float x, float t) {
  uint32_t r;
  asm("v_cmp_nle_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %3, %3, vcc" : "=v"(r) : "v"(x), "v"(t), "v"(u) : "vcc");
  return r;
}
// The last step of the binned quantiser: leaf 16 + s + !(x <= t), again a
// compare into VCC and one add-with-carry.
__device__ __forceinline__ uint32_t bin_step(uint32_t s, float x, float t) {
  uint32_t r;
  asm("v_cmp_nle_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, 16, %3, vcc" : "=v"(r) : "v"(x), "v"(t), "v"(s) : "vcc");
  return r;
}

// Sort key of one FP16 value of a group, from the 32-bit word holding it
// (HI: the upper half): |x| in bits 17..31, the sign in bit 0, and
// (15 - i) << 1 for the value's place i among the lane's 16.  A funnel shift
// brings |x| and the sign into place (the other half's bits land in 1..16 and
// are masked off).  The lane's part of the group index is OR-ed in where keys
// of different lanes meet (OR of (7 - lane) << 5): keys then order by |x|,
// ties going to the lower index, and are unique within a group.
template <bool HI>
__device__ __forceinline__ uint32_t value_key(uint32_t w, uint32_t i) {
  const uint32_t f = __builtin_amdgcn_alignbit(w, w, HI ? 31u : 15u);
  return (f & 0xfffe0001u) | ((15u - i) << 1);
}
__device__ __forceinline__ float key_value(uint32_t k) { return f16_value((k >> 17) | ((k & 1u) << 15)); }

// (At least four waves per SIMD: the compiler is held to 128 VGPRs.)
template <int GS>
__global__ __launch_bounds__(kEncWaves * 64, 4) void encode_kernel(EncodeArgs args) {
  const EncodeJob a = args.job[find_job<kMaxJobs>(args, blockIdx.x)];         // one copy, kept in scalar registers
  const uint32_t lw = blockIdx.x - a.wg_first;
  using Geo = GroupGeom<GS>;
  using EG = EncGeom<GS>;
  constexpr int NV = EG::NV, NL = EG::NL, LPG = EG::LPG, GPW = EG::GPW;
  static_assert((LPG == 8 || LPG == 4) && GPW <= 16, "EncodeSmem holds 16 groups per wave");
  static_assert(NV == 16, "value_key places 16 values per lane");
  constexpr uint32_t RB = Geo::kRecBits;
  constexpr int NSLOT = 16 / LPG;           // outlier records (and thresholds) per lane
  __shared__ EncodeSmem sm;
  const uint32_t tid = threadIdx.x;
  // Table staging: every global load is issued before the first LDS write,
  // so the loads' latencies overlap (the quantiser bins are copied whether
  // or not they are used).
  constexpr uint32_t NT = kEncWaves * 64;
  Stage16<S * 16 / 4, NT> st_mid;
  Stage16<S * 2 / 4, NT> st_c;
  Stage16<S * A / 4, NT> st_len;
  Stage16<S * H * A / 4, NT> st_enc;
  Stage16<S * kQBins / 16, NT> st_qb;
  Stage16<S * 2 / 4, NT> st_qa;
  Stage16<(GS == 64 ? kPGrid * kPGrid * kPCand / 16 : 1), NT> st_pc;
  st_mid.load(&a.tab->midpoints[0][0], tid);
  st_c.load(&a.tab->c0c14[0][0], tid);
  st_len.load(&a.tab->len4[0][0], tid);
  st_enc.load(&a.tab->enc[0][0][0], tid);
  st_qb.load(&a.tab->qbin[0][0], tid);
  st_qa.load(&a.tab->qaxis[0][0], tid);
  if constexpr (GS == 64) st_pc.load(&a.tab->pcand[0][0], tid);
  const bool qbins_ok = a.tab->qbins_ok != 0u;
  const float4 pgrid = make_float4(a.tab->pgrid[0], a.tab->pgrid[1], a.tab->pgrid[2], a.tab->pgrid[3]);
  st_mid.store(sm.mid, tid);
  st_c.store(sm.c0c14, tid);
  st_len.store(sm.len4 + 16, tid);
  st_enc.store(sm.enc + 16, tid);
  st_qb.store(sm.qbin, tid);
  st_qa.store(sm.qaxis, tid);
  if constexpr (GS == 64) st_pc.store(sm.pcand, tid);
  __syncthreads();

  const uint32_t lane = lane_id(), wave = tid >> 6;
  const uint32_t q = lane / LPG, tl = lane % LPG;
  const uint32_t lane_bits = (7u - tl) << 5;    // the lane's part of a key's index field
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
  // whole rows back to back (input and blocks): a group's place is its
  // index times its size, with no row / column split
  const bool contig = a.x_stride == (uint64_t)a.gpr.d * GS && a.blk_stride == a.gpr.d;
  auto load_group = [&](uint32_t g) -> Raw {
    g = min(g, a.n_groups - 1u);
    uint64_t off = (uint64_t)g * GS;
    if (!contig) {
      const uint32_t row = div_magic(g, a.gpr), col = g - row * a.gpr.d;
      off = (uint64_t)row * a.x_stride + (uint64_t)col * GS;
    }
    const uint16_t* src = a.x + off + NV * tl;
    Raw r;
#pragma unroll
    for (int c = 0; c < NL; ++c) r.v[c] = load_stream(src + 8 * c);
    return r;
  };
  const uint32_t ustride = a.wg_count * kEncWaves;
  uint32_t unit = lw * kEncWaves + wave;
  // one unit of GPW groups, whose input raw was loaded one unit ahead
  auto encode_unit = [&](uint32_t unit, const Raw& raw) {
    const uint32_t gidx = unit * GPW + q;
    const bool valid = gidx < a.n_groups;
    uint64_t bidx = gidx;                  // the block's index in a.blocks
    if (valid && !contig) {
      const uint32_t row = div_magic(gidx, a.gpr), col = gidx - row * a.gpr.d;
      bidx = (uint64_t)row * a.blk_stride + col;
    }
    uint32_t wd[NV / 2];                   // the lane's values as 8 words of two FP16 each
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      wd[4 * c + 0] = raw.v[c].x;
      wd[4 * c + 1] = raw.v[c].y;
      wd[4 * c + 2] = raw.v[c].z;
      wd[4 * c + 3] = raw.v[c].w;
    }
    float xf[NV];
    uint32_t key[NV];
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) {
      xf[2 * k] = f16_value(wd[k] & 0xffffu);
      xf[2 * k + 1] = f16_value(wd[k] >> 16);
      key[2 * k] = value_key<false>(wd[k], 2 * k);
      key[2 * k + 1] = value_key<true>(wd[k], 2 * k + 1);
    }
    // 1. scale element: largest |x|, lowest index on ties
    uint32_t km = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) km = max(km, key[i]);
    km = seg_max_u32<LPG>(km | lane_bits);
    // the lane that holds it compares its own keys with km's lane-free part;
    // the others with a value no key takes
    const uint32_t km_own = ((km ^ lane_bits) & 0xe0u) == 0u ? (km & ~0xe0u) : 0xffffffffu;
    const float xs = key_value(km);
    const uint32_t s8 = fp8_encode(xs * inv_t);
    const float S = fp8_decode<0>(s8) * t;
    const float aa = fabsf(S);
    // 2. min / max of the other GS - 1 values.  xq, the values with a quiet
    //    NaN in the scale element's place, serves both: fminf and fmaxf
    //    return the other operand of a NaN.  It is also the quantiser's
    //    input, whose steps test "not x <= t" (true for NaN, x > t for the
    //    rest): the NaN walks to the tree's last leaf, which no finite value
    //    reaches, and that leaf is symbol 15.
    float mn = __builtin_inff(), mx = -__builtin_inff();
    float xq[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      xq[i] = key[i] == km_own ? __builtin_nanf("") : xf[i];
      mn = fminf(mn, xq[i]);
      mx = fmaxf(mx, xq[i]);
    }
    mn = seg_min_f32<LPG>(mn);
    mx = seg_max_f32<LPG>(mx);
    // 3. pattern: min/max squared error, lowest p on ties.  Each lane keeps its
    //    best of 64 / LPG (p rising, so a strict < keeps the lowest); the
    //    segment then takes the least fitness (non-negative, so its bits
    //    order like it) and the least p among the lanes that reach it.
    //    64-value groups (four lanes, 16 patterns each) need not try all 64:
    //    the tables list, for each cell of a grid over (min / a, max / a), the
    //    patterns that can have the least fitness in it (the fitness
    //    differences are affine there), at most eight, which the group's
    //    lanes try (lane tl: slots tl, tl + LPG; the list rises, so a strict
    //    < still keeps the lowest p).  A wave with a group off the grid, at
    //    a = 0, or in a cell of more candidates tries every pattern.  (With
    //    eight lanes a group tries only eight patterns a lane anyway, and the
    //    two dependent LDS reads of the cell's list cost the 128-value
    //    encoder more time than the instructions they save: 278 -> 287 us on
    //    the layer, 18.9 -> 20.0 us on the KV append.)
    float bf = __builtin_inff();
    uint32_t bp;
    bool grid = false;
    const uint8_t* cand = sm.pcand;
    if constexpr (GS == 64) {
      const float ra = __builtin_amdgcn_rcpf(aa);
      int gx, gy;                          // floor, saturating (and 0 for NaN)
      asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(gx) : "v"(fmaf(mn, ra * pgrid.x, pgrid.y)));
      asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(gy) : "v"(fmaf(mx, ra * pgrid.z, pgrid.w)));
      const bool on_grid = aa > 0.0f && (uint32_t)gx < (uint32_t)kPGrid && (uint32_t)gy < (uint32_t)kPGrid;
      cand += (on_grid ? (uint32_t)(gy * kPGrid + gx) : 0u) * kPCand;
      grid = !__any(!on_grid || cand[0] == kPCandMany);
    }
    if (grid) {
      bp = 63u;
#pragma unroll
      for (int k = 0; k < kPCand / LPG; ++k) {
        const uint32_t p = cand[tl + LPG * k];
        if (p != kPCandNone) {
          const float2 c = reinterpret_cast<const float2*>(sm.c0c14)[p];
          const float d1 = mn - c.x * aa;
          const float d2 = mx - c.y * aa;
          const float f = d1 * d1 + d2 * d2;
          if (f < bf) {
            bf = f;
            bp = p;
          }
        }
      }
    } else {
      uint32_t bk = 0;                     // the lane's best pattern is tl + LPG * bk
      // the lane's end-centroid pairs: one address from an opaque copy of tl,
      // each pattern's offset a constant that the 8-byte load's offset field
      // takes (kept addresses per pattern cost registers); the pattern count
      // also goes through an opaque copy, so that each step's test is one
      // scalar compare rather than a mask kept from before the loop
      uint32_t tl_op = tl;
      asm volatile("" : "+v"(tl_op));
      const float2* cb = reinterpret_cast<const float2*>(sm.c0c14) + tl_op;
      int nsl = n_search_lane;
      asm volatile("" : "+s"(nsl));
#pragma unroll
      for (int k = 0; k < 64 / LPG; ++k) {
        if (k >= nsl) break;            // later patterns repeat earlier ones' end centroids
        const float2 c = cb[LPG * k];
        const float d1 = mn - c.x * aa;
        const float d2 = mx - c.y * aa;
        const float f = d1 * d1 + d2 * d2;
        if (f < bf) {
          bf = f;
          bk = k;
        }
      }
      bp = tl + LPG * bk;
    }
    const uint32_t fmin = seg_min_u32<LPG>(__float_as_uint(bf));
    const uint32_t pstar = seg_min_u32<LPG>(__float_as_uint(bf) == fmin ? bp : 63u) & 63u;
    // 4. quantise: sym = #{k : x > m_pk * a}, as leaf u = 16 + sym.  The 15
    //    thresholds (m_p14 * a taken as the largest finite float, which no
    //    finite x exceeds) are written to LDS by the group's lanes (lane tl:
    //    thresholds tl, tl + LPG, ...).
    //    With the tables' quantiser bins (and no group of the wave at a = 0),
    //    a value's bin j = min(floor(x * B / a + C), last) gives the count of
    //    thresholds surely below it, s = qbin[p][j], and one compare with
    //    threshold s finishes the count; the NaN in the scale element's place
    //    goes to the last bin (s = 14), whose compare it passes: symbol 15.
    //    Otherwise the thresholds form an implicit binary tree, node 1 the
    //    root and node u's children 2u and 2u + 1, which four compares walk,
    //    the root one against a register copy.
    const uint32_t* len_p = sm.len4 + 16u * pstar;       // len_p[u] = lengths of symbol u - 16
    uint32_t leaf[NV];
    uint32_t l4c[NL * 2];                  // per 4 values: four byte counters (codebooks 0..3)
#pragma unroll
    for (int c = 0; c < NL * 2; ++c) l4c[c] = 0;
    // (the lane's threshold slots are addressed from an opaque copy of tl:
    // addresses kept from before the loop cost registers)
    uint32_t tlq = tl;
    asm volatile("" : "+v"(tlq));
    if (qbins_ok && !__any(aa == 0.0f)) {
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl) {
        const uint32_t k = tl + LPG * sl;
        if (k < 15u) thr[tlq + LPG * sl] = k < 14u ? sm.mid[pstar * 16u + k] * aa : 3.40282347e38f;
      }
      wave_sync();
      const float2 ax = reinterpret_cast<const float2*>(sm.qaxis)[pstar];
      const float qa = ax.x * __builtin_amdgcn_rcpf(aa);
      const uint8_t* qb = sm.qbin + pstar * (uint32_t)kQBins;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float pos = fminf(fmaf(xq[i], qa, ax.y), (float)(kQBins - 1));
        uint32_t j;
        asm("v_cvt_u32_f32 %0, %1" : "=v"(j) : "v"(pos));   // saturates: below 0 -> bin 0
        const uint32_t sb = qb[j];
        const uint32_t u = bin_step(sb, xq[i], thr[sb]);
        leaf[i] = u;
        l4c[i / 4] += len_p[u];
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl) {
        const uint32_t k = tl + LPG * sl;
        if (k < 15u) thr[enode(tlq + LPG * sl)] = k < 14u ? sm.mid[pstar * 16u + k] * aa : 3.40282347e38f;
      }
      wave_sync();
      const float root = thr[1];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        uint32_t u = !(xq[i] <= root) ? 3u : 2u;
        u = tree_step(u, xq[i], thr[u]);
        u = tree_step(u, xq[i], thr[u]);
        u = tree_step(u, xq[i], thr[u]);
        leaf[i] = u;
        l4c[i / 4] += len_p[u];
      }
    }
    // 5. codebook with the shortest stream, lowest h on ties
    const uint32_t l4 = (l4c[0] + l4c[1]) + (l4c[2] + l4c[3]);
    uint32_t l02 = seg_add_u32<LPG>(l4 & 0x00ff00ffu), l13 = seg_add_u32<LPG>((l4 >> 8) & 0x00ff00ffu);
    uint32_t Lh[4] = {l02 & 0xffffu, l13 & 0xffffu, l02 >> 16, l13 >> 16};
    uint32_t hstar = 0, L = Lh[0];
#pragma unroll
    for (int h = 1; h < 4; ++h)
      if (Lh[h] < L) { L = Lh[h]; hstar = h; }
    // 6. codewords, four values (at most 32 bits) at a time: an entry holds
    //    the canonical codeword left-aligned and 32 - len in its low bits, so
    //    one funnel shift appends it (acc = acc << len | code); the part's
    //    bits are then reversed into stream order.  A segment scan gives each
    //    lane's position; the parts are OR-ed into the block's words, and
    //    bits past 511 land in the sink words after them and are never
    //    stored, which is exactly the clipping rule.
    const uint32_t* enc_ph = sm.enc + 16u * (pstar * 4u + hstar);   // enc_ph[u] for symbol u - 16
    uint32_t part[NL * 2], plen[NL * 2];
    uint32_t off = 0;
#pragma unroll
    for (int c = 0; c < NL * 2; ++c) {
      uint32_t acc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t e = enc_ph[leaf[4 * c + i]];
        acc = __builtin_amdgcn_alignbit(acc, e, e);
      }
      plen[c] = (l4c[c] >> (8u * hstar)) & 0xffu;
      part[c] = __builtin_bitreverse32(acc) >> ((0u - plen[c]) & 31u);
      off += plen[c];
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) out[tl + LPG * sl] = 0;
    const uint32_t incl = seg_scan_add<LPG>(off, tl);
    const uint32_t pos = 16u + incl - off;
    wave_sync();
    {
      uint32_t pp = pos;
#pragma unroll
      for (int c = 0; c < NL * 2; ++c) {
        const uint32_t w = pp >> 5;
        const uint64_t v = (uint64_t)part[c] << (pp & 31u);
        atomicOr(&out[w], (uint32_t)v);          // (rarely 0, and OR-ing 0 changes nothing)
        if ((uint32_t)(v >> 32)) atomicOr(&out[w + 1u], (uint32_t)(v >> 32));
        pp += plen[c];
      }
    }
    const bool clipped = 16u + L > 512u;
    const uint32_t n = clipped ? 0u : min(16u, (496u - L) / RB);
    // 7. outliers: n largest |x| (j != i*), lower j first on ties.  With the
    //    lane's index bits OR-ed in, keys are unique in the group and order
    //    like that rule, and the scale element holds the largest (km); so the
    //    outliers are the n keys that follow km, and round rr takes the
    //    group's largest key below the previous round's (km for the first):
    //    each lane offers its own largest key below it, a segment max picks
    //    the round's key, and lane rr % LPG keeps it in slot rr / LPG.  The
    //    rounds are unrolled, so that each updates one slot and compares the
    //    lane with a constant.  For at most kOutlierSortRounds rounds a lane
    //    finds its offer by one pass over its keys (the largest key below m
    //    is m - 1 - min(m - 1 - key), unsigned: keys not below m wrap to
    //    values above m - 1; m, one of the group's 17 largest keys, which
    //    are unique, is never 0).  For more, the lane first sorts its two 8-key
    //    halves (descending, 19 compare-exchanges each); a round then
    //    compares the two heads, and the half that held the previous round's
    //    key shifts up by one (km's half first).  Rounds go on until no group
    //    of the wave needs another.
    uint32_t mykey[NSLOT];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) mykey[sl] = 0;
    if (__any(n > kOutlierSortRounds)) {
      uint32_t k8[NL][8];
#pragma unroll
      for (int c = 0; c < NL; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) k8[c][i] = key[8 * c + i] | lane_bits;
        sort8_desc(k8[c]);
      }
      uint32_t m = km;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const bool own = k8[c][0] == m;
#pragma unroll
          for (int i = 0; i < 7; ++i) k8[c][i] = own ? k8[c][i + 1] : k8[c][i];
          k8[c][7] = own ? 0u : k8[c][7];
        }
        uint32_t head = k8[0][0];
#pragma unroll
        for (int c = 1; c < NL; ++c) head = max(head, k8[c][0]);
        m = seg_max_u32<LPG>(head);
        mykey[rr / LPG] = tl == (uint32_t)(rr % LPG) ? m : mykey[rr / LPG];
        if (!__any((uint32_t)rr + 1u < n)) break;
      }
    } else if (__any(n > 0u)) {
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] |= lane_bits;
      uint32_t m = km;
#pragma unroll
      for (int rr = 0; rr < (int)kOutlierSortRounds; ++rr) {
        const uint32_t m1 = m - 1u;
        uint32_t d = m1 - key[0];
#pragma unroll
        for (int i = 1; i < NV; ++i) d = min(d, m1 - key[i]);
        m = seg_max_u32<LPG>(d <= m1 ? m1 - d : 0u);
        mykey[rr / LPG] = tl == (uint32_t)(rr % LPG) ? m : mykey[rr / LPG];
        if (!__any((uint32_t)rr + 1u < n)) break;
      }
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const uint32_t r = tl + LPG * sl;
      if (r < n) {
        const uint32_t mk = mykey[sl];
        const uint32_t j = 127u - ((mk >> 1) & 127u);
        const uint32_t myrec = j | (fp8_encode(key_value(mk) * inv_t) << Geo::kPosBits);
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
      uint8_t* dst = a.blocks + bidx * 64u;
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
        e += 32u - (enc_ph[leaf[i]] & 31u);
        ends += e <= 512u ? 1u : 0u;
      }
      const uint32_t k = seg_add_u32<LPG>(ends);
      bool nonfin = false;
#pragma unroll
      for (int i = 0; i < NV / 2; ++i)
        nonfin |= (wd[i] & 0x7c00u) == 0x7c00u || (wd[i] & 0x7c000000u) == 0x7c000000u;
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
    wave_sync();
  };
  // the next unit's input is loaded before this one is worked on, into the
  // other of two register sets: unrolled by two, the loop copies neither.
  // (64-value groups keep the plain loop and one copy: unrolled, their
  // kernel spills a threshold address.)
  Raw ra = load_group(unit * GPW + q);
  if constexpr (GS == 128) {
    Raw rb;
    while (unit < a.n_units) {
      rb = load_group((unit + ustride) * GPW + q);
      encode_unit(unit, ra);
      unit += ustride;
      if (unit >= a.n_units) break;
      ra = load_group((unit + ustride) * GPW + q);
      encode_unit(unit, rb);
      unit += ustride;
    }
  } else {
    for (; unit < a.n_units; unit += ustride) {
      const Raw nraw = load_group((unit + ustride) * GPW + q);
      encode_unit(unit, ra);
      ra = nraw;
    }
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
  uint64_t total = 0;
  if (!group_count(n_rows, gpr, &total)) return ECCO_ESIZE;
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

// Up to 8 workgroups of kEncWaves = 8 waves per CU (two are resident at a
// time; the later ones even out the tail), and at least two units per wave,
// so a small launch does not stage the tables in LDS more often than it
// needs (eight waves share one staging): each
// job gets its share of the grid in proportion to its units (at least one
// workgroup), and the few workgroups the rounding leaves go one by one to the
// job whose workgroups carry the most units.
void assign_encode_workgroups(EncodeArgs& args, uint32_t cus) {
  uint64_t want[kMaxJobs], total = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) {
    want[j] = (args.job[j].n_units + 2 * kEncWaves - 1) / (2 * kEncWaves);
    total += want[j];
  }
  const uint64_t grid = std::max<uint64_t>(args.n_jobs, std::min<uint64_t>(total, (uint64_t)cus * 8));
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
  uint64_t total = 0;
  if (!group_count(n_rows, gpr, &total)) return ECCO_ESIZE;
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
