// Speculative block decode for gfx950: the pages' parallel Huffman decoder
// mapped onto one wavefront per block, kept beside the lane-serial decoder of
// ecco_kernels.hip for comparison (both give identical output).
//
// The pages' decompressor cuts a block's codeword stream into segments and
// decodes every segment from every possible start offset at once, then a
// merge network picks, segment by segment, the one decode that continues the
// previous segment's, and the symbol counts give each segment its place in
// the output (Ecco review, "The pith"; Fig. 8 caption: 64-way parallel
// decoder).  Here:
//   segments  lane i owns stream bits 16 + 8 i .. 16 + 8 i + 7 (62 lanes cover
//             bits 16..511); a codeword is at most 8 bits, so for each of the
//             8 start offsets a lane meets at most 4 codeword starts and the
//             decode leaves the segment at offset 0..7 of the next one; the
//             lane looks up the codeword at each of its 8 bits once and runs
//             the 8 decodes from those entries
//   resolve   a six-step scan over the lanes composes the
//             segments' 8-entry exit maps and sums their symbol counts, so
//             lane i learns where segments 0 .. i - 1 leave the stream when
//             segment 0 is entered at offset 0 (its own entry) and how many
//             codewords they hold (its first output index): the pages' merge
//             stages, one per doubling of the span
//   emit      each lane follows its segment's decode from its true entry and
//             writes the symbols whose index is below 128; the 128th
//             codeword's end fixes the outlier-record count as in the format
// The rest (value table, records, FP16 store) is the format's dequantisation.
// Every block costs 8 table look-ups per lane (one per stream bit) and a
// six-step merge, against one look-up per codeword (2 per lane-block) for
// the lane-serial decoder; the latter is the library's decoder because it
// does far less work per block.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ecco_device.h"

namespace ecco {

constexpr int kSpecWaves = 8;                     // waves (blocks in flight) per workgroup
constexpr int kSegments = (512 - 16) / 8;         // 62 segments of 8 stream bits
// DPP controls (GFX9 encoding) of the merge scan
constexpr int kRowBcast15 = 0x142;                // lane 15 of each row -> the next row
constexpr int kRowBcast31 = 0x143;                // lane 31 -> rows 2 and 3
constexpr int kWaveShr1 = 0x138;                  // lane i - 1 -> lane i, across rows

struct SpecArgs {
  const uint8_t* blocks;
  uint16_t* y;
  const Tables* tab;
  uint64_t blk_stride, y_stride;
  DivMagic gpr;
  uint32_t n_groups;
  float t;
};

struct SpecSmem {
  uint8_t lut[S * H * 256];
  float cent[S * 16];
  uint32_t blk[kSpecWaves][20];                   // 16 block words + zero pad (windows past bit 512)
  uint8_t sym[kSpecWaves][128 + 16];              // value-table byte offset per position (+ pad)
  uint16_t vtab[kSpecWaves][32];
};

__global__ __launch_bounds__(kSpecWaves * 64) void decode_spec_kernel(SpecArgs a) {
  __shared__ SpecSmem sm;
  {
    const uint4* src = reinterpret_cast<const uint4*>(&a.tab->lut[0][0][0]);
    uint4* dst = reinterpret_cast<uint4*>(sm.lut);
    for (uint32_t i = threadIdx.x; i < S * H * 256 / 16; i += blockDim.x) dst[i] = src[i];
    const float* c = &a.tab->centroids[0][0];
    for (uint32_t i = threadIdx.x; i < S * 16; i += blockDim.x) sm.cent[i] = c[i];
  }
  __syncthreads();
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t* W = sm.blk[wave];
  uint8_t* sym = sm.sym[wave];
  uint16_t* vt = sm.vtab[wave];
  const float t = a.t;
  const uint32_t stride = gridDim.x * kSpecWaves;
  // word lane % 16 of block gg; past the last block, the last block's (loaded
  // unconditionally so that the load overlaps the current block's decode)
  auto block_word = [&](uint64_t gg) -> uint32_t {
    const uint32_t gc = (uint32_t)min(gg, (uint64_t)a.n_groups - 1u);
    const uint32_t r = div_magic(gc, a.gpr), c = gc - r * a.gpr.d;
    return reinterpret_cast<const uint32_t*>(a.blocks + ((uint64_t)r * a.blk_stride + c) * 64u)[lane & 15u];
  };
  uint32_t cur = block_word(blockIdx.x * kSpecWaves + wave);
  for (uint32_t g = blockIdx.x * kSpecWaves + wave; g < a.n_groups; g += stride) {
    const uint32_t row = div_magic(g, a.gpr), col = g - row * a.gpr.d;
    const uint32_t nxt = block_word((uint64_t)g + stride);
    if (lane < 20u) W[lane] = lane < 16u ? cur : 0u;
    if (lane < 36u) reinterpret_cast<uint32_t*>(sym)[lane] = 0x20202020u;   // entry 16: +0 past a clip
    wave_sync();
    const uint32_t head = W[0];
    const uint32_t lutb = ((head & 63u) * 4u + ((head >> 6) & 3u)) * 256u;
    bool full;                                      // 128 codewords read
    uint32_t E;                                     // stream end after codeword 128
    if (a.tab->complete) {
      // the two words holding bits seg0 .. seg0 + 15 of this lane's segment
      const uint32_t seg0 = 16u + 8u * min(lane, (uint32_t)kSegments - 1u);
      const uint32_t wlo = W[seg0 >> 5], whi = W[(seg0 >> 5) + 1u], wbase = seg0 & ~31u;
      const bool last = lane == (uint32_t)kSegments - 1u;
      // 1. speculative decode.  A codeword may start at any of the segment's
      //    8 bits: one look-up each gives its table entry (bytes of Elo, Ehi)
      //    and the place q + length it ends (bytes of Nlo, Nhi; in the last
      //    segment 16 marks a codeword that does not fit before bit 512, where
      //    the stream is clipped).  The 8 decodes, one per entry offset o, then
      //    run side by side in the bytes of P (position reached from o), a byte
      //    gather per step; byte o of the map M is where decode o leaves the
      //    segment (offset into the next one), byte o of K how many codewords
      //    it read.  A codeword is at least 2 bits, so 4 steps finish them all.
      uint32_t Elo = 0, Ehi = 0, Nlo = 0, Nhi = 0;
  #pragma unroll
      for (uint32_t q = 0; q < 8u; ++q) {
        const uint32_t e = sm.lut[lutb + (window(wlo, whi, seg0 + q - wbase) & 255u)];
        uint32_t nq = q + (e >> 5) + 1u;
        if (last && nq > 8u) nq = 16u;
        const uint32_t sh = 8u * (q & 3u);
        if (q < 4u) {
          Elo |= e << sh;
          Nlo |= nq << sh;
        } else {
          Ehi |= e << sh;
          Nhi |= nq << sh;
        }
      }
      uint32_t Plo = 0x03020100u, Phi = 0x07060504u, Klo = 0, Khi = 0;
      auto step = [&](uint32_t& P, uint32_t& K) {
        const uint32_t out = ((P >> 3) | (P >> 4)) & 0x01010101u;      // 1 in each byte whose decode has ended
        const uint32_t G = __builtin_amdgcn_perm(Nhi, Nlo, P & 0x07070707u);
        const uint32_t live = (out ^ 0x01010101u) * 0xffu;
        K += (live & 0x01010101u) & (~G >> 4);                          // a codeword read unless it does not fit
        P = (G & live) | (P & ~live);
      };
  #pragma unroll
      for (int k = 0; k < 4; ++k) {
        step(Plo, Klo);
        step(Phi, Khi);
      }
      uint32_t Mlo = (Plo - 0x08080808u) & 0x07070707u, Mhi = (Phi - 0x08080808u) & 0x07070707u;
      // 2. resolve.  An inclusive scan over the lanes composes the spans: a
      //    lane that holds the map of segments j .. i (entry offset of the
      //    first -> entry offset of the one after the last) and their codeword
      //    counts per entry offset takes in the span that ends at j - 1 from a
      //    lower lane: M(o) = M_i(M_prev(o)), a byte gather that v_perm_b32 does
      //    for four entries at once (selectors 0..7 pick bytes of the 8-byte
      //    map), and K(o) = K_prev(o) + K_i(M_prev(o)), bytewise (a count is at
      //    most 4 per segment, so no byte carries over).  Six DPP steps: shifts
      //    by 1, 2, 4, 8 inside each row of 16 lanes, then the last lane of row
      //    0 (2) into row 1 (3), then lane 31 into rows 2 and 3.
      auto join = [&](uint32_t plo, uint32_t phi, uint32_t qlo, uint32_t qhi, bool take) {
        if (take) {
          const uint32_t nlo = __builtin_amdgcn_perm(Mhi, Mlo, plo), nhi = __builtin_amdgcn_perm(Mhi, Mlo, phi);
          const uint32_t klo = qlo + __builtin_amdgcn_perm(Khi, Klo, plo);
          const uint32_t khi = qhi + __builtin_amdgcn_perm(Khi, Klo, phi);
          Mlo = nlo;
          Mhi = nhi;
          Klo = klo;
          Khi = khi;
        }
      };
      join(dpp_u32<kRowShr1>(Mlo), dpp_u32<kRowShr1>(Mhi), dpp_u32<kRowShr1>(Klo), dpp_u32<kRowShr1>(Khi),
           (lane & 15u) >= 1u);
      join(dpp_u32<kRowShr2>(Mlo), dpp_u32<kRowShr2>(Mhi), dpp_u32<kRowShr2>(Klo), dpp_u32<kRowShr2>(Khi),
           (lane & 15u) >= 2u);
      join(dpp_u32<kRowShr4>(Mlo), dpp_u32<kRowShr4>(Mhi), dpp_u32<kRowShr4>(Klo), dpp_u32<kRowShr4>(Khi),
           (lane & 15u) >= 4u);
      join(dpp_u32<kRowShr8>(Mlo), dpp_u32<kRowShr8>(Mhi), dpp_u32<kRowShr8>(Klo), dpp_u32<kRowShr8>(Khi),
           (lane & 15u) >= 8u);
      join(dpp_u32<kRowBcast15>(Mlo), dpp_u32<kRowBcast15>(Mhi), dpp_u32<kRowBcast15>(Klo),
           dpp_u32<kRowBcast15>(Khi), (lane & 16u) != 0u);
      join(dpp_u32<kRowBcast31>(Mlo), dpp_u32<kRowBcast31>(Mhi), dpp_u32<kRowBcast31>(Klo),
           dpp_u32<kRowBcast31>(Khi), lane >= 32u);
      // entry 0 of segment 0: lane i enters where segments 0 .. i - 1 leave
      const uint32_t pm = dpp_u32<kWaveShr1>(Mlo), pk = dpp_u32<kWaveShr1>(Klo);
      const uint32_t my_entry = lane ? (pm & 255u) : 0u;
      const uint32_t my_start = lane ? (pk & 255u) : 0u;
      const uint32_t my_cnt = (Klo & 255u) - my_start;
      const uint32_t start = __builtin_amdgcn_readlane(Klo, kSegments - 1) & 255u;
      full = start >= 128u;               // 128 whole codewords fit: not clipped
      // 3. emit: the codewords of the decode from the true entry, from the
      //    entries already looked up
      uint32_t end = 0;                               // stream end after codeword 128 (its lane only)
      if (lane < (uint32_t)kSegments) {
        uint32_t q = my_entry;
  #pragma unroll
        for (uint32_t s = 0; s < 4u; ++s) {
          if (s < my_cnt) {
            const uint32_t e = __builtin_amdgcn_perm(Ehi, Elo, q) & 255u;   // the entry looked up at bit q
            const uint32_t idx = my_start + s;
            q += (e >> 5) + 1u;
            if (idx < 128u) sym[idx] = (uint8_t)((e & 31u) << 1);
            if (idx == 127u) end = seg0 + q;
          }
        }
      }
      const uint64_t has_end = __ballot(end != 0u);
      E = has_end ? __builtin_amdgcn_readlane(end, (int)__builtin_ctzll(has_end)) : 0u;
    } else {
      // tables with an incomplete codebook: lane 0 reads the stream alone,
      // stopping at a codeword that does not fit before bit 512 or at a
      // window that no codeword starts (kLutNoCode, bit 4 of the entry)
      uint32_t k = 0, pos = 16;
      if (lane == 0u) {
        uint32_t kw = 0, lo = W[0], hi = W[1];
        for (; k < 128u; ++k) {
          const uint32_t e = sm.lut[lutb + (window(lo, hi, pos - 32u * kw) & 255u)];
          const uint32_t np = pos + (e >> 5) + 1u;
          if ((e & 0x10u) != 0u || np > 512u) break;
          sym[k] = (uint8_t)((e & 31u) << 1);
          pos = np;
          if (pos - 32u * kw >= 32u) {              // pos <= 512: kw <= 16, W[kw + 1] within the 20 words
            ++kw;
            lo = hi;
            hi = W[kw + 1u];
          }
        }
      }
      full = __builtin_amdgcn_readfirstlane(k) == 128u;
      E = __builtin_amdgcn_readfirstlane(pos);
    }
    const uint32_t RB = 15u;
    const uint32_t n = full ? min(16u, (512u - E) / RB) : 0u;
    // 4. value table: [0..14] fp16(c * a), [15] fp16(S), [16 + r] record r or +0
    const uint32_t p = head & 63u;
    const float Sv = fp8_decode<1>(head) * t;
    const float aa = fabsf(Sv);
    if (lane < 15u) vt[lane] = (uint16_t)f16_bits(sm.cent[p * 16u + lane] * aa);
    if (lane == 15u) vt[15] = (uint16_t)f16_bits(Sv);
    uint32_t jrec = 0;
    if (lane >= 16u && lane < 32u) {
      const uint32_t r = lane - 16u;
      uint32_t hv = 0;
      if (r < n) {
        const uint32_t bpos = 512u - RB * (r + 1u);
        const uint32_t rec = window(W[bpos >> 5], W[(bpos >> 5) + 1u], bpos & 31u) & 0x7fffu;
        hv = f16_bits(fp8_decode<0>(rec >> 7) * t);
        jrec = rec & 127u;
      }
      vt[16u + r] = (uint16_t)hv;
    }
    wave_sync();
    // outlier positions take entry 16 + r, in record order (a later record wins)
    for (uint32_t r = 0; r < n; ++r) {
      if (lane == 16u + r) sym[jrec] = (uint8_t)(2u * (16u + r));
      wave_sync();
    }
    // 5. FP16 store: two values per lane, one 256-byte row per wave
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(vt);
    const uint32_t v0 = *reinterpret_cast<const uint16_t*>(tb + sym[2u * lane]);
    const uint32_t v1 = *reinterpret_cast<const uint16_t*>(tb + sym[2u * lane + 1u]);
    reinterpret_cast<uint32_t*>(a.y + (uint64_t)row * a.y_stride + (uint64_t)col * 128u)[lane] = v0 | (v1 << 16);
    wave_sync();
    cur = nxt;
  }
}


// ------------------------------------------------ segments of 2, 4 or 8 lanes
//
// The middle ground between one lane per block (ecco_decode) and one wave per
// block (above): L lanes share a block, lane k owning stream bits
// 16 + k * SB .. 16 + (k + 1) * SB - 1 (SB = 496 / L: 248, 124 or 62 bits).
//   speculate  each lane decodes its segment from its first bit, as if a
//              codeword started there, keeping the look-up entries (symbol
//              and length) in LDS, until a codeword ends at or past the
//              segment's end (in the last segment: until the next codeword
//              would end past bit 512, the clip rule); the overshoot is the
//              exit offset into the next segment
//   resolve    segment k's true entry is segment k - 1's exit.  A lane whose
//              entry differs from its guess decodes again from the true
//              entry until the new path meets a codeword boundary of the
//              speculative one (prefix codes fall back into step within a
//              few codewords, and from there the two paths agree), keeping
//              only the new prefix.  If the new path leaves the segment
//              without meeting the old one, its exit differs too, and the
//              next segment redoes its decode in the next round; L rounds
//              settle every block (the pages' merge, one segment at a time)
//   emit       a segmented scan of the lanes' codeword counts gives each
//              lane its first output index; each lane writes the value-table
//              offsets of its codewords below index 128 and the one holding
//              codeword 127 reports where it ends (the outlier records'
//              start); then the value table, the records and the FP16 store
//              as in the other decoders
// One look-up per codeword as in the lane-serial decoder, plus the re-decoded
// prefixes, an LDS write and read per codeword, and a wave holds 64 / L
// blocks instead of 64.
template <int L>
struct SegGeom {
  static_assert(L == 2 || L == 4 || L == 8, "2, 4 or 8 lanes per block");
  static constexpr uint32_t kBlocks = 64 / L;                 // blocks per wave pass
  static constexpr uint32_t kSegBits = (512 - 16) / L;        // stream bits per segment
  static constexpr int kWaves = L == 2 ? 2 : L == 4 ? 4 : 8;  // waves per workgroup (LDS bound)
  static constexpr uint32_t kChunks = kBlocks * 4;            // 16-byte pieces of a pass
  static constexpr uint32_t kChunksPerLane = (kChunks + 63) / 64;
};

template <int L>
struct SegSmem {
  using G = SegGeom<L>;
  uint8_t lut[S * H * 256];
  float cent[S * 16];
  uint32_t blk[G::kWaves][G::kBlocks][20];            // 16 block words + zero pad (windows past bit 512)
  uint8_t spec[G::kWaves][64][G::kSegBits];           // speculative look-up entries per lane
  uint8_t pre[G::kWaves][64][G::kSegBits];            // re-decoded prefix per lane
  uint32_t sym[G::kWaves][G::kBlocks][36];            // value-table byte offset per position (+ pad)
  uint16_t vt[G::kWaves][G::kBlocks][32];
};

template <int L>
__global__ __launch_bounds__(SegGeom<L>::kWaves * 64) void decode_seg_kernel(SpecArgs a) {
  using G = SegGeom<L>;
  constexpr uint32_t SB = G::kSegBits, NB = G::kBlocks;
  __shared__ SegSmem<L> sm;
  {
    const uint4* src = reinterpret_cast<const uint4*>(&a.tab->lut[0][0][0]);
    uint4* dst = reinterpret_cast<uint4*>(sm.lut);
    for (uint32_t i = threadIdx.x; i < S * H * 256 / 16; i += blockDim.x) dst[i] = src[i];
    const float* c = &a.tab->centroids[0][0];
    for (uint32_t i = threadIdx.x; i < S * 16; i += blockDim.x) sm.cent[i] = c[i];
  }
  __syncthreads();
  const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t stride = (uint64_t)gridDim.x * G::kWaves * NB;
  const uint64_t n_groups = a.n_groups;
  // piece c of the pass starting at group gb: bytes 16 (c & 3) .. + 15 of
  // group gb + (c >> 2); past the last group, the last group's (never stored)
  auto load = [&](uint64_t gb, uint32_t c) -> uint4 {
    const uint32_t gg = (uint32_t)min(gb + min(c, G::kChunks - 1u) / 4u, n_groups - 1u);
    const uint32_t r = div_magic(gg, a.gpr), col = gg - r * a.gpr.d;
    return load_stream(a.blocks + ((uint64_t)r * a.blk_stride + col) * 64u + 16u * (c & 3u));
  };
  uint64_t g0 = ((uint64_t)blockIdx.x * G::kWaves + wave) * NB;
  uint4 cur[G::kChunksPerLane];
#pragma unroll
  for (uint32_t i = 0; i < G::kChunksPerLane; ++i) cur[i] = load(g0, lane + 64u * i);
  uint32_t (*B)[20] = sm.blk[wave];
  uint8_t* sp = sm.spec[wave][lane];
  uint8_t* pr = sm.pre[wave][lane];
  const uint32_t bi = lane / L, k = lane % L;
  const bool last = k == L - 1u;
  const uint32_t s = 16u + k * SB, ek = last ? 512u : s + SB;
  const float t = a.t;
  for (; g0 < n_groups; g0 += stride) {
    uint4 nxt[G::kChunksPerLane];
#pragma unroll
    for (uint32_t i = 0; i < G::kChunksPerLane; ++i) nxt[i] = load(g0 + stride, lane + 64u * i);
#pragma unroll
    for (uint32_t i = 0; i < G::kChunksPerLane; ++i) {
      const uint32_t c = lane + 64u * i;
      if (c < G::kChunks) {
        uint32_t* d = &B[c >> 2][4u * (c & 3u)];
        d[0] = cur[i].x;
        d[1] = cur[i].y;
        d[2] = cur[i].z;
        d[3] = cur[i].w;
      }
    }
    if (lane < NB) {
      B[lane][16] = 0u;
      B[lane][17] = 0u;
      B[lane][18] = 0u;
      B[lane][19] = 0u;
    }
    for (uint32_t i = lane; i < NB * 36u; i += 64u) (&sm.sym[wave][0][0])[i] = 0x20202020u;  // entry 16: +0
    wave_sync();
    const uint32_t* W = B[bi];
    const uint32_t head = W[0];
    const uint32_t lutb = ((head & 63u) * 4u + ((head >> 6) & 3u)) * 256u;
    // decodes from bit `pos` while pos < ek and the codeword fits before bit
    // 512, handing each entry to put(); returns the position reached
    auto run = [&](uint32_t pos, auto put) -> uint32_t {
      uint32_t kw = pos >> 5, lo = W[kw], hi = W[kw + 1u];
      while (pos < ek) {
        const uint32_t e = sm.lut[lutb + (window(lo, hi, pos - 32u * kw) & 255u)];
        const uint32_t np = pos + (e >> 5) + 1u;
        if (np > 512u) break;
        put(e);
        pos = np;
        if (pos - 32u * kw >= 32u) {
          ++kw;
          lo = hi;
          hi = W[kw + 1u];
        }
      }
      return pos;
    };
    uint8_t* row = reinterpret_cast<uint8_t*>(sm.sym[wave][bi]);
    bool full;                                       // 128 codewords read
    uint32_t E;                                      // stream end after codeword 128
    if (a.tab->complete) {
      // 1. speculate
      uint32_t cnt = 0;
      const uint32_t spos = run(s, [&](uint32_t e) { sp[cnt++] = (uint8_t)e; });
      uint32_t xit = last ? 0u : spos - ek;           // exit offset into the next segment
      // 2. resolve: final codewords = pr[0 .. n_new) then sp[jo .. cnt)
      uint32_t ent = 0, n_new = 0, jo = 0;
      for (uint32_t round = 0; round < (uint32_t)L; ++round) {
        const uint32_t left = __shfl(xit, k == 0u ? lane : lane - 1u);
        const uint32_t want = k == 0u ? 0u : left;
        const bool redo = want != ent;
        if (!__any(redo)) break;
        if (redo) {
          ent = want;
          n_new = 0;
          uint32_t end;
          if (round == 0u) {
            // meet the speculative path: po walks its codeword boundaries
            uint32_t pn = s + ent, po = s;
            jo = 0;
            uint32_t kw = pn >> 5, lo = W[kw], hi = W[kw + 1u];
            while (true) {
              while (po < pn && jo < cnt) po += (uint32_t)(sp[jo++] >> 5) + 1u;
              if (po == pn || pn >= ek) break;
              const uint32_t e = sm.lut[lutb + (window(lo, hi, pn - 32u * kw) & 255u)];
              const uint32_t np = pn + (e >> 5) + 1u;
              if (np > 512u) break;
              pr[n_new++] = (uint8_t)e;
              pn = np;
              if (pn - 32u * kw >= 32u) {
                ++kw;
                lo = hi;
                hi = W[kw + 1u];
              }
            }
            if (po == pn) {
              end = spos;                              // met: the rest is the speculative decode
            } else {
              end = pn;
              jo = cnt;
            }
          } else {
            end = run(s + ent, [&](uint32_t e) { pr[n_new++] = (uint8_t)e; });
            jo = cnt;
          }
          if (!last) xit = end - ek;
        }
      }
      // 3. output indices: inclusive scan of the codeword counts over the block's lanes
      const uint32_t mine = n_new + (cnt - jo);
      uint32_t incl = mine;
  #pragma unroll
      for (uint32_t d = 1; d < (uint32_t)L; d <<= 1) {
        const uint32_t v = __shfl_up(incl, d, L);
        if (k >= d) incl += v;
      }
      const uint32_t base = incl - mine;
      const uint32_t total = __shfl(incl, L - 1, L);
      full = total >= 128u;
      E = 0;                                           // end of codeword 127 (its lane only)
      {
        uint32_t pe = s + ent;
        const uint32_t m = base < 128u ? min(mine, 128u - base) : 0u;
        for (uint32_t i = 0; i < m; ++i) {
          const uint32_t e = i < n_new ? pr[i] : sp[jo + i - n_new];
          row[base + i] = (uint8_t)((e & 31u) << 1);
          pe += (e >> 5) + 1u;
          if (base + i == 127u) E = pe;
        }
      }
  #pragma unroll
      for (uint32_t d = 1; d < (uint32_t)L; d <<= 1) E = max(E, (uint32_t)__shfl_xor(E, d, L));
    } else {
      // tables with an incomplete codebook: the block's first lane reads the
      // stream alone, stopping at a codeword that does not fit before bit
      // 512 or at a window that no codeword starts (kLutNoCode, bit 4)
      uint32_t nk = 0, pos = 16;
      if (k == 0u) {
        uint32_t kw = 0, lo = W[0], hi = W[1];
        for (; nk < 128u; ++nk) {
          const uint32_t e = sm.lut[lutb + (window(lo, hi, pos - 32u * kw) & 255u)];
          const uint32_t np = pos + (e >> 5) + 1u;
          if ((e & 0x10u) != 0u || np > 512u) break;
          row[nk] = (uint8_t)((e & 31u) << 1);
          pos = np;
          if (pos - 32u * kw >= 32u) {               // pos <= 512: kw <= 16, W[kw + 1] within the 20 words
            ++kw;
            lo = hi;
            hi = W[kw + 1u];
          }
        }
      }
      full = (uint32_t)__shfl(nk, 0, L) == 128u;
      E = (uint32_t)__shfl(pos, 0, L);
    }
    // 4. value table: [0..14] fp16(c * a), [15] fp16(S), [16 + r] record r or +0
    const uint32_t n = full ? min(16u, (512u - E) / 15u) : 0u;
    const uint32_t p = head & 63u;
    const float Sv = fp8_decode<1>(head) * t;
    const float aa = fabsf(Sv);
    uint16_t* vt = sm.vt[wave][bi];
    for (uint32_t j = k; j < 32u; j += L) {
      uint32_t hv;
      if (j < 15u) {
        hv = f16_bits(sm.cent[p * 16u + j] * aa);
      } else if (j == 15u) {
        hv = f16_bits(Sv);
      } else {
        const uint32_t r = j - 16u;
        hv = 0u;
        if (r < n) {
          const uint32_t bpos = 512u - 15u * (r + 1u);
          const uint32_t rec = window(W[bpos >> 5], W[(bpos >> 5) + 1u], bpos & 31u) & 0x7fffu;
          hv = f16_bits(fp8_decode<0>(rec >> 7) * t);
        }
      }
      vt[j] = (uint16_t)hv;
    }
    wave_sync();
    // outlier positions take entry 16 + r, in record order (a later record wins)
    if (k == 0u) {
      for (uint32_t r = 0; r < n; ++r) {
        const uint32_t bpos = 512u - 15u * (r + 1u);
        const uint32_t rec = window(W[bpos >> 5], W[(bpos >> 5) + 1u], bpos & 31u) & 0x7fffu;
        row[rec & 127u] = (uint8_t)(2u * (16u + r));
      }
    }
    wave_sync();
    // 5. FP16 store: 8 values per lane, four 256-byte rows per step
#pragma unroll
    for (uint32_t it = 0; it < NB / 4u; ++it) {
      const uint32_t b = 4u * it + lane / 16u, j0 = 8u * (lane % 16u);
      const uint64_t gg = g0 + b;
      const uint2 sv = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(sm.sym[wave][b]) + j0);
      const uint8_t* tb = reinterpret_cast<const uint8_t*>(sm.vt[wave][b]);
      auto v = [&](uint32_t w, int q) -> uint32_t {
        return *reinterpret_cast<const uint16_t*>(tb + ((w >> (8 * q)) & 0xffu));
      };
      const uint4 o = make_uint4(v(sv.x, 0) | (v(sv.x, 1) << 16), v(sv.x, 2) | (v(sv.x, 3) << 16),
                                 v(sv.y, 0) | (v(sv.y, 1) << 16), v(sv.y, 2) | (v(sv.y, 3) << 16));
      if (gg < n_groups) {
        const uint32_t r = div_magic((uint32_t)gg, a.gpr), col = (uint32_t)gg - r * a.gpr.d;
        store_stream(a.y + (uint64_t)r * a.y_stride + (uint64_t)col * 128u + j0, o);
      }
    }
    wave_sync();
#pragma unroll
    for (uint32_t i = 0; i < G::kChunksPerLane; ++i) cur[i] = nxt[i];
  }
}

}  // namespace ecco

using namespace ecco;

extern "C" int ecco_decode_speculative(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride,
                                       uint64_t y_stride, const void* tables, float tensor_scale, uint16_t* y,
                                       void* stream) {
  if (!blocks || !tables || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  uint64_t total = 0;
  if (!group_count(n_rows, gpr, &total)) return ECCO_ESIZE;
  if (n_rows > 1 && (y_stride < gpr * 128 || blk_stride < gpr)) return ECCO_ESIZE;
  if (!host_aligned(y, 16) || (y_stride % 8) != 0 || !host_aligned(blocks, 64) || !host_aligned(tables, 256))
    return ECCO_EALIGN;
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  SpecArgs a;
  a.blocks = static_cast<const uint8_t*>(blocks);
  a.y = y;
  a.tab = static_cast<const Tables*>(tables);
  a.blk_stride = n_rows > 1 ? blk_stride : gpr;
  a.y_stride = n_rows > 1 ? y_stride : gpr * 128;
  a.gpr = make_magic((uint32_t)gpr);
  a.n_groups = (uint32_t)total;
  a.t = tensor_scale;
  const uint64_t want = (total + kSpecWaves - 1) / kSpecWaves;
  const uint32_t grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)cus * 2));
  (void)hipGetLastError();
  hipLaunchKernelGGL(decode_spec_kernel, dim3(grid), dim3(kSpecWaves * 64), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}


extern "C" int ecco_decode_segmented(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride,
                                     uint64_t y_stride, const void* tables, float tensor_scale, uint16_t* y,
                                     uint32_t lanes_per_block, void* stream) {
  if (!blocks || !tables || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  if (lanes_per_block != 2 && lanes_per_block != 4 && lanes_per_block != 8) return ECCO_EINVAL;
  uint64_t total = 0;
  if (!group_count(n_rows, gpr, &total)) return ECCO_ESIZE;
  if (n_rows > 1 && (y_stride < gpr * 128 || blk_stride < gpr)) return ECCO_ESIZE;
  if (!host_aligned(y, 16) || (y_stride % 8) != 0 || !host_aligned(blocks, 64) || !host_aligned(tables, 256))
    return ECCO_EALIGN;
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  SpecArgs a;
  a.blocks = static_cast<const uint8_t*>(blocks);
  a.y = y;
  a.tab = static_cast<const Tables*>(tables);
  a.blk_stride = n_rows > 1 ? blk_stride : gpr;
  a.y_stride = n_rows > 1 ? y_stride : gpr * 128;
  a.gpr = make_magic((uint32_t)gpr);
  a.n_groups = (uint32_t)total;
  a.t = tensor_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // one workgroup per CU (the LDS holds one), each wave 64 / L blocks per pass
  auto launch = [&](auto kernel, uint64_t per_wg, int waves) {
    const uint64_t want = (total + per_wg - 1) / per_wg;
    const uint32_t grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)cus));
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(waves * 64), 0, s, a);
  };
  switch (lanes_per_block) {
    case 2: launch(decode_seg_kernel<2>, SegGeom<2>::kWaves * SegGeom<2>::kBlocks, SegGeom<2>::kWaves); break;
    case 4: launch(decode_seg_kernel<4>, SegGeom<4>::kWaves * SegGeom<4>::kBlocks, SegGeom<4>::kWaves); break;
    default: launch(decode_seg_kernel<8>, SegGeom<8>::kWaves * SegGeom<8>::kBlocks, SegGeom<8>::kWaves); break;
  }
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}
