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
    const bool full = start >= 128u;               // 128 whole codewords fit: not clipped
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
    const uint32_t E = has_end ? __builtin_amdgcn_readlane(end, (int)__builtin_ctzll(has_end)) : 0u;
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
