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
//             decode leaves the segment at offset 0..7 of the next one
//   resolve   from offset 0 in segment 0, the chain of exit offsets picks each
//             segment's entry; a uniform loop over the 62 segments reads every
//             lane's 8-entry exit and count tables with readlane (the merge),
//             and the running count gives each lane its first output index
//   emit      each lane decodes its segment again from its true entry and
//             writes the symbols whose index is below 128; the 128th
//             codeword's end fixes the outlier-record count as in the format
// The rest (value table, records, FP16 store) is the format's dequantisation.
// Every block costs about 32 table look-ups per lane and a 62-step merge,
// against 2 look-ups per lane-block for the lane-serial decoder; the latter
// is the library's decoder because it does far less work per block.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ecco_device.h"

namespace ecco {

constexpr int kSpecWaves = 8;                     // waves (blocks in flight) per workgroup
constexpr int kSegments = (512 - 16) / 8;         // 62 segments of 8 stream bits

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
  for (uint32_t g = blockIdx.x * kSpecWaves + wave; g < a.n_groups; g += gridDim.x * kSpecWaves) {
    const uint32_t row = div_magic(g, a.gpr), col = g - row * a.gpr.d;
    if (lane < 16u) W[lane] = reinterpret_cast<const uint32_t*>(a.blocks + ((uint64_t)row * a.blk_stride + col) * 64u)[lane];
    else if (lane < 20u) W[lane] = 0u;
    if (lane < 36u) reinterpret_cast<uint32_t*>(sym)[lane] = 0x20202020u;   // entry 16: +0 past a clip
    wave_sync();
    const uint32_t head = W[0];
    const uint32_t lutb = ((head & 63u) * 4u + ((head >> 6) & 3u)) * 256u;
    // the two words holding bits seg0 .. seg0 + 15 of this lane's segment
    const uint32_t seg0 = 16u + 8u * min(lane, (uint32_t)kSegments - 1u), seg1 = seg0 + 8u;
    const uint32_t wlo = W[seg0 >> 5], whi = W[(seg0 >> 5) + 1u], wbase = seg0 & ~31u;
    const bool last = lane == (uint32_t)kSegments - 1u;
    // 1. speculative decode from each entry offset: exit offset and count
    uint32_t F = 0, C = 0;
#pragma unroll
    for (uint32_t o = 0; o < 8u; ++o) {
      uint32_t pos = seg0 + o, cnt = 0;
      bool go = true;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (go && pos < seg1) {
          const uint32_t e = sm.lut[lutb + (window(wlo, whi, pos - wbase) & 255u)];
          const uint32_t len = (e >> 5) + 1u;
          if (last && pos + len > 512u) {
            go = false;                            // the codeword does not fit: the stream is clipped
          } else {
            pos += len;
            ++cnt;
          }
        }
      }
      F |= ((pos - seg1) & 7u) << (3u * o);
      C |= cnt << (3u * o);
    }
    // 2. resolve: follow the exit offsets from offset 0 of segment 0
    uint32_t entry = 0, start = 0, my_entry = 0, my_start = 0, my_cnt = 0;
    for (uint32_t i = 0; i < (uint32_t)kSegments; ++i) {
      const uint32_t f = __builtin_amdgcn_readlane(F, i), c = __builtin_amdgcn_readlane(C, i);
      const uint32_t n_i = (c >> (3u * entry)) & 7u;
      if (lane == i) {
        my_entry = entry;
        my_start = start;
        my_cnt = n_i;
      }
      start += n_i;
      entry = (f >> (3u * entry)) & 7u;
    }
    const bool full = start >= 128u;               // 128 whole codewords fit: not clipped
    // 3. emit: decode the segment again from its true entry
    uint32_t end = 0;                               // stream end after codeword 128 (its lane only)
    if (lane < (uint32_t)kSegments) {
      uint32_t pos = seg0 + my_entry;
#pragma unroll
      for (uint32_t s = 0; s < 4u; ++s) {
        if (s < my_cnt) {
          const uint32_t e = sm.lut[lutb + (window(wlo, whi, pos - wbase) & 255u)];
          const uint32_t idx = my_start + s;
          pos += (e >> 5) + 1u;
          if (idx < 128u) sym[idx] = (uint8_t)((e & 31u) << 1);
          if (idx == 127u) end = pos;
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
  }
}

}  // namespace ecco

using namespace ecco;

extern "C" int ecco_decode_speculative(const void* blocks, uint64_t n_rows, uint64_t gpr, uint64_t blk_stride,
                                       uint64_t y_stride, const void* tables, float tensor_scale, uint16_t* y,
                                       void* stream) {
  if (!blocks || !tables || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  const uint64_t total = n_rows * gpr;
  if (n_rows == 0 || gpr == 0 || total >= (1ull << 32) || gpr >= (1ull << 32)) return ECCO_ESIZE;
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
