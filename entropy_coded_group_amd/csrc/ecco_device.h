// Device helpers and the block-decode core shared by the decode and fused
// decode+GEMV kernels of libecco (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include "ecco_internal.h"

namespace ecco {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Wave-level ordering of LDS traffic: all lanes of the wave reach this point
// and their earlier LDS writes are visible to later LDS reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// All-reduce over the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  v = max(v, dpp_u32<kRowHalfMirror>(v));
  v = max(v, dpp_u32<kRowMirror>(v));
  return v;
}
__device__ __forceinline__ uint32_t row_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kQuadXor1>(v));
  v = min(v, dpp_u32<kQuadXor2>(v));
  v = min(v, dpp_u32<kRowHalfMirror>(v));
  v = min(v, dpp_u32<kRowMirror>(v));
  return v;
}
__device__ __forceinline__ uint32_t row_add_u32(uint32_t v) {
  v += dpp_u32<kQuadXor1>(v);
  v += dpp_u32<kQuadXor2>(v);
  v += dpp_u32<kRowHalfMirror>(v);
  v += dpp_u32<kRowMirror>(v);
  return v;
}
__device__ __forceinline__ float row_min_f32(float v) {
  v = fminf(v, dpp_f32<kQuadXor1>(v));
  v = fminf(v, dpp_f32<kQuadXor2>(v));
  v = fminf(v, dpp_f32<kRowHalfMirror>(v));
  v = fminf(v, dpp_f32<kRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kRowMirror>(v));
  return v;
}
template <int CTRL>
__device__ __forceinline__ uint64_t min_u64_dpp(uint64_t v) {
  uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  uint64_t o = ((uint64_t)hi << 32) | lo;
  return o < v ? o : v;
}
__device__ __forceinline__ uint64_t row_min_u64(uint64_t v) {
  v = min_u64_dpp<kQuadXor1>(v);
  v = min_u64_dpp<kQuadXor2>(v);
  v = min_u64_dpp<kRowHalfMirror>(v);
  v = min_u64_dpp<kRowMirror>(v);
  return v;
}
// acc + sum of the products of 8 FP16 pairs, FP32 accumulation
// (v_dot2_f32_f16: two products summed into an FP32 accumulator).
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, x.w), acc, false);
  return acc;
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kQuadXor1>(v);
  v += dpp_f32<kQuadXor2>(v);
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kRowMirror>(v);
  return v;
}

// Sum over the whole wave, in a fixed order: rows first, then the four row
// totals read back in row order.  The result is uniform.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kQuadXor1>(v);
  v += dpp_f32<kQuadXor2>(v);
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kRowMirror>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kRowMirror>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// All-reduce over aligned segments of LPG = 16 lanes (a DPP row) or 8 lanes
// (half a row: the quad swaps and the half-row mirror stay inside it).
template <int LPG>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "segment of 4, 8 or 16 lanes");
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  if constexpr (LPG >= 8) v = max(v, dpp_u32<kRowHalfMirror>(v));
  if constexpr (LPG == 16) v = max(v, dpp_u32<kRowMirror>(v));
  return v;
}
template <int LPG>
__device__ __forceinline__ uint32_t seg_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kQuadXor1>(v));
  v = min(v, dpp_u32<kQuadXor2>(v));
  if constexpr (LPG >= 8) v = min(v, dpp_u32<kRowHalfMirror>(v));
  if constexpr (LPG == 16) v = min(v, dpp_u32<kRowMirror>(v));
  return v;
}
template <int LPG>
__device__ __forceinline__ uint32_t seg_add_u32(uint32_t v) {
  v += dpp_u32<kQuadXor1>(v);
  v += dpp_u32<kQuadXor2>(v);
  if constexpr (LPG >= 8) v += dpp_u32<kRowHalfMirror>(v);
  if constexpr (LPG == 16) v += dpp_u32<kRowMirror>(v);
  return v;
}
// Float min / max over a segment of non-NaN values.  Written with the DPP
// form of v_min_f32 / v_max_f32 directly: through fminf the compiler moves
// the neighbour's value and quiets it (a possible signalling NaN) before the
// min, three instructions a step instead of one.  Each step waits the two
// cycles a DPP read of a just-written register needs.
#define ECCO_DPP_STEP(op, ctrl) "s_nop 1\n\t" op " %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define ECCO_DPP_QX1 "quad_perm:[1,0,3,2]"
#define ECCO_DPP_QX2 "quad_perm:[2,3,0,1]"
#define ECCO_DPP_RHM "row_half_mirror"
#define ECCO_DPP_RM "row_mirror"
template <int LPG>
__device__ __forceinline__ float seg_min_f32(float v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "segment of 4, 8 or 16 lanes");
  if constexpr (LPG == 4)
    asm(ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX2) : "+v"(v));
  else if constexpr (LPG == 8)
    asm(ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX2)
        ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_RHM) : "+v"(v));
  else
    asm(ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_QX2)
        ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_RHM) ECCO_DPP_STEP("v_min_f32_dpp", ECCO_DPP_RM) : "+v"(v));
  return v;
}
template <int LPG>
__device__ __forceinline__ float seg_max_f32(float v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "segment of 4, 8 or 16 lanes");
  if constexpr (LPG == 4)
    asm(ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX2) : "+v"(v));
  else if constexpr (LPG == 8)
    asm(ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX2)
        ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_RHM) : "+v"(v));
  else
    asm(ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX1) ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_QX2)
        ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_RHM) ECCO_DPP_STEP("v_max_f32_dpp", ECCO_DPP_RM) : "+v"(v));
  return v;
}

// Inclusive prefix sum over the 16 lanes of a row (Hillis-Steele).
__device__ __forceinline__ uint32_t row_scan_add(uint32_t v) {
  v += dpp_u32<kRowShr1>(v);
  v += dpp_u32<kRowShr2>(v);
  v += dpp_u32<kRowShr4>(v);
  v += dpp_u32<kRowShr8>(v);
  return v;
}
// The same over aligned segments of LPG lanes; tl = lane index in the segment
// (a shifted-in value from the previous segment is dropped).
template <int LPG>
__device__ __forceinline__ uint32_t seg_scan_add(uint32_t v, uint32_t tl) {
  if constexpr (LPG == 16) {
    return row_scan_add(v);
  } else {
    uint32_t u = dpp_u32<kRowShr1>(v);
    v += tl >= 1u ? u : 0u;
    u = dpp_u32<kRowShr2>(v);
    v += tl >= 2u ? u : 0u;
    if constexpr (LPG == 8) {
      u = dpp_u32<kRowShr4>(v);
      v += tl >= 4u ? u : 0u;
    }
    return v;
  }
}

// OCP FP8 E4M3FN encode of a non-NaN float: saturate to +-448, round to
// nearest even (the subnormal grid is 2^-9).  gfx950's v_cvt_pk_fp8_f32
// converts to that format with round-to-nearest-even; the clamp first makes
// out-of-range values saturate.  (Checked against a bit-level software
// encoder over every non-NaN binary32 input.)
__device__ __forceinline__ uint32_t fp8_encode(float v) {
  const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}

// OCP FP8 E4M3FN decode of byte B of x (exact; 0x7F / 0xFF give NaN) with
// gfx950's v_cvt_f32_fp8, which implements that format.
template <int B>
__device__ __forceinline__ float fp8_decode(uint32_t x) {
  return __builtin_amdgcn_cvt_f32_fp8((int)x, B);
}

// FP16 <-> FP32 through the native half type: v_cvt_f16_f32 rounds to nearest
// even, v_cvt_f32_f16 is exact.
// The empty asm pins v as a rounded binary32 value: without it the compiler
// may fuse a preceding multiply into v_fma_mixlo_f16, which rounds the exact
// product to FP16 once instead of rounding to FP32 first as the format defines.
__device__ __forceinline__ uint32_t f16_bits(float v) {
  asm volatile("" : "+v"(v));
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ float f16_value(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Streaming (non-temporal) 16-byte global accesses: decoded rows and
// compressed blocks are touched once, and marking them so keeps them from
// displacing cached lines; for a stream that is 80 % writes this matters
// more than anything else in the memory system.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

// Index of the job whose workgroup range holds workgroup w: the number of
// jobs after the first whose range starts at or before w (the ranges are in
// order).  Every job's first workgroup is read at once, so the search waits
// for one scalar load instead of one per job passed.
template <int MAXJ, class Args>
__device__ __forceinline__ uint32_t find_job(const Args& args, uint32_t w) {
  uint32_t j = 0;
#pragma unroll
  for (int k = 1; k < MAXJ; ++k) j += ((uint32_t)k < args.n_jobs && w >= args.job[k].wg_first) ? 1u : 0u;
  return __builtin_amdgcn_readfirstlane(j);      // uniform: the job descriptor stays in scalar registers
}

// 64-bit window shift: bits [r, r + 32) of hi:lo, r < 64.
__device__ __forceinline__ uint32_t window(uint32_t lo, uint32_t hi, uint32_t r) {
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> r);
}

// Row / column of a linear group index by a precomputed reciprocal
// (n / d = (n + umulhi(n, m)) >> s, exact for every 32-bit n).
struct DivMagic {
  uint32_t d, m, s;
};
inline __host__ DivMagic make_magic(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t M = ((1ull << (32 + s)) / d) + 1;     // in (2^32, 2^33]
  return DivMagic{d, (uint32_t)(M - (1ull << 32)), s};
}
__device__ __forceinline__ uint32_t div_magic(uint32_t n, DivMagic q) {
  return (uint32_t)(((uint64_t)n + __umulhi(n, q.m)) >> q.s);
}


// ------------------------------------------------------------- decode core
//
// A wavefront decodes batches of up to 64 blocks.  The look-up tables live in
// LDS for the whole workgroup; each wave has a private staging area:
//   blk   64 x 17 dwords: the batch's blocks; after a lane has decoded its
//         block, the block's 32-entry FP16 value table overwrites its words
//   qsym  16 x 36 dwords: the symbol bytes of 16 blocks at a time (128 per
//         block, or 64 in a row of 20 dwords for 64-value groups)

constexpr int kDecWaves = 12;                    // decode kernel: waves per workgroup (one workgroup per CU)
constexpr int kGemvWaves = 12;                   // fused decode+GEMV: waves per workgroup
constexpr int kBlkStride = 17;                   // dwords per staged block: 16 + 1 pad (column reads spread over banks)
constexpr int kBlkWords = 64 * kBlkStride + 48;  // slack for reads past the last block
constexpr int kDeadLut = S * H * 256;            // byte offset of the all-"clipped" look-up table
constexpr int kSymStride = 36;                   // dwords per staged symbol row: 32 + 4 pad, keeps 16-byte
                                                 // row writes of several lanes off a single group of banks
constexpr int kPassBlocks = 16;                  // blocks whose symbols are staged at a time
constexpr int kPasses = 64 / kPassBlocks;

// Geometry of a group size: 128 values (weights, KV cache: 15-bit outlier
// records with a 7-bit position) or 64 (activations: 14-bit records, 6-bit
// position).  Eight values per lane in the transposed step, so a block's
// output row takes GS / 8 lanes.
template <int GS>
struct GroupGeom {
  static_assert(GS == 128 || GS == 64, "group of 128 or 64 values");
  static constexpr uint32_t kPosBits = GS == 128 ? 7 : 6;
  static constexpr uint32_t kRecBits = kPosBits + 8;
  static constexpr int kChunks = GS / 4;                     // 4-codeword refill steps per block
  static constexpr int kSymStride = GS == 128 ? 36 : 20;     // dwords per staged symbol row (GS bytes + 16 pad bytes + pad)
  static constexpr int kLanesPerBlock = GS / 8;
  static constexpr int kBlocksPerIter = 64 / kLanesPerBlock;
  static constexpr int kPassIters = kPassBlocks / kBlocksPerIter;
};

template <int NW>
struct DecodeSmem {
  alignas(16) uint8_t lut[S * H * 256 + 256];   // decode look-up tables + the clipped-stream table
  alignas(16) float cent[S * 16];
  alignas(16) uint32_t blk[NW][kBlkWords];
  uint32_t qsym[NW][kPassBlocks * kSymStride];
};

// The look-up tables' global loads of the full rounds are issued before the
// first LDS write, so their latencies overlap instead of adding up one loop
// trip at a time (NW * 64 threads at most, so each full round stays in
// bounds; the remainder loop covers the rest at any workgroup size).
template <int NW>
__device__ __forceinline__ void stage_decode_tables(DecodeSmem<NW>& sm, const Tables* tab) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  constexpr uint32_t NL = S * H * 256 / 16;                  // 16-byte pieces of the look-up tables
  constexpr uint32_t IT = NL / (NW * 64);                    // full rounds
  const uint4* src = reinterpret_cast<const uint4*>(&tab->lut[0][0][0]);
  uint4* dst = reinterpret_cast<uint4*>(sm.lut);
  uint4 v[IT];
#pragma unroll
  for (uint32_t k = 0; k < IT; ++k) v[k] = src[tid + k * nt];
  for (uint32_t i = tid + IT * nt; i < NL; i += nt) dst[i] = src[i];
  const uint4* csrc = reinterpret_cast<const uint4*>(&tab->centroids[0][0]);
  for (uint32_t i = tid; i < S * 16 / 4; i += nt) reinterpret_cast<uint4*>(sm.cent)[i] = csrc[i];
  // a clipped stream reads as symbol 16 ("+0" in a clipped block), one bit per step
  if (tid < 16) dst[NL + tid] = make_uint4(0x10101010u, 0x10101010u, 0x10101010u, 0x10101010u);
  uint4* blk = reinterpret_cast<uint4*>(&sm.blk[0][0]);
  for (uint32_t i = tid; i < NW * kBlkWords / 4; i += nt) blk[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (uint32_t k = 0; k < IT; ++k) dst[tid + k * nt] = v[k];
}

// The 64 blocks of a batch as four 16-byte chunks per lane: chunk i of lane l
// is bytes 16 (l & 3) .. + 15 of block l / 4 + 16 i (coalesced when the
// blocks are contiguous).  Issued early so the loads overlap the previous
// batch's decode.
struct BatchRegs {
  uint4 v[4];
};

// Blocks past n_valid read the last valid block instead (their output is
// never stored), so the loads are unconditional: a conditional load would
// make the compiler wait for it at once instead of letting it overlap.
template <class Load>
__device__ __forceinline__ BatchRegs fetch_batch(uint32_t lane, uint32_t n_valid, Load load) {
  BatchRegs r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (lane >> 2) + 16u * i;
    r.v[i] = load(min(b, n_valid - 1u), lane & 3u);
  }
  return r;
}

// The default pass prologue of decode_batch: nothing to load.
struct NoPrologue {
  __device__ void operator()(uint32_t) const {}
};

// Decode one staged batch of GS-value blocks (FULL: all 64 blocks exist, so
// no store is predicated).
//   pre(k)                    called as write-out pass k (0..3) starts, before
//                             its LDS work: a sink that needs other data for
//                             the pass (the GEMV's x) loads it here
//   sink(b, j0, v, k, it)     8 decoded FP16 values of block b at positions
//                             j0 .. j0 + 7 (v.x holds values j0, j0 + 1, ...),
//                             in iteration it of pass k
// Steps: stage the batch in LDS; each lane decodes one block's codeword
// stream with the 8-bit-window look-up table, four codewords per bit-window
// refill, and marks a clipped stream; builds the block's value table (15
// centroids * a, the scale S, up to 16 outlier values, or +0 for a clipped
// block); then, 16 blocks at a time, stages the symbol bytes -- each as the
// byte offset of its value-table entry, outlier positions overwritten by that
// of entry 16 + r -- and hands 8 values per lane to the sink,
// GS / 8 lanes per block, so every store instruction writes whole rows (four
// of 256 bytes, or eight of 128).
// STOP adds the stop at a window that no codeword starts, which only tables
// with an incomplete codebook have (kLutNoCode entries); complete tables run
// the instance without it.
// PRIO sets the wave's issue priority by step: the staging and the
// lane-serial chain, a dependent series of LDS look-ups that bounds the
// batch's latency, go first; the write-out passes next; the value-table work
// last.  (The decode gains 6-8 % from it and the attention kernels 5 %;
// the GEMV does not.)
template <bool FULL, int NW, int GS = 128, bool PRIO = false, bool STOP = false, class Sink, class Pre = NoPrologue>
__device__ __forceinline__ void decode_batch(DecodeSmem<NW>& sm, uint32_t wave, uint32_t lane, uint32_t n_valid,
                                             float t, const BatchRegs& in, Sink sink, Pre pre = Pre{}) {
  using Geo = GroupGeom<GS>;
  constexpr uint32_t RB = Geo::kRecBits;
  constexpr int SST = Geo::kSymStride;
  constexpr int LPB = Geo::kLanesPerBlock;
  constexpr int BPI = Geo::kBlocksPerIter;
  uint32_t* blk = sm.blk[wave];
  uint32_t* qs = sm.qsym[wave];
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t* d = blk + ((lane >> 2) + 16u * i) * kBlkStride + 4u * (lane & 3u);
    d[0] = in.v[i].x;
    d[1] = in.v[i].y;
    d[2] = in.v[i].z;
    d[3] = in.v[i].w;
  }
  wave_sync();

  // 1. lane-serial decode of block `lane`
  uint32_t* W = blk + lane * kBlkStride;
  uint32_t lo = W[0], hi = W[1];
  const uint32_t head = lo;
  uint32_t lutb = ((head & 63u) * 4u + ((head >> 6) & 3u)) * 256u;   // lut[p][h]
  uint32_t r = 16, kw = 2, lim = 512;
  uint32_t E[Geo::kChunks];
#pragma unroll
  for (int c = 0; c < Geo::kChunks; ++c) {
    const uint32_t nxt = W[kw];
    const uint32_t base = (kw - 2u) * 32u;
    uint32_t x = window(lo, hi, r);
    const uint32_t e0 = sm.lut[lutb + (x & 255u)];
    const uint32_t r1 = r + (e0 >> 5) + 1u;
    x = window(lo, hi, r1);
    const uint32_t e1 = sm.lut[lutb + (x & 255u)];
    const uint32_t r2 = r1 + (e1 >> 5) + 1u;
    x = window(lo, hi, r2);
    const uint32_t e2 = sm.lut[lutb + (x & 255u)];
    const uint32_t r3 = r2 + (e2 >> 5) + 1u;
    x = window(lo, hi, r3);
    const uint32_t e3 = sm.lut[lutb + (x & 255u)];
    const uint32_t r4 = r3 + (e3 >> 5) + 1u;
    // the four entries' low bytes, packed by three byte permutes
    uint32_t ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(e3, e2, 0x0c0c0400u),
                                        __builtin_amdgcn_perm(e1, e0, 0x0c0c0400u), 0x05040100u);
    asm volatile("" : "+v"(ev));                 // pack now: keeps one register per 4 symbols
    // The stream stops in this chunk if a codeword of it ends past bit 512
    // (clipped) or, with STOP (tables with an incomplete codebook), a window
    // has no codeword: the kLutNoCode entry, the only one with bit 4 set
    // while the stream is live (~lim masks the test off once it stopped).
    if (base + r4 > lim || (STOP && (ev & ~lim & 0x10101010u) != 0u)) {
      // The codewords read are a prefix of f: the ends rise, so those that
      // fit come first (8 f counted by inline constants: the byte masks, as
      // literals, took four registers of the whole kernel), and none is
      // read from the first window without a codeword on.  The bytes from f
      // on become 16.
      uint32_t f8 = (base + r1 <= 512u ? 8u : 0u) + (base + r2 <= 512u ? 8u : 0u) + (base + r3 <= 512u ? 8u : 0u);
      if constexpr (STOP) {
        const uint32_t nc = ev & 0x10101010u;    // bit 8 i + 4: codeword i's window has no codeword
        f8 = min(f8 + (base + r4 <= 512u ? 8u : 0u), nc ? ((uint32_t)__builtin_ctz(nc) & 0x38u) : 32u);
      }
      const uint32_t m = 0xffffffffu << f8;
      ev = (ev & ~m) | (0x10101010u & m);
      lim = 0xffffffffu;
      lutb = kDeadLut;
    }
    E[c] = (ev & 0x1f1f1f1fu) << 1;             // symbol -> byte offset of its FP16 value-table entry
    const bool adv = r4 >= 32u;
    lo = adv ? hi : lo;
    hi = adv ? nxt : hi;
    r = r4 & 31u;
    kw += adv ? 1u : 0u;
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  const bool full = lim == 512u;
  const uint32_t end = (kw - 2u) * 32u + r;
  const uint32_t n = full ? min(16u, (512u - end) / RB) : 0u;

  // 2. value table: [0..14] fp16(c * a), [15] fp16(S), [16 + r] outlier r (or +0 if clipped)
  const uint32_t p = head & 63u;
  const float S = fp8_decode<1>(head) * t;
  const float aa = fabsf(S);
  uint32_t vtab[16];
  {
    const float* cp = sm.cent + p * 16u;
#pragma unroll
    for (int s = 0; s < 15; s += 2) {
      const float v0 = cp[s] * aa;
      const float v1 = s + 1 < 15 ? cp[s + 1] * aa : S;
      vtab[s / 2] = f16_bits(v0) | (f16_bits(v1) << 16);
    }
  }
  // all 16 record slots at once (records sit in words 8..15 at fixed places);
  // slots r >= n are dropped
  uint32_t tail[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) tail[i] = W[8 + i];
  // jp: byte r of jp[r / 4] is the symbol-row byte that slot r patches: the
  // record's position, or a pad byte past the row's GS symbols if r >= n
  uint32_t jp[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 8; i < 16; ++i) vtab[i] = 0;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    if ((rr & 3) == 0 && !__any((uint32_t)rr < n)) break;
    const uint32_t pos = 512u - RB * (rr + 1);
    const uint32_t wi = (pos >> 5) - 8u, sh = pos & 31u;
    const uint32_t rec = window(tail[wi], tail[wi + 1], sh) & ((1u << RB) - 1u);
    const uint32_t hv = f16_bits(fp8_decode<0>(rec >> Geo::kPosBits) * t);
    const bool use = (uint32_t)rr < n;
    vtab[8 + rr / 2] |= (use ? hv : 0u) << (16 * (rr & 1));
    jp[rr / 4] |= (use ? (rec & (GS - 1u)) : GS + (uint32_t)rr) << (8 * (rr & 3));
  }
  // the block's words are consumed: its value table takes their place
#pragma unroll
  for (int i = 0; i < 16; ++i) W[i] = vtab[i];

  if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
  // 3. passes of kPassBlocks blocks
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    pre((uint32_t)k);
    if (lane / kPassBlocks == (uint32_t)k) {
      uint32_t* Q = qs + (lane % kPassBlocks) * SST;
#pragma unroll
      for (int i = 0; i < Geo::kChunks; i += 4)
        *reinterpret_cast<uint4*>(Q + i) = make_uint4(E[i], E[i + 1], E[i + 2], E[i + 3]);
      // outlier positions take value-table entry 16 + r, in record order so
      // that a later record wins a repeated position
      uint8_t* Qb = reinterpret_cast<uint8_t*>(Q);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        if ((rr & 3) == 0 && !__any((uint32_t)rr < n)) break;
        Qb[(jp[rr / 4] >> (8 * (rr & 3))) & 0xffu] = (uint8_t)(2 * (16 + rr));
      }
    }
    wave_sync();
    uint2 sv[Geo::kPassIters];
#pragma unroll
    for (int it = 0; it < Geo::kPassIters; ++it)
      sv[it] = *reinterpret_cast<const uint2*>(qs + (it * BPI + lane / LPB) * SST + 2u * (lane % LPB));
    uint4 o[Geo::kPassIters];
#pragma unroll
    for (int it = 0; it < Geo::kPassIters; ++it) {
      // the block's value table: this lane's row base plus a constant
      // (k, it) offset, which goes last so that the look-up instruction's
      // offset field takes it (a per-step address per lane cost registers)
      const uint8_t* tb = reinterpret_cast<const uint8_t*>(blk + (lane / LPB) * kBlkStride);
      const uint32_t off = (kPassBlocks * (uint32_t)k + (uint32_t)(it * BPI)) * kBlkStride * 4u;
      // each staged byte is already the entry's byte offset (< 64)
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      auto v = [&](uint32_t s, int b) -> _Float16 {
        return *reinterpret_cast<const _Float16*>(tb + ((s >> (8 * b)) & 0xffu) + off);
      };
      auto pr = [&](uint32_t s, int b) -> uint32_t {
        h2 q;
        q.x = v(s, b);
        q.y = v(s, b + 1);
        return __builtin_bit_cast(uint32_t, q);
      };
      const uint32_t s0 = sv[it].x, s1 = sv[it].y;
      o[it].x = pr(s0, 0);
      o[it].y = pr(s0, 2);
      o[it].z = pr(s1, 0);
      o[it].w = pr(s1, 2);
    }
    wave_sync();
#pragma unroll
    for (int it = 0; it < Geo::kPassIters; ++it) {
      const uint32_t bl = kPassBlocks * k + it * BPI + lane / LPB;
      if (FULL || bl < n_valid) sink(bl, 8u * (lane % LPB), o[it], (uint32_t)k, (uint32_t)it);
    }
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

}  // namespace ecco
