// Decode-phase attention over Ecco-compressed K and V caches, for gfx950.
//
// The pages' online codec compresses the KV cache so that each decoding step
// reads a quarter of the bytes (Ecco review, "Core claim"; KV-cache
// compression with the min/max pattern choice).  Here the blocks are decoded
// inside the attention kernels themselves, so the FP16 cache is never written:
//
//   scores   one wave per 64 tokens of one (sequence, kv head): the shared
//            decode core hands each lane 8 values of one token's K row;
//            v_dot2_f32_f16 against the G query heads' matching 8 values, a
//            DPP row sum over the token's 16 lanes, times scale * log2(e)
//            -> s[pair][t][g] (scores in base-2 units), and each head's
//            largest score of the 64 tokens -> bmax[pair][t / 64][g]
//   p . V    one wave per 128 tokens (a unit) of one pair: with m the unit's
//            largest score (of its two bmax entries), p_t = 2^(s_t - m)
//            times the decoded V values, FP32 accumulators for the G heads
//            and the lane's 8 positions, a cross-row reduction; the unit's
//            partial sums, m and z = sum of its p_t
//   combine  per output row: M = the largest unit m, then the units' partial
//            sums and z, each weighted by 2^(m - M), added in unit order;
//            out = sum / z (the softmax normalisation, applied once)
//
// Every sum is taken in a fixed order, so results do not depend on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "ecco_device.h"

namespace ecco {

constexpr uint32_t kUnitTokens = 128;   // tokens per p . V work unit (two batches)
// waves per workgroup of the scores kernel: three per SIMD; at G = 8 the
// eight scores per token need more registers than that leaves, so two
template <int G>
constexpr int score_waves() { return G > 4 ? 8 : 12; }
constexpr int kPvWaves = 12;            // waves per workgroup of the p . V kernel

// DPP row rotations (GFX9 encoding)
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

struct AttnArgs {
  const uint8_t* kb;
  const uint8_t* vb;
  const Tables* kt;
  const Tables* vt;
  const uint16_t* q;
  float* probs;          // [pairs][S][G] scores, base-2 units
  float* part;           // [pairs][n_units][G][128] unnormalised partial sums
  float* bmax;           // [pairs][n_kb][G] largest score of each 64-token batch
  float* mz;             // [pairs][n_units][G] (m, z) of each unit
  float* out;            // [pairs * G][128]
  uint32_t pairs, S, stride, n_kb, n_units, G;
  float kts, vts, scale;
};

// The 64 blocks of batch t0 .. t0 + 63 of one pair (clamped at S); with
// live == false the cached table blob is read instead (a prefetch past the
// end that must stay unconditional).
// The lane index goes through an opaque copy, so that the four block
// indices (lane / 4 + 16 i) are computed at each fetch rather than kept in
// registers across the batch (the score kernel spilled them).
__device__ __forceinline__ BatchRegs fetch_tokens(uint32_t lane, const uint8_t* rows, const uint8_t* idle,
                                                  uint32_t n_valid, bool live) {
  asm volatile("" : "+v"(lane));
  return fetch_batch(lane, n_valid, [&](uint32_t i, uint32_t q) {
    return load_stream((live ? rows + (uint64_t)i * 64u : idle + 64u * (i & 63u)) + 16u * q);
  });
}

// The scores kernel's work; STOP: the decode core's instance for tables
// with an incomplete codebook.
template <int G, bool STOP>
__device__ __forceinline__ void attn_scores_body(const AttnArgs& a, DecodeSmem<score_waves<G>()>& sm) {
  constexpr int kScoreWaves = score_waves<G>();
  // the wave index is uniform: held in a scalar register, so are the batch
  // counters and the addresses derived from them
  const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t total = a.pairs * a.n_kb;
  const uint32_t stride = gridDim.x * kScoreWaves;
  const uint8_t* idle = reinterpret_cast<const uint8_t*>(a.kt);
  uint32_t batch = wave * gridDim.x + blockIdx.x;   // batches go round the CUs first
  if (batch >= total) return;
  auto fetch = [&](uint32_t bt, bool live) {
    const uint32_t pair = bt / a.n_kb, t0 = (bt % a.n_kb) * 64u;
    return fetch_tokens(lane, a.kb + ((uint64_t)pair * a.stride + t0) * 64u, idle, min(64u, a.S - t0), live);
  };
  BatchRegs cur = fetch(batch, true);
  const uint32_t j0 = 8u * (lane & 15u);
  for (; batch < total; batch += stride) {
    const uint32_t nb = batch + stride;
    const bool more = nb < total;
    const BatchRegs nxt = fetch(more ? nb : batch, more);
    const uint32_t pair = batch / a.n_kb, t0 = (batch % a.n_kb) * 64u;
    const uint32_t n_valid = min(64u, a.S - t0);
    // The G query slices (8 values each) are loaded as each write-out pass
    // starts, from an opaque copy of their address: held across the whole
    // batch (the lane-serial chain included), they made the kernel spill.
    // A load under a run-time condition is not moved earlier than written.
    const uint16_t* qb = a.q + (uint64_t)pair * G * 128u;
    uint4 qv[G];
    auto load_q = [&]() {
      const uint16_t* qp = qb;
      asm volatile("" : "+s"(qp));
      if (n_valid != 0u) {
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g] = *reinterpret_cast<const uint4*>(qp + (uint32_t)g * 128u + j0);
      }
    };
    auto pre = [&](uint32_t) { load_q(); };
    // this lane's token's scores within a write-out step; step (k, it) adds
    // 16 k + 4 it tokens, a constant that the store's offset field takes
    // (written as one 64-bit product, the 16 offsets were kept in registers)
    float* sp = a.probs + ((uint64_t)pair * a.S + t0 + lane / 16u) * G;
    // the largest score of head lane % G over the tokens this lane sees
    // (every lane of a row holds all G scores of the row's token; one
    // register instead of G)
    float mloc = -__builtin_inff();
    auto sink = [&](uint32_t b, uint32_t, uint4 w, uint32_t, uint32_t) {
      float d[G];
#pragma unroll
      for (int g = 0; g < G; ++g) d[g] = row_sum_f32(dot8(w, qv[g], 0.0f)) * a.scale;
      float mine = d[0];
#pragma unroll
      for (int g = 1; g < G; ++g) mine = (lane & (G - 1u)) == (uint32_t)g ? d[g] : mine;
      mloc = fmaxf(mloc, mine);
      // one vector store of the token's G scores (whole 16-byte pieces, so the
      // four tokens of an instruction fill their 64 bytes without partial writes)
      if ((lane & 15u) == 0) {
        float* dst = sp + (b - lane / 16u) * G;
        if constexpr (G == 1) {
          dst[0] = d[0];
        } else if constexpr (G == 2) {
          *reinterpret_cast<float2*>(dst) = make_float2(d[0], d[1]);
        } else {
#pragma unroll
          for (int g = 0; g < G; g += 4)
            *reinterpret_cast<float4*>(dst + g) = make_float4(d[g], d[g + 1], d[g + 2], d[g + 3]);
        }
      }
    };
    if (n_valid == 64u)
      decode_batch<true, kScoreWaves, 128, true, STOP>(sm, wave, lane, 64u, a.kts, cur, sink, pre);
    else
      decode_batch<false, kScoreWaves, 128, true, STOP>(sm, wave, lane, n_valid, a.kts, cur, sink, pre);
    // the batch's largest score per head: rotations of each row by G, 2G,
    // ... keep a lane's residue mod G, so lane g of every row ends with its
    // row's maximum of head g (a lane that saw no token holds -inf); then
    // the four rows' values of each head, read out as scalars
    if constexpr (G < 2) mloc = fmaxf(mloc, dpp_f32<kRowRor1>(mloc));
    if constexpr (G < 4) mloc = fmaxf(mloc, dpp_f32<kRowRor2>(mloc));
    if constexpr (G < 8) mloc = fmaxf(mloc, dpp_f32<kRowRor4>(mloc));
    mloc = fmaxf(mloc, dpp_f32<kRowRor8>(mloc));
    float bm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      auto rd = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mloc), l)); };
      bm[g] = fmaxf(fmaxf(rd(g), rd(16 + g)), fmaxf(rd(32 + g), rd(48 + g)));
    }
    if (lane == 0u) {
#pragma unroll
      for (int g = 0; g < G; ++g) a.bmax[(uint64_t)batch * G + g] = bm[g];
    }
    cur = nxt;
  }
}

template <int G>
__global__ __launch_bounds__(score_waves<G>() * 64) void attn_scores_kernel(AttnArgs a) {
  __shared__ DecodeSmem<score_waves<G>()> sm;
  stage_decode_tables(sm, a.kt);
  __syncthreads();
  if (a.kt->complete)
    attn_scores_body<G, false>(a, sm);
  else
    attn_scores_body<G, true>(a, sm);
}

// p . V for heads g_off .. g_off + GH - 1 of G.
// The value kernel's work; STOP as for the scores.
template <int GH, bool STOP>
__device__ __forceinline__ void attn_pv_body(const AttnArgs& a, uint32_t g_off, DecodeSmem<kPvWaves>& sm) {
  // the wave index is uniform: held in a scalar register, so are the batch
  // counters and the addresses derived from them
  const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t total = a.pairs * a.n_units;
  const uint32_t stride = gridDim.x * kPvWaves;
  const uint8_t* idle = reinterpret_cast<const uint8_t*>(a.vt);
  uint32_t unit = wave * gridDim.x + blockIdx.x;
  if (unit >= total) return;
  // the wave's batches: two per unit (the second empty past S)
  auto fetch = [&](uint32_t un, uint32_t half, bool live) {
    const uint32_t pair = un / a.n_units, t0 = (un % a.n_units) * kUnitTokens + 64u * half;
    const uint32_t nv = t0 < a.S ? min(64u, a.S - t0) : 0u;
    return fetch_tokens(lane, a.vb + ((uint64_t)pair * a.stride + min(t0, a.S - 1u)) * 64u, idle, max(nv, 1u),
                        live && nv > 0u);
  };
  BatchRegs cur = fetch(unit, 0, true);
  const uint32_t j0 = 8u * (lane & 15u);
  float acc[GH][8], z[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    z[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  }
  // slots (unit, half) in order; a unit's sums are flushed after its second half
  for (uint32_t half = 0; unit < total;) {
    const uint32_t pair = unit / a.n_units, u = unit % a.n_units;
    const uint32_t nu = unit + stride;
    // the unit's largest score per head: the larger of its batches' maxima
    // (the second batch only if the unit reaches past 64 tokens)
    float m[GH];
    {
      const float* bm = a.bmax + ((uint64_t)pair * a.n_kb + 2u * u) * a.G + g_off;
      const bool two = u * kUnitTokens + 64u < a.S;
#pragma unroll
      for (int g = 0; g < GH; ++g) m[g] = two ? fmaxf(bm[g], bm[a.G + g]) : bm[g];
    }
    const BatchRegs nxt = half == 0u ? fetch(unit, 1, true) : fetch(nu < total ? nu : unit, 0, nu < total);
    const uint32_t t0 = u * kUnitTokens + 64u * half;
    if (t0 < a.S) {
      const uint32_t n_valid = min(64u, a.S - t0);
      // the weights p = 2^(s - m) of a pass's four tokens per lane, their
      // scores loaded as the pass starts (from an opaque copy of the address,
      // under a run-time condition, so the loads are neither hoisted to the
      // batch's start nor held across the decode).  Step (k, it) takes token 16 k + 4 it +
      // lane / 16; tl is an opaque copy of lane / 16, so that the compiler
      // does not keep the 16 token indices of a batch in registers; a token
      // past n_valid reads token 0 (its products are never used).
      const float* pb = a.probs + ((uint64_t)pair * a.S + t0) * a.G + g_off;
      uint32_t tl = lane / 16u;
      asm volatile("" : "+v"(tl));
      const float* pl = pb + tl * a.G;
      float pq[4][GH];
      auto pre = [&](uint32_t k) {
        const float* pp = pl;
        asm volatile("" : "+v"(pp));
        if (n_valid != 0u) {
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int c = (int)(16u * k) + 4 * it;
            const float* src = (int)tl < (int)n_valid - c ? pp + (uint32_t)c * a.G : pb;
#pragma unroll
            for (int g = 0; g < GH; ++g) pq[it][g] = __builtin_amdgcn_exp2f(src[g] - m[g]);
          }
        }
      };
      auto sink = [&](uint32_t, uint32_t, uint4 w, uint32_t, uint32_t it) {
        float p[GH];
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          p[g] = pq[it][g];
          z[g] += p[g];
        }
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = f16_value((wv[i / 2] >> (16 * (i & 1))) & 0xffffu);
#pragma unroll
          for (int g = 0; g < GH; ++g) acc[g][i] = fmaf(p[g], v, acc[g][i]);
        }
      };
      // one instantiation of the decode core (with a second one for whole
      // batches, the accumulators were copied between the two and spilled)
      decode_batch<false, kPvWaves, 128, true, STOP>(sm, wave, lane, n_valid, a.vts, cur, sink, pre);
    }
    cur = nxt;
    if (half == 1u) {
      // lanes l, l + 16, l + 32, l + 48 hold the same positions of different tokens
#pragma unroll
      for (int g = 0; g < GH; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v = acc[g][i];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          acc[g][i] = v;
        }
      // the lanes of a row summed the same tokens' weights: add the rows
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        z[g] += __shfl_xor(z[g], 16);
        z[g] += __shfl_xor(z[g], 32);
      }
      if (lane < 16u) {
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float* dst = a.part + (((uint64_t)pair * a.n_units + u) * a.G + g_off + g) * 128u + j0;
          *reinterpret_cast<float4*>(dst) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
      }
      if (lane == 0u) {
#pragma unroll
        for (int g = 0; g < GH; ++g)
          *reinterpret_cast<float2*>(a.mz + (((uint64_t)pair * a.n_units + u) * a.G + g_off + g) * 2u) =
              make_float2(m[g], z[g]);
      }
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        z[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
      }
      unit = nu;
      half = 0;
    } else {
      half = 1;
    }
  }
}

template <int GH>
__global__ __launch_bounds__(kPvWaves * 64) void attn_pv_kernel(AttnArgs a, uint32_t g_off) {
  __shared__ DecodeSmem<kPvWaves> sm;
  stage_decode_tables(sm, a.vt);
  __syncthreads();
  if (a.vt->complete)
    attn_pv_body<GH, false>(a, g_off, sm);
  else
    attn_pv_body<GH, true>(a, g_off, sm);
}

// out[pair * G + g][d]: with M the largest of the units' maxima m_u, the
// units' partial sums and weight sums z_u, each times 2^(m_u - M), summed;
// then the partial-sum total over the z total.  One workgroup per output
// row: thread t adds units t / 32, t / 32 + 8, ... (in that order) for the
// four values 4 (t % 32) .. + 3 with 16-byte loads, and one pass over the
// eight threads' sums (in order) finishes the row; so the order of the
// additions is fixed.
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  __shared__ float4 red[kCombineThreads / 32][32];
  __shared__ float zred[kCombineThreads / 32];
  __shared__ float mred[kCombineThreads / 64];
  const uint32_t row = blockIdx.x;        // < pairs * G
  const uint32_t pair = row / a.G, g = row % a.G;
  const uint32_t t = threadIdx.x, q = t & 31u, ug = t >> 5;
  const uint64_t base = (uint64_t)pair * a.n_units * a.G + g;     // unit 0's (pair, g) entry
  const float2* mz = reinterpret_cast<const float2*>(a.mz) + base;
  // M: each thread's units t, t + 256, ..., then a butterfly over the wave
  // and the waves' maxima (max is exact, so its order does not matter)
  float M = -__builtin_inff();
  for (uint32_t u = t; u < a.n_units; u += kCombineThreads) M = fmaxf(M, mz[(uint64_t)u * a.G].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((t & 63u) == 0) mred[t >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) M = fmaxf(M, mred[i]);
  const float4* src = reinterpret_cast<const float4*>(a.part + base * 128u) + q;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float zt = 0.0f;
#pragma unroll 4
  for (uint32_t u = ug; u < a.n_units; u += kCombineThreads / 32) {
    const float2 e = mz[(uint64_t)u * a.G];
    const float w = __builtin_amdgcn_exp2f(e.x - M);
    const float4 v = src[(uint64_t)u * a.G * 32u];
    acc.x += v.x * w;
    acc.y += v.y * w;
    acc.z += v.z * w;
    acc.w += v.w * w;
    zt += e.y * w;
  }
  red[ug][q] = acc;
  if (q == 0) zred[ug] = zt;
  __syncthreads();
  if (t < 32) {
    float4 s4 = red[0][t];
    float z = zred[0];
#pragma unroll
    for (int i = 1; i < kCombineThreads / 32; ++i) {
      const float4 r = red[i][t];
      s4.x += r.x;
      s4.y += r.y;
      s4.z += r.z;
      s4.w += r.w;
      z += zred[i];
    }
    reinterpret_cast<float4*>(a.out + (uint64_t)row * 128u)[t] = make_float4(s4.x / z, s4.y / z, s4.z / z, s4.w / z);
  }
}

}  // namespace ecco

using namespace ecco;

namespace {
constexpr uint64_t kWsAlign = 256;
uint64_t round_up(uint64_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
uint64_t probs_bytes(uint64_t pairs, uint64_t g, uint64_t s) { return round_up(pairs * s * g * 4u); }
uint64_t bmax_bytes(uint64_t pairs, uint64_t g, uint64_t s) { return round_up(pairs * ((s + 63) / 64) * g * 4u); }
uint64_t mz_bytes(uint64_t pairs, uint64_t g, uint64_t s) {
  return round_up(pairs * ((s + kUnitTokens - 1) / kUnitTokens) * g * 8u);
}
uint64_t part_bytes(uint64_t pairs, uint64_t g, uint64_t s) {
  return round_up(pairs * ((s + kUnitTokens - 1) / kUnitTokens) * g * 128u * 4u);
}
// workspace: scores, partial sums, batch maxima, unit (m, z), each 256-aligned
uint64_t workspace_bytes(uint64_t pairs, uint64_t g, uint64_t s) {
  return probs_bytes(pairs, g, s) + part_bytes(pairs, g, s) + bmax_bytes(pairs, g, s) + mz_bytes(pairs, g, s);
}
}  // namespace

extern "C" size_t ecco_attention_workspace_size(uint64_t batch, uint64_t kv_heads, uint64_t group, uint64_t seq) {
  if (batch >= (1ull << 20) || kv_heads >= (1ull << 20) || seq >= (1ull << 24) || group > 8) return 0;
  const uint64_t pairs = batch * kv_heads;
  return (size_t)workspace_bytes(pairs, group, seq);
}

namespace {

// Checks the arguments of an attention call (all but the workspace);
// *pairs_out = batch * kv_heads.
int check_attention_args(const void* k_blocks, const void* k_tables, float k_scale, const void* v_blocks,
                         const void* v_tables, float v_scale, const uint16_t* q, uint64_t batch,
                         uint64_t kv_heads, uint64_t group, uint64_t seq, uint64_t kv_stride, float scale,
                         float* out, uint64_t* pairs_out) {
  if (!k_blocks || !k_tables || !v_blocks || !v_tables || !q || !out) return ECCO_EINVAL;
  for (float t : {k_scale, v_scale})
    if (!(t > 0.0f) || !(t < __builtin_huge_valf())) return ECCO_EINVAL;
  if (!(std::fabs(scale) < __builtin_huge_valf())) return ECCO_EINVAL;
  if (batch == 0 || kv_heads == 0 || seq == 0 || kv_stride < seq) return ECCO_ESIZE;
  if (group != 1 && group != 2 && group != 4 && group != 8) return ECCO_ESIZE;
  // each factor bounded before any product, so none of them wraps
  if (batch >= (1ull << 20) || kv_heads >= (1ull << 20) || kv_stride >= (1ull << 32)) return ECCO_ESIZE;
  const uint64_t pairs = batch * kv_heads;
  if (pairs >= (1ull << 20) || seq >= (1ull << 24) || pairs * kv_stride >= (1ull << 32) ||
      pairs * ((seq + 63) / 64) >= (1ull << 31))
    return ECCO_ESIZE;
  if (!host_aligned(k_blocks, 64) || !host_aligned(v_blocks, 64) || !host_aligned(k_tables, 256) ||
      !host_aligned(v_tables, 256) || !host_aligned(q, 16) || !host_aligned(out, 16))
    return ECCO_EALIGN;
  *pairs_out = pairs;
  return ECCO_OK;
}

// Enqueues the attention kernels (scores, p . V, combine) with `workspace`
// (device memory of ecco_attention_workspace_size bytes) for the scores,
// partial sums and maxima.
int launch_attention(const void* k_blocks, const void* k_tables, float k_scale, const void* v_blocks,
                     const void* v_tables, float v_scale, const uint16_t* q, uint64_t pairs, uint64_t group,
                     uint64_t seq, uint64_t kv_stride, float scale, void* workspace, float* out, void* stream) {
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  AttnArgs a;
  a.kb = static_cast<const uint8_t*>(k_blocks);
  a.vb = static_cast<const uint8_t*>(v_blocks);
  a.kt = static_cast<const Tables*>(k_tables);
  a.vt = static_cast<const Tables*>(v_tables);
  a.q = q;
  a.probs = static_cast<float*>(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.part = reinterpret_cast<float*>(ws + probs_bytes(pairs, group, seq));
  a.bmax = reinterpret_cast<float*>(ws + probs_bytes(pairs, group, seq) + part_bytes(pairs, group, seq));
  a.mz = reinterpret_cast<float*>(ws + probs_bytes(pairs, group, seq) + part_bytes(pairs, group, seq) +
                                  bmax_bytes(pairs, group, seq));
  a.out = out;
  a.pairs = (uint32_t)pairs;
  a.S = (uint32_t)seq;
  a.stride = (uint32_t)kv_stride;
  a.n_kb = (uint32_t)((seq + 63) / 64);
  a.n_units = (uint32_t)((seq + kUnitTokens - 1) / kUnitTokens);
  a.G = (uint32_t)group;
  a.kts = k_scale;
  a.vts = v_scale;
  a.scale = (float)((double)scale * 1.4426950408889634);   // scores in base-2 units: exp(x) = 2^(x log2 e)
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const uint32_t kgrid = std::max<uint32_t>(1, std::min<uint32_t>(a.pairs * a.n_kb, (uint32_t)cus));
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_scores_kernel<1>, dim3(kgrid), dim3(score_waves<1>() * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_scores_kernel<2>, dim3(kgrid), dim3(score_waves<2>() * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_scores_kernel<4>, dim3(kgrid), dim3(score_waves<4>() * 64), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_scores_kernel<8>, dim3(kgrid), dim3(score_waves<8>() * 64), 0, s, a); break;
  }
  const uint32_t rows = a.pairs * a.G;
  const uint32_t vgrid = std::max<uint32_t>(1, std::min<uint32_t>(a.pairs * a.n_units, (uint32_t)cus));
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_pv_kernel<1>, dim3(vgrid), dim3(kPvWaves * 64), 0, s, a, 0u); break;
    case 2: hipLaunchKernelGGL(attn_pv_kernel<2>, dim3(vgrid), dim3(kPvWaves * 64), 0, s, a, 0u); break;
    case 4: hipLaunchKernelGGL(attn_pv_kernel<4>, dim3(vgrid), dim3(kPvWaves * 64), 0, s, a, 0u); break;
    default:   // eight heads as two launches of four (accumulators for all eight do not fit)
      hipLaunchKernelGGL(attn_pv_kernel<4>, dim3(vgrid), dim3(kPvWaves * 64), 0, s, a, 0u);
      hipLaunchKernelGGL(attn_pv_kernel<4>, dim3(vgrid), dim3(kPvWaves * 64), 0, s, a, 4u);
      break;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(rows), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}

constexpr uint64_t kScratchBytes = ECCO_ATTENTION_NOALLOC_MAX_WORKSPACE;
static_assert(kScratchBytes % kWsAlign == 0, "scratch size");

}  // namespace

namespace ecco {
// Scratch of the allocation-free entry point: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` only names
// the symbol; its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
}  // namespace ecco

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The calling thread's current device's copy of `scratch`, or nullptr.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int ecco_attention_decode(const void* k_blocks, const void* k_tables, float k_scale, const void* v_blocks,
                                     const void* v_tables, float v_scale, const uint16_t* q, uint64_t batch,
                                     uint64_t kv_heads, uint64_t group, uint64_t seq, uint64_t kv_stride,
                                     float scale, void* workspace, float* out, void* stream) {
  uint64_t pairs = 0;
  const int rc = check_attention_args(k_blocks, k_tables, k_scale, v_blocks, v_tables, v_scale, q, batch, kv_heads,
                                      group, seq, kv_stride, scale, out, &pairs);
  if (rc) return rc;
  if (!workspace) return ECCO_EINVAL;
  if (!host_aligned(workspace, kWsAlign)) return ECCO_EALIGN;
  return launch_attention(k_blocks, k_tables, k_scale, v_blocks, v_tables, v_scale, q, pairs, group, seq, kv_stride,
                          scale, workspace, out, stream);
}

extern "C" int ecco_attention_decode_noalloc(const void* k_blocks, const void* k_tables, float k_scale,
                                             const void* v_blocks, const void* v_tables, float v_scale,
                                             const uint16_t* q, uint64_t batch, uint64_t kv_heads, uint64_t group,
                                             uint64_t seq, uint64_t kv_stride, float scale, float* out,
                                             void* stream) {
  uint64_t pairs = 0;
  int rc = check_attention_args(k_blocks, k_tables, k_scale, v_blocks, v_tables, v_scale, q, batch, kv_heads, group,
                                seq, kv_stride, scale, out, &pairs);
  if (rc) return rc;
  if (workspace_bytes(pairs, group, seq) > kScratchBytes) return ECCO_ESIZE;
  int cus = 0;
  rc = check_gfx950(&cus);
  if (rc) return rc;
  void* ws = scratch_address();
  if (!ws) return ECCO_EHIP;
  return launch_attention(k_blocks, k_tables, k_scale, v_blocks, v_tables, v_scale, q, pairs, group, seq, kv_stride,
                          scale, ws, out, stream);
}
