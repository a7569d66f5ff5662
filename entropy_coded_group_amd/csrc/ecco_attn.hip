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
//            DPP row sum over the token's 16 lanes, scale -> s[pair][t][g]
//   softmax  one workgroup per pair: max, sum of exp, normalise in place
//   p . V    one wave per 128 tokens of one pair: decoded V values times the
//            token's probabilities, FP32 accumulators for the G heads and the
//            lane's 8 positions, a cross-row reduction, partial sums per unit
//   combine  the units' partial sums of each output row added in order
//
// Every sum is taken in a fixed order, so results do not depend on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "ecco_device.h"

namespace ecco {

constexpr uint32_t kUnitTokens = 128;   // tokens per p . V work unit (two batches)
constexpr int kScoreWaves = 12;         // waves per workgroup of the scores kernel (at G = 4 the compiler
                                        // spills 24 registers to fit 3 waves per SIMD, still 4.5 % faster
                                        // than 2 waves per SIMD without spills)
constexpr int kPvWaves = 8;             // waves per workgroup of the p . V kernel

struct AttnArgs {
  const uint8_t* kb;
  const uint8_t* vb;
  const Tables* kt;
  const Tables* vt;
  const uint16_t* q;
  float* probs;          // [pairs][S][G]
  float* part;           // [pairs][n_units][G][128]
  float* out;            // [pairs * G][128]
  uint32_t pairs, S, stride, n_kb, n_units, G;
  float kts, vts, scale;
};

// The 64 blocks of batch t0 .. t0 + 63 of one pair (clamped at S); with
// live == false the cached table blob is read instead (a prefetch past the
// end that must stay unconditional).
__device__ __forceinline__ BatchRegs fetch_tokens(uint32_t lane, const uint8_t* rows, const uint8_t* idle,
                                                  uint32_t n_valid, bool live) {
  return fetch_batch(lane, n_valid, [&](uint32_t i, uint32_t q) {
    return load_stream((live ? rows + (uint64_t)i * 64u : idle + 64u * (i & 63u)) + 16u * q);
  });
}

template <int G>
__global__ __launch_bounds__(kScoreWaves * 64) void attn_scores_kernel(AttnArgs a) {
  __shared__ DecodeSmem<kScoreWaves> sm;
  stage_decode_tables(sm, a.kt);
  __syncthreads();
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
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
    uint4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g] = *reinterpret_cast<const uint4*>(a.q + ((uint64_t)pair * G + g) * 128u + j0);
    float* sp = a.probs + ((uint64_t)pair * a.S + t0) * G;
    auto sink = [&](uint32_t b, uint32_t, uint4 w, uint32_t, uint32_t) {
      float d[G];
#pragma unroll
      for (int g = 0; g < G; ++g) d[g] = row_sum_f32(dot8(w, qv[g], 0.0f)) * a.scale;
      // one vector store of the token's G scores (whole 16-byte pieces, so the
      // four tokens of an instruction fill their 64 bytes without partial writes)
      if ((lane & 15u) == 0) {
        float* dst = sp + (uint64_t)b * G;
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
      decode_batch<true, kScoreWaves, 128, true>(sm, wave, lane, 64u, a.kts, cur, sink);
    else
      decode_batch<false, kScoreWaves, 128, true>(sm, wave, lane, n_valid, a.kts, cur, sink);
    cur = nxt;
  }
}

// Softmax of one pair's G rows, [S][G] with g innermost, by one workgroup:
// three coalesced passes over the pair's scores (max, sum of exp, then exp
// again divided by the sum, written in place), which stay in the L2 cache
// between them; workgroup reductions through LDS.  Recomputing exp in the
// last pass gives the same values as the second and saves a write pass.
constexpr int kSmThreads = 1024;

template <int G>
__global__ __launch_bounds__(kSmThreads) void attn_softmax_kernel(AttnArgs a) {
  __shared__ float red[kSmThreads / 64][G];
  __shared__ float fin[G];
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  float* base = a.probs + (uint64_t)blockIdx.x * a.S * G;
  auto wg_reduce = [&](float (&v)[G], bool is_max) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float w = is_max ? wave_max_f32(v[g]) : wave_sum_f32(v[g]);
      if (lane == 0) red[wave][g] = w;
    }
    __syncthreads();
    if (tid < (uint32_t)G) {
      float r = red[0][tid];
      for (int w = 1; w < kSmThreads / 64; ++w) r = is_max ? fmaxf(r, red[w][tid]) : r + red[w][tid];
      fin[tid] = r;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = fin[g];
    __syncthreads();
  };
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -__builtin_inff();
  for (uint32_t t = tid; t < a.S; t += kSmThreads)
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = fmaxf(m[g], base[(uint64_t)t * G + g]);
  wg_reduce(m, true);
  float z[G];
#pragma unroll
  for (int g = 0; g < G; ++g) z[g] = 0.0f;
  for (uint32_t t = tid; t < a.S; t += kSmThreads)
#pragma unroll
    for (int g = 0; g < G; ++g) z[g] += expf(base[(uint64_t)t * G + g] - m[g]);
  wg_reduce(z, false);
  float inv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) inv[g] = 1.0f / z[g];
  for (uint32_t t = tid; t < a.S; t += kSmThreads)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* q = base + (uint64_t)t * G + g;
      *q = expf(*q - m[g]) * inv[g];
    }
}

// p . V for heads g_off .. g_off + GH - 1 of G.
template <int GH>
__global__ __launch_bounds__(kPvWaves * 64) void attn_pv_kernel(AttnArgs a, uint32_t g_off) {
  __shared__ DecodeSmem<kPvWaves> sm;
  stage_decode_tables(sm, a.vt);
  __syncthreads();
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
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
  float acc[GH][8];
#pragma unroll
  for (int g = 0; g < GH; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  // slots (unit, half) in order; a unit's sums are flushed after its second half
  for (uint32_t half = 0; unit < total;) {
    const uint32_t pair = unit / a.n_units, u = unit % a.n_units;
    const uint32_t nu = unit + stride;
    const BatchRegs nxt = half == 0u ? fetch(unit, 1, true) : fetch(nu < total ? nu : unit, 0, nu < total);
    const uint32_t t0 = u * kUnitTokens + 64u * half;
    if (t0 < a.S) {
      const uint32_t n_valid = min(64u, a.S - t0);
      const float* pp = a.probs + ((uint64_t)pair * a.S + t0) * a.G + g_off;
      auto sink = [&](uint32_t b, uint32_t, uint4 w, uint32_t, uint32_t) {
        float p[GH];
#pragma unroll
        for (int g = 0; g < GH; ++g) p[g] = pp[(uint64_t)b * a.G + g];
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = f16_value((wv[i / 2] >> (16 * (i & 1))) & 0xffffu);
#pragma unroll
          for (int g = 0; g < GH; ++g) acc[g][i] = fmaf(p[g], v, acc[g][i]);
        }
      };
      if (n_valid == 64u)
        decode_batch<true, kPvWaves, 128, true>(sm, wave, lane, 64u, a.vts, cur, sink);
      else
        decode_batch<false, kPvWaves, 128, true>(sm, wave, lane, n_valid, a.vts, cur, sink);
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
      if (lane < 16u) {
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float* dst = a.part + (((uint64_t)pair * a.n_units + u) * a.G + g_off + g) * 128u + j0;
          *reinterpret_cast<float4*>(dst) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
      }
#pragma unroll
      for (int g = 0; g < GH; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
      unit = nu;
      half = 0;
    } else {
      half = 1;
    }
  }
}

// out[pair * G + g][d] = sum over units, in unit order.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const uint64_t idx = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const uint64_t rows = (uint64_t)a.pairs * a.G;
  if (idx >= rows * 128u) return;
  const uint32_t d = (uint32_t)(idx & 127u);
  const uint64_t row = idx >> 7;
  const uint32_t pair = (uint32_t)(row / a.G), g = (uint32_t)(row % a.G);
  const float* src = a.part + ((uint64_t)pair * a.n_units * a.G + g) * 128u + d;
  float s = 0.0f;
#pragma unroll 8
  for (uint32_t u = 0; u < a.n_units; ++u) s += src[(uint64_t)u * a.G * 128u];
  a.out[row * 128u + d] = s;
}

}  // namespace ecco

using namespace ecco;

namespace {
constexpr uint64_t kWsAlign = 256;
uint64_t round_up(uint64_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
uint64_t probs_bytes(uint64_t pairs, uint64_t g, uint64_t s) { return round_up(pairs * s * g * 4u); }
uint64_t part_bytes(uint64_t pairs, uint64_t g, uint64_t s) {
  return round_up(pairs * ((s + kUnitTokens - 1) / kUnitTokens) * g * 128u * 4u);
}
}  // namespace

extern "C" size_t ecco_attention_workspace_size(uint64_t batch, uint64_t kv_heads, uint64_t group, uint64_t seq) {
  const uint64_t pairs = batch * kv_heads;
  return (size_t)(probs_bytes(pairs, group, seq) + part_bytes(pairs, group, seq));
}

extern "C" int ecco_attention_decode(const void* k_blocks, const void* k_tables, float k_scale, const void* v_blocks,
                                     const void* v_tables, float v_scale, const uint16_t* q, uint64_t batch,
                                     uint64_t kv_heads, uint64_t group, uint64_t seq, uint64_t kv_stride,
                                     float scale, void* workspace, float* out, void* stream) {
  if (!k_blocks || !k_tables || !v_blocks || !v_tables || !q || !workspace || !out) return ECCO_EINVAL;
  for (float t : {k_scale, v_scale})
    if (!(t > 0.0f) || !(t < __builtin_huge_valf())) return ECCO_EINVAL;
  if (!(std::fabs(scale) < __builtin_huge_valf())) return ECCO_EINVAL;
  if (batch == 0 || kv_heads == 0 || seq == 0 || kv_stride < seq) return ECCO_ESIZE;
  if (group != 1 && group != 2 && group != 4 && group != 8) return ECCO_ESIZE;
  const uint64_t pairs = batch * kv_heads;
  if (pairs >= (1ull << 20) || seq >= (1ull << 24) || pairs * kv_stride >= (1ull << 32) ||
      pairs * ((seq + 63) / 64) >= (1ull << 31))
    return ECCO_ESIZE;
  if (!host_aligned(k_blocks, 64) || !host_aligned(v_blocks, 64) || !host_aligned(k_tables, 256) ||
      !host_aligned(v_tables, 256) || !host_aligned(q, 16) || !host_aligned(workspace, kWsAlign) ||
      !host_aligned(out, 16))
    return ECCO_EALIGN;
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  AttnArgs a;
  a.kb = static_cast<const uint8_t*>(k_blocks);
  a.vb = static_cast<const uint8_t*>(v_blocks);
  a.kt = static_cast<const Tables*>(k_tables);
  a.vt = static_cast<const Tables*>(v_tables);
  a.q = q;
  a.probs = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + probs_bytes(pairs, group, seq));
  a.out = out;
  a.pairs = (uint32_t)pairs;
  a.S = (uint32_t)seq;
  a.stride = (uint32_t)kv_stride;
  a.n_kb = (uint32_t)((seq + 63) / 64);
  a.n_units = (uint32_t)((seq + kUnitTokens - 1) / kUnitTokens);
  a.G = (uint32_t)group;
  a.kts = k_scale;
  a.vts = v_scale;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const uint32_t kgrid = std::max<uint32_t>(1, std::min<uint32_t>(a.pairs * a.n_kb, (uint32_t)cus));
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_scores_kernel<1>, dim3(kgrid), dim3(kScoreWaves * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_scores_kernel<2>, dim3(kgrid), dim3(kScoreWaves * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_scores_kernel<4>, dim3(kgrid), dim3(kScoreWaves * 64), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_scores_kernel<8>, dim3(kgrid), dim3(kScoreWaves * 64), 0, s, a); break;
  }
  const uint32_t rows = a.pairs * a.G;
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_softmax_kernel<1>, dim3(a.pairs), dim3(kSmThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_softmax_kernel<2>, dim3(a.pairs), dim3(kSmThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_softmax_kernel<4>, dim3(a.pairs), dim3(kSmThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_softmax_kernel<8>, dim3(a.pairs), dim3(kSmThreads), 0, s, a); break;
  }
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
  const uint64_t n = (uint64_t)rows * 128u;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}
