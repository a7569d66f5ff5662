// Fused decode + GEMV for gfx950: y[b][o] = sum_i W[o][i] * x[b][i], W held as
// Ecco blocks.  The pages' consumer of compressed weights is the decode-phase
// GEMM, memory-bound at small batch (Ecco review, "If this is right"; Fig. 12
// caption: memory requests of a GEMM kernel).  At batch 1..8 the product is
// not a dense contraction worth the matrix cores, so the decoded FP16 weights
// are multiplied on the vector ALUs (v_dot2_f32_f16: two FP16 products summed
// into an FP32 accumulator) straight out of the decoder, without writing W.
//
// Work split: a wavefront owns one output row at a time and decodes the row's
// blocks 64 at a time with the shared decode core; each lane accumulates the
// products of the 8 weights it is handed for every batch column, and a wave
// reduction finishes the row.
#include <hip/hip_runtime.h>

#include "ecco_device.h"

namespace ecco {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, x.w), acc, false);
  return acc;
}

struct GemvArgs {
  const uint8_t* blocks;
  const Tables* tab;
  const uint16_t* x;
  float* y;
  uint32_t out_f, in_f, gpr, batch;
  float t;
};

template <int BM>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_kernel(GemvArgs a) {
  __shared__ DecodeSmem<kGemvWaves> sm;
  stage_decode_tables(sm, a.tab);
  __syncthreads();
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t stride = gridDim.x * kGemvWaves;
  uint32_t row = wave * gridDim.x + blockIdx.x;   // rows go round the CUs first
  if (row >= a.out_f) return;
  auto fetch = [&](uint32_t rw, uint32_t c0) {
    const uint8_t* rowblk = a.blocks + ((uint64_t)rw * a.gpr + c0) * 64u;
    return fetch_batch(lane, min(64u, a.gpr - c0), [&](uint32_t b, uint32_t q) {
      return *reinterpret_cast<const uint4*>(rowblk + (uint64_t)b * 64u + 16u * q);
    });
  };
  float part[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) part[b] = 0.0f;
  uint32_t c0 = 0;
  BatchRegs cur = fetch(row, 0);
  while (true) {
    uint32_t nrow = row, nc0 = c0 + 64u;
    if (nc0 >= a.gpr) {
      nrow = row + stride;
      nc0 = 0;
    }
    const BatchRegs nxt = nrow < a.out_f ? fetch(nrow, nc0) : fetch(row, c0);
    auto sink = [&](uint32_t b, uint32_t j0, uint4 w) {
      const uint16_t* xp = a.x + (uint64_t)(c0 + b) * 128u + j0;
#pragma unroll
      for (int b2 = 0; b2 < BM; ++b2) {
        if ((uint32_t)b2 < a.batch) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xp + (uint64_t)b2 * a.in_f);
          part[b2] = dot8(w, xv, part[b2]);
        }
      }
    };
    const uint32_t n_valid = min(64u, a.gpr - c0);
    if (n_valid == 64u)
      decode_batch<true>(sm, wave, lane, 64u, a.t, cur, sink);
    else
      decode_batch<false>(sm, wave, lane, n_valid, a.t, cur, sink);
    if (c0 + 64u >= a.gpr) {
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        float v = part[b];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0 && (uint32_t)b < a.batch) a.y[(uint64_t)b * a.out_f + row] = v;
        part[b] = 0.0f;
      }
    }
    if (nrow >= a.out_f) break;
    row = nrow;
    c0 = nc0;
    cur = nxt;
  }
}

}  // namespace ecco

using namespace ecco;

extern "C" int ecco_decode_gemv(const void* blocks, const void* tables, float tensor_scale, int64_t out_f,
                                int64_t in_f, const uint16_t* x, int64_t batch, float* y, void* stream) {
  if (!blocks || !tables || !x || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  if (out_f < 1 || in_f < 128 || in_f % 128 != 0 || batch < 1 || batch > ECCO_GEMV_MAX_BATCH) return ECCO_ESIZE;
  if ((uint64_t)out_f * (uint64_t)(in_f / 128) >= (1ull << 32) || out_f >= (1ll << 31)) return ECCO_ESIZE;
  if (!host_aligned(blocks, 64) || !host_aligned(tables, 256) || !host_aligned(x, 16) || !host_aligned(y, 4))
    return ECCO_EALIGN;
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  GemvArgs a;
  a.blocks = static_cast<const uint8_t*>(blocks);
  a.tab = static_cast<const Tables*>(tables);
  a.x = x;
  a.y = y;
  a.out_f = (uint32_t)out_f;
  a.in_f = (uint32_t)in_f;
  a.gpr = (uint32_t)(in_f / 128);
  a.batch = (uint32_t)batch;
  a.t = tensor_scale;
  const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(a.out_f, (uint32_t)cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (batch == 1)
    hipLaunchKernelGGL(gemv_kernel<1>, dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
  else if (batch <= 2)
    hipLaunchKernelGGL(gemv_kernel<2>, dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
  else if (batch <= 4)
    hipLaunchKernelGGL(gemv_kernel<4>, dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(gemv_kernel<8>, dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}
