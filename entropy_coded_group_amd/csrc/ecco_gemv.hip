// Fused decode + GEMV for gfx950: y[b][o] = sum_i W[o][i] * x[b][i], W held as
// Ecco blocks.  The pages' consumer of compressed weights is the decode-phase
// GEMM, memory-bound at small batch (Ecco review, "If this is right"; Fig. 12
// caption: memory requests of a GEMM kernel).  At batch 1..8 the product is
// not a dense contraction worth the matrix cores, so the decoded FP16 weights
// are multiplied on the vector ALUs (v_dot2_f32_f16: two FP16 products summed
// into an FP32 accumulator) straight out of the decoder, without writing W.
//
// Work split at batch 1 with rows of 16, 32 or 64 blocks (in_features 2048,
// 4096, 8192): the matrix is cut into batches of 64 consecutive blocks, i.e.
// 4, 2 or 1 whole rows, dealt round the waves of all CUs.  The decode core
// hands the weights over in four passes of 16 blocks and each pass lies inside
// one row, so every lane keeps one accumulator per row of the batch; wave sums
// finish the rows.  Otherwise a wavefront owns one output row at a time and
// decodes its blocks 64 at a time (the last batch of a row partly filled).
// Either way each lane accumulates the products of the 8 weights it is
// handed, and the sums are taken in a fixed order.
#include <hip/hip_runtime.h>

#include "ecco_device.h"

namespace ecco {

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
    auto sink = [&](uint32_t b, uint32_t j0, uint4 w, uint32_t) {
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
        const float v = wave_sum_f32(part[b]);
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

// Rows of 64 / RB blocks: RB whole rows per 64-block batch.
template <int BM, int RB>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_rows_kernel(GemvArgs a) {
  __shared__ DecodeSmem<kGemvWaves> sm;
  stage_decode_tables(sm, a.tab);
  __syncthreads();
  constexpr uint32_t kGpr = 64 / RB;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t n_groups = a.out_f * kGpr;
  const uint32_t n_batches = (n_groups + 63u) / 64u;
  const uint32_t stride = gridDim.x * kGemvWaves;
  uint32_t batch = wave * gridDim.x + blockIdx.x;   // batches go round the CUs first
  if (batch >= n_batches) return;
  auto fetch = [&](uint32_t bt) {
    const uint32_t g0 = bt * 64u;
    return fetch_batch(lane, min(64u, n_groups - g0), [&](uint32_t i, uint32_t q) {
      return load_stream(a.blocks + (uint64_t)(g0 + i) * 64u + 16u * q);
    });
  };
  BatchRegs cur = fetch(batch);
  for (; batch < n_batches; batch += stride) {
    const uint32_t nb = batch + stride;
    const BatchRegs nxt = fetch(nb < n_batches ? nb : batch);
    float acc[RB][BM];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int b2 = 0; b2 < BM; ++b2) acc[r][b2] = 0.0f;
    // pass k covers blocks 16 k .. 16 k + 15: row k * RB / 4 of the batch
    // an opaque copy of x per batch: otherwise the compiler hoists the 16
    // loop-invariant x addresses of a batch out of the loop (32 registers)
    const uint16_t* xb = a.x;
    asm volatile("" : "+s"(xb));
    auto sink = [&](uint32_t b, uint32_t j0, uint4 w, uint32_t k) {
      const uint16_t* xp = xb + (uint64_t)(b & (kGpr - 1u)) * 128u + j0;
      const uint32_t r = k * RB / 4u;
#pragma unroll
      for (int b2 = 0; b2 < BM; ++b2) {
        if ((uint32_t)b2 < a.batch) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xp + (uint64_t)b2 * a.in_f);
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
            if ((uint32_t)rr == r) acc[rr][b2] = dot8(w, xv, acc[rr][b2]);
        }
      }
    };
    const uint32_t n_valid = min(64u, n_groups - batch * 64u);
    if (n_valid == 64u)
      decode_batch<true>(sm, wave, lane, 64u, a.t, cur, sink);
    else
      decode_batch<false>(sm, wave, lane, n_valid, a.t, cur, sink);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const uint32_t row = batch * RB + r;
#pragma unroll
      for (int b2 = 0; b2 < BM; ++b2) {
        const float v = wave_sum_f32(acc[r][b2]);
        if (lane == 0 && (uint32_t)b2 < a.batch && row < a.out_f) a.y[(uint64_t)b2 * a.out_f + row] = v;
      }
    }
    cur = nxt;
  }
}

}  // namespace ecco

using namespace ecco;

namespace {
template <int BM>
void launch_gemv(const GemvArgs& a, uint32_t cus, hipStream_t s) {
  // (one accumulator per row and batch column: with more columns the
  // registers run out, and those launches use the row-per-wave kernel)
  if constexpr (BM == 1) {
    if (a.gpr == 16 || a.gpr == 32 || a.gpr == 64) {
      const uint32_t rb = 64u / a.gpr;
      const uint32_t n_batches = (a.out_f * a.gpr + 63u) / 64u;
      const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(n_batches, cus));
      if (rb == 4)
        hipLaunchKernelGGL((gemv_rows_kernel<1, 4>), dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
      else if (rb == 2)
        hipLaunchKernelGGL((gemv_rows_kernel<1, 2>), dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
      else
        hipLaunchKernelGGL((gemv_rows_kernel<1, 1>), dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
      return;
    }
  }
  const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(a.out_f, cus));
  hipLaunchKernelGGL(gemv_kernel<BM>, dim3(grid), dim3(kGemvWaves * 64), 0, s, a);
}
}  // namespace

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
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (batch == 1)
    launch_gemv<1>(a, (uint32_t)cus, s);
  else if (batch <= 2)
    launch_gemv<2>(a, (uint32_t)cus, s);
  else if (batch <= 4)
    launch_gemv<4>(a, (uint32_t)cus, s);
  else
    launch_gemv<8>(a, (uint32_t)cus, s);
  return hipGetLastError() == hipSuccess ? ECCO_OK : ECCO_EHIP;
}
