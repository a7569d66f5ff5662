// Fused decode + GEMV for gfx950: y[b][o] = sum_i W[o][i] * x[b][i], W held as
// Ecco blocks.  The pages' consumer of compressed weights is the decode-phase
// GEMM, memory-bound at small batch (Ecco review, "If this is right"; Fig. 12
// caption: memory requests of a GEMM kernel).  At batch 1..8 the product is
// not a dense contraction worth the matrix cores, so the decoded FP16 weights
// are multiplied on the vector ALUs (v_dot2_f32_f16: two FP16 products summed
// into an FP32 accumulator) straight out of the decoder, without writing W.
//
// Work splits:
//  * batch 1 with rows of 16, 32 or 64 blocks (in_features 2048, 4096,
//    8192): the matrix is cut into batches of 64 consecutive blocks, i.e. 4,
//    2 or 1 whole rows, dealt round the waves of all CUs.  The decode core
//    hands the weights over in four passes of 16 blocks and each pass lies
//    inside one row, so every lane keeps one accumulator per row of the
//    batch; wave sums finish the rows.
//  * otherwise, with out_features a multiple of 4 and rows a multiple of 16
//    blocks: row groups.  A wavefront owns 4 rows and walks their columns 16
//    blocks at a time; a 64-block batch holds the 4 x 16 blocks in
//    column-major order (block 4c + r), so the decode core's write-out hands
//    lane l always a weight slice of row l / 16, and the four blocks of one
//    write-out step share their column: the x slices a step needs are the
//    same for the four rows, so every x load instruction touches a quarter
//    of the bytes it would with one row per batch.  DPP row sums (one DPP row
//    = one output row) finish the rows.
//  * otherwise a wavefront owns one output row at a time and decodes its
//    blocks 64 at a time (the last batch of a row partly filled).
// Each lane accumulates the products of the 8 weights it is handed, and the
// sums are taken in a fixed order.
//
// One launch can cover several matrices (the q, k and v projections of a
// layer read the same x): each workgroup stages one matrix's tables and the
// CUs are shared out in proportion to the matrices' work, so small matrices
// run beside large ones instead of leaving most CUs idle.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ecco_device.h"

namespace ecco {

// One matrix of a launch, and the contiguous range of workgroups that work
// on it.
struct GemvJob {
  const uint8_t* blocks;
  const Tables* tab;
  const uint16_t* x;
  float* y;
  uint32_t out_f, in_f, gpr;
  uint32_t rb;         // whole rows per 64-block batch (1, 2 or 4); kRowGroups: row groups; 0: one row per wave
  uint32_t n_units;    // 64-block batches (rb 1, 2, 4), row groups of 4 (kRowGroups) or rows (0)
  uint32_t wg_first, wg_count;
  float t;
};

constexpr int kMaxGemvJobs = ECCO_GEMV_MAX_JOBS;
constexpr uint32_t kRowGroups = 8;   // GemvJob::rb of the row-group split

struct GemvArgs {
  GemvJob job[kMaxGemvJobs];
  uint32_t n_jobs, batch;
};

// acc[b2] += the 8 weights w . x[b2][the same 8 columns] for b2 < BM, x[b2]
// at xp + b2 * in_f.  The BM loads sit together under one run-time
// condition (always true: batch >= 1), so they issue together and their
// latency is paid once, and the compiler does not move them (or their
// addresses) ahead of the write-out pass they belong to; a column past the
// batch reads the last row, and its sums are never stored.  Under a
// condition per column, each load was waited for on its own, and each wait
// also covered the next batch's block prefetch.
template <int BM>
__device__ __forceinline__ void gemv_dot_x(float (&acc)[BM], uint4 w, const uint16_t* xp, uint32_t in_f,
                                           uint32_t batch) {
  if (batch != 0u) {
    uint4 xv[BM];
#pragma unroll
    for (int b2 = 0; b2 < BM; ++b2)
      xv[b2] = *reinterpret_cast<const uint4*>(xp + (uint64_t)min((uint32_t)b2, batch - 1u) * in_f);
#pragma unroll
    for (int b2 = 0; b2 < BM; ++b2) acc[b2] = dot8(w, xv[b2], acc[b2]);
  }
}

// A wavefront owns one output row at a time and decodes its blocks 64 at a
// time (the last batch of a row partly filled).  Rows go round the job's
// workgroups first, then their waves.
template <int BM, bool STOP>
__device__ __forceinline__ void gemv_rows_per_wave(DecodeSmem<kGemvWaves>& sm, const GemvJob& a, uint32_t lw,
                                                   uint32_t batch) {
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t stride = a.wg_count * kGemvWaves;
  uint32_t row = wave * a.wg_count + lw;
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
    auto sink = [&](uint32_t b, uint32_t j0, uint4 w, uint32_t, uint32_t) {
      const uint16_t* xp = a.x + (uint64_t)(c0 + b) * 128u + j0;
      gemv_dot_x<BM>(part, w, xp, a.in_f, batch);
    };
    const uint32_t n_valid = min(64u, a.gpr - c0);
    if (n_valid == 64u)
      decode_batch<true, kGemvWaves, 128, false, STOP>(sm, wave, lane, 64u, a.t, cur, sink);
    else
      decode_batch<false, kGemvWaves, 128, false, STOP>(sm, wave, lane, n_valid, a.t, cur, sink);
    if (c0 + 64u >= a.gpr) {
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        const float v = wave_sum_f32(part[b]);
        if (lane == 0 && (uint32_t)b < batch) a.y[(uint64_t)b * a.out_f + row] = v;
        part[b] = 0.0f;
      }
    }
    if (nrow >= a.out_f) break;
    row = nrow;
    c0 = nc0;
    cur = nxt;
  }
}

// Batch 1, rows of 64 / RB blocks: RB whole rows per 64-block batch.  The
// decode core hands the weights over in four passes of 16 blocks and each
// pass lies inside one row (pass k: row k * RB / 4 of the batch), so every
// lane keeps one accumulator per row; wave sums finish the rows.
template <int RB, bool STOP>
__device__ __forceinline__ void gemv_whole_rows(DecodeSmem<kGemvWaves>& sm, const GemvJob& a, uint32_t lw,
                                                uint32_t batch_cols) {
  constexpr uint32_t kGpr = 64 / RB;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t n_groups = a.out_f * kGpr;
  const uint32_t n_batches = a.n_units;
  const uint32_t stride = a.wg_count * kGemvWaves;
  uint32_t batch = wave * a.wg_count + lw;          // batches go round the workgroups first
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
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.0f;
    // an opaque copy of x per batch: otherwise the compiler hoists the 16
    // loop-invariant x addresses of a batch out of the loop (32 registers)
    const uint16_t* xb = a.x;
    asm volatile("" : "+s"(xb));
    // rows of 32 or 64 blocks: the pass's four x slices are loaded as the
    // pass starts, so their latency runs under the pass's LDS work (with
    // four rows per batch the extra registers spill, and the loads stay in
    // the sink).  A load under a run-time condition is not started earlier
    // than written; unconditional, all 16 of a batch would be issued first
    // and held across the decode.
    constexpr bool kPre = RB <= 2;
    uint4 xpre[4];
    auto pre = [&](uint32_t k) {
      if constexpr (kPre) {
        if (batch_cols != 0u) {
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const uint32_t b = 16u * k + 4u * (uint32_t)it + lane / 16u;
            xpre[it] = *reinterpret_cast<const uint4*>(xb + (uint64_t)(b & (kGpr - 1u)) * 128u + 8u * (lane % 16u));
          }
        }
      }
    };
    auto sink = [&](uint32_t b, uint32_t j0, uint4 w, uint32_t k, uint32_t it) {
      const uint32_t r = k * RB / 4u;
      if (batch_cols != 0u) {
        uint4 xv;
        if constexpr (kPre) {
          xv = xpre[it];
        } else {
          xv = *reinterpret_cast<const uint4*>(xb + (uint64_t)(b & (kGpr - 1u)) * 128u + j0);
        }
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
          if ((uint32_t)rr == r) acc[rr] = dot8(w, xv, acc[rr]);
      }
    };
    const uint32_t n_valid = min(64u, n_groups - batch * 64u);
    if (n_valid == 64u)
      decode_batch<true, kGemvWaves, 128, false, STOP>(sm, wave, lane, 64u, a.t, cur, sink, pre);
    else
      decode_batch<false, kGemvWaves, 128, false, STOP>(sm, wave, lane, n_valid, a.t, cur, sink, pre);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const uint32_t row = batch * RB + r;
      const float v = wave_sum_f32(acc[r]);
      if (lane == 0 && row < a.out_f) a.y[row] = v;
    }
    cur = nxt;
  }
}

// Row groups: 4 rows x 16 block columns per 64-block batch, column-major (see
// the file header).  Lane l's row is l / 16 and its 8 weights are positions
// 8 (l % 16) .. + 7 of its block; block b of the batch is column b / 4.
//
// A unit is one batch: (row group, column chunk).  Each workgroup takes a
// contiguous share of the job's row groups and works through it in rounds of
// up to kGemvUnits units (whole row groups); the units of a round are dealt
// round the workgroup's waves, so every wave gets as many batches as the
// others give or take one, whatever the rows' length.  Each unit's row sums
// go to LDS; after a barrier the sums of a row group's chunks are added in
// chunk order.  The order of every sum depends only on the matrix, not on
// how many workgroups the launch gives the job, so a call with several jobs
// gives the same bits as one call per job.
constexpr uint32_t kGemvUnits = 84;     // units per round (row sums of a round in LDS)

// The row sums of a round (one array for both decode instances of a kernel).
template <int BM>
__device__ __forceinline__ float (&gemv_round_sums())[kGemvUnits][4][BM] {
  __shared__ float part[kGemvUnits][4][BM];
  return part;
}

template <int BM, bool STOP>
__device__ __forceinline__ void gemv_row_groups(DecodeSmem<kGemvWaves>& sm, const GemvJob& a, uint32_t lw,
                                                uint32_t batch) {
  float (&part)[kGemvUnits][4][BM] = gemv_round_sums<BM>();
  // the wave index is uniform: held in a scalar register, so are the unit counters
  const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t n_cc = a.gpr / 16u;              // column chunks of a row group
  const uint32_t rg_lo = (uint32_t)((uint64_t)a.n_units * lw / a.wg_count);
  const uint32_t rg_hi = (uint32_t)((uint64_t)a.n_units * (lw + 1u) / a.wg_count);
  const uint32_t R = kGemvUnits / n_cc;           // row groups per round (>= 1: the host checks n_cc)
  // The decode core takes chunk i of lane l as bytes 16 (l & 3) .. + 15 of
  // batch block (l >> 2) + 16 i, i.e. column (l >> 4) + 4 i of row (l >> 2) & 3:
  // one offset per lane, then 256 bytes (4 columns) per chunk.  A prefetch
  // past the wave's last unit reads the (cached) table blob instead.
  const uint32_t lane_off = (((lane >> 2) & 3u) * a.gpr + (lane >> 4)) * 64u + 16u * (lane & 3u);
  const uint8_t* idle = reinterpret_cast<const uint8_t*>(a.tab) + 64u * (lane >> 2) + 16u * (lane & 3u);
  auto fetch = [&](uint32_t rg, uint32_t cc, bool live) {
    const uint8_t* p = live ? a.blocks + ((uint64_t)rg * 4u * a.gpr + (uint64_t)cc * 16u) * 64u + lane_off
                            : idle;
    BatchRegs r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = load_stream(p + (live ? 256u : 1024u) * (uint32_t)i);
    return r;
  };
  const uint32_t j0 = 8u * (lane & 15u);
  uint32_t g0 = rg_lo;
  if (g0 >= rg_hi) return;                        // the whole workgroup has no share (uniform)
  // units of the round starting at row group g0; this wave's are wave, wave + kGemvWaves, ...
  uint32_t U = min(R, rg_hi - g0) * n_cc, u = wave;
  BatchRegs cur = fetch(g0 + u / n_cc, u % n_cc, u < U);
  while (true) {
    for (; u < U; u += kGemvWaves) {
      // the next unit: this round's, else this wave's first of the next round
      uint32_t nu = u + kGemvWaves, ng = g0, nU = U;
      if (nu >= U && g0 + R < rg_hi) {
        ng = g0 + R;
        nU = min(R, rg_hi - ng) * n_cc;
        nu = wave;
      }
      const bool live = nu < nU;
      const BatchRegs nxt = fetch(ng + (live ? nu / n_cc : 0u), live ? nu % n_cc : 0u, live);
      const uint32_t cc = u % n_cc;
      const uint16_t* xc = a.x + (uint64_t)cc * (16u * 128u) + j0;
      float acc[BM];
#pragma unroll
      for (int b = 0; b < BM; ++b) acc[b] = 0.0f;
      auto sink = [&](uint32_t b, uint32_t, uint4 w, uint32_t, uint32_t) {
        gemv_dot_x<BM>(acc, w, xc + (uint64_t)(b >> 2) * 128u, a.in_f, batch);
      };
      decode_batch<true, kGemvWaves, 128, false, STOP>(sm, wave, lane, 64u, a.t, cur, sink);
#pragma unroll
      for (int b2 = 0; b2 < BM; ++b2) {
        const float v = row_sum_f32(acc[b2]);
        if ((lane & 15u) == 0u) part[u][lane >> 4][b2] = v;
      }
      cur = nxt;
    }
    __syncthreads();
    // row (g0 + j, q), batch column b2: its chunks' sums in chunk order
    const uint32_t n_rg = U / n_cc;
    for (uint32_t o = threadIdx.x; o < n_rg * 4u * batch; o += blockDim.x) {
      const uint32_t b2 = o % batch, q = (o / batch) & 3u, jg = o / (4u * batch);
      float s = 0.0f;
      for (uint32_t cc = 0; cc < n_cc; ++cc) s += part[jg * n_cc + cc][q][b2];
      a.y[(uint64_t)b2 * a.out_f + 4u * (g0 + jg) + q] = s;
    }
    __syncthreads();
    g0 += R;
    if (g0 >= rg_hi) break;
    // a wave that had a unit in the round has prefetched its first of this one
    const bool prefetched = wave < U;
    U = min(R, rg_hi - g0) * n_cc;
    u = wave;
    if (!prefetched) cur = fetch(g0 + u / n_cc, u % n_cc, u < U);
  }
}

// The kernel's work split.  Tables with an incomplete codebook take the
// decode core's STOP instance, in the simplest split only (a row per wave,
// which serves every shape): a second instance of the larger splits made
// the kernels spill.
template <int BM, int RB>
__device__ __forceinline__ void gemv_split(DecodeSmem<kGemvWaves>& sm, const GemvJob& a, uint32_t lw, uint32_t batch) {
  if (!a.tab->complete) {
    gemv_rows_per_wave<BM, true>(sm, a, lw, batch);
  } else if constexpr (RB == (int)kRowGroups) {
    gemv_row_groups<BM, false>(sm, a, lw, batch);
  } else if constexpr (RB > 0) {
    static_assert(BM == 1, "whole rows per batch at batch 1 only");
    gemv_whole_rows<RB, false>(sm, a, lw, batch);
  } else {
    gemv_rows_per_wave<BM, false>(sm, a, lw, batch);
  }
}

// Each workgroup works on one matrix, so the look-up tables it stages in LDS
// serve every block it sees.  BM: accumulators per lane (batch <= BM); RB:
// whole rows per batch (every job of the launch alike), 0 for a row per wave.
// (One kernel per work split: a kernel holding both splits spills.)
template <int BM, int RB>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_kernel(GemvArgs args) {
  __shared__ DecodeSmem<kGemvWaves> sm;
  uint32_t j = 0;
  while (j + 1 < args.n_jobs && blockIdx.x >= args.job[j + 1].wg_first) ++j;
  const GemvJob a = args.job[j];            // one copy, kept in scalar registers
  stage_decode_tables(sm, a.tab);
  __syncthreads();
  const uint32_t lw = blockIdx.x - a.wg_first;
  gemv_split<BM, RB>(sm, a, lw, args.batch);
}

}  // namespace ecco

using namespace ecco;

namespace {

// Checks one matrix and fills its descriptor (all but the workgroup range).
int make_gemv_job(const void* blocks, const void* tables, float tensor_scale, int64_t out_f, int64_t in_f,
                  const uint16_t* x, float* y, int64_t batch, GemvJob* out) {
  if (!blocks || !tables || !x || !y) return ECCO_EINVAL;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < __builtin_huge_valf())) return ECCO_EINVAL;
  if (out_f < 1 || in_f < 128 || in_f % 128 != 0 || batch < 1 || batch > ECCO_GEMV_MAX_BATCH) return ECCO_ESIZE;
  uint64_t n_groups = 0;
  if (out_f >= (1ll << 31) || !group_count((uint64_t)out_f, (uint64_t)(in_f / 128), &n_groups)) return ECCO_ESIZE;
  if (!host_aligned(blocks, 64) || !host_aligned(tables, 256) || !host_aligned(x, 16) || !host_aligned(y, 4))
    return ECCO_EALIGN;
  GemvJob& a = *out;
  a.blocks = static_cast<const uint8_t*>(blocks);
  a.tab = static_cast<const Tables*>(tables);
  a.x = x;
  a.y = y;
  a.out_f = (uint32_t)out_f;
  a.in_f = (uint32_t)in_f;
  a.gpr = (uint32_t)(in_f / 128);
  a.t = tensor_scale;
  // batch 1 with rows of 16, 32 or 64 blocks packs whole rows into a batch (with
  // more batch columns the registers run out for one accumulator per row and
  // column, and those launches go one row per wave)
  const bool whole = batch == 1 && (a.gpr == 16 || a.gpr == 32 || a.gpr == 64);
  // row groups where a row is not a whole number of batches (a row per wave
  // would leave lanes idle, or its waves would each read x at another place);
  // rows of 64k blocks keep a row per wave, which measures a little faster
  const bool groups = !whole && a.gpr % 64u != 0u && a.out_f % 4u == 0u && a.gpr % 16u == 0u &&
                      a.gpr / 16u <= kGemvUnits;
  a.rb = whole ? 64u / a.gpr : groups ? kRowGroups : 0u;
  a.n_units = whole ? (a.out_f * a.gpr + 63u) / 64u : groups ? a.out_f / 4u : a.out_f;
  a.wg_first = a.wg_count = 0;
  return ECCO_OK;
}

// 64-block batches of decode work in a job.
uint64_t gemv_cost(const GemvJob& a) {
  if (a.rb == kRowGroups) return (uint64_t)a.n_units * (a.gpr / 16u);
  return a.rb ? a.n_units : (uint64_t)a.out_f * ((a.gpr + 63u) / 64u);
}

// Splits the workgroups (at most one per CU) among the jobs: one each, then
// each further workgroup to the job whose workgroups carry the most work; a
// job gets no more workgroups than it has units.
void assign_gemv_workgroups(GemvArgs& args, uint32_t cus) {
  uint64_t total = 0;
  for (uint32_t j = 0; j < args.n_jobs; ++j) total += args.job[j].n_units;
  const uint32_t grid = (uint32_t)std::max<uint64_t>(args.n_jobs, std::min<uint64_t>(total, cus));
  for (uint32_t j = 0; j < args.n_jobs; ++j) args.job[j].wg_count = 1;
  for (uint32_t k = args.n_jobs; k < grid; ++k) {
    uint32_t best = 0;
    uint64_t best_load = 0;
    for (uint32_t j = 0; j < args.n_jobs; ++j) {
      const GemvJob& a = args.job[j];
      if (a.wg_count >= a.n_units) continue;
      const uint64_t load = (gemv_cost(a) + a.wg_count - 1) / a.wg_count;
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

// One launch per work split present among the jobs (jobs of one split share
// the GPU's workgroups); launches follow each other on the stream.
int launch_gemv(const GemvArgs& all, void* stream) {
  int cus = 0, rc = check_gfx950(&cus);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 block(kGemvWaves * 64);
  (void)hipGetLastError();
  for (uint32_t rb : {0u, 1u, 2u, 4u, kRowGroups}) {
    GemvArgs args;
    std::memset(&args, 0, sizeof(args));
    args.batch = all.batch;
    for (uint32_t j = 0; j < all.n_jobs; ++j)
      if (all.job[j].rb == rb) args.job[args.n_jobs++] = all.job[j];
    if (args.n_jobs == 0) continue;
    assign_gemv_workgroups(args, (uint32_t)cus);
    const GemvJob& last = args.job[args.n_jobs - 1];
    const dim3 grid(last.wg_first + last.wg_count);
    if (rb == kRowGroups) {
      if (args.batch == 1)
        hipLaunchKernelGGL((gemv_kernel<1, kRowGroups>), grid, block, 0, s, args);
      else if (args.batch <= 2)
        hipLaunchKernelGGL((gemv_kernel<2, kRowGroups>), grid, block, 0, s, args);
      else if (args.batch <= 4)
        hipLaunchKernelGGL((gemv_kernel<4, kRowGroups>), grid, block, 0, s, args);
      else
        hipLaunchKernelGGL((gemv_kernel<8, kRowGroups>), grid, block, 0, s, args);
    } else if (rb == 4)
      hipLaunchKernelGGL((gemv_kernel<1, 4>), grid, block, 0, s, args);
    else if (rb == 2)
      hipLaunchKernelGGL((gemv_kernel<1, 2>), grid, block, 0, s, args);
    else if (rb == 1)
      hipLaunchKernelGGL((gemv_kernel<1, 1>), grid, block, 0, s, args);
    else if (args.batch == 1)
      hipLaunchKernelGGL((gemv_kernel<1, 0>), grid, block, 0, s, args);
    else if (args.batch <= 2)
      hipLaunchKernelGGL((gemv_kernel<2, 0>), grid, block, 0, s, args);
    else if (args.batch <= 4)
      hipLaunchKernelGGL((gemv_kernel<4, 0>), grid, block, 0, s, args);
    else
      hipLaunchKernelGGL((gemv_kernel<8, 0>), grid, block, 0, s, args);
    if (hipGetLastError() != hipSuccess) return ECCO_EHIP;
  }
  return ECCO_OK;
}

}  // namespace

extern "C" int ecco_decode_gemv(const void* blocks, const void* tables, float tensor_scale, int64_t out_f,
                                int64_t in_f, const uint16_t* x, int64_t batch, float* y, void* stream) {
  GemvArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = 1;
  args.batch = (uint32_t)std::max<int64_t>(0, std::min<int64_t>(batch, 1 << 16));
  int rc = make_gemv_job(blocks, tables, tensor_scale, out_f, in_f, x, y, batch, &args.job[0]);
  if (rc) return rc;
  return launch_gemv(args, stream);
}

extern "C" int ecco_decode_gemv_many(const ecco_gemv_job_t* jobs, uint32_t n_jobs, int64_t batch, void* stream) {
  if (!jobs) return ECCO_EINVAL;
  if (n_jobs == 0 || n_jobs > (uint32_t)kMaxGemvJobs) return ECCO_ESIZE;
  GemvArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_jobs = n_jobs;
  args.batch = (uint32_t)std::max<int64_t>(0, std::min<int64_t>(batch, 1 << 16));
  for (uint32_t j = 0; j < n_jobs; ++j) {
    const ecco_gemv_job_t& q = jobs[j];
    if (q.reserved != 0) return ECCO_EINVAL;
    int rc = make_gemv_job(q.blocks_dev, q.tables_dev, q.tensor_scale, q.out_features, q.in_features, q.x_dev,
                           q.y_dev, batch, &args.job[j]);
    if (rc) return rc;
  }
  return launch_gemv(args, stream);
}
