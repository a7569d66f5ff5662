/*
 * ecco.h -- C ABI of libecco, an MI355X (gfx950) implementation of the Ecco
 * entropy-coded block codec for LLM weights and KV caches.
 *
 * Source of the method: the pith.science review of "Ecco: Improving Memory
 * Bandwidth and Capacity for LLMs via Entropy-aware Cache Compression"
 * (arXiv 2505.06901).  Each group of 128 FP16 values is normalised by a
 * per-group FP8 scale derived from a per-tensor FP16-to-FP8 scale (Fig. 4
 * caption), quantised onto one of 64 shared patterns of 15 sorted k-means
 * centroids with index 15 reserved for the scale ("What carries the
 * argument"; "free parameters"), the pattern being chosen by comparing only
 * the group's min and max with each pattern's (same section; compressor,
 * section 4.3), Huffman coded with the shortest of 4 codebooks per pattern
 * whose code lengths are 2..8 bits (referee report, major comment 1), clipped
 * to, or padded with the largest remaining values up to, a fixed 512-bit
 * block ("Core claim"; "free parameters": top-16 outliers, 240 bits at most).
 *
 * ------------------------------------------------------------------------
 * BLOCK FORMAT v1 (64 bytes per group of 128 values)
 * ------------------------------------------------------------------------
 * Bit i of a block is bit (i & 7) of byte (i >> 3).  Integer fields are
 * stored least-significant bit first.
 *
 *   bits   0..5    pattern p            (0..63)
 *   bits   6..7    codebook h           (0..3)
 *   bits   8..15   group scale s8       FP8 E4M3FN of x[i*] * inv_t (signed)
 *   bits  16..E-1  codewords of symbols 0..127 in position order; each
 *                  canonical codeword (RFC 1951 3.2.2 ordering) is written
 *                  most-significant code bit first.  L = total code length.
 *                  Unclipped: E = 16 + L <= 512.  Clipped (16 + L > 512):
 *                  the stream fills bits 16..511 and ends with a proper
 *                  prefix of the first codeword that did not fit; k < 128
 *                  whole codewords are decodable.
 *   bits   E..512-15n-1  zero
 *   bits   512-15(r+1) .. 512-15r-1   outlier record r, r = 0..n-1:
 *                  bits 0..6 = position j, bits 7..14 = FP8 E4M3FN(x_j * inv_t)
 *   n = min(16, floor((512 - E) / 15)) for an unclipped block, 0 if clipped.
 *
 * Encode of a group x[0..127] (FP16 promoted exactly to FP32; every step
 * below is one IEEE binary32 operation, round-to-nearest-even, no FMA):
 *   t      per-tensor scale (amax / 448, see ecco_tensor_scale_from_amax);
 *          inv_t = 1.0f / t computed by the library on the host
 *   i*     = argmax_j |x_j|, lowest j on ties; s8 = FP8(x_i* * inv_t)
 *            (saturating to +-448, round to nearest even, never NaN)
 *   S      = f32(s8) * t; a = |S|
 *   p      = argmin_p (gmin - c_p0*a)^2 + (gmax - c_p14*a)^2 (squares summed
 *            in that order), gmin/gmax over the 127 values j != i*; lowest p
 *   sym_j  = #{k in 0..13 : x_j > m_pk * a}, m_pk = (c_pk + c_p,k+1) * 0.5f;
 *            sym_i* = 15
 *   h      = argmin_h sum_j len[p][h][sym_j]; lowest h on ties
 *   outliers: the n values j != i* of largest |x_j| (lower j first on ties),
 *            record r holding the r-th of them
 * Decode: symbols are read while a whole codeword fits in bits 16..511, at
 * most 128 of them (with an incomplete codebook, reading also stops where
 * no codeword starts the remaining bits); k = the symbols read; value
 * j = fp16(S) for symbol 15, fp16(c[p][sym] * a) otherwise, +0 for j >= k;
 * if k == 128 the n records are applied in order r = 0..n-1:
 * value[j_r] = fp16(f32(v8_r) * t).  Any 512 bits decode.
 *
 * ------------------------------------------------------------------------
 * ACTIVATION FORMAT (64 bytes per group of 64 values, about 8 bits/value)
 * ------------------------------------------------------------------------
 * The 2x format for activations: groups of 64 values ("free parameters":
 * activation group size 64 for a 2x target) coded by the same steps
 * and the same kind of table blob (the low-ratio compressor reuses the
 * high-ratio one's hardware, Fig. 9 caption).  Everything above holds with
 * 128 replaced by 64, except the records: 14 bits each, bits 0..5 = position
 * j, bits 6..13 = FP8 value; bits 512-14(r+1) .. 512-14r-1 hold record r and
 * n = min(16, floor((512 - E) / 14)).  Symmetric like the 4x format: one
 * figure caption mentions zero points, but the pages never define them, so
 * none are stored.
 *
 * ------------------------------------------------------------------------
 * CONVENTIONS
 * ------------------------------------------------------------------------
 * - "_dev" pointers are HIP device memory owned by the caller; "_host"
 *   pointers are host memory owned by the caller.  The library allocates,
 *   frees and synchronises nothing: every device call only enqueues kernels
 *   on `stream` (a hipStream_t, passed as void*; NULL = the default stream)
 *   and returns.  Calls are reentrant; overlapping calls that write the same
 *   memory race.
 * - Return value: ECCO_OK (0) or a negative ECCO_E* code.  Arguments are
 *   checked before anything is enqueued; no C++ exception crosses the ABI.
 * - Alignment: FP16 tensors and row strides 16-byte aligned, blocks 64-byte
 *   aligned, the table blob 256-byte aligned (ECCO_EALIGN otherwise).
 * - Device entry points require a gfx950 device (ECCO_EDEVICE otherwise).
 */
#ifndef ECCO_H
#define ECCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ECCO_GROUP 128
#define ECCO_BLOCK_BYTES 64
#define ECCO_N_PATTERNS 64
#define ECCO_N_CENTROIDS 15
#define ECCO_N_CODEBOOKS 4
#define ECCO_N_SYMBOLS 16
#define ECCO_LEN_MIN 2
#define ECCO_LEN_MAX 8
#define ECCO_GEMV_MAX_BATCH 8
#define ECCO_DECODE_MAX_JOBS 16
#define ECCO_GEMV_MAX_JOBS 16
#define ECCO_AMAX_MAX_JOBS 16

enum {
  ECCO_OK = 0,
  ECCO_EINVAL = -1,   /* null pointer where one is required, bad option value   */
  ECCO_EALIGN = -2,   /* pointer or stride alignment violated                   */
  ECCO_ESIZE = -3,    /* size out of range (see each call)                      */
  ECCO_ETABLES = -4,  /* table blob or table contents invalid                   */
  ECCO_EHIP = -5,     /* a HIP runtime call or kernel launch failed             */
  ECCO_EDEVICE = -6   /* current device is not gfx950                           */
};

/* Device-side counters accumulated by ecco_encode (atomics; caller zeroes). */
typedef struct {
  unsigned long long groups;           /* groups encoded                                */
  unsigned long long clipped_groups;   /* groups with 16 + L > 512                      */
  unsigned long long clipped_values;   /* sum over groups of 128 - k (64 - k)           */
  unsigned long long padded_outliers;  /* sum of n                                      */
  unsigned long long pad_bits;         /* sum of 15 n (14 n in the activation format)   */
  unsigned long long fill_bits;        /* zero bits between stream end and records      */
  unsigned long long nonfinite_groups; /* groups holding Inf/NaN (their blocks are unspecified) */
} ecco_stats_t;

/* Options of ecco_train_patterns; NULL selects the defaults shown. */
typedef struct {
  uint32_t kmeans_iters;  /* Lloyd iterations of the 64-pattern k-means (25)      */
  uint32_t huff_iters;    /* codebook Lloyd iterations per pattern (10)           */
  uint64_t seed;          /* k-means++ seed (0)                                   */
  uint32_t max_groups;    /* use at most this many sample groups, 0 = all (0)     */
  uint32_t threads;       /* host threads, 0 = hardware concurrency (0)           */
  uint32_t n_patterns;    /* distinct patterns learned: 16, 32 or 64, 0 = 64 (0);
                             the blob's 64 slots repeat them (slot p holds
                             pattern p mod n_patterns), so blocks keep the
                             6-bit pattern field and the encoder searches only
                             the distinct ones                                  */
  uint32_t group;         /* values per group of the sample: 128 (weights, KV
                             cache) or 64 (the 2x activation format of
                             ecco_encode_act); 0 = 128 (0)                       */
} ecco_train_opts_t;

/* ---- tables --------------------------------------------------------------
 * The per-tensor side data is an opaque, position-independent blob of
 * ecco_tables_size() bytes: the inputs (centroids, code lengths) plus tables
 * the kernels derive from them (canonical codes, decode look-up table,
 * midpoints).  Build it on the host, then copy the bytes to device memory
 * (256-byte aligned) for the device calls.
 */
size_t ecco_tables_size(void);

/* Build a blob from the per-tensor side data the pages describe: 64 shared
 * patterns of 15 sorted centroids and 4 Huffman codebooks per pattern ("What
 * carries the argument"; "Assumptions & free parameters": S = 64, H = 4),
 * with code lengths of 2..8 bits (referee report, major comment 1).
 * Build it from centroids[64][15] (float32, each exactly representable in
 * FP16, non-decreasing per pattern, within [-1, 1]) and code_len[64][4][16]
 * (each in [2, 8], every codebook a prefix code: Kraft sum at most 1; an
 * incomplete codebook leaves bit strings that no codeword starts, where the
 * decoder stops the stream, see ecco_decode).  Returns ECCO_ETABLES if the
 * contents violate these rules (the blob is then left unspecified),
 * ECCO_EINVAL for NULL pointers.
 * The blob records how many patterns the encoder has to search: the least
 * of 16, 32 and 64 such that every later pattern p has the same first and
 * last centroid as pattern p mod that number (the min/max fitness then ties
 * and the lower pattern wins, so the shorter search gives the same blocks). */
int ecco_tables_build(const float* centroids_host, const uint8_t* code_len_host, void* tables_host);

/* Check a host blob: header, checksum, and the rules of ecco_tables_build. */
int ecco_tables_validate(const void* tables_host);

/* Copy the centroids and code lengths back out of a valid host blob. */
int ecco_tables_get(const void* tables_host, float* centroids_host, uint8_t* code_len_host);

/* Learn tables offline from an FP16 sample (n_values a positive multiple of
 * 128) -- the pages' calibration step, in which patterns and codebooks are
 * learned once, offline, and then kept fixed ("Load-bearing premise";
 * "Assumptions & free parameters": S = 64, H = 4; the pages give no
 * procedure).  The steps taken here: exact 1-D k-means of each normalised
 * group, Lloyd k-means of those 15-vectors into 64 patterns, then per pattern
 * 4 codebooks by Lloyd iterations on code length with optimal 2..8-bit
 * lengths (referee report, major comment 1).  Host only; writes a valid blob
 * to tables_host. */
int ecco_train_patterns(const uint16_t* sample_fp16_host, uint64_t n_values,
                        const ecco_train_opts_t* opts, void* tables_host);

/* Per-tensor scale t = amax / 448 (1 if amax == 0 or not finite): the one
 * scale per tensor that maps FP16 values onto the FP8 range (Fig. 4 caption). */
float ecco_tensor_scale_from_amax(float amax);

/* ---- device calls ---------------------------------------------------------- */

/* amax_dev[0] = max |x| over n_values FP16 values (n_values >= 1; NaN
 * ignored): the tensor's largest magnitude, from which its FP16-to-FP8 scale
 * t is taken (Fig. 4 caption; see ecco_tensor_scale_from_amax).  amax_dev is
 * overwritten. */
int ecco_amax(const uint16_t* x_dev, uint64_t n_values, float* amax_dev, void* stream);

/* One tensor of an ecco_amax_many call: the arguments of ecco_amax. */
typedef struct {
  const uint16_t* x_dev;
  uint64_t n_values;
  float* amax_dev;
} ecco_amax_job_t;

/* The maxima of several tensors (the amax each per-tensor scale is derived
 * from) in two launches in all -- one that zeroes the outputs and one that
 * reads every tensor -- e.g. all matrices of a layer before they are
 * encoded.  Each job follows the rules of ecco_amax; jobs_host (n_jobs in
 * 1..ECCO_AMAX_MAX_JOBS) is read before the call returns.  If any job is
 * invalid the call returns that job's error and enqueues nothing.  Jobs that
 * name the same amax_dev leave there the maximum over all of them.  The
 * workgroups are shared out in proportion to the jobs' sizes.  Results are
 * identical to one ecco_amax call per job. */
int ecco_amax_many(const ecco_amax_job_t* jobs_host, uint32_t n_jobs, void* stream);

/* Encode: each group of 128 FP16 values becomes one self-contained 64-byte
 * block -- FP8 group scale, pattern chosen from the group's min and max,
 * centroid indices coded with the shortest of the pattern's 4 codebooks,
 * overflow clipped and spare bits filled with the largest remaining values
 * ("Core claim"; "What carries the argument"; "Assumptions & free
 * parameters": 128-value groups, 64-byte blocks, up to 16 padded values;
 * compressor of Fig. 9 caption).  The rules are those of the block format
 * above.
 * Encode n_rows x groups_per_row groups.  Group (r, g) is the 128 FP16
 * values at x_dev + r * x_row_stride_elems + g * 128; its block goes to
 * blocks_dev + (r * blk_row_stride_blocks + g) * 64.  Weights [out, in]:
 * n_rows = out, groups_per_row = in / 128.  KV append in [B, H, S, D=128]:
 * n_rows = B * H, groups_per_row = tokens, x_row_stride_elems = S * 128,
 * blk_row_stride_blocks = S, pointers offset to the first new token.
 * tensor_scale must be finite and > 0.  stats_dev may be NULL.
 * ECCO_ESIZE if n_rows or groups_per_row is 0 or >= 2^32, or their product
 * is >= 2^32; ECCO_ESIZE also if n_rows > 1 and a row stride is shorter than
 * a row. */
int ecco_encode(const uint16_t* x_dev, uint64_t n_rows, uint64_t groups_per_row,
                uint64_t x_row_stride_elems, uint64_t blk_row_stride_blocks,
                const void* tables_dev, float tensor_scale, void* blocks_dev,
                ecco_stats_t* stats_dev, void* stream);

/* One tensor of an ecco_encode_many call: the arguments of ecco_encode. */
typedef struct {
  const uint16_t* x_dev;
  void* blocks_dev;
  const void* tables_dev;
  ecco_stats_t* stats_dev;    /* may be NULL */
  uint64_t n_rows;
  uint64_t groups_per_row;
  uint64_t x_row_stride_elems;
  uint64_t blk_row_stride_blocks;
  float tensor_scale;
  uint32_t reserved;          /* must be 0 */
} ecco_encode_job_t;

/* Encode several tensors, each with its own tables and scale, in one launch
 * -- e.g. the K and V rows a decode step appends to the caches.  Each job
 * follows the rules of ecco_encode; jobs_host (n_jobs in
 * 1..ECCO_DECODE_MAX_JOBS) is read before the call returns.  If any job is
 * invalid the call returns that job's error and enqueues nothing.  Blocks of
 * different jobs must not overlap (statistics buffers may be shared).  The
 * workgroups are shared out in proportion to the jobs' sizes.  Results are
 * identical to one ecco_encode call per job. */
int ecco_encode_many(const ecco_encode_job_t* jobs_host, uint32_t n_jobs, void* stream);

/* Decode: every block is expanded back to 128 FP16 values on load, from its
 * own bits and the tensor's side data alone ("The pith"; "Core claim";
 * decompressor of Fig. 8 caption): codewords read while they fit (and,
 * with an incomplete codebook, while one starts the remaining bits), values
 * c * |S| or S, positions past the last codeword read +0, then the padded
 * values, exactly as the block format above states.
 * The inverse layout of ecco_encode; group (r, g) is written to
 * y_dev + r * y_row_stride_elems + g * 128.  Every block decodes (the
 * decoder is total on arbitrary bits).  Same size rules as ecco_encode. */
int ecco_decode(const void* blocks_dev, uint64_t n_rows, uint64_t groups_per_row,
                uint64_t blk_row_stride_blocks, uint64_t y_row_stride_elems,
                const void* tables_dev, float tensor_scale, uint16_t* y_dev, void* stream);

/* Activation format: encode / decode groups of 64 values.  Arguments, layout
 * (with 128 replaced by 64: group (r, g) is the 64 FP16 values at
 * x_dev + r * x_row_stride_elems + g * 64), size rules, statistics and errors
 * as for ecco_encode / ecco_decode.  The tables should come from
 * ecco_train_patterns with group = 64; any valid blob is accepted. */
int ecco_encode_act(const uint16_t* x_dev, uint64_t n_rows, uint64_t groups_per_row,
                    uint64_t x_row_stride_elems, uint64_t blk_row_stride_blocks,
                    const void* tables_dev, float tensor_scale, void* blocks_dev,
                    ecco_stats_t* stats_dev, void* stream);
int ecco_decode_act(const void* blocks_dev, uint64_t n_rows, uint64_t groups_per_row,
                    uint64_t blk_row_stride_blocks, uint64_t y_row_stride_elems,
                    const void* tables_dev, float tensor_scale, uint16_t* y_dev, void* stream);

/* Decode by the pages' parallel method (Fig. 8 caption, 64-way parallel
 * decoder): one wavefront per block, the codeword stream cut into 62 segments
 * of 8 bits, each segment decoded speculatively from all 8 start offsets, the
 * true entries resolved by following the exit offsets from bit 16, then each
 * segment emitted at its running symbol count.  Arguments, layout, rules and
 * output as ecco_decode, and the same output bit for bit; it does about 16
 * times the table look-ups per block, so ecco_decode is the one to use. */
int ecco_decode_speculative(const void* blocks_dev, uint64_t n_rows, uint64_t groups_per_row,
                            uint64_t blk_row_stride_blocks, uint64_t y_row_stride_elems,
                            const void* tables_dev, float tensor_scale, uint16_t* y_dev, void* stream);

/* Decode by speculation over a few long segments (the pages' overlapping
 * segments and merge, Fig. 8 caption and "What carries the argument", with
 * fewer, longer segments): lanes_per_block (2, 4 or 8) lanes share a block,
 * each decoding 496 / lanes_per_block stream bits from their first bit as if
 * a codeword started there; a lane whose true entry (the exit of the segment
 * before it) differs decodes again from it until its path meets a codeword
 * boundary of the first one; the symbol counts, scanned over the block's
 * lanes, place each segment's symbols.  Arguments, layout, rules and output
 * as ecco_decode, and the same output bit for bit; ECCO_EINVAL for another
 * lanes_per_block.  A comparison decoder: each block costs more look-ups and
 * LDS traffic than in ecco_decode, which is the one to use. */
int ecco_decode_segmented(const void* blocks_dev, uint64_t n_rows, uint64_t groups_per_row,
                          uint64_t blk_row_stride_blocks, uint64_t y_row_stride_elems,
                          const void* tables_dev, float tensor_scale, uint16_t* y_dev,
                          uint32_t lanes_per_block, void* stream);

/* One tensor of an ecco_decode_many call: the arguments of ecco_decode. */
typedef struct {
  const void* blocks_dev;
  uint16_t* y_dev;
  const void* tables_dev;
  uint64_t n_rows;
  uint64_t groups_per_row;
  uint64_t blk_row_stride_blocks;
  uint64_t y_row_stride_elems;
  float tensor_scale;
  uint32_t reserved;          /* must be 0 */
} ecco_decode_job_t;

/* Decode several tensors, each with its own tables and scale, in one launch
 * -- e.g. every weight matrix of a decoder layer.  Blocks carry everything
 * their decode needs except the per-tensor side data ("Core claim"), so
 * tensors with different tables can share one launch.  Each job follows the
 * rules of ecco_decode; jobs_host (n_jobs in 1..ECCO_DECODE_MAX_JOBS) is read
 * before the call returns.  If any job is invalid the call returns that
 * job's error and enqueues nothing.  Outputs of different jobs must not
 * overlap.  The GPU's workgroups are shared out in proportion to the jobs'
 * sizes, so small tensors are decoded beside large ones rather than after
 * them. */
int ecco_decode_many(const ecco_decode_job_t* jobs_host, uint32_t n_jobs, void* stream);

/* Fused decode + GEMV -- the decode-phase matrix-vector product whose weight
 * traffic the format cuts (Fig. 12 caption: memory requests of a GEMM
 * kernel; Fig. 11 caption and "If this is right": the gain is largest at
 * small batch): the blocks are decoded on load and never written out.
 * y[b][o] = sum_i W[o][i] * x[b][i] with W the decoded
 * FP16 weights, products and sums in FP32 (plain FMA on the vector ALUs).
 * blocks_dev holds W as [out_features][in_features / 128] blocks; x_dev is
 * [batch][in_features] FP16; y_dev is [batch][out_features] FP32 and is
 * overwritten.  ECCO_ESIZE unless in_features is a positive multiple of 128,
 * out_features in 1 .. 2^31 - 1, 1 <= batch <= ECCO_GEMV_MAX_BATCH and
 * out_features * in_features / 128 < 2^32. */
int ecco_decode_gemv(const void* blocks_dev, const void* tables_dev, float tensor_scale,
                     int64_t out_features, int64_t in_features,
                     const uint16_t* x_dev, int64_t batch, float* y_dev, void* stream);

/* One matrix of an ecco_decode_gemv_many call: the arguments of
 * ecco_decode_gemv except the batch, which all jobs share. */
typedef struct {
  const void* blocks_dev;
  const void* tables_dev;
  const uint16_t* x_dev;
  float* y_dev;
  int64_t out_features;
  int64_t in_features;
  float tensor_scale;
  uint32_t reserved;          /* must be 0 */
} ecco_gemv_job_t;

/* Fused decode + GEMV of several matrices in one launch, each with its own
 * blocks, tables, scale, x and y -- e.g. the q, k and v projections of a
 * layer, which read the same x.  Each job follows the rules of
 * ecco_decode_gemv with the common batch; jobs_host (n_jobs in
 * 1..ECCO_GEMV_MAX_JOBS) is read before the call returns.  If any job is
 * invalid the call returns that job's error and enqueues nothing.  The y
 * outputs of different jobs must not overlap.  Jobs whose rows split the same
 * way -- at batch 1, rows of 16, 32 or 64 blocks pack 4, 2 or 1 whole rows
 * into a 64-block batch; otherwise one row per wave -- share one launch, the
 * GPU's workgroups shared out in proportion to their decode work; each other
 * split present takes a launch of its own, in order on the stream.  Results
 * are identical to one ecco_decode_gemv call per job. */
int ecco_decode_gemv_many(const ecco_gemv_job_t* jobs_host, uint32_t n_jobs, int64_t batch, void* stream);

/* Decode-phase attention over Ecco-compressed K and V caches, one query token
 * per sequence -- the consumer of the online KV codec ("Core claim": KV cache
 * blocks decompressed on load).  For b < B, kv head h < H_kv and g < G (query
 * heads per kv head, query head hq = h * G + g):
 *   s_t   = scale * sum_d q[b][hq][d] * K[b][h][t][d]        t < S
 *   p_t   = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
 *   out[b][hq][d] = sum_t p_t * V[b][h][t][d]
 * with K and V the decoded FP16 values; products and sums in FP32.
 * k_blocks_dev / v_blocks_dev: [B][H_kv][kv_stride_tokens] blocks (the layout
 * ecco_encode writes for a [B, H_kv, S_max, 128] cache, kv_stride_tokens =
 * S_max >= S); q_dev: [B][H_kv * G][128] FP16; out_dev: [B][H_kv * G][128]
 * FP32, overwritten.  workspace_dev (256-byte aligned) holds
 * ecco_attention_workspace_size(B, H_kv, G, S) bytes of caller memory that
 * the call uses for scores, per-unit partial sums and the maxima and weight
 * sums of the softmax (taken per 64- and 128-token block, combined at the
 * end); its contents are unspecified afterwards.  ECCO_ESIZE unless B, H_kv, S >= 1, G is 1, 2, 4 or 8,
 * B, H_kv and B * H_kv are below 2^20, S is below 2^24, S <= kv_stride_tokens
 * < 2^32 and B * H_kv * kv_stride_tokens < 2^32.  The workspace size is 0 for
 * B, H_kv or G beyond those limits. */
size_t ecco_attention_workspace_size(uint64_t batch, uint64_t kv_heads, uint64_t group, uint64_t seq);
int ecco_attention_decode(const void* k_blocks_dev, const void* k_tables_dev, float k_scale,
                          const void* v_blocks_dev, const void* v_tables_dev, float v_scale,
                          const uint16_t* q_dev, uint64_t batch, uint64_t kv_heads, uint64_t group,
                          uint64_t seq, uint64_t kv_stride_tokens, float scale,
                          void* workspace_dev, float* out_dev, void* stream);

/* ecco_attention_decode without the workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The workspace contents go to
 * a static device array of ECCO_ATTENTION_NOALLOC_MAX_WORKSPACE bytes that
 * the library holds on each GPU it runs on until the process ends; the call
 * allocates and frees nothing.  Everything else -- arguments, layout,
 * results, errors -- is as for ecco_attention_decode; in addition
 * ECCO_ESIZE when ecco_attention_workspace_size(B, H_kv, G, S) exceeds
 * ECCO_ATTENTION_NOALLOC_MAX_WORKSPACE, and ECCO_EHIP if the array's device
 * address cannot be obtained.  Calls on one GPU share its array: calls that
 * overlap on that GPU (different streams, or host threads) race, so a
 * caller orders them on one stream.  Every byte a call reads from the array
 * it has written earlier in the same call, so nothing needs clearing. */
#define ECCO_ATTENTION_NOALLOC_MAX_WORKSPACE (64ull << 20)
int ecco_attention_decode_noalloc(const void* k_blocks_dev, const void* k_tables_dev, float k_scale,
                                  const void* v_blocks_dev, const void* v_tables_dev, float v_scale,
                                  const uint16_t* q_dev, uint64_t batch, uint64_t kv_heads, uint64_t group,
                                  uint64_t seq, uint64_t kv_stride_tokens, float scale, float* out_dev,
                                  void* stream);

const char* ecco_strerror(int code);

/* Library version string, e.g. "ecco 1.0 (format v1, gfx950)". */
const char* ecco_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ECCO_H */
