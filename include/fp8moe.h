/*
 * fp8moe.h -- C ABI of the MI355X (gfx950) FP8 MoE quantization and grouped-GEMM library.
 *
 * What the library computes
 *   Dynamic FP8 quantization as one fused pass (absolute max -> scale -> apply ->
 *   clip -> cast) in rowwise, colwise and MXFP8 (1x32 blocks, e8m0 scales)
 *   forms, over the e4m3fn (max 448) and e4m3fnuz (max 240) codecs, feeding an
 *   offset-routed grouped GEMM for the forward, dgrad and wgrad products of an
 *   MoE expert layer.  Sources (cited by page and section):
 *     [P1] AI Trends summary (aitrends.kr/articles/95981) of the PyTorch post
 *          "FP8 Training on AMD GPUs with TorchTitan and TorchAO".
 *     [P2] AI Trends summary (aitrends.kr/articles/16888) of the TorchAO MXFP8
 *          MoE training post on Llama4 Scout.
 *     [P3] aihirek.info, "Az AMD GPU-kon is gyorsult az FP8-as PyTorch-tréning".
 *     [P4] aixai.ru blog post on FP8 training on AMD with TorchTitan.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer allocated by the caller; the
 *     library allocates no device memory, keeps no per-call state and never
 *     takes ownership of a buffer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on that stream; none synchronizes it.  Results are
 *     visible once the caller synchronizes the stream.
 *   - Layouts are row-major ("phys [a][b]": b contiguous).  bf16 inputs are
 *     passed as their 16-bit patterns; FP8 data and e8m0 scales are bytes.
 *   - Every argument check the host can do (null pointers, enums, negative
 *     sizes, alignment, divisibility) runs BEFORE any HIP call and returns a
 *     non-zero status; nothing is then enqueued.  FP8MOE_ERR_LAUNCH reports a
 *     failed launch.  Device-resident data (the offsets) is not validated; it is
 *     read with the clamping rule below, so malformed offsets cannot cause an
 *     out-of-bounds access.  Device faults surface at the caller's synchronize.
 *   - Group offsets `offs[n_groups]` (int32, device) are the inclusive
 *     cumulative row counts of the groups (experts).  Group e covers rows
 *     [hi(e-1), hi(e)), hi(e) = max(hi(e-1), clamp(offs[e], 0, rows)),
 *     hi(-1) = 0: groups are disjoint, a decreasing entry gives an empty group,
 *     and rows at or past hi(n_groups-1) belong to no group.  The host never
 *     reads the offsets.  [P1 Details, MoE paragraph: tokens placed per expert
 *     by offsets; P4 "MoE: почему DeepSeek-V3 ломал пайплайн".]
 *   - Scales.  fp32 scales are multipliers: q ~= x * s with s = fmax / max(amax,
 *     1e-12f), computed with an IEEE fp32 division; dequantized value = dec(q)/s.
 *     e8m0 scales are dequantization factors 2^(code-127): dequantized value =
 *     dec(q) * 2^(code-127).
 *   - Rounding: y = fp32(x * s) (round to nearest even), clamp to
 *     [-fmax, fmax], then round to the nearest FP8 value, ties to the even code.
 *     e4m3fn keeps the sign of a zero result (0x80); e4m3fnuz has one unsigned
 *     zero and never emits 0x80.  No subnormal is flushed.
 *   - Calls on different streams may run concurrently from several host
 *     threads.  The only mutable library state is the device array the
 *     single-pass colwise quantizer exchanges column maxima through (see
 *     quantize_colwise: its values are tagged per call, so overlapping calls
 *     stay correct) and that quantizer's poll budget and chunk height, test
 *     hooks (fp8moe_set_colwise_poll_budget, fp8moe_set_colwise_chunk_rows).
 *     Everything else a call needs is in
 *     its arguments.
 */
#ifndef FP8MOE_H
#define FP8MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FP8MOE_OK 0
#define FP8MOE_ERR_NULL 1          /* a required pointer is NULL */
#define FP8MOE_ERR_SHAPE 2         /* a size is negative or sizes are inconsistent */
#define FP8MOE_ERR_ENUM 3          /* an enum argument is out of range */
#define FP8MOE_ERR_ALIGN 4         /* a pointer, leading dimension or size violates its alignment */
#define FP8MOE_ERR_UNSUPPORTED 5   /* a valid combination this library does not implement */
#define FP8MOE_ERR_LAUNCH 6        /* the HIP runtime rejected a launch */
#define FP8MOE_ERR_DEVICE 7        /* a HIP device query failed */
#define FP8MOE_ERR_SCRATCH 8       /* the allocation-free entry point's fixed scratch is too small */

/* FP8 codecs.  e4m3fn: OCP, bias 7, max 448, NaN 0x7F/0xFF, signed zero.
 * e4m3fnuz: bias 8, max 240, no NaN/Inf among finite codes, unsigned zero.
 * [P1 Details, e4m3fnuz property table; P1 glossary "FNUZ"; P3 "Az AMD
 * FP8-formátumának támogatása"; P4 "Тихая порча градиентов: проблема формата FNUZ".] */
#define FP8MOE_E4M3FN 0
#define FP8MOE_E4M3FNUZ 1

/* MX shared-exponent rule X for a 1x32 block with |x| max `amax` (e8m0 code X+127):
 * FLOOR_OCP: X = floor(log2 amax) - 8 (OCP MX rule for e4m3; values above
 *            448*2^X saturate in the clamp).   CEIL: the smallest X with
 * amax*2^-X <= 448.  amax == 0 gives X = -127.  X is clamped to [-127, 127].
 * [P2 Details, MXFP8 data/scale layout diagram: e4m3 data, one e8m0 scale per 1x32 block.] */
#define FP8MOE_MX_FLOOR_OCP 0
#define FP8MOE_MX_CEIL 1

/* e8m0 scale layouts of quantize_mx.  A scale matrix has R rows (the rows of
 * the operand that a GEMM contracts along) and NB = L / 32 blocks per row:
 *   ROWS: row-major, byte (r, b) at r * NB + b.
 *   K4:   the four blocks of one 128-wide contraction stage of all rows
 *         together: byte (r, b) at ((b / 4) * R + r) * 4 + b % 4, size
 *         4 * R * ceil(NB / 4); bytes of blocks NB .. 4 ceil(NB / 4) - 1 are
 *         written as 0.  One GEMM stage then reads its scales as one
 *         contiguous run per operand tile instead of one word per row.
 * [P2 Details, MXFP8 data/scale layout diagram: one e8m0 scale per 1x32 block;
 * the K4 arrangement is this library's choice for its GEMM.] */
#define FP8MOE_MX_LAYOUT_ROWS 0
#define FP8MOE_MX_LAYOUT_K4 1

/* grouped GEMM modes */
#define FP8MOE_GROUPED_M 0         /* 2D x 3D -> 2D: forward and dgrad */
#define FP8MOE_GROUPED_K 1         /* 2D x 2D -> 3D: wgrad, contracting over tokens */

/* operand formats */
#define FP8MOE_OPD_E4M3FN 0
#define FP8MOE_OPD_E4M3FNUZ 1
#define FP8MOE_OPD_BF16 2

/* scale kinds */
#define FP8MOE_SCALE_F32 0         /* fp32 multipliers (divide in the epilogue) */
#define FP8MOE_SCALE_E8M0 1        /* e8m0 per 32-block along the contraction (MXFP8) */
#define FP8MOE_SCALE_NONE 2        /* unscaled bf16 operands */
#define FP8MOE_SCALE_E8M0_K4 3     /* e8m0 as SCALE_E8M0, in the K4 layout of quantize_mx */

/* output dtypes */
#define FP8MOE_OUT_BF16 0          /* round to nearest even */
#define FP8MOE_OUT_F32 1

/*
 * quantize_rowwise -- one fp32 scale per row, over the last dimension.
 *   [P1 Details: rowwise FP8 recipe and fused quantization kernels; P4 "Скейлы:
 *   от тензора до микроблока" (rowwise granularity); P4 "Три уровня оптимизации
 *   Triton-ядер" (one fused absmax/scale/clip/cast pass; expert weights quantized
 *   by one kernel parallel over experts and output-dimension blocks).]
 *   Expert weights W[E][N][K] are passed as rows = E*N, giving the per-expert
 *   output-column scales [E][N] the grouped GEMM takes.
 *   x      bf16 [rows][ld_x] (only the first `cols` of each row are read)
 *   q      u8   [rows][cols]   FP8 codes (written)
 *   scale  f32  [rows]         s = fmax/max(amax, 1e-12f) (written)
 *   Requires: rows, cols >= 0; ld_x >= cols; cols % 8 == 0; ld_x % 8 == 0;
 *   x and q 16-byte aligned, scale 4-byte aligned.
 */
int quantize_rowwise(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                     int codec, void *q, float *scale, void *stream);

/*
 * swiglu_quantize_rowwise -- the SwiGLU activation between the two expert
 * GEMMs, fused with the rowwise quantization of its output for the W2 GEMM.
 *   [P1 Details: the MoE layer's grouped GEMMs on dynamically quantized
 *   operands, fused quantization kernels; P4 "MoE" (routed experts between two
 *   grouped GEMMs) and "Три уровня оптимизации Triton-ядер" (quantization fused
 *   into the kernel that produces the tensor).]
 *   h1     bf16 [rows][ld_h1]  W1's output: gate in columns [0, F), up in [F, 2F)
 *   a2     bf16 [rows][F]      bf16(silu(gate) * up), silu(g) = g / (1 + e^-g),
 *                              fp32 arithmetic, round to nearest even (written)
 *   q      u8   [rows][F]      FP8 codes of a2, as quantize_rowwise(a2) (written), or
 *                              NULL together with scale: a2 only (for a caller that
 *                              quantizes a2 another way, e.g. MXFP8)
 *   scale  f32  [rows]         as quantize_rowwise(a2) (written)
 *   Requires: rows, F >= 0; ld_h1 >= 2F; F % 8 == 0; ld_h1 % 8 == 0; h1, a2 and
 *   q 16-byte aligned, scale 4-byte aligned.  The caller owns every buffer.
 */
int swiglu_quantize_rowwise(const void *h1_bf16, int64_t rows, int64_t F, int64_t ld_h1,
                            int codec, void *a2_bf16, void *q, float *scale, void *stream);

/*
 * swiglu_backward_quantize_rowwise -- the gradient of W1's output through the
 * SwiGLU, fused with its rowwise quantization for the W1 dgrad GEMM.
 *   [as swiglu_quantize_rowwise]
 *   da2    bf16 [rows][F]      gradient of a2 (the W2 dgrad output)
 *   h1     bf16 [rows][ld_h1]  as above
 *   dh1    bf16 [rows][2F]     [bf16(da2 up s (1 + g (1 - s))) | bf16(da2 g s)],
 *                              s = sigmoid(gate), fp32 arithmetic (written)
 *   q      u8   [rows][2F]     FP8 codes of dh1, as quantize_rowwise(dh1) (written), or
 *                              NULL together with scale: dh1 only
 *   scale  f32  [rows]         as quantize_rowwise(dh1) (written)
 *   Requires: as swiglu_quantize_rowwise, and da2 16-byte aligned.
 */
int swiglu_backward_quantize_rowwise(const void *da2_bf16, const void *h1_bf16, int64_t rows,
                                     int64_t F, int64_t ld_h1, int codec, void *dh1_bf16,
                                     void *q, float *scale, void *stream);

/*
 * quantize_tensorwise -- one fp32 scale for the whole tensor: the coarsest and
 * fastest scaling granularity, next to rowwise, blockwise and MXFP8.
 *   [P4 "Скейлы: от тензора до микроблока" (one scale per tensor); P4 FAQ
 *   (tensorwise is faster and coarser than rowwise); P3, the four scaling
 *   strategies TorchAO and TorchTitan support.]
 *   The rowwise recipe with every element as the one reduction set:
 *   s = fmax/max(amax, 1e-12f), codes = enc(clamp(fp32(x*s))).
 *   x       bf16 [batch][rows][cols], contiguous
 *   q       u8   [batch*rows][cols]    row-major codes, or NULL (written)
 *   q_t     u8   phys [batch][cols][ld_q]  the same codes transposed, as
 *           quantize_colwise lays them out for the backward GEMMs, or NULL;
 *           bytes [rows, ld_q) of each output row untouched (written)
 *   scale   f32  [n_scale]  every entry s (written).  Size it as the fp32 scale
 *           vector grouped_mm_scaled takes for this operand (rows of A, E*N of
 *           3D weights, n_groups*cols of a transposed operand): the grouped GEMM
 *           then runs tensorwise with no change.
 *   workspace  device memory of quantize_tensorwise_workspace_bytes() bytes,
 *           owned by the caller; contents on entry do not matter
 *   Requires: batch >= 1, rows, cols >= 0, n_scale >= 1, cols % 8 == 0; x, q,
 *   q_t 16-byte aligned; with q_t: ld_q >= rows, ld_q % 16 == 0.  Two or three
 *   kernels (maxima, row-major cast + broadcast, transposed cast), no allocation.
 */
int quantize_tensorwise(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols, int codec,
                        void *q, void *q_t, int64_t ld_q, float *scale, int64_t n_scale,
                        void *workspace, void *stream);

/* Workspace bytes quantize_tensorwise needs (a fixed size). */
int64_t quantize_tensorwise_workspace_bytes(void);

/*
 * quantize_blockwise -- one fp32 scale per fixed tile: 1 x 128 (block_rows = 1)
 * for activations, 128 x 128 (block_rows = 128) for weights.
 *   [P4 "Скейлы: от тензора до микроблока" (a scale per fixed-size tile,
 *   between rowwise and MXFP8; blockwise kernels for MI300 and MI350); P3, the
 *   four scaling strategies.  The pages give no tile shape.]
 *   Each tile (the last of a row or column range may be partial) follows the
 *   rowwise recipe: s = fmax/max(amax, 1e-12f), codes = enc(clamp(fp32(x*s))).
 *   x      bf16 [batch][rows][cols], contiguous
 *   q      u8   [batch][rows][cols] (written)
 *   scale  f32  [batch][ceil(rows/block_rows)][ceil(cols/128)] (written)
 *   Requires: batch >= 1, rows, cols >= 0, block_rows 1 or 128, cols % 8 == 0;
 *   x and q 16-byte aligned, scale 4-byte aligned.
 */
int quantize_blockwise(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                       int block_rows, int codec, void *q, float *scale, void *stream);

/*
 * grouped_mm_blockwise -- GROUPED_M (2D x 3D -> 2D) over blockwise-scaled FP8
 * operands: out[m][n] = sum over 128-wide contraction blocks kb of
 * (sum of a[m][k] b[e][n][k] over kb) / (a_scale[m][kb] * b_scale[e][n/128][kb]),
 * e the group of row m.
 *   [as quantize_blockwise; P1 Details (the grouped GEMM over an offsets tensor).]
 *   a        e4m3fn [M][K]            from quantize_blockwise(block_rows = 1)
 *   a_scale  f32 [M][ceil(K/128)]
 *   b        e4m3fn [n_groups][N][K]  from quantize_blockwise(batch = n_groups, block_rows = 128)
 *   b_scale  f32 [n_groups][ceil(N/128)][ceil(K/128)]
 *   offs     int32 [n_groups], groups as in grouped_mm_scaled (rows of no group untouched)
 *   out      bf16 (round to nearest even) or f32 [M][N] (written)
 *   Per block, the FP8 products are summed in fp32 (MFMA), and the partial sum is
 *   scaled and added to an fp32 running result.  Requires: a_fmt = b_fmt =
 *   FP8MOE_OPD_E4M3FN (others: FP8MOE_ERR_UNSUPPORTED), K % 16 == 0, a and b
 *   16-byte aligned.
 */
int grouped_mm_blockwise(const void *a, int a_fmt, const float *a_scale, const void *b, int b_fmt,
                         const float *b_scale, const int32_t *offs, int32_t n_groups, int64_t M,
                         int64_t N, int64_t K, void *out, int out_dtype, void *stream);

/*
 * quantize_blockwise_tokens -- the blockwise tiles of a token-major operand of
 * the weight gradient (dY, X), which contracts over tokens: one fp32 scale per
 * column and 128-token block, the blocks restarting at every group start (a
 * block never spans two experts; a group's last block may be partial).
 *   [as quantize_blockwise]
 *   x      bf16 [tokens][cols]
 *   offs   int32 [n_groups], groups as in quantize_colwise
 *   q_t    u8 phys [cols][ld_q]: q_t[c][t] = code of x[t][c] (tokens of no group untouched) (written)
 *   scale  f32 [blockwise_token_blocks_bound(tokens, n_groups)][cols]: row b = the b-th
 *          block in group order; rows past the last block untouched (written)
 *   Requires: cols % 8 == 0, ld_q >= tokens, ld_q % 16 == 0; x and q_t 16-byte aligned.
 */
int quantize_blockwise_tokens(const void *x_bf16, int64_t tokens, int64_t cols, const int32_t *offs,
                              int32_t n_groups, int codec, void *q_t, int64_t ld_q, float *scale,
                              void *stream);

/* Most 128-token blocks a grouping of `tokens` tokens into n_groups groups can have
 * (-1: invalid sizes). */
int64_t blockwise_token_blocks_bound(int64_t tokens, int32_t n_groups);

/*
 * grouped_mm_blockwise_k -- GROUPED_K (2D x 2D -> 3D, the weight gradient) over
 * blockwise e4m3fn operands from quantize_blockwise_tokens:
 * out[e][n][k] = sum over the 128-token blocks b of group e of
 * (sum of a_t[n][t] b_t[k][t] over b) / (a_scale[b][n] * b_scale[b][k]).
 *   a_t phys [N][ld], b_t phys [K][ld], a_scale [blocks][N], b_scale [blocks][K];
 *   out bf16 or f32 [n_groups][N][K] (written; an empty group gives zeros).
 *   Blocks whose first token is 16-byte aligned in the transposed rows move 16
 *   bytes at a time, others byte by byte.  Requires: ld >= tokens, ld % 16 == 0,
 *   a_t and b_t 16-byte aligned.
 */
int grouped_mm_blockwise_k(const void *a_t, const float *a_scale, const void *b_t,
                           const float *b_scale, const int32_t *offs, int32_t n_groups,
                           int64_t tokens, int64_t ld, int64_t N, int64_t K, void *out,
                           int out_dtype, void *stream);

/*
 * moe_route -- group the token slots of a top-k routing by expert: per-expert
 * counts, the offsets tensor the grouped GEMMs take, and for every slot the
 * grouped row it lands in (and the inverse map).
 *   [P1 Details (the grouped GEMM over token groups split by an offsets
 *   tensor); P4 "MoE" (tokens routed to experts, grouped GEMMs over the routed
 *   rows); P2 Details (groups padded to the MX block size).]
 *   Slot i = t*topk + j is token t's j-th choice.  Within an expert the slots
 *   keep their order (a stable grouping); each group's row count is rounded up
 *   to a multiple of `pad` (1: no padding), its padding rows after its slots.
 *   An id outside [0, n_experts) drops its slot: not counted, dest -1.
 *   expert_ids  int32 [tokens][topk]
 *   counts      int32 [n_experts]   valid slots per expert (written)
 *   offs        int32 [n_experts]   inclusive cumsum of the padded counts (written)
 *   dest        int32 [tokens*topk] grouped row of each slot, or -1 (written)
 *   src         int32 [moe_route_rows_bound(...)]  slot whose row lands at each
 *               grouped row; -1 for padding and for rows past offs[n_experts-1] (written)
 *   workspace   device memory of moe_route_workspace_bytes(tokens*topk, n_experts)
 *               bytes, owned by the caller; contents on entry do not matter
 *   Requires: tokens >= 0, topk >= 1, 1 <= n_experts, pad >= 1, tokens*topk and
 *   the rows bound within int32; int32 pointers 4-byte aligned.  More than
 *   1024 experts: FP8MOE_ERR_UNSUPPORTED.  Three kernels, no allocation.
 */
int moe_route(const int32_t *expert_ids, int64_t tokens, int32_t topk, int32_t n_experts,
              int32_t pad, int32_t *counts, int32_t *offs, int32_t *dest, int32_t *src,
              void *workspace, void *stream);

/*
 * moe_route_noalloc -- moe_route for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, results and kernels, with the
 * workspace replaced by a fixed scratch array the library owns on each GPU
 * (4 MiB, held until the process ends; routings whose
 * moe_route_workspace_bytes exceed it return FP8MOE_ERR_SCRATCH before any
 * HIP call).  It calls no allocating routine.  Every call on a GPU shares
 * that GPU's scratch, which keeps the last call's contents (a call rewrites
 * all it uses, so nothing needs clearing): calls that overlap on one GPU race.
 * The scratch's device address is looked up once per device, at the first
 * call with that device current.
 */
int moe_route_noalloc(const int32_t *expert_ids, int64_t tokens, int32_t topk, int32_t n_experts,
                      int32_t pad, int32_t *counts, int32_t *offs, int32_t *dest, int32_t *src,
                      void *stream);

/* Workspace bytes moe_route needs for `slots` = tokens*topk slots (-1: invalid sizes). */
int64_t moe_route_workspace_bytes(int64_t slots, int32_t n_experts);

/* Most grouped rows a routing of `slots` slots can need: slots + n_experts*(pad-1)
 * (-1: invalid sizes or beyond int32).  The length of moe_route's src. */
int64_t moe_route_rows_bound(int64_t slots, int32_t n_experts, int32_t pad);

/*
 * moe_permute -- gather token rows into the grouped layout.
 *   [as moe_route]
 *   x      bf16 [tokens][cols]
 *   src    int32 [rows_out]   as written by moe_route
 *   xg     bf16 [rows_out][cols]  row r = x[src[r] / topk], zeros where src[r] < 0
 *          or src[r] >= tokens*topk (written)
 *   Requires: cols % 8 == 0; x and xg 16-byte aligned, src 4-byte aligned.
 */
int moe_permute(const void *x_bf16, int64_t tokens, int64_t cols, int32_t topk,
                const int32_t *src, int64_t rows_out, void *xg_bf16, void *stream);

/*
 * moe_permute_quantized -- gather rowwise-quantized token rows (FP8 codes and
 * their fp32 row scales) into the grouped layout: quantize the tokens once,
 * then move one byte per element, instead of gathering bf16 rows and
 * quantizing every routed copy.
 *   [as moe_route; the rowwise recipe as quantize_rowwise]
 *   q        u8  [tokens][cols]   codes of quantize_rowwise(x)
 *   scale    f32 [tokens]         its row scales
 *   src      int32 [rows_out]     as written by moe_route
 *   qg       u8  [rows_out][cols] row r = q[src[r] / topk]; zero codes for a padding
 *            row (src[r] < 0 or >= tokens*topk) (written)
 *   scale_g  f32 [rows_out]       scale[src[r] / topk]; for a padding row the scale the
 *            rowwise recipe gives an all-zero row, fmax/1e-12f (written)
 *   With that padding rule the result has the bits of quantize_rowwise applied to
 *   moe_permute(x).  Requires: cols % 16 == 0; q and qg 16-byte aligned; src,
 *   scale, scale_g 4-byte aligned.
 */
int moe_permute_quantized(const void *q, const float *scale, int64_t tokens, int64_t cols,
                          int32_t topk, const int32_t *src, int64_t rows_out, int codec,
                          void *qg, float *scale_g, void *stream);

/*
 * moe_permute_rowwise -- gather token rows into the grouped layout and
 * quantize them rowwise in the same pass: one read of each routed token row
 * gives the gathered bf16 row (kept for the backward's colwise operand) and
 * its FP8 codes and scale for the forward GEMM.
 *   [as moe_route; P1 Details, MoE paragraph, and P4 "Три уровня
 *   оптимизации Triton-ядер": quantization fused into the kernel that
 *   produces the operand, ahead of the grouped GEMM.]
 *   x        bf16 [tokens][cols]
 *   src      int32 [rows_out]      as written by moe_route
 *   xg       bf16 [rows_out][cols] as moe_permute(x) (written), or NULL when not
 *            wanted (then cols <= 16384: longer rows are cast from that copy)
 *   qg       u8   [rows_out][cols] codes of quantize_rowwise(xg) (written)
 *   scale_g  f32  [rows_out]       its row scales; a padding row takes fmax/1e-12f (written)
 *   Requires: cols % 8 == 0; x, xg and qg 16-byte aligned, src and scale_g
 *   4-byte aligned.  One kernel, no allocation.
 */
int moe_permute_rowwise(const void *x_bf16, int64_t tokens, int64_t cols, int32_t topk,
                        const int32_t *src, int64_t rows_out, int codec, void *xg_bf16, void *qg,
                        float *scale_g, void *stream);

/*
 * moe_combine -- weighted sum of each token's expert outputs.
 *   [P4 "MoE" (the routed experts' outputs summed per token with the router's
 *   weights).]
 *   yg       bf16 [rows_in][cols]  expert outputs in the grouped layout
 *   dest     int32 [tokens*topk]   as written by moe_route; a slot whose dest
 *                                  is < 0 or >= rows_in contributes nothing
 *   weights  f32 [tokens][topk], or NULL: every weight 1 (the backward's sum of a
 *            token's routed input gradients)
 *   y        bf16 [tokens][cols]   y[t] = sum over j in order 0..topk-1 of
 *            weights[t][j] * yg[dest[t*topk+j]], each product and sum one fp32
 *            operation rounded to nearest, then rounded to bf16 (nearest even) (written)
 *   Requires: cols % 8 == 0; yg and y 16-byte aligned, dest and weights 4-byte aligned.
 */
int moe_combine(const void *yg_bf16, int64_t rows_in, const int32_t *dest,
                const float *weights, int64_t tokens, int32_t topk, int64_t cols,
                void *y_bf16, void *stream);

/*
 * moe_combine_backward -- the gradients through moe_combine, for the loss
 * gradient dy of its output: each routed row's gradient in the grouped layout
 * (optionally quantized rowwise in the same pass, for the W2 dgrad GEMM) and
 * each router weight's gradient.
 *   [P4 "MoE" (the routed experts' outputs summed per token with the router's
 *   weights); P1 Details, MoE paragraph (the backward's grouped GEMMs on
 *   dynamically quantized operands).]
 *   dy       bf16 [tokens][cols]   gradient of moe_combine's output
 *   yg       bf16 [rows][cols]     the expert outputs moe_combine summed
 *   dest     int32 [tokens*topk], src int32 [rows]  from one moe_route call
 *   weights  f32  [tokens][topk]
 *   dyg      bf16 [rows][cols]     for grouped row r holding slot s = src[r] of
 *            token t = s / topk: bf16(weights[s] * dy[t]), one fp32 product
 *            rounded to nearest even; zeros for a row holding no slot (written),
 *            or NULL: not written (moe_permute_quantize_mx_dual forms the same
 *            rows from dy itself)
 *   q        u8   [rows][cols]     codes of quantize_rowwise(dyg), or NULL (written)
 *   scale    f32  [rows]           its row scales, NULL exactly when q is (written)
 *   dweights f32  [tokens*topk]    sum over columns of dy[t] * yg[dest[s]] (exact
 *            bf16 products, fp32 sums in an unspecified order); 0 for a slot whose
 *            dest is < 0 or >= rows (written)
 *   Requires: cols % 8 == 0 and cols <= 16384 (else FP8MOE_ERR_UNSUPPORTED);
 *   dy, yg, dyg and q 16-byte aligned, the int32 and f32 arrays 4-byte
 *   aligned.  One kernel, no allocation.
 */
int moe_combine_backward(const void *dy_bf16, const void *yg_bf16, int64_t rows,
                         const int32_t *dest, const int32_t *src, const float *weights,
                         int64_t tokens, int32_t topk, int64_t cols, int codec, void *dyg_bf16,
                         void *q, float *scale, float *dweights, void *stream);

/*
 * quantize_colwise -- one fp32 scale per (group, column), reduced over the
 * group's rows, with the FP8 output written transposed (contraction-contiguous)
 * so the backward GEMMs read it directly, with no separate transpose copy.
 *   [P1 Details: colwise scales kernel, output tile transposed through LDS
 *   before the store, single-pass variant without the second HBM read; P4 "Три
 *   уровня оптимизации Triton-ядер" (removal of the .t().contiguous().t() copy,
 *   fused scale-and-cast for backward); P2 Details, wgrad layout along the
 *   contracting dimension.]
 *   Grouped 2D form (batch == 1, offs != NULL):
 *     x     bf16 [rows][cols], offs int32 [n_groups]
 *     q_t   u8   phys [cols][ld_q]   q_t[c][r] = code of x[r][c] (rows of no group untouched)
 *     scale f32  [n_groups][cols]    empty group: fmax/1e-12f
 *   Batched 3D form (offs == NULL, n_groups ignored):
 *     x     bf16 [batch][rows][cols]
 *     q_t   u8   phys [batch][cols][ld_q]
 *     scale f32  [batch][cols]
 *   Requires: batch >= 1 (== 1 with offs), n_groups >= 1 with offs, rows, cols >= 0,
 *   ld_q >= rows, cols % 8 == 0, ld_q % 16 == 0, x and q_t 16-byte aligned.
 *   Normally the call enqueues one kernel: every 64-column chunk of 512 rows
 *   (256 rows when the groups or batch items average at most 512 rows, 128
 *   when at most 128, so a short group does not occupy a mostly empty chunk)
 *   is read once into
 *   registers, and the chunks of a group exchange their column
 *   maxima through a fixed library-owned device array (32768 chunk slots, no
 *   allocation) before casting from registers.  Values in that array carry a
 *   per-call tag (a host counter), so calls need no reset and leave nothing
 *   behind.  Calls that overlap on one device (other streams) stay correct: a
 *   chunk whose peers do not all publish within a bounded number of polls
 *   recomputes the maxima from x itself, at the cost of a second read.  A
 *   group taller than 128 chunks of 512 rows, a call with more than 32768 chunks, or a
 *   call made while `stream` is being captured into a graph (where a replay
 *   would repeat the tag) instead takes three kernels (amax reset, partial
 *   amax, cast): x is read twice, and no state carries between launches.
 */
int quantize_colwise(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                     const int32_t *offs, int32_t n_groups, int codec,
                     void *q_t, int64_t ld_q, float *scale, void *stream);

/*
 * moe_permute_quantize_colwise -- the gather of token rows into moe_route's
 * grouped layout fused with quantize_colwise of the gathered tensor: the rows
 * are formed at load time and never go to memory.  With router weights it
 * forms, the same way, the routed-row gradients of moe_combine_backward from
 * the output gradient dy (the weight gradient's colwise operand; the rowwise
 * one comes from moe_combine_backward in the same backward pass).
 *   [as quantize_colwise; P1 Details, MoE paragraph (the routed rows quantized
 *   by a fused kernel ahead of the grouped GEMM); P4 "MoE" (the experts' outputs
 *   summed with the router's weights); P4 "Три уровня оптимизации
 *   Triton-ядер" (fused backward scale-and-cast).]
 *   x        bf16 [tokens][cols]  token rows (or dy)
 *   src      int32 [rows]         from moe_route: grouped row r holds slot
 *                                 s = src[r] of token s / topk; a row whose
 *                                 src is < 0 or >= tokens*topk is zeros
 *   weights  f32 [tokens*topk], or NULL: row r = bf16(weights[s] * x[s / topk]),
 *            one fp32 product rounded to nearest even; NULL: row r = x[s / topk]
 *   q_t, ld_q, scale, offs, n_groups, codec: as quantize_colwise of the gathered
 *   [rows][cols] tensor in its grouped form (offs required, non-NULL); the same
 *   kernels, paths and shared-state rules.
 *   Requires: tokens*topk <= INT32_MAX; x 16-byte aligned, src and weights
 *   4-byte aligned; the rest as quantize_colwise.  No allocation.
 */
int moe_permute_quantize_colwise(const void *x_bf16, int64_t tokens, int64_t cols, int32_t topk,
                                 const int32_t *src, const float *weights, int64_t rows,
                                 const int32_t *offs, int32_t n_groups, int codec, void *q_t,
                                 int64_t ld_q, float *scale, void *stream);

/*
 * quantize_mx -- MXFP8: e4m3fn codes with one e8m0 scale per 1x32 block.
 *   [P2 Details: _to_mxfp8_then_scaled_grouped_mm quantizes activations and
 *   weights dynamically; MXFP8 data/scale layout diagram; wgrad quantized along
 *   the contracting (token) dimension.  P4 "Скейлы: от тензора до микроблока".]
 *   axis == 1 (blocks along cols; offs must be NULL):
 *     x [batch*rows][cols] -> q [batch*rows][cols], scale [batch*rows][cols/32]; cols % 32 == 0.
 *   axis == 0, offs == NULL (blocks along rows, per batch item):
 *     x [batch][rows][cols] -> q phys [batch][cols][rows], scale [batch][cols][rows/32];
 *     rows % 32 == 0.
 *   axis == 0, offs != NULL (batch == 1; blocks restart at every group):
 *     x [rows][cols] -> q phys [cols][rows_pad], scale [cols][rows_pad/32],
 *     offs_pad_out int32 [n_groups] = inclusive cumsum of ceil(M_e/32)*32.
 *     Each group is zero-padded to a multiple of 32 rows (pad counted as +0);
 *     columns past the last padded group are written as data 0 and scale 0.
 *     rows_pad % 32 == 0 and rows_pad >= quantize_mx_rows_bound(rows, n_groups).
 *   scale_layout: FP8MOE_MX_LAYOUT_ROWS gives the row-major scale shapes above;
 *     FP8MOE_MX_LAYOUT_K4 the K4 layout of the same matrices, with
 *     R = batch*rows, NB = cols/32 (axis 1); R = batch*cols, NB = rows/32
 *     (axis 0 without offs); R = cols, NB = rows_pad/32 (axis 0 with offs).
 *   Requires cols % 8 == 0 for axis == 0; x and q 16-byte aligned.
 *   MX is defined for e4m3fn only (there is no codec argument).
 */
int quantize_mx(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols, int axis,
                const int32_t *offs, int32_t n_groups, int rule, int scale_layout,
                void *q, void *scale_e8m0, int64_t rows_pad, int32_t *offs_pad_out,
                void *stream);

/*
 * quantize_mx_dual -- both MXFP8 forms of one tensor from a single read: the
 * last-dim blocks (a weight's forward operand, an activation gradient's dgrad
 * operand) and the row blocks (the same weight's dgrad operand, the wgrad
 * operands).  Every 1x32 block is local to its 32 elements, so one pass over a
 * tile of x gives both; HBM sees x read once instead of twice.
 *   [as quantize_mx; P2 Details (the forward and both backward GEMMs take
 *   MXFP8 operands blocked along their own contraction dimension); P4 "Три
 *   уровня оптимизации Triton-ядер" (fused scale-and-cast, no second read).]
 *   q, scale_e8m0     the outputs of quantize_mx(x, batch, rows, cols, axis = 1)
 *                     over x viewed as [batch*rows][cols] (written).  With offs,
 *                     only the rows inside groups (rows < offs[n_groups-1]) are
 *                     written; rows past the last group are left untouched.
 *   q_t, scale_t_e8m0 the outputs of quantize_mx(x, ..., axis = 0, offs, n_groups,
 *                     rows_pad, offs_pad_out) (written)
 *   Every other argument and every requirement is that of the two quantize_mx
 *   calls (cols % 32 == 0; without offs, rows % 32 == 0); scale_layout applies
 *   to both scale matrices; q 16-byte aligned.  One kernel (128 x 128 work
 *   items, so every row's last-dim codes leave in whole 128-byte lines), no
 *   allocation.
 */
int quantize_mx_dual(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                     const int32_t *offs, int32_t n_groups, int rule, int scale_layout, void *q,
                     void *scale_e8m0, void *q_t, void *scale_t_e8m0, int64_t rows_pad,
                     int32_t *offs_pad_out, void *stream);

/*
 * moe_permute_quantize_mx_dual -- the gather of token rows into moe_route's
 * grouped layout fused with both MXFP8 forms of the gathered tensor: the rows
 * are formed at load time and never go to memory (an optional bf16 copy
 * exists).  With router weights it forms, the same way, the routed-row
 * gradients of moe_combine_backward from the output gradient dy.
 *   [P1 Details, MoE paragraph (the routed rows quantized by a fused kernel
 *   ahead of the grouped GEMM); P2 Details (MXFP8 operands blocked along each
 *   GEMM's contraction dimension); P4 "MoE" (the experts' outputs summed with
 *   the router's weights, whose backward scales each routed row).]
 *   x        bf16 [tokens][cols]  token rows (or dy)
 *   src      int32 [rows]         from moe_route: grouped row r holds slot
 *                                 s = src[r] of token s / topk; a row whose
 *                                 src is < 0 or >= tokens*topk is zeros
 *   weights  f32 [tokens*topk], or NULL: row r = bf16(weights[s] * x[s / topk]),
 *            one fp32 product rounded to nearest even; NULL: row r = x[s / topk]
 *   xg       bf16 [rows][cols]    optional copy of the gathered rows (NULL: not
 *                                 written); rows past the last group untouched
 *   q, scale_e8m0, q_t, scale_t_e8m0, offs, n_groups, rows_pad, offs_pad_out,
 *   rule, scale_layout: as quantize_mx_dual of the gathered [rows][cols] tensor
 *   with offs (required, non-NULL).
 *   Requires: tokens*topk <= INT32_MAX; x, xg and q 16-byte aligned, src and
 *   weights 4-byte aligned; the rest as quantize_mx_dual.  One kernel, no
 *   allocation.
 */
int moe_permute_quantize_mx_dual(const void *x_bf16, int64_t tokens, int64_t cols, int32_t topk,
                                 const int32_t *src, const float *weights, int64_t rows,
                                 const int32_t *offs, int32_t n_groups, int rule, int scale_layout,
                                 void *xg_bf16, void *q, void *scale_e8m0, void *q_t, void *scale_t_e8m0,
                                 int64_t rows_pad, int32_t *offs_pad_out, void *stream);

/*
 * swiglu_quantize_mx_dual -- the SwiGLU between the two expert GEMMs fused with
 * both MXFP8 forms of its output (the W2 forward operand and the W2 wgrad
 * operand): A2 = bf16(silu(gate) * up) is computed from W1's output as
 * swiglu_quantize_rowwise computes it and quantized as quantize_mx_dual(A2)
 * would, without A2 ever going to memory.
 *   [P1 Details and P4 "Три уровня оптимизации Triton-ядер": quantization
 *   fused into the kernel that produces the tensor; P2 Details: MXFP8 operands
 *   blocked along each GEMM's contraction dimension.]
 *   h1      bf16 [rows][ld_h1]  gate in columns [0, F), up in [F, 2F)
 *   a2      bf16 [rows][F]      optional copy of A2 (NULL: not written)
 *   q, scale_e8m0, q_t, scale_t_e8m0, offs, n_groups, rows_pad, offs_pad_out,
 *   rule, scale_layout: as quantize_mx_dual of A2 ([rows][F], so with offs
 *   only the rows inside groups get last-dim codes).
 *   Requires: F % 32 == 0; ld_h1 >= 2F, ld_h1 % 8 == 0; h1, a2 and q 16-byte
 *   aligned; the rest as quantize_mx_dual.  One kernel, no allocation.
 */
int swiglu_quantize_mx_dual(const void *h1_bf16, int64_t rows, int64_t F, int64_t ld_h1,
                            const int32_t *offs, int32_t n_groups, int rule, int scale_layout,
                            void *a2_bf16, void *q, void *scale_e8m0, void *q_t, void *scale_t_e8m0,
                            int64_t rows_pad, int32_t *offs_pad_out, void *stream);

/*
 * swiglu_backward_quantize_mx_dual -- SwiGLU's backward fused with both MXFP8
 * forms of its result (the W1 dgrad operand and the W1 wgrad operand): dH1 =
 * [d gate | d up] ([rows][2F]) as swiglu_backward_quantize_rowwise computes it,
 * quantized as quantize_mx_dual(dH1) would, without dH1 going to memory.
 *   [as swiglu_quantize_mx_dual]
 *   da2     bf16 [rows][F]      gradient of A2
 *   dh1     bf16 [rows][2F]     optional copy of dH1 (NULL: not written)
 *   The rest as swiglu_quantize_mx_dual, for the [rows][2F] tensor dH1, except
 *   that F % 128 == 0 (each work item evaluates the product rule once for 128
 *   columns of F and emits the matching d gate and d up tiles).
 */
int swiglu_backward_quantize_mx_dual(const void *da2_bf16, const void *h1_bf16, int64_t rows,
                                     int64_t F, int64_t ld_h1, const int32_t *offs, int32_t n_groups,
                                     int rule, int scale_layout, void *dh1_bf16, void *q,
                                     void *scale_e8m0, void *q_t, void *scale_t_e8m0, int64_t rows_pad,
                                     int32_t *offs_pad_out, void *stream);

/* Host-side allocation bound for quantize_mx's padded rows: round_up(rows + 31*n_groups, 32).
 * Returns -1 for negative arguments. */
int64_t quantize_mx_rows_bound(int64_t rows, int32_t n_groups);

/*
 * grouped_mm_scaled -- offset-routed grouped GEMM with the quantization scales
 * applied in the epilogue (fp32) or per 32-block (e8m0).
 *   [P1 Details, MoE paragraph: variable-size expert batches, per-expert weight
 *   column scales, per-row activation scales, routing offsets, one launch;
 *   P4 "MoE: почему DeepSeek-V3 ломал пайплайн"; P3 and P4 on the three GEMMs of a
 *   linear layer (forward, input gradient, weight gradient); P2 Details, MoE
 *   forward diagram (2D activations x 3D expert weights grouped by offsets) and
 *   scaled MXFP8 grouped GEMM; P1 Details, Figure 1 "+GW" run with the weight
 *   gradient kept in BF16.]
 *   mode GROUPED_M (fwd/dgrad):  out[m][n] = sum_k A(m,k) B(e,n,k), m in group e
 *     a [M][K], b [E][N][K] (E = n_groups), out [M][N]; rows of no group untouched.
 *     SCALE_F32:  a_scale f32 [M], b_scale f32 [E][N]; A = dec(a)/sa, B = dec(b)/sb.
 *     SCALE_E8M0: a_scale u8 [M][K/32], b_scale u8 [E][N][K/32]; K % 32 == 0.
 *   mode GROUPED_K (wgrad):  out[e][n][k] = sum_{m in group e} A(n,m) B(k,m)
 *     a phys [N][M], b phys [K][M] (token-contiguous), out [E][N][K]; empty group -> 0.
 *     SCALE_F32:  a_scale f32 [E][N], b_scale f32 [E][K].
 *     SCALE_E8M0: a_scale u8 [N][M/32], b_scale u8 [K][M/32]; M = padded rows and
 *                 offs = padded offsets from quantize_mx (multiples of 32).
 *   SCALE_E8M0_K4: the same e8m0 scales in quantize_mx's K4 layout, the operand's
 *     scale rows being R = M and E*N (GROUPED_M: a, b) or N and K (GROUPED_K);
 *     4-byte aligned, 4 * R * ceil(L/128) bytes each (L = K or M) and below 2^31.
 *     SCALE_NONE with OPD_BF16 operands: a bf16 [M][N], b bf16 [M][K] (token-major).
 *   offs may be NULL only when n_groups == 1 (one group of all M rows).
 *   Formats: both operands FP8 (e4m3fn or e4m3fnuz, mixed allowed; e8m0 scales
 *   need e4m3fn) or both BF16 (GROUPED_K with SCALE_NONE only).
 *   Accumulation is fp32; out is bf16 (round to nearest even) or fp32.
 *   Requires: M, N, K >= 0; FP8 operands: K % 16 == 0 and K <= 2^23 (GROUPED_M) or
 *   M % 16 == 0 and M <= 2^23 (GROUPED_K); BF16 operands: M, N, K % 8 == 0;
 *   all pointers 16-byte aligned.
 */
int grouped_mm_scaled(int mode, const void *a, int a_fmt, const void *a_scale,
                      const void *b, int b_fmt, const void *b_scale, int scale_kind,
                      const int32_t *offs, int32_t n_groups, int64_t M, int64_t N, int64_t K,
                      void *out, int out_dtype, void *stream);

/*
 * fp8moe_encode_f32 -- the device FP8 encoder alone: q[i] = enc(y[i]) for
 * values already inside [-fmax, fmax] (round to nearest, ties to the even
 * code; e4m3fn keeps the sign of zero, e4m3fnuz has one unsigned zero).  The
 * same encoder the quantization kernels use; exposed so the codec can be
 * checked on the device over whole value ranges.  Values outside the range or
 * NaN give unspecified codes.  y f32 [n] (4-byte aligned), q u8 [n].
 */
int fp8moe_encode_f32(const float *y, int64_t n, int codec, void *q, void *stream);

/* Static string for a status code (never NULL). */
const char *fp8moe_status_string(int status);

/* FP8 codec native to a device: gfx950 -> E4M3FN, gfx942 -> E4M3FNUZ.  Queries
 * the device (a HIP call).  Returns FP8MOE_ERR_UNSUPPORTED for other architectures.
 * [P1 Details and P4 "Тихая порча градиентов": the FP8 dtype and its maximum are
 * chosen from the hardware.] */
int fp8moe_default_codec(int hip_device, int *codec_out);

/* Library ABI version (major*100 + minor). */
int fp8moe_version(void);

/*
 * fp8moe_set_colwise_poll_budget -- test hook: the number of polls a chunk of
 * the single-pass colwise quantizer makes for its peers' column maxima before
 * it recomputes them from x (0: recompute at once; negative: restore the
 * default, 4096).  Results do not depend on it, only the time a call takes;
 * tests use 0 to run the recomputation path.  It applies to calls enqueued
 * after it returns.  Returns the previous budget.  Host only, no HIP call.
 */
int fp8moe_set_colwise_poll_budget(int polls);

/*
 * fp8moe_set_colwise_chunk_rows -- test and tuning hook: the chunk height of
 * the single-pass colwise quantizer (128, 256 or 512 rows: forced; any other
 * value: chosen per call from the average rows per group or batch item, 128
 * rows up to 128, 256 rows up to 512, else 512).  A forced height that a call
 * cannot use (too many chunks)
 * falls back to 512 rows, then to the two-pass path.  Results do not depend on
 * it.  Process-wide; returns the previous setting (0 for per-call choice).
 */
int fp8moe_set_colwise_chunk_rows(int rows);

#ifdef __cplusplus
}
#endif

#endif /* FP8MOE_H */
