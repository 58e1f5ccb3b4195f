/*
 * q4k.h -- C ABI of libq4k.so, the MI355X (gfx950) fused-dequantize Q4_K
 * matrix-vector product, its batched (prefill) form, the Q4_0 and Q6_K
 * matrix-vector products and the ternary BitNet b1.58 sibling.
 *
 * Common contract for every compute entry point:
 *   - x, w_blocks/codes and y are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees, synchronizes or keeps state; it
 *     validates the arguments, enqueues its kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and returns.
 *   - Arguments are validated before anything is launched, in this order:
 *     dimensions, then NULL pointers, then alignment.  On any error nothing
 *     is launched and y is left untouched.
 *   - y must not overlap x or the weights (not checked).
 *   - Stateless and safe to call from any host thread on any stream.
 *   - Every call is deterministic: each output has exactly one writer and
 *     the summation order depends only on the shapes.
 *   - No C++ exception crosses this interface.
 */
#ifndef Q4K_H
#define Q4K_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define Q4K_OK 0
#define Q4K_EINVAL_DIM (-1) /* a dimension is <= 0 or not a multiple of the block size */
#define Q4K_ENULL (-2)      /* a required pointer is NULL */
#define Q4K_EALIGN (-3)     /* a pointer is not 16-byte aligned where required */
#define Q4K_EHIP (-4)       /* the HIP runtime reported an error (see q4k_strerror) */
#define Q4K_ESCRATCH (-5)   /* q4k_matmul_noalloc: the call needs more than its fixed scratch */

/*
 * Q4_K weight format (block_q4_K, 256 weights in 144 bytes), as the Q4_K
 * page (SKaiNET PR #562, "feat(kernel): SIMD-fused Q4_K matmul kernel +
 * Q4KMatmulKernel SPI", section "Pipeline") uses it:
 *   bytes 0..1    d     binary16, little-endian
 *   bytes 2..3    dmin  binary16, little-endian
 *   bytes 4..15   eight 6-bit scales sc[s] and eight 6-bit mins m[s] in the
 *                 ggml packing: s<4: sc=S[s]&63, m=S[s+4]&63; s>=4:
 *                 sc=(S[s+4]&15)|(S[s-4]>>6)<<4, m=(S[s+4]>>4)|(S[s]>>6)<<4
 *   bytes 16..143 qs; byte 32j+l holds position l of sub-block 2j in its low
 *                 nibble and position l of sub-block 2j+1 in its high nibble
 * Weight k of a block (sub-block s = k/32, code q) is d*sc[s]*q - dmin*m[s].
 * The matrix is row-major [output_dim][input_dim/256] blocks: row o is the
 * input_dim/256 consecutive blocks starting at byte o*(input_dim/256)*144.
 */

/*
 * q4k_gemv -- y[o] = sum_k W[o,k] * x[k] for o < output_dim (batch 1).
 * The fused Q4_K matrix-vector product of the Q4_K page, sections "Summary"
 * and "Pipeline": every output is the per-sub-block lazy-dmin sum
 * sum_s (d*sc[s]*sum_l q*x - dmin*m[s]*sum_l x), accumulated in fp32.
 *   x          fp32 [input_dim], 16-byte aligned
 *   w_blocks   uint8 [output_dim * input_dim/256 * 144], 16-byte aligned
 *   input_dim  K; must be > 0 and a multiple of 256 (the page's test plan
 *              rejects any other inputDim) and at most 2^24, else
 *              Q4K_EINVAL_DIM
 *   output_dim N > 0
 *   y          fp32 [output_dim]
 * fp32 accumulation; agreement with the exact product is within about 1e-4
 * relative (elementwise against 1e-4*|y| + 1e-4*rms(y)).  |x| should stay
 * above ~1e-30 for full precision (the vector form's codes enter the
 * multiply scaled by 2^-24).
 * Three kernels compute it: a vector form (lanes own 32-byte slabs of a row
 * and walk rows), a matrix-core form (16x16x32 f16 MFMA over 16 rows x
 * one sub-block; each 32-activation sub-block is scaled by a power of two
 * and split into exact fp16 hi and lo halves, which holds for |x| < 2^96,
 * about 7.9e28) and a persistent matrix-core walk (the same arithmetic;
 * workgroups walk groups of 16 rows x one super-block, the next ones in
 * flight).  Where each measured fastest on MI355X, the call picks the walk
 * for large matrices (output_dim >= 3072 with input_dim >= 5120, or
 * output_dim >= 11008 with input_dim >= 4096), the matrix-core form when
 * ceil(output_dim/16) is 192..256 and input_dim/256 is 12..19, else the
 * vector form; q4k_gemv_shaped and q4k_gemv_walk_shaped select one
 * explicitly.
 */
int q4k_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
             int64_t output_dim, float *y, void *stream);

/*
 * q4k_matmul -- Y[r, o] = sum_k W[o,k] * X[r,k] for r < n_tokens: the
 * batched (prefill) form.  Row r of X starts at X + r*input_dim and row r
 * of Y at Y + r*output_dim, the row offsets of the ternary page's prefill
 * row loop (SKaiNET issue #1138, section "Tasks").  Following the tiling
 * page (llama.cpp fork PR #37, "ggml-cpu: cache-aware tiling in
 * ggml_compute_forward_mul_mat", section "Summary", fix 1), the weights
 * are not re-streamed per token: each kernel reads a weight tile once for
 * a whole tile of tokens, and the workgroups that share a weight tile run
 * on one XCD, so HBM delivers each weight byte once per call; the
 * activations (4 bytes each) are fetched into every XCD's L2 that uses
 * them.
 *   X          fp32 [n_tokens, input_dim], 16-byte aligned
 *   w_blocks   as for q4k_gemv
 *   n_tokens   M > 0 (M == 1 runs q4k_gemv)
 *   input_dim, output_dim as for q4k_gemv
 *   Y          fp32 [n_tokens, output_dim]
 * Same error behaviour and tolerance as q4k_gemv.  The kernels serving it:
 * M == 1 is q4k_gemv; a few tokens (M <= 2 at any shape, M <= 8 with
 * output_dim <= 4096) run on a batched matrix-core GEMV that reads each
 * weight once for all of them; from 33 tokens (from 17 with output_dim > 4096, from 9 with
 * input_dim >= 8192) 128-row x 32-token tiles whose input_dim is split
 * across workgroups when the tiles alone would leave CUs idle; otherwise
 * prefill tiles of 64 rows x 16 tokens (narrowed to 32 or 16 rows when
 * 64-row tiles would leave CUs idle).  The batched and tiled kernels pass
 * the activations through fp16: each token's 256 activations of a
 * super-block are scaled by a power of two, then split into a high and a
 * low half, both exact MFMA operands (any |x| < 2^96).  The split tiles add
 * their ranges' partial results in a fixed order, so results do not depend
 * on timing.  Their partial tiles go to a workspace of 32 MiB + 4 KiB that
 * the library allocates once per device, on the first call that needs it,
 * and keeps until the process ends; a call that would allocate it while its
 * stream is being captured into a graph fails with Q4K_EHIP (make one such
 * call outside the capture first).  Every call on a device shares that
 * workspace, so calls that use it (q4k_matmul and q4k_matmul_shaped on the
 * split tiles, graphs holding such calls) must not run at the same time on
 * one device: on different streams, order them with events.  Y must not
 * alias X or the weights.
 */
int q4k_matmul(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
               int64_t input_dim, int64_t output_dim, float *Y, void *stream);

/*
 * Q4_0 weight format (block_q4_0, 32 weights in 18 bytes): the simpler
 * block the Q4_K page names as its follow-up (section "Out of scope": same
 * algorithm, 32 / 18 bytes).  The page prints no more; this library reads
 * it as ggml's block_q4_0:
 *   bytes 0..1    d   binary16, little-endian
 *   bytes 2..17   qs; byte i holds element i in its low nibble and element
 *                 16+i in its high nibble
 * Weight k of a block (code q) is d*(q - 8).  The matrix is row-major
 * [output_dim][input_dim/32] blocks, row o starting at byte
 * o*(input_dim/32)*18.
 */

/*
 * q4_0_gemv -- y[o] = sum_k W[o,k] * x[k] for a Q4_0 matrix (batch 1), the
 * same fused product as q4k_gemv: every block adds d*(sum q*x - 8*sum x),
 * accumulated in fp32.
 *   x          fp32 [input_dim], 16-byte aligned
 *   w_blocks   uint8 [output_dim * input_dim/32 * 18], 16-byte aligned
 *   input_dim  K > 0, a multiple of 256 and at most 2^24, else
 *              Q4K_EINVAL_DIM.  The format itself only needs multiples of
 *              32; this kernel walks rows in 144-byte groups of eight
 *              blocks, which keeps every row 16-byte aligned.
 *   output_dim N > 0
 *   y          fp32 [output_dim]
 * Same error behaviour, determinism and tolerance as q4k_gemv.  Two kernels
 * compute it: the vector form (|x| should stay above ~1e-30 for full
 * precision) and a matrix-core form (16x16x32 f16 MFMA over 16 rows and
 * eight blocks; each block's activations scaled by a power of two and split
 * into exact fp16 hi and lo halves, for any |x| < 2^96), taken where it
 * measured fastest on MI355X: ceil(output_dim/16) 192..256 and
 * input_dim/256 12..24.
 */
int q4_0_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
              int64_t output_dim, float *y, void *stream);

/*
 * q4_0_gemv_shaped -- q4_0_gemv with an explicit launch shape; the values
 * of rows_per_lane, k_waves and workgroup_waves are those of
 * q4k_gemv_shaped, workgroup_waves = 16 selecting the matrix-core form
 * (rows_per_lane and k_waves then 0), which takes input_dim up to 65536
 * (256 groups of eight blocks; more is Q4K_EINVAL_DIM) and any |x| < 2^96.
 */
int q4_0_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                     int64_t output_dim, float *y, void *stream,
                     int rows_per_lane, int k_waves, int workgroup_waves);

/*
 * Q6_K weight format (block_q6_K, 256 weights in 210 bytes): the Q4_K page's
 * other follow-up (section "Out of scope": ql holds the codes' low bits, qh
 * their high bits, four codes per qh byte, in two interleaved halves).  Read
 * as ggml's block_q6_K:
 *   bytes 0..127    ql
 *   bytes 128..191  qh
 *   bytes 192..207  sixteen int8 scales
 *   bytes 208..209  d   binary16, little-endian
 * Element 128n + 32c + l (n < 2, c < 4, l < 32) has code q = lo | hi<<4: lo
 * the low (c < 2) or high (c >= 2) nibble of ql[64n + 32*(c%2) + l], hi bits
 * 2c..2c+1 of qh[32n + l]; its weight is d*scale[8n + 2c + l/16]*(q - 32).
 * The matrix is row-major [output_dim][input_dim/256] blocks, row o
 * starting at byte o*(input_dim/256)*210 (rows need not be 16-byte
 * aligned; the matrix must).
 */

/*
 * q6k_gemv -- y[o] = sum_k W[o,k] * x[k] for a Q6_K matrix (batch 1): every
 * 16-weight group adds d*scale*(sum q*x - 32*sum x), accumulated in fp32.
 *   x          fp32 [input_dim], 16-byte aligned
 *   w_blocks   uint8 [output_dim * input_dim/256 * 210], 16-byte aligned
 *   input_dim  K > 0, a multiple of 256 and at most 2^24, else Q4K_EINVAL_DIM
 *   output_dim N > 0
 *   y          fp32 [output_dim]
 * Same error behaviour, determinism and tolerance as q4k_gemv (vector
 * form; |x| should stay above ~1e-30 for full precision).
 */
int q6k_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
             int64_t output_dim, float *y, void *stream);

/*
 * q6k_gemv_shaped -- q6k_gemv with an explicit launch shape; the values are
 * those of q4k_gemv_shaped without the matrix-core form, except that
 * rows_per_lane 8 with k_waves 4 and 4-wave workgroups is rejected for long
 * rows (Q4K_EINVAL_DIM: the tiles would not fit in LDS).
 */
int q6k_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                    int64_t output_dim, float *y, void *stream,
                    int rows_per_lane, int k_waves, int workgroup_waves);

/*
 * Ternary BitNet b1.58 format (ternary page, SKaiNET issue #1138, section
 * "Tasks"): four codes per byte in sequence; element i of a row is
 * ((byte[i/4] >> 2*(i%4)) & 3) - 1, so field values 0, 1, 2 decode to
 * -1, 0, +1 (field value 3 decodes to +2 by the same formula).  The matrix
 * is row-major: row o is input_dim/4 bytes starting at o*input_dim/4.
 */

/*
 * ternary_gemv_codes -- t[o] = sum_i code(o,i) * x[i]: the codes-dot with
 * the scale NOT applied, the gemvPacked contract of the ternary page.
 *   x          fp32 [input_dim] (any alignment; 16-byte alignment, together
 *              with input_dim % 64 == 0 and 16-byte aligned codes, selects
 *              the fast kernel)
 *   codes      uint8 [output_dim * input_dim/4]
 *   input_dim  K > 0, a multiple of 4 and at most 2^24, else Q4K_EINVAL_DIM
 *   output_dim N > 0
 *   y          fp32 [output_dim]
 * fp32 accumulation.  Exact (bit-equal to the exact result) whenever every
 * x[i] is an integer and sum_i |x[i]| * 2 < 2^22.
 */
int ternary_gemv_codes(const float *x, const uint8_t *codes, int64_t input_dim,
                       int64_t output_dim, float *y, void *stream);

/*
 * ternary_gemv -- y[o] = scale * t[o]: the per-tensor scale is multiplied
 * after the codes-dot, as the ternary page's reference view kernel does
 * (one fp32 rounding of scale * t).  Arguments as ternary_gemv_codes.
 */
int ternary_gemv(const float *x, const uint8_t *codes, float scale,
                 int64_t input_dim, int64_t output_dim, float *y,
                 void *stream);

/*
 * ternary_matmul -- Y[r, o] = scale * sum_i code(o,i) * X[r,i] for r <
 * n_tokens: the batched (prefill) ternary product, the row loop of the
 * ternary page's prefill path (SKaiNET issue #1138, section "Tasks"), with
 * each code read once for a tile of 16 tokens.
 *   X          fp32 [n_tokens, input_dim] (row r at X + r*input_dim)
 *   codes      as for ternary_gemv_codes
 *   scale      per-tensor scale, multiplied after each dot
 *   n_tokens   M > 0 (M == 1 runs ternary_gemv), else Q4K_EINVAL_DIM
 *   input_dim, output_dim as for ternary_gemv_codes
 *   Y          fp32 [n_tokens, output_dim] (row r at Y + r*output_dim)
 * With input_dim % 64 == 0, 16-byte aligned X and codes, and more than 2
 * tokens (more than 3 when input_dim > 8192) the products run on 16x16x32
 * f16 MFMA tiles (64, 32 or 16 rows x 16 tokens per workgroup, the height
 * chosen as for q4k_matmul's prefill tiles): the codes enter exactly, and
 * X, after each token's 256-position block is scaled by a power of two, as
 * exact fp16 hi and lo halves (any |X| < 2^96); the sum is fp32 (tolerance as q4k_gemv;
 * exact for integer X with sum_i |X[r,i]| * 3 < 2^22).  Otherwise it runs
 * one ternary_gemv launch per token row.  Y must not alias X or the codes.
 * Error behaviour as for the other calls, with one exception: on the row
 * loop every launch has the same dimensions, so anything the library
 * rejects is rejected before the first row, but a failure that the HIP
 * runtime reports part-way through the loop (Q4K_EHIP) can leave the
 * earlier token rows of Y written.
 */
int ternary_matmul(const float *X, const uint8_t *codes, float scale, int64_t n_tokens,
                   int64_t input_dim, int64_t output_dim, float *Y, void *stream);

/*
 * ternary_matmul_shaped -- ternary_matmul with its kernel forced, for
 * sweeps and tests: form 1 runs the row loop (one ternary_gemv launch per
 * token row); form 16, 32 or 64 runs the matrix-core tiles with that many
 * rows per workgroup (x 16 tokens; input_dim a multiple of 64 else
 * Q4K_EINVAL_DIM, X and codes 16-byte aligned else Q4K_EALIGN); 0 is
 * ternary_matmul itself.  Any other value gives Q4K_EINVAL_DIM.
 */
int ternary_matmul_shaped(const float *X, const uint8_t *codes, float scale, int64_t n_tokens,
                          int64_t input_dim, int64_t output_dim, float *Y, void *stream,
                          int form);

/*
 * q4k_gemv_shaped -- q4k_gemv with an explicit launch shape, for sweeps and
 * for the benchmark's launch configuration.  rows_per_lane in {1, 2, 4, 8}
 * (rows whose partial sums one lane carries), k_waves in {1, 2, 4} (waves
 * of one workgroup that split input_dim between them), workgroup_waves in
 * {1, 2, 4, 8} (a multiple of k_waves; with 8 waves k_waves <= 2 and
 * rows_per_lane <= 4).  A value of 0 lets the library choose (k_waves = 0
 * never exceeds the workgroup size).  workgroup_waves = 16 selects the
 * matrix-core form instead (rows_per_lane and k_waves must then be 0).  Any
 * other value gives Q4K_EINVAL_DIM.  Results are within the q4k_gemv
 * tolerance for every shape (the summation order depends on the shape).
 */
int q4k_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                    int64_t output_dim, float *y, void *stream,
                    int rows_per_lane, int k_waves, int workgroup_waves);

/*
 * q4k_gemv_walk_shaped -- q4k_gemv's product on the persistent matrix-core
 * walk, with its launch shape: waves per workgroup in {4, 8, 16}, row_groups
 * (consecutive groups of 16 rows per workgroup) in 1..4, depth (units of 16
 * rows x one super-block each wave loads ahead) in {2, 4}, with 4 waves
 * only depth 4 and with 16 waves only depth 2; 0 lets the library choose
 * that value.  Any other value gives Q4K_EINVAL_DIM.  Arguments, layouts,
 * range of x and results as for q4k_gemv (within its tolerance for every
 * shape).
 */
int q4k_gemv_walk_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                         int64_t output_dim, float *y, void *stream, int waves,
                         int row_groups, int depth);

/*
 * Q4_K tiled block order.  SKaiNET docs, "Eager execution: backends and
 * kernels": a packed weight reaches a kernel by declaring its block order,
 * and a canonical weight is relayouted into that order once, not per call.
 * The tiled order is this library's GPU block order; it holds the canonical
 * bytes, moved and never changed:
 *   - rows in groups of 16: group G is rows 16G .. 16G+15, ceil(output_dim/16)
 *     groups; rows at or past output_dim are zero bytes;
 *   - super-block b of group G is one 2304-byte tile at byte (G*nb + b)*2304,
 *     nb = input_dim/256;
 *   - tile bytes 0..2047: the 16 rows' qs in two halves of 1024 bytes; qs
 *     byte 32j + 8g + t (j, g < 4, t < 8) of row 16G + n is at tile byte
 *     1024*(j/2) + 16*(n + 16g) + 8*(j%2) + t (so the 16 bytes at 16*lane of
 *     a half are one lane's MFMA operand bytes for two sub-block pairs);
 *   - tile bytes 2048..2303: the 16 rows' block headers (bytes 0..15 of the
 *     block: d, dmin, the 12 scale bytes), row n at 2048 + 16n.
 */

/*
 * q4k_tiled_size -- bytes of a matrix in the tiled order:
 * ceil(output_dim/16) * (input_dim/256) * 2304, or Q4K_EINVAL_DIM (negative)
 * when a dimension is invalid as for q4k_gemv.  Host-only; touches no GPU.
 */
int64_t q4k_tiled_size(int64_t input_dim, int64_t output_dim);

/*
 * q4k_relayout_tiled -- the one-time move of a canonical Q4_K matrix into
 * the tiled order (meant for load time, not per call).
 *   w_blocks   canonical uint8 [output_dim * input_dim/256 * 144], 16-byte
 *              aligned (as for q4k_gemv)
 *   input_dim, output_dim as for q4k_gemv
 *   w_tiled    uint8 [q4k_tiled_size(input_dim, output_dim)], 16-byte
 *              aligned, every byte written (padding rows as zeros); must not
 *              overlap w_blocks (not checked)
 * Errors as for q4k_gemv (dimensions, then NULL, then alignment); on error
 * nothing is launched and w_tiled is untouched.  Pure byte moves: the
 * result is bit-exact.
 */
int q4k_relayout_tiled(const uint8_t *w_blocks, int64_t input_dim, int64_t output_dim,
                       uint8_t *w_tiled, void *stream);

/*
 * q4k_gemv_tiled -- q4k_gemv's product, y[o] = sum_k W[o,k] * x[k], with W
 * given in the tiled order (the product of the Q4_K page, sections
 * "Summary" and "Pipeline", in the lazy-dmin form).
 *   x          fp32 [input_dim], 16-byte aligned
 *   w_tiled    uint8 [q4k_tiled_size(input_dim, output_dim)], 16-byte
 *              aligned, written by q4k_relayout_tiled (or laid out so)
 *   input_dim, output_dim, y as for q4k_gemv
 * Computed on 16x16x32 f16 MFMA tiles: each tile is three coalesced
 * 16-byte loads per lane straight into registers; each 32-activation
 * sub-block is scaled by a power of two and split into exact fp16 hi and lo
 * halves (any |x| < 2^96); fp32 accumulation.  Errors and tolerance as for
 * q4k_gemv.  Deterministic; the summation order depends only on the shape.
 */
int q4k_gemv_tiled(const float *x, const uint8_t *w_tiled, int64_t input_dim,
                   int64_t output_dim, float *y, void *stream);

/*
 * q4k_matmul_tiled -- q4k_matmul's batched product, Y[r, o] = sum_k W[o,k] *
 * X[r,k] for r < n_tokens, with W in the tiled order: a weight relayouted
 * once serves both the single-token and the batched (prefill) calls.
 *   X          fp32 [n_tokens, input_dim], 16-byte aligned (row r at
 *              X + r*input_dim)
 *   w_tiled    as for q4k_gemv_tiled
 *   n_tokens   M > 0 (M == 1 runs q4k_gemv_tiled)
 *   input_dim, output_dim, Y as for q4k_matmul
 * The kernels are q4k_matmul's on this layout, with a hand-over measured
 * for it: a few tokens (M <= 4, or M <= 8 with output_dim <= 4096 and
 * input_dim >= 4096) on the batched matrix-core GEMV
 * (any |X| < 2^96), more on the prefill tiles of q4k_matmul (64, 32 or 16
 * rows x 16 tokens, any |X| < 2^96), which give q4k_matmul's bits: 64-row tiles
 * with input_dim below 8192 load each wave's tiles straight into registers,
 * the rest stage whole tiles through LDS.  Errors and tolerance as for
 * q4k_matmul.
 */
int q4k_matmul_tiled(const float *X, const uint8_t *w_tiled, int64_t n_tokens,
                     int64_t input_dim, int64_t output_dim, float *Y, void *stream);

/*
 * q4k_gemv_tiled_shaped -- q4k_gemv_tiled with an explicit launch shape:
 * waves per workgroup in {4, 8, 16}, row_groups (consecutive groups of 16
 * rows per workgroup) in 1..4, depth (tiles each wave loads ahead) in
 * {2, 4} ({2} with 16 waves); 0 lets the library choose that value.  Any
 * other value gives Q4K_EINVAL_DIM.  Results are within the q4k_gemv
 * tolerance for every shape.
 */
int q4k_gemv_tiled_shaped(const float *x, const uint8_t *w_tiled, int64_t input_dim,
                          int64_t output_dim, float *y, void *stream, int waves,
                          int row_groups, int depth);

/*
 * q4k_matmul_noalloc -- q4k_matmul for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, kernels, results and
 * error behaviour as q4k_matmul, except that the split tiles' counters and
 * partial tiles live in a fixed scratch array reserved with the library's
 * code object (4 MiB + 4 KiB per GPU, held until the process ends) instead
 * of the library's allocated workspace: the call performs no allocation of
 * any kind.  A call whose tiles would need more scratch than that returns
 * Q4K_ESCRATCH and launches nothing (the library's own choice of input_dim
 * ranges always fits: at most 256 partial tiles of 16 KiB).  Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams, concurrent graphs) race and must be ordered by the
 * caller.  The counters in it start at zero and every call leaves them at
 * zero.
 */
int q4k_matmul_noalloc(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
                       int64_t input_dim, int64_t output_dim, float *Y, void *stream);

/*
 * q4k_matmul_shaped -- q4k_matmul with its kernel forced, for sweeps and
 * tests: form 1 runs the few-token matrix-core GEMV (n_tokens <= 8, any
 * |X| < 2^96); form 16, 32 or 64 runs the prefill tiles with that many
 * weight rows per workgroup (x 16 tokens, any |X| < 2^96) at any token count;
 * form 65 runs 64-row x 16-token tiles whose waves each own whole
 * super-blocks of all 64 rows, with the activations loaded straight into
 * matrix-core operand registers (same arithmetic and range); form 128 runs
 * the 128-row x 32-token tiles with the library's number S of input_dim
 * ranges, and form 128 + S (S = 1..8) fixes it (clamped to at most
 * input_dim/512 ranges, and to 1 from 256 tiles on; same arithmetic and
 * range, workspace as for q4k_matmul); 0 is q4k_matmul itself.  Any other value (or form 1 with more than 8
 * tokens) gives Q4K_EINVAL_DIM.  Results are within the q4k_matmul
 * tolerance for every form.
 */
int q4k_matmul_shaped(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
                      int64_t input_dim, int64_t output_dim, float *Y, void *stream,
                      int form);

/*
 * q4k_matmul_tiled_shaped -- q4k_matmul_tiled with its kernel forced: form
 * as for q4k_matmul_shaped (1 = the few-token GEMV, 16 / 32 / 64 = the
 * prefill tiles, 0 = q4k_matmul_tiled itself; forms 65 and 128 .. 136 are
 * canonical-only and give Q4K_EINVAL_DIM here).
 */
int q4k_matmul_tiled_shaped(const float *X, const uint8_t *w_tiled, int64_t n_tokens,
                            int64_t input_dim, int64_t output_dim, float *Y, void *stream,
                            int form);

/* Static description of a return code; for Q4K_EHIP it includes the HIP
 * error text of the failing call on this host thread. */
const char *q4k_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
