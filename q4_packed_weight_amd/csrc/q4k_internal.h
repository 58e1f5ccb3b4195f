// q4k_internal.h -- declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

// Launch shape of the vector GEMV kernel (Q4_K, Q4_0, Q6_K).
struct GemvShape {
  int lanes = 64;         // lanes spanning the slabs of one row: 16, 32 or 64
  int rows_per_lane = 4;  // rows whose partial sums one lane carries: 1, 2, 4, 8
  int k_waves = 1;        // waves of a workgroup splitting input_dim: 1, 2, 4
  int waves = 4;          // waves per workgroup: 1, 2, 4 (a multiple of k_waves)
};

// min_lanes: 32 for Q6_K, whose 210-byte blocks make whole 16-byte chunks
// only in groups of eight (a step of 32 lanes).
GemvShape choose_gemv_shape(int64_t nb, int64_t N, int rows_per_lane, int k_waves,
                            int waves, int min_lanes = 16);
hipError_t gemv_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                       int64_t N, const GemvShape &s, hipStream_t stream);
// The same kernels on Q4_0 rows: ngroups = input_dim/256 groups of eight
// 18-byte blocks per row.
hipError_t gemv_q4_0_launch(const float *x, const uint8_t *w, float *y, int64_t ngroups,
                            int64_t N, const GemvShape &s, hipStream_t stream);
// The same kernels on Q6_K rows of nb 210-byte blocks (rows need not start
// 16-byte aligned; w must).
hipError_t gemv_q6k_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                           int64_t N, const GemvShape &s, hipStream_t stream);

// The Q4_0 products on the matrix cores (q4_0_gemv_mfma.hip): 16 rows per
// workgroup, rows of at most kQ40MfmaMaxGroups groups of eight blocks (the
// codes enter as fp16 subnormals, as in the Q4_K form below).
constexpr int kQ40MfmaMaxGroups = 256;
hipError_t gemv_q4_0_mfma_launch(const float *x, const uint8_t *w, float *y, int64_t ngroups,
                                 int64_t N, hipStream_t stream);

// Q4_K GEMV with the multiplies on the matrix cores (16 rows per workgroup).
hipError_t gemv_mfma_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                            int64_t N, hipStream_t stream);
// Whether q4k_gemv's automatic choice is the matrix-core form (measured on
// MI355X: it wins with 12 to 19 super-blocks a row, so that every wave owns
// at most one super-block and the row is long enough, and 192 to 256
// workgroups, all resident at once).
bool use_gemv_mfma(int64_t nb, int64_t N);
// The persistent matrix-core walk over canonical rows: workgroups of
// `waves` waves own `row_groups` consecutive groups of 16 rows; each wave
// keeps `depth` units (16 rows x one super-block) loaded ahead.
struct WalkShape {
  int waves = 8;       // 4, 8 or 16
  int row_groups = 1;  // 1 .. 4
  int depth = 2;       // 2 or 4 (4 waves: 4; 16 waves: 2)
};
// Zero fields of the request are chosen by the library.
WalkShape choose_walk_shape(int64_t nb, int64_t N, int waves, int row_groups, int depth);
hipError_t gemv_walk_launch(const float *x, const uint8_t *w, float *y, int64_t nb, int64_t N,
                            const WalkShape &s, hipStream_t stream);
// Whether q4k_gemv's automatic choice is the walk (measured on MI355X: large
// matrices, from output_dim 3072 with input_dim 5120, or output_dim 11008
// with input_dim 4096).
bool use_gemv_walk(int64_t nb, int64_t N);

// The tiled block order (q4k_tiled.hip): bytes of an N-row matrix of nb
// super-blocks per row, the one-time relayout, and the matrix-core GEMV
// that streams it.
struct TiledShape {
  int waves = 8;       // waves per workgroup: 4, 8 or 16
  int row_groups = 1;  // consecutive groups of 16 rows per workgroup: 1 .. 4
  int depth = 4;       // tiles each wave loads ahead: 2 or 4 (16 waves: 2)
};
int64_t tiled_bytes(int64_t nb, int64_t N);
hipError_t relayout_tiled_launch(const uint8_t *w, uint8_t *out, int64_t nb, int64_t N,
                                 hipStream_t stream);
// Zero fields of the request are chosen by the library.
TiledShape choose_tiled_shape(int64_t nb, int64_t N, int waves, int row_groups, int depth);
hipError_t gemv_tiled_launch(const float *x, const uint8_t *wt, float *y, int64_t nb, int64_t N,
                             const TiledShape &s, hipStream_t stream);
// Batched products on tiled weights: 1 <= M <= 8 tokens (one row group per
// workgroup), and the 64-row x 16-token prefill tiles.
hipError_t gemv_tiled_batch_launch(const float *X, const uint8_t *wt, float *Y, int64_t M,
                                   int64_t nb, int64_t N, hipStream_t stream);
hipError_t prefill_tiled_launch(const float *X, const uint8_t *wt, int64_t M, int64_t nb,
                                int64_t N, float *Y, hipStream_t stream, int rows = 0);

hipError_t ternary_launch(const float *x, const uint8_t *codes, float scale,
                          bool apply_scale, int64_t K, int64_t N, float *y,
                          hipStream_t stream);

// Batched ternary product on the matrix cores (ternary_matmul.hip); K a
// multiple of 64, X and codes 16-byte aligned.
hipError_t ternary_matmul_launch(const float *X, const uint8_t *codes, float scale, int64_t M,
                                 int64_t K, int64_t N, float *Y, hipStream_t stream,
                                 int rows = 0);

// rows: weight rows per workgroup (64, 32 or 16); 0 = prefill_rows(M, N).
hipError_t prefill_launch(const float *X, const uint8_t *w, int64_t M,
                          int64_t K, int64_t N, float *Y, hipStream_t stream, int rows = 0);
int prefill_rows(int64_t M, int64_t N);
// The 64-row x 16-token prefill with each wave owning whole super-blocks and
// its activations loaded straight into MFMA operand registers
// (q4k_prefill_direct.hip).
hipError_t prefill_direct_launch(const float *X, const uint8_t *w, int64_t M, int64_t K,
                                 int64_t N, float *Y, hipStream_t stream);
// The same kernel reading tiled weights (q4k_tiled.hip's order): whole tiles
// are staged through LDS into the canonical block layout, same bits.
hipError_t prefill_staged_tiled_launch(const float *X, const uint8_t *wt, int64_t M, int64_t K,
                                       int64_t N, float *Y, hipStream_t stream, int rows = 0);

// The 128-row x 32-token prefill with input_dim split into S ranges across
// workgroups (q4k_prefill_splitk.hip).  With S > 1 it needs a workspace of
// workspace_bytes: kSplitkCounterBytes of counters, zero before the first
// call (every call leaves them zero again), then one partial tile per
// (output tile, range).  Calls sharing a workspace must not overlap in time.
constexpr int kSplitkMaxRanges = 8;
constexpr int64_t kSplitkCounterBytes = 4096;  // one per (tile, wave); S > 1 only below 256 tiles
// below 256 tiles, at most 8 ranges of 16 KiB partial tiles each
constexpr int64_t kSplitkWorkspaceBytes = kSplitkCounterBytes + 255 * 8 * 16384;
struct SplitkPlan {
  int64_t n_rt = 0, n_tt = 0;  // 128-row and 32-token tiles
  int S = 1;                   // ranges of input_dim
  int64_t counter_bytes = 0;   // counters at the start of the workspace
  int64_t workspace_bytes = 0; // 0 when S == 1
};
// ranges: S itself (clamped to 1 .. min(8, nb/2), and 1 from 256 tiles on);
// 0 = the library's choice.
SplitkPlan splitk_plan(int64_t M, int64_t K, int64_t N, int ranges = 0);
bool splitk_fits(int64_t M, int64_t K, int64_t N);
hipError_t prefill_splitk_launch(const float *X, const uint8_t *w, int64_t M, int64_t K,
                                 int64_t N, float *Y, void *workspace, int64_t workspace_bytes,
                                 hipStream_t stream, int ranges = 0);

// 1 <= M <= 8 tokens on the matrix cores (q4k_gemv_batch.hip); X is
// [M][nb*256], Y is [M][N].
hipError_t gemv_batch_launch(const float *X, const uint8_t *w, float *Y, int64_t M, int64_t nb,
                             int64_t N, hipStream_t stream);

}  // namespace q4k
