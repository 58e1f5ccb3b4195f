// q4k_capi.hip -- the C ABI of libq4k.so: argument validation, launch-shape
// selection and dispatch to the kernels.  Declarations and the contract are
// in include/q4k.h.
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "q4k.h"
#include "q4k_internal.h"

namespace {

thread_local char g_hip_detail[256] = "";

int hip_fail(hipError_t e, const char *what) {
  snprintf(g_hip_detail, sizeof g_hip_detail, "%s: %s (%d)", what,
           hipGetErrorString(e), (int)e);
  return Q4K_EHIP;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest input_dim accepted (2^24): every buffer offset a kernel forms
// (up to 128 rows of one workgroup, the whole activation vector) then stays
// below 2^31.
constexpr int64_t kMaxInputDim = (int64_t)1 << 24;


int check_q4k(const void *x, const uint8_t *w, const void *y, int64_t M,
              int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || N <= 0 || K % 256 != 0 || K > kMaxInputDim)
    return Q4K_EINVAL_DIM;
  if (!x || !w || !y) return Q4K_ENULL;
  if (!aligned16(x) || !aligned16(w)) return Q4K_EALIGN;
  return Q4K_OK;
}

int check_ternary(const void *x, const uint8_t *c, const void *y, int64_t K,
                  int64_t N) {
  if (K <= 0 || N <= 0 || K % 4 != 0 || K > kMaxInputDim) return Q4K_EINVAL_DIM;
  if (!x || !c || !y) return Q4K_ENULL;
  return Q4K_OK;
}



// The split-K prefill's workspace, owned by the library: one per device, of
// the largest size any call needs, allocated by the first call that needs
// it (outside stream capture) and never freed or moved, so graphs that
// captured calls keep a valid pointer.  Calls that use it must not overlap
// in time (include/q4k.h).
struct DeviceWorkspace {
  int device;
  void *ptr;
};
std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

hipError_t device_workspace(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  for (const auto &w : g_ws)
    if (w.device == dev) {
      *out = w.ptr;
      return hipSuccess;
    }
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return e;
  if (st != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  void *p = nullptr;
  e = hipMalloc(&p, q4k::kSplitkWorkspaceBytes);
  if (e != hipSuccess) return e;
  // the counters start at zero (every call leaves them zero again); done
  // before any stream can use the workspace
  e = hipMemsetAsync(p, 0, q4k::kSplitkCounterBytes, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return e;
  }
  g_ws.push_back(DeviceWorkspace{dev, p});
  *out = p;
  return hipSuccess;
}

// Scratch of q4k_matmul_noalloc (for callers that cannot allocate): the
// split tiles' counters and up to 256 partial tiles in device memory that
// comes with the code object, one copy per GPU.  Host code uses the address
// hipGetSymbolAddress gives on each device, never the array's name.
constexpr int64_t kNoAllocScratchBytes = q4k::kSplitkCounterBytes + 256 * 16384;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void zero_words_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct DeviceScratch {
  int device;
  void *ptr;
};
std::mutex g_scratch_mutex;
std::vector<DeviceScratch> g_scratch;

// This device's copy of `scratch`, looked up on the first call on the
// device; that call also zeroes the counters with a kernel on its stream
// (capturable, unlike a memset; every later call leaves them zero).
hipError_t device_scratch(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  for (const auto &s : g_scratch)
    if (s.device == dev) {
      *out = s.ptr;
      return hipSuccess;
    }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  const int words = (int)(q4k::kSplitkCounterBytes / 4);
  hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t *>(p), words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  g_scratch.push_back(DeviceScratch{dev, p});
  *out = p;
  return hipSuccess;
}

// The split-K prefill on the library's workspace for this device.
int matmul_splitk(const float *X, const uint8_t *w, int64_t M, int64_t K, int64_t N, float *Y,
                  void *stream, int ranges = 0) {
  if (!q4k::splitk_fits(M, K, N)) return Q4K_EINVAL_DIM;
  const q4k::SplitkPlan p = q4k::splitk_plan(M, K, N, ranges);
  void *ws = nullptr;
  if (p.workspace_bytes > 0) {
    hipError_t e = device_workspace((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_fail(e, "q4k_matmul workspace");
  }
  hipError_t e = q4k::prefill_splitk_launch(X, w, M, K, N, Y, ws, p.workspace_bytes,
                                            (hipStream_t)stream, ranges);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul launch");
}

// Validates an explicit vector-kernel launch shape (see q4k_gemv_shaped).
bool valid_vector_shape(int rows_per_lane, int k_waves, int workgroup_waves) {
  const auto pow2_le = [](int v, int hi) {
    return v == 0 || ((v & (v - 1)) == 0 && v > 0 && v <= hi);
  };
  if (!pow2_le(rows_per_lane, 8) || !pow2_le(k_waves, 4) ||
      !pow2_le(workgroup_waves, 8))
    return false;
  const int wg = workgroup_waves ? workgroup_waves : 4;
  return !(k_waves > wg || (wg == 8 && (k_waves == 4 || rows_per_lane == 8)));
}

}  // namespace

extern "C" {

int q4k_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                    int64_t output_dim, float *y, void *stream,
                    int rows_per_lane, int k_waves, int workgroup_waves) {
  int rc = check_q4k(x, w_blocks, y, 1, input_dim, output_dim);
  if (rc) return rc;
  if (workgroup_waves == 16) {  // the matrix-core form
    if (rows_per_lane != 0 || k_waves != 0) return Q4K_EINVAL_DIM;
    hipError_t e = q4k::gemv_mfma_launch(x, w_blocks, y, input_dim / 256, output_dim,
                                         (hipStream_t)stream);
    return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_gemv launch");
  }
  if (!valid_vector_shape(rows_per_lane, k_waves, workgroup_waves)) return Q4K_EINVAL_DIM;
  const int64_t nb = input_dim / 256;
  const q4k::GemvShape s = q4k::choose_gemv_shape(nb, output_dim, rows_per_lane,
                                                  k_waves, workgroup_waves);
  hipError_t e = q4k::gemv_launch(x, w_blocks, y, nb, output_dim, s,
                                  (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_gemv launch");
}

// Q4_0 rows of input_dim/32 18-byte blocks; a multiple of 256 keeps them
// whole 144-byte groups (validation as for Q4_K).
int q4_0_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                     int64_t output_dim, float *y, void *stream,
                     int rows_per_lane, int k_waves, int workgroup_waves) {
  int rc = check_q4k(x, w_blocks, y, 1, input_dim, output_dim);
  if (rc) return rc;
  const int64_t ng = input_dim / 256;
  if (workgroup_waves == 16) {  // the matrix-core form
    if (rows_per_lane != 0 || k_waves != 0 || ng > q4k::kQ40MfmaMaxGroups) return Q4K_EINVAL_DIM;
    hipError_t e = q4k::gemv_q4_0_mfma_launch(x, w_blocks, y, ng, output_dim,
                                              (hipStream_t)stream);
    return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4_0_gemv launch");
  }
  if (!valid_vector_shape(rows_per_lane, k_waves, workgroup_waves)) return Q4K_EINVAL_DIM;
  const q4k::GemvShape s = q4k::choose_gemv_shape(ng, output_dim, rows_per_lane,
                                                  k_waves, workgroup_waves);
  hipError_t e = q4k::gemv_q4_0_launch(x, w_blocks, y, ng, output_dim, s,
                                       (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4_0_gemv launch");
}

// Measured on MI355X (graph-replayed calls over rotating weights, us/call,
// vector / matrix-core form): the matrix-core form wins on 192 to 256
// workgroups with 12 to 24 groups of eight blocks a row, 3072x3072 3.93 /
// 3.56, 4096->3072 4.03 / 3.66, 3072->4096 4.07 / 3.80, 4096x4096 4.32 /
// 3.93, 4864->4096 6.02 / 4.80, 5120->4096 5.92 / 5.34 (Q4_0 has no walk to
// take over from 20 groups); it loses with 8 groups (2048->4096 3.07 /
// 3.43), on 128 workgroups (4096->2048 3.26 / 3.46) and past 256
// (4096->5120 5.47 / 5.92).
static bool use_q4_0_mfma(int64_t ng, int64_t N) {
  const int64_t grid = (N + 15) / 16;
  return grid >= 192 && grid <= 256 && ng >= 12 && ng <= 24;
}

int q4_0_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
              int64_t output_dim, float *y, void *stream) {
  return q4_0_gemv_shaped(x, w_blocks, input_dim, output_dim, y, stream, 0, 0,
                          use_q4_0_mfma(input_dim / 256, output_dim) ? 16 : 0);
}

// Q6_K rows of input_dim/256 210-byte blocks (validation as for Q4_K).  The
// kernel runs 32 or 64 lanes per row; 64 lanes with 8 rows per lane and a
// 4-way split of input_dim would need more LDS than a CU has.
int q6k_gemv_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                    int64_t output_dim, float *y, void *stream,
                    int rows_per_lane, int k_waves, int workgroup_waves) {
  int rc = check_q4k(x, w_blocks, y, 1, input_dim, output_dim);
  if (rc) return rc;
  if (!valid_vector_shape(rows_per_lane, k_waves, workgroup_waves)) return Q4K_EINVAL_DIM;
  const int64_t nb = input_dim / 256;
  const q4k::GemvShape s = q4k::choose_gemv_shape(nb, output_dim, rows_per_lane,
                                                  k_waves, workgroup_waves, 32);
  if (s.lanes == 64 && s.rows_per_lane == 8 && s.k_waves == 4) return Q4K_EINVAL_DIM;
  hipError_t e = q4k::gemv_q6k_launch(x, w_blocks, y, nb, output_dim, s,
                                      (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q6k_gemv launch");
}

// Measured on MI355X (graph-replayed calls over rotating weights, 13.8 to
// 48 MB per matrix): no split of input_dim across waves (the Q6_K tiles
// leave room for one workgroup per CU only when split) and at most 2 rows
// per lane: 4096x4096 5.6 us, 4096->14336 14.0, 14336->4096 15.4,
// 11008->4096 12.3, against 6.4 / 15.3 / 20.5 / 19.6 with the Q4_K rule.
int q6k_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
             int64_t output_dim, float *y, void *stream) {
  int rc = check_q4k(x, w_blocks, y, 1, input_dim, output_dim);
  if (rc) return rc;
  const q4k::GemvShape s = q4k::choose_gemv_shape(input_dim / 256, output_dim, 0, 1, 0, 32);
  return q6k_gemv_shaped(x, w_blocks, input_dim, output_dim, y, stream,
                         s.rows_per_lane < 2 ? s.rows_per_lane : 2, 1, 0);
}

int q4k_gemv_walk_shaped(const float *x, const uint8_t *w_blocks, int64_t input_dim,
                         int64_t output_dim, float *y, void *stream, int waves,
                         int row_groups, int depth) {
  int rc = check_q4k(x, w_blocks, y, 1, input_dim, output_dim);
  if (rc) return rc;
  if (!(waves == 0 || waves == 4 || waves == 8 || waves == 16) || row_groups < 0 ||
      row_groups > 4 || !(depth == 0 || depth == 2 || depth == 4))
    return Q4K_EINVAL_DIM;
  const q4k::WalkShape s = q4k::choose_walk_shape(input_dim / 256, output_dim, waves,
                                                  row_groups, depth);
  if ((s.waves == 4 && s.depth != 4) || (s.waves == 16 && s.depth != 2)) return Q4K_EINVAL_DIM;
  hipError_t e = q4k::gemv_walk_launch(x, w_blocks, y, input_dim / 256, output_dim, s,
                                       (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_gemv_walk launch");
}

int q4k_gemv(const float *x, const uint8_t *w_blocks, int64_t input_dim,
             int64_t output_dim, float *y, void *stream) {
  if (input_dim > 0 && output_dim > 0 && input_dim % 256 == 0 &&
      q4k::use_gemv_walk(input_dim / 256, output_dim))
    return q4k_gemv_walk_shaped(x, w_blocks, input_dim, output_dim, y, stream, 0, 0, 0);
  return q4k_gemv_shaped(x, w_blocks, input_dim, output_dim, y, stream, 0, 0,
                         q4k::use_gemv_mfma(input_dim / 256, output_dim) ? 16 : 0);
}

// Few tokens run on the batched matrix-core GEMV, one launch of up to 8
// tokens, where it beats the prefill tiles (at the height prefill_rows
// picks).  Measured on MI355X (graph-replayed calls over rotating weights,
// batched / prefill us/call): with output_dim 4096, 16 waves per workgroup
// up to 4 tokens, 8 above: 4096x4096 with 2 tokens 4.9 / 10.4, 3-4 tokens
// 5.9 / 10.4, 5-8 tokens 8.7-8.8 / 10.4; 11008->4096 with 8 tokens 19.2 /
// 23.7; 14336->4096 with 5-8 tokens 21.7-22.6 / 22.0-22.6; 2048->4096 with 6
// tokens 4.9 / 6.6; 4096->2048 with 8 tokens 8.3 / 10.2.  Wider outputs (8
// waves per workgroup) keep the prefill from 3 tokens on (4096->8192 with 3
// tokens 12.6 / 10.7, 4096->14336 with 4 tokens 22.7 / 15.4); 2 tokens win
// everywhere (4096->14336: 13.6 / 16.8).
static bool use_gemv_batch(int64_t M, int64_t K, int64_t N) {
  (void)K;
  return M <= 2 || (M <= 8 && N <= 4096);
}

// Valid explicit forms of the batched products: 1 = the few-token GEMV
// (at most 8 tokens), 16 / 32 / 64 = the prefill tiles with that many
// weight rows per workgroup.
static bool valid_matmul_form(int form, int64_t n_tokens) {
  return (form == 1 && n_tokens <= 8) || form == 16 || form == 32 || form == 64 || form == 65 ||
         (form >= 128 && form <= 128 + q4k::kSplitkMaxRanges);
}

int q4k_matmul_shaped(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
                      int64_t input_dim, int64_t output_dim, float *Y, void *stream, int form) {
  int rc = check_q4k(X, w_blocks, Y, n_tokens, input_dim, output_dim);
  if (rc) return rc;
  if (form == 0) return q4k_matmul(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream);
  if (!valid_matmul_form(form, n_tokens)) return Q4K_EINVAL_DIM;
  if (form >= 128)
    return matmul_splitk(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream, form - 128);
  hipError_t e = form == 1
      ? q4k::gemv_batch_launch(X, w_blocks, Y, n_tokens, input_dim / 256, output_dim,
                               (hipStream_t)stream)
      : form == 65
      ? q4k::prefill_direct_launch(X, w_blocks, n_tokens, input_dim, output_dim, Y,
                                   (hipStream_t)stream)
      : q4k::prefill_launch(X, w_blocks, n_tokens, input_dim, output_dim, Y,
                            (hipStream_t)stream, form);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul launch");
}

// The 128-row x 32-token tiles with input_dim split across workgroups win
// from 33 tokens on, from 17 with output_dim above 4096 and from 9 with
// input_dim from 8192.  Measured on MI355X (graph-replayed calls over
// rotating weights, the other kernels' best / these tiles, us/call):
// 64x4096x4096 17.3 / 16.4, 128x4096x4096 31.3 / 22.1, 512x4096x4096 117.3
// / 67.9, 64x4096->14336 62.7 / 35.5, 64x14336->4096 46.1 / 35.3,
// 32x4096->14336 33.7 / 23.8, 32x4096->8192 18.1 / 17.1, 16x14336->4096
// 36.3 / 23.7, 16x11008->4096 28.6 / 20.5; against 16x4096x4096 12.1 /
// 14.5, 16x4096->14336 20.0 / 22.7 and 24x4096x4096 14.3 / 14.8.
static bool use_splitk(int64_t M, int64_t K, int64_t N) {
  return q4k::splitk_fits(M, K, N) && M >= 9 && (M > 32 || K >= 8192 || (M > 16 && N > 4096));
}

int q4k_matmul(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
               int64_t input_dim, int64_t output_dim, float *Y, void *stream) {
  int rc = check_q4k(X, w_blocks, Y, n_tokens, input_dim, output_dim);
  if (rc) return rc;
  if (n_tokens == 1) return q4k_gemv(X, w_blocks, input_dim, output_dim, Y, stream);
  if (use_splitk(n_tokens, input_dim, output_dim))
    return matmul_splitk(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream);
  if (use_gemv_batch(n_tokens, input_dim, output_dim)) {
    hipError_t e = q4k::gemv_batch_launch(X, w_blocks, Y, n_tokens, input_dim / 256, output_dim,
                                          (hipStream_t)stream);
    return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul launch");
  }
  hipError_t e = q4k::prefill_launch(X, w_blocks, n_tokens, input_dim,
                                     output_dim, Y, (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul launch");
}

int q4k_matmul_noalloc(const float *X, const uint8_t *w_blocks, int64_t n_tokens,
                       int64_t input_dim, int64_t output_dim, float *Y, void *stream) {
  int rc = check_q4k(X, w_blocks, Y, n_tokens, input_dim, output_dim);
  if (rc) return rc;
  // every other kernel q4k_matmul may pick uses no scratch and allocates nothing
  if (!use_splitk(n_tokens, input_dim, output_dim))
    return q4k_matmul(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream);
  const q4k::SplitkPlan p = q4k::splitk_plan(n_tokens, input_dim, output_dim);
  if (p.workspace_bytes > kNoAllocScratchBytes) {
    snprintf(g_hip_detail, sizeof g_hip_detail,
             "q4k_matmul_noalloc: the split tiles need %lld bytes of scratch, more than the "
             "%lld reserved", (long long)p.workspace_bytes, (long long)kNoAllocScratchBytes);
    return Q4K_ESCRATCH;
  }
  void *ws = nullptr;
  if (p.workspace_bytes > 0) {
    hipError_t e = device_scratch((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_fail(e, "q4k_matmul_noalloc scratch");
  }
  hipError_t e = q4k::prefill_splitk_launch(X, w_blocks, n_tokens, input_dim, output_dim, Y, ws,
                                            kNoAllocScratchBytes, (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul_noalloc launch");
}

int ternary_gemv_codes(const float *x, const uint8_t *codes, int64_t input_dim,
                       int64_t output_dim, float *y, void *stream) {
  int rc = check_ternary(x, codes, y, input_dim, output_dim);
  if (rc) return rc;
  hipError_t e = q4k::ternary_launch(x, codes, 1.0f, false, input_dim,
                                     output_dim, y, (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "ternary_gemv_codes launch");
}

int ternary_gemv(const float *x, const uint8_t *codes, float scale,
                 int64_t input_dim, int64_t output_dim, float *y,
                 void *stream) {
  int rc = check_ternary(x, codes, y, input_dim, output_dim);
  if (rc) return rc;
  hipError_t e = q4k::ternary_launch(x, codes, scale, true, input_dim,
                                     output_dim, y, (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "ternary_gemv launch");
}

// Batched ternary product: one token is ternary_gemv; rows of whole 16-byte
// code chunks with aligned X and codes run on the matrix-core tiles (every
// code byte read once per 16 tokens); anything else is the ternary page's
// row loop, one ternary_gemv launch per token row.  The row loop also wins
// for very few tokens (measured on MI355X, graph-replayed calls over
// rotating codes, loop / tiles at the height prefill_rows picks: 4096x4096
// with 2 tokens 8.1 / 10.9 and with 3 tokens 12.1 / 10.9; 14336->4096 with
// 3 tokens 31.1 / 33.7 and with 4 tokens 41.0 / 33.7).
static bool ternary_row_loop_wins(int64_t M, int64_t K) {
  return M <= 2 || (M <= 3 && K > 8192);
}

// Every launch of the loop has the same dimensions, so a launch that the
// library itself rejects is rejected for the first row, before anything is
// written; only a failure reported by the HIP runtime part-way through can
// leave earlier token rows written (include/q4k.h, ternary_matmul).
static int ternary_row_loop(const float *X, const uint8_t *codes, float scale, int64_t n_tokens,
                            int64_t input_dim, int64_t output_dim, float *Y, void *stream) {
  for (int64_t r = 0; r < n_tokens; ++r) {
    hipError_t e = q4k::ternary_launch(X + r * input_dim, codes, scale, true, input_dim,
                                       output_dim, Y + r * output_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ternary_matmul launch");
  }
  return Q4K_OK;
}

// form 1 = the row loop of ternary_gemv launches; 16 / 32 / 64 = the matrix-
// core tiles with that many rows per workgroup (input_dim a multiple of 64,
// X and codes 16-byte aligned); 0 = ternary_matmul's own choice.
int ternary_matmul_shaped(const float *X, const uint8_t *codes, float scale, int64_t n_tokens,
                          int64_t input_dim, int64_t output_dim, float *Y, void *stream,
                          int form) {
  if (n_tokens <= 0) return Q4K_EINVAL_DIM;
  int rc = check_ternary(X, codes, Y, input_dim, output_dim);
  if (rc) return rc;
  if (form == 0) return ternary_matmul(X, codes, scale, n_tokens, input_dim, output_dim, Y, stream);
  if (form == 1)
    return ternary_row_loop(X, codes, scale, n_tokens, input_dim, output_dim, Y, stream);
  if ((form != 16 && form != 32 && form != 64) || input_dim % 64 != 0) return Q4K_EINVAL_DIM;
  if (!aligned16(X) || !aligned16(codes)) return Q4K_EALIGN;
  hipError_t e = q4k::ternary_matmul_launch(X, codes, scale, n_tokens, input_dim, output_dim, Y,
                                            (hipStream_t)stream, form);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "ternary_matmul launch");
}

int ternary_matmul(const float *X, const uint8_t *codes, float scale, int64_t n_tokens,
                   int64_t input_dim, int64_t output_dim, float *Y, void *stream) {
  if (n_tokens <= 0) return Q4K_EINVAL_DIM;
  int rc = check_ternary(X, codes, Y, input_dim, output_dim);
  if (rc) return rc;
  if (n_tokens == 1) return ternary_gemv(X, codes, scale, input_dim, output_dim, Y, stream);
  if (input_dim % 64 == 0 && aligned16(X) && aligned16(codes) &&
      !ternary_row_loop_wins(n_tokens, input_dim)) {
    hipError_t e = q4k::ternary_matmul_launch(X, codes, scale, n_tokens, input_dim, output_dim,
                                              Y, (hipStream_t)stream);
    return e == hipSuccess ? Q4K_OK : hip_fail(e, "ternary_matmul launch");
  }
  return ternary_row_loop(X, codes, scale, n_tokens, input_dim, output_dim, Y, stream);
}

int64_t q4k_tiled_size(int64_t input_dim, int64_t output_dim) {
  if (input_dim <= 0 || output_dim <= 0 || input_dim % 256 != 0 || input_dim > kMaxInputDim)
    return Q4K_EINVAL_DIM;
  return q4k::tiled_bytes(input_dim / 256, output_dim);
}

int q4k_relayout_tiled(const uint8_t *w_blocks, int64_t input_dim, int64_t output_dim,
                       uint8_t *w_tiled, void *stream) {
  int rc = check_q4k(w_blocks, w_blocks, w_tiled, 1, input_dim, output_dim);
  if (rc) return rc;
  if (!aligned16(w_tiled)) return Q4K_EALIGN;
  hipError_t e = q4k::relayout_tiled_launch(w_blocks, w_tiled, input_dim / 256, output_dim,
                                            (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_relayout_tiled launch");
}

int q4k_gemv_tiled_shaped(const float *x, const uint8_t *w_tiled, int64_t input_dim,
                          int64_t output_dim, float *y, void *stream, int waves,
                          int row_groups, int depth) {
  int rc = check_q4k(x, w_tiled, y, 1, input_dim, output_dim);
  if (rc) return rc;
  if (!(waves == 0 || waves == 4 || waves == 8 || waves == 16) || row_groups < 0 ||
      row_groups > 4 || !(depth == 0 || depth == 2 || depth == 4) ||
      (waves == 16 && depth == 4))
    return Q4K_EINVAL_DIM;
  const q4k::TiledShape s = q4k::choose_tiled_shape(input_dim / 256, output_dim, waves,
                                                    row_groups, depth);
  hipError_t e = q4k::gemv_tiled_launch(x, w_tiled, y, input_dim / 256, output_dim, s,
                                        (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_gemv_tiled launch");
}

int q4k_gemv_tiled(const float *x, const uint8_t *w_tiled, int64_t input_dim,
                   int64_t output_dim, float *y, void *stream) {
  return q4k_gemv_tiled_shaped(x, w_tiled, input_dim, output_dim, y, stream, 0, 0, 0);
}

// On tiled weights the batched kernel streams its tiles without LDS staging
// and wins over the prefill tiles further out than on canonical weights.
// Measured (graph-replayed calls over rotating tiled copies, batched /
// prefill at the height prefill_rows picks, us/call): 4096x4096 with 8
// tokens 8.6 / 9.9; 14336->4096 with 8 tokens 22.1 / 30.3; 4096->14336
// with 4 tokens 15.6 / 16.0 and with 5 tokens 16.1 / 16.0; 4096->8192 with
// 4 tokens 9.2 / 12.1 and with 5 to 8 tokens 12.6-12.8 / 12.0.
static bool use_tiled_batch(int64_t M, int64_t K, int64_t N) {
  return M <= 4 || (M <= 8 && N <= 4096 && K >= 4096);
}

int q4k_matmul_tiled_shaped(const float *X, const uint8_t *w_tiled, int64_t n_tokens,
                            int64_t input_dim, int64_t output_dim, float *Y, void *stream,
                            int form) {
  int rc = check_q4k(X, w_tiled, Y, n_tokens, input_dim, output_dim);
  if (rc) return rc;
  if (form == 0) return q4k_matmul_tiled(X, w_tiled, n_tokens, input_dim, output_dim, Y, stream);
  if (!valid_matmul_form(form, n_tokens) || form == 65 || form >= 128) return Q4K_EINVAL_DIM;
  hipError_t e = form == 1
      ? q4k::gemv_tiled_batch_launch(X, w_tiled, Y, n_tokens, input_dim / 256, output_dim,
                                     (hipStream_t)stream)
      : q4k::prefill_tiled_launch(X, w_tiled, n_tokens, input_dim / 256, output_dim, Y,
                                  (hipStream_t)stream, form);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul_tiled launch");
}

// One token is q4k_gemv_tiled, a few tokens the batched kernel, more the
// prefill tiles.
int q4k_matmul_tiled(const float *X, const uint8_t *w_tiled, int64_t n_tokens, int64_t input_dim,
                     int64_t output_dim, float *Y, void *stream) {
  int rc = check_q4k(X, w_tiled, Y, n_tokens, input_dim, output_dim);
  if (rc) return rc;
  if (n_tokens == 1) return q4k_gemv_tiled(X, w_tiled, input_dim, output_dim, Y, stream);
  if (use_tiled_batch(n_tokens, input_dim, output_dim)) {
    hipError_t e = q4k::gemv_tiled_batch_launch(X, w_tiled, Y, n_tokens, input_dim / 256,
                                                output_dim, (hipStream_t)stream);
    return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul_tiled launch");
  }
  hipError_t e = q4k::prefill_tiled_launch(X, w_tiled, n_tokens, input_dim / 256, output_dim, Y,
                                           (hipStream_t)stream);
  return e == hipSuccess ? Q4K_OK : hip_fail(e, "q4k_matmul_tiled launch");
}

const char *q4k_strerror(int code) {
  switch (code) {
    case Q4K_OK: return "ok";
    case Q4K_EINVAL_DIM:
      return "invalid dimension: every dimension must be > 0, input_dim a "
             "multiple of 256 for Q4_K, Q4_0 and Q6_K (of 4 for ternary) and at "
             "most 2^24";
    case Q4K_ENULL: return "a required pointer is NULL";
    case Q4K_EALIGN: return "x and the Q4_K, Q4_0 or Q6_K blocks must be 16-byte aligned";
    case Q4K_EHIP: return g_hip_detail[0] ? g_hip_detail : "HIP runtime error";
    case Q4K_ESCRATCH:
      return g_hip_detail[0] ? g_hip_detail
                             : "q4k_matmul_noalloc: the call needs more than its fixed scratch";
    default: return "unknown error code";
  }
}

}  // extern "C"
