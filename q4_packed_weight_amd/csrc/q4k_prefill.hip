// q4k_prefill.hip -- batched (prefill) Q4_K product Y = X W^T.
//
// Provisional form: one GEMV launch per token row (the row loop of the
// ternary page's prefill path).  It re-reads W once per token.
#include "q4k_internal.h"

namespace q4k {

hipError_t prefill_launch(const float *X, const uint8_t *w, int64_t M,
                          int64_t K, int64_t N, float *Y, hipStream_t stream) {
  const int64_t nb = K / 256;
  const GemvShape s = choose_gemv_shape(nb, N, 0, 0, 0);
  for (int64_t r = 0; r < M; ++r) {
    hipError_t e = gemv_launch(X + r * K, w, Y + r * N, nb, N, s, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace q4k
