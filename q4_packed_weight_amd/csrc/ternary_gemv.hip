// ternary_gemv.hip -- BitNet b1.58 ternary matrix-vector product for gfx950.
//
// What it computes (ternary page: SKaiNET issue #1138, "[ternary-f32] Phase
// 2: TernaryF32GemvNative SPI + reference ViewKernel + TernaryF32KernelPack",
// section "Tasks"): t[o] = sum_i code(o,i) * x[i], code = field - 1 with
// field = (byte[i/4] >> 2*(i%4)) & 3, fp32 accumulation; optionally
// y[o] = scale * t[o] with the per-tensor scale applied after the dot.
//
// Same skeleton as the Q4_K GEMV: a lane owns a 16-byte slice of a row (64
// codes) and keeps the 64 activations of that slice in VGPRs while it walks
// R rows.  The code offset is lazy: sum (u - 1)*x = sum u*x - sum x, and the
// activation sum is row-independent, so it is computed once per slice and
// reduced once per wave, not once per row.  Fields are never converted: a
// dword masked with 0x00030003 << 2f holds two fp16 subnormals 4^f*u*2^-24
// that v_fma_mix_f32 multiplies into one of four per-field accumulators;
// the powers of two are removed when the accumulators are combined.  With
// integer activations every partial sum is a multiple of 2^-24 of bounded
// size, so the codes-dot is exact.
//
// A generic kernel (one wave per row, byte loads) serves input_dim not a
// multiple of 64 and unaligned pointers.

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float comp(float4 v, int f) {
  return f == 0 ? v.x : (f == 1 ? v.y : (f == 2 ? v.z : v.w));
}

// ONE: input_dim fits one iteration (n_items <= 64); its loads then leave
// before the rest of the set-up, with no loop around them.
template <int R, bool ONE>
__global__ __launch_bounds__(kThreads) void ternary_gemv_kernel(
    const float *x, const uint8_t *codes, float *__restrict__ y, float scale,
    int apply_scale, int n_items, int64_t N) {
  // x and codes are deliberately not __restrict__: that keeps their loads
  // ordered before the compiler fence that closes each load phase.
  constexpr int S = 64;                     // 16-byte items staged per iteration
  constexpr int SP = S + 1;                 // padded row of the staged layout
  constexpr int XQ = 16 * S / kThreads;     // staged float4 per thread
  // Staged activations: float4 k of item it at slot k*SP + it (consecutive
  // items in consecutive slots for the per-lane reads; the pad spreads the
  // staging writes), and the activation sum of each staged item.
  __shared__ float4 xs4[16 * SP];
  __shared__ float xsum_item[S];

  // The host validates input_dim >= 64 here; saying so lets the compiler
  // fetch every kernel argument in one round trip.
  __builtin_assume(n_items >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t wg_row0 = (int64_t)blockIdx.x * (kThreads / 64) * R;
  const int64_t row0 = wg_row0 + (int64_t)wave * R;
  const int row_bytes = n_items * 16;
  // Range-checked views: rows past N and items past the end read as zeros.
  // The workgroup reads its own 4R rows only; they and x stay below 2^31
  // bytes (input_dim <= 2^24, checked by the host), so the sizes need no
  // 64-bit clamp ahead of the first load.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc32(x, (uint32_t)n_items * 256u);
  const int64_t rows_left = N - wg_row0;
  const __amdgpu_buffer_rsrc_t cr = make_rsrc32(
      codes + wg_row0 * row_bytes,
      (uint32_t)(rows_left < (kThreads / 64) * R ? rows_left : (kThreads / 64) * R) *
          (uint32_t)row_bytes);
  const int wave_off = wave * R * row_bytes;

  // Load phase of iteration it: activations for staging (coalesced), then
  // the 16 code bytes of this lane's item in each of the R rows (coalesced
  // rows).
  float4 xv[XQ];
  uint4 cw[R];
  auto load_phase = [&](int it) {
    const int item_base = it * S;
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int f = tid + kThreads * q;
      xv[q] = load_buf_f4(xr, 4 * (64 * (item_base + (f >> 4)) + 4 * (f & 15)));
    }
    const int i = item_base + lane;
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = load_buf_stream16(cr, wave_off + r * row_bytes + 16 * i);
  };
  if constexpr (ONE) {
    load_phase(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[r][f] = 0.f;
  float xsum = 0.f;

  const int iters = ONE ? 1 : (n_items + S - 1) / S;
  for (int it = 0; it < iters; ++it) {
    if constexpr (!ONE) load_phase(it);
    const int i = it * S + lane;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // Stage the activations and the per-item sums (the 16 float4 of an item
    // sit in 16 aligned lanes).
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int f = tid + kThreads * q;
      const int itm = f >> 4, k = f & 15;
      xs4[k * SP + itm] = xv[q];
      const float part = group_sum<16>(sum4(xv[q]));
      if (k == 0) xsum_item[itm] = part;
    }
    __syncthreads();

    if (i < n_items) {
      float4 xq[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) xq[k] = xs4[k * SP + lane];
      xsum += xsum_item[lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t dw[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // dword t holds positions 16t..16t+15: byte kb, field f -> 16t+4kb+f
          const uint32_t w0 = dw[t];
          const uint32_t w8 = w0 >> 8;
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const uint32_t mask = 0x00030003u << (2 * f);
            const uint32_t a = w0 & mask;  // bytes 0 and 2
            const uint32_t b = w8 & mask;  // bytes 1 and 3
            acc[r][f] = __builtin_fmaf(half_lo(a), comp(xq[4 * t + 0], f), acc[r][f]);
            acc[r][f] = __builtin_fmaf(half_lo(b), comp(xq[4 * t + 1], f), acc[r][f]);
            acc[r][f] = __builtin_fmaf(half_hi(a), comp(xq[4 * t + 2], f), acc[r][f]);
            acc[r][f] = __builtin_fmaf(half_hi(b), comp(xq[4 * t + 3], f), acc[r][f]);
          }
        }
      }
    }
    if (it + 1 < iters) __syncthreads();
  }

  xsum = group_sum<64>(xsum);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // sum u*x in units of 2^-24
    float s = __builtin_fmaf(acc[r][3], 0x1p-6f,
              __builtin_fmaf(acc[r][2], 0x1p-4f,
              __builtin_fmaf(acc[r][1], 0x1p-2f, acc[r][0])));
    s = group_sum<64>(s);
    const int64_t row = row0 + r;
    if (lane == 0 && row < N) {
      const float t = __builtin_fmaf(s, 0x1p24f, -xsum);
      y[row] = apply_scale ? scale * t : t;
    }
  }
}

// Any input_dim % 4 == 0 and any alignment: one wave per row, each lane
// walks bytes lane, lane+64, ...
__global__ __launch_bounds__(kThreads) void ternary_gemv_generic_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ codes,
    float *__restrict__ y, float scale, int apply_scale, int64_t K,
    int64_t N) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const int64_t row_bytes = K / 4;
  const uint8_t *rp = codes + row * row_bytes;
  float acc = 0.f;
  for (int64_t bi = lane; bi < row_bytes; bi += 64) {
    const uint32_t byte = rp[bi];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float c = (float)(int)((byte >> (2 * f)) & 3u) - 1.0f;
      acc = __builtin_fmaf(c, x[4 * bi + f], acc);
    }
  }
  acc = group_sum<64>(acc);
  if (lane == 0) y[row] = apply_scale ? scale * acc : acc;
}

template <int R>
hipError_t launch_fast(const float *x, const uint8_t *codes, float scale,
                       bool apply, int64_t K, int64_t N, float *y,
                       hipStream_t s) {
  const int64_t rows_per_wg = (kThreads / 64) * R;
  const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
  // per-workgroup code offsets must stay below 2^31
  if (rows_per_wg * (K / 4) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (K <= 64 * 64)
    hipLaunchKernelGGL((ternary_gemv_kernel<R, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, x, codes, y, scale, apply ? 1 : 0,
                       (int)(K / 64), N);
  else
    hipLaunchKernelGGL((ternary_gemv_kernel<R, false>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, x, codes, y, scale, apply ? 1 : 0,
                       (int)(K / 64), N);
  return hipGetLastError();
}

}  // namespace

hipError_t ternary_launch(const float *x, const uint8_t *codes, float scale,
                          bool apply_scale, int64_t K, int64_t N, float *y,
                          hipStream_t stream) {
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 16 == 0);
  if (K % 64 == 0 && aligned) {
    // Rows per lane, measured on MI355X (graph-replayed calls over rotating
    // codes, us/call at R = 4 / 2 / 1): 4096x4096 4.25 / 3.88 / 3.96,
    // 14336->4096 10.55 / 8.97 / 10.07, 8192->4096 6.35 / 5.54 / 5.85,
    // 4096->8192 5.44 / 5.15 / 5.81, 14336->8192 13.46 / 13.98 / 17.85,
    // 4096->14336 7.30 / 7.8 / 8.8, 14336->2048 - / 7.78 / 7.25: two waves
    // per SIMD beat one until the grid is large.
    if (N >= 12288 || (N >= 8192 && K >= 12288))
      return launch_fast<4>(x, codes, scale, apply_scale, K, N, y, stream);
    if (N >= 4096) return launch_fast<2>(x, codes, scale, apply_scale, K, N, y, stream);
    return launch_fast<1>(x, codes, scale, apply_scale, K, N, y, stream);
  }
  const int64_t grid = (N + 3) / 4;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ternary_gemv_generic_kernel, dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, x, codes, y, scale,
                     apply_scale ? 1 : 0, K, N);
  return hipGetLastError();
}

}  // namespace q4k
