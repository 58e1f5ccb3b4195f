// q4k_gemv.hip -- fused-dequantize Q4_K matrix-vector product for gfx950.
//
// What it computes (Q4_K page: SKaiNET PR #562, "feat(kernel): SIMD-fused
// Q4_K matmul kernel + Q4KMatmulKernel SPI", sections "Summary" and
// "Pipeline"):  y[o] = sum over super-blocks b and sub-blocks s of
//     d*sc[s] * sum_l q[l]*x[l]  -  dmin*m[s] * sum_l x[l]
// i.e. the lazy-dmin form: the offset term uses the activation sum of the
// sub-block instead of dequantizing each weight.
//
// Work mapping (MI355X, wave64):
//   * A lane owns one "slab" of a super-block: the 32 qs bytes 32j..32j+31,
//     i.e. 32 positions of sub-block 2j (low nibbles) and of sub-block 2j+1
//     (high nibbles) -- one byte load feeds both nibble accumulators, as on
//     the page.  A super-block is 4 slabs, so L lanes cover L/4 blocks.
//   * The 64 activations a slab needs stay in VGPRs while the lane walks R
//     rows (x reuse across rows), and their two sub-block sums (the lazy-dmin
//     input sums) are computed once per slab, not once per row.
//   * L = 16, 32 or 64 lanes span the slabs of one row (small input_dim packs
//     64/L rows into one wave instruction); KW waves of a workgroup split the
//     slab range of the same rows and combine through LDS.
//   * Weights arrive as three 16-byte non-temporal loads per (row, slab):
//     the block header (d, dmin, packed scales) and the two halves of the
//     slab.  All loads of a step are issued before any arithmetic.
//   * Nibbles never go through an integer->float convert: a masked dword
//     (w & 0x000F000F) is two fp16 subnormals q*2^-24, multiplied into fp32
//     accumulators by v_fma_mix_f32; high nibbles are masked in place
//     (w & 0x00F000F0 = 16q*2^-24).  The powers of two are folded back into
//     the scales, so the arithmetic is exact up to fp32 accumulation.
//   * Per-row partial sums are reduced across the L lanes with DPP, then
//     across the KW waves through LDS.  Each output has exactly one writer.

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int kThreads = 256;

// Per-lane decoded header values for the lane's two sub-blocks.
struct SlabScales {
  float d, dmin, sc_lo16, sc_hi, m_lo, m_hi;
};

// Decode d, dmin and the scale/min pair of sub-blocks 2j and 2j+1 from a
// 16-byte block header.  `sh` = 16*(j&1) selects the byte pair inside each
// scale dword and `jhi` = (j >= 2) selects the 4+2-bit packing of
// sub-blocks 4..7; both are fixed per lane.
__device__ __forceinline__ SlabScales decode_header(uint4 h, uint32_t sh,
                                                    bool jhi) {
  // h.y = S[0..3], h.z = S[4..7], h.w = S[8..11]
  const uint32_t p1 = h.y >> sh;  // S[2j'], S[2j'+1] with j' = j & 1
  const uint32_t p2 = h.z >> sh;  // S[2j'+4], S[2j'+5]
  const uint32_t t3 = h.w >> sh;  // S[2j'+8], S[2j'+9]
  const uint32_t lo_src_sc = jhi ? t3 : p1;
  const uint32_t lo_src_m = jhi ? (t3 >> 4) : p2;
  const uint32_t mask_lo = jhi ? 0x0F0Fu : 0x3F3Fu;
  const uint32_t mask_hi = jhi ? 0x3030u : 0u;
  const uint32_t scp = (lo_src_sc & mask_lo) | ((p1 >> 2) & mask_hi);
  const uint32_t mp = (lo_src_m & mask_lo) | ((p2 >> 2) & mask_hi);
  SlabScales s;
  s.d = half_lo(h.x);
  s.dmin = half_hi(h.x);
  s.sc_lo16 = (float)(scp & 0xFFu) * 16.0f;
  s.sc_hi = (float)((scp >> 8) & 0xFFu);
  s.m_lo = (float)(mp & 0xFFu);
  s.m_hi = (float)((mp >> 8) & 0xFFu);
  return s;
}

// Code dots of one qs dword (slab bytes 4t..4t+3): low nibbles against
// xl[0..3], high nibbles against xh[0..3].  acc_lo is in units of 2^-24,
// acc_hi in units of 2^-20 (the high nibble is used in place, times 16).
__device__ __forceinline__ void nibble_dots(uint32_t w, float4 xl, float4 xh,
                                            float &acc_lo, float &acc_hi) {
  const uint32_t lo02 = w & 0x000F000Fu;
  const uint32_t hi02 = w & 0x00F000F0u;
  const uint32_t w8 = w >> 8;
  const uint32_t lo13 = w8 & 0x000F000Fu;
  const uint32_t hi13 = w8 & 0x00F000F0u;
  acc_lo = __builtin_fmaf(half_lo(lo02), xl.x, acc_lo);
  acc_hi = __builtin_fmaf(half_lo(hi02), xh.x, acc_hi);
  acc_lo = __builtin_fmaf(half_lo(lo13), xl.y, acc_lo);
  acc_hi = __builtin_fmaf(half_lo(hi13), xh.y, acc_hi);
  acc_lo = __builtin_fmaf(half_hi(lo02), xl.z, acc_lo);
  acc_hi = __builtin_fmaf(half_hi(hi02), xh.z, acc_hi);
  acc_lo = __builtin_fmaf(half_hi(lo13), xl.w, acc_lo);
  acc_hi = __builtin_fmaf(half_hi(hi13), xh.w, acc_hi);
}

__device__ __forceinline__ float sum4(float4 v) { return (v.x + v.y) + (v.z + v.w); }

template <int L, int R, int KW>
__global__ __launch_bounds__(kThreads) void q4k_gemv_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ w,
    float *__restrict__ y, int nb, int64_t N) {
  constexpr int G = 64 / L;         // rows side by side in one wave instruction
  constexpr int RG = (kThreads / 64) / KW;  // row groups (of KW waves) per workgroup
  constexpr int ROWS_W = G * R;     // rows per wave
  __shared__ float partial[KW > 1 ? (kThreads / 64) * ROWS_W * 2 : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = wave % KW;
  const int rg = wave / KW;
  const int g = lane / L;
  const int u = lane % L;
  const int64_t row0 = (int64_t)blockIdx.x * (RG * ROWS_W) + (int64_t)rg * ROWS_W;
  const int n_slabs = 4 * nb;
  const int steps = (n_slabs + L - 1) / L;
  const int64_t row_bytes = (int64_t)nb * kBlockBytes;

  float acc_c[R], acc_m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc_c[r] = acc_m[r] = 0.0f;

  for (int t = kw; t < steps; t += KW) {
    const int i = t * L + u;
    // Lanes past the last slab of a row add nothing; the whole slab body is
    // predicated on this (no zero fill needed).
    if (i >= n_slabs) continue;
    const int b = i >> 2;
    const int j = i & 3;
    const uint32_t sh = (uint32_t)(j & 1) * 16u;
    const bool jhi = j >= 2;

    // Weight loads for all R rows first (the HBM stream), then activations.
    // Rows past N read row N-1 instead: their sums are never stored.
    uint4 hdr[R], q0[R], q1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t row = row0 + (int64_t)r * G + g;
      row = row < N ? row : N - 1;
      const uint8_t *blk = w + row * row_bytes + (int64_t)b * kBlockBytes;
      hdr[r] = load_stream16(blk);
      q0[r] = load_stream16(blk + 16 + 32 * j);
      q1[r] = load_stream16(blk + 32 + 32 * j);
    }
    float4 xl[8], xh[8];
    const float *xs = x + 256 * (int64_t)b + 64 * j;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xl[k] = load_f4(xs + 4 * k);
      xh[k] = load_f4(xs + 32 + 4 * k);
    }
    // Lazy-dmin input sums of the two sub-blocks, once per slab.
    float xsum_lo = 0.f, xsum_hi = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xsum_lo += sum4(xl[k]);
      xsum_hi += sum4(xh[k]);
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s_lo = 0.f, s_hi = 0.f;
      const uint32_t qw[8] = {q0[r].x, q0[r].y, q0[r].z, q0[r].w,
                              q1[r].x, q1[r].y, q1[r].z, q1[r].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) nibble_dots(qw[k], xl[k], xh[k], s_lo, s_hi);
      const SlabScales sc = decode_header(hdr[r], sh, jhi);
      // code part in units of 2^-20: 16*sc_lo*s_lo + sc_hi*s_hi
      const float tc = __builtin_fmaf(sc.sc_lo16, s_lo, sc.sc_hi * s_hi);
      const float tm = __builtin_fmaf(sc.m_lo, xsum_lo, sc.m_hi * xsum_hi);
      acc_c[r] = __builtin_fmaf(sc.d, tc, acc_c[r]);
      acc_m[r] = __builtin_fmaf(sc.dmin, tm, acc_m[r]);
    }
  }

  // Reduce each row over the L lanes of its group.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc_c[r] = group_sum<L>(acc_c[r]);
    acc_m[r] = group_sum<L>(acc_m[r]);
  }

  if constexpr (KW == 1) {
    if (u == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + (int64_t)r * G + g;
        if (row < N) y[row] = __builtin_fmaf(acc_c[r], 0x1p20f, -acc_m[r]);
      }
    }
  } else {
    // partial[wave][row_in_wave][c|m]
    if (u == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = (wave * ROWS_W + r * G + g) * 2;
        partial[idx] = acc_c[r];
        partial[idx + 1] = acc_m[r];
      }
    }
    __syncthreads();
    if (kw == 0 && lane < ROWS_W) {
      float c = 0.f, m = 0.f;
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int idx = ((wave + k) * ROWS_W + lane) * 2;
        c += partial[idx];
        m += partial[idx + 1];
      }
      const int64_t row = row0 + lane;
      if (row < N) y[row] = __builtin_fmaf(c, 0x1p20f, -m);
    }
  }
}

template <int L, int R, int KW>
hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, int nb,
                       int64_t N, hipStream_t stream) {
  constexpr int G = 64 / L;
  constexpr int RG = (kThreads / 64) / KW;
  constexpr int64_t rows_per_wg = (int64_t)RG * G * R;
  const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((q4k_gemv_kernel<L, R, KW>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, x, w, y, nb, N);
  return hipGetLastError();
}

template <int L, int R>
hipError_t launch_kw(int kw, const float *x, const uint8_t *w, float *y,
                     int nb, int64_t N, hipStream_t s) {
  switch (kw) {
    case 1: return launch_gemv<L, R, 1>(x, w, y, nb, N, s);
    case 2: return launch_gemv<L, R, 2>(x, w, y, nb, N, s);
    default: return launch_gemv<L, R, 4>(x, w, y, nb, N, s);
  }
}

template <int L>
hipError_t launch_r(int r, int kw, const float *x, const uint8_t *w, float *y,
                    int nb, int64_t N, hipStream_t s) {
  switch (r) {
    case 1: return launch_kw<L, 1>(kw, x, w, y, nb, N, s);
    case 2: return launch_kw<L, 2>(kw, x, w, y, nb, N, s);
    case 4: return launch_kw<L, 4>(kw, x, w, y, nb, N, s);
    default: return launch_kw<L, 8>(kw, x, w, y, nb, N, s);
  }
}

}  // namespace

GemvShape choose_gemv_shape(int64_t nb, int64_t N, int rows_per_lane,
                            int k_waves) {
  GemvShape s;
  const int64_t slabs = 4 * nb;
  s.lanes = slabs <= 16 ? 16 : (slabs <= 32 ? 32 : 64);
  const int64_t steps = (slabs + s.lanes - 1) / s.lanes;
  const int64_t g = 64 / s.lanes;
  if (k_waves > 0) {
    s.k_waves = k_waves;
  } else {
    s.k_waves = steps >= 4 ? 4 : (steps >= 2 ? 2 : 1);
  }
  if (rows_per_lane > 0) {
    s.rows_per_lane = rows_per_lane;
  } else {
    // Enough waves to give every SIMD of the 256 CUs at least one.
    const int64_t target_waves = 1024;
    int r = 4;
    while (r > 1 && (N + g * r - 1) / (g * r) * s.k_waves < target_waves) r /= 2;
    s.rows_per_lane = r;
  }
  return s;
}

hipError_t gemv_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                       int64_t N, const GemvShape &s, hipStream_t stream) {
  const int nbi = (int)nb;
  switch (s.lanes) {
    case 16: return launch_r<16>(s.rows_per_lane, s.k_waves, x, w, y, nbi, N, stream);
    case 32: return launch_r<32>(s.rows_per_lane, s.k_waves, x, w, y, nbi, N, stream);
    default: return launch_r<64>(s.rows_per_lane, s.k_waves, x, w, y, nbi, N, stream);
  }
}

}  // namespace q4k
