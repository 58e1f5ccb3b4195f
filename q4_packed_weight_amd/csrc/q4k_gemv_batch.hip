// q4k_gemv_batch.hip -- Q4_K product for a few tokens at once (2 to 8) on
// the gfx950 matrix cores: the decode-batch regime between the batch-1
// GEMV and the 16-token prefill tiles.
//
// What it computes is q4k_matmul's product (Q4_K page: SKaiNET PR #562,
// "feat(kernel): SIMD-fused Q4_K matmul kernel + Q4KMatmulKernel SPI",
// sections "Summary" and "Pipeline", applied to every token row as in the
// ternary page's prefill row loop, SKaiNET issue #1138, section "Tasks"):
//     Y[t, o] = sum_b d * sum_s sc_s * sum_l q * X[t, k] - dmin * m_s * sum_l X[t, k].
// Every weight byte is read once for all tokens of the call.
//
// Layout: a workgroup owns 16 weight rows (the MFMA's column tile); its 8
// or 16 waves split the row's super-blocks and walk them one at a time, loading
// the next one ahead (coalesced 16-byte loads into a wave-private LDS tile).
// The nibbles enter the MFMA's B operand masked into fp16 subnormals (q *
// 2^-24 low, 16q * 2^-24 high), or as exact normal codes for very long rows
// (code_operand_pair).  The A operand's 16 rows carry the
// tokens: row 2t the fp16 hi part of token t's activations, row 2t + 1 the
// lo part (hi = fp16(x), lo = fp16(x - hi), both exact), so one 16x16x32
// MFMA serves up to 8 tokens and every product is exact.  Before the split
// each token's 256 activations of a super-block are scaled by a power of
// two that puts their largest |x| in [2^14, 2^15) (no fp16 overflow for any
// |x| < 2^96); it is undone once per token and super-block.
//
// Lane (n = lane % 16, g = lane / 16) holds D rows 4g .. 4g+3 of row n, i.e.
// the hi and lo dots of tokens 2g and 2g + 1, and applies all eight
// sub-block scales of row n to them in fp32 with the lazy-dmin term; at the
// end the waves are summed in a fixed order (one writer per output).
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int MB_ROWS = 16;                      // rows per workgroup
// Waves per workgroup: 8, or 16 for up to 4 tokens when the grid fills the
// 256 CUs at most once and rows hold at least 16 super-blocks (four waves per
// SIMD, so that one wave's LDS and MFMA latencies hide under another's work).
// Measured (graph-replayed calls over rotating weights, us/call, 8 / 16
// waves): 2x4096x4096 6.15 / 4.84, 4x4096x4096 6.85 / 5.84, 4x11008->4096
// 14.2 / 13.0, 4x14336->4096 17.1 / 17.6 (even within noise), but
// 2x4096->14336 (896 workgroups) 14.6 / 15.5 and 4x2048->4096 (8
// super-blocks a row, half the waves idle) 4.02 / 5.00.
constexpr int MB_WCH = MB_ROWS * 9;              // 16-byte weight pieces per super-block
constexpr int MB_WPL = (MB_WCH + 63) / 64;       // weight loads per lane
// LDS dwords per staged row, unpadded: each lane's 16-byte chunk lands in
// one contiguous 16-byte store and the operand reads of 16 rows hit
// distinct banks (no bank conflict cycles, against 4 per chunk store and 2
// per code read with rows of 38)
constexpr int MB_WROW = 36;

// T: tokens of the launch, 2, 4 or 8 (rows of X past M read as zeros); NC:
// exact normal code operands (rows of more than 256 super-blocks)
template <int T, bool NC, int MB_WAVES>
__global__ __launch_bounds__(64 * MB_WAVES) void q4k_gemv_batch_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, int M, int nb, int N) {
  // Per wave: the staged weight rows of its super-block, each token's fp16 hi
  // and lo activations of it (operand order: pairs (0,2), (1,3), (4,6),
  // (5,7) of every 8), their sums per sub-block and the token's scaling
  // exponent; then the waves' partial outputs.
  __shared__ __align__(16) uint32_t wt[MB_WAVES][MB_ROWS * MB_WROW];
  // [wave][2t] token t's hi part, [wave][2t + 1] its lo part, rows of 136
  // dwords: the A rows of all lane groups, read by one instruction, then
  // fall in different banks (measured with the bank conflict counter: no
  // conflict cycles for 2, 4 or 8 tokens, against 4 to 28 per read with
  // rows of 128 or 132)
  __shared__ __align__(16) uint32_t xhl[MB_WAVES][2 * T][136];
  __shared__ __align__(16) float xs[MB_WAVES][T][8];
  __shared__ int xe[MB_WAVES][T];
  __shared__ float part[MB_WAVES][T][MB_ROWS];

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // weight row of the tile; A row
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7; tokens 2g, 2g+1
  const int row0 = blockIdx.x * MB_ROWS;
  const int K = nb * 256;
  const int row_bytes = nb * kBlockBytes;
  // this wave's super-blocks [b_lo, b_hi)
  const int b_lo = (nb * wave) / MB_WAVES;
  const int n_chunks = (nb * (wave + 1)) / MB_WAVES - b_lo;

  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)min(N - row0, MB_ROWS) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (int64_t)M * K * 4);

  int woff[MB_WPL];
#pragma unroll
  for (int m = 0; m < MB_WPL; ++m) {
    const int q = min(lane + 64 * m, MB_WCH - 1);
    const int row = q / 9;
    woff[m] = row * row_bytes + 16 * (q - 9 * row);
  }
  uint4 wa[MB_WPL], wb[MB_WPL];
  float4 xa[T], xb[T];
  auto load_x = [&](int c, float4 (&xv)[T]) {
    const int b0 = __builtin_amdgcn_readfirstlane(b_lo + c);  // wave-uniform
#pragma unroll
    for (int t = 0; t < T; ++t) xv[t] = load_buf_f4(xr, t * K * 4 + 16 * lane, 1024 * b0);
  };
  auto load_w = [&](int c, uint4 (&wv)[MB_WPL]) {
    const int b0 = __builtin_amdgcn_readfirstlane(b_lo + c);  // wave-uniform
#pragma unroll
    for (int m = 0; m < MB_WPL; ++m) wv[m] = load_buf_stream16(wr, woff[m], kBlockBytes * b0);
  };

  uint32_t *wtw = wt[wave];
  auto stage_chunk = [&](const uint4 (&wv)[MB_WPL], const float4 (&xv)[T]) {
    // the activations first: they were loaded first (and come from L2), so
    // their split runs while the weight bytes are still arriving
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4 v0 = xv[t];  // positions 4 lane .. 4 lane + 3
      const float mx = wave_max_nonneg_v(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))));
      const int e = __builtin_amdgcn_frexp_expf(mx) - 15;  // |x| * 2^-e < 2^15
      const float4 v = make_float4(__builtin_ldexpf(v0.x, -e), __builtin_ldexpf(v0.y, -e),
                                   __builtin_ldexpf(v0.z, -e), __builtin_ldexpf(v0.w, -e));
      half2_t h02, h13;
      h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
      h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
      const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
      *reinterpret_cast<uint2 *>(&xhl[wave][2 * t][2 * lane]) = make_uint2(hw02, hw13);
      *reinterpret_cast<uint2 *>(&xhl[wave][2 * t + 1][2 * lane]) =
          make_uint2(lo_pair(hw02, v.x, v.z), lo_pair(hw13, v.y, v.w));
      // sub-block lane / 8: 8 aligned lanes, which all hold the same sum
      xs[wave][t][lane >> 3] = group_sum<8>(sum4(v0));
      xe[wave][t] = e;  // every lane, one value
    }
#pragma unroll
    for (int m = 0; m < MB_WPL; ++m) {
      const int q = lane + 64 * m;
      if (MB_WCH % 64 != 0 && q >= MB_WCH) break;  // only the last load is partial
      const int row = q / 9;
      uint32_t *dst = &wtw[row * MB_WROW + 4 * (q - 9 * row)];
      *reinterpret_cast<uint4 *>(dst) = wv[m];
    }
  };

  // A operand: row n is token n / 2 (rows past 2T repeat token T - 1 and
  // are never read back), hi part in even rows, lo part in odd rows.
  const int ta = min(n >> 1, T - 1);
  const uint32_t *xa_src = xhl[wave][2 * ta + (n & 1)];
  // this lane's tokens (D rows 4g, 4g+1 and 4g+2, 4g+3)
  const int t0 = min(2 * g, T - 1), t1 = min(2 * g + 1, T - 1);
  float y0 = 0.f, y1 = 0.f;

  // Code reads: one 8-byte read per sub-block pair, each from its own base
  // register (8-byte units).  Sharing one base, the compiler pairs them
  // into ds_read2_b64 (offsets 32 bytes apart), which measured 8
  // bank-conflict cycles per pair; single reads of the same bytes none.
  int qoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qoff[j] = (n * MB_WROW + 4 + 8 * j + 2 * g) >> 1;
    asm volatile("" : "+v"(qoff[j]));
  }
  const uint2 *const wt2 = reinterpret_cast<const uint2 *>(wtw);

  auto compute_chunk = [&]() {
    const uint32_t *rowp = &wtw[n * MB_WROW];
    // header of row n: d, dmin and all eight 6-bit scales and mins
    const uint2 h01 = *reinterpret_cast<const uint2 *>(rowp);
    const uint2 h23 = *reinterpret_cast<const uint2 *>(rowp + 2);
    const uint32_t sc03 = h01.y & 0x3F3F3F3Fu;
    const uint32_t mn03 = h23.x & 0x3F3F3F3Fu;
    const uint32_t sc47 = (h23.y & 0x0F0F0F0Fu) | ((h01.y >> 2) & 0x30303030u);
    const uint32_t mn47 = ((h23.y >> 4) & 0x0F0F0F0Fu) | ((h23.x >> 2) & 0x30303030u);
    const float d = half_lo(h01.x), dmin = half_hi(h01.x);
    // Eight independent MFMAs (two per sub-block pair j), then the combine.
    floatx4 dlo[4], dhi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 qbj = wt2[qoff[j]];
      const half8_t alo = *reinterpret_cast<const half8_t *>(&xa_src[(64 * j + 8 * g) / 2]);
      const half8_t ahi = *reinterpret_cast<const half8_t *>(&xa_src[(64 * j + 32 + 8 * g) / 2]);
      const uint32_t s0 = qbj.x >> 8, s1 = qbj.y >> 8;
      uint4 blo, bhi;
      blo.x = code_operand_pair<NC>(qbj.x, 0x000F000Fu); blo.y = code_operand_pair<NC>(s0, 0x000F000Fu);
      blo.z = code_operand_pair<NC>(qbj.y, 0x000F000Fu); blo.w = code_operand_pair<NC>(s1, 0x000F000Fu);
      bhi.x = code_operand_pair<NC>(qbj.x, 0x00F000F0u); bhi.y = code_operand_pair<NC>(s0, 0x00F000F0u);
      bhi.z = code_operand_pair<NC>(qbj.y, 0x00F000F0u); bhi.w = code_operand_pair<NC>(s1, 0x00F000F0u);
      dlo[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          alo, __builtin_bit_cast(half8_t, blo), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      dhi[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          ahi, __builtin_bit_cast(half8_t, bhi), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    // Scaled code dots of this super-block: sub-block 2j (low nibbles, q *
    // 2^-c) weighs sc, sub-block 2j+1 (high nibbles, 16q * 2^-c) sc / 16.
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t scw = j < 2 ? sc03 : sc47;
      const float sl = (float)((scw >> (16 * (j & 1))) & 0xFFu);
      const float sh = (float)((scw >> (16 * (j & 1) + 8)) & 0xFFu) * 0.0625f;
      c0 = __builtin_fmaf(sl, dlo[j][0] + dlo[j][1], __builtin_fmaf(sh, dhi[j][0] + dhi[j][1], c0));
      c1 = __builtin_fmaf(sl, dlo[j][2] + dlo[j][3], __builtin_fmaf(sh, dhi[j][2] + dhi[j][3], c1));
    }
    // lazy-dmin term: dmin * sum_s m_s * (sum of x over sub-block s)
    const float4 sa0 = *reinterpret_cast<const float4 *>(&xs[wave][t0][0]);
    const float4 sa1 = *reinterpret_cast<const float4 *>(&xs[wave][t0][4]);
    const float4 sb0 = *reinterpret_cast<const float4 *>(&xs[wave][t1][0]);
    const float4 sb1 = *reinterpret_cast<const float4 *>(&xs[wave][t1][4]);
    const float m0 = (float)(mn03 & 0xFFu), m1 = (float)((mn03 >> 8) & 0xFFu);
    const float m2 = (float)((mn03 >> 16) & 0xFFu), m3 = (float)(mn03 >> 24);
    const float m4 = (float)(mn47 & 0xFFu), m5 = (float)((mn47 >> 8) & 0xFFu);
    const float m6 = (float)((mn47 >> 16) & 0xFFu), m7 = (float)(mn47 >> 24);
    const float z0 = m0 * sa0.x + m1 * sa0.y + m2 * sa0.z + m3 * sa0.w +
                     m4 * sa1.x + m5 * sa1.y + m6 * sa1.z + m7 * sa1.w;
    const float z1 = m0 * sb0.x + m1 * sb0.y + m2 * sb0.z + m3 * sb0.w +
                     m4 * sb1.x + m5 * sb1.y + m6 * sb1.z + m7 * sb1.w;
    // the activations entered as x * 2^-e, the codes as q * 2^-c
    y0 += __builtin_ldexpf(d * c0, xe[wave][t0] + kCodeShift<NC>) - dmin * z0;
    y1 += __builtin_ldexpf(d * c1, xe[wave][t1] + kCodeShift<NC>) - dmin * z1;
  };

  // With 16 waves the next chunk's activations go to the same registers,
  // loaded once the current ones are staged (they come from L2): a second
  // buffer would not fit the 128 registers of a 16-wave lane (from 3
  // tokens on).
  constexpr bool XSINGLE = MB_WAVES == 16 && T > 2;
  if (n_chunks > 0) {  // wave-uniform
    load_x(0, xa);
    load_w(0, wa);
    for (int c = 0;;) {
      const bool more = c + 1 < n_chunks;
      if (more) {
        if constexpr (!XSINGLE) load_x(c + 1, xb);
        load_w(c + 1, wb);
      }
      stage_chunk(wa, xa);
      if constexpr (XSINGLE) {
        if (more) load_x(c + 1, xa);
      }
      compute_chunk();
      if (!more) break;
      ++c;
      const bool more2 = c + 1 < n_chunks;
      if (more2) {
        if constexpr (!XSINGLE) load_x(c + 1, xa);
        load_w(c + 1, wa);
      }
      if constexpr (XSINGLE) {
        stage_chunk(wb, xa);
        if (more2) load_x(c + 1, xa);
      } else {
        stage_chunk(wb, xb);
      }
      compute_chunk();
      if (!more2) break;
      ++c;
    }
  }

  // Lane (n, g) holds tokens 2g and 2g+1 of row n (lane groups past the
  // launch's tokens hold repeats and write nothing); sum the waves.
  if (2 * g < T) part[wave][2 * g][n] = y0;
  if (2 * g + 1 < T) part[wave][2 * g + 1][n] = y1;
  __syncthreads();
  if (tid < T * MB_ROWS) {
    const int t = tid >> 4, r = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < MB_WAVES; ++k) v += part[k][t][r];
    if (t < M && row0 + r < N) Y[(int64_t)t * N + row0 + r] = v;
  }
}

}  // namespace

hipError_t gemv_batch_launch(const float *X, const uint8_t *w, float *Y, int64_t M, int64_t nb,
                             int64_t N, hipStream_t stream) {
  // Offsets formed in the kernel: 16 rows of weights and 8 token rows of X
  // stay below 2^31 bytes.
  if (M < 1 || M > 8 || N > 0x7FFFFFFF ||
      (int64_t)MB_ROWS * nb * kBlockBytes >= ((int64_t)1 << 31) ||
      (int64_t)8 * nb * 1024 + 1024 * nb >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + MB_ROWS - 1) / MB_ROWS));
  const bool nc = nb > kNormalCodesAbove;
  const bool wide = grid.x <= 256 && nb >= 16;
#define Q4K_BATCH_LAUNCH(T_, W_)                                                              \
  if (nc)                                                                                     \
    hipLaunchKernelGGL((q4k_gemv_batch_kernel<T_, true, W_>), grid, dim3(64 * W_), 0, stream, \
                       X, w, Y, (int)M, (int)nb, (int)N);                                     \
  else                                                                                        \
    hipLaunchKernelGGL((q4k_gemv_batch_kernel<T_, false, W_>), grid, dim3(64 * W_), 0, stream, \
                       X, w, Y, (int)M, (int)nb, (int)N);
  if (M <= 2) {
    if (wide) {
      Q4K_BATCH_LAUNCH(2, 16)
    } else {
      Q4K_BATCH_LAUNCH(2, 8)
    }
  } else if (M <= 4) {
    if (wide) {
      Q4K_BATCH_LAUNCH(4, 16)
    } else {
      Q4K_BATCH_LAUNCH(4, 8)
    }
  } else {
    Q4K_BATCH_LAUNCH(8, 8)
  }
#undef Q4K_BATCH_LAUNCH
  return hipGetLastError();
}

}  // namespace q4k
