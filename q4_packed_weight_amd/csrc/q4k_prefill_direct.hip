// q4k_prefill_direct.hip -- batched (prefill) Q4_K product Y = X W^T on the
// gfx950 matrix cores, with each wave owning whole super-blocks of the
// workgroup's rows and its activations loaded straight into MFMA operand
// registers.
//
// What it computes is q4k_matmul's product (Q4_K page: SKaiNET PR #562,
// "feat(kernel): SIMD-fused Q4_K matmul kernel + Q4KMatmulKernel SPI",
// sections "Summary" and "Pipeline", in the lazy-dmin form, for every token
// row as in the ternary page's prefill row loop, SKaiNET issue #1138, section
// "Tasks"):
//     Y[r, o] = sum_b d * sum_s sc_s * sum_l q * X[r, k] - dmin * sum_s m_s * sum_l X[r, k],
// with every weight byte read once per workgroup for its 16 tokens (the
// tiling page: llama.cpp fork PR #37, "ggml-cpu: cache-aware tiling in
// ggml_compute_forward_mul_mat", section "Summary", fix 1).
//
// Work decomposition: a workgroup owns 64 weight rows (4 MFMA row tiles) and
// 16 tokens (one token tile) over the whole of input_dim; its 8 waves split
// the super-blocks (wave w takes w, w + 8, ...), each wave computing all 64
// rows x 16 tokens of its super-blocks.  There is no barrier until the waves'
// partial tiles are added at the end (fixed order, one writer per output).
// Per super-block a wave
//   - stages the 64 rows' 144-byte blocks in a wave-private LDS tile
//     (coalesced 16-byte streaming loads, one super-block ahead);
//   - loads its 16 tokens' 256 activations straight into B-operand layout
//     (lane (r, g): token r, positions 8g .. 8g+7 of each sub-block), one
//     super-block ahead, and splits them in registers: each token's block
//     is scaled by the power of two that brings its largest |x| into
//     [2^14, 2^15) and split into exact fp16 hi + lo halves, the scaling
//     folded into the v_fma_mix that rounds each half (two operations per
//     activation);
//   - decodes each row's header once (lane l, row l) into a small LDS
//     table: the packed fp16 (mul, add) pair that turns a code masked under
//     0x6400 into sc*q, and 32*m of each sub-block;
//   - runs 16x16x32 f16 MFMAs: A = sc*q (exact in fp16), B = hi and lo
//     halves, one accumulator per row tile and super-block; an all-ones A
//     operand gives the sums of x per sub-block, and one more MFMA per row
//     tile (A = 32*m, B = those sums times 2^-5 as hi and lo halves in two
//     lane groups) gives sum_s m_s * (sum of x over s);
//   - adds 2^e * (d * tile - dmin * min tile) to the running result.
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int PD_ROWS = 64;            // weight rows per workgroup (4 row tiles)
constexpr int PD_TOK = 16;             // tokens per workgroup (one token tile)
constexpr int PD_WAVES = 8;
constexpr int PD_THREADS = 64 * PD_WAVES;
// LDS dwords per staged row: the rows' blocks are staged in chunk order
// (row n at 144 n bytes), so chunk q of a super-block lands at 16 q and the
// writes take immediate offsets.  With a 36-dword pitch the 16 rows that a
// row tile's lanes read start in 16 different banks.
constexpr int PD_WROW = 36;
constexpr int PD_WCH = PD_ROWS * 9;    // 16-byte chunks of one super-block of the rows
constexpr int PD_WPL = PD_WCH / 64;    // per lane: 9
constexpr int PD_TREC = 12;            // header record: 8 scale pairs + 4 dwords of 32*m
constexpr int PD_RROW = PD_ROWS + 4;   // reduction row pitch (floats)
static_assert(PD_WCH % 64 == 0, "a super-block of the rows must be whole wave loads");

// 32*m for the two 6-bit mins in bytes 0 and 2 of `v` (bytes 1 and 3 zero),
// as an fp16 pair: v | 0x6400 in each half is 1024 + m, and
// 32 * (1024 + m) - 32768 is exact in fp16.
__device__ __forceinline__ uint32_t mins32(uint32_t v, uint32_t hi64) {
  const half2_t t = as_h2(v | hi64);
  return as_u32h(__builtin_elementwise_fma(t, half2_t{(_Float16)32.0f, (_Float16)32.0f},
                                           half2_t{(_Float16)-32768.0f, (_Float16)-32768.0f}));
}

// REUSE: more than one token group reads each row tile, so the weights are
// ordinary cached loads that the other groups' workgroups (on the same XCD)
// find in L2; a single token group streams them.
template <bool REUSE>
__global__ __launch_bounds__(PD_THREADS) void q4k_prefill_direct_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, int M, int nb, int N) {
  // Per wave: the staged rows of its current super-block, the decoded
  // header records and the (d, dmin) pairs of the 64 rows.
  __shared__ __align__(16) uint32_t wt[PD_WAVES][PD_ROWS * PD_WROW];
  __shared__ __align__(16) uint32_t tab[PD_WAVES][PD_ROWS * PD_TREC];
  __shared__ __align__(16) uint32_t dd[PD_WAVES][PD_ROWS];
  static_assert(PD_WAVES * PD_TOK * PD_RROW <= PD_WAVES * PD_ROWS * PD_WROW,
                "the partial tiles must fit in the weight tiles");

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;  // A: row of a row tile; B and D: token
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7 of a sub-block
  const int row0 = blockIdx.x * PD_ROWS;
  const int tok0 = blockIdx.y * PD_TOK;
  const int K = nb * 256;
  const int row_bytes = nb * kBlockBytes;
  // super-blocks wave, wave + 8, ... (wave-uniform; 0 when nb <= wave)
  const int n_steps = (nb - wave + PD_WAVES - 1) / PD_WAVES;

  // Range-checked views: rows past N and tokens past M read as zeros.
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // Weight chunk q = lane + 64 m of a super-block (row q / 9, piece q % 9;
  // staged at dword 4 q of the wave's tile).  Since 64 = 7 * 9 + 1, chunk
  // lane + 64 m lies m * (7 row_bytes + 16) bytes past chunk lane (a
  // wave-uniform part, in the loads' scalar offset), plus row_bytes - 144
  // once lane % 9 + m passes 8 (its piece index wrapped into the next row).
  const int lane9 = lane % 9;
  const int wbase = (lane / 9) * row_bytes + 16 * lane9;
  const int wwrap = wbase + row_bytes - kBlockBytes;
  const int wstep = 7 * row_bytes + 16;
  // Activations: float4 (s, h) of a lane is token r, positions 32 s + 8 g +
  // 4 h .. +3 of the super-block.
  const int xoff = r * K * 4 + 32 * g;

  uint4 wv[PD_WPL];
  float4 xv[16];
  auto load_step = [&](int b) {  // b wave-uniform
    // the nine offsets are formed at each step (held across the loop they
    // would not fit the registers)
    int wb = wbase, ww = wwrap;
    asm volatile("" : "+v"(wb), "+v"(ww));
#pragma unroll
    for (int m = 0; m < PD_WPL; ++m) {
      const int vo = lane9 + m > 8 ? ww : wb;
      const int so = kBlockBytes * b + wstep * m;
      if constexpr (REUSE)
        wv[m] = __builtin_bit_cast(uint4, load_buf_f4(wr, vo, so));
      else
        wv[m] = load_buf_stream16(wr, vo, so);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      xv[k] = load_buf_f4(xr, xoff + 128 * (k >> 1) + 16 * (k & 1), 1024 * b);
  };

  uint32_t *wtw = wt[wave];
  uint32_t *tbw = tab[wave];
  uint32_t *ddw = dd[wave];
  const uint32_t hi64 = vgpr_const(0x64006400u);
  half8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  floatx4 yacc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) yacc[a] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (n_steps > 0) {  // wave-uniform
    load_step(wave);
    for (int i = 0; i < n_steps; ++i) {
      // ---- this super-block's weights into the wave's LDS tile
#pragma unroll
      for (int m = 0; m < PD_WPL; ++m)
        *reinterpret_cast<uint4 *>(&wtw[4 * (lane + 64 * m)]) = wv[m];

      // ---- token r's block maximum (lanes r, r+16, r+32, r+48) and scale
      // two chains of v_max3 over the lane's 64 values
      float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        mx0 = absmax3(absmax3(mx0, xv[k].x, xv[k].y), xv[k].z, xv[k].w);
        mx1 = absmax3(absmax3(mx1, xv[k + 1].x, xv[k + 1].y), xv[k + 1].z, xv[k + 1].w);
      }
      const float mx = fmaxf(mx0, mx1);
      uint32_t mb = __builtin_bit_cast(uint32_t, mx);
      {
        const auto h = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
        mb = h[0] > h[1] ? h[0] : h[1];
        const auto q = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);
        mb = q[0] > q[1] ? q[0] : q[1];
      }
      // |x| * 2^-e < 2^15; e >= -126 keeps both powers of two normal floats
      int e = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mb)) - 15;
      e = e < -126 ? -126 : e;
      const float sdown = __builtin_ldexpf(1.0f, -e);
      const float sup = __builtin_ldexpf(1.0f, e);

      // ---- B operands: positions in operand order (0,2), (1,3), (4,6), (5,7)
      half8_t bh[8], bl[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float4 a = xv[2 * s], c = xv[2 * s + 1];
        uint4 h, l;
        split_pair(a.x, a.z, sdown, h.x, l.x);
        split_pair(a.y, a.w, sdown, h.y, l.y);
        split_pair(c.x, c.z, sdown, h.z, l.z);
        split_pair(c.y, c.w, sdown, h.w, l.w);
        bh[s] = __builtin_bit_cast(half8_t, h);
        bl[s] = __builtin_bit_cast(half8_t, l);
      }


      // ---- headers: lane l decodes row l once for the whole wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      {
        const uint4 hd = *reinterpret_cast<const uint4 *>(&wtw[lane * PD_WROW]);
        const uint2 h01 = make_uint2(hd.x, hd.y), h23 = make_uint2(hd.z, hd.w);
        const uint32_t sc03 = h01.y & 0x3F3F3F3Fu;
        const uint32_t mn03 = h23.x & 0x3F3F3F3Fu;
        const uint32_t sc47 = (h23.y & 0x0F0F0F0Fu) | ((h01.y >> 2) & 0x30303030u);
        const uint32_t mn47 = ((h23.y >> 4) & 0x0F0F0F0Fu) | ((h23.x >> 2) & 0x30303030u);
        uint4 r0, r1, r2;
        // even sub-blocks are low nibbles, odd ones high nibbles kept in place
        r0.x = scale_pair(sc03 & 255u, false);
        r0.y = scale_pair((sc03 >> 8) & 255u, true);
        r0.z = scale_pair((sc03 >> 16) & 255u, false);
        r0.w = scale_pair(sc03 >> 24, true);
        r1.x = scale_pair(sc47 & 255u, false);
        r1.y = scale_pair((sc47 >> 8) & 255u, true);
        r1.z = scale_pair((sc47 >> 16) & 255u, false);
        r1.w = scale_pair(sc47 >> 24, true);
        // 32*m in the operand order of the sums: m0, m2 | m1, m3 | m4, m6 | m5, m7
        r2.x = mins32(mn03 & 0x00FF00FFu, hi64);
        r2.y = mins32((mn03 >> 8) & 0x00FF00FFu, hi64);
        r2.z = mins32(mn47 & 0x00FF00FFu, hi64);
        r2.w = mins32((mn47 >> 8) & 0x00FF00FFu, hi64);
        uint4 *rec = reinterpret_cast<uint4 *>(&tbw[lane * PD_TREC]);
        rec[0] = r0;
        rec[1] = r1;
        rec[2] = r2;
        ddw[lane] = h01.x;  // d | dmin << 16
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- MFMAs: the four row tiles' chains interleaved with the sums
      floatx4 acc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
      float sums[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int s = 2 * j + h;
          floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bh[s],
                                                              floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bl[s], sx, 0, 0, 0);
          // two row tiles at a time keep the operand registers few
#pragma unroll
          for (int a0 = 0; a0 < 4; a0 += 2) {
            half8_t A[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int row = 16 * (a0 + a) + r;
              const uint2 qb = *reinterpret_cast<const uint2 *>(&wtw[row * PD_WROW + 4 + 8 * j + 2 * g]);
              const uint32_t sp = tbw[row * PD_TREC + s];
              A[a] = dequant8_ma(qb.x, qb.y, h != 0, sp, hi64);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
              acc[a0 + a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], bh[s], acc[a0 + a], 0, 0, 0);
#pragma unroll
            for (int a = 0; a < 2; ++a)
              acc[a0 + a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], bl[s], acc[a0 + a], 0, 0, 0);
          }
          sums[s] = sx[0];  // sum of token r's scaled x over sub-block s
        }
        // the next super-block's loads leave half way through the MFMAs:
        // the weight registers and the first half of the B operands are
        // free by then, which keeps two waves per SIMD within the register
        // file
        if (j == 1 && i + 1 < n_steps) load_step(wave + PD_WAVES * (i + 1));
      }

      // ---- lazy-dmin term: B rows 8g + k hold the sums times 2^-5 (below
      //      2^15) of sub-blocks 0, 2, 1, 3, 4, 6, 5, 7: their hi halves in
      //      lane group 0, their lo halves in group 1, zeros in groups 2, 3
      const float s5 = opaque_f32(0.03125f);
      uint4 mh, ml;
      split_pair(sums[0], sums[2], s5, mh.x, ml.x);
      split_pair(sums[1], sums[3], s5, mh.y, ml.y);
      split_pair(sums[4], sums[6], s5, mh.z, ml.z);
      split_pair(sums[5], sums[7], s5, mh.w, ml.w);
      const uint4 bmv = g == 0 ? mh : (g == 1 ? ml : make_uint4(0u, 0u, 0u, 0u));
      const half8_t bm = __builtin_bit_cast(half8_t, bmv);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const half8_t am =
            *reinterpret_cast<const half8_t *>(&tbw[(16 * a + r) * PD_TREC + 8]);
        const floatx4 mt =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bm, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        // (d, dmin) of rows 16a + 4g + k, this lane's D rows
        const uint4 dv = *reinterpret_cast<const uint4 *>(&ddw[16 * a + 4 * g]);
        const uint32_t dk[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float t = half_lo(dk[k]) * acc[a][k] - half_hi(dk[k]) * mt[k];
          yacc[a][k] = __builtin_fmaf(t, sup, yacc[a][k]);
        }
      }
    }
  }

  // ---- add the waves' partial tiles in a fixed order and store.  Lane
  //      (token r, group g) holds rows 16a + 4g + k of its token.
  __syncthreads();  // every wave is done with its LDS tiles
  float *red = reinterpret_cast<float *>(&wt[0][0]);  // [wave][token][PD_RROW]
#pragma unroll
  for (int a = 0; a < 4; ++a)
    *reinterpret_cast<float4 *>(&red[(wave * PD_TOK + r) * PD_RROW + 16 * a + 4 * g]) =
        make_float4(yacc[a][0], yacc[a][1], yacc[a][2], yacc[a][3]);
  __syncthreads();
  for (int o = tid; o < PD_TOK * PD_ROWS; o += PD_THREADS) {
    const int tok = o / PD_ROWS, rr = o % PD_ROWS;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < PD_WAVES; ++k) v += red[(k * PD_TOK + tok) * PD_RROW + rr];
    if (tok0 + tok < M && row0 + rr < N) Y[(int64_t)(tok0 + tok) * N + row0 + rr] = v;
  }
}

}  // namespace

hipError_t prefill_direct_launch(const float *X, const uint8_t *w, int64_t M, int64_t K,
                                 int64_t N, float *Y, hipStream_t stream) {
  const int64_t nb = K / 256;
  // Offsets formed in the kernel (64 rows of weights, 16 rows of X) stay
  // below 2^31 bytes.
  if ((int64_t)PD_ROWS * nb * kBlockBytes >= ((int64_t)1 << 31) ||
      (int64_t)PD_TOK * K * 4 >= ((int64_t)1 << 31) || N > 0x7FFFFFFF || M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + PD_ROWS - 1) / PD_ROWS), (unsigned)((M + PD_TOK - 1) / PD_TOK));
  if (grid.y > 65535) return hipErrorInvalidConfiguration;
  if (grid.y > 1)
    hipLaunchKernelGGL(q4k_prefill_direct_kernel<true>, grid, dim3(PD_THREADS), 0, stream, X, w,
                       Y, (int)M, (int)nb, (int)N);
  else
    hipLaunchKernelGGL(q4k_prefill_direct_kernel<false>, grid, dim3(PD_THREADS), 0, stream, X,
                       w, Y, (int)M, (int)nb, (int)N);
  return hipGetLastError();
}

}  // namespace q4k
