// q4_0_gemv_mfma.hip -- Q4_0 matrix-vector product with the multiplies on
// the gfx950 matrix cores.
//
// What it computes is q4_0_gemv's product: the Q4_K page's fused GEMV
// (SKaiNET PR #562, "feat(kernel): SIMD-fused Q4_K matmul kernel +
// Q4KMatmulKernel SPI", sections "Summary" and "Pipeline") on the simpler
// block its section "Out of scope" names, ggml's block_q4_0: 32 weights in
// 18 bytes, d (fp16) then 16 bytes whose byte i holds element i in its low
// nibble and element 16 + i in its high nibble; weight = d * (q - 8).  So
//     y[o] = sum over blocks of d * sum_l q * x - 8 d * sum_l x.
//
// Eight blocks take 144 bytes, the size of a Q4_K super-block, and a block's
// 32 weights are 32 consecutive positions, like a Q4_K sub-block.  The work
// decomposition is that of the Q4_K matrix-core form: a workgroup owns 16
// rows; its 16 waves split the row's groups of eight blocks (contiguous
// ranges); a wave walks its range one group at a time, loading it (16 rows
// x 144 bytes, 256 activations) with coalesced 16-byte loads one ahead,
// stages it in a wave-private LDS area (activations already split into
// exact fp16 hi + lo halves in operand order, each block's 32 activations
// first scaled by the power of two that brings its largest |x| into
// [2^14, 2^15), with the block sums of x), then runs 8 MFMAs per group.
//
// Operands (16x16x32 f16 MFMA, lane (n, g) = (lane % 16, lane / 16)): the B
// operand's column n is weight row n.  MFMA j (0..3) takes from lane group g
// code bytes 8 (g % 2) .. 8 (g % 2) + 7 of block 2j + g / 2: low nibbles in
// the first MFMA of the pair (elements 8 (g % 2) + e), high nibbles kept in
// place in the second (elements 16 + 8 (g % 2) + e, entering as 16 q).  The
// codes enter as fp16 subnormals q * 2^-24.  A row i = 4j' + 2p + h carries
// the hi (h = 0) or lo (h = 1) activations of block 2j' + p at those
// positions in MFMA j = j' and the lane groups g / 2 = p, zeros elsewhere;
// so lane (n, g) finds in its D rows 4g .. 4g+3 blocks 2g and 2g + 1 of row
// n alone and applies their scales in fp32.  The four lane groups and the
// 16 waves are summed at the end in a fixed order (one writer per output).
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int Q0_GROUP_BYTES = 144;   // eight blocks of 18 bytes
constexpr int Q0_ROWS = 16;           // rows per workgroup (one MFMA column tile)
constexpr int Q0_WAVES = 16;
constexpr int Q0_WCH = Q0_ROWS * 9;   // 16-byte weight chunks of a group of 16 rows
constexpr int Q0_WPL = (Q0_WCH + 63) / 64;
constexpr int Q0_WROW = 36;           // LDS dwords per staged row (144 bytes)
constexpr int Q0_XLO = 128 + 16;      // lo part of a wave's activations
constexpr int Q0_XZ = 2 * Q0_XLO;     // zeros that A rows read where they feed nothing
constexpr int Q0_XW = Q0_XZ + 64;     // dwords per wave

// 16-byte loads without the non-temporal hint: a row's 144-byte piece shares
// its 128-byte lines with the neighbouring groups, which other waves load
// at about the same time (as in the Q4_K matrix-core form).
__device__ __forceinline__ uint4 load_w16(__amdgpu_buffer_rsrc_t r, int off, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(64 * Q0_WAVES) void q4_0_gemv_mfma_kernel(
    const float *x, const uint8_t *w, float *__restrict__ y, int ng, int N) {
  // Per wave: the staged weight rows of its group; the fp16 hi part of the
  // group's activations at 0, the lo part at Q0_XLO (positions in operand
  // order: pairs (0,2), (1,3), (4,6), (5,7) of every 8), then zeros; per
  // block pair p: the two blocks' x sums, then their scaling exponents.
  __shared__ __align__(16) uint32_t wt[Q0_WAVES][Q0_ROWS * Q0_WROW];
  __shared__ __align__(16) uint32_t xhl[Q0_WAVES][Q0_XW];
  __shared__ __align__(16) float xse[Q0_WAVES][16];
  __shared__ float part[Q0_WAVES][Q0_ROWS];

  __builtin_assume(ng >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * Q0_ROWS;
  const int row_bytes = ng * Q0_GROUP_BYTES;
  // this wave's groups [b_lo, b_hi) (ng * 16 < 2^31)
  const int b_lo = (int)((unsigned)(ng * wave) / Q0_WAVES);
  const int b_hi = (int)((unsigned)(ng * (wave + 1)) / Q0_WAVES);
  const int n_chunks = b_hi - b_lo;

  // The workgroup's own 16 rows and x stay below 2^31 bytes (input_dim <=
  // 2^24, checked by the host); rows past N read as zeros.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc32(
      w + (int64_t)row0 * row_bytes, (uint32_t)min(N - row0, Q0_ROWS) * (uint32_t)row_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc32(x, (uint32_t)ng * 1024u);

  // weight chunk q (clamped; the duplicates are never stored) is chunk q % 9
  // of row q / 9; activation float4 of this lane: positions 4 lane .. +3
  int woff[Q0_WPL];
#pragma unroll
  for (int m = 0; m < Q0_WPL; ++m) {
    const int q = min(lane + 64 * m, Q0_WCH - 1);
    const int row = q / 9;
    woff[m] = row * row_bytes + 16 * (q - row * 9);
  }
  uint4 wa[Q0_WPL], wb[Q0_WPL];
  float4 xa, xb;
  auto load_chunk = [&](int c, uint4 (&wv)[Q0_WPL], float4 &xv) {
    const int b0 = __builtin_amdgcn_readfirstlane(b_lo + c);  // wave-uniform
    xv = load_buf_f4(xr, 16 * lane, 1024 * b0);
#pragma unroll
    for (int m = 0; m < Q0_WPL; ++m) wv[m] = load_w16(wr, woff[m], Q0_GROUP_BYTES * b0);
  };
  if (n_chunks > 0) load_chunk(0, wa, xa);
  __builtin_amdgcn_sched_barrier(0);

  uint32_t *wtw = wt[wave];
  auto stage_chunk = [&](const uint4 (&wv)[Q0_WPL], const float4 v0) {
    // block lane / 8 (8 aligned lanes): |x| * 2^-e < 2^15
    float mx = fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w)));
    mx = group_max_nonneg<8>(mx);
    const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    const float4 v = make_float4(__builtin_ldexpf(v0.x, -e), __builtin_ldexpf(v0.y, -e),
                                 __builtin_ldexpf(v0.z, -e), __builtin_ldexpf(v0.w, -e));
    half2_t h02, h13;
    h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
    h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
    const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
    *reinterpret_cast<uint2 *>(&xhl[wave][2 * lane]) = make_uint2(hw02, hw13);
    *reinterpret_cast<uint2 *>(&xhl[wave][Q0_XLO + 2 * lane]) =
        make_uint2(lo_pair(hw02, v.x, v.z), lo_pair(hw13, v.y, v.w));
    const float s = group_sum<8>(sum4(v0));
    if ((lane & 7) == 0) {
      const int blk = lane >> 3;
      xse[wave][4 * (blk >> 1) + (blk & 1)] = s;
      xse[wave][4 * (blk >> 1) + 2 + (blk & 1)] = __builtin_bit_cast(float, e);
    }
#pragma unroll
    for (int m = 0; m < Q0_WPL; ++m) {
      const int q = lane + 64 * m;
      if (Q0_WCH % 64 != 0 && q >= Q0_WCH) break;  // only the last load is partial
      const int row = q / 9;
      *reinterpret_cast<uint4 *>(&wtw[row * Q0_WROW + 4 * (q - row * 9)]) = wv[m];
    }
  };

  // A operand indices (16-byte units of the wave's area): this lane feeds
  // MFMA j when its row n is block 2j + g/2's hi or lo row; the high-nibble
  // positions sit 16 positions (2 units) further.  Zeros otherwise.
  const int p_mine = (n >> 1) & 1;
  int aidx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    aidx[j] = ((n >> 2) == j && p_mine == (g >> 1))
                  ? ((n & 1) * Q0_XLO + 32 * j + 16 * (g >> 1) + 4 * (g & 1)) >> 2
                  : (Q0_XZ + 32 * (j & 1)) >> 2;
  const uint4 *const xa4 = reinterpret_cast<const uint4 *>(xhl[wave]);
  // Code bytes of MFMA j: row bytes 36j + 18 (g/2) + 2 + 8 (g%2) .. +7,
  // 2-byte aligned for g < 2: read from three dwords (two when aligned,
  // which keeps every read inside the row) and funnel-shifted.
  const int c_dw = (18 * (g >> 1) + 2 + 8 * (g & 1)) >> 2;  // + 9j
  const uint32_t c_sh = g < 2 ? 2u : 0u;                  // byte shift
  const int c_dw3 = g < 2 ? 2 : 1;                         // third dword, or the second again
  float yacc = 0.f;

  auto compute_chunk = [&](int c) {
    (void)c;
    const uint32_t *rowp = &wtw[n * Q0_WROW];
    // d of blocks 2g (bytes 36g, 36g+1) and 2g + 1 (bytes 36g+18, 36g+19)
    const float d0 = half_lo(rowp[9 * g]);
    const float d1 = half_hi(rowp[9 * g + 4]);
    const float4 xsp = *reinterpret_cast<const float4 *>(&xse[wave][4 * g]);
    // codes enter as q * 2^-24 (low nibbles) and 16 q * 2^-24 (high), the
    // activations as x * 2^-e
    const float s0 = __builtin_ldexpf(d0, __builtin_bit_cast(int, xsp.z) + 24);
    const float s1 = __builtin_ldexpf(d1, __builtin_bit_cast(int, xsp.w) + 24);
    yacc = __builtin_fmaf(-8.f * d0, xsp.x, __builtin_fmaf(-8.f * d1, xsp.y, yacc));
    uint2 qb[4];
    half8_t alo[4], ahi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w0 = rowp[c_dw + 9 * j], w1 = rowp[c_dw + 9 * j + 1];
      const uint32_t w2 = rowp[c_dw + 9 * j + c_dw3];
      qb[j] = make_uint2(__builtin_amdgcn_alignbyte(w1, w0, c_sh),
                         __builtin_amdgcn_alignbyte(w2, w1, c_sh));
      alo[j] = __builtin_bit_cast(half8_t, xa4[aidx[j]]);
      ahi[j] = __builtin_bit_cast(half8_t, xa4[aidx[j] + 2]);
    }
    floatx4 dlo = {0.f, 0.f, 0.f, 0.f}, dhi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t t0 = qb[j].x >> 8, t1 = qb[j].y >> 8;
      uint4 blo, bhi;
      blo.x = qb[j].x & 0x000F000Fu; blo.y = t0 & 0x000F000Fu;
      blo.z = qb[j].y & 0x000F000Fu; blo.w = t1 & 0x000F000Fu;
      bhi.x = qb[j].x & 0x00F000F0u; bhi.y = t0 & 0x00F000F0u;
      bhi.z = qb[j].y & 0x00F000F0u; bhi.w = t1 & 0x00F000F0u;
      dlo = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[j], __builtin_bit_cast(half8_t, blo),
                                                    dlo, 0, 0, 0);
      dhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[j], __builtin_bit_cast(half8_t, bhi),
                                                    dhi, 0, 0, 0);
    }
    // D rows 4g, 4g+1: block 2g (hi, lo); 4g+2, 4g+3: block 2g + 1
    const float t_0 = (dlo[0] + dlo[1]) + 0.0625f * (dhi[0] + dhi[1]);
    const float t_1 = (dlo[2] + dlo[3]) + 0.0625f * (dhi[2] + dhi[3]);
    yacc = __builtin_fmaf(s0, t_0, __builtin_fmaf(s1, t_1, yacc));
  };

  xhl[wave][Q0_XZ + lane] = 0u;  // the zero area (read after this wave's own stores)
  if (n_chunks > 0) {  // wave-uniform
    for (int c = 0;;) {
      const bool more = c + 1 < n_chunks;
      if (more) load_chunk(c + 1, wb, xb);
      stage_chunk(wa, xa);
      compute_chunk(c);
      if (!more) break;
      ++c;
      const bool more2 = c + 1 < n_chunks;
      if (more2) load_chunk(c + 1, wa, xa);
      stage_chunk(wb, xb);
      compute_chunk(c);
      if (!more2) break;
      ++c;
    }
  }

  // Sum the four lane groups (lanes n, n+16, n+32, n+48), then the waves.
  yacc = add_partner_row<32>(yacc);
  yacc = add_partner_row<64>(yacc);
  if (lane < Q0_ROWS) part[wave][lane] = yacc;
  __syncthreads();
  if (tid < Q0_ROWS) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < Q0_WAVES; ++k) v += part[k][tid];
    if (row0 + tid < N) y[row0 + tid] = v;
  }
}

}  // namespace

hipError_t gemv_q4_0_mfma_launch(const float *x, const uint8_t *w, float *y, int64_t ngroups,
                                 int64_t N, hipStream_t stream) {
  const int64_t grid = (N + Q0_ROWS - 1) / Q0_ROWS;
  // Offsets formed in the kernel: 16 rows of weights and the activation
  // vector stay below 2^31 bytes; the codes enter as fp16 subnormals, so
  // rows are limited as in the Q4_K matrix-core form.
  if (grid > 0x7FFFFFFF || N > 0x7FFFFFFF || ngroups > kQ40MfmaMaxGroups ||
      (int64_t)Q0_ROWS * ngroups * Q0_GROUP_BYTES >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(q4_0_gemv_mfma_kernel, dim3((unsigned)grid), dim3(64 * Q0_WAVES), 0, stream,
                     x, w, y, (int)ngroups, (int)N);
  return hipGetLastError();
}

}  // namespace q4k
