// q4k_prefill.hip -- batched (prefill) Q4_K product Y = X W^T on gfx950 MFMA.
//
// What it computes: for every token row r, the same lazy-dmin sum as the
// GEMV (Q4_K page: SKaiNET PR #562, "feat(kernel): SIMD-fused Q4_K matmul
// kernel + Q4KMatmulKernel SPI", sections "Summary" and "Pipeline"),
//     Y[r, o] = sum_b d[o,b] * sum_s sc[o,b,s] * sum_l q * X[r, k]
//             - sum_b dmin[o,b] * sum_s m[o,b,s] * sum_l X[r, k]
// with the weights of a tile read once for all tokens of the tile (the
// tiling page: llama.cpp fork PR #37, "ggml-cpu: cache-aware tiling in
// ggml_compute_forward_mul_mat", section "Summary", fix 1).
//
// Work decomposition (MI355X): a workgroup owns 64 weight rows (4 MFMA row
// tiles) and 16 tokens (one MFMA token tile) over the WHOLE of input_dim, so
// every output has exactly one writer: plain stores, no zero fill, no
// atomics, and the result does not depend on scheduling.  For 256
// workgroups the 64x16 tile keeps the bytes a CU pulls from L2 near their
// minimum (64 rows of weights and 16 rows of activations per unit of
// input_dim).  The token groups of a row tile are gridDim.x workgroup ids
// apart, which puts them on the same XCD (and its L2) whenever the number
// of row tiles is a multiple of 8.
//
// Pipeline: input_dim is walked in stages of 4 super-blocks.  All 256
// threads load a stage with coalesced 16-byte loads (every wave instruction
// reads 1 KB of one activation row, or consecutive 16-byte chunks of the
// weight rows) into registers one stage ahead, then write it to LDS: the
// activations already split into fp16 hi + lo in MFMA operand order, the
// weight blocks raw.  Wave w then computes super-block w of the stage:
// decodes the 64 block headers (one row per lane), dequantizes A operands
// from LDS and runs the MFMAs, while the next stage's loads are in flight.
//
// MFMA layout (16x16x32 f16): lane (r = lane % 16, g = lane / 16) holds for
// the A operand row 16a + r of row tile a, positions 8g .. 8g+7 of one
// sub-block (the qs bytes 32j + 8g .. +7 give sub-block 2j in their low
// nibbles and 2j+1 in their high nibbles); for the B operand token r at the
// same positions.  The D tile has rows 16a + 4g + e and token r in lane
// (r, g), element e.
//
// Precision: A = sc*q (<= 945) is exact in fp16.  The activations are split
// into fp16 hi + lo (hi = fp16(x), lo = fp16(x - hi)), two MFMAs per tile,
// so every product is exact and the MFMA's fp32 accumulation gives
// fp32-level results (|x| must stay below 65504).  The per-block tile is
// scaled by d once.  The sums of x over each sub-block come from an MFMA
// with an all-ones A operand, and the lazy-dmin term sum_s (dmin*m_s) *
// (sum of x over sub-block s) runs on the fp32 MFMA (16x16x4) with exact
// fp32 operands.
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int PF_ROWS = 64;           // weight rows per workgroup (4 row tiles)
constexpr int PF_TOK = 16;            // tokens per workgroup (one token tile)
constexpr int PF_BLKS = 4;            // super-blocks per stage
constexpr int PF_WAVES = 8;           // two waves per block: row tiles {0,1} and {2,3}
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_RPAD = PF_ROWS + 4;  // padded row dimension of the header tables
// LDS row pitches in dwords: an activation row (256 fp16 positions) + 16 B,
// a staged weight block (144 B) + 8 B, and one super-block of all 64 rows
// + 32 B; the pads spread consecutive rows over the banks.
constexpr int XROW = 128 + 4;
constexpr int WROW = 36 + 2;
constexpr int WBLK = PF_ROWS * WROW + 8;
// Loads of a stage: waves 0-3 (256 threads) bring the weights, 16-byte
// chunk q = t + 256 m of the 64 rows' 576-byte stage pieces; all 8 waves
// bring the activations, float4 i of thread tid = token 2i + (tid >= 256),
// positions 4t .. 4t+3 of the stage (t = tid % 256).
constexpr int W_CHUNKS = PF_ROWS * PF_BLKS * 9;           // 2304
constexpr int W_PER_THREAD = W_CHUNKS / 256;              // 9
constexpr int X_PER_THREAD = PF_TOK / 2;                  // 8
static_assert(W_CHUNKS % 256 == 0, "weight chunks must divide evenly");

__global__ __launch_bounds__(PF_THREADS) void q4k_prefill_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, int M, int nb,
    int N) {
  // xh/xl: fp16 hi and lo activations [block of stage][token][position
  // pairs in operand order]; wt: raw weight blocks [block of stage][row];
  // header tables of the stage's blocks: fp16 scale pairs (mul, add) per
  // sub-block and row, dmin*m, d.
  __shared__ __align__(16) uint32_t xh[PF_BLKS][PF_TOK][XROW];
  __shared__ __align__(16) uint32_t xl[PF_BLKS][PF_TOK][XROW];
  __shared__ __align__(16) uint32_t wt[PF_BLKS * WBLK];
  __shared__ uint2 sc_tab[PF_BLKS][8][PF_RPAD];
  __shared__ float c_tab[PF_BLKS][8][PF_RPAD];
  __shared__ __align__(16) float d_tab[PF_BLKS][PF_ROWS];

  // The host validates nb >= 1; saying so lets the compiler fetch every
  // kernel argument in one round trip.
  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool w_loader = wave < 4;
  const int t = tid & 255;  // thread index within its loader half
  const int bb = wave & 3;  // block of the stage this wave computes
  const int half = wave >> 2;  // row tiles 2*half and 2*half + 1
  const int r = lane & 15;  // A: row within a row tile; B and D: token
  const int g = lane >> 4;  // lane group
  const int row0 = blockIdx.x * PF_ROWS;
  const int tok0 = blockIdx.y * PF_TOK;
  const int K = nb * 256;
  const int row_bytes = nb * kBlockBytes;
  const int n_stages = (nb + PF_BLKS - 1) / PF_BLKS;

  // Range-checked views: rows past N and tokens past M read as zeros.
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // Prefetch registers.  The per-thread part of every load offset is fixed;
  // the stage part is wave-uniform and goes into the loads' scalar offset.
  // Chunks past a row's last block (ragged last stage) are never consumed.
  uint4 wv[W_PER_THREAD];
  float4 xv[X_PER_THREAD];
  int woff[W_PER_THREAD];
#pragma unroll
  for (int m = 0; m < W_PER_THREAD; ++m) {
    const int q = t + 256 * m;
    const int row = q / 36;
    woff[m] = row * row_bytes + 16 * (q - 36 * row);
  }
  const int tok_lo = tid >> 8;  // tokens 2i + tok_lo
  auto load_stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < X_PER_THREAD; ++i)
      xv[i] = load_buf_f4(xr, 16 * t + 4 * K * (2 * i + tok_lo), 4096 * st);
    if (w_loader) {
#pragma unroll
      for (int m = 0; m < W_PER_THREAD; ++m)
        wv[m] = __builtin_bit_cast(uint4, load_buf_f4(wr, woff[m], st * (4 * kBlockBytes)));
    }
  };
  auto stage_to_lds = [&]() {
    // float4 i: token 2i + tok_lo, block (t / 64), positions 4*lane ..
    // 4*lane+3; stored as pairs (0,2) and (1,3): operand order
    const int xb = t >> 6;
#pragma unroll
    for (int i = 0; i < X_PER_THREAD; ++i) {
      const float4 v = xv[i];
      half2_t h02, h13;
      h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
      h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
      const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
      const int tok = 2 * i + tok_lo;
      *reinterpret_cast<uint2 *>(&xh[xb][tok][2 * lane]) = make_uint2(hw02, hw13);
      *reinterpret_cast<uint2 *>(&xl[xb][tok][2 * lane]) =
          make_uint2(lo_pair(hw02, v.x, v.z), lo_pair(hw13, v.y, v.w));
    }
    if (w_loader) {
#pragma unroll
      for (int m = 0; m < W_PER_THREAD; ++m) {
        const int q = t + 256 * m;
        const int row = q / 36;
        const int cc = q - 36 * row;
        const int b = cc / 9;
        uint32_t *dst = &wt[b * WBLK + row * WROW + 4 * (cc - 9 * b)];
        *reinterpret_cast<uint2 *>(dst) = make_uint2(wv[m].x, wv[m].y);
        *reinterpret_cast<uint2 *>(dst + 2) = make_uint2(wv[m].z, wv[m].w);
      }
    }
  };

  floatx4 y_acc[2], m_acc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) y_acc[a] = m_acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  half8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  const uint32_t *wblk = &wt[bb * WBLK];
  const int hrow = 32 * half + (lane & 31);  // header row decoded by this lane

  // The token groups of a row tile start at different stages (and wrap
  // around), so that together they read whole weight rows at any moment
  // (contiguous DRAM pages) rather than the same quarter of every row.
  const int st0 = blockIdx.y % n_stages;
  load_stage(st0);
  for (int it = 0; it < n_stages; ++it) {
    const int st = st0 + it < n_stages ? st0 + it : st0 + it - n_stages;
    stage_to_lds();
    __syncthreads();
    if (it + 1 < n_stages) load_stage(st + 1 < n_stages ? st + 1 : 0);  // in flight during the MFMAs

    if (st * PF_BLKS + bb < nb) {
      // ---- headers of this wave's 32 rows of block bb (lanes 32-63 repeat
      //      lanes 0-31 and write the same values)
      {
        const uint2 h01 = *reinterpret_cast<const uint2 *>(&wblk[hrow * WROW]);
        const uint2 h23 = *reinterpret_cast<const uint2 *>(&wblk[hrow * WROW + 2]);
        const float d = half_lo(h01.x), dmin = half_hi(h01.x);
        // 6-bit scales and mins, four per dword (one per byte)
        const uint32_t sc03 = h01.y & 0x3F3F3F3Fu;
        const uint32_t mn03 = h23.x & 0x3F3F3F3Fu;
        const uint32_t sc47 = (h23.y & 0x0F0F0F0Fu) | ((h01.y >> 2) & 0x30303030u);
        const uint32_t mn47 = ((h23.y >> 4) & 0x0F0F0F0Fu) | ((h23.x >> 2) & 0x30303030u);
        d_tab[bb][hrow] = d;
        const uint32_t scw[2] = {sc03, sc47}, mnw[2] = {mn03, mn47};
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 4 * hw + e;
            const float scf = (float)((scw[hw] >> (8 * e)) & 255u);
            const float mnf = (float)((mnw[hw] >> (8 * e)) & 255u);
            c_tab[bb][s][hrow] = dmin * mnf;
            // even sub-blocks are low nibbles, odd ones high nibbles (16 v)
            const float mulf = (s & 1) ? scf * 0.0625f : scf;
            const float addf = (s & 1) ? scf * -64.0f : scf * -1024.0f;
            half2_t m2, a2;
            m2.x = m2.y = (_Float16)mulf;
            a2.x = a2.y = (_Float16)addf;
            sc_tab[bb][s][hrow] = make_uint2(as_u32h(m2), as_u32h(a2));
          }
        }
      }

      // ---- MFMAs for row tiles 2*half + a.  The two accumulator chains are
      //      interleaved with the sub-block-sum chain.
      floatx4 acc[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
      // xsb[c]: the B operand of the fp32 MFMA, the sum of x over
      // sub-block 4c + g for token r (lane group g picks its sub-block)
      float xsb[2] = {0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 qb[2], tl[2], th[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int row = 16 * (2 * half + a) + r;
          qb[a] = *reinterpret_cast<const uint2 *>(&wblk[row * WROW + 4 + 8 * j + 2 * g]);
          tl[a] = sc_tab[bb][2 * j][row];
          th[a] = sc_tab[bb][2 * j + 1][row];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int s = 2 * j + h;
          const half8_t Bh = *reinterpret_cast<const half8_t *>(&xh[bb][r][16 * s + 4 * g]);
          const half8_t Bl = *reinterpret_cast<const half8_t *>(&xl[bb][r][16 * s + 4 * g]);
          half8_t A[2];
#pragma unroll
          for (int a = 0; a < 2; ++a)
            A[a] = h ? dequant8(qb[a].x, qb[a].y, true, th[a].x, th[a].y)
                     : dequant8(qb[a].x, qb[a].y, false, tl[a].x, tl[a].y);
          floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int a = 0; a < 2; ++a)
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bh, acc[a], 0, 0, 0);
          sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bl, sx, 0, 0, 0);
#pragma unroll
          for (int a = 0; a < 2; ++a)
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bl, acc[a], 0, 0, 0);
          // sum of x over sub-block s for token r (every row of the tile)
          if ((s & 3) == g) xsb[s >> 2] = sx[0];
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int rt = 2 * half + a;
        // d of rows 16 rt + 4g + e (the rows of this lane's D elements)
        const float4 dv = *reinterpret_cast<const float4 *>(&d_tab[bb][16 * rt + 4 * g]);
        y_acc[a][0] = __builtin_fmaf(dv.x, acc[a][0], y_acc[a][0]);
        y_acc[a][1] = __builtin_fmaf(dv.y, acc[a][1], y_acc[a][1]);
        y_acc[a][2] = __builtin_fmaf(dv.z, acc[a][2], y_acc[a][2]);
        y_acc[a][3] = __builtin_fmaf(dv.w, acc[a][3], y_acc[a][3]);
        // lazy-dmin term: A[row][kk] = dmin*m of sub-block 4c + kk, B = sums
#pragma unroll
        for (int c = 0; c < 2; ++c)
          m_acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(c_tab[bb][4 * c + g][16 * rt + r], xsb[c],
                                                          m_acc[a], 0, 0, 0);
      }
    }
    __syncthreads();  // the next stage overwrites the LDS tiles
  }

  // ---- add the four blocks' partial tiles (through the activation tiles,
  //      no longer needed) and store.  Lane (token r, group g) holds rows
  //      16 rt + 4g + e of its token.
  float4 *red = reinterpret_cast<float4 *>(&xh[0][0][0]);  // [block][token][17]
#pragma unroll
  for (int a = 0; a < 2; ++a)
    red[(bb * PF_TOK + r) * 17 + 4 * (2 * half + a) + g] =
        make_float4(y_acc[a][0] - m_acc[a][0], y_acc[a][1] - m_acc[a][1],
                    y_acc[a][2] - m_acc[a][2], y_acc[a][3] - m_acc[a][3]);
  __syncthreads();
  const float *redf = reinterpret_cast<const float *>(red);
  for (int o = tid; o < PF_TOK * PF_ROWS; o += PF_THREADS) {
    const int tok = o / PF_ROWS, rr = o % PF_ROWS;
    float v = 0.f;
#pragma unroll
    for (int b = 0; b < PF_BLKS; ++b) v += redf[(b * PF_TOK + tok) * 68 + rr];
    if (tok0 + tok < M && row0 + rr < N) Y[(int64_t)(tok0 + tok) * N + row0 + rr] = v;
  }
}

}  // namespace

hipError_t prefill_launch(const float *X, const uint8_t *w, int64_t M,
                          int64_t K, int64_t N, float *Y, hipStream_t stream) {
  const int64_t nb = K / 256;
  // Offsets formed in the kernel (a row tile of 64 rows plus one stage past
  // its end, 16 rows of X plus one stage) must stay below 2^31 bytes.
  if ((int64_t)PF_ROWS * nb * kBlockBytes + 4096 >= ((int64_t)1 << 31) ||
      ((int64_t)PF_TOK * K + 2048) * 4 >= ((int64_t)1 << 31) || N > 0x7FFFFFFF ||
      M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + PF_ROWS - 1) / PF_ROWS), (unsigned)((M + PF_TOK - 1) / PF_TOK));
  if (grid.y > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(q4k_prefill_kernel, grid, dim3(PF_THREADS), 0, stream, X, w, Y, (int)M,
                     (int)nb, (int)N);
  return hipGetLastError();
}

}  // namespace q4k
