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
// input_dim).  With few token tiles 64-row workgroups leave CUs idle (16
// tokens x 4096 rows is 64 workgroups), so the launch can narrow them to 32
// or 16 rows (prefill_rows: the height with the fewest rounds of 256
// workgroups times the measured per-workgroup time).  The token groups of a
// row tile are gridDim.x workgroup ids apart, which puts them on the same
// XCD (and its L2) whenever the number of row tiles is a multiple of 8.
//
// Pipeline: input_dim is walked in stages of 4 super-blocks.  The 512
// threads load a stage with coalesced 16-byte loads (every wave instruction
// reads 1 KB of one activation row, or consecutive 16-byte chunks of the
// weight rows, or of whole tiles in the tiled block order) into registers
// one stage ahead, then write it to LDS: the activations already split into
// fp16 hi + lo in MFMA operand order, the weight blocks raw.  Waves w and
// w + 4 then compute super-block w of the stage (two row tiles each, or at
// 32 and 16 rows half of its sub-blocks each): they decode their rows'
// block headers into LDS tables, each (row, sub-block) once, dequantize A
// operands from LDS and run the MFMAs while the next stage's loads are in
// flight.
//
// MFMA layout (16x16x32 f16): lane (r = lane % 16, g = lane / 16) holds for
// the A operand row 16a + r of row tile a, positions 8g .. 8g+7 of one
// sub-block (the qs bytes 32j + 8g .. +7 give sub-block 2j in their low
// nibbles and 2j+1 in their high nibbles); for the B operand token r at the
// same positions.  The D tile has rows 16a + 4g + e and token r in lane
// (r, g), element e.
//
// Precision: A = sc*q (<= 945) is exact in fp16.  Each token's 256
// activations of a super-block are first scaled by the power of two that
// puts their largest |x| into [2^14, 2^15), then split into fp16 hi + lo
// (hi = fp16(x), lo = fp16(x - hi)), two MFMAs per tile: the halves can
// neither overflow fp16 nor, for any element within 2^-17 of the block's
// largest, lose bits of lo to fp16's subnormal range, so every product is
// exact and the MFMA's fp32 accumulation gives fp32-level results for any
// |x| < 2^96.  The per-block tile is scaled by d once and the power of two
// undone (d * tile, then the exponent).  The sums of x over each sub-block
// come from an MFMA with an all-ones A operand (scaled back the same way),
// and the lazy-dmin term sum_s (dmin*m_s) * (sum of x over sub-block s)
// runs on the fp32 MFMA (16x16x4) with exact fp32 operands.
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int kTileRows = 16;                      // tiled block order: rows per group
constexpr int kTileBytes = 16 * kBlockBytes;       // one tile: a group's super-block
constexpr int kTileChunks = kTileBytes / 16;
constexpr int PF_TOK = 16;            // tokens per workgroup (one token tile)
constexpr int PF_BLKS = 4;            // super-blocks per stage
constexpr int PF_WAVES = 8;           // two waves per block of a stage
constexpr int PF_THREADS = 64 * PF_WAVES;
// LDS row pitches in dwords: an activation row (256 fp16 positions) + 16 B,
// a staged weight block (144 B) + 8 B; the pads spread consecutive rows over
// the banks.
constexpr int XROW = 128 + 4;
constexpr int WROW = 36 + 2;
constexpr int X_PER_THREAD = PF_TOK / 2;                  // 8

// ROWS weight rows (RT = ROWS / 16 MFMA row tiles) per workgroup.  The
// waves of a stage are (block bb, half): with 4 row tiles half h computes
// row tiles 2h, 2h+1 over all eight sub-blocks; with 2 or 1, all row tiles
// over sub-blocks 4h .. 4h+3.  Loads: 16-byte chunk q of the rows' 576-byte
// stage pieces is brought by thread q % W_STRIDE (all 8 waves at 64 rows,
// the first RT waves otherwise); all 8 waves bring the activations, float4 i
// of thread tid = token 2i + (tid >= 256), positions 4t .. 4t+3 of the
// stage (t = tid % 256).
// TILED: w holds the weights in the tiled block order (16-row groups, one
// 2304-byte tile per group and super-block: 16-byte chunk c < 128 carries
// qs bytes 8g .. 8g+7 of pairs 2h and 2h+1 of row n, h = c / 64, n = c % 16,
// g = (c % 64) / 16; chunks 128 + n the header of row n).  The stage's
// chunks are then whole tiles, read contiguously, and staging scatters each
// into the same LDS block layout, so both orders give the same bits.
template <int ROWS, bool TILED>
__global__ __launch_bounds__(PF_THREADS) void q4k_prefill_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, int M, int nb,
    int N) {
  constexpr int RT = ROWS / 16;
  // Up to 2 row tiles the block's two waves split its sub-blocks (each wave:
  // all row tiles, half the sub-blocks), so each activation operand and sub-
  // block sum is produced once per workgroup; measured at 32 rows, 16 and 32
  // tokens, 4096 and 14336 inputs: 6-7% faster than one row tile per wave.
  // At 4 row tiles splitting the sub-blocks measured no faster (and needs
  // more registers), so each wave takes two row tiles over all sub-blocks.
  constexpr bool SPLIT = RT <= 2;
  constexpr int TPW = SPLIT ? RT : (RT == 4 ? 2 : 1);  // row tiles per wave
  constexpr int NJ = SPLIT ? 2 : 4;                    // sub-block pairs per wave
  constexpr int NS = SPLIT ? 2 : 1;                    // waves sharing a block's rows
  constexpr int RPAD = ROWS + 4;          // padded row dimension of the header tables
  constexpr int WBLK = ROWS * WROW + 8;   // one super-block of all rows + 32 B
  // Two choices measured per height (MI355X, graph-replayed calls at input_
  // dim 4096 and 14336): at 64 rows every wave loads weight chunks (chunk
  // q = tid + 512 m; the last round covers the first W_LAST threads, whole
  // waves) and the next stage's loads leave after the barrier, 3-7% faster
  // than 4 loader waves; at 32 and 16 rows the 4 ROWS threads of the first
  // RT waves load 9 chunks each and the next stage's loads leave before the
  // barrier, 3-8% faster.  Each choice slowed the other height.
  constexpr bool SPREAD = ROWS == 64;
  constexpr bool EARLY = !SPREAD;
  constexpr int W_CHUNKS = ROWS * 36;  // 16-byte weight chunks of a stage
  constexpr int W_STRIDE = SPREAD ? PF_THREADS : 4 * ROWS;
  constexpr int W_ITERS = (W_CHUNKS + W_STRIDE - 1) / W_STRIDE;
  constexpr int W_LAST = W_CHUNKS - W_STRIDE * (W_ITERS - 1);
  static_assert(W_CHUNKS % 64 == 0 && W_LAST % 64 == 0, "weight rounds must cover whole waves");
  // xh/xl: fp16 hi and lo activations [block of stage][token][position
  // pairs in operand order]; wt: raw weight blocks [block of stage][row];
  // header tables of the stage's blocks: the fp16 scale pair (mul, add) of
  // each sub-block and row packed in a dword, dmin*m, d.
  __shared__ __align__(16) uint32_t xh[PF_BLKS][PF_TOK][XROW];
  __shared__ __align__(16) uint32_t xl[PF_BLKS][PF_TOK][XROW];
  __shared__ __align__(16) uint32_t wt[PF_BLKS * WBLK];
  __shared__ uint2 sc_tab[PF_BLKS][4][RPAD];  // (even, odd) sub-block of a pair
  __shared__ float c_tab[PF_BLKS][8][RPAD];
  __shared__ __align__(16) float d_tab[PF_BLKS][ROWS];
  __shared__ int xe[PF_BLKS][PF_TOK];  // scaling exponent per (block, token) of the stage

  // The host validates nb >= 1; saying so lets the compiler fetch every
  // kernel argument in one round trip.
  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // wave-uniform: takes part in the weight loads of round m
  auto w_round = [&](int m) { return wave < (m + 1 < W_ITERS ? W_STRIDE : W_LAST) / 64; };
  const int t = tid & 255;  // thread index within its activation-loader half
  const int bb = wave & 3;  // block of the stage this wave computes
  const int half = wave >> 2;
  const int rt0 = SPLIT ? 0 : (RT == 4 ? 2 * half : half);  // first row tile of this wave
  const int j0 = SPLIT ? 2 * half : 0;                      // first sub-block pair
  const int r = lane & 15;  // A: row within a row tile; B and D: token
  const int g = lane >> 4;  // lane group
  const int row0 = blockIdx.x * ROWS;
  const int tok0 = blockIdx.y * PF_TOK;
  const int K = nb * 256;
  const int row_bytes = nb * kBlockBytes;
  const int n_stages = (nb + PF_BLKS - 1) / PF_BLKS;

  // Range-checked views: rows past N and tokens past M read as zeros (the
  // tiled order pads its last row group with zero rows).
  const int ng_left = (N - row0 + kTileRows - 1) / kTileRows;  // row groups from row0 on
  const __amdgpu_buffer_rsrc_t wr =
      TILED ? make_rsrc(w + (int64_t)(row0 / kTileRows) * nb * kTileBytes,
                        (int64_t)min(RT, ng_left) * nb * kTileBytes)
            : make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // Prefetch registers.  The per-thread part of every load offset is fixed;
  // the stage part is wave-uniform and goes into the loads' scalar offset.
  // Chunks past a row's last block (ragged last stage) are never consumed.
  uint4 wv[W_ITERS];
  float4 xv[X_PER_THREAD];
  int woff[W_ITERS];
#pragma unroll
  for (int m = 0; m < W_ITERS; ++m) {
    const int q = tid + W_STRIDE * m;
    if constexpr (TILED) {
      // chunk q: tile q / 144 = (row group a, block bb of the stage)
      const int tile = q / kTileChunks;
      woff[m] = ((tile >> 2) * nb + (tile & 3)) * kTileBytes + 16 * (q - kTileChunks * tile);
    } else {
      const int row = q / 36;
      woff[m] = row * row_bytes + 16 * (q - 36 * row);
    }
  }
  constexpr int W_STAGE_BYTES = PF_BLKS * (TILED ? kTileBytes : kBlockBytes);
  const int tok_lo = tid >> 8;  // tokens 2i + tok_lo
  // activations: wave w stages block w % 4 of the stage for the tokens of
  // parity w / 4, lane (token 2 (lane / 8) + w / 4, column j = lane % 8)
  // taking positions 32c + 4j .. +3 of the block (c = 0..7): a token's 8
  // lanes read whole 128-byte lines and hold its whole block
  const int xb = t >> 6;
  const int xj = lane & 7;
  const int xtok = 2 * (lane >> 3) + tok_lo;
  const int xoff = 4 * K * xtok + 1024 * xb + 16 * xj;
  auto load_stage = [&](int st) {
#pragma unroll
    for (int c = 0; c < X_PER_THREAD; ++c)
      xv[c] = load_buf_f4(xr, xoff + 128 * c, 4096 * st);
#pragma unroll
    for (int m = 0; m < W_ITERS; ++m)
      if (w_round(m))
        wv[m] = __builtin_bit_cast(uint4, load_buf_f4(wr, woff[m], st * W_STAGE_BYTES));
  };
  auto stage_to_lds = [&]() {
    // the token's block maximum: a chain over the lane's 32 values, then a
    // maximum over its 8 lanes; halves stored as pairs (0,2) and (1,3):
    // operand order
    float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
    for (int c = 0; c < X_PER_THREAD; c += 2) {
      mx0 = absmax3(absmax3(mx0, xv[c].x, xv[c].y), xv[c].z, xv[c].w);
      mx1 = absmax3(absmax3(mx1, xv[c + 1].x, xv[c + 1].y), xv[c + 1].z, xv[c + 1].w);
    }
    const float mx = group_max_nonneg<8>(fmaxf(mx0, mx1));
    // |x| * 2^-e < 2^15; e >= -126 keeps both powers of two normal floats
    int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    e = e < -126 ? -126 : e;
    const float sdown = __builtin_ldexpf(1.0f, -e);
    if (xj == 0) xe[xb][xtok] = e;
#pragma unroll
    for (int c = 0; c < X_PER_THREAD; ++c) {
      uint2 h, l;
      split_pair(xv[c].x, xv[c].z, sdown, h.x, l.x);
      split_pair(xv[c].y, xv[c].w, sdown, h.y, l.y);
      *reinterpret_cast<uint2 *>(&xh[xb][xtok][2 * (xj + 8 * c)]) = h;
      *reinterpret_cast<uint2 *>(&xl[xb][xtok][2 * (xj + 8 * c)]) = l;
    }
#pragma unroll
    for (int m = 0; m < W_ITERS; ++m) {
      if (w_round(m)) {
        const int q = tid + W_STRIDE * m;
        uint32_t *d0, *d1;  // LDS homes of the chunk's two 8-byte halves
        if constexpr (TILED) {
          const int tile = q / kTileChunks;
          const int c = q - kTileChunks * tile;
          uint32_t *blk = &wt[(tile & 3) * WBLK + 16 * (tile >> 2) * WROW];
          if (c < 128) {  // pair 2h at dword 4 + 16h + 2g of row n, pair 2h+1 8 dwords on
            d0 = blk + (c & 15) * WROW + 4 + 16 * (c >> 6) + 2 * ((c >> 4) & 3);
            d1 = d0 + 8;
          } else {  // header of row c - 128
            d0 = blk + (c - 128) * WROW;
            d1 = d0 + 2;
          }
        } else {
          const int row = q / 36;
          const int cc = q - 36 * row;
          const int b = cc / 9;
          d0 = &wt[b * WBLK + row * WROW + 4 * (cc - 9 * b)];
          d1 = d0 + 2;
        }
        *reinterpret_cast<uint2 *>(d0) = make_uint2(wv[m].x, wv[m].y);
        *reinterpret_cast<uint2 *>(d1) = make_uint2(wv[m].z, wv[m].w);
      }
    }
  };

  floatx4 y_acc[TPW], m_acc[TPW];
#pragma unroll
  for (int a = 0; a < TPW; ++a) y_acc[a] = m_acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  half8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  const uint32_t *wblk = &wt[bb * WBLK];
  const uint32_t hi64 = vgpr_const(0x64006400u);
  // Header decoding: the wave's HROWS rows x NSUB sub-blocks, SPL sub-
  // blocks per lane (4, 2 or 1), each (row, sub-block) once.
  constexpr int HROWS = 16 * TPW;
  constexpr int NSUB = SPLIT ? 4 : 8;
  constexpr int SPL = HROWS * NSUB / 64;
  static_assert(SPL >= 1 && HROWS * NSUB == 64 * SPL, "header work must split evenly");
  const int hrow = 16 * rt0 + lane % HROWS;
  const int s_first = (SPLIT ? 4 * half : 0) + SPL * (lane / HROWS);  // lane's first sub-block

  // The token groups of a row tile start at different stages (and wrap
  // around), so that together they read whole weight rows at any moment
  // (contiguous DRAM pages) rather than the same quarter of every row.
  const int st0 = blockIdx.y % n_stages;
  load_stage(st0);
  for (int it = 0; it < n_stages; ++it) {
    const int st = st0 + it < n_stages ? st0 + it : st0 + it - n_stages;
    stage_to_lds();
    // the registers are free again; the next stage's loads stay in flight
    // during the MFMAs
    if (EARLY && it + 1 < n_stages) load_stage(st + 1 < n_stages ? st + 1 : 0);
    __syncthreads();
    if (!EARLY && it + 1 < n_stages) load_stage(st + 1 < n_stages ? st + 1 : 0);

    if (st * PF_BLKS + bb < nb) {
      // ---- headers of this wave's rows of block bb
      {
        const uint2 h01 = *reinterpret_cast<const uint2 *>(&wblk[hrow * WROW]);
        const uint2 h23 = *reinterpret_cast<const uint2 *>(&wblk[hrow * WROW + 2]);
        const float d = half_lo(h01.x), dmin = half_hi(h01.x);
        // 6-bit scales and mins of sub-blocks 4hw .. 4hw+3, one per byte
        const bool hw = s_first >= 4;
        const uint32_t scw = hw ? (h23.y & 0x0F0F0F0Fu) | ((h01.y >> 2) & 0x30303030u)
                                : h01.y & 0x3F3F3F3Fu;
        const uint32_t mnw = hw ? ((h23.y >> 4) & 0x0F0F0F0Fu) | ((h23.x >> 2) & 0x30303030u)
                                : h23.x & 0x3F3F3F3Fu;
        const int sh = 8 * (s_first & 3);
        if (s_first == (SPLIT ? 4 * half : 0)) d_tab[bb][hrow] = d;
        uint32_t pk[SPL];
#pragma unroll
        for (int e = 0; e < SPL; ++e) {
          const int s = s_first + e;
          const float mnf = (float)((mnw >> (sh + 8 * e)) & 255u);
          c_tab[bb][s][hrow] = dmin * mnf;
          // even sub-blocks are low nibbles, odd ones high nibbles (16 v)
          pk[e] = scale_pair((scw >> (sh + 8 * e)) & 255u, SPL > 1 ? (e & 1) : (s & 1));
        }
        uint32_t *tab = reinterpret_cast<uint32_t *>(&sc_tab[bb][s_first >> 1][hrow]);
        if constexpr (SPL == 1) {
          tab[s_first & 1] = pk[0];
        } else {
#pragma unroll
          for (int e = 0; e < SPL; e += 2)
            *reinterpret_cast<uint2 *>(tab + 2 * RPAD * (e >> 1)) = make_uint2(pk[e], pk[e + 1]);
        }
      }

      // ---- MFMAs for the wave's row tiles.  The accumulator chains are
      //      interleaved with the sub-block-sum chain.
      floatx4 acc[TPW];
#pragma unroll
      for (int a = 0; a < TPW; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
      // xsb[c]: the B operand of the fp32 MFMA, the sum of x over
      // sub-block 4c + g for token r (lane group g picks its sub-block)
      float xsb[2] = {0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int j = j0 + jj;
        uint2 qb[TPW], sp[TPW];
#pragma unroll
        for (int a = 0; a < TPW; ++a) {
          const int row = 16 * (rt0 + a) + r;
          qb[a] = *reinterpret_cast<const uint2 *>(&wblk[row * WROW + 4 + 8 * j + 2 * g]);
          sp[a] = sc_tab[bb][j][row];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int s = 2 * j + h;
          const half8_t Bh = *reinterpret_cast<const half8_t *>(&xh[bb][r][16 * s + 4 * g]);
          const half8_t Bl = *reinterpret_cast<const half8_t *>(&xl[bb][r][16 * s + 4 * g]);
          half8_t A[TPW];
#pragma unroll
          for (int a = 0; a < TPW; ++a)
            A[a] = dequant8_ma(qb[a].x, qb[a].y, h != 0, h ? sp[a].y : sp[a].x, hi64);
          floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int a = 0; a < TPW; ++a)
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bh, acc[a], 0, 0, 0);
          sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bl, sx, 0, 0, 0);
#pragma unroll
          for (int a = 0; a < TPW; ++a)
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bl, acc[a], 0, 0, 0);
          // sum of x over sub-block s for token r (every row of the tile)
          if ((s & 3) == g) xsb[s >> 2] = sx[0];
        }
      }
      // token r (this lane's D column) entered block bb as x * 2^-e
      const int er = xe[bb][r];
      const float xs0 = __builtin_ldexpf(xsb[0], er), xs1 = __builtin_ldexpf(xsb[1], er);
#pragma unroll
      for (int a = 0; a < TPW; ++a) {
        const int rt = rt0 + a;
        // d of rows 16 rt + 4g + e (the rows of this lane's D elements)
        const float4 dv = *reinterpret_cast<const float4 *>(&d_tab[bb][16 * rt + 4 * g]);
        y_acc[a][0] += __builtin_ldexpf(dv.x * acc[a][0], er);
        y_acc[a][1] += __builtin_ldexpf(dv.y * acc[a][1], er);
        y_acc[a][2] += __builtin_ldexpf(dv.z * acc[a][2], er);
        y_acc[a][3] += __builtin_ldexpf(dv.w * acc[a][3], er);
        // lazy-dmin term: A[row][kk] = dmin*m of sub-block 4c + kk, B = sums
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (SPLIT && c != half) continue;  // wave-uniform: its own sub-blocks
          m_acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(c_tab[bb][4 * c + g][16 * rt + r],
                                                          c ? xs1 : xs0, m_acc[a], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next stage overwrites the LDS tiles
  }

  // ---- add the waves' partial tiles (through the activation tiles, no
  //      longer needed) and store.  Lane (token r, group g) holds rows
  //      16 rt + 4g + e of its token; partial slot (bb, s) of the rows.
  constexpr int RROW = ROWS + 4;
  // [block][token][RROW] per share: the first share in xh, the second in xl
  float *red0 = reinterpret_cast<float *>(&xh[0][0][0]);
  float *red1 = reinterpret_cast<float *>(&xl[0][0][0]);
  static_assert(PF_BLKS * PF_TOK * RROW <= PF_BLKS * PF_TOK * XROW,
                "the partial tiles must fit in the activation tiles");
  float *red = NS == 2 && half ? red1 : red0;
#pragma unroll
  for (int a = 0; a < TPW; ++a)
    *reinterpret_cast<float4 *>(&red[(bb * PF_TOK + r) * RROW + 16 * (rt0 + a) + 4 * g]) =
        make_float4(y_acc[a][0] - m_acc[a][0], y_acc[a][1] - m_acc[a][1],
                    y_acc[a][2] - m_acc[a][2], y_acc[a][3] - m_acc[a][3]);
  __syncthreads();
  for (int o = tid; o < PF_TOK * ROWS; o += PF_THREADS) {
    const int tok = o / ROWS, rr = o % ROWS;
    float v = 0.f;
#pragma unroll
    for (int b = 0; b < PF_BLKS; ++b) {
      v += red0[(b * PF_TOK + tok) * RROW + rr];
      if (NS == 2) v += red1[(b * PF_TOK + tok) * RROW + rr];
    }
    if (tok0 + tok < M && row0 + rr < N) Y[(int64_t)(tok0 + tok) * N + row0 + rr] = v;
  }
}

template <int ROWS, bool TILED>
hipError_t prefill_launch_rows(const float *X, const uint8_t *w, int64_t M, int64_t K, int64_t N,
                               float *Y, hipStream_t stream) {
  const int64_t nb = K / 256;
  // Offsets formed in the kernel (a row tile of ROWS rows plus one stage
  // past its end, 16 rows of X plus one stage) must stay below 2^31 bytes.
  if ((int64_t)ROWS * nb * kBlockBytes + 4 * kTileBytes >= ((int64_t)1 << 31) ||
      ((int64_t)PF_TOK * K + 2048) * 4 >= ((int64_t)1 << 31) || N > 0x7FFFFFFF ||
      M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)((M + PF_TOK - 1) / PF_TOK));
  if (grid.y > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((q4k_prefill_kernel<ROWS, TILED>), grid, dim3(PF_THREADS), 0, stream, X, w,
                     Y, (int)M, (int)nb, (int)N);
  return hipGetLastError();
}

template <bool TILED>
hipError_t prefill_launch_any(const float *X, const uint8_t *w, int64_t M, int64_t K, int64_t N,
                              float *Y, hipStream_t stream, int rows) {
  if (rows == 0) rows = prefill_rows(M, N);
  switch (rows) {
    case 64: return prefill_launch_rows<64, TILED>(X, w, M, K, N, Y, stream);
    case 32: return prefill_launch_rows<32, TILED>(X, w, M, K, N, Y, stream);
    case 16: return prefill_launch_rows<16, TILED>(X, w, M, K, N, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_rows(int64_t M, int64_t N) {
  // One workgroup per CU at a time (the LDS tiles allow no second), so a
  // height costs rounds of 256 workgroups x its per-workgroup time.  The
  // per-workgroup times measured on MI355X (graph-replayed calls, input_dim
  // 4096, 256 workgroups each, less the 1.4 us between graph nodes): 64 rows
  // 13.4 us, 32 rows 9.4, 16 rows 7.4, i.e. 100 : 70 : 55.  Measured
  // us/call, 64-row tiles vs the chosen height: 16 tokens x 4096 rows 14.6
  // vs 8.8 (16 rows), 32 x 4096 14.5 vs 10.8 (32 rows), 16 tokens 14336 ->
  // 4096 44.4 vs 25.5 (16 rows); 48 x 4096 and 16 x 14336 stay at 64 rows
  // (the 32-row grid, past one round, cost 19.6 vs 14.6 and 20.7 vs 15.8).
  const int64_t tok_groups = (M + PF_TOK - 1) / PF_TOK;
  const int rows[3] = {64, 32, 16};
  const int64_t cost[3] = {100, 70, 55};
  int best = 64;
  int64_t best_cost = INT64_MAX;
  for (int i = 0; i < 3; ++i) {
    const int64_t grid = (N + rows[i] - 1) / rows[i] * tok_groups;
    const int64_t c = (grid + 255) / 256 * cost[i];
    if (c < best_cost) { best_cost = c; best = rows[i]; }
  }
  return best;
}

hipError_t prefill_launch(const float *X, const uint8_t *w, int64_t M,
                          int64_t K, int64_t N, float *Y, hipStream_t stream, int rows) {
  // The library's own choice of 64-row tiles runs the kernel whose waves own
  // whole super-blocks (q4k_prefill_direct.hip): measured on MI355X
  // (graph-replayed calls over rotating weights, this file's kernel / that
  // one, us/call): 64x4096x4096 18.9 / 16.9, 48 tokens 18.2 / 16.9,
  // 64x14336->4096 60.0 / 42.9, 64x11008->4096 47.2 / 35.0, 64x4096->14336
  // 68.3 / 61.2, 128x4096x4096 34.4 / 31.0.  Here the per-(token,
  // super-block) maximum for the activations' scaling spans a whole wave,
  // there it is a maximum within each lane.  rows == 64 still forces this
  // file's kernel.
  if (rows == 0 && prefill_rows(M, N) == 64)
    return prefill_direct_launch(X, w, M, K, N, Y, stream);
  return prefill_launch_any<false>(X, w, M, K, N, Y, stream, rows);
}

hipError_t prefill_staged_tiled_launch(const float *X, const uint8_t *wt, int64_t M, int64_t K,
                                       int64_t N, float *Y, hipStream_t stream, int rows) {
  return prefill_launch_any<true>(X, wt, M, K, N, Y, stream, rows);
}

}  // namespace q4k
