// ternary_matmul.hip -- batched (prefill) ternary product on gfx950 MFMA.
//
// What it computes: the ternary page's prefill path (SKaiNET issue #1138,
// "[ternary-f32] Phase 2: TernaryF32GemvNative SPI + reference ViewKernel +
// TernaryF32KernelPack", section "Tasks") is a loop over token rows of the
// codes-dot; here every weight is read once for all tokens of a tile:
//     Y[r, o] = scale * sum_i (u(o, i) - 1) * X[r, i]
// with u the 2-bit field of element i (byte i/4, bits 2*(i%4)).
//
// Work decomposition and pipeline follow the Q4_K prefill kernel: a
// workgroup owns 64 rows (4 MFMA row tiles; 32 or 16 when few token tiles
// would leave CUs idle) and 16 tokens (one token tile) over the whole of
// input_dim and walks it in stages of 1024 positions.
// Every thread loads two 16-byte code chunks and eight activation float4
// of the next stage while the current one is computed; the activations go
// to LDS already split into exact fp16 hi + lo halves in MFMA operand order
// (positions paired (0,2), (1,3) within each group of four), each token's
// 256-position block first scaled by the power of two that brings its
// largest |x| into [2^14, 2^15) (so the halves neither overflow fp16 nor
// lose bits of lo to its subnormal range, for any |x| below 2^96).  Wave w takes
// positions 256*(w%4) .. +255 of the stage for its row tiles.
//
// Operands (16x16x32 f16 MFMA; lane (r, g) = (lane % 16, lane / 16)): MFMA
// step s = 2 s2 + h of a block takes from lane group g the code dword q =
// 4 s2 + g of row 16a + r (positions 16q .. 16q+15) and from it the fields
// of bytes h and h + 2: shifted right by 8h + 2p and masked with 0x00030003,
// the dword leaves positions 16q + 4h + p and 16q + 8 + 4h + p (p = 0..3) in
// its two halves, one shift and one AND-OR per pair.  The activations are
// staged in that operand order.  Each field u becomes the fp16 1024 + u
// (bits 0x6400 | u), and a packed subtraction of 1025 leaves the code u - 1
// in {-1, 0, 1, 2}, exactly.  (Feeding the raw fields as fp16
// subnormals u*2^-24 loses products of the lo halves on the matrix cores.)
// The MFMA products are exact and the accumulation is fp32: one tile per
// block, scaled back by the token's power of two into the running sum; the
// epilogue is Y = scale * D, one writer per output.
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int TR_TOK = 16;             // tokens per workgroup
constexpr int TR_WAVES = 8;
constexpr int TR_THREADS = 64 * TR_WAVES;
constexpr int TR_STAGE = 1024;         // positions per stage
constexpr int TR_CB = TR_STAGE / 4;    // code bytes of one row per stage
// LDS pitches in dwords: a token's activation row of one 256-position block
// (128 fp16 pairs) + 16 B; a row's codes of one stage (256 B) + 8 B.
constexpr int XROW = 128 + 4;
constexpr int CROW = TR_CB / 4 + 2;
constexpr int X_PER_THREAD = TR_TOK / 2;                          // 8

// The A operand from a dword of 16 codes (positions 0..15 of its range):
// for H = 0 the pairs (p, 8 + p), for H = 1 the pairs (4 + p, 12 + p), p =
// 0..3 (fields p of bytes H and H + 2), as the fp16 codes u - 1.  hi64 =
// 0x64006400 held in a vector register (vgpr_const), so that each
// mask-and-insert is one AND-OR.
template <int H>
__device__ __forceinline__ half8_t code_operand(uint32_t w, uint32_t hi64) {
  uint4 v;  // fp16 1024 + u in each half
  v.x = ((w >> (8 * H)) & 0x00030003u) | hi64;
  v.y = ((w >> (8 * H + 2)) & 0x00030003u) | hi64;
  v.z = ((w >> (8 * H + 4)) & 0x00030003u) | hi64;
  v.w = ((w >> (8 * H + 6)) & 0x00030003u) | hi64;
  half8_t a = __builtin_bit_cast(half8_t, v);
  const _Float16 off = (_Float16)1025.0f;
  return a - half8_t{off, off, off, off, off, off, off, off};
}

// ROWS = 64, 32 or 16 rows (RT row tiles) per workgroup.  Wave (bb, half):
// with 4 row tiles, tiles 2 half and 2 half + 1 over the block's eight
// 32-position steps; with 2, tile half; with 1, the one tile over steps
// 4 half .. 4 half + 3.
template <int ROWS>
__global__ __launch_bounds__(TR_THREADS) void ternary_matmul_kernel(
    const float *X, const uint8_t *codes, float *__restrict__ Y, float scale, int M, int K,
    int N) {
  constexpr int RT = ROWS / 16;
  constexpr int TPW = RT == 4 ? 2 : 1;       // row tiles per wave
  constexpr int NSTEP = RT == 1 ? 4 : 8;     // 32-position steps per wave and block
  constexpr int NS = RT == 1 ? 2 : 1;        // waves sharing a block's rows
  constexpr int CHUNKS = ROWS * TR_CB / 16;  // 16-byte code chunks per stage
  constexpr int C_PER_THREAD = CHUNKS > TR_THREADS ? CHUNKS / TR_THREADS : 1;
  constexpr int C_WAVES = CHUNKS >= TR_THREADS ? TR_WAVES : CHUNKS / 64;  // waves that load codes
  static_assert(C_PER_THREAD * 64 * C_WAVES == CHUNKS, "code chunks must divide evenly");
  // xh/xl: fp16 hi and lo activations [block of stage][token][pairs in
  // operand order]; ct: the stage's codes [row][dword].
  __shared__ __align__(16) uint32_t xh[4][TR_TOK][XROW];
  __shared__ __align__(16) uint32_t xl[4][TR_TOK][XROW];
  __shared__ __align__(16) uint32_t ct[ROWS * CROW];
  __shared__ int xe[4][TR_TOK];  // scaling exponent per (block, token) of the stage

  // The host validates K >= 64; saying so lets the compiler fetch every
  // kernel argument in one round trip.
  __builtin_assume(K >= 64);
  const uint32_t hi64 = vgpr_const(0x64006400u);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = tid & 255;     // thread index within its half of the workgroup
  const int bb = wave & 3;     // 256-position block of the stage this wave computes
  const int half = wave >> 2;
  const int rt0 = RT == 4 ? 2 * half : (RT == 2 ? half : 0);  // first row tile of this wave
  const int s0 = RT == 1 ? 4 * half : 0;                      // first step of this wave
  const bool c_loader = wave < C_WAVES;
  const int r = lane & 15;     // A: row within a row tile; B and D: token
  const int g = lane >> 4;
  const int row0 = blockIdx.x * ROWS;
  const int tok0 = blockIdx.y * TR_TOK;
  const int row_bytes = K / 4;
  const int n_stages = (K + TR_STAGE - 1) / TR_STAGE;

  // Range-checked views: rows past N and tokens past M read as zeros;
  // positions past K are zeroed in the load offsets below (a zero
  // activation makes any code byte harmless).
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(codes + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // code chunk q = t + 256*m + ...: row q / 16, chunk q % 16 of the row's
  // 256 stage bytes; activations: wave w stages block w % 4 of the stage for
  // the tokens of parity w / 4, lane (token 2 (lane / 8) + w / 4, j = lane %
  // 8) taking positions P .. P+3 and P+8 .. P+11 of the block, P = 64 s2 +
  // 16 (j / 2) + 4 (j % 2) (s2 = 0..3): the operand pairs of MFMA step 2 s2
  // + j % 2, lane group j / 2, and a token's 8 lanes hold its whole block.
  uint4 cv[C_PER_THREAD];
  float4 xv[X_PER_THREAD];
  int coff[C_PER_THREAD];
#pragma unroll
  for (int m = 0; m < C_PER_THREAD; ++m) {
    const int q = tid + TR_THREADS * m;
    coff[m] = (q >> 4) * row_bytes + 16 * (q & 15);
  }
  const int tok_lo = tid >> 8;
  const int xb = t >> 6;                     // block of the stage this wave stages
  const int xj = lane & 7;
  const int xg = xj >> 1, xh2 = xj & 1;       // the operand lane group and half it feeds
  const int xtok = 2 * (lane >> 3) + tok_lo;  // this lane's token
  const int xpos = 256 * xb + 16 * xg + 4 * xh2;  // + 64 s2 (+ 8): its positions in the stage
  auto load_stage = [&](int st) {
    // positions past K (a ragged last stage, K a multiple of 64) read as
    // zeros: their offsets are moved past the end of the view, since the
    // bytes there would be the next token's activations
#pragma unroll
    for (int c = 0; c < X_PER_THREAD; ++c) {
      const int pos = xpos + 64 * (c >> 1) + 8 * (c & 1);
      const bool in_k = st * TR_STAGE + pos < K;
      xv[c] = load_buf_f4(xr, in_k ? 4 * K * xtok + 4 * pos : 0x7FFFFFF0, 4096 * st);
    }
#pragma unroll
    for (int m = 0; m < C_PER_THREAD; ++m)
      if (c_loader) cv[m] = __builtin_bit_cast(uint4, load_buf_f4(cr, coff[m], TR_CB * st));
  };
  auto stage_to_lds = [&]() {
    // the token's block maximum: a chain over the lane's 32 values, then a
    // maximum over its 8 lanes
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
    for (int s2 = 0; s2 < X_PER_THREAD / 2; ++s2) {
      const float4 a = xv[2 * s2], b = xv[2 * s2 + 1];  // positions P + p, P + 8 + p
      uint4 h, l;
      split_pair(a.x, b.x, sdown, h.x, l.x);
      split_pair(a.y, b.y, sdown, h.y, l.y);
      split_pair(a.z, b.z, sdown, h.z, l.z);
      split_pair(a.w, b.w, sdown, h.w, l.w);
      const int d = 16 * (2 * s2 + xh2) + 4 * xg;  // step 2 s2 + xh2, lane group xg
      *reinterpret_cast<uint4 *>(&xh[xb][xtok][d]) = h;
      *reinterpret_cast<uint4 *>(&xl[xb][xtok][d]) = l;
    }
    if (c_loader) {
#pragma unroll
      for (int m = 0; m < C_PER_THREAD; ++m) {
        const int q = tid + TR_THREADS * m;
        uint32_t *dst = &ct[(q >> 4) * CROW + 4 * (q & 15)];
        *reinterpret_cast<uint2 *>(dst) = make_uint2(cv[m].x, cv[m].y);
        *reinterpret_cast<uint2 *>(dst + 2) = make_uint2(cv[m].z, cv[m].w);
      }
    }
  };

  floatx4 acc[TPW];
#pragma unroll
  for (int a = 0; a < TPW; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  // this lane's codes for step s of block bb: dword 16 bb + 4 (s / 2) + g of
  // its row in the stage

  load_stage(0);
  for (int st = 0; st < n_stages; ++st) {
    stage_to_lds();
    // The registers are free again: the next stage's loads leave before the
    // barrier and stay in flight during the MFMAs (measured 5-7% faster than
    // after it at every height).
    if (st + 1 < n_stages) load_stage(st + 1);
    __syncthreads();
    // per row tile: the block's hi and lo products in separate accumulators
    // (four independent MFMA chains)
    floatx4 bh[TPW], bl[TPW];
#pragma unroll
    for (int a = 0; a < TPW; ++a) bh[a] = bl[a] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < NSTEP; ++ss) {
      const int s = s0 + ss;
      const half8_t Bh = *reinterpret_cast<const half8_t *>(&xh[bb][r][16 * s + 4 * g]);
      const half8_t Bl = *reinterpret_cast<const half8_t *>(&xl[bb][r][16 * s + 4 * g]);
#pragma unroll
      for (int a = 0; a < TPW; ++a) {
        const int row = 16 * (rt0 + a) + r;
        const uint32_t w = ct[row * CROW + 16 * bb + 4 * (s >> 1) + g];
        const half8_t A = (ss & 1) ? code_operand<1>(w, hi64) : code_operand<0>(w, hi64);
        bh[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, bh[a], 0, 0, 0);
        bl[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, bl[a], 0, 0, 0);
      }
    }
    // undo the scaling of token r's block (the D column of this lane)
    const int e = xe[bb][r];
#pragma unroll
    for (int a = 0; a < TPW; ++a)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[a][k] += __builtin_ldexpf(bh[a][k] + bl[a][k], e);
    __syncthreads();  // the next stage overwrites the LDS tiles
  }

  // Add the waves' partial tiles (through the activation tiles, no longer
  // needed); lane (token r, group g) holds rows 16 rt + 4g + e; partial slot
  // (block, share) of the rows.
  constexpr int RROW = ROWS + 4;
  float *red = reinterpret_cast<float *>(&xh[0][0][0]);  // [block][share][token][RROW]
  static_assert(4 * NS * TR_TOK * RROW <= 4 * TR_TOK * XROW,
                "the partial tiles must fit in the activation tile");
  const int shr = RT == 1 ? half : 0;
#pragma unroll
  for (int a = 0; a < TPW; ++a)
    *reinterpret_cast<float4 *>(&red[((bb * NS + shr) * TR_TOK + r) * RROW + 16 * (rt0 + a) + 4 * g]) =
        make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
  __syncthreads();
  for (int o = tid; o < TR_TOK * ROWS; o += TR_THREADS) {
    const int tok = o / ROWS, rr = o % ROWS;
    float v = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) v += red[((b * NS + s2) * TR_TOK + tok) * RROW + rr];
    if (tok0 + tok < M && row0 + rr < N) Y[(int64_t)(tok0 + tok) * N + row0 + rr] = scale * v;
  }
}

template <int ROWS>
hipError_t ternary_matmul_launch_rows(const float *X, const uint8_t *codes, float scale,
                                      int64_t M, int64_t K, int64_t N, float *Y,
                                      hipStream_t stream) {
  const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)((M + TR_TOK - 1) / TR_TOK));
  if (grid.y > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ternary_matmul_kernel<ROWS>, grid, dim3(TR_THREADS), 0, stream, X, codes, Y,
                     scale, (int)M, (int)K, (int)N);
  return hipGetLastError();
}

}  // namespace

hipError_t ternary_matmul_launch(const float *X, const uint8_t *codes, float scale, int64_t M,
                                 int64_t K, int64_t N, float *Y, hipStream_t stream, int rows) {
  // Offsets formed in the kernel (64 rows of codes, 16 rows of X, plus one
  // stage) must stay below 2^31 bytes; K must be whole 16-byte code chunks.
  if (K % 64 != 0 || (int64_t)64 * (K / 4) + 4096 >= ((int64_t)1 << 31) ||
      ((int64_t)TR_TOK * K + 4096) * 4 >= ((int64_t)1 << 31) || N > 0x7FFFFFFF ||
      M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  if (rows == 0) rows = prefill_rows(M, N);
  switch (rows) {
    case 64: return ternary_matmul_launch_rows<64>(X, codes, scale, M, K, N, Y, stream);
    case 32: return ternary_matmul_launch_rows<32>(X, codes, scale, M, K, N, Y, stream);
    case 16: return ternary_matmul_launch_rows<16>(X, codes, scale, M, K, N, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4k
