// q4k_prefill_splitk.hip -- batched (prefill) Q4_K product Y = X W^T on the
// gfx950 matrix cores with 128-row x 32-token tiles whose input_dim may be
// split across workgroups.
//
// What it computes is q4k_matmul's product (Q4_K page: SKaiNET PR #562,
// "feat(kernel): SIMD-fused Q4_K matmul kernel + Q4KMatmulKernel SPI",
// sections "Summary" and "Pipeline", in the lazy-dmin form, for every token
// row as in the ternary page's prefill row loop, SKaiNET issue #1138, section
// "Tasks"):
//     Y[r, o] = sum_b d * sum_s sc_s * sum_l q * X[r, k] - dmin * sum_s m_s * sum_l X[r, k].
// Each workgroup reads every weight byte of its tile once for 32 tokens, and
// with 64 tokens two workgroups on one XCD share the tile through its L2 (the
// tiling page: llama.cpp fork PR #37, "ggml-cpu: cache-aware tiling in
// ggml_compute_forward_mul_mat", section "Summary", fix 1).
//
// Work decomposition.  A work item is 128 weight rows (8 MFMA row tiles) x 32
// tokens (2 token tiles) x one of S equal ranges of super-blocks; S > 1 when
// the (rows, tokens) tiles alone would leave CUs idle.  Work items are
// numbered token tile fastest, then row tile, then range, and consecutive
// numbers are given to workgroups on the same XCD (workgroups are dealt to the
// 8 XCDs in turn), so the token tiles of a row tile share its weights in one
// L2 and each XCD fetches the activations of few ranges.
//
// A workgroup's 8 waves form two halves of 4; in each step half h takes the
// next super-block of the range (b0 + 2i + h), and wave v of a half owns rows
// 32v .. 32v+31 of the tile for all 32 tokens.  Per step and half:
//   - the 256 lanes split the 32 tokens' activations once for all rows:
//     lane (token, column c) loads 16 bytes of each of the 8 sub-blocks (the
//     token's 8 lanes read whole 128-byte lines), scales the token's block by
//     the power of two that brings its largest |x| into [2^14, 2^15) (a
//     maximum over the 8 lanes) and writes exact fp16 hi and lo halves into
//     B-operand images in LDS; the 8 lanes' partial sums are reduced so that
//     lane c ends with sub-block c's sum, written (times 2^-5, also as hi +
//     lo) for the min term;
//   - every wave decodes its 32 rows' headers into a wave-private table,
//     then turns each lane's qs bytes into A = sc*q (exact in fp16, masked
//     under 0x6400 and one packed fma per pair) and runs 16x16x32 f16 MFMAs
//     against the hi and lo images: one A operand feeds both token tiles;
//   - one 16x16x16 MFMA per (row tile, token tile) gives sum_s m_s * (sum of
//     x over s) from 32*m and the sums' images;
//   - 2^e * (d * tile - dmin * min tile) goes into the running result.
// The images are double-buffered, one barrier per step.  Activations are
// loaded two steps ahead and weights one step ahead, and the next step's
// activations are split between this step's MFMAs (sub-block t alongside
// MFMA t), so that a wave's VALU and matrix-core work overlap.
//
// The MFMA contraction order.  A lane (row i, lane group g) holds 32 qs
// bytes of its row: [16g, 16g+16) and [64+16g, 64+16g+16).  MFMA t = 2dp+n
// (dp = 0..3, n = nibble) takes 8 of their codes, bytes 8(dp&1) .. +7 of
// load dp>>1, so its 32 contraction slots cover positions
//     k = 128(dp>>1) + 64(g>>1) + 32n + 16(g&1) + 8(dp&1) + e
// (two sub-blocks per MFMA; A carries each one's scale).  The images hold x
// at those positions, in the operand order of the codes ((0,2), (1,3), ...).
//
// End: the halves' results are added (half 0 + half 1), and each wave of
// half 0 finishes its 32 rows on its own.  With S = 1 it stores them to Y.
// With S > 1 it stores them to its range's workspace slot with the
// agent-coherent cache policy and, once those stores are complete, counts
// its arrival at the counter of (tile, wave); the wave that finds itself the
// S-th arrival reads the S slots' rows back (same policy), adds them in range
// order, stores them to Y and resets the counter to zero, so every output has
// one writer and the same bits whatever the arrival order.  Y is stored from
// the MFMA layout directly: 16 bytes (4 rows of one token) per lane.
#include <type_traits>

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

constexpr int kBlockBytes = 144;
constexpr int SK_ROWS = 128;
constexpr int SK_TOK = 32;
constexpr int SK_WAVES = 8;
constexpr int SK_THREADS = 64 * SK_WAVES;
constexpr int SK_TILE = SK_ROWS * SK_TOK;  // floats of one workspace slot
// cache policy (aux) of the workspace accesses: sc1, coherent across XCDs
constexpr int kCoherent = 16;

// One half's image buffer (bytes).  Image I = (t*2 + tt)*2 + hl holds MFMA
// t's B operand for token tile tt (hl: hi or lo halves) at I*SK_IMG +
// SK_ISHIFT*(I >> 3), lane (token j, group g) 16 (j + 16 g) into it: every
// 16-lane quarter reads 256 contiguous bytes.  The pad and the shift were
// picked with the bank-conflict counter: the splitting lanes' 8-byte stores
// cost 4 conflict cycles each, 12 without the shift (every stride tried that
// keeps the images 16-byte aligned).
constexpr int SK_IMG = 1024 + 16;
constexpr int SK_ISHIFT = 32;                   // added per 8 images: img_off(I)
constexpr int SK_MIMG = 32 * SK_IMG + 4 * SK_ISHIFT;  // sums' images: 2 token tiles x 64 lanes x 8 B
constexpr int SK_ETAB = SK_MIMG + 2 * 512;      // 32 exponents e
constexpr int SK_HBUF = SK_ETAB + SK_TOK * 4;
// A wave's header table (dwords): 32 rows x 8 scale pairs, 32 rows x 4
// dwords of 32*m (operand order m0, m2 | m1, m3 | m4, m6 | m5, m7), 32 rows
// of (d | dmin << 16).
constexpr int SK_TSC = 0;
constexpr int SK_TMN = 32 * 8;
constexpr int SK_TDD = SK_TMN + 32 * 4;
constexpr int SK_TAB = SK_TDD + 32;
constexpr int SK_LDS = 4 * SK_HBUF + SK_WAVES * SK_TAB * 4;
static_assert(SK_LDS <= 160 * 1024, "LDS of one workgroup");
static_assert(SK_WAVES / 2 * 4 * 64 * 16 <= SK_LDS, "half 1's sums must fit in the image buffers");

// 32*m for the two 6-bit mins in bytes 0 and 2 of `v` (bytes 1 and 3 zero),
// as an fp16 pair: v | 0x6400 in each half is 1024 + m, and
// 32 * (1024 + m) - 32768 is exact in fp16.
__device__ __forceinline__ uint32_t mins32(uint32_t v, uint32_t hi64) {
  const half2_t t = as_h2(v | hi64);
  return as_u32h(__builtin_elementwise_fma(t, half2_t{(_Float16)32.0f, (_Float16)32.0f},
                                           half2_t{(_Float16)-32768.0f, (_Float16)-32768.0f}));
}

// v, from the lane that DPP control CTRL names (within rows of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, true));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(SK_THREADS) void q4k_prefill_splitk_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, float *part, unsigned *cnt,
    int M, int nb, int N, int S, int n_rt, int n_tt) {
  __shared__ __align__(16) uint8_t lds[SK_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, wv = wave & 3;
  const int i16 = lane & 15;  // A: row of a row tile; B and D: token of a token tile
  const int g = lane >> 4;

  // ---- work item (consecutive numbers on one XCD)
  // Every quantity here is non-negative and below 2^31 (the launcher
  // checks the grid; s * nb < 8 * 2^17), so unsigned 32-bit divisions give
  // the same values as signed or 64-bit ones at a fraction of the
  // instructions, all of which run before the first load.
  const unsigned G = gridDim.x, L = blockIdx.x;
  const unsigned xcd = L & 7, q8 = G >> 3, r8 = G & 7;
  const unsigned work = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + (L >> 3);
  const unsigned rest = work / (unsigned)n_tt;
  const int tti = (int)(work - rest * (unsigned)n_tt);
  const unsigned sq = rest / (unsigned)n_rt;
  const int rti = (int)(rest - sq * (unsigned)n_rt);
  const int s = (int)sq;
  const int tile = rti * n_tt + tti;
  const int row0 = rti * SK_ROWS, tok0 = tti * SK_TOK;
  const int b0 = (int)((unsigned)(s * nb) / (unsigned)S);
  const int b1 = (int)((unsigned)((s + 1) * nb) / (unsigned)S);
  const int n_steps = (b1 - b0 + 1) >> 1;
  const int K = nb * 256;
  const int row_bytes = nb * kBlockBytes;

  // Range-checked views: rows past N and tokens past M read as zeros.
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // weights: qs bytes [16g, 16g+16) and [64+16g, ...) of rows 32wv + 16rt + i16;
  // lane l's header: row 32wv + (l & 31)
  const int wq_off = (32 * wv + i16) * row_bytes + 16 + 16 * g;
  const int wq_off1 = wq_off + 16 * row_bytes;
  const int hd_off = (32 * wv + (lane & 31)) * row_bytes;
  // activations: lane (token tl, column j) of the half takes x[tl][32c + 4j
  // .. +3] of sub-blocks c = 0..7
  const int tl = 8 * wv + (lane >> 3);
  const int j = lane & 7;
  const int x_off = tl * K * 4 + 16 * j;

  auto load_w = [&](int b, uint4 (&q)[2][2], uint4 &h) {  // b wave-uniform
    const int so = kBlockBytes * b;
    q[0][0] = __builtin_bit_cast(uint4, load_buf_f4(wr, wq_off, so));
    q[0][1] = __builtin_bit_cast(uint4, load_buf_f4(wr, wq_off + 64, so));
    q[1][0] = __builtin_bit_cast(uint4, load_buf_f4(wr, wq_off1, so));
    q[1][1] = __builtin_bit_cast(uint4, load_buf_f4(wr, wq_off1 + 64, so));
    h = __builtin_bit_cast(uint4, load_buf_f4(wr, hd_off, so));
  };
  auto load_x = [&](int b, float4 (&xv)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) xv[c] = load_buf_f4(xr, x_off + 128 * c, 1024 * b);
  };

  const uint32_t hi64 = vgpr_const(0x64006400u);

  // ---- split this lane's 32 activations into the images of buffer hb, in
  //      three parts so that the middle one can run between a step's MFMAs:
  //      the token's exponent e, then sub-block c's hi and lo halves (and
  //      the lane's partial sum of it), then the sums and e themselves
  auto split_exponent = [&](const float4 (&xv)[8]) {
    float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      mx0 = absmax3(absmax3(mx0, xv[c].x, xv[c].y), xv[c].z, xv[c].w);
      mx1 = absmax3(absmax3(mx1, xv[c + 1].x, xv[c + 1].y), xv[c + 1].z, xv[c + 1].w);
    }
    const float mx = group_max_nonneg<8>(fmaxf(mx0, mx1));  // the token's 8 lanes
    // |x| * 2^-e < 2^15; e >= -126 keeps both powers of two normal floats
    const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    return e < -126 ? -126 : e;
  };
  // x[32c + 4j .. +3] is half (j & 1) of 8-position segment 4c + (j >> 1),
  // MFMA t's slots of lane group gg (operand order (0,2), (1,3) | (4,6),
  // (5,7): the low or high 8 bytes of the image entry)
  const int x_tt = tl >> 4, x_tok16 = tl & 15;
  const int x_img = (x_tt * 2 + 8 * ((j >> 1) & 1)) * SK_IMG + SK_ISHIFT * ((j >> 1) & 1) +
                    256 * (j >> 2) + 16 * x_tok16 +
                    8 * (j & 1);
  auto split_chunk = [&](uint8_t *hb, const float4 &v, int c, float sdown) {
    uint2 h, l;
    split_pair(v.x, v.z, sdown, h.x, l.x);
    split_pair(v.y, v.w, sdown, h.y, l.y);
    const int t0 = 4 * (c >> 2) + (c & 1);  // t = t0 + 2 ((j >> 1) & 1)
    // group 2((c>>1)&1) + (j>>2); images 4 t0 + ... sit 2 (c >> 2) shifts on
    const int off = x_img + t0 * 4 * SK_IMG + 2 * SK_ISHIFT * (c >> 2) + 512 * ((c >> 1) & 1);
    *reinterpret_cast<uint2 *>(hb + off) = h;
    *reinterpret_cast<uint2 *>(hb + off + SK_IMG) = l;
    return sum4(v);
  };
  // sub-block sums: a reduce-scatter of the lane's partial sums over the
  // token's 8 lanes (lane j <-> 7 - j, then j ^ 2, then j ^ 1, each lane
  // keeping half of what it holds) leaves sub-block j's sum in lane j
  auto split_sums = [&](uint8_t *hb, const float (&ps)[8], int e) {
    float r4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a0 = ps[k] + dpp_f32<0x141>(ps[k]);          // row_half_mirror
      const float a1 = ps[k + 4] + dpp_f32<0x141>(ps[k + 4]);
      r4[k] = j < 4 ? a0 : a1;
    }
    float r2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float a0 = r4[k] + dpp_f32<0x4E>(r4[k]);           // quad_perm [2,3,0,1]
      const float a1 = r4[k + 2] + dpp_f32<0x4E>(r4[k + 2]);
      r2[k] = (j & 2) ? a1 : a0;
    }
    const float c0 = r2[0] + dpp_f32<0xB1>(r2[0]);             // quad_perm [1,0,3,2]
    const float c1 = r2[1] + dpp_f32<0xB1>(r2[1]);
    const float sum = (j & 1) ? c1 : c0;
    // sub-block j's sum times 2^-e * 2^-5 (below 2^15) as hi + lo: slot
    // order 0, 2, 1, 3 within each group of four sub-blocks, hi halves in
    // lane groups 0 and 1, lo halves in 2 and 3
    const float s5 = __builtin_ldexpf(sum, -e - 5);
    const _Float16 mh = (_Float16)s5;
    const _Float16 ml = (_Float16)(s5 - (float)mh);
    const int qq = j & 3, pos = ((qq & 1) << 1) | (qq >> 1);
    _Float16 *mi = reinterpret_cast<_Float16 *>(hb + SK_MIMG + x_tt * 512);
    mi[(x_tok16 + 16 * (j >> 2)) * 4 + pos] = mh;
    mi[(x_tok16 + 16 * (2 + (j >> 2))) * 4 + pos] = ml;
    if (j == 0) reinterpret_cast<int *>(hb + SK_ETAB)[tl] = e;
  };
  auto split_write = [&](uint8_t *hb, const float4 (&xv)[8]) {
    const int e = split_exponent(xv);
    const float sdown = __builtin_ldexpf(1.0f, -e);
    float ps[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ps[c] = split_chunk(hb, xv[c], c, sdown);
    split_sums(hb, ps, e);
  };

  uint32_t *tab = reinterpret_cast<uint32_t *>(lds + 4 * SK_HBUF) + wave * SK_TAB;
  floatx4 yacc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) yacc[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- one super-block of the wave's 32 rows against the images of hb
  // With SPLIT, the next step's activations xs are split into buffer hs
  // between this step's MFMAs (sub-block c = t alongside MFMA t).
  auto mfma_step = [&](const uint8_t *hb, const uint4 (&q)[2][2], const uint4 &hd, auto split_tag,
                       uint8_t *hs, const float4 (&xs)[8]) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    int xe = 0;
    float sdown = 0.f;
    float ps[8];
    if constexpr (SPLIT) {
      xe = split_exponent(xs);
      sdown = __builtin_ldexpf(1.0f, -xe);
    }
    // headers: lanes 0-31 decode scales and (d, dmin) of row lane, lanes
    // 32-63 the mins of row lane - 32
    wave_sync_lds();
    if (lane < 32) {
      const uint32_t sc03 = hd.y & 0x3F3F3F3Fu;
      const uint32_t sc47 = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
      uint4 r0, r1;
      // even sub-blocks are low nibbles, odd ones high nibbles kept in place
      r0.x = scale_pair(sc03 & 255u, false);
      r0.y = scale_pair((sc03 >> 8) & 255u, true);
      r0.z = scale_pair((sc03 >> 16) & 255u, false);
      r0.w = scale_pair(sc03 >> 24, true);
      r1.x = scale_pair(sc47 & 255u, false);
      r1.y = scale_pair((sc47 >> 8) & 255u, true);
      r1.z = scale_pair((sc47 >> 16) & 255u, false);
      r1.w = scale_pair(sc47 >> 24, true);
      *reinterpret_cast<uint4 *>(&tab[SK_TSC + 8 * lane]) = r0;
      *reinterpret_cast<uint4 *>(&tab[SK_TSC + 8 * lane + 4]) = r1;
      tab[SK_TDD + lane] = hd.x;  // d | dmin << 16
    } else {
      const uint32_t mn03 = hd.z & 0x3F3F3F3Fu;
      const uint32_t mn47 = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
      uint4 r2;
      r2.x = mins32(mn03 & 0x00FF00FFu, hi64);
      r2.y = mins32((mn03 >> 8) & 0x00FF00FFu, hi64);
      r2.z = mins32(mn47 & 0x00FF00FFu, hi64);
      r2.w = mins32((mn47 >> 8) & 0x00FF00FFu, hi64);
      *reinterpret_cast<uint4 *>(&tab[SK_TMN + 4 * (lane - 32)]) = r2;
    }
    wave_sync_lds();

    // scale pairs of sub-blocks 4h + 2(g>>1) + {0, 1} of the lane's rows
    uint2 sp[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = 16 * rt + i16;
      sp[rt][0] = *reinterpret_cast<const uint2 *>(&tab[SK_TSC + 8 * row + 2 * (g >> 1)]);
      sp[rt][1] = *reinterpret_cast<const uint2 *>(&tab[SK_TSC + 8 * row + 4 + 2 * (g >> 1)]);
    }
    floatx4 acc[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dp = 0; dp < 4; ++dp) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int t = 2 * dp + n;
        half8_t bh[2], bl[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int off = (t * 2 + tt) * 2 * SK_IMG + SK_ISHIFT * (t >> 1) + 16 * lane;
          bh[tt] = *reinterpret_cast<const half8_t *>(hb + off);
          bl[tt] = *reinterpret_cast<const half8_t *>(hb + off + SK_IMG);
        }
        if constexpr (SPLIT) ps[t] = split_chunk(hs, xs[t], t, sdown);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const uint4 &qv = q[rt][dp >> 1];
          const uint32_t w0 = (dp & 1) ? qv.z : qv.x;
          const uint32_t w1 = (dp & 1) ? qv.w : qv.y;
          const uint32_t ma = n ? sp[rt][dp >> 1].y : sp[rt][dp >> 1].x;
          const half8_t A = dequant8_ma(w0, w1, n != 0, ma, hi64);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[tt], acc[rt][tt], 0, 0, 0);
            acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[tt], acc[rt][tt], 0, 0, 0);
          }
        }
      }
    }

    // min term: A = 32*m of the lane's row (slots 4g .. 4g+3), B = the sums'
    // images
    half4_t bm[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      bm[tt] = *reinterpret_cast<const half4_t *>(hb + SK_MIMG + tt * 512 + 8 * lane);
    const int *et = reinterpret_cast<const int *>(hb + SK_ETAB);
    float sup[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) sup[tt] = __builtin_ldexpf(1.0f, et[16 * tt + i16]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const half4_t am = *reinterpret_cast<const half4_t *>(
          &tab[SK_TMN + 4 * (16 * rt + i16) + 2 * (g & 1)]);
      // (d, dmin) of rows 16rt + 4g + k, this lane's D rows
      const uint4 dv = *reinterpret_cast<const uint4 *>(&tab[SK_TDD + 16 * rt + 4 * g]);
      const uint32_t dk[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const floatx4 mt = __builtin_amdgcn_mfma_f32_16x16x16f16(
            am, bm[tt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float tv = half_lo(dk[k]) * acc[rt][tt][k] - half_hi(dk[k]) * mt[k];
          yacc[rt][tt][k] = __builtin_fmaf(tv, sup[tt], yacc[rt][tt][k]);
        }
      }
    }
    if constexpr (SPLIT) split_sums(hs, ps, xe);
  };

  auto hbuf = [&](int p) { return lds + (p * 2 + half) * SK_HBUF; };

  // ---- steps: half h takes super-blocks b0 + h, b0 + h + 2, ...  Loads run
  // ahead: the activations two steps (split at the end of the step before
  // their own), the weights one step (issued once this step's MFMAs have
  // read the registers they go to).  Two register sets alternate, so the
  // loop body is written for a pair of steps.
  uint4 wA[2][2], hA, wB[2][2], hB;
  float4 xA[8], xB[8];
  auto sb = [&](int i) { return b0 + 2 * i + half; };  // wave-uniform
  if (sb(0) < b1) {
    load_w(sb(0), wA, hA);
    load_x(sb(0), xA);
    split_write(hbuf(0), xA);
  }
  // the second step's loads leave once the first step's activations are
  // in: issued together they share the bandwidth and hold up the first
  if (sb(1) < b1) {
    load_w(sb(1), wB, hB);
    load_x(sb(1), xB);
  }
  __syncthreads();
  // step i: weights of i in (wc, hc), of i + 1 in flight in (wn, hn);
  // activations of i + 1 in xn (split at the end), xf free for i + 2
  auto step = [&](int i, uint4 (&wc)[2][2], uint4 &hc, float4 (&xn)[8], float4 (&xf)[8]) {
    if (sb(i + 2) < b1) load_x(sb(i + 2), xf);
    if (sb(i + 1) < b1)  // then sb(i) < b1 too
      mfma_step(hbuf(i & 1), wc, hc, std::true_type{}, hbuf((i + 1) & 1), xn);
    else if (sb(i) < b1)
      mfma_step(hbuf(i & 1), wc, hc, std::false_type{}, hbuf((i + 1) & 1), xn);
    if (sb(i + 2) < b1) load_w(sb(i + 2), wc, hc);
    __syncthreads();
  };
  for (int i = 0; i < n_steps; i += 2) {
    step(i, wA, hA, xB, xA);
    if (i + 1 < n_steps) step(i + 1, wB, hB, xA, xB);
  }

  // ---- half 0 + half 1 (the loop ended with a barrier: the images are free)
  float *red = reinterpret_cast<float *>(lds);
  if (half == 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<floatx4 *>(&red[((wv * 4 + c) * 64 + lane) * 4]) = yacc[c >> 1][c & 1];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      yacc[c >> 1][c & 1] += *reinterpret_cast<const floatx4 *>(&red[((wv * 4 + c) * 64 + lane) * 4]);
  }

  if (half == 1) return;  // half 0 holds the workgroup's sums

  if (S > 1) {
    // Per wave: this range's 32 rows into its workspace slot (lane order),
    // then the arrival count of (tile, wave).  The slots are written and
    // read with the agent-coherent cache policy (sc1: written through the
    // XCD's L2, read past stale L2 lines), each writer waits for its stores
    // to complete before its arrival is counted, and the last arrival reads
    // the slots only after its own count returned; so no L2 write-back or
    // invalidate is needed (an agent-scope release fence per workgroup costs
    // a whole-L2 write-back, measured at ~20 us per 64x4096x4096 call).
    // Every slot is read back, this wave's own included: the same additions
    // in range order whichever wave comes last.
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part + (int64_t)tile * S * SK_TILE, (int64_t)S * SK_TILE * 4);
    const int pv = ((wv * 4) * 64 + lane) * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yacc[c >> 1][c & 1]), pr,
                                             pv + 1024 * c, s * SK_TILE * 4, kCoherent);
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&cnt[tile * 4 + wv], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    old = (unsigned)__builtin_amdgcn_readfirstlane((int)old);
    if (old != (unsigned)(S - 1)) return;  // wave-uniform
    if (lane == 0)
      __hip_atomic_store(&cnt[tile * 4 + wv], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      yacc[c >> 1][c & 1] = __builtin_bit_cast(
          floatx4, __builtin_amdgcn_raw_buffer_load_b128(pr, pv + 1024 * c, 0, kCoherent));
    for (int s2 = 1; s2 < S; ++s2) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        yacc[c >> 1][c & 1] += __builtin_bit_cast(
            floatx4,
            __builtin_amdgcn_raw_buffer_load_b128(pr, pv + 1024 * c, s2 * SK_TILE * 4, kCoherent));
    }
  }

  // lane (token i16, group g) holds rows 4g .. 4g+3 of each (row tile, token tile)
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = tok0 + 16 * tt + i16, row = row0 + 32 * wv + 16 * rt + 4 * g;
      if (tok >= M) continue;
      float *yr = Y + (int64_t)tok * N + row;
      if (vec && row < N) {
        *reinterpret_cast<floatx4 *>(yr) = yacc[rt][tt];
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (row + k < N) yr[k] = yacc[rt][tt][k];
      }
    }
}

}  // namespace

SplitkPlan splitk_plan(int64_t M, int64_t K, int64_t N, int ranges) {
  SplitkPlan p;
  const int64_t nb = K / 256;
  p.n_rt = (N + SK_ROWS - 1) / SK_ROWS;
  p.n_tt = (M + SK_TOK - 1) / SK_TOK;
  const int64_t tiles = p.n_rt * p.n_tt;
  // the most ranges that keep the grid within one workgroup per CU (256):
  // a second, partial round of workgroups costs more than the ranges save
  // (measured on MI355X, graph-replayed calls, us/call at S = 1 / 2 / 3 / 4
  // / 6 / 8: 64x4096x4096 34.4 / 21.6 / 18.6 / 16.4 / 24.0 / 24.1,
  // 128x4096x4096 34.1 / 22.1 / 31.5 / 28.4 / 33.5 / 41.6, 64x4096->14336
  // 35.5 / 41.5 / 47.1 / 53.4 / 62.4 / 71.3, 16x14336->4096 109.3 / 58.8 /
  // 43.1 / 33.9 / 27.5 / 23.7)
  int64_t S = ranges;
  if (S <= 0) S = tiles < 256 ? 256 / tiles : 1;
  const int64_t smax = nb / 2 < 1 ? 1 : nb / 2;  // at least one super-block per half
  if (S > smax) S = smax;
  if (S > kSplitkMaxRanges) S = kSplitkMaxRanges;
  if (tiles >= 256) S = 1;  // the counters' region holds 4 per tile for 256 tiles
  p.S = (int)S;
  // S > 1 only below 256 tiles, so the counters fit their fixed region
  p.counter_bytes = S > 1 ? kSplitkCounterBytes : 0;
  p.workspace_bytes = S > 1 ? p.counter_bytes + tiles * S * SK_TILE * 4 : 0;
  static_assert(kSplitkCounterBytes + 255 * kSplitkMaxRanges * SK_TILE * 4 <= kSplitkWorkspaceBytes,
                "the library's workspace holds every plan");
  static_assert(255 * (SK_WAVES / 2) * 4 <= kSplitkCounterBytes, "one counter per (tile, wave)");
  return p;
}

bool splitk_fits(int64_t M, int64_t K, int64_t N) {
  const int64_t nb = K / 256;
  // offsets formed in the kernel (128 rows of weights, 32 rows of X) stay
  // below 2^31 bytes
  return (int64_t)SK_ROWS * nb * kBlockBytes < ((int64_t)1 << 31) &&
         (int64_t)SK_TOK * K * 4 < ((int64_t)1 << 31) && N <= 0x7FFFFFFF && M <= 0x7FFFFFFF;
}

hipError_t prefill_splitk_launch(const float *X, const uint8_t *w, int64_t M, int64_t K,
                                 int64_t N, float *Y, void *workspace, int64_t workspace_bytes,
                                 hipStream_t stream, int ranges) {
  if (!splitk_fits(M, K, N)) return hipErrorInvalidValue;
  const SplitkPlan p = splitk_plan(M, K, N, ranges);
  if (p.workspace_bytes > workspace_bytes || (p.S > 1 && workspace == nullptr))
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)p.n_rt * p.n_tt * p.S;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  unsigned *cnt = static_cast<unsigned *>(workspace);
  float *part = p.S > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                                    p.counter_bytes)
                        : nullptr;
  hipLaunchKernelGGL(q4k_prefill_splitk_kernel, dim3((unsigned)grid), dim3(SK_THREADS), 0, stream,
                     X, w, Y, part, cnt, (int)M, (int)(K / 256), (int)N, p.S, (int)p.n_rt,
                     (int)p.n_tt);
  return hipGetLastError();
}

}  // namespace q4k
