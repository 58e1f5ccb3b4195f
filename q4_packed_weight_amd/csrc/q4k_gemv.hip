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
// xl[0..3], high nibbles against xh[0..3].  The lo accumulators are in units
// of 2^-24, the hi ones in units of 2^-20 (the high nibble is used in place,
// times 16); bytes 0/2 and 1/3 feed separate accumulators so that four
// independent chains hide the FMA latency.
__device__ __forceinline__ void nibble_dots(uint32_t w, float4 xl, float4 xh,
                                            float (&lo)[2], float (&hi)[2]) {
  const uint32_t lo02 = w & 0x000F000Fu;
  const uint32_t hi02 = w & 0x00F000F0u;
  const uint32_t w8 = w >> 8;
  const uint32_t lo13 = w8 & 0x000F000Fu;
  const uint32_t hi13 = w8 & 0x00F000F0u;
  lo[0] = __builtin_fmaf(half_lo(lo02), xl.x, lo[0]);
  hi[0] = __builtin_fmaf(half_lo(hi02), xh.x, hi[0]);
  lo[1] = __builtin_fmaf(half_lo(lo13), xl.y, lo[1]);
  hi[1] = __builtin_fmaf(half_lo(hi13), xh.y, hi[1]);
  lo[0] = __builtin_fmaf(half_hi(lo02), xl.z, lo[0]);
  hi[0] = __builtin_fmaf(half_hi(hi02), xh.z, hi[0]);
  lo[1] = __builtin_fmaf(half_hi(lo13), xl.w, lo[1]);
  hi[1] = __builtin_fmaf(half_hi(hi13), xh.w, hi[1]);
}

// Per-format parts of the GEMV kernels.  Each format defines
//   kBlockBytes  bytes of one block (a Q4_K super-block, eight Q4_0 blocks,
//                one Q6_K block); four lanes share a block, one 64-position
//                slab each;
//   kUnaligned   whether a row can start off a 16-byte boundary (then the
//                tile holds each row piece from its aligned-down start, with
//                one more chunk, and the lane adds the row's offset);
//   load_x       the lane's 64 activations from the staged slabs, as two
//                float4[8] (xl, xh), and the sums the format's offset term
//                needs (xs);
//   slab         acc plus the lane's slab contribution to a row, reading the
//                block that starts `boff` bytes into the wave's LDS tile.
// Staged layout: float4 k (positions 4k..4k+3) of staged slab ls is
// xs4[k*SP + ls]; xsum[ls] holds the sums over positions 0..31 and 32..63.

// The lane's staged slab as positions 0..31 (xl) and 32..63 (xh) with their
// two 32-position sums (Q4_K sub-blocks 2j and 2j+1, Q4_0 blocks 2j and
// 2j+1).
__device__ __forceinline__ void load_x_slab(const float4 *xs4, int SP, int ls,
                                            const float2 *xsum, float4 (&xl)[8],
                                            float4 (&xh)[8], float4 &xs) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    xl[k] = xs4[k * SP + ls];
    xh[k] = xs4[(k + 8) * SP + ls];
  }
  const float2 t = xsum[ls];
  xs = make_float4(t.x, t.y, 0.f, 0.f);
}

// Q4_K: the block is one super-block; the lane reads the header and the 32
// qs bytes 32j..32j+31 (positions l of sub-blocks 2j and 2j+1).
struct Q4K {
  static constexpr int kBlockBytes = 144;
  static constexpr bool kUnaligned = false;
  __device__ __forceinline__ static void load_x(const float4 *xs4, int SP, int ls, int,
                                                const float2 *xsum, float4 (&xl)[8],
                                                float4 (&xh)[8], float4 &xs) {
    load_x_slab(xs4, SP, ls, xsum, xl, xh, xs);
  }
  __device__ __forceinline__ static float slab(const uint4 *tile, int boff, int j, uint32_t sh,
                                               bool jhi, const float4 (&xl)[8],
                                               const float4 (&xh)[8], float4 xs, float acc) {
    const uint4 *grp = tile + (boff >> 4);
    const uint4 hdr = grp[0];
    const uint4 q0 = grp[1 + 2 * j];
    const uint4 q1 = grp[2 + 2 * j];
    float lo[2] = {0.f, 0.f}, hi[2] = {0.f, 0.f};
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) nibble_dots(qw[k], xl[k], xh[k], lo, hi);
    const float s_lo = lo[0] + lo[1], s_hi = hi[0] + hi[1];
    const SlabScales sc = decode_header(hdr, sh, jhi);
    // code part in units of 2^-20: 16*sc_lo*s_lo + sc_hi*s_hi
    const float tc = __builtin_fmaf(sc.sc_lo16, s_lo, sc.sc_hi * s_hi);
    const float tm = __builtin_fmaf(sc.m_lo, xs.x, sc.m_hi * xs.y);
    // this slab's contribution: d * 2^20 * tc - dmin * tm
    return __builtin_fmaf(sc.d * 0x1p20f, tc, __builtin_fmaf(-sc.dmin, tm, acc));
  }
};

// Q4_0 (the Q4_K page's follow-up format, section "Out of scope": 32
// weights in 18 bytes; fp16 d, then 16 qs bytes whose low nibbles are
// elements 0..15 and high nibbles elements 16..31, weight d*(q - 8)).
// Eight blocks make one 144-byte group, so a slab of 64 positions is the
// two blocks 2j, 2j+1 at bytes 36j..36j+35: nine dwords.  The first block's
// qs start 2 bytes into its first dword and are realigned; the second's
// are dword-aligned.  Each block contributes d*(sum q*x - 8*sum x).
struct Q40 {
  static constexpr int kBlockBytes = 144;
  static constexpr bool kUnaligned = false;
  __device__ __forceinline__ static void load_x(const float4 *xs4, int SP, int ls, int,
                                                const float2 *xsum, float4 (&xl)[8],
                                                float4 (&xh)[8], float4 &xs) {
    load_x_slab(xs4, SP, ls, xsum, xl, xh, xs);
  }
  __device__ __forceinline__ static float slab(const uint4 *tile, int boff, int j, uint32_t, bool,
                                               const float4 (&xl)[8], const float4 (&xh)[8],
                                               float4 xs, float acc) {
    const uint32_t *g32 = reinterpret_cast<const uint32_t *>(tile + (boff >> 4)) + 9 * j;
    uint32_t dw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) dw[i] = g32[i];
    float lo0[2] = {0.f, 0.f}, hi0[2] = {0.f, 0.f}, lo1[2] = {0.f, 0.f}, hi1[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // block 2j: qs bytes 4t..4t+3 sit at bytes 2+4t.. of the slab
      nibble_dots(__builtin_amdgcn_alignbyte(dw[t + 1], dw[t], 2), xl[t], xl[4 + t], lo0, hi0);
      // block 2j+1: qs bytes 4t.. are dword 5+t
      nibble_dots(dw[5 + t], xh[t], xh[4 + t], lo1, hi1);
    }
    const float d0 = half_lo(dw[0]), d1 = half_hi(dw[4]);
    // sum q*x in units of 2^-20: 16*(low-nibble sums) + (high-nibble sums)
    const float t0 = __builtin_fmaf(16.0f, lo0[0] + lo0[1], hi0[0] + hi0[1]);
    const float t1 = __builtin_fmaf(16.0f, lo1[0] + lo1[1], hi1[0] + hi1[1]);
    acc = __builtin_fmaf(d0 * 0x1p20f, t0, __builtin_fmaf(-8.0f * d0, xs.x, acc));
    return __builtin_fmaf(d1 * 0x1p20f, t1, __builtin_fmaf(-8.0f * d1, xs.y, acc));
  }
};

// Q6_K (the Q4_K page's other follow-up format, section "Out of scope": ql
// holds each code's low 4 bits, qh its high 2 bits, four codes per qh byte,
// in two interleaved halves).  Read as ggml's block_q6_K, 210 bytes: ql[128],
// qh[64], 16 int8 scales, fp16 d.  Element 128n + 32c + l (half n, quadrant
// c) has the low (c < 2) or high (c >= 2) nibble of ql[64n + 32(c&1) + l],
// bits 2c..2c+1 of qh[32n + l] on top, and scale 8n + 2c + l/16; weight
// d*scale*(q - 32).  Lane j of a block takes half n = j/2 and quadrants
// p = j%2 and p + 2: the same 32 ql bytes (low and high nibbles) and the
// same 32 qh bytes, four 16-position scale groups.  Blocks start on even
// bytes only, so every field is read as dwords from its aligned-down start
// and shifted back by the block's offset (0 or 2 bytes).
struct Q6K {
  static constexpr int kBlockBytes = 210;
  static constexpr bool kUnaligned = true;
  // positions 32p..32p+31 of staged slabs 4b + 2n (xl: quadrant p) and
  // 4b + 2n + 1 (xh: quadrant p + 2), and their four 16-position sums
  __device__ __forceinline__ static void load_x(const float4 *xs4, int SP, int ls, int j,
                                                const float2 *, float4 (&xl)[8],
                                                float4 (&xh)[8], float4 &xs) {
    const int p = j & 1;
    const int a = ls - p;  // slab 4b + 2n of this lane's block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xl[i] = xs4[(8 * p + i) * SP + a];
      xh[i] = xs4[(8 * p + i) * SP + a + 1];
    }
    xs.x = (sum4(xl[0]) + sum4(xl[1])) + (sum4(xl[2]) + sum4(xl[3]));
    xs.y = (sum4(xl[4]) + sum4(xl[5])) + (sum4(xl[6]) + sum4(xl[7]));
    xs.z = (sum4(xh[0]) + sum4(xh[1])) + (sum4(xh[2]) + sum4(xh[3]));
    xs.w = (sum4(xh[4]) + sum4(xh[5])) + (sum4(xh[6]) + sum4(xh[7]));
  }
  __device__ __forceinline__ static float slab(const uint4 *tile, int boff, int j, uint32_t, bool,
                                               const float4 (&xl)[8], const float4 (&xh)[8],
                                               float4 xs, float acc) {
    const uint32_t *t32 = reinterpret_cast<const uint32_t *>(tile);
    const int n = j >> 1, p = j & 1;
    const uint32_t sb = (uint32_t)boff & 3u;  // 0 or 2: the block's byte offset in a dword
    const int oq = (boff + 64 * n + 32 * p) >> 2;
    const int oh = (boff + 128 + 32 * n) >> 2;
    const int os = (boff + 192 + 8 * n) >> 2;
    const int od = (boff + 208) >> 2;
    uint32_t q[9], h[9], sd[3];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      q[i] = t32[oq + i];
      h[i] = t32[oh + i];
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) sd[i] = t32[os + i];
    const float d = half_lo(t32[od] >> (8u * sb));
    // the four scales: bytes 2p, 2p+1 (quadrant p) and 2p+4, 2p+5 (p + 2)
    const uint32_t s0 = __builtin_amdgcn_alignbyte(sd[1], sd[0], sb);
    const uint32_t s1 = __builtin_amdgcn_alignbyte(sd[2], sd[1], sb);
    // sign-extended bytes (the builtin's result type is unsigned: convert
    // through int32_t)
    const uint32_t sp = 16u * (uint32_t)p;
    const float ds0 = d * (float)(int32_t)__builtin_amdgcn_sbfe(s0, sp, 8);
    const float ds1 = d * (float)(int32_t)__builtin_amdgcn_sbfe(s0, sp + 8, 8);
    const float ds2 = d * (float)(int32_t)__builtin_amdgcn_sbfe(s1, sp, 8);
    const float ds3 = d * (float)(int32_t)__builtin_amdgcn_sbfe(s1, sp + 8, 8);
    // code sums in units of 2^-24 (6-bit codes enter as fp16 subnormals):
    // [quadrant p | p + 2][positions 0..15 | 16..31][two chains]
    float c[2][2][2] = {};
    const uint32_t hs = 2u * (uint32_t)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ql = __builtin_amdgcn_alignbyte(q[i + 1], q[i], sb);
      const uint32_t hq = __builtin_amdgcn_alignbyte(h[i + 1], h[i], sb) >> hs;
      // four 6-bit codes per dword, one per byte
      const uint32_t clo = (ql & 0x0F0F0F0Fu) | ((hq << 4) & 0x30303030u);
      const uint32_t chi = ((ql >> 4) & 0x0F0F0F0Fu) | (hq & 0x30303030u);
      const int hf = i >> 2;
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const uint32_t cw = qd ? chi : clo;
        const float4 xv = qd ? xh[i] : xl[i];
        const uint32_t a02 = cw & 0x003F003Fu, a13 = (cw >> 8) & 0x003F003Fu;
        c[qd][hf][0] = __builtin_fmaf(half_lo(a02), xv.x, c[qd][hf][0]);
        c[qd][hf][1] = __builtin_fmaf(half_lo(a13), xv.y, c[qd][hf][1]);
        c[qd][hf][0] = __builtin_fmaf(half_hi(a02), xv.z, c[qd][hf][0]);
        c[qd][hf][1] = __builtin_fmaf(half_hi(a13), xv.w, c[qd][hf][1]);
      }
    }
    // each 16-position group adds d*scale*(2^24 * codes.x - 32 * sum x)
    acc = __builtin_fmaf(ds0 * 0x1p24f, c[0][0][0] + c[0][0][1], __builtin_fmaf(-32.0f * ds0, xs.x, acc));
    acc = __builtin_fmaf(ds1 * 0x1p24f, c[0][1][0] + c[0][1][1], __builtin_fmaf(-32.0f * ds1, xs.y, acc));
    acc = __builtin_fmaf(ds2 * 0x1p24f, c[1][0][0] + c[1][0][1], __builtin_fmaf(-32.0f * ds2, xs.z, acc));
    return __builtin_fmaf(ds3 * 0x1p24f, c[1][1][0] + c[1][1][1], __builtin_fmaf(-32.0f * ds3, xs.w, acc));
  }
};

// ONE: every wave's part of input_dim fits one iteration (4 nb <= L KW).
// Its loads then leave before the rest of the set-up, with no loop around
// them (a load phase peeled off a general loop keeps its registers live
// through the body and costs occupancy at large grids).
template <class F, int L, int R, int KW, int W, bool ONE>
__global__ __launch_bounds__(64 * W) void q4k_gemv_kernel(
    const float *x, const uint8_t *w, float *__restrict__ y, int nb,
    int64_t N) {
  // x and w are deliberately not __restrict__: that keeps their loads
  // ordered before the compiler fence that closes each load phase.
  constexpr int kThreads = 64 * W;          // W waves per workgroup
  constexpr int G = 64 / L;                 // rows side by side in one wave instruction
  constexpr int RG = W / KW;                // row groups (of KW waves) per workgroup
  constexpr int ROWS_W = G * R;             // rows per wave
  constexpr int BPS = L / 4;                // blocks of one row covered by one step
  static_assert(BPS * F::kBlockBytes % 16 == 0, "a row piece must be whole 16-byte chunks");
  constexpr int CH_ROW = BPS * F::kBlockBytes / 16;   // 16-byte chunks of one row per step
  constexpr int CH_ROWP = CH_ROW + (F::kUnaligned ? 1 : 0);  // tile chunks per row piece
  constexpr int TILE = ROWS_W * CH_ROWP;    // chunks of a wave's weight tile
  constexpr int NM = (TILE + 63) / 64;      // load instructions per tile
  constexpr int S = KW * L;                 // slabs whose activations are staged together
  constexpr int SP = S + 1;                 // padded row of the staged layout (float4)
  constexpr int XF = 16 * S;                // staged float4 per iteration
  constexpr int XQ = (XF + kThreads - 1) / kThreads;  // staged float4 per thread
  static_assert(XF % 64 == 0, "staging guard must be wave-uniform");

  // Staged activations: float4 k of slab ls at slot k*SP + ls.  A wave
  // reading float4 k of consecutive slabs touches consecutive slots, and the
  // one-slot pad per k-row spreads the staging writes (16 k of one slab per
  // 16 lanes) over distinct banks.  Then the two sub-block sums of each
  // staged slab, and one weight tile per wave.
  __shared__ float4 xs4[16 * SP];
  __shared__ float2 xsum[S];
  __shared__ uint4 wt[W][TILE];
  __shared__ float partial[KW > 1 ? W * ROWS_W : 1];

  // The host validates nb >= 1; saying so lets the compiler fetch every
  // kernel argument in one round trip instead of two (the loop-entry test
  // would otherwise sit between them).
  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = wave % KW;
  const int rg = wave / KW;
  const int g = lane / L;
  const int u = lane % L;
  const int64_t row0 = (int64_t)blockIdx.x * (RG * ROWS_W) + (int64_t)rg * ROWS_W;
  const int n_slabs = 4 * nb;
  const int steps = (n_slabs + L - 1) / L;
  const int iters = ONE ? 1 : (steps + KW - 1) / KW;
  const int64_t row_bytes = (int64_t)nb * F::kBlockBytes;
  const int j = u & 3;
  const uint32_t sh = (uint32_t)(j & 1) * 16u;
  const bool jhi = j >= 2;
  const int ls = kw * L + u;  // this lane's slab within the staged range
  // Range-checked buffer views: activations, and this workgroup's rows of
  // the weight matrix (rows past N read as zeros, so no clamping).
  // Rows of an unaligned format are read from the workgroup's first byte
  // rounded down to 16 (w itself is 16-byte aligned); wave_off is the
  // wave's first row relative to that base.  The view ends at the matrix's
  // end rounded up to a dword: the range check zeroes every dword that
  // crosses the view's end, and the last bytes of a Q6_K matrix can share
  // a dword with up to two bytes past it (never a page of their own).
  const int64_t wg_row0 = (int64_t)blockIdx.x * (RG * ROWS_W);
  const int64_t wg_byte0 = wg_row0 * row_bytes;
  const int64_t wg_base = F::kUnaligned ? (wg_byte0 & ~(int64_t)15) : wg_byte0;
  // The view covers this workgroup's rows (fewer at the end of the matrix)
  // to their last byte rounded up to a dword; the launcher keeps that below
  // 2^31 bytes, so the size needs no 64-bit clamp ahead of the first load.
  const int64_t rows_here = N - wg_row0 < RG * ROWS_W ? N - wg_row0 : RG * ROWS_W;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc32(x, (uint32_t)nb * 1024u);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc32(
      w + wg_base, (uint32_t)(((wg_byte0 + rows_here * row_bytes + 3) & ~(int64_t)3) - wg_base));
  const int wave_off = (int)(wg_byte0 - wg_base + (row0 - wg_row0) * row_bytes);

  // 1. Load phase of iteration it.  Activations for staging first
  //    (coalesced, L2-resident, they return first), then this wave's weight
  //    tile as a coalesced stream: chunk q of the tile is row q / CH_ROWP of
  //    the wave, chunk q % CH_ROWP of this step's piece of that row (from
  //    the piece's first byte rounded down to 16).  Slabs past the end of x
  //    and rows past N read as zeros; blocks past the end of a row read the
  //    next row's bytes and are never consumed.
  float4 xv[XQ];
  uint4 wv[NM];
  auto load_phase = [&](int it) {
    const int slab_base = it * S;
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int f = min(tid + kThreads * q, XF - 1);
      xv[q] = load_buf_f4(xr, 4 * (64 * (slab_base + (f >> 4)) + 4 * (f & 15)));
    }
    const int b0 = (it * KW + kw) * BPS;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int q = 64 * m + lane;
      const int rt = q / CH_ROWP;
      const int within = q - rt * CH_ROWP;
      const int start = wave_off + rt * (int)row_bytes + b0 * F::kBlockBytes;
      wv[m] = load_buf_stream16(wr, (start & ~15) + 16 * within);
    }
  };
  if constexpr (ONE) {
    load_phase(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  for (int it = 0; it < iters; ++it) {
    if constexpr (!ONE) load_phase(it);
    const int t = it * KW + kw;
    const int b0 = t * BPS;
    // Keep the LDS stores below from being hoisted above the load phase.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. Stage the activations and their sub-block sums (the 8 float4 of a
    //    sub-block sit in 8 aligned lanes); only the activation loads are
    //    waited for, the weight stream keeps flowing.
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int f = tid + kThreads * q;
      if (XF % kThreads != 0 && f >= XF) break;  // wave-uniform
      const int sl = f >> 4, k = f & 15;
      xs4[k * SP + sl] = xv[q];
      if constexpr (!F::kUnaligned) {  // Q6_K sums its own 16-position groups
        const float part = group_sum<8>(sum4(xv[q]));
        if (k == 0) xsum[sl].x = part;
        if (k == 8) xsum[sl].y = part;
      }
    }
    __syncthreads();

    // 3. Compute.  Before row slot r, the tile chunks that carry its rows
    //    are written to this wave's LDS tile (waiting only for those loads),
    //    then each lane reads its slab's header and 32 qs bytes back.
    const int i = t * L + u;
    const bool active = t < steps && i < n_slabs;
    float4 xl[8], xh[8];
    float4 xs = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) F::load_x(xs4, SP, ls, j, xsum, xl, xh, xs);
    const int bl = u >> 2;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int prev_last = r == 0 ? -1 : (r * G * CH_ROWP - 1) / 64;
      const int last_m = ((r + 1) * G * CH_ROWP - 1) / 64;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (m > prev_last && m <= last_m && 64 * m + lane < TILE) wt[wave][64 * m + lane] = wv[m];
      if (active) {
        const int rr = r * G + g;  // row of the wave
        int boff = rr * CH_ROWP * 16 + bl * F::kBlockBytes;
        if constexpr (F::kUnaligned)
          boff += (wave_off + rr * (int)row_bytes + b0 * F::kBlockBytes) & 15;
        acc[r] = F::slab(wt[wave], boff, j, sh, jhi, xl, xh, xs, acc[r]);
      }
    }
    // every wave must be done with the staged activations before the next
    // iteration overwrites them (the weight tile is private to the wave)
    if (it + 1 < iters) __syncthreads();
  }

  // Reduce each row over the L lanes of its group.
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = group_sum<L>(acc[r]);

  if constexpr (KW == 1) {
    if (u == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + (int64_t)r * G + g;
        if (row < N) y[row] = acc[r];
      }
    }
  } else {
    // partial[wave][row_in_wave], summed over the KW waves in wave order
    if (u == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) partial[wave * ROWS_W + r * G + g] = acc[r];
    }
    __syncthreads();
    if (kw == 0 && lane < ROWS_W) {
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < KW; ++k) v += partial[(wave + k) * ROWS_W + lane];
      const int64_t row = row0 + lane;
      if (row < N) y[row] = v;
    }
  }
}

// Persistent form for rows that fit in one step (4*nb <= L slabs) and
// more row groups than stay resident: a workgroup stages the activations
// once, then walks units u = blockIdx.x, blockIdx.x + gridDim.x, ... (a unit
// is the W*R*G rows one launch of the kernel above would give a
// workgroup), loading the weight tile of the next unit while it computes
// the current one.  Arithmetic and summation order per row are those of
// q4k_gemv_kernel with KW = 1, so results are identical.
template <class F, int L, int R, int W>
__global__ __launch_bounds__(64 * W) void q4k_gemv_persist_kernel(
    const float *x, const uint8_t *w, float *__restrict__ y, int nb,
    int64_t N, int n_units) {
  constexpr int kThreads = 64 * W;
  constexpr int G = 64 / L;
  constexpr int ROWS_W = G * R;
  constexpr int BPS = L / 4;
  static_assert(BPS * F::kBlockBytes % 16 == 0, "a row piece must be whole 16-byte chunks");
  constexpr int CH_ROW = BPS * F::kBlockBytes / 16;
  constexpr int CH_ROWP = CH_ROW + (F::kUnaligned ? 1 : 0);
  constexpr int TILE = ROWS_W * CH_ROWP;
  constexpr int NM = (TILE + 63) / 64;
  constexpr int S = L;
  constexpr int SP = S + 1;
  constexpr int XF = 16 * S;
  constexpr int XQ = (XF + kThreads - 1) / kThreads;
  static_assert(XF % 64 == 0, "staging guard must be wave-uniform");
  __shared__ float4 xs4[16 * SP];
  __shared__ float2 xsum[S];
  __shared__ uint4 wt[W][TILE];

  __builtin_assume(nb >= 1);
  __builtin_assume(n_units >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane / L;
  const int u = lane % L;
  const int n_slabs = 4 * nb;
  const int64_t row_bytes = (int64_t)nb * F::kBlockBytes;
  const int j = u & 3;
  const uint32_t sh = (uint32_t)(j & 1) * 16u;
  const bool jhi = j >= 2;
  const int64_t unit_rows = (int64_t)W * ROWS_W;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)nb * 1024);

  // Weight tile of a unit: chunk q of this wave's tile is row q / CH_ROWP
  // of the wave, chunk q % CH_ROWP of the row (the whole row: one step),
  // counted from the row's first byte rounded down to 16.  wave_off(unit)
  // is the wave's first row relative to the unit's base.
  auto unit_base = [&](int unit) {
    const int64_t b = (int64_t)unit * unit_rows * row_bytes;
    return F::kUnaligned ? (b & ~(int64_t)15) : b;
  };
  auto wave_off = [&](int unit) {
    const int64_t b = (int64_t)unit * unit_rows * row_bytes;
    return (int)(b - unit_base(unit) + wave * ROWS_W * row_bytes);
  };
  auto load_tile = [&](int unit, uint4 (&wv)[NM]) {
    const int64_t base = unit_base(unit);
    // ends at the matrix's end rounded up to a dword (see q4k_gemv_kernel)
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + base, ((N * row_bytes + 3) & ~(int64_t)3) - base);
    const int woff = wave_off(unit);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int q = 64 * m + lane;
      const int rt = q / CH_ROWP;
      const int within = q - rt * CH_ROWP;
      const int start = woff + rt * (int)row_bytes;
      wv[m] = load_buf_stream16(wr, (start & ~15) + 16 * within);
    }
  };

  // Activations (all slabs) and the first unit's tile.
  float4 xv[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int f = min(tid + kThreads * q, XF - 1);
    xv[q] = load_buf_f4(xr, 4 * (64 * (f >> 4) + 4 * (f & 15)));
  }
  uint4 wa[NM], wb[NM];
  int unit = blockIdx.x;
  load_tile(unit, wa);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int f = tid + kThreads * q;
    if (XF % kThreads != 0 && f >= XF) break;  // wave-uniform
    const int sl = f >> 4, k = f & 15;
    xs4[k * SP + sl] = xv[q];
    if constexpr (!F::kUnaligned) {
      const float part = group_sum<8>(sum4(xv[q]));
      if (k == 0) xsum[sl].x = part;
      if (k == 8) xsum[sl].y = part;
    }
  }
  __syncthreads();
  const bool active = u < n_slabs;
  float4 xl[8], xh[8];
  float4 xs = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active) F::load_x(xs4, SP, u, j, xsum, xl, xh, xs);
  const int bl = u >> 2;

  auto compute = [&](int cur, const uint4 (&wv)[NM]) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int prev_last = r == 0 ? -1 : (r * G * CH_ROWP - 1) / 64;
      const int last_m = ((r + 1) * G * CH_ROWP - 1) / 64;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (m > prev_last && m <= last_m && 64 * m + lane < TILE) wt[wave][64 * m + lane] = wv[m];
      acc[r] = 0.0f;
      if (active) {
        const int rr = r * G + g;
        int boff = rr * CH_ROWP * 16 + bl * F::kBlockBytes;
        if constexpr (F::kUnaligned) boff += (wave_off(cur) + rr * (int)row_bytes) & 15;
        acc[r] = F::slab(wt[wave], boff, j, sh, jhi, xl, xh, xs, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum<L>(acc[r]);
    if (u == 0) {
      const int64_t row0 = (int64_t)cur * unit_rows + (int64_t)wave * ROWS_W;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + (int64_t)r * G + g;
        if (row < N) y[row] = acc[r];
      }
    }
  };

  // Ping-pong over the two tile registers: the next unit's loads are in
  // flight while the current unit is computed.
  for (;;) {
    const int nxt = unit + (int)gridDim.x;
    if (nxt < n_units) load_tile(nxt, wb);
    compute(unit, wa);
    if (nxt >= n_units) break;
    unit = nxt;
    const int nxt2 = unit + (int)gridDim.x;
    if (nxt2 < n_units) load_tile(nxt2, wa);
    compute(unit, wb);
    if (nxt2 >= n_units) break;
    unit = nxt2;
  }
}

// Workgroups of the persistent form that stay resident on the 256 CUs (two
// per CU, the LDS limit of the 4-wave form).
constexpr int64_t kPersistSlots = 512;

// Static LDS of q4k_gemv_kernel<F, L, R, KW, W> (staged activations and
// sums, the waves' tiles, the cross-wave partials).
template <class F, int L, int R, int KW, int W>
constexpr int gemv_lds_bytes() {
  constexpr int rows_w = (64 / L) * R;
  constexpr int ch_rowp = L / 4 * F::kBlockBytes / 16 + (F::kUnaligned ? 1 : 0);
  return 16 * 16 * (KW * L + 1) + 8 * KW * L + 16 * W * rows_w * ch_rowp +
         4 * (KW > 1 ? W * rows_w : 1);
}
constexpr int kMaxLds = 160 * 1024;

template <class F, int L, int R, int KW, int W>
hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, int nb,
                       int64_t N, hipStream_t stream) {
  if constexpr (gemv_lds_bytes<F, L, R, KW, W>() > kMaxLds) {
    return hipErrorInvalidConfiguration;  // the callers reject these shapes first
  } else {
  constexpr int G = 64 / L;
  constexpr int64_t rows_per_wg = (int64_t)(W / KW) * G * R;
  const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // a workgroup's rows (its buffer view, plus alignment) stay below 2^31
  // bytes; every shape the library picks for input_dim <= 2^24 does
  if (rows_per_wg * nb * F::kBlockBytes + 32 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if constexpr (KW == 1 && W == 4) {
    // One step per row and more units than resident slots: walk the units
    // with as few workgroups as give every workgroup the same unit count.
    if (4 * (int64_t)nb <= L && grid > kPersistSlots) {
      const int64_t per = (grid + kPersistSlots - 1) / kPersistSlots;
      const int64_t pgrid = (grid + per - 1) / per;
      hipLaunchKernelGGL((q4k_gemv_persist_kernel<F, L, R, W>), dim3((unsigned)pgrid),
                         dim3(64 * W), 0, stream, x, w, y, nb, N, (int)grid);
      return hipGetLastError();
    }
  }
  if (4 * (int64_t)nb <= L * KW) {
    hipLaunchKernelGGL((q4k_gemv_kernel<F, L, R, KW, W, true>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, w, y, nb, N);
  } else if constexpr (L == 64) {
    hipLaunchKernelGGL((q4k_gemv_kernel<F, L, R, KW, W, false>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, w, y, nb, N);
  } else {
    // 16 or 32 lanes are only chosen for rows of one step (4 nb <= L)
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
  }
}

template <class F, int L, int R>
hipError_t launch_w(int waves, int kw, const float *x, const uint8_t *w,
                    float *y, int nb, int64_t N, hipStream_t s) {
  if (waves == 8) {
    if constexpr (R <= 4) {  // 8 waves x 8 rows would exceed the 160 KB of LDS
      if (kw == 1) return launch_gemv<F, L, R, 1, 8>(x, w, y, nb, N, s);
      return launch_gemv<F, L, R, 2, 8>(x, w, y, nb, N, s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (waves == 1) return launch_gemv<F, L, R, 1, 1>(x, w, y, nb, N, s);
  if (waves == 2) {
    if (kw == 1) return launch_gemv<F, L, R, 1, 2>(x, w, y, nb, N, s);
    return launch_gemv<F, L, R, 2, 2>(x, w, y, nb, N, s);
  }
  if (kw == 1) return launch_gemv<F, L, R, 1, 4>(x, w, y, nb, N, s);
  if (kw == 2) return launch_gemv<F, L, R, 2, 4>(x, w, y, nb, N, s);
  return launch_gemv<F, L, R, 4, 4>(x, w, y, nb, N, s);
}

template <class F, int L>
hipError_t launch_r(const GemvShape &sh, const float *x, const uint8_t *w,
                    float *y, int nb, int64_t N, hipStream_t s) {
  switch (sh.rows_per_lane) {
    case 1: return launch_w<F, L, 1>(sh.waves, sh.k_waves, x, w, y, nb, N, s);
    case 2: return launch_w<F, L, 2>(sh.waves, sh.k_waves, x, w, y, nb, N, s);
    case 4: return launch_w<F, L, 4>(sh.waves, sh.k_waves, x, w, y, nb, N, s);
    default: return launch_w<F, L, 8>(sh.waves, sh.k_waves, x, w, y, nb, N, s);
  }
}

}  // namespace

GemvShape choose_gemv_shape(int64_t nb, int64_t N, int rows_per_lane,
                            int k_waves, int waves, int min_lanes) {
  // Defaults measured on MI355X (graph-replayed calls over rotating
  // weights): 4-wave workgroups, 4 rows per lane while that still gives
  // every SIMD a wave, and a 2-way split of input_dim across the waves of a
  // workgroup once a row needs several steps; small problems fall back to
  // smaller workgroups so that every CU gets one.
  GemvShape s;
  const int64_t slabs = 4 * nb;
  s.lanes = slabs <= 16 ? 16 : (slabs <= 32 ? 32 : 64);
  if (s.lanes < min_lanes) s.lanes = min_lanes;
  const int64_t steps = (slabs + s.lanes - 1) / s.lanes;
  const int64_t g = 64 / s.lanes;
  s.k_waves = k_waves > 0 ? k_waves : (steps >= 2 ? 2 : 1);
  if (rows_per_lane > 0) {
    s.rows_per_lane = rows_per_lane;
  } else {
    const int64_t target_waves = 1024;
    int r = 4;
    while (r > 1 && (N + g * r - 1) / (g * r) * s.k_waves < target_waves) r /= 2;
    // Where the persistent walk runs (one step per row, more than 512
    // workgroups of 4 waves x 4 rows), 2 rows per lane balances the walk
    // better: measured 0.4-2.1 us faster at input_dim 3072-4096 and
    // output_dim 11008-28672, slower at input_dim 2048.
    if (r == 4 && s.k_waves == 1 && s.lanes == 64 && nb >= 12 && N > 512 * 16) r = 2;
    s.rows_per_lane = r;
  }
  if (waves > 0) {
    s.waves = waves;
  } else {
    s.waves = 4;
    while (s.waves > s.k_waves &&
           (N + (s.waves / s.k_waves) * g * s.rows_per_lane - 1) /
                   ((s.waves / s.k_waves) * g * s.rows_per_lane) < 256)
      s.waves /= 2;
  }
  if (s.k_waves > s.waves) s.k_waves = s.waves;
  return s;
}

template <class F>
hipError_t gemv_launch_fmt(const float *x, const uint8_t *w, float *y, int64_t nb,
                           int64_t N, const GemvShape &s, hipStream_t stream) {
  const int nbi = (int)nb;
  switch (s.lanes) {
    case 16:
      // 16 lanes cover 4 blocks per step: whole 16-byte chunks for 144-byte
      // blocks only
      if constexpr (4 * F::kBlockBytes % 16 == 0) return launch_r<F, 16>(s, x, w, y, nbi, N, stream);
      else return hipErrorInvalidValue;
    case 32: return launch_r<F, 32>(s, x, w, y, nbi, N, stream);
    default: return launch_r<F, 64>(s, x, w, y, nbi, N, stream);
  }
}

hipError_t gemv_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                       int64_t N, const GemvShape &s, hipStream_t stream) {
  return gemv_launch_fmt<Q4K>(x, w, y, nb, N, s, stream);
}

hipError_t gemv_q4_0_launch(const float *x, const uint8_t *w, float *y, int64_t ngroups,
                            int64_t N, const GemvShape &s, hipStream_t stream) {
  return gemv_launch_fmt<Q40>(x, w, y, ngroups, N, s, stream);
}

hipError_t gemv_q6k_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                           int64_t N, const GemvShape &s, hipStream_t stream) {
  return gemv_launch_fmt<Q6K>(x, w, y, nb, N, s, stream);
}

}  // namespace q4k
