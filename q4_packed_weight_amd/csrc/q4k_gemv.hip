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

// Per-lane work of one (row, slab) pair, by weight format.  `grp` is the
// 144-byte group (9 uint4 of the staged tile) holding this lane's slab; j
// (0..3) is the slab within the group; xl/xh are the slab's 64 activations
// (float4 k of xl is positions 4k..4k+3, of xh positions 32+4k..) and xsm
// their sums over positions 0..31 and 32..63.  Returns acc plus the slab's
// contribution to the row.
//
// Q4_K: the group is one super-block; the lane reads the header and the 32
// qs bytes 32j..32j+31 (positions l of sub-blocks 2j and 2j+1).
struct Q4K {
  __device__ __forceinline__ static float slab(const uint4 *grp, int j, uint32_t sh, bool jhi,
                                               const float4 (&xl)[8], const float4 (&xh)[8],
                                               float2 xsm, float acc) {
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
    const float tm = __builtin_fmaf(sc.m_lo, xsm.x, sc.m_hi * xsm.y);
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
  __device__ __forceinline__ static float slab(const uint4 *grp, int j, uint32_t, bool,
                                               const float4 (&xl)[8], const float4 (&xh)[8],
                                               float2 xsm, float acc) {
    const uint32_t *g32 = reinterpret_cast<const uint32_t *>(grp) + 9 * j;
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
    acc = __builtin_fmaf(d0 * 0x1p20f, t0, __builtin_fmaf(-8.0f * d0, xsm.x, acc));
    return __builtin_fmaf(d1 * 0x1p20f, t1, __builtin_fmaf(-8.0f * d1, xsm.y, acc));
  }
};

template <class F, int L, int R, int KW, int W>
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
  constexpr int CH_ROW = BPS * 9;           // 16-byte chunks of one row per step
  constexpr int TILE = ROWS_W * CH_ROW;     // chunks of a wave's weight tile
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
  const int iters = (steps + KW - 1) / KW;
  const int64_t row_bytes = (int64_t)nb * kBlockBytes;
  const int j = u & 3;
  const uint32_t sh = (uint32_t)(j & 1) * 16u;
  const bool jhi = j >= 2;
  const int ls = kw * L + u;  // this lane's slab within the staged range
  // Range-checked buffer views: activations, and this workgroup's rows of
  // the weight matrix (rows past N read as zeros, so no clamping).
  const int64_t wg_row0 = (int64_t)blockIdx.x * (RG * ROWS_W);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)nb * 1024);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + wg_row0 * row_bytes, (N - wg_row0) * row_bytes);
  const int wave_off = (int)((row0 - wg_row0) * row_bytes);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  for (int it = 0; it < iters; ++it) {
    // 1. Load phase.  Activations for staging first (coalesced, L2-resident,
    //    they return first), then this wave's weight tile as a coalesced
    //    stream: chunk q of the tile is row q / CH_ROW of the wave, chunk
    //    q % CH_ROW of this step's piece of that row.  Slabs past the end of
    //    x and rows past N read as zeros; blocks past the end of a row read
    //    the next row's bytes and are never consumed.
    const int slab_base = it * S;
    float4 xv[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int f = min(tid + kThreads * q, XF - 1);
      xv[q] = load_buf_f4(xr, 4 * (64 * (slab_base + (f >> 4)) + 4 * (f & 15)));
    }
    const int t = it * KW + kw;
    const int b0 = t * BPS;
    uint4 wv[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int q = 64 * m + lane;
      const int rt = q / CH_ROW;
      const int within = q - rt * CH_ROW;
      wv[m] = load_buf_stream16(wr, wave_off + rt * (int)row_bytes + b0 * kBlockBytes + 16 * within);
    }
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
      const float part = group_sum<8>(sum4(xv[q]));
      if (k == 0) xsum[sl].x = part;
      if (k == 8) xsum[sl].y = part;
    }
    __syncthreads();

    // 3. Compute.  Before row slot r, the tile chunks that carry its rows
    //    are written to this wave's LDS tile (waiting only for those loads),
    //    then each lane reads its slab's header and 32 qs bytes back.
    const int i = t * L + u;
    const bool active = t < steps && i < n_slabs;
    float4 xl[8], xh[8];
    float2 xsm = make_float2(0.f, 0.f);
    if (active) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xl[k] = xs4[k * SP + ls];
        xh[k] = xs4[(k + 8) * SP + ls];
      }
      xsm = xsum[ls];
    }
    const int bl = u >> 2;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int prev_last = r == 0 ? -1 : (r * G * CH_ROW - 1) / 64;
      const int last_m = ((r + 1) * G * CH_ROW - 1) / 64;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (m > prev_last && m <= last_m && 64 * m + lane < TILE) wt[wave][64 * m + lane] = wv[m];
      if (active)
        acc[r] = F::slab(&wt[wave][((r * G + g) * BPS + bl) * 9], j, sh, jhi, xl, xh, xsm, acc[r]);
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
  constexpr int CH_ROW = BPS * 9;
  constexpr int TILE = ROWS_W * CH_ROW;
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
  const int64_t row_bytes = (int64_t)nb * kBlockBytes;
  const int j = u & 3;
  const uint32_t sh = (uint32_t)(j & 1) * 16u;
  const bool jhi = j >= 2;
  const int64_t unit_rows = (int64_t)W * ROWS_W;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)nb * 1024);

  // Weight tile of a unit: chunk q of this wave's tile is row q / CH_ROW of
  // the wave, chunk q % CH_ROW of the row (the whole row: one step).
  auto load_tile = [&](int unit, uint4 (&wv)[NM]) {
    const int64_t r0 = (int64_t)unit * unit_rows;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + r0 * row_bytes, (N - r0) * row_bytes);
    const int wave_off = (int)(wave * ROWS_W * row_bytes);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int q = 64 * m + lane;
      const int rt = q / CH_ROW;
      const int within = q - rt * CH_ROW;
      wv[m] = load_buf_stream16(wr, wave_off + rt * (int)row_bytes + 16 * within);
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
    const float part = group_sum<8>(sum4(xv[q]));
    if (k == 0) xsum[sl].x = part;
    if (k == 8) xsum[sl].y = part;
  }
  __syncthreads();
  const bool active = u < n_slabs;
  float4 xl[8], xh[8];
  float2 xsm = make_float2(0.f, 0.f);
  if (active) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xl[k] = xs4[k * SP + u];
      xh[k] = xs4[(k + 8) * SP + u];
    }
    xsm = xsum[u];
  }
  const int bl = u >> 2;

  auto compute = [&](int cur, const uint4 (&wv)[NM]) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int prev_last = r == 0 ? -1 : (r * G * CH_ROW - 1) / 64;
      const int last_m = ((r + 1) * G * CH_ROW - 1) / 64;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (m > prev_last && m <= last_m && 64 * m + lane < TILE) wt[wave][64 * m + lane] = wv[m];
      acc[r] = 0.0f;
      if (active)
        acc[r] = F::slab(&wt[wave][((r * G + g) * BPS + bl) * 9], j, sh, jhi, xl, xh, xsm, acc[r]);
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

template <class F, int L, int R, int KW, int W>
hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, int nb,
                       int64_t N, hipStream_t stream) {
  constexpr int G = 64 / L;
  constexpr int64_t rows_per_wg = (int64_t)(W / KW) * G * R;
  const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
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
  hipLaunchKernelGGL((q4k_gemv_kernel<F, L, R, KW, W>), dim3((unsigned)grid),
                     dim3(64 * W), 0, stream, x, w, y, nb, N);
  return hipGetLastError();
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
                            int k_waves, int waves) {
  // Defaults measured on MI355X (graph-replayed calls over rotating
  // weights): 4-wave workgroups, 4 rows per lane while that still gives
  // every SIMD a wave, and a 2-way split of input_dim across the waves of a
  // workgroup once a row needs several steps; small problems fall back to
  // smaller workgroups so that every CU gets one.
  GemvShape s;
  const int64_t slabs = 4 * nb;
  s.lanes = slabs <= 16 ? 16 : (slabs <= 32 ? 32 : 64);
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
    case 16: return launch_r<F, 16>(s, x, w, y, nbi, N, stream);
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

}  // namespace q4k
