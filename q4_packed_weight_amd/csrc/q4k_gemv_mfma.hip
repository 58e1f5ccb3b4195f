// q4k_gemv_mfma.hip -- Q4_K matrix-vector product with the multiplies on the
// gfx950 matrix cores.
//
// What it computes is q4k_gemv's product (Q4_K page: SKaiNET PR #562,
// "feat(kernel): SIMD-fused Q4_K matmul kernel + Q4KMatmulKernel SPI",
// sections "Summary" and "Pipeline"): y[o] = sum over super-blocks and
// sub-blocks of d*sc*sum_l q*x - dmin*m*sum_l x, the lazy-dmin form.
//
// Why MFMA for a batch of one: on the vector path every weight costs a
// mask and an fma_mix; here the nibbles are only masked into fp16
// subnormals (q * 2^-24, high nibbles in place as 16q * 2^-24; exact normal
// codes for very long rows, see code_operand_pair) and one 16x16x32 f16
// MFMA takes 512 of them.  The MFMA's B
// operand is 16 weight rows x 32 positions of one sub-block; its A operand carries the activations: rows 0, 2, 4, ... hold
// the fp16 hi part of x and rows 1, 3, 5, ... the lo part (hi = fp16(x),
// lo = fp16(x - hi), both exact as MFMA inputs), so D rows 4g and 4g + 1
// of every lane hold the hi and lo halves of the same dot product and one
// instruction does both.  Before the split each 32-activation sub-block is
// scaled by a power of two that brings its largest |x| into [2^14, 2^15):
// the halves can neither overflow fp16 nor, for any element within 2^-17 of
// the sub-block's largest, lose bits of lo to fp16's subnormal range.  The
// power of two is folded into the per-sub-block scale d*sc, which (like the
// lazy-dmin term) is applied once per sub-block in fp32; that scale stays
// finite for every |x| < 2^96 (d*sc < 2^22).
//
// Work decomposition: a workgroup owns 16 rows; its 16 waves (four per
// SIMD, so that one wave's LDS and MFMA latencies hide under another's
// work) split the super-blocks of input_dim (contiguous ranges).  A wave
// walks its range one super-block at a time: it loads it (16 rows x 144
// bytes of weights, 256 activations) with coalesced 16-byte loads one ahead,
// stores it in a wave-private LDS area (activations already split and in
// operand order, with their sub-block sums), then runs the MFMAs.  Lane
// (n = lane % 16, g = lane / 16) applies the scales of sub-blocks 2g and
// 2g+1 of row n; the four lane groups and the four waves are summed at the
// end, so every output has one writer and a fixed summation order.
#include <algorithm>

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int MV_ROWS = 16;           // rows per workgroup (one MFMA column tile)
constexpr int MV_WAVES = 16;
constexpr int MV_CB = 1;              // super-blocks per chunk
constexpr int MV_WCH = MV_ROWS * MV_CB * 9;             // 16-byte weight chunks per chunk
constexpr int MV_WPL = (MV_WCH + 63) / 64;              // weight loads per lane
constexpr int MV_XPL = MV_CB * 256 / 4 / 64;            // activation float4 per lane
// LDS dwords per staged row, unpadded: each lane's 16-byte chunk lands in
// one contiguous 16-byte store and the operand reads of 16 rows hit
// distinct banks (measured with the bank conflict counter: no conflict
// cycles, against 4 per chunk store and 2 per code read with rows of 38)
constexpr int MV_WROW = MV_CB * 36;
constexpr int MV_XLO = MV_CB * 128 + 16;                // lo part of a wave's activations
constexpr int MV_XZ = 2 * MV_XLO;                       // zeros for even MFMAs j; + 32: odd
constexpr int MV_XW = MV_XZ + 64;                       // dwords per wave
static_assert(MV_CB == 1 && MV_XZ % 64 == 32, "zero areas in the bank halves the reads leave free");
static_assert(MV_XPL * 64 * 4 == MV_CB * 256, "activation chunk must split evenly");

// 16-byte weight loads of both kernels here, without the non-temporal hint
// the other GEMVs use.  A 144-byte row piece shares its 128-byte lines with
// the neighbouring super-blocks, which other waves load at about the same
// time; with the hint, 4096x4096 measured 4.11 us per call against 3.91
// without it, and the FFN pair 18.8 against 17.8 (MI355X, graph replay;
// the same with the rotation widened to 4 GiB: 4.03 / 3.83 and 18.4 /
// 17.3).  Kernels whose waves read whole lines keep the hint.
__device__ __forceinline__ uint4 load_buf16(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool NC>  // exact normal code operands (rows of more than 256 super-blocks)
__global__ __launch_bounds__(64 * MV_WAVES) void q4k_gemv_mfma_kernel(
    const float *x, const uint8_t *w, float *__restrict__ y, int nb, int N) {
  // Per wave: staged weight rows, fp16 hi and lo activations of the chunk
  // (positions in operand order: pairs (0,2), (1,3), (4,6), (5,7) of every
  // 8), the chunk's sub-block sums; then the cross-wave partials.
  __shared__ __align__(16) uint32_t wt[MV_WAVES][MV_ROWS * MV_WROW];
  // Per wave: the hi part at 0, the lo part at MV_XLO (16 dwords further
  // modulo the banks: the hi and lo A rows of the four lane groups, read by
  // one instruction, then fall in different banks; measured with the bank
  // conflict counter, 4 conflict cycles per read with the parts a multiple
  // of the banks or 4 dwords apart, none at 8 to 48), then two zeroed areas
  // that A rows read in the MFMAs they do not feed (see compute_chunk), in
  // the bank half the real reads of that MFMA leave free.
  __shared__ __align__(16) uint32_t xhl[MV_WAVES][MV_XW];
  // per sub-block pair p (sub-blocks 2p, 2p+1): their x sums, then their
  // scaling exponents (int bits), read by one lane as one 16-byte word
  __shared__ __align__(16) float xse[MV_WAVES][MV_CB * 16];
  __shared__ float part[MV_WAVES][MV_ROWS];

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // B column / D column: weight row; A row
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7
  const int row0 = blockIdx.x * MV_ROWS;
  const int row_bytes = nb * kBlockBytes;
  // this wave's super-blocks [b_lo, b_hi) (nb * 16 < 2^31)
  const int b_lo = (int)((unsigned)(nb * wave) / MV_WAVES);
  const int b_hi = (int)((unsigned)(nb * (wave + 1)) / MV_WAVES);
  const int n_chunks = (b_hi - b_lo + MV_CB - 1) / MV_CB;

  // A workgroup reads its own 16 rows only; 16 rows and x stay below 2^31
  // bytes (input_dim <= 2^24, checked by the host).
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc32(w + (int64_t)row0 * row_bytes, (uint32_t)min(N - row0, MV_ROWS) * (uint32_t)row_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc32(x, (uint32_t)nb * 1024u);

  // Load roles: weight chunk q (clamped; the duplicates are never stored)
  // is row q / (9 MV_CB), chunk q % (9 MV_CB) of the row's piece of the chunk;
  // activation float4 i is positions 4*(lane + 64 i) of the chunk.
  int woff[MV_WPL];
#pragma unroll
  for (int m = 0; m < MV_WPL; ++m) {
    const int q = min(lane + 64 * m, MV_WCH - 1);
    const int row = q / (9 * MV_CB);
    woff[m] = row * row_bytes + 16 * (q - row * 9 * MV_CB);
  }
  uint4 wa[MV_WPL], wb[MV_WPL];
  float4 xa[MV_XPL], xb[MV_XPL];
  auto load_chunk = [&](int c, uint4 (&wv)[MV_WPL], float4 (&xv)[MV_XPL]) {
    const int b0 = __builtin_amdgcn_readfirstlane(b_lo + c * MV_CB);  // wave-uniform
#pragma unroll
    for (int i = 0; i < MV_XPL; ++i) xv[i] = load_buf_f4(xr, 16 * (lane + 64 * i), 1024 * b0);
#pragma unroll
    for (int m = 0; m < MV_WPL; ++m) wv[m] = load_buf16(wr, woff[m], kBlockBytes * b0);
  };

  // The first chunk's loads leave before the rest of the set-up below (the
  // operand indices, the zero areas), which then runs while they are in
  // flight.
  if (n_chunks > 0) load_chunk(0, wa, xa);
  __builtin_amdgcn_sched_barrier(0);

  uint32_t *wtw = wt[wave];
  auto stage_chunk = [&](const uint4 (&wv)[MV_WPL], const float4 (&xv)[MV_XPL]) {
    // the activations first: they were loaded first (and come from L2), so
    // their split runs while the weight bytes are still arriving
#pragma unroll
    for (int i = 0; i < MV_XPL; ++i) {
      const float4 v0 = xv[i];
      // sub-block (f / 8, 8 aligned lanes) scaling: |x| * 2^-e < 2^15
      float mx = fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w)));
      mx = group_max_nonneg<8>(mx);
      const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
      const float4 v = make_float4(__builtin_ldexpf(v0.x, -e), __builtin_ldexpf(v0.y, -e),
                                   __builtin_ldexpf(v0.z, -e), __builtin_ldexpf(v0.w, -e));
      half2_t h02, h13;
      h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
      h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
      const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
      const int f = lane + 64 * i;  // float4 index: positions 4f .. 4f+3
      *reinterpret_cast<uint2 *>(&xhl[wave][2 * f]) = make_uint2(hw02, hw13);
      *reinterpret_cast<uint2 *>(&xhl[wave][MV_XLO + 2 * f]) =
          make_uint2(lo_pair(hw02, v.x, v.z), lo_pair(hw13, v.y, v.w));
      // sub-block f / 8: the 8 float4 of a sub-block sit in 8 aligned lanes
      const float s = group_sum<8>(sum4(v0));
      if ((lane & 7) == 0) {
        const int sb = f >> 3;
        xse[wave][4 * (sb >> 1) + (sb & 1)] = s;
        xse[wave][4 * (sb >> 1) + 2 + (sb & 1)] = __builtin_bit_cast(float, e);
      }
    }
#pragma unroll
    for (int m = 0; m < MV_WPL; ++m) {
      const int q = lane + 64 * m;
      if (MV_WCH % 64 != 0 && q >= MV_WCH) break;  // only the last load is partial
      const int row = q / (9 * MV_CB);
      uint32_t *dst = &wtw[row * MV_WROW + 4 * (q - row * 9 * MV_CB)];
      *reinterpret_cast<uint4 *>(dst) = wv[m];
    }
  };

  // A operand: row n carries the hi part (n even) or the lo part (n odd) of
  // sub-block 2j (MFMA on low nibbles) or 2j+1 (high nibbles) only in the
  // MFMAs j = n / 4; in the other three it reads zeros.  So D rows 4j ..
  // 4j+3 hold sub-block pair j alone, one accumulator per nibble half sums
  // the four MFMAs, and lane (n, g) finds its pair j = g in its own rows 4g
  // (hi) and 4g+1 (lo): no selection among four results.  aidx: 16-byte
  // units of the wave's area.
  const int j_mine = g;  // sub-blocks 2g, 2g+1 are scaled by this lane
  int aidx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    aidx[j] = (n >> 2) == j ? ((n & 1) * MV_XLO + 32 * j + 4 * g) >> 2 : (MV_XZ + 32 * (j & 1)) >> 2;
  const uint4 *const xa4 = reinterpret_cast<const uint4 *>(xhl[wave]);
  const uint32_t sh = (uint32_t)(g & 1) * 16u;
  const bool jhi = g >= 2;
  // Code reads: one 8-byte read per sub-block pair, each from its own base
  // register (8-byte units).  Sharing one base, the compiler pairs them
  // into ds_read2_b64 (offsets 32 bytes apart), which measured 8
  // bank-conflict cycles per pair; single reads of the same bytes none.
  int qoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qoff[j] = (n * MV_WROW + 4 + 8 * j + 2 * g) >> 1;
    asm volatile("" : "+v"(qoff[j]));
  }
  const uint2 *const wt2 = reinterpret_cast<const uint2 *>(wtw);
  float yacc = 0.f;

  auto compute_chunk = [&](int c) {
    const int nblk = min(MV_CB, b_hi - (b_lo + c * MV_CB));
#pragma unroll
    for (int bb = 0; bb < MV_CB; ++bb) {
      if (bb >= nblk) break;  // wave-uniform
      const uint32_t *rowp = &wtw[n * MV_WROW + 36 * bb];
      // header of row n: d, dmin and the scale/min of sub-blocks 2g, 2g+1
      const uint2 h01 = *reinterpret_cast<const uint2 *>(rowp);
      const uint2 h23 = *reinterpret_cast<const uint2 *>(rowp + 2);
      const uint32_t p1 = h01.y >> sh, p2 = h23.x >> sh, t3 = h23.y >> sh;
      const uint32_t sc_src = jhi ? t3 : p1;
      const uint32_t m_src = jhi ? (t3 >> 4) : p2;
      const uint32_t mask_lo = jhi ? 0x0F0Fu : 0x3F3Fu;
      const uint32_t mask_hi = jhi ? 0x3030u : 0u;
      const uint32_t scp = (sc_src & mask_lo) | ((p1 >> 2) & mask_hi);
      const uint32_t mp = (m_src & mask_lo) | ((p2 >> 2) & mask_hi);
      const float d = half_lo(h01.x), dmin = half_hi(h01.x);
      const float4 xsp = *reinterpret_cast<const float4 *>(&xse[wave][4 * (4 * bb + j_mine)]);
      // codes enter as q * 2^-c (low nibbles) and 16q * 2^-c (high), c =
      // kCodeShift<NC>; the activations as x * 2^-e
      const float s_lo = __builtin_ldexpf(d * (float)(scp & 0xFFu),
                                          __builtin_bit_cast(int, xsp.z) + kCodeShift<NC>);
      const float s_hi = __builtin_ldexpf(d * (float)((scp >> 8) & 0xFFu),
                                          __builtin_bit_cast(int, xsp.w) + kCodeShift<NC> - 4);
      yacc = __builtin_fmaf(-dmin, __builtin_fmaf((float)(mp & 0xFFu), xsp.x,
                                                  (float)((mp >> 8) & 0xFFu) * xsp.y), yacc);
      // All operands of the block first, then eight independent MFMAs, then
      // the combine: no read waits on a just-issued MFMA.
      uint2 qb[4];
      half8_t alo[4], ahi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qb[j] = wt2[qoff[j] + 18 * bb];
        alo[j] = __builtin_bit_cast(half8_t, xa4[aidx[j]]);      // positions 8g.. of 2j
        ahi[j] = __builtin_bit_cast(half8_t, xa4[aidx[j] + 4]);  // of 2j + 1 (32 on)
      }
      floatx4 dlo = {0.f, 0.f, 0.f, 0.f}, dhi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t s0 = qb[j].x >> 8, s1 = qb[j].y >> 8;
        uint4 blo, bhi;
        blo.x = code_operand_pair<NC>(qb[j].x, 0x000F000Fu); blo.y = code_operand_pair<NC>(s0, 0x000F000Fu);
        blo.z = code_operand_pair<NC>(qb[j].y, 0x000F000Fu); blo.w = code_operand_pair<NC>(s1, 0x000F000Fu);
        bhi.x = code_operand_pair<NC>(qb[j].x, 0x00F000F0u); bhi.y = code_operand_pair<NC>(s0, 0x00F000F0u);
        bhi.z = code_operand_pair<NC>(qb[j].y, 0x00F000F0u); bhi.w = code_operand_pair<NC>(s1, 0x00F000F0u);
        dlo = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[j], __builtin_bit_cast(half8_t, blo),
                                                      dlo, 0, 0, 0);
        dhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[j], __builtin_bit_cast(half8_t, bhi),
                                                      dhi, 0, 0, 0);
      }
      // D rows 4g (hi part) and 4g + 1 (lo part) of row n: sub-block pair
      // j = g, the other MFMAs having added exact zeros to them
      const float t_lo = dlo[0] + dlo[1], t_hi = dhi[0] + dhi[1];
      yacc = __builtin_fmaf(s_lo, t_lo, __builtin_fmaf(s_hi, t_hi, yacc));
    }
  };

  // the zero areas (64 dwords per wave, read after this wave's own stores)
  xhl[wave][MV_XZ + lane] = 0u;
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
  if (lane < MV_ROWS) part[wave][lane] = yacc;
  __syncthreads();
  if (tid < MV_ROWS) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < MV_WAVES; ++k) v += part[k][tid];
    if (row0 + tid < N) y[row0 + tid] = v;
  }
}

// The persistent walk: the same product for matrices that the form above
// does not fill the chip with, i.e. long rows (one workgroup's 16 waves
// would each walk several super-blocks with one loaded ahead) or many rows
// (more 16-wave workgroups than fit at once).  A W-wave workgroup owns
// rg_per_wg consecutive groups of 16 rows and walks input_dim in chunks of
// up to CAP super-blocks.  Wave w takes units w, w + W, w + 2W, ... of a
// chunk's (row group, super-block) units in row-group-major order and keeps
// D units loaded ahead in registers (a unit is the 16 x 144 weight bytes of
// one super-block of the group: three coalesced 16-byte loads per lane,
// rows of 9 chunks); computing a unit first moves its bytes through the
// wave's LDS tile into operand order.  The chunk's activations are staged
// in LDS as fp16 hi and lo in operand order with their sub-block sums and
// scaling exponents:
//   - cooperatively (PRIV false), by the whole workgroup before the chunk's
//     units and behind a barrier, their loads issued before the first tiles';
//   - per wave (PRIV, when input_dim / 256 is above 16 and within one
//     chunk, and a multiple of W or the workgroup owns one row group): wave
//     w then only ever uses super-blocks w, w + W, ..., and stages each on
//     first use (in the first row group), its activations loaded with the
//     unit.
// A wave's partial sums go to LDS whenever its row group changes; the
// lanes' and waves' partials are summed in a fixed order at the end (one
// writer per output).
constexpr int WK_MAX_RG = 4;  // row groups per workgroup

template <int W, int D, int CAP, bool PRIV, bool NC>
__global__ __launch_bounds__(64 * W) void q4k_gemv_walk_kernel(
    const float *x, const uint8_t *w, float *__restrict__ y, int nb, int N, int rg_per_wg) {
  constexpr int XPL = CAP / W;  // activation float4 per thread of a chunk
  static_assert(XPL * 64 * W == CAP * 64, "a chunk's activations must split evenly");
  // the hi part, then the lo part 16 dwords further modulo the banks: the
  // hi and lo A rows of the four lane groups, read by one instruction, then
  // fall in different banks (4 conflict cycles per read otherwise); then
  // the zero areas that A rows read in the MFMAs they do not feed, in the
  // bank half the real reads of that MFMA leave free (as in the form above)
  constexpr int XZ = 2 * CAP * 128 + 32;  // even MFMAs j; + 32: odd
  __shared__ __align__(16) uint32_t xhl[XZ + 64];
  uint32_t *const xh = xhl;
  uint32_t *const xl = xhl + CAP * 128 + 16;
  // per sub-block pair p: its two x sums, then its two exponents (int bits)
  __shared__ __align__(16) float xse[CAP * 16];
  __shared__ __align__(16) uint32_t wt[W][MV_ROWS * MV_WROW];
  __shared__ float part[W][WK_MAX_RG][64];

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // B / D column: weight row of the group; A row
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7 of a sub-block
  const int NG = (N + MV_ROWS - 1) / MV_ROWS;
  const int rg0 = blockIdx.x * rg_per_wg;
  const int rgn = min(rg_per_wg, NG - rg0);
  const int row_bytes = nb * kBlockBytes;
  const int rg_bytes = MV_ROWS * row_bytes;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(
      w + (int64_t)rg0 * rg_bytes, (int64_t)(N - rg0 * MV_ROWS) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)nb * 1024);
  constexpr int kPastEnd = 0x7FFFF000;  // a unit or activation offset that reads zeros

#pragma unroll
  for (int r = 0; r < WK_MAX_RG; ++r) part[wave][r][lane] = 0.f;

  // weight chunk q of a unit (clamped; the duplicates are never stored) is
  // chunk q % 9 of row q / 9
  int woff[MV_WPL];
#pragma unroll
  for (int m = 0; m < MV_WPL; ++m) {
    const int q = min(lane + 64 * m, MV_WCH - 1);
    const int row = q / 9;
    woff[m] = row * row_bytes + 16 * (q - 9 * row);
  }
  uint4 wq[D][MV_WPL];
  float4 xq[PRIV ? D : 1];

  // A operand: row n feeds only MFMAs j = n / 4, reading the hi (n even)
  // or lo (n odd) part there and zeros in the other three, so one
  // accumulator per nibble half collects sub-block pair j in D rows 4j ..
  // 4j+3 and lane (n, g) finds its pair g in its rows 4g, 4g+1.  16-byte
  // units: this lane's part at a_own + 32 * super-block.
  const int a_own = ((n & 1) * (CAP * 128 + 16) + 32 * (n >> 2) + 4 * g) >> 2;
  const uint4 *const xa4 = reinterpret_cast<const uint4 *>(xhl);
  const uint32_t sh = (uint32_t)(g & 1) * 16u;
  const bool jhi = g >= 2;
  uint32_t *wtw = wt[wave];
  xhl[XZ + lane] = 0u;  // each wave before its own reads (same values)
  // Code reads: one 8-byte read per sub-block pair, each from its own base
  // register (8-byte units).  Sharing one base, the compiler pairs them
  // into ds_read2_b64 (offsets 32 bytes apart), which measured 8
  // bank-conflict cycles per pair; single reads of the same bytes none.
  int qoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qoff[j] = (n * MV_WROW + 4 + 8 * j + 2 * g) >> 1;
    asm volatile("" : "+v"(qoff[j]));
  }
  const uint2 *const wt2 = reinterpret_cast<const uint2 *>(wtw);

  // Stage float4 f of a chunk (positions 4f .. 4f+3; its sub-block f / 8
  // sits in 8 aligned lanes): scale the sub-block by 2^-e so that
  // |x| * 2^-e < 2^15, split into fp16 hi + lo, store its sum and e.
  auto stage4 = [&](float4 v0, int f) {
    float mx = fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w)));
    mx = group_max_nonneg<8>(mx);
    const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    const float4 v = make_float4(__builtin_ldexpf(v0.x, -e), __builtin_ldexpf(v0.y, -e),
                                 __builtin_ldexpf(v0.z, -e), __builtin_ldexpf(v0.w, -e));
    half2_t h02, h13;
    h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
    h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
    const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
    *reinterpret_cast<uint2 *>(&xh[2 * f]) = make_uint2(hw02, hw13);
    *reinterpret_cast<uint2 *>(&xl[2 * f]) =
        make_uint2(lo_pair(hw02, v.x, v.z), lo_pair(hw13, v.y, v.w));
    const float sum = group_sum<8>(sum4(v0));
    if ((lane & 7) == 0) {
      const int sb = f >> 3;
      xse[4 * (sb >> 1) + (sb & 1)] = sum;
      xse[4 * (sb >> 1) + 2 + (sb & 1)] = __builtin_bit_cast(float, e);
    }
  };
  // the wave reads what its own lanes wrote: LDS executes one wave's
  // instructions in order; keep the compiler from moving them
  auto wave_lds_order = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  for (int c0 = 0; c0 < nb; c0 += CAP) {
    const int nbc = min(CAP, nb - c0);
    const int U = rgn * nbc;
    const int T = wave < U ? (U - wave + W - 1) / W : 0;
    // unit (i, bl): row group i, super-block c0 + bl
    auto advance = [&](int &i, int &bl) {
      bl += W;
      while (bl >= nbc) { bl -= nbc; ++i; }
    };
    auto load_unit = [&](int s, int i, int bl, bool valid) {
      const int off = valid ? i * rg_bytes + (c0 + bl) * kBlockBytes : kPastEnd;
      if constexpr (PRIV)  // activations of super-block bl, needed in the first row group only
        xq[s] = load_buf_f4(xr, 16 * lane, valid && i == 0 ? 1024 * bl : kPastEnd);
#pragma unroll
      for (int m = 0; m < MV_WPL; ++m) wq[s][m] = load_buf16(wr, woff[m], off);
    };

    // Cooperative staging loads the chunk's activations first, then the
    // first D units: staging waits only for the activation loads.
    float4 xv[PRIV ? 1 : XPL];
    if constexpr (!PRIV) {
#pragma unroll
      for (int r = 0; r < XPL; ++r) xv[r] = load_buf_f4(xr, 16 * (tid + 64 * W * r), 1024 * c0);
    }
    int li = 0, lbl = wave;
    while (lbl >= nbc) { lbl -= nbc; ++li; }
    int ci = li, cbl = lbl;
#pragma unroll
    for (int s = 0; s < D; ++s) {
      load_unit(s, li, lbl, s < T);
      advance(li, lbl);
    }
    if constexpr (!PRIV) {
      if (c0 > 0) __syncthreads();  // the previous chunk's operands are no longer read
#pragma unroll
      for (int r = 0; r < XPL; ++r) stage4(xv[r], tid + 64 * W * r);
      __syncthreads();
    }

    float acc = 0.f;
    int acc_i = ci;
    auto compute = [&](int s, int bl) {
      if constexpr (PRIV) {
        if (ci == 0) stage4(xq[s], 64 * bl + lane);  // wave-uniform: first use of bl
      }
      // the unit's weight bytes into the wave's tile, read back in operand order
#pragma unroll
      for (int m = 0; m < MV_WPL; ++m) {
        const int q = lane + 64 * m;
        if (MV_WCH % 64 != 0 && q >= MV_WCH) break;  // only the last load is partial
        const int row = q / 9;
        uint32_t *dst = &wtw[row * MV_WROW + 4 * (q - 9 * row)];
        *reinterpret_cast<uint4 *>(dst) = wq[s][m];
      }
      wave_lds_order();
      const uint32_t *rowp = &wtw[n * MV_WROW];
      // header of row n: d, dmin and the scale/min of sub-blocks 2g, 2g+1
      const uint2 h01 = *reinterpret_cast<const uint2 *>(rowp);
      const uint2 h23 = *reinterpret_cast<const uint2 *>(rowp + 2);
      const uint32_t p1 = h01.y >> sh, p2 = h23.x >> sh, t3 = h23.y >> sh;
      const uint32_t sc_src = jhi ? t3 : p1;
      const uint32_t m_src = jhi ? (t3 >> 4) : p2;
      const uint32_t mask_lo = jhi ? 0x0F0Fu : 0x3F3Fu;
      const uint32_t mask_hi = jhi ? 0x3030u : 0u;
      const uint32_t scp = (sc_src & mask_lo) | ((p1 >> 2) & mask_hi);
      const uint32_t mp = (m_src & mask_lo) | ((p2 >> 2) & mask_hi);
      const float d = half_lo(h01.x), dmin = half_hi(h01.x);
      const float4 xsp = *reinterpret_cast<const float4 *>(&xse[4 * (4 * bl + g)]);
      // codes enter as q * 2^-c (low nibbles) and 16q * 2^-c (high), c =
      // kCodeShift<NC>; the activations as x * 2^-e
      const float s_lo = __builtin_ldexpf(d * (float)(scp & 0xFFu),
                                          __builtin_bit_cast(int, xsp.z) + kCodeShift<NC>);
      const float s_hi = __builtin_ldexpf(d * (float)((scp >> 8) & 0xFFu),
                                          __builtin_bit_cast(int, xsp.w) + kCodeShift<NC> - 4);
      acc = __builtin_fmaf(-dmin, __builtin_fmaf((float)(mp & 0xFFu), xsp.x,
                                                 (float)((mp >> 8) & 0xFFu) * xsp.y), acc);
      uint2 qb[4];
      half8_t alo[4], ahi[4];
      const int a_real = a_own + 32 * bl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qb[j] = wt2[qoff[j]];
        const int ai = (n >> 2) == j ? a_real : (XZ + 32 * (j & 1)) >> 2;
        alo[j] = __builtin_bit_cast(half8_t, xa4[ai]);      // positions 8g.. of 2j
        ahi[j] = __builtin_bit_cast(half8_t, xa4[ai + 4]);  // of 2j + 1
      }
      floatx4 dlo = {0.f, 0.f, 0.f, 0.f}, dhi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t s0 = qb[j].x >> 8, s1 = qb[j].y >> 8;
        uint4 blo, bhi;
        blo.x = code_operand_pair<NC>(qb[j].x, 0x000F000Fu); blo.y = code_operand_pair<NC>(s0, 0x000F000Fu);
        blo.z = code_operand_pair<NC>(qb[j].y, 0x000F000Fu); blo.w = code_operand_pair<NC>(s1, 0x000F000Fu);
        bhi.x = code_operand_pair<NC>(qb[j].x, 0x00F000F0u); bhi.y = code_operand_pair<NC>(s0, 0x00F000F0u);
        bhi.z = code_operand_pair<NC>(qb[j].y, 0x00F000F0u); bhi.w = code_operand_pair<NC>(s1, 0x00F000F0u);
        dlo = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[j], __builtin_bit_cast(half8_t, blo),
                                                      dlo, 0, 0, 0);
        dhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[j], __builtin_bit_cast(half8_t, bhi),
                                                      dhi, 0, 0, 0);
      }
      // D rows 4g (hi part) and 4g + 1 (lo part) of row n: pair j = g
      const float t_lo = dlo[0] + dlo[1], t_hi = dhi[0] + dhi[1];
      acc = __builtin_fmaf(s_lo, t_lo, __builtin_fmaf(s_hi, t_hi, acc));
      // the next unit's stores into the tile come after these reads
      wave_lds_order();
    };

    for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        if (t0 + s < T) {  // wave-uniform
          if (ci != acc_i) {
            part[wave][acc_i][lane] += acc;
            acc = 0.f;
            acc_i = ci;
          }
          compute(s, cbl);
          advance(ci, cbl);
        }
        // always issued (zeros past the wave's units): the number of loads
        // in flight is the same on every path
        load_unit(s, li, lbl, t0 + s + D < T);
        advance(li, lbl);
      }
    }
    if (T > 0) part[wave][acc_i][lane] += acc;
  }

  __syncthreads();
  if (tid < rgn * MV_ROWS) {
    const int i = tid >> 4, r = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k)
      v += (part[k][i][r] + part[k][i][r + 16]) + (part[k][i][r + 32] + part[k][i][r + 48]);
    const int row = (rg0 + i) * MV_ROWS + r;
    if (row < N) y[row] = v;
  }
}

template <int W, int D, int CAP>
void launch_walk(const float *x, const uint8_t *w, float *y, int64_t nb, int64_t N, int rg,
                 hipStream_t stream) {
  const int64_t NG = (N + MV_ROWS - 1) / MV_ROWS;
  const dim3 grid((unsigned)((NG + rg - 1) / rg));
  if (CAP > 16 && nb > 16 && (nb % W == 0 || rg == 1) && nb <= CAP)
    hipLaunchKernelGGL((q4k_gemv_walk_kernel<W, D, CAP, CAP != 16, false>), grid, dim3(64 * W), 0,
                       stream, x, w, y, (int)nb, (int)N, rg);
  else if (CAP > 16 && nb > kNormalCodesAbove)
    hipLaunchKernelGGL((q4k_gemv_walk_kernel<W, D, CAP, false, CAP != 16>), grid, dim3(64 * W), 0,
                       stream, x, w, y, (int)nb, (int)N, rg);
  else
    hipLaunchKernelGGL((q4k_gemv_walk_kernel<W, D, CAP, false, false>), grid, dim3(64 * W), 0,
                       stream, x, w, y, (int)nb, (int)N, rg);
}

}  // namespace

bool use_gemv_mfma(int64_t nb, int64_t N) {
  // Measured (graph-replayed calls over rotating weights, input_dim and
  // output_dim 2048 to 8192; us/call, vector form / this form): the
  // matrix-core form wins when its grid fills 192 to 256 CUs once, one
  // 16-wave workgroup each, with 12 to 16 super-blocks a row (3072x3072
  // 4.06 / 3.56, 4096->3072 4.16 / 3.64, 3072->4096 4.11 / 3.77, 4096x4096
  // 4.39 / 3.91); with 8 super-blocks (2048->4096 3.12 / 3.46), on 128
  // workgroups (4096->2048 3.31 / 3.42) or past 256 the vector kernel's
  // several-per-CU occupancy wins, and from 20 super-blocks the walk does.
  const int64_t grid = (N + MV_ROWS - 1) / MV_ROWS;
  return grid >= 192 && grid <= 256 && nb >= 12 && nb <= 19;
}

hipError_t gemv_mfma_launch(const float *x, const uint8_t *w, float *y, int64_t nb,
                            int64_t N, hipStream_t stream) {
  const int64_t grid = (N + MV_ROWS - 1) / MV_ROWS;
  // Offsets formed in the kernel: 16 rows of weights and the activation
  // vector stay below 2^31 bytes.
  if (grid > 0x7FFFFFFF || N > 0x7FFFFFFF ||
      (int64_t)MV_ROWS * nb * kBlockBytes >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  if (nb > kNormalCodesAbove)
    hipLaunchKernelGGL(q4k_gemv_mfma_kernel<true>, dim3((unsigned)grid), dim3(64 * MV_WAVES), 0,
                       stream, x, w, y, (int)nb, (int)N);
  else
    hipLaunchKernelGGL(q4k_gemv_mfma_kernel<false>, dim3((unsigned)grid), dim3(64 * MV_WAVES), 0,
                       stream, x, w, y, (int)nb, (int)N);
  return hipGetLastError();
}

WalkShape choose_walk_shape(int64_t nb, int64_t N, int waves, int row_groups, int depth) {
  WalkShape s;
  const int64_t NG = (N + MV_ROWS - 1) / MV_ROWS;
  s.row_groups = row_groups ? row_groups
                            : (int)std::min<int64_t>(WK_MAX_RG, std::max<int64_t>(1, (NG + 255) / 256));
  s.waves = waves ? waves : 8;
  s.depth = depth ? depth : (s.waves == 4 ? 4 : 2);
  return s;
}

bool use_gemv_walk(int64_t nb, int64_t N) {
  // Measured (graph-replayed calls over rotating weights, input_dim 2048 to
  // 28672, output_dim 1024 to 28672; best other form / walk with 8 waves
  // and 2 units ahead, us/call): the walk wins once rows hold 20
  // super-blocks or more and output_dim is 3072 or more, 5120->3072 5.17 /
  // 4.77, 5120x5120 8.10 / 7.03, 6144->4096 5.95 / 5.67, 6144->8192 10.22 /
  // 7.71, 8192x8192 10.73 / 9.45, 14336->4096 11.37 / 9.89, 28672->28672
  // 123.0 / 98.1, and for 16 super-blocks from output_dim 11008 (4096->14336
  // 10.17 / 9.62); it loses at output_dim 2048 (8192->2048 4.27 / 5.79,
  // 14336->2048 7.89 / 8.78) and with 16 super-blocks below 11008 rows
  // (4096x4096 3.91 / 4.71, 4096->8192 5.95 / 6.28).  The offsets its launch
  // forms must fit (four row groups).
  if ((int64_t)WK_MAX_RG * MV_ROWS * nb * kBlockBytes > 0x7FFF0000 || nb * 1024 > 0x7FFF0000)
    return false;
  return (N >= 3072 && nb >= 20) || (N >= 11008 && nb >= 16);
}

hipError_t gemv_walk_launch(const float *x, const uint8_t *w, float *y, int64_t nb, int64_t N,
                            const WalkShape &s, hipStream_t stream) {
  const int64_t NG = (N + MV_ROWS - 1) / MV_ROWS;
  // Offsets formed in the kernel: a workgroup's rows stay below the
  // past-the-end offset its idle loads use, and the activations below 2^31.
  if (NG > 0x7FFFFFFF || s.row_groups < 1 || s.row_groups > WK_MAX_RG ||
      (int64_t)s.row_groups * MV_ROWS * nb * kBlockBytes > 0x7FFF0000 ||
      nb * 1024 > 0x7FFF0000)
    return hipErrorInvalidValue;
  const bool small = nb <= 16;
#define Q4K_WALK_CASE(W_, D_)                                                             \
  if (s.waves == W_ && s.depth == D_) {                                                   \
    if (small)                                                                            \
      launch_walk<W_, D_, 16>(x, w, y, nb, N, s.row_groups, stream);                      \
    else                                                                                  \
      launch_walk<W_, D_, 64>(x, w, y, nb, N, s.row_groups, stream);                      \
    return hipGetLastError();                                                             \
  }
  Q4K_WALK_CASE(4, 4)
  Q4K_WALK_CASE(8, 2)
  Q4K_WALK_CASE(8, 4)
  Q4K_WALK_CASE(16, 2)
#undef Q4K_WALK_CASE
  return hipErrorInvalidValue;
}

}  // namespace q4k
