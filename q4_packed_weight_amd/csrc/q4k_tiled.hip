// q4k_tiled.hip -- the tiled block order of a Q4_K matrix: the one-time
// relayout from the canonical layout, and the matrix-vector, few-token and
// 64-row prefill products that stream the tiled order (narrower prefill
// tiles, and 64-row ones from input_dim 8192 on, run q4k_prefill.hip's
// kernel on it).
//
// SKaiNET docs, "Eager execution: backends and kernels": a packed weight
// reaches a kernel by declaring its block order, and a canonical weight is
// relayouted into that order once, not per call.  The tiled order is this
// library's GPU block order.  It moves the canonical bytes and changes none:
// rows in groups of 16 (rows past output_dim are zero bytes), super-block b
// of group G one 2304-byte tile at (G * nb + b) * 2304, and inside a tile
//   bytes    0..2047  qs, two halves of 1024: the 16 bytes at 1024h + 16L
//                     (n = L % 16, g = L / 16) are qs bytes 8g..8g+7 of
//                     sub-block pairs 2h and 2h+1 of row 16G + n
//   bytes 2048..2303  the 16-byte block headers of the 16 rows, in order.
// So the 64 lanes of a wave, loading 16 bytes each at 16 * lane of a half,
// receive exactly their B operands of the 16x16x32 f16 MFMA (column n =
// weight row, positions 8g..8g+7 of a sub-block) for two sub-block pairs:
// a tile is three fully coalesced wave loads straight into registers, with
// no LDS staging of weights (the canonical form must stage through LDS,
// because a lane's operand bytes are spread over 16 rows' lines).
//
// The arithmetic is the canonical matrix-core GEMV's (Q4_K page: SKaiNET PR
// #562, "feat(kernel): SIMD-fused Q4_K matmul kernel + Q4KMatmulKernel SPI",
// sections "Summary" and "Pipeline", in the lazy-dmin form): nibbles masked
// into fp16 subnormals (exact normal codes for very long rows,
// code_operand_pair), activations split into exact fp16 hi + lo
// parts (A rows of alternating parity), every 32-activation sub-block scaled
// by a power of two first, scales applied per sub-block in fp32 after the
// MFMAs.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

constexpr int kBlockBytes = 144;
constexpr int kTileRows = 16;
constexpr int kTileBytes = 2304;
constexpr int kTileChunks = kTileBytes / 16;
constexpr int kMaxRowGroups = 4;  // row groups per workgroup

// One thread per 16-byte chunk of the tiled matrix: a gather of two 8-byte
// qs pieces (or one header) of the canonical row, or zeros for a padding row.
__global__ __launch_bounds__(256) void q4k_relayout_tiled_kernel(
    const uint8_t *__restrict__ w, uint8_t *__restrict__ out, int64_t nb, int64_t N,
    int64_t n_chunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  const int64_t tile = c / kTileChunks;
  const int within = (int)(c - tile * kTileChunks);
  const int64_t G = tile / nb, b = tile - G * nb;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (within < 128) {
    const int h = within >> 6, L = within & 63;
    const int64_t row = G * kTileRows + (L & 15);
    if (row < N) {
      // qs byte 32j + 8g of pair j = 2h sits at block byte 16 + 64h + 8g
      const uint8_t *src = w + (row * nb + b) * kBlockBytes + 16 + 64 * h + 8 * (L >> 4);
      const uint2 a = *reinterpret_cast<const uint2 *>(src);
      const uint2 e = *reinterpret_cast<const uint2 *>(src + 32);
      v = make_uint4(a.x, a.y, e.x, e.y);
    }
  } else {
    const int64_t row = G * kTileRows + (within - 128);
    if (row < N) v = *reinterpret_cast<const uint4 *>(w + (row * nb + b) * kBlockBytes);
  }
  *reinterpret_cast<uint4 *>(out + c * 16) = v;
}

// Workgroup: W waves, `rg_per_wg` consecutive row groups (their tiles are
// one contiguous stream), input_dim walked in chunks of up to CAP
// super-blocks.  Wave w takes units w, w + W, w + 2W, ... of a chunk's (row
// group, super-block) units in row-group-major order, D tiles loaded ahead.
// The activations of a chunk are staged in LDS as fp16 hi and lo in operand
// order, with sub-block sums and scaling exponents:
//   - cooperative (PRIV false): by the whole workgroup before the chunk's
//     units, behind a barrier;
//   - per wave (PRIV, when input_dim/256 is a multiple of W, above 16 and
//     within one chunk): unit (i, b) then always has b = w (mod W), so wave
//     w uses only super-blocks w, w + W, ...; it stages each on first use (the first
//     row group), its activations riding in the tile prefetch ring, with no
//     barrier and no start-up wait for all of x.
// A wave's partial sums go to LDS whenever its row group changes; the
// waves' partials are summed in a fixed order at the end (one writer per
// output, deterministic).
template <int W, int D, int CAP, bool PRIV, bool NC>
__global__ __launch_bounds__(64 * W) void q4k_gemv_tiled_kernel(
    const float *x, const uint8_t *wt, float *__restrict__ y, int nb, int N, int rg_per_wg) {
  constexpr int XPL = CAP * 64 / (64 * W);  // activation float4 per thread per chunk
  static_assert(XPL * 64 * W == CAP * 64, "a chunk's activations must split evenly");
  // the hi part, then the lo part 16 dwords further modulo the banks: the
  // hi and lo A rows of the four lane groups, read by one instruction, then
  // fall in different banks (4 conflict cycles per read otherwise)
  __shared__ __align__(16) uint32_t xhl[2 * CAP * 128 + 16];
  uint32_t *const xh = xhl;
  uint32_t *const xl = xhl + CAP * 128 + 16;
  // per sub-block pair p: its two x sums, then its two exponents (int bits)
  __shared__ __align__(16) float xse[CAP * 16];
  __shared__ float part[W][kMaxRowGroups][64];

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // B / D column: weight row of the group; A row
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7 of a sub-block
  const int NG = (N + kTileRows - 1) / kTileRows;
  const int rg0 = blockIdx.x * rg_per_wg;
  const int rgn = min(rg_per_wg, NG - rg0);

  // The workgroup's tiles (at most four row groups) and x stay below 2^31
  // bytes (input_dim <= 2^24), so the sizes need no 64-bit clamp ahead of
  // the first load and kPastEnd lies past the view's end.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc32(
      wt + (int64_t)rg0 * nb * kTileBytes, (uint32_t)rgn * (uint32_t)nb * (uint32_t)kTileBytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc32(x, (uint32_t)nb * 1024u);
  constexpr int kPastEnd = 0x7FFFF000;  // a tile or activation offset that reads zeros

  const int vq0 = 16 * lane, vq1 = 1024 + 16 * lane, vhd = 2048 + 16 * n;
  uint4 wq0[D], wq1[D], whd[D];
  float4 xq[PRIV ? D : 1];

  // A operand rows: even rows the hi part, odd rows the lo part.
  const uint32_t *xa_src = (n & 1) ? xl : xh;
  const uint32_t sh = (uint32_t)(g & 1) * 16u;
  const bool jhi = g >= 2;

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

  for (int c0 = 0; c0 < nb; c0 += CAP) {
    const int nbc = min(CAP, nb - c0);
    const int U = rgn * nbc;
    const int T = wave < U ? (U - wave + W - 1) / W : 0;
    // unit (i, bl) -> tile i * nb + c0 + bl of the workgroup's stream
    auto advance = [&](int &i, int &bl) {
      bl += W;
      while (bl >= nbc) { bl -= nbc; ++i; }
    };
    auto load_unit = [&](int s, int i, int bl, bool valid) {
      const int off = valid ? (i * nb + c0 + bl) * kTileBytes : kPastEnd;
      if constexpr (PRIV)  // activations of super-block bl, needed in the first row group only
        xq[s] = load_buf_f4(xr, 16 * lane, valid && i == 0 ? 1024 * bl : kPastEnd);
      wq0[s] = load_buf_stream16(wr, vq0, off);
      wq1[s] = load_buf_stream16(wr, vq1, off);
      whd[s] = load_buf_stream16(wr, vhd, off);
    };

    // Cooperative staging loads the chunk's activations first, then the
    // first D tiles: staging waits only for the activation loads.
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
    if (c0 == 0) {  // once the first loads have left
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < kMaxRowGroups; ++r) part[wave][r][lane] = 0.f;
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
        if (ci == 0) {  // wave-uniform: first use of super-block bl
          stage4(xq[s], 64 * bl + lane);
          // the wave reads what its own lanes wrote: LDS executes one wave's
          // instructions in order; keep the compiler from moving them
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
      const uint4 hd = whd[s];
      // header of row n: d, dmin and the scale/min of sub-blocks 2g, 2g+1
      const uint32_t p1 = hd.y >> sh, p2 = hd.z >> sh, t3 = hd.w >> sh;
      const uint32_t sc_src = jhi ? t3 : p1;
      const uint32_t m_src = jhi ? (t3 >> 4) : p2;
      const uint32_t mask_lo = jhi ? 0x0F0Fu : 0x3F3Fu;
      const uint32_t mask_hi = jhi ? 0x3030u : 0u;
      const uint32_t scp = (sc_src & mask_lo) | ((p1 >> 2) & mask_hi);
      const uint32_t mp = (m_src & mask_lo) | ((p2 >> 2) & mask_hi);
      const float d = half_lo(hd.x), dmin = half_hi(hd.x);
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
      qb[0] = make_uint2(wq0[s].x, wq0[s].y);
      qb[1] = make_uint2(wq0[s].z, wq0[s].w);
      qb[2] = make_uint2(wq1[s].x, wq1[s].y);
      qb[3] = make_uint2(wq1[s].z, wq1[s].w);
      half8_t alo[4], ahi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = 128 * bl + 32 * j + 4 * g;  // dword of sub-block 2j, positions 8g..
        alo[j] = *reinterpret_cast<const half8_t *>(&xa_src[pos]);
        ahi[j] = *reinterpret_cast<const half8_t *>(&xa_src[pos + 16]);
      }
      floatx4 dlo[4], dhi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t s0 = qb[j].x >> 8, s1 = qb[j].y >> 8;
        uint4 blo, bhi;
        blo.x = code_operand_pair<NC>(qb[j].x, 0x000F000Fu); blo.y = code_operand_pair<NC>(s0, 0x000F000Fu);
        blo.z = code_operand_pair<NC>(qb[j].y, 0x000F000Fu); blo.w = code_operand_pair<NC>(s1, 0x000F000Fu);
        bhi.x = code_operand_pair<NC>(qb[j].x, 0x00F000F0u); bhi.y = code_operand_pair<NC>(s0, 0x00F000F0u);
        bhi.z = code_operand_pair<NC>(qb[j].y, 0x00F000F0u); bhi.w = code_operand_pair<NC>(s1, 0x00F000F0u);
        dlo[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            alo[j], __builtin_bit_cast(half8_t, blo), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        dhi[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            ahi[j], __builtin_bit_cast(half8_t, bhi), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
      // D rows 4g (hi part) and 4g + 1 (lo part) of row n; this lane keeps
      // sub-block pair j = g
      float t_lo = dlo[0][0] + dlo[0][1], t_hi = dhi[0][0] + dhi[0][1];
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        if (j == g) {
          t_lo = dlo[j][0] + dlo[j][1];
          t_hi = dhi[j][0] + dhi[j][1];
        }
      }
      acc = __builtin_fmaf(s_lo, t_lo, __builtin_fmaf(s_hi, t_hi, acc));
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
  if (tid < rgn * kTileRows) {
    const int i = tid >> 4, r = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k)
      v += (part[k][i][r] + part[k][i][r + 16]) + (part[k][i][r + 32] + part[k][i][r + 48]);
    const int row = (rg0 + i) * kTileRows + r;
    if (row < N) y[row] = v;
  }
}

// A few tokens (2 to 8) on tiled weights: the batched product of
// q4k_gemv_batch.hip (A rows 2t and 2t + 1 carry token t's fp16 hi and lo
// parts, each token's super-block scaled by a power of two first; lane (n,
// g) applies all eight sub-block scales of row n to tokens 2g and 2g + 1),
// with each tile streamed straight into registers.  A workgroup owns one
// row group; wave w takes its super-blocks w, w + W, ..., D ahead, with the
// T tokens' activations of each super-block riding in the same ring and
// staged in a wave-private LDS slot just before use (every super-block's
// activations are staged once per workgroup, as in the canonical form).
template <int T, int W, int D, bool NC>
__global__ __launch_bounds__(64 * W) void q4k_gemv_tiled_batch_kernel(
    const float *X, const uint8_t *wt, float *__restrict__ Y, int M, int nb, int N) {
  // [wave][2t] token t's hi part, [wave][2t + 1] its lo part, rows of 136
  // dwords: the A rows of all lane groups, read by one instruction, then
  // fall in different banks (measured with the bank conflict counter: no
  // conflict cycles for 2, 4 or 8 tokens, against 4 to 28 per read with
  // rows of 128 or 132)
  __shared__ __align__(16) uint32_t xhl[W][2 * T][136];
  __shared__ __align__(16) float xs[W][T][8];
  __shared__ int xe[W][T];
  __shared__ float part[W][T][kTileRows];

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // weight row of the group; A row
  const int g = lane >> 4;  // lane group: positions 8g .. 8g+7; tokens 2g, 2g+1
  const int K = nb * 256;
  const int rg = blockIdx.x;
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(wt + (int64_t)rg * nb * kTileBytes, (int64_t)nb * kTileBytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (int64_t)M * K * 4);
  constexpr int kPastEnd = 0x7FFFF000;
  const int nt = wave < nb ? (nb - wave + W - 1) / W : 0;  // this wave's super-blocks

  const int vq0 = 16 * lane, vq1 = 1024 + 16 * lane, vhd = 2048 + 16 * n;
  uint4 wq0[D], wq1[D], whd[D];
  float4 xq[D][T];
  // slot s <- super-block b (its tile and the tokens' activations); idle
  // slots read zeros from past the end
  auto load_unit = [&](int s, int b, bool valid) {
    const int off = valid ? b * kTileBytes : kPastEnd;
#pragma unroll
    for (int t = 0; t < T; ++t)
      xq[s][t] = load_buf_f4(xr, t * K * 4 + 16 * lane, valid ? 1024 * b : kPastEnd);
    wq0[s] = load_buf_stream16(wr, vq0, off);
    wq1[s] = load_buf_stream16(wr, vq1, off);
    whd[s] = load_buf_stream16(wr, vhd, off);
  };

  // A operand: row n is token n / 2 (rows past 2T repeat token T - 1 and are
  // never read back), hi part in even rows, lo part in odd rows.
  const int ta = min(n >> 1, T - 1);
  const uint32_t *xa_src = xhl[wave][2 * ta + (n & 1)];
  const int t0 = min(2 * g, T - 1), t1 = min(2 * g + 1, T - 1);
  float y0 = 0.f, y1 = 0.f;

  auto compute = [&](int s) {
    // stage the tokens' activations of this super-block (positions 4 lane ..)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4 v0 = xq[s][t];
      const float mx = wave_max_nonneg_v(
          fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))));
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
      xs[wave][t][lane >> 3] = group_sum<8>(sum4(v0));  // 8 lanes write one value
      xe[wave][t] = e;                                  // every lane, one value
    }
    // the wave reads what its own lanes wrote: LDS executes one wave's
    // instructions in order; keep the compiler from moving them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const uint4 hd = whd[s];
    // header of row n: d, dmin and all eight 6-bit scales and mins
    const uint32_t sc03 = hd.y & 0x3F3F3F3Fu;
    const uint32_t mn03 = hd.z & 0x3F3F3F3Fu;
    const uint32_t sc47 = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mn47 = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    const float d = half_lo(hd.x), dmin = half_hi(hd.x);
    uint2 qb[4];
    qb[0] = make_uint2(wq0[s].x, wq0[s].y);
    qb[1] = make_uint2(wq0[s].z, wq0[s].w);
    qb[2] = make_uint2(wq1[s].x, wq1[s].y);
    qb[3] = make_uint2(wq1[s].z, wq1[s].w);
    half8_t alo[4], ahi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      alo[j] = *reinterpret_cast<const half8_t *>(&xa_src[32 * j + 4 * g]);
      ahi[j] = *reinterpret_cast<const half8_t *>(&xa_src[32 * j + 16 + 4 * g]);
    }
    floatx4 dlo[4], dhi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t s0 = qb[j].x >> 8, s1 = qb[j].y >> 8;
      uint4 blo, bhi;
      blo.x = code_operand_pair<NC>(qb[j].x, 0x000F000Fu); blo.y = code_operand_pair<NC>(s0, 0x000F000Fu);
      blo.z = code_operand_pair<NC>(qb[j].y, 0x000F000Fu); blo.w = code_operand_pair<NC>(s1, 0x000F000Fu);
      bhi.x = code_operand_pair<NC>(qb[j].x, 0x00F000F0u); bhi.y = code_operand_pair<NC>(s0, 0x00F000F0u);
      bhi.z = code_operand_pair<NC>(qb[j].y, 0x00F000F0u); bhi.w = code_operand_pair<NC>(s1, 0x00F000F0u);
      dlo[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          alo[j], __builtin_bit_cast(half8_t, blo), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      dhi[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          ahi[j], __builtin_bit_cast(half8_t, bhi), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    // sub-block 2j (low nibbles, q * 2^-c) weighs sc, 2j+1 (16q * 2^-c) sc/16
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t scw = j < 2 ? sc03 : sc47;
      const float sl = (float)((scw >> (16 * (j & 1))) & 0xFFu);
      const float shh = (float)((scw >> (16 * (j & 1) + 8)) & 0xFFu) * 0.0625f;
      c0 = __builtin_fmaf(sl, dlo[j][0] + dlo[j][1], __builtin_fmaf(shh, dhi[j][0] + dhi[j][1], c0));
      c1 = __builtin_fmaf(sl, dlo[j][2] + dlo[j][3], __builtin_fmaf(shh, dhi[j][2] + dhi[j][3], c1));
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
    // the next staging overwrites this slot's activations only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  int lb = wave;
#pragma unroll
  for (int s = 0; s < D; ++s, lb += W) load_unit(s, lb, s < nt);
  for (int u0 = 0; u0 < nt; u0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (u0 + s < nt) compute(s);  // wave-uniform
      load_unit(s, lb, u0 + s + D < nt);  // always issued: equal loads in flight on every path
      lb += W;
    }
  }

  // Lane (n, g) holds tokens 2g and 2g+1 of row n (lane groups past the
  // launch's tokens hold repeats and write nothing); sum the waves.
  if (2 * g < T) part[wave][2 * g][n] = y0;
  if (2 * g + 1 < T) part[wave][2 * g + 1][n] = y1;
  __syncthreads();
  if (tid < T * kTileRows) {
    const int t = tid >> 4, r = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) v += part[k][t][r];
    const int row = rg * kTileRows + r;
    if (t < M && row < N) Y[(int64_t)t * N + row] = v;
  }
}

// Prefill on tiled weights, 64 rows (4 row groups) x 16 tokens per
// workgroup: the 64-row prefill tiles of q4k_prefill.hip (the same
// arithmetic: A = sc*q exact in fp16, activations split into fp16 hi + lo,
// d applied per block, the lazy-dmin term on the fp32 MFMA) with the
// weights no longer staged through LDS.  Wave (bb, half) computes
// super-block bb of each 4-super-block stage for row groups 2 half and
// 2 half + 1, as in q4k_prefill.hip.  It loads its tiles straight into
// registers one stage ahead (its A operand bytes are its own 16-byte slots)
// and decodes its rows' headers in registers; only the activations go
// through LDS.  (Narrower tiles, and 64-row tiles from input_dim 8192 on,
// run q4k_prefill.hip's kernel on the tiled order instead: measured faster
// there.)

// A 16-byte tile load, cached (REUSE) or streaming.
template <bool REUSE>
__device__ __forceinline__ uint4 load_tile16(__amdgpu_buffer_rsrc_t r, int off, int soff) {
  if constexpr (REUSE) return __builtin_bit_cast(uint4, load_buf_f4(r, off, soff));
  else return load_buf_stream16(r, off, soff);
}

constexpr int TP_ROWS = 64;   // weight rows per workgroup
constexpr int TP_TOK = 16;    // tokens per workgroup (one MFMA token tile)
constexpr int TP_BLKS = 4;    // super-blocks per stage
constexpr int TP_WAVES = 8;
constexpr int TP_XROW = 128 + 4;  // LDS dwords per staged activation row (+ 16 B)

// REUSE: more than one token group reads each weight tile, so the tiles are
// loaded as ordinary cached loads that the later groups find in L2 (64
// tokens x 4096 -> 4096 measured 15.0 us with streaming loads, 13.7
// cached); a single token group streams them (10.0 vs 10.3 us at 16 tokens).
template <bool REUSE>
__global__ __launch_bounds__(64 * TP_WAVES) void q4k_prefill_tiled_kernel(
    const float *X, const uint8_t *wt, float *__restrict__ Y, int M, int nb, int N) {
  constexpr int ROWS = TP_ROWS;
  constexpr int RT = ROWS / 16;  // row groups per workgroup
  constexpr int TPW = 2;         // row groups per wave
  constexpr int NJ = 4;          // sub-block pairs per wave
  __shared__ __align__(16) uint32_t xh[TP_BLKS][TP_TOK][TP_XROW];
  __shared__ __align__(16) uint32_t xl[TP_BLKS][TP_TOK][TP_XROW];
  __shared__ __align__(16) float dtab[TP_WAVES][TPW][16];
  __shared__ int xe[TP_BLKS][TP_TOK];  // scaling exponent per (block, token) of the stage

  __builtin_assume(nb >= 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bb = wave & 3;     // super-block of the stage this wave computes
  const int half = wave >> 2;
  const int rt0 = 2 * half;    // first row group of this wave
  const int r = lane & 15;     // A: row within a row group; B and D: token
  const int g = lane >> 4;
  const int t = tid & 255;
  const int NG = (N + kTileRows - 1) / kTileRows;
  const int rg0 = blockIdx.x * RT;
  const int tok0 = blockIdx.y * TP_TOK;
  const int K = nb * 256;
  const int n_stages = (nb + TP_BLKS - 1) / TP_BLKS;

  // the workgroup's (up to) RT row groups, one contiguous tile stream
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(
      wt + (int64_t)rg0 * nb * kTileBytes, (int64_t)min(RT, NG - rg0) * nb * kTileBytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);
  constexpr int kPastEnd = 0x7FFFF000;

  // qs half hs of a tile at 1024 hs + 16 lane, the header at 2048 + 16 r
  const int vq[2] = {16 * lane, 1024 + 16 * lane};
  const int vhd = 2048 + 16 * r;
  uint4 qs[2][TPW][2], hd[2][TPW];  // [buffer][row group a][qs half]
  float4 xv[8];
  const int tok_lo = tid >> 8;
  // activations: wave w stages block w % 4 of the stage for the tokens of
  // parity w / 4, lane (token 2 (lane / 8) + w / 4, column j = lane % 8)
  // taking positions 32c + 4j .. +3 of the block (c = 0..7): a token's 8
  // lanes read whole 128-byte lines and hold its whole block
  const int xb = t >> 6;
  const int xj = (t & 63) & 7;
  const int xtok = 2 * ((t & 63) >> 3) + tok_lo;
  const int xoff = 4 * K * xtok + 1024 * xb + 16 * xj;
  auto load_stage = [&](int st, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int c = 0; c < 8; ++c) xv[c] = load_buf_f4(xr, xoff + 128 * c, 4096 * st);
    const int b = st * TP_BLKS + bb;
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      const int off = b < nb ? ((rt0 + a) * nb + b) * kTileBytes : kPastEnd;
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) qs[buf][a][hs] = load_tile16<REUSE>(wr, vq[hs], off);
      hd[buf][a] = load_tile16<REUSE>(wr, vhd, off);
    }
  };
  auto stage_x = [&]() {
    // As in the canonical prefill, each token's block is first scaled by the
    // power of two that puts its largest |x| (a chain over the lane's 32
    // values, then a maximum over its 8 lanes) into [2^14, 2^15); halves
    // stored as pairs (0,2) and (1,3): operand order.
    float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
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
    for (int c = 0; c < 8; ++c) {
      uint2 h, l;
      split_pair(xv[c].x, xv[c].z, sdown, h.x, l.x);
      split_pair(xv[c].y, xv[c].w, sdown, h.y, l.y);
      *reinterpret_cast<uint2 *>(&xh[xb][xtok][2 * (xj + 8 * c)]) = h;
      *reinterpret_cast<uint2 *>(&xl[xb][xtok][2 * (xj + 8 * c)]) = l;
    }
  };

  floatx4 y_acc[TPW], m_acc[TPW];
#pragma unroll
  for (int a = 0; a < TPW; ++a) y_acc[a] = m_acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  half8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  const uint32_t hi64 = vgpr_const(0x64006400u);

  auto compute = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // headers of row r of this wave's row groups: the packed fp16 (mul, add)
    // pairs of its sub-blocks, dmin*m of sub-blocks g and 4 + g (the lazy-
    // dmin MFMA's A operand), and d into the wave's table for the D rows
    uint32_t ma[TPW][2 * NJ];  // by the wave's own sub-block index
    float cm[TPW][2];
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      const uint4 h = hd[buf][a];
      const float d = half_lo(h.x), dmin = half_hi(h.x);
      const uint32_t sc03 = h.y & 0x3F3F3F3Fu;
      const uint32_t mn03 = h.z & 0x3F3F3F3Fu;
      const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
      const uint32_t mn47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
      for (int ls = 0; ls < 2 * NJ; ++ls) {  // sub-block ls
        const uint32_t scw = ls < 4 ? sc03 : sc47;
        // even sub-blocks are low nibbles, odd ones high nibbles (16 v)
        ma[a][ls] = scale_pair((scw >> (8 * (ls & 3))) & 255u, ls & 1);
      }
      cm[a][0] = dmin * (float)((mn03 >> (8 * g)) & 255u);  // sub-block g
      cm[a][1] = dmin * (float)((mn47 >> (8 * g)) & 255u);  // sub-block 4 + g
      dtab[wave][a][r] = d;  // the four lane groups write the same value
    }
    floatx4 acc[TPW];
#pragma unroll
    for (int a = 0; a < TPW; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
    float xsb[2] = {0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = jj;
      uint2 qb[TPW];
#pragma unroll
      for (int a = 0; a < TPW; ++a) {
        const uint4 v = qs[buf][a][jj >> 1];
        qb[a] = (jj & 1) ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int sb = 2 * j + hh;
        const half8_t Bh = *reinterpret_cast<const half8_t *>(&xh[bb][r][16 * sb + 4 * g]);
        const half8_t Bl = *reinterpret_cast<const half8_t *>(&xl[bb][r][16 * sb + 4 * g]);
        half8_t A[TPW];
#pragma unroll
        for (int a = 0; a < TPW; ++a)
          A[a] = dequant8_ma(qb[a].x, qb[a].y, hh != 0, ma[a][2 * jj + hh], hi64);
        floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int a = 0; a < TPW; ++a)
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bh, acc[a], 0, 0, 0);
        sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bl, sx, 0, 0, 0);
#pragma unroll
        for (int a = 0; a < TPW; ++a)
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[a], Bl, acc[a], 0, 0, 0);
        // sum of x over sub-block sb for token r (every row of the tile)
        if ((sb & 3) == g) xsb[sb >> 2] = sx[0];
      }
    }
    // d of the D rows 4g + e, written above by this wave's lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // token r (this lane's D column) entered block bb as x * 2^-e
    const int er = xe[bb][r];
    const float xs0 = __builtin_ldexpf(xsb[0], er), xs1 = __builtin_ldexpf(xsb[1], er);
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      const float4 dv = *reinterpret_cast<const float4 *>(&dtab[wave][a][4 * g]);
      y_acc[a][0] += __builtin_ldexpf(dv.x * acc[a][0], er);
      y_acc[a][1] += __builtin_ldexpf(dv.y * acc[a][1], er);
      y_acc[a][2] += __builtin_ldexpf(dv.z * acc[a][2], er);
      y_acc[a][3] += __builtin_ldexpf(dv.w * acc[a][3], er);
      // lazy-dmin term: A[row][kk] = dmin*m of sub-block 4c + kk, B = sums
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        m_acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(cm[a][c], c ? xs1 : xs0, m_acc[a], 0, 0, 0);
      }
    }
    // the next block's d values overwrite the table only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // The token groups of a row tile start at different stages (and wrap).
  // Two stages per trip, so that each tile buffer is a fixed set of
  // registers.
  const int st0 = blockIdx.y % n_stages;
  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int st = st0 + it < n_stages ? st0 + it : st0 + it - n_stages;
    stage_x();
    __syncthreads();
    // the next stage's loads leave after the barrier (measured faster than
    // before it for 64-row tiles, as for the canonical prefill)
    if (it + 1 < n_stages)
      load_stage(st + 1 < n_stages ? st + 1 : 0, std::integral_constant<int, buf ^ 1>());
    if (st * TP_BLKS + bb < nb) compute(bufc);  // wave-uniform
    __syncthreads();  // the next stage overwrites the activation tiles
  };
  load_stage(st0, std::integral_constant<int, 0>());
  for (int it = 0; it < n_stages; it += 2) {
    step(it, std::integral_constant<int, 0>());
    if (it + 1 >= n_stages) break;
    step(it + 1, std::integral_constant<int, 1>());
  }

  // Add the waves' partial tiles (through the activation tiles, no longer
  // needed) and store.  Lane (token r, group g) holds rows 16 (rt0 + a) +
  // 4g + e of its token; partial slot bb of the rows.
  constexpr int RROW = ROWS + 4;
  // [block][token][RROW]
  float *red = reinterpret_cast<float *>(&xh[0][0][0]);
  static_assert(TP_BLKS * TP_TOK * RROW <= TP_BLKS * TP_TOK * TP_XROW,
                "the partial tiles must fit in the activation tiles");
#pragma unroll
  for (int a = 0; a < TPW; ++a)
    *reinterpret_cast<float4 *>(&red[(bb * TP_TOK + r) * RROW + 16 * (rt0 + a) + 4 * g]) =
        make_float4(y_acc[a][0] - m_acc[a][0], y_acc[a][1] - m_acc[a][1],
                    y_acc[a][2] - m_acc[a][2], y_acc[a][3] - m_acc[a][3]);
  __syncthreads();
  for (int o = tid; o < TP_TOK * ROWS; o += 64 * TP_WAVES) {
    const int tok = o / ROWS, rr = o % ROWS;
    float v = 0.f;
#pragma unroll
    for (int b = 0; b < TP_BLKS; ++b) v += red[(b * TP_TOK + tok) * RROW + rr];
    const int row = rg0 * kTileRows + rr;
    if (tok0 + tok < M && row < N) Y[(int64_t)(tok0 + tok) * N + row] = v;
  }
}

hipError_t prefill_tiled_launch_64(const float *X, const uint8_t *wt, int64_t M, int64_t nb,
                                   int64_t N, float *Y, hipStream_t stream) {
  const int64_t NG = (N + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)((NG + TP_ROWS / 16 - 1) / (TP_ROWS / 16)),
                  (unsigned)((M + TP_TOK - 1) / TP_TOK));
  if (grid.y > 65535) return hipErrorInvalidConfiguration;
  if (grid.y > 1)
    hipLaunchKernelGGL(q4k_prefill_tiled_kernel<true>, grid, dim3(64 * TP_WAVES), 0, stream, X,
                       wt, Y, (int)M, (int)nb, (int)N);
  else
    hipLaunchKernelGGL(q4k_prefill_tiled_kernel<false>, grid, dim3(64 * TP_WAVES), 0, stream, X,
                       wt, Y, (int)M, (int)nb, (int)N);
  return hipGetLastError();
}

template <int W, int D, int CAP>
hipError_t launch_tiled(const float *x, const uint8_t *wt, float *y, int64_t nb, int64_t N,
                        int rg, hipStream_t stream) {
  const int64_t NG = (N + kTileRows - 1) / kTileRows;
  const int64_t grid = (NG + rg - 1) / rg;
  // Per-wave staging measured faster only for long rows (14336 -> 4096:
  // 8.67 vs 9.02 us/call); with 16 super-blocks per row the cooperative
  // staging, which overlaps the first tiles' loads, wins by 0.1 - 0.35 us.
  if (CAP > 16 && nb > 16 && nb % W == 0 && nb <= CAP)
    hipLaunchKernelGGL((q4k_gemv_tiled_kernel<W, D, CAP, CAP != 16, false>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, wt, y, (int)nb, (int)N, rg);
  else if (CAP > 16 && nb > kNormalCodesAbove)
    hipLaunchKernelGGL((q4k_gemv_tiled_kernel<W, D, CAP, false, CAP != 16>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, wt, y, (int)nb, (int)N, rg);
  else
    hipLaunchKernelGGL((q4k_gemv_tiled_kernel<W, D, CAP, false, false>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, wt, y, (int)nb, (int)N, rg);
  return hipGetLastError();
}

}  // namespace

int64_t tiled_bytes(int64_t nb, int64_t N) {
  return (N + kTileRows - 1) / kTileRows * nb * kTileBytes;
}

hipError_t relayout_tiled_launch(const uint8_t *w, uint8_t *out, int64_t nb, int64_t N,
                                 hipStream_t stream) {
  const int64_t n_chunks = tiled_bytes(nb, N) / 16;
  const int64_t grid = (n_chunks + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(q4k_relayout_tiled_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w,
                     out, nb, N, n_chunks);
  return hipGetLastError();
}

// Measured on MI355X (graph-replayed calls over rotating tiled copies,
// sweeping waves x row groups x depth): the best grid holds one workgroup
// per CU or just under (ceil(row groups / 256) groups per workgroup), and
// the wave count follows the tiles per workgroup: up to 16 tiles, 4 waves
// with 4 tiles ahead; more, 8 waves with 2 ahead.  us/call, canonical auto
// vs tiled chosen: 4096x4096 4.60 / 4.32, 4096->14336 10.79 / 8.07,
// 14336->4096 11.81 / 9.26, 11008->4096 11.69 / 8.09, 4096->11008 8.80 /
// 6.92, 2048->8192 4.78 / 4.42.
TiledShape choose_tiled_shape(int64_t nb, int64_t N, int waves, int row_groups, int depth) {
  TiledShape s;
  const int64_t NG = (N + kTileRows - 1) / kTileRows;
  s.row_groups = row_groups ? row_groups
                            : (int)std::min<int64_t>(kMaxRowGroups, std::max<int64_t>(1, (NG + 255) / 256));
  const bool few = (int64_t)s.row_groups * nb <= 16;
  s.waves = waves ? waves : (few ? 4 : 8);
  s.depth = depth ? depth : (s.waves == 4 ? 4 : 2);
  return s;
}

hipError_t gemv_tiled_launch(const float *x, const uint8_t *wt, float *y, int64_t nb, int64_t N,
                             const TiledShape &s, hipStream_t stream) {
  const int64_t NG = (N + kTileRows - 1) / kTileRows;
  // Offsets formed in the kernel: a workgroup's tiles stay below the
  // past-the-end offset its idle loads use (and the activations below 2^31).
  if (NG > 0x7FFFFFFF || (int64_t)s.row_groups * nb * kTileBytes > 0x7FFF0000 ||
      s.row_groups < 1 || s.row_groups > kMaxRowGroups)
    return hipErrorInvalidValue;
  const bool small = nb <= 16;
#define Q4K_TILED_CASE(W_, D_)                                                            \
  if (s.waves == W_ && s.depth == D_)                                                     \
    return small ? launch_tiled<W_, D_, 16>(x, wt, y, nb, N, s.row_groups, stream)        \
                 : launch_tiled<W_, D_, 64>(x, wt, y, nb, N, s.row_groups, stream);
  Q4K_TILED_CASE(4, 2)
  Q4K_TILED_CASE(4, 4)
  Q4K_TILED_CASE(8, 2)
  Q4K_TILED_CASE(8, 4)
  Q4K_TILED_CASE(16, 2)
#undef Q4K_TILED_CASE
  return hipErrorInvalidValue;
}

hipError_t gemv_tiled_batch_launch(const float *X, const uint8_t *wt, float *Y, int64_t M,
                                   int64_t nb, int64_t N, hipStream_t stream) {
  // Offsets formed in the kernel: a row group's tiles and 8 token rows of X
  // stay below the past-the-end offset.
  if (M < 1 || M > 8 || N > 0x7FFFFFFF || nb * kTileBytes > 0x7FFF0000 ||
      (int64_t)8 * nb * 1024 + 1024 * nb > 0x7FFF0000)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + kTileRows - 1) / kTileRows));
  constexpr int W = 8, D = 2;
  const bool nc = nb > kNormalCodesAbove;
#define Q4K_TBATCH_CASE(T_)                                                                 \
  if (nc)                                                                                   \
    hipLaunchKernelGGL((q4k_gemv_tiled_batch_kernel<T_, W, D, true>), grid, dim3(64 * W), 0,  \
                       stream, X, wt, Y, (int)M, (int)nb, (int)N);                          \
  else                                                                                      \
    hipLaunchKernelGGL((q4k_gemv_tiled_batch_kernel<T_, W, D, false>), grid, dim3(64 * W), 0, \
                       stream, X, wt, Y, (int)M, (int)nb, (int)N);
  if (M <= 2) {
    Q4K_TBATCH_CASE(2)
  } else if (M <= 4) {
    Q4K_TBATCH_CASE(4)
  } else {
    Q4K_TBATCH_CASE(8)
  }
#undef Q4K_TBATCH_CASE
  return hipGetLastError();
}

hipError_t prefill_tiled_launch(const float *X, const uint8_t *wt, int64_t M, int64_t nb,
                               int64_t N, float *Y, hipStream_t stream, int rows) {
  // Offsets formed in the kernel: four row groups' tiles, and 16 rows of X
  // plus one stage, stay below the past-the-end offset.
  if (4 * nb * kTileBytes > 0x7FFF0000 || ((int64_t)TP_TOK * nb * 256 + 2048) * 4 > 0x7FFF0000 ||
      N > 0x7FFFFFFF || M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  if (rows == 0) rows = prefill_rows(M, N);
  if (rows != 64 && rows != 32 && rows != 16) return hipErrorInvalidValue;
  // The canonical prefill kernel staging whole tiles through LDS, or this
  // file's kernel loading each wave's tiles into registers: measured on
  // MI355X (graph-replayed calls, register / staged us/call), staging wins
  // at 32 and 16 rows (16 tokens: 4096x4096 10.0 / 9.1, 14336->4096 30.8 /
  // 25.7; 32 tokens 14336->4096 36.7 / 32.6) and at 64 rows from input_dim
  // 8192 on (8192->4096 27.0 / 26.1, 14336->4096 46.4 / 43.9), registers at
  // 64 rows below it (4096x4096 13.7 / 14.5, 2048->8192 14.7 / 16.0).
  if (rows < 64 || nb >= 32)
    return prefill_staged_tiled_launch(X, wt, M, nb * 256, N, Y, stream, rows);
  return prefill_tiled_launch_64(X, wt, M, nb, N, Y, stream);
}

}  // namespace q4k
