// q4k_tiled.hip -- the tiled block order of a Q4_K matrix: the one-time
// relayout from the canonical layout, and the matrix-vector product that
// streams the tiled order.
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
// into exact fp16 subnormals, activations split into exact fp16 hi + lo
// parts (A rows of alternating parity), every 32-activation sub-block scaled
// by a power of two first, scales applied per sub-block in fp32 after the
// MFMAs.
#include <algorithm>

#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ uint32_t as_u32h(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// lo = fp16(x - hi) for the two halves of `hi2` (fp16 hi parts of x0, x1):
// v_fma_mix evaluates x - hi exactly in fp32 and rounds once to fp16.
__device__ __forceinline__ uint32_t lo_pair_t(uint32_t hi2, float x0, float x1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hi2), "v"(x0));
  asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(r) : "v"(hi2), "v"(x1));
  return r;
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
template <int W, int D, int CAP, bool PRIV>
__global__ __launch_bounds__(64 * W) void q4k_gemv_tiled_kernel(
    const float *x, const uint8_t *wt, float *__restrict__ y, int nb, int N, int rg_per_wg) {
  constexpr int XPL = CAP * 64 / (64 * W);  // activation float4 per thread per chunk
  static_assert(XPL * 64 * W == CAP * 64, "a chunk's activations must split evenly");
  __shared__ __align__(16) uint32_t xh[CAP * 128];
  __shared__ __align__(16) uint32_t xl[CAP * 128];
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

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(
      wt + (int64_t)rg0 * nb * kTileBytes, (int64_t)rgn * nb * kTileBytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)nb * 1024);
  constexpr int kPastEnd = 0x7FFFF000;  // a tile or activation offset that reads zeros

#pragma unroll
  for (int r = 0; r < kMaxRowGroups; ++r) part[wave][r][lane] = 0.f;

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
    mx = group_max<8>(mx);
    const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    const float4 v = make_float4(__builtin_ldexpf(v0.x, -e), __builtin_ldexpf(v0.y, -e),
                                 __builtin_ldexpf(v0.z, -e), __builtin_ldexpf(v0.w, -e));
    half2_t h02, h13;
    h02.x = (_Float16)v.x; h02.y = (_Float16)v.z;
    h13.x = (_Float16)v.y; h13.y = (_Float16)v.w;
    const uint32_t hw02 = as_u32h(h02), hw13 = as_u32h(h13);
    *reinterpret_cast<uint2 *>(&xh[2 * f]) = make_uint2(hw02, hw13);
    *reinterpret_cast<uint2 *>(&xl[2 * f]) =
        make_uint2(lo_pair_t(hw02, v.x, v.z), lo_pair_t(hw13, v.y, v.w));
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
      // codes enter as q * 2^-24 (low nibbles) and 16q * 2^-24 (high), the
      // activations as x * 2^-e
      const float s_lo = __builtin_ldexpf(d * (float)(scp & 0xFFu),
                                          __builtin_bit_cast(int, xsp.z) + 24);
      const float s_hi = __builtin_ldexpf(d * (float)((scp >> 8) & 0xFFu),
                                          __builtin_bit_cast(int, xsp.w) + 20);
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
        blo.x = qb[j].x & 0x000F000Fu; blo.y = s0 & 0x000F000Fu;
        blo.z = qb[j].y & 0x000F000Fu; blo.w = s1 & 0x000F000Fu;
        bhi.x = qb[j].x & 0x00F000F0u; bhi.y = s0 & 0x00F000F0u;
        bhi.z = qb[j].y & 0x00F000F0u; bhi.w = s1 & 0x00F000F0u;
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

template <int W, int D, int CAP>
hipError_t launch_tiled(const float *x, const uint8_t *wt, float *y, int64_t nb, int64_t N,
                        int rg, hipStream_t stream) {
  const int64_t NG = (N + kTileRows - 1) / kTileRows;
  const int64_t grid = (NG + rg - 1) / rg;
  // Per-wave staging measured faster only for long rows (14336 -> 4096:
  // 8.67 vs 9.02 us/call); with 16 super-blocks per row the cooperative
  // staging, which overlaps the first tiles' loads, wins by 0.1 - 0.35 us.
  if (CAP > 16 && nb > 16 && nb % W == 0 && nb <= CAP)
    hipLaunchKernelGGL((q4k_gemv_tiled_kernel<W, D, CAP, CAP != 16>), dim3((unsigned)grid),
                       dim3(64 * W), 0, stream, x, wt, y, (int)nb, (int)N, rg);
  else
    hipLaunchKernelGGL((q4k_gemv_tiled_kernel<W, D, CAP, false>), dim3((unsigned)grid),
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

}  // namespace q4k
