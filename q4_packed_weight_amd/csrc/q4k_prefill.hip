// q4k_prefill.hip -- batched (prefill) Q4_K product Y = X W^T on gfx950 MFMA.
//
// What it computes: for every token row r, the same lazy-dmin sum as the
// GEMV (Q4_K page: SKaiNET PR #562, "feat(kernel): SIMD-fused Q4_K matmul
// kernel + Q4KMatmulKernel SPI", sections "Summary" and "Pipeline"),
//     Y[r, o] = sum_b d[o,b] * sum_s sc[o,b,s] * sum_l q * X[r, k]
//             - sum_b dmin[o,b] * sum_s m[o,b,s] * sum_l X[r, k]
// with every weight tile read once for all tokens of the call (the tiling
// page: llama.cpp fork PR #37, "ggml-cpu: cache-aware tiling in
// ggml_compute_forward_mul_mat", section "Summary", fix 1).
//
// Work decomposition (MI355X): a workgroup of 4 waves owns 128 weight rows
// (8 MFMA row tiles of 16), PF_KB super-blocks of input_dim and up to 64
// tokens (4 MFMA column tiles); input_dim is split across workgroups so that
// no CU has to pull the whole activation matrix out of L2 (a CU reads L2 at
// roughly 120 GB/s, so 1 MB of activations per CU would cost ~8 us).
// Partial results are added into Y with fp32 atomics after a zero fill, so
// the low bits of Y can depend on the order in which the splits land
// (results are exact whenever the arithmetic is, e.g. integer inputs).
//
// Precision: the A operand is the exact integer sc*q (<= 945) in fp16.  The
// activations are split into fp16 hi + lo (hi = fp16(x), lo = fp16(x - hi)),
// two MFMAs per tile, so every product is exact and the MFMA's fp32
// accumulation gives fp32-level results (|x| must stay below 65504).  A
// k-step of 32 is exactly one sub-block; the 8 sub-blocks of a super-block
// accumulate into one tile that is scaled by d once per super-block.  The
// lazy-dmin term sum_s (dmin*m_s) * (sum of x over sub-block s) is itself a
// small contraction and runs on the fp32 MFMA (16x16x4) with exact fp32
// operands.
#include "device_common.h"
#include "q4k_internal.h"

namespace q4k {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBlockBytes = 144;
constexpr int PF_ROWS = 128;   // weight rows per workgroup
constexpr int PF_KB = 2;       // super-blocks of input_dim per workgroup
constexpr int PF_TOK = 64;     // tokens per workgroup
constexpr int PF_THREADS = 256;
constexpr int CH_PER_ROW = PF_KB * 9;                 // 16-byte chunks per row piece
constexpr int W_CHUNKS = PF_ROWS * CH_PER_ROW;        // 2304
constexpr int W_PER_THREAD = W_CHUNKS / PF_THREADS;   // 9
static_assert(W_CHUNKS % PF_THREADS == 0, "tile must divide evenly");

// The 8 activations a lane feeds to one MFMA are positions 8g + perm[e] of a
// sub-block, in the order the weight side produces its fp16 pairs:
// (byte0, byte2), (byte1, byte3), (byte4, byte6), (byte5, byte7).
__device__ constexpr int kPerm[8] = {0, 2, 1, 3, 4, 6, 5, 7};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Eight codes of one sub-block as fp16 sc*q: `p` holds 1024 + q pairs built
// with the 0x6400 exponent bias; fma(1024+q, sc, -1024*sc) = sc*q exactly.
__device__ __forceinline__ half8_t dequant8(uint32_t p0, uint32_t p1, uint32_t p2,
                                            uint32_t p3, half2_t sc, half2_t nsc) {
  const half2_t a = __builtin_elementwise_fma(as_h2(p0), sc, nsc);
  const half2_t b = __builtin_elementwise_fma(as_h2(p1), sc, nsc);
  const half2_t c = __builtin_elementwise_fma(as_h2(p2), sc, nsc);
  const half2_t d = __builtin_elementwise_fma(as_h2(p3), sc, nsc);
  half8_t r;
  r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
  r[4] = c.x; r[5] = c.y; r[6] = d.x; r[7] = d.y;
  return r;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ y, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) y[i] = 0.f;
}

__global__ __launch_bounds__(PF_THREADS) void q4k_prefill_kernel(
    const float *X, const uint8_t *w, float *__restrict__ Y, int M, int nb,
    int N) {
  // LDS: weight tile (row r, block kb at chunks (r*PF_KB + kb)*9 ..), the
  // activation fragments of one super-block [s][token tile][hi|lo][lane],
  // sub-block activation sums, and the decoded block headers.
  __shared__ uint4 wt[W_CHUNKS];
  __shared__ uint4 bfrag[8][4][2][64];
  __shared__ float xs_tab[8][PF_TOK];
  __shared__ float d_tab[PF_KB][PF_ROWS];
  __shared__ float c_tab[PF_KB][8][PF_ROWS];
  __shared__ uint32_t sc_tab[PF_KB][8][PF_ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * PF_ROWS;
  const int kb0 = blockIdx.y * PF_KB;
  const int tok0 = blockIdx.z * PF_TOK;
  const int K = nb * 256;
  const int64_t row_bytes = (int64_t)nb * kBlockBytes;

  // Range-checked views: rows past N and tokens past M read as zeros.
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w + (int64_t)row0 * row_bytes, (int64_t)(N - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)tok0 * K, (int64_t)(M - tok0) * K * 4);

  // 1. Weight tile: each row's PF_KB blocks are one contiguous 288-byte
  //    piece; chunk q = row (q / CH_PER_ROW), piece chunk (q % CH_PER_ROW).
  //    Blocks past nb read the next row's bytes and are never consumed.
  uint4 wv[W_PER_THREAD];
#pragma unroll
  for (int m = 0; m < W_PER_THREAD; ++m) {
    const int q = tid + PF_THREADS * m;
    const int r = q / CH_PER_ROW;
    const int within = q - r * CH_PER_ROW;
    wv[m] = load_buf_stream16(wr, (int)(r * row_bytes) + kb0 * kBlockBytes + 16 * within);
  }

  // Activation staging roles: thread -> token tok = tid / 4, group g = tid % 4
  // (positions 8g..8g+7 of every sub-block).
  const int s_tok = tid >> 2;
  const int s_g = tid & 3;

  float4 xv[16];
  auto load_x = [&](int kb) {
    const int kbase = (kb0 + kb) * 256;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int off = 4 * (s_tok * K + kbase + 32 * s + 8 * s_g);
      xv[2 * s] = load_buf_f4(xr, off);
      xv[2 * s + 1] = load_buf_f4(xr, off + 16);
    }
  };
  auto stage_x = [&]() {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float v[8] = {xv[2 * s].x, xv[2 * s].y, xv[2 * s].z, xv[2 * s].w,
                          xv[2 * s + 1].x, xv[2 * s + 1].y, xv[2 * s + 1].z, xv[2 * s + 1].w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a = v[kPerm[e]], b = v[kPerm[e + 1]];
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
        half2_t h2, l2;
        h2.x = ha; h2.y = hb;
        l2.x = la; l2.y = lb;
        hi[e / 2] = as_u32(h2);
        lo[e / 2] = as_u32(l2);
      }
      const int flane = 16 * s_g + (s_tok & 15);
      bfrag[s][s_tok >> 4][0][flane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      bfrag[s][s_tok >> 4][1][flane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      // sub-block activation sum over the 4 groups of this token
      float part = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      part = group_sum<4>(part);
      if (s_g == 0) xs_tab[s][s_tok] = part;
    }
  };

  load_x(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // 2. Weight tile and activations of the first block into LDS.
#pragma unroll
  for (int m = 0; m < W_PER_THREAD; ++m) wt[tid + PF_THREADS * m] = wv[m];
  stage_x();
  __syncthreads();

  // 3. Decode the PF_ROWS * PF_KB block headers once: thread -> (row, kb).
  {
    const int r = tid >> 1, kb = tid & 1;
    const uint4 h = wt[(r * PF_KB + kb) * 9];
    const float d = half_lo(h.x), dmin = half_hi(h.x);
    const uint32_t S[12] = {h.y & 255u, (h.y >> 8) & 255u, (h.y >> 16) & 255u, h.y >> 24,
                            h.z & 255u, (h.z >> 8) & 255u, (h.z >> 16) & 255u, h.z >> 24,
                            h.w & 255u, (h.w >> 8) & 255u, (h.w >> 16) & 255u, h.w >> 24};
    d_tab[kb][r] = d;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t sc = s < 4 ? (S[s] & 63u) : ((S[s + 4] & 15u) | ((S[s - 4] >> 6) << 4));
      const uint32_t mm = s < 4 ? (S[s + 4] & 63u) : ((S[s + 4] >> 4) | ((S[s] >> 6) << 4));
      c_tab[kb][s][r] = dmin * (float)mm;
      half2_t sc2;
      sc2.x = (_Float16)(float)sc;
      sc2.y = sc2.x;
      sc_tab[kb][s][r] = as_u32(sc2);
    }
  }
  __syncthreads();

  // 4. MFMA main loop.  Wave w owns row tiles 2w and 2w+1; lane l works on
  //    row l % 16 of a tile and activation group g = l / 16.
  const int lr = lane & 15;
  const int g = lane >> 4;
  floatx4 y_acc[2][4], m_acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) y_acc[a][t] = m_acc[a][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < PF_KB; ++kb) {
    if (kb0 + kb >= nb) break;  // ragged last split (uniform)
    if (kb > 0) {
      __syncthreads();  // everyone is done with the previous block's fragments
      load_x(kb);
      stage_x();
      __syncthreads();
    }
    floatx4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[a][t] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // qs bytes 32j + 8g .. +7 of each of the wave's two rows (this lane's)
      uint2 qb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int r = (2 * wave + a) * 16 + lr;
        const uint8_t *blk = reinterpret_cast<const uint8_t *>(&wt[(r * PF_KB + kb) * 9]);
        qb[a] = *reinterpret_cast<const uint2 *>(blk + 16 + 32 * j + 8 * g);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // h = 0: sub-block 2j (low nibbles), 1: 2j+1 (high)
        const int s = 2 * j + h;
        uint4 bh[4], bl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bh[t] = bfrag[s][t][0][lane];
          bl[t] = bfrag[s][t][1][lane];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int r = (2 * wave + a) * 16 + lr;
          const uint32_t w0 = h ? (qb[a].x >> 4) : qb[a].x;
          const uint32_t w1 = h ? (qb[a].y >> 4) : qb[a].y;
          const uint32_t p0 = (w0 & 0x000F000Fu) | 0x64006400u;
          const uint32_t p1 = ((w0 >> 8) & 0x000F000Fu) | 0x64006400u;
          const uint32_t p2 = (w1 & 0x000F000Fu) | 0x64006400u;
          const uint32_t p3 = ((w1 >> 8) & 0x000F000Fu) | 0x64006400u;
          const half2_t sc = as_h2(sc_tab[kb][s][r]);
          const half2_t nsc = sc * (_Float16)(-1024.0f);
          const half8_t A = dequant8(p0, p1, p2, p3, sc, nsc);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(half8_t, bh[t]), acc[a][t], 0, 0, 0);
            acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(half8_t, bl[t]), acc[a][t], 0, 0, 0);
          }
        }
      }
    }

    // Epilogue of this super-block: scale by d (per row) into y_acc, and the
    // lazy-dmin term on the fp32 MFMA: sum_s (dmin*m_s)[row] * xs[s][token].
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int rt0 = (2 * wave + a) * 16;
      float dv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[e] = d_tab[kb][rt0 + 4 * g + e];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y_acc[a][t][e] = __builtin_fmaf(dv[e], acc[a][t][e], y_acc[a][t][e]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const float ca = c_tab[kb][4 * mi + g][rt0 + lr];
          const float xb = xs_tab[4 * mi + g][16 * t + lr];
          m_acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ca, xb, m_acc[a][t], 0, 0, 0);
        }
      }
    }
  }

  // 5. Add this split's partial results into Y.  Each wave first transposes
  //    its 32 rows x 64 tokens through LDS (row stride 33 floats against
  //    bank conflicts) so that one atomic instruction covers 2 tokens x 32
  //    consecutive rows (2 cache lines) instead of 16 scattered lines.  Rows
  //    past N and tokens past M are dropped.
  __syncthreads();  // every wave is done reading the activation fragments
  float *T = reinterpret_cast<float *>(&bfrag[0][0][0][0]) + wave * (PF_TOK * 33);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        T[(16 * t + lr) * 33 + 16 * a + 4 * g + e] = y_acc[a][t][e] - m_acc[a][t][e];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
  const int rr = lane & 31;
  const int row = row0 + wave * 32 + rr;
#pragma unroll 4
  for (int i = 0; i < PF_TOK / 2; ++i) {
    const int tl = 2 * i + (lane >> 5);
    const int tok = tok0 + tl;
    const float v = T[tl * 33 + rr];
    if (tok < M && row < N) unsafeAtomicAdd(Y + (int64_t)tok * N + row, v);
  }
}

}  // namespace

hipError_t prefill_launch(const float *X, const uint8_t *w, int64_t M,
                          int64_t K, int64_t N, float *Y, hipStream_t stream) {
  const int64_t nb = K / 256;
  // Offsets formed in the kernel: row tile of 128 rows and a token group of
  // 64 rows of X must stay below 2^31 bytes.
  if ((int64_t)PF_ROWS * nb * kBlockBytes >= ((int64_t)1 << 31) ||
      (int64_t)PF_TOK * K * 4 >= ((int64_t)1 << 31) || N > 0x7FFFFFFF || M > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const int64_t total = M * N;
  int64_t fill_grid = (total + 255) / 256;
  if (fill_grid > 4096) fill_grid = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)fill_grid), dim3(256), 0, stream, Y, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + PF_ROWS - 1) / PF_ROWS), (unsigned)((nb + PF_KB - 1) / PF_KB),
                  (unsigned)((M + PF_TOK - 1) / PF_TOK));
  if (grid.y > 65535 || grid.z > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(q4k_prefill_kernel, grid, dim3(PF_THREADS), 0, stream, X, w, Y, (int)M,
                     (int)nb, (int)N);
  return hipGetLastError();
}

}  // namespace q4k
