// device_common.h -- small gfx950 device helpers shared by the GEMV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));  // one MFMA f16 operand
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));  // one 16x16 MFMA D tile per lane

__device__ __forceinline__ uint32_t as_u32h(half2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// The register holding c, as a value the compiler cannot see through: an
// fma by it is not folded into a plain add (which would lose the single
// v_fma_mix rounding below).
__device__ __forceinline__ float opaque_f32(float c) {
  float v = c;
  asm("" : "+v"(v));
  return v;
}

// hi = fp16(x * s) and lo = fp16(x * s - hi) for two values, s a power of
// two: each half is one v_fma_mix that evaluates the product (and the
// difference) exactly in fp32 and rounds once to fp16, so hi + lo carries
// x * s to 22 significant bits and both are exact MFMA inputs.  Written in
// C (no inline assembly) so that the compiler sees these register writes
// and keeps its matrix-core hazard waits around them.
__device__ __forceinline__ void split_pair(float x0, float x1, float s, uint32_t &hi,
                                           uint32_t &lo) {
  const _Float16 h0 = (_Float16)__builtin_fmaf(x0, s, 0.0f);
  const _Float16 h1 = (_Float16)__builtin_fmaf(x1, s, 0.0f);
  const _Float16 l0 = (_Float16)__builtin_fmaf(x0, s, -(float)h0);
  const _Float16 l1 = (_Float16)__builtin_fmaf(x1, s, -(float)h1);
  hi = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
  lo = __builtin_bit_cast(uint32_t, half2_t{l0, l1});
}

// lo = fp16(x - hi) for the two halves of `hi2` (fp16 hi parts of x0, x1):
// v_fma_mix evaluates x - hi exactly in fp32 and rounds once to fp16, so
// hi + lo carries x to 22 significant bits and both are exact MFMA inputs.
// Two instructions reading hi2's halves through op_sel (the compiler's own
// selection of the same arithmetic re-converts each half first).  Inline
// assembly gets no matrix-core hazard waits from the compiler, so this is
// for staging code that runs while no MFMA is in flight (every earlier
// MFMA result already read by ordinary code); split_pair is the form for
// code interleaved with MFMAs.
__device__ __forceinline__ uint32_t lo_pair(uint32_t hi2, float x0, float x1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hi2), "v"(x0));
  asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(r) : "v"(hi2), "v"(x1));
  return r;
}

// A three-operand AND-OR takes at most one scalar operand and no literal on
// this target, so the 0x64 bytes come from a register the caller holds
// (`hi64` = 0x64006400, made by vgpr_const).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t v = c;
  asm volatile("" : "+v"(v));
  return v;
}
// The same without volatile, for helpers called many times: the compiler
// may then share one register among all the uses of a constant.
__device__ __forceinline__ uint32_t vgpr_const_shared(uint32_t c) {
  uint32_t v = c;
  asm("" : "+v"(v));
  return v;
}

// Two codes of a qs dword as exact *normal* fp16 MFMA operands: with mask
// 0x000F000F the low nibbles of bytes 0 and 2 as q, with 0x00F000F0 their
// high nibbles, kept in place, as 16 q (shift the dword right by 8 first for
// bytes 1 and 3).  (w & mask) | 0x6400 is the fp16 number 1024 + v, and a
// packed subtraction of 1024 leaves v exactly.  Normal operands matter: with
// the codes as fp16 subnormals (v * 2^-24, only masked) the 16x16x32 f16
// MFMA measured a biased loss of up to 4e-6 of a dot whose products span a
// wide range, against about one fp32 ulp with normal codes.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t mask) {
  const half2_t v = as_h2((w & mask) | vgpr_const_shared(0x64006400u));
  return as_u32h(v - half2_t{(_Float16)1024.0f, (_Float16)1024.0f});
}

// The code operands of the matrix-core GEMV kernels.  Masked into fp16
// subnormals (v * 2^-24) a pair costs one AND; its measured bias is about
// 1.6e-7 of a dot, which stays within fp32-level error up to a few hundred
// super-blocks per row but reaches ~1e-4 at input_dim 2^24.  Rows longer
// than kNormalCodesAbove super-blocks therefore use exact normal codes
// (NC), one packed subtraction more per pair.
constexpr int kNormalCodesAbove = 256;
template <bool NC>
__device__ __forceinline__ uint32_t code_operand_pair(uint32_t w, uint32_t mask) {
  if constexpr (NC) return code_pair(w, mask);
  else return w & mask;
}
// the power of two the codes carry: a low nibble enters as q * 2^-kCodeShift,
// a high nibble in place as 16 q * 2^-kCodeShift
template <bool NC> constexpr int kCodeShift = NC ? 0 : 24;

// The packed fp16 pair (mul, add) of a sub-block with 6-bit scale sc:
// (sc, -1024 sc) for its low nibbles, (sc/16, -64 sc) for high nibbles kept
// in place.  Every value is exact in fp16 (|1024 sc| <= 64512).
__device__ __forceinline__ uint32_t scale_pair(uint32_t sc, bool odd) {
  const _Float16 f = (_Float16)(uint16_t)sc;
  const half2_t k = odd ? half2_t{(_Float16)0.0625f, (_Float16)-64.0f}
                        : half2_t{(_Float16)1.0f, (_Float16)-1024.0f};
  return as_u32h(half2_t{f, f} * k);
}

// One MFMA A operand (8 codes of one sub-block) from two qs dwords: their
// low nibbles (hi_nib false) or their high nibbles kept in place, i.e. as
// 16 v (true).  Each pair of codes is masked straight under the 0x64 high
// byte of two fp16 halves (bytes 0 and 2 of a dword in place, bytes 1 and 3
// after a shift right by 8 that a dword's low and high nibbles share), the
// fp16 number 1024 + v or 1024 + 16 v; one AND-OR per pair.  `ma` packs the
// sub-block's fp16 pair (mul, add) (scale_pair), and the fused multiply-add,
// reading each half for both lanes, turns 1024 + v into sc*v, exact in
// fp16.  Codes come out in operand order: positions (0,2), (1,3), (4,6),
// (5,7) of the 8.
__device__ __forceinline__ half8_t dequant8_ma(uint32_t w0, uint32_t w1, bool hi_nib,
                                               uint32_t ma, uint32_t hi64) {
  const uint32_t mask = hi_nib ? 0x00F000F0u : 0x000F000Fu;
  const half2_t pr = as_h2(ma);
  const half2_t m2 = {pr.x, pr.x}, a2 = {pr.y, pr.y};
  const half2_t p0 = __builtin_elementwise_fma(as_h2((w0 & mask) | hi64), m2, a2);
  const half2_t p1 = __builtin_elementwise_fma(as_h2(((w0 >> 8) & mask) | hi64), m2, a2);
  const half2_t p2 = __builtin_elementwise_fma(as_h2((w1 & mask) | hi64), m2, a2);
  const half2_t p3 = __builtin_elementwise_fma(as_h2(((w1 >> 8) & mask) | hi64), m2, a2);
  half8_t v;
  v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
  v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  return v;
}

// The two binary16 halves of a dword as fp32.  When the result feeds an FMA
// with an fp32 operand, the compiler folds the conversion into
// v_fma_mix_f32 (op_sel picks the half), so a masked nibble or 2-bit field
// sitting in a half's low bits acts as an exact fp16 subnormal
// (value * 2^-24) at no conversion cost.
__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(half2_t, v).x;
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(half2_t, v).y;
}

// Streaming (non-temporal) 16-byte load for data read exactly once.
__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 load_f4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}

// Raw buffer view of `bytes` bytes at `base` (gfx9 descriptor word 3):
// loads at offsets past the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                          int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n,
                                           0x00020000);
}

// The same view when the caller knows 0 <= bytes < 2^31: no 64-bit clamp,
// so fewer scalar instructions ahead of a kernel's first load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte loads through a buffer view at a byte offset; the streaming form
// sets the non-temporal hint (aux bit 1 on gfx94x/gfx950).
// `soff` is an optional wave-uniform part of the offset (the instruction's
// scalar offset operand).
__device__ __forceinline__ uint4 load_buf_stream16(__amdgpu_buffer_rsrc_t r, int off,
                                                   int soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_buf_f4(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float sum4(float4 v) { return (v.x + v.y) + (v.z + v.w); }

// max(m, |a|, |b|) for m >= 0: one v_maximum3_f32 with absolute-value
// modifiers (the IEEE maximum needs no NaN quieting of loaded values)
__device__ __forceinline__ float absmax3(float m, float a, float b) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(a)),
                                       __builtin_fabsf(b));
}

// Maximum of non-negative values (NaN included) over aligned groups of
// `width` lanes, every lane of the group receiving it: the maximum of the bit
// patterns as unsigned integers is the float maximum, and an integer
// maximum takes its DPP operand directly (one v_max_u32_dpp per step, where
// the float maximum needs a move and two NaN-quieting maxima besides).
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_step(uint32_t b) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, true);
  return b > o ? b : o;
}
template <int width>
__device__ __forceinline__ float group_max_nonneg(float v) {
  static_assert(width == 2 || width == 4 || width == 8 || width == 16,
                "group_max_nonneg covers 2, 4, 8 or 16 lanes");
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  b = max_dpp_step<0xB1>(b);                             // quad_perm [1,0,3,2]
  if constexpr (width >= 4) b = max_dpp_step<0x4E>(b);   // quad_perm [2,3,0,1]
  if constexpr (width >= 8) b = max_dpp_step<0x141>(b);  // row_half_mirror
  if constexpr (width >= 16) b = max_dpp_step<0x140>(b); // row_mirror
  return __builtin_bit_cast(float, b);
}

// Maximum of a non-negative value over the 64 lanes of a wave, as a
// wave-uniform value: DPP within each row of 16 lanes, then the four row
// results through scalar registers (for non-negative floats, NaN included,
// the integer order of the bit patterns is the float order); no LDS round
// trip.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = group_max_nonneg<16>(v);
  const int b = __builtin_bit_cast(int, v);
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readlane(b, 0);
  const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane(b, 16);
  const uint32_t m2 = (uint32_t)__builtin_amdgcn_readlane(b, 32);
  const uint32_t m3 = (uint32_t)__builtin_amdgcn_readlane(b, 48);
  const uint32_t m01 = m0 > m1 ? m0 : m1, m23 = m2 > m3 ? m2 : m3;
  return __builtin_bit_cast(float, m01 > m23 ? m01 : m23);
}

// The same maximum without the scalar round trip: after the 16-lane DPP
// steps, gfx950's lane-swap instructions exchange the two 32-lane halves
// (lane i with lane i ^ 32) and then neighbouring 16-lane rows (i with
// i ^ 16), each followed by an integer maximum; every lane ends with the
// wave's maximum in a vector register.
__device__ __forceinline__ float wave_max_nonneg_v(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, group_max_nonneg<16>(v));
  const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  b = h[0] > h[1] ? h[0] : h[1];
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  b = r[0] > r[1] ? r[0] : r[1];
  return __builtin_bit_cast(float, b);
}

// v + v of lane i ^ 16 (width 32) or i ^ 32 (width 64), in every lane:
// gfx950's lane-swap instructions exchange neighbouring 16-lane rows (or
// the two 32-lane halves) in a vector register, so the partner's value
// arrives without an LDS round trip; fp32 addition is commutative, so the
// bits are those of v + partner in either order.  The two results are
// copied into integers before the float conversion: this compiler turns
// __builtin_bit_cast(float, h[1]) of the swap's result pair into a second
// read of h[0] (the sum then comes out as 2 * h[0]).
template <int width>
__device__ __forceinline__ float add_partner_row(float v) {
  static_assert(width == 32 || width == 64, "rows of 16 or halves of 32 lanes");
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto h = width == 32 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                             : __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const uint32_t own_or_partner0 = h[0], own_or_partner1 = h[1];
  return __uint_as_float(own_or_partner0) + __uint_as_float(own_or_partner1);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64);
// every lane of the group receives the group sum.  Steps below 16 lanes use
// DPP quad permutes and row mirrors; the 16- and 32-lane steps use the lane
// swaps (add_partner_row).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (width >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
  if constexpr (width >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
  if constexpr (width >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)); // row_half_mirror
  if constexpr (width >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)); // row_mirror
  if constexpr (width >= 32) v = add_partner_row<32>(v);
  if constexpr (width >= 64) v = add_partner_row<64>(v);
  return v;
}

}  // namespace q4k
