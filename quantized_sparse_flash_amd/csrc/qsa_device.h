// qsa_device.h -- gfx950 device helpers shared by the QSA kernels.
//
// Only the HIP library includes this header; the CPU oracle shares nothing
// with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace qsa {

constexpr int kHeadDim = 256;     // dims per head
constexpr int kHpg = 12;          // query heads per KV group
constexpr int kBlk = 64;          // dims per fp16 scale
constexpr int kNBlk = kHeadDim / kBlk;
constexpr int kChunk = 64;        // selected cells per chunk
constexpr int kRec = kHeadDim + 2;  // floats per partial record (o, m, l)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// S = 0.0625 * q.k, and the softmax runs in base 2: x = S * log2(e).
constexpr float kScoreScaleLog2 = 0.0625f * kLog2e;
// Buffer-resource word 3 for raw 32-bit loads on gfx9-family parts: the
// hardware range check then returns 0 for offsets at or past the size.
constexpr int kBufferFlags = 0x00020000;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled
// at compile time (the index stays a constant expression inside f).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] B[32x16].  Lane l holds
// A row (l % 16) and B column (l % 16), eight k values each at k slots
// selected by (l / 16, element); D element (4*(l/16) + i, l % 16) sits in
// register i of lane l.
__device__ __forceinline__ f32x4 mfma16(half8_t a, half8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// v_mfma_i32_16x16x64_i8: the same shape with 64 int8 k values, sixteen
// bytes per lane in A and B (exact int32 accumulation).  A and B hold their
// k values in the same lane and byte positions, so any fixed assignment of
// dims to those positions, used by both operands, computes the dot product.
__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ------------------------------------------------- int8 -> fp16 convert
// Two signed bytes of dwords `lo_src`/`hi_src` (byte selectors as template
// arguments) become the two halves of one packed fp16 pair.  One SDWA
// convert per element: the selected byte is sign-extended to 16 bits and
// converted exactly (|code| <= 128 is exact in fp16).
template <int BL, int BH>
__device__ __forceinline__ uint32_t i8pair_to_h2(uint32_t lo_src, uint32_t hi_src) {
  uint32_t r;
  static_assert(BL >= 0 && BL < 4 && BH >= 0 && BH < 4, "byte select");
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_%c3\n\t"
      "v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_%c4"
      : "=&v"(r)
      : "v"(lo_src), "v"(hi_src), "i"(BL), "i"(BH));  // pure: no side effects
  return r;
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// 4 codes of one dword, scaled by s (fp16 rounding of code*s), as 2 dwords.
__device__ __forceinline__ void dq4(uint32_t w, half2_t s, uint32_t& o0, uint32_t& o1) {
  o0 = as_u32(as_h2(i8pair_to_h2<0, 1>(w, w)) * s);
  o1 = as_u32(as_h2(i8pair_to_h2<2, 3>(w, w)) * s);
}

// Byte `b` (runtime-uniform constant after unrolling) of two dwords.
template <int B>
__device__ __forceinline__ half2_t col_pair(uint32_t w_lo, uint32_t w_hi) {
  return as_h2(i8pair_to_h2<B, B>(w_lo, w_hi));
}

// --------------------------------------------------------- wave helpers
// Reductions over the four lanes n, n + 16, n + 32, n + 48 on the VALU:
// v_permlane16_swap with both operands holding v leaves rows (0, 1) of v in
// one register and rows (1, 0) in the other (likewise rows 2 and 3), so
// combining the two gives every lane its xor-16 partner's value;
// v_permlane32_swap does the same for the halves.  Each lane combines the
// same pair of values in the same order, so all four lanes end with one
// result.  Written as asm: the compiler's builtin for these swaps, when
// both results feed one operation, hands that operation the first result
// twice.  The s_nops give the swap the wait states it needs after the
// copy and before its results are read.
template <bool X32>
__device__ __forceinline__ void swap_pair(float v, float& a, float& b) {
  a = v;
  if constexpr (X32)
    asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1"
        : "+v"(a), "=&v"(b));
  else
    asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1"
        : "+v"(a), "=&v"(b));
}
__device__ __forceinline__ float xor_pair_max(float v, auto x32) {
  float a, b;
  swap_pair<decltype(x32)::value>(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor_pair_sum(float v, auto x32) {
  float a, b;
  swap_pair<decltype(x32)::value>(v, a, b);
  return a + b;
}
__device__ __forceinline__ float wave_max_xor16_32(float v) {
  return xor_pair_max(xor_pair_max(v, std::false_type{}), std::true_type{});
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  return xor_pair_sum(xor_pair_sum(v, std::false_type{}), std::true_type{});
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace qsa
