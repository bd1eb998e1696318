// Device-side building blocks shared by the gfx950 kernels of libjetlong.
//
// Method: "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
// RoPE" (gist.science summaries of arXiv 2607.07740), section "Dynamic
// Bifocal RoPE": G = max(1, ceil(L / w_pretrained)) (eq. G), remote position
// f(x) = floor(x / G) (eq. f), classic RoPE inside the local window w0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jl {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// Two floats -> packed IEEE half (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// x rounded to IEEE half (nearest even), or NaN where x lies outside half
// range (|x| >= 65520 would round to infinity).  An operand the matrix cores
// cannot represent then poisons every result that uses it instead of
// turning it into a wrong finite value.
__device__ __forceinline__ _Float16 half_or_nan(float x) {
  return fabsf(x) < 65520.f ? static_cast<_Float16>(x) : static_cast<_Float16>(__builtin_nanf(""));
}

// Two floats -> packed half_or_nan.
__device__ __forceinline__ uint32_t pack_f16x2_or_nan(float lo, float hi) {
  const f16x2 h = {half_or_nan(lo), half_or_nan(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- rotations

// Table row and sign of sin for rotating a vector that sits at position p to
// angle position a.  Raw inputs: R(a) itself.  Inputs already rotated at p
// (a pre-rotated cache): the correction R(a - p), with R(-x) read as
// (cos x, -sin x) from row x ("On-the-Fly Correction Rotation").
struct RotRow {
  int row;
  float sgn;
};
__device__ __forceinline__ RotRow rot_row(int a, int p, bool prerot) {
  if (!prerot) return {a, 1.f};
  const int d = a - p;
  return d >= 0 ? RotRow{d, 1.f} : RotRow{-d, -1.f};
}

// ---------------------------------------------------------------- eq. G / f

// G = max(1, ceil(L / w_pretrained)), exact integers (eq. G).
__device__ __forceinline__ int group_size(int L, int w_pretrained) {
  const int64_t g = (static_cast<int64_t>(L) + w_pretrained - 1) / w_pretrained;
  return g < 1 ? 1 : static_cast<int>(g);
}

// ---------------------------------------------------------------- routing

enum : int { kSkip = 0, kLocal = 1, kRemote = 2, kStraddle = 3, kDiag = 4 };

// Class of the block of query positions [i0, i1] against key positions
// [j0, j1] (both inclusive, i0 <= i1, j0 <= j1): decided from the nearest
// and farthest causal distances, which is exactly the pair-by-pair routing of
// the local window (distance < w0 -> classic RoPE, else grouped positions).
__device__ __host__ __forceinline__ int classify_tile(int i0, int i1, int j0, int j1, int w0) {
  if (j0 > i1) return kSkip;
  const int far = i1 - j0;                 // largest causal distance
  const int near = i0 > j1 ? i0 - j1 : 0;  // smallest causal distance
  int c;
  if (far < w0) c = kLocal;
  else if (near >= w0) c = kRemote;
  else c = kStraddle;
  if (j1 > i0) c |= kDiag;                 // some key after some query
  return c;
}

}  // namespace jl
