// Device-side helpers shared by the HIP translation units of libmuon.so
// (gfx950, CDNA4, wave64): element types, bf16 conversions with
// round-to-nearest-even, the weight step with (cautious) decay, streaming
// accesses and a compile-time loop.  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <cstring>
#include <utility>

#include "muon_kernels.h"

namespace muon {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Kernel arguments are read in place from the kernarg segment: indexing a
// per-matrix table with the matrix index must not copy the table to scratch.
template <typename Arg>
__device__ __forceinline__ const __attribute__((address_space(4))) Arg& kernarg() {
  return *(const __attribute__((address_space(4))) Arg*)__builtin_amdgcn_kernarg_segment_ptr();
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return static_cast<bf16_t>(x);  // v_cvt_pk_bf16_f32: round to nearest even
}

// x as the sum of two bf16 values: hi = bf16(x), lo = bf16(x - hi) (the
// difference is exact in fp32), 16 significant bits in all.  (A's residual
// in the Q A Q Gram steps.)
__device__ __forceinline__ void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
  hi = from_f32<bf16_t>(x);
  lo = from_f32<bf16_t>(x - to_f32(hi));
}

// The X state of the bf16 path between Newton-Schulz steps: hi = bf16(x) and
// one signed byte q, x - hi in units of 1/256 of hi's bf16 spacing.  With
// hi = f * 2^e, f in [0.5, 1) (frexp), the spacing is 2^(e - 8) and the unit
// 2^(e - 16):
//   q = round((x - hi) * 2^(16 - e)) (to nearest even), clamped to [-128, 127],
//   x = hi + q * 2^(e - 16) to within 2^(e - 17), ulp/512,
// 16 significant bits, as hi + bf16(x - hi) would hold, in 3 bytes instead
// of 4.  |x - hi| <= ulp/2, so only q = 128 is clamped (x - hi within ulp/512
// below +ulp/2, about one element in 512; error up to ulp/256).  The decode
// takes the unit from hi's exponent bits, so a zero or subnormal hi (|x| <
// 2^-126, outside the library's input range) comes back as hi, and a
// non-finite x as NaN (as hi + bf16(x - hi) did).  The encode is a frexp, an
// ldexp, a clamp and an add; the decode a mask, a multiply and an fma.
__device__ __forceinline__ unsigned lo8_of(float x, float hi) {
  const int e = __builtin_amdgcn_frexp_expf(hi);
  const float q = __builtin_fminf(
      __builtin_fmaxf(__builtin_amdgcn_ldexpf(x - hi, 16 - e), -128.f), 127.f);
  // round to nearest even by adding 1.5 * 2^23: the sum's low mantissa bits
  // are the rounded integer, its low byte q's two's complement byte
  return __float_as_uint(q + 0x1.8p23f) & 0xffu;
}
// x from hi and the signed byte q: the unit 2^(e - 16) is hi's exponent
// bits times 2^-15 (0 for a zero or subnormal hi, whose q is then ignored)
__device__ __forceinline__ float lo8_x(float hi, int q) {
  return __builtin_fmaf((float)q, __uint_as_float(__float_as_uint(hi) & 0x7f800000u) * 0x1p-15f,
                        hi);
}
// the signed byte b (0..3) of a packed word
__device__ __forceinline__ int lo8_byte(unsigned w, int b) {
  return (int)(w << (24 - 8 * b)) >> 24;
}

// One weight element: W' = W + wscale*x (wscale = -lr*scale, x the update
// direction), minus lr*wd*W where the decay applies: everywhere, or with
// the cautious decay (web3.cnoyu.systems review of karpathy/autoresearch's
// train.py, paragraph after the Muon one) only where x*W >= 0.  neg_lrwd = -lr*wd; with 0
// the decay term is skipped (so that non-finite weights propagate as in the
// plain update).
__device__ __forceinline__ float weight_step(float w, float x, float wscale, float neg_lrwd,
                                             int cautious) {
  const float nw = fmaf(wscale, x, w);
  const bool decay = neg_lrwd != 0.f && (!cautious || x * w >= 0.f);
  return decay ? fmaf(neg_lrwd, w, nw) : nw;
}

// Streaming (nontemporal) loads and stores, for data that a launch touches
// once: the X state in the update and final epilogues and in NorMuon's
// weight pass, the weights, and the gradient, momentum and X_0 of prep.
// Kept out of the caches, they leave L2 to the operand panels that the GEMM
// main loops re-read.  The UPDATE / FINAL and prep kernels take them (STRM)
// for groups whose X state is larger than the last-level cache; smaller
// groups keep X cached for the next launch.
template <typename V>
__device__ __forceinline__ V ld_nt(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void st_nt(V v, V* p) { __builtin_nontemporal_store(v, p); }

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>), so that
// register arrays are never indexed at run time (which would put them in
// scratch memory).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace muon
