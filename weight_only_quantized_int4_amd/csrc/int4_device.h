// int4_device.h -- device helpers of the MatMulNBits int4 kernels (the
// original layout in int4_gemv.hip and the load-time packed layout in
// int4_packed.hip): nibble unpack to exact fp16 (q - zp) pairs and the
// staging order of x.
#pragma once

#include "qgemv_device.h"

namespace qg {

struct Pairs8 {
  f16x2 a, b, c, d;  // (e0,e4)-zp, (e1,e5)-zp, (e2,e6)-zp, (e3,e7)-zp
};

// Eight 4-bit codes of one 32-bit word (element 2i in the low nibble of byte
// i) -> four exact fp16 pairs of (code - zero point).  `magic` is fp16 1024.0
// in both halves, held in a VGPR so that each mask-and-or is one v_and_or_b32.
__device__ __forceinline__ Pairs8 unpack8(uint32_t word, uint32_t magic, uint32_t bias_lo,
                                          uint32_t bias_hi) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = word >> 8;
  Pairs8 r;
  r.a = bitcast<f16x2>((word & 0x000F000Fu) | magic) + bitcast<f16x2>(bias_lo);
  r.b = __builtin_elementwise_fma(bitcast<f16x2>((word & 0x00F000F0u) | magic), sixteenth,
                                  bitcast<f16x2>(bias_hi));
  r.c = bitcast<f16x2>((w8 & 0x000F000Fu) | magic) + bitcast<f16x2>(bias_lo);
  r.d = __builtin_elementwise_fma(bitcast<f16x2>((w8 & 0x00F000F0u) | magic), sixteenth,
                                  bitcast<f16x2>(bias_hi));
  return r;
}

// Eight consecutive halves of x (one 16-byte load when x is 16-byte aligned
// with a row stride that keeps it so).
__device__ __forceinline__ uint4 load_x8(const uint16_t* src, int vec16) {
  if (vec16) return *reinterpret_cast<const uint4*>(src);
  return make_uint4(src[0] | ((uint32_t)src[1] << 16), src[2] | ((uint32_t)src[3] << 16),
                    src[4] | ((uint32_t)src[5] << 16), src[6] | ((uint32_t)src[7] << 16));
}

// x0..x7 -> (x0,x4 | x1,x5 | x2,x6 | x3,x7), the order of unpack8's pairs.
__device__ __forceinline__ uint4 pair_halves(uint4 v) {
  return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                    (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace qg
