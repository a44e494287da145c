// Device helpers shared by the gfx950 kernels: bf16 / E4M3 / E8M0 conversions
// and wave-level reductions. All conversions are exact bit manipulations of
// the format definitions (bf16: 8 significant bits in fp32's exponent range;
// OCP E4M3 "FN": bias 7, 3 fraction bits, max 448, subnormal step 2^-9).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

constexpr int kWave = 64;  // CDNA wavefront width

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) hint: data read once per call.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even. Inputs are finite by
// construction; a NaN is kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

// Eight bf16 values packed in a 16-byte vector <-> eight floats.
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint32_t pack2_bits(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Round eight floats to bf16 and pack them.
__device__ __forceinline__ uint4 pack8_round(const float (&f)[8]) {
  uint4 v;
  v.x = pack2_bits(f32_to_bf16_bits(f[0]), f32_to_bf16_bits(f[1]));
  v.y = pack2_bits(f32_to_bf16_bits(f[2]), f32_to_bf16_bits(f[3]));
  v.z = pack2_bits(f32_to_bf16_bits(f[4]), f32_to_bf16_bits(f[5]));
  v.w = pack2_bits(f32_to_bf16_bits(f[6]), f32_to_bf16_bits(f[7]));
  return v;
}

// E4M3 (FN) code of a finite float, nearest-even; |f| >= 448 saturates to 0x7E.
// Below 2^-6 the code is the subnormal count round(|f| * 2^9) (8 is the
// smallest normal); above, the fp32 fraction is rounded to 3 bits and the
// exponent re-biased from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {            // 448.0
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {      // 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
  } else {
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;     // exponent:3-bit fraction, RNE
    code = r - ((127u - 7u) << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// E8M0 block exponent e of a non-negative finite amax given as fp32 bits:
// the smallest integer with amax <= 448 * 2^e, i.e. E - 8 + [fraction > 0.75]
// for amax = 1.f * 2^E; -127 for zero and for anything below 2^-126 (the
// exact value would be below the E8M0 range, which clamps at -127).
__device__ __forceinline__ int e8m0_exponent(uint32_t amax_bits) {
  const uint32_t ef = amax_bits >> 23;
  if (ef == 0) return -127;
  int e = (int)ef - 127 - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Cross-lane moves on the DPP path (no LDS round trip). Quad permutations act
// within each group of 4 lanes; row rotations within each row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppQuadXor3 = 0x1B;   // quad_perm [3,2,1,0]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint4 dpp_u4(const uint4& v) {
  return make_uint4(dpp_u32<CTRL>(v.x), dpp_u32<CTRL>(v.y), dpp_u32<CTRL>(v.z), dpp_u32<CTRL>(v.w));
}

// Sum over the 64 lanes on the DPP path: within each row of 16 (quad xors, then row
// rotations), then the four row sums read into scalars. Every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace mhc
