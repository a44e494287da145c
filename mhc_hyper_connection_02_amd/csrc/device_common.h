// Device helpers shared by the gfx950 kernels: bf16 / E4M3 / E8M0 conversions
// and wave-level reductions. Narrowing to bf16 (8 significant bits in fp32's
// exponent range) and to OCP E4M3 "FN" (bias 7, 3 fraction bits, max 448,
// subnormal step 2^-9) runs on gfx950's packed conversion instructions, round
// to nearest even; widening and the E8M0 exponent are bit manipulations.
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

// Stores of the outputs (written once, read by a later kernel) with the non-temporal
// hint: measured 0.3-0.6 us less per boundary call than plain stores, by leaving
// fewer dirty lines in L2 for the end of the kernel.
__device__ __forceinline__ void store_nt(uint4* p, const uint4& v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(uint2* p, const uint2& v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ void store_nt(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}

// 4-byte load with the non-temporal hint (two bf16 values).
__device__ __forceinline__ uint32_t load_nt(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void store_nt(uint16_t* p, uint16_t v) {
  __builtin_nontemporal_store(v, p);
}

// 8-byte load with the non-temporal hint (four bf16 values).
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 values packed in a 16-byte vector <-> eight floats.
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (lo in bits 0..15), round to nearest even, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}


// Round eight floats to bf16 and pack them.
__device__ __forceinline__ uint4 pack8_round(const float (&f)[8]) {
  uint4 v;
  v.x = cvt_pk_bf16(f[0], f[1]);
  v.y = cvt_pk_bf16(f[2], f[3]);
  v.z = cvt_pk_bf16(f[4], f[5]);
  v.w = cvt_pk_bf16(f[6], f[7]);
  return v;
}

// Round eight floats to bf16 precision in place (they stay floats).
__device__ __forceinline__ void round8_bf16(float (&f)[8]) {
  unpack8(pack8_round(f), f);
}

// The same for a lane's 16-byte (eight bf16) or 8-byte (four bf16) vector, by overload.
__device__ __forceinline__ void unpack_bf16(const uint4& v, float (&f)[8]) { unpack8(v, f); }
__device__ __forceinline__ void unpack_bf16(const uint2& v, float (&f)[4]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
}
__device__ __forceinline__ void unpack_bf16(const uint32_t& v, float (&f)[2]) {
  f[0] = bf16_lo(v); f[1] = bf16_hi(v);
}
__device__ __forceinline__ uint4 pack_bf16(const float (&f)[8]) { return pack8_round(f); }
__device__ __forceinline__ uint32_t pack_bf16(const float (&f)[2]) {
  return cvt_pk_bf16(f[0], f[1]);
}
__device__ __forceinline__ uint2 pack_bf16(const float (&f)[4]) {
  return make_uint2(cvt_pk_bf16(f[0], f[1]), cvt_pk_bf16(f[2], f[3]));
}
template <int N>
__device__ __forceinline__ void round_bf16(float (&f)[N]) {
  unpack_bf16(pack_bf16(f), f);
}

// Four floats -> four OCP E4M3 (FN) codes (byte i = f[i]), round to nearest even,
// in two v_cvt_pk_fp8_f32. Inputs must be finite with |f| <= 448 (the E8M0 scale
// guarantees it), where no saturation or NaN case arises; below 2^-6 the codes are
// the subnormals.
__device__ __forceinline__ uint32_t cvt_pk4_e4m3(float f0, float f1, float f2, float f3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, lo, true);
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

// Byte offset of the E8M0 scale of row r, 32-element block kb, in the MXFP8 scale
// output. kt == 0: plain row-major [rows][kblocks]. kt > 0: the swizzled 128x4
// layout that the boundary page names for its MXFP8 layer input (FlashInfer's, the
// block-scale layout of the published block-scaled GEMM interfaces): rows padded to
// 128, blocks to 4, one 512-byte tile per 128 rows x 4 blocks, tiles row-major with
// kt = padded blocks / 4 tiles per tile row; inside a tile, byte
// (r % 32) * 16 + ((r / 32) % 4) * 4 + kb % 4.
__device__ __forceinline__ size_t mx_scale_offset(int r, int kb, int kblocks, int kt) {
  if (kt == 0) return (size_t)r * kblocks + kb;
  return (((size_t)(r >> 7) * kt + (kb >> 2)) << 9) + ((r & 31) << 4) + (((r >> 5) & 3) << 2) +
         (kb & 3);
}

// Cross-lane moves on the DPP path (no LDS round trip). Quad permutations act
// within each group of 4 lanes; row rotations within each row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each eight

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
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

// Touches every 64-byte line of the kernel's argument block in one round of scalar loads.
// The compiler reads a large argument block in several rounds, each waiting for its loads
// (it parks the values in VGPR lanes between them); with the lines already in the scalar
// cache those rounds no longer wait for memory. BYTES: the summed sizes of the explicit
// arguments, at most the argument segment's size; the first word of each line is read, and
// only where it lies inside those bytes.
template <int BYTES>
__device__ __forceinline__ void prefetch_kernargs() {
  static_assert(BYTES >= 4, "an argument block of at least one word");
  const uint32_t* ka = (const uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < (BYTES - 4) / 64 + 1; ++i) t ^= ka[i * 16];
  asm volatile("" ::"s"(t));
}

// base plus a byte offset held in 32 bits: a global access then takes its 64-bit base from
// scalar registers and only a 32-bit offset per lane, with no 64-bit address arithmetic per
// lane. Callers keep the offset below 2^32.
template <typename T>
__device__ __forceinline__ const T* byte_at(const T* base, uint32_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ T* byte_at(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// Reciprocal, reciprocal square root and exp on the hardware approximations (about one
// ulp; exp through exp2 of x log2 e): the coefficient epilogue and the row norms are chains
// of dependent steps, where the exactly rounded sequences cost 10 to 20 instructions each.
// The results stay far inside the tolerances (1e-5 for the coefficients, the bf16 rounding
// of the layer input).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// A row handoff word, stored and polled either at device scope or, where every workgroup of
// the row runs on one XCD, through that XCD's L2: the store then needs only workgroup scope
// (the CU's L1 is write-through) and the poll is a non-temporal load, which the L1 does not
// keep, so each poll reads the L2, where the other workgroups' stores land. The empty asm
// keeps the compiler from merging polls of a loop into one load.
__device__ __forceinline__ void publish_word(unsigned long long* p, unsigned long long v,
                                             bool xcd) {
  if (xcd)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long poll_word(const unsigned long long* p, bool xcd) {
  if (xcd) {
    asm volatile("" ::: "memory");
    return __builtin_nontemporal_load(p);
  }
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mhc
