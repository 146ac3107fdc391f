// Internal helpers shared by the HIP sources of the library (not part of
// the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride.  Loads past num_records return zero without
// touching memory, which is how padding slots are kept out of every read.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, kBufferRsrcWord3);
}

// Cache policy of K/V loads (the buffer instruction's aux bits).  Rows are
// read once per decode step and every load fetches whole 128-byte lines, so
// they use the non-temporal policy (kLoadNt, aux bit 1 -> `nt`): on MI355X
// this lifts a paged 256-byte-segment read stream from ~6.0 to ~6.8 TB/s.
constexpr int kLoadNt = 2;

template <int AUX = kLoadNt>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r,
                                        uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, AUX);
}

template <int AUX = kLoadNt>
__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t r,
                                       uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, AUX);
}

// Eight OCP fp8 e4m3 codes (bytes in order) to eight fp16 values, exactly:
// every e4m3 value (|x| <= 448, subnormals 2^-9 .. 7*2^-9) is an fp16
// value.  (On gfx950 the fp8 conversions use the OCP formats.)
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(u32x2 w) {
  // gfx950's scaled conversion turns two e4m3 codes (one 16-bit half of the
  // word) into two fp16 values; with scale 1 it is exact, since every e4m3
  // value is an fp16 number
  const unsigned w0 = w.x, w1 = w.y;
  u32x4 r;
  r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false));
  r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true));
  r.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false));
  r.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true));
  return r;
}

// e4m3 code pair of x*inv and y*inv: the conversion rounds to nearest even
// and gives NaN above the largest finite code, so values are clamped to
// +-448 first (NaN inputs stay NaN).  Result in the low or high 16 bits of
// `old` as `hi` says.
__device__ __forceinline__ int fp8_pair(float x, float y, float inv, int old,
                                        bool hi) {
  float u = x * inv, v = y * inv;
  u = u > 448.f ? 448.f : (u < -448.f ? -448.f : u);
  v = v > 448.f ? 448.f : (v < -448.f ? -448.f : v);
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(u, v, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(u, v, old, false);
}

__device__ __forceinline__ u32x2 f16x8_to_fp8x8(u32x4 h, float inv) {
  const unsigned w[4] = {h.x, h.y, h.z, h.w};
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[k] & 0xffffu));
    f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[k] >> 16));
  }
  int lo = fp8_pair(f[0], f[1], inv, 0, false);
  lo = fp8_pair(f[2], f[3], inv, lo, true);
  int hi = fp8_pair(f[4], f[5], inv, 0, false);
  hi = fp8_pair(f[6], f[7], inv, hi, true);
  u32x2 r;
  r.x = (unsigned)lo;
  r.y = (unsigned)hi;
  return r;
}

// Cross-lane moves inside a 16-lane DPP row (all lanes must be active).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;      // row_ror:8 = lane ^ 8 within a row of 16
constexpr int kRowRor4 = 0x124;      // row_ror:4

// Sum over aligned groups of LANES (8 or 16) lanes; every lane of a group
// ends with the bitwise-identical total (each step adds two equal-order
// partial sums, so the result does not depend on the lane).
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LANES == 8 || LANES == 16, "group of 8 or 16 lanes");
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  if (LANES == 16) v += dpp<kRowMirror>(v);
  return v;
}

// Reinterpret one 32-bit word as two fp16 values.  The word must arrive as
// a scalar: with this compiler, bit-casting a vector element expression in
// place (v.y, v.z, v.w) reads element x instead.
__device__ __forceinline__ f16x2 as_h2(unsigned w) {
  return __builtin_bit_cast(f16x2, w);
}

// One 32-bit word as fp32 (the word must arrive as a scalar, as for as_h2)
__device__ __forceinline__ float as_f32(unsigned w) {
  return __builtin_bit_cast(float, w);
}

// Eight fp16 products of two 16-byte chunks accumulated in fp32
// (v_dot2_f32_f16: exact fp16 products, fp32 sums).
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
  const unsigned a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w;
  const unsigned b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
  float s = __builtin_amdgcn_fdot2(as_h2(a0), as_h2(b0), 0.f, false);
  s = __builtin_amdgcn_fdot2(as_h2(a1), as_h2(b1), s, false);
  s = __builtin_amdgcn_fdot2(as_h2(a2), as_h2(b2), s, false);
  s = __builtin_amdgcn_fdot2(as_h2(a3), as_h2(b3), s, false);
  return s;
}

__device__ __forceinline__ float half_at(u32x4 v, int e) {
  const unsigned w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (float)as_h2(w)[e & 1];
}

// v_readlane of an fp32 value (the builtin takes and returns int, so the
// bits are moved, not converted)
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

}  // namespace pa
