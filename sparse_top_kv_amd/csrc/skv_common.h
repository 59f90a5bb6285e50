// skv_common.h -- device helpers shared by the libsparsekv kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Row geometry of one K or V row: each lane moves 16 bytes per load.
template <int DT, int D>
struct RowGeom {
  static constexpr int kElem = DT == 1 ? 2 : 4;     // bytes per element
  static constexpr int kRowBytes = D * kElem;       // bytes per cache row
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kElemsPerLane = 16 / kElem;
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // rows one wave load covers
};

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // reverse within 8 lanes
constexpr int kDppMirror = 0x140;     // reverse within 16 lanes

// Lane l and lane l ^ 16 (resp. l ^ 32) combined with VALU lane swaps
// (v_permlane16_swap / v_permlane32_swap) instead of an LDS-routed shuffle.
// Both lanes of a pair compute the same expression on the same operands (the
// lower lane's value first), so they hold bit-identical results.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of N lanes (N in 1..64, power of two); every lane
// of the group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }

// 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9 word 3: 32-bit data
// format); loads past `bytes` return zeros instead of faulting.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte buffer load at byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Same with the non-temporal hint (cache policy bit 1): for data read once.
__device__ __forceinline__ uint4 buf_load16_stream(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

// Dot product of this lane's 16-byte slice of a row with the matching query
// slice.  bf16: q holds 4 packed pairs; fp32: q holds 4 floats (as bits).
template <int DT>
__device__ __forceinline__ float slice_dot(const uint32_t (&q)[4], const uint4& k) {
  if constexpr (DT == 1) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[0]),
                                              __builtin_bit_cast(bf16x2_t, k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[1]),
                                        __builtin_bit_cast(bf16x2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[2]),
                                        __builtin_bit_cast(bf16x2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[3]),
                                        __builtin_bit_cast(bf16x2_t, k.w), s, false);
    return s;
  } else {
    float s = __uint_as_float(q[0]) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q[1]), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q[2]), __uint_as_float(k.z), s);
    s = fmaf(__uint_as_float(q[3]), __uint_as_float(k.w), s);
    return s;
  }
}

// Widen this lane's 16-byte slice of a row to fp32 (8 values for bf16, 4 for fp32).
template <int DT>
__device__ __forceinline__ void slice_to_f32(const uint4& v, float* out) {
  if constexpr (DT == 1) {
    out[0] = bf16lo(v.x); out[1] = bf16hi(v.x);
    out[2] = bf16lo(v.y); out[3] = bf16hi(v.y);
    out[4] = bf16lo(v.z); out[5] = bf16hi(v.z);
    out[6] = bf16lo(v.w); out[7] = bf16hi(v.w);
  } else {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
}

// Order-preserving map of an fp32 score to uint32: larger float -> larger key;
// -0.0 is folded onto +0.0 first.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace skv
