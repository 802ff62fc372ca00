// Matrix-core helpers shared by the chunked kernels (gfx950, wave64):
// bf16 fragment types, LDS fragment and transpose reads, hi / lo bf16
// splits, the 16x16x32 bf16 product and a forward substitution on DPP row
// broadcasts.
#pragma once

#include "kda_device.h"

namespace kda {
namespace mx {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Storage position of contracted index c inside its block of 32: the
// fragment slot 8g + e (g = lane / 16, e = 0..7) of a contraction fed from
// accumulator tiles holds row 4g + e (e < 4) of the upper tile and row
// 16 + 4g + e - 4 (e >= 4) of the lower tile.
__host__ __device__ constexpr int pos32(int c) {
  return (c & ~31) | (8 * ((c & 15) >> 2)) | (4 * ((c >> 4) & 1)) | (c & 3);
}

// Workgroup barrier that orders LDS traffic only.  Waves exchange data
// through LDS alone, so outstanding global loads (the prefetched next tile)
// and stores may stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// fp32 -> bf16 bits (hardware round to nearest even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float hi_of(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

// An opaque copy of x: values derived from it cannot be hoisted out of a loop.
__device__ __forceinline__ int launder(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 frag_lds(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ s16x4 tr4(const bf16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 a, s16x4 b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// store 4 floats as bf16 (8 bytes)
__device__ __forceinline__ void st4b(bf16_t* p, const float* x) {
  uint2 u;
  u.x = cvt2(x[0], x[1]);
  u.y = cvt2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = u;
}
// store 8 floats as bf16 (16 bytes)
__device__ __forceinline__ void st8b(bf16_t* p, const float* x) {
  uint4 u;
  u.x = cvt2(x[0], x[1]);
  u.y = cvt2(x[2], x[3]);
  u.z = cvt2(x[4], x[5]);
  u.w = cvt2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// x += bcast_S(x) * a, where bcast_S(x) is x of lane S of the lane's row of
// 16 lanes: one v_fmac_f32 with a DPP row_newbcast source.  A DPP source
// must not be written by either of the two preceding VALU instructions; the
// callers interleave at least three independent updates between writes.
template <int S>
__device__ __forceinline__ void fmac_bcast16(float& x, float a) {
  asm volatile("v_fmac_f32_dpp %0, %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf" : "+v"(x) : "v"(a), "n"(S));
}

// Forward substitution down the 16 lanes of each lane row: lane r holds x_r
// of NG right-hand sides per system and na[s] = -L[r][s] of the unit lower
// triangular L (zero for s >= r); steps S..14 apply x_r += na[s] x_s with
// x_s final.  Two independent systems (x, na) and (y, nb) are interleaved.
template <int S, int NG>
__device__ __forceinline__ void fsub16x2(float (&x)[NG], const float (&na)[16], float (&y)[NG], const float (&nb)[16]) {
  if constexpr (S < 15) {
#pragma unroll
    for (int g = 0; g < NG; ++g) fmac_bcast16<S>(x[g], na[S]);
#pragma unroll
    for (int g = 0; g < NG; ++g) fmac_bcast16<S>(y[g], nb[S]);
    fsub16x2<S + 1, NG>(x, na, y, nb);
  }
}
template <int S, int NG>
__device__ __forceinline__ void fsub16(float (&x)[NG], const float (&na)[16]) {
  static_assert(NG >= 3, "DPP source hazard: at least three interleaved updates");
  if constexpr (S < 15) {
#pragma unroll
    for (int g = 0; g < NG; ++g) fmac_bcast16<S>(x[g], na[S]);
    fsub16<S + 1, NG>(x, na);
  }
}

// hi / lo bf16 pair of two floats, each packed in 32 bits: hi = bf16(x),
// lo = bf16(x - hi); the packed hi is unpacked by shifts, not converted back
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt2(a, b);
  lo = cvt2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// fragment (and hi / lo pair) from two vertically adjacent accumulator tiles
__device__ __forceinline__ void frag_pair(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  uint4 uh, ul;
  split2(a[0], a[1], uh.x, ul.x);
  split2(a[2], a[3], uh.y, ul.y);
  split2(b[0], b[1], uh.z, ul.z);
  split2(b[2], b[3], uh.w, ul.w);
  hi = __builtin_bit_cast(bf16x8, uh);
  lo = __builtin_bit_cast(bf16x8, ul);
}

// 8 floats as hi / lo bf16 pairs (16 bytes each)
__device__ __forceinline__ void st8b_pair(bf16_t* ph, bf16_t* pl, const float* x) {
  uint4 uh, ul;
  split2(x[0], x[1], uh.x, ul.x);
  split2(x[2], x[3], uh.y, ul.y);
  split2(x[4], x[5], uh.z, ul.z);
  split2(x[6], x[7], uh.w, ul.w);
  *reinterpret_cast<uint4*>(ph) = uh;
  *reinterpret_cast<uint4*>(pl) = ul;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16 product: lane l holds row (A) or column (B) l % 16 and the
// four contracted indices 4 (l / 16) .. 4 (l / 16) + 3 -- the accumulator
// layout of a 16x16 tile read along its rows
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

}  // namespace mx
}  // namespace kda
