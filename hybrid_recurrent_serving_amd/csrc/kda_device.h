// Device-side helpers shared by the libkda kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (the hardware convert; a NaN
// stays a NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> struct io;

template <> struct io<float> {
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float x) { *p = x; }
  // load 4 consecutive elements (16-byte aligned for float)
  __device__ static __forceinline__ void ld4(const float* p, float (&x)[4]) {
    float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  }
  __device__ static __forceinline__ void st4(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <> struct io<bf16_t> {
  __device__ static __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void st(bf16_t* p, float x) { *p = f32_to_bf16(x); }
  // 4 consecutive elements = 8 bytes (8-byte aligned)
  __device__ static __forceinline__ void ld4(const bf16_t* p, float (&x)[4]) {
    uint2 t = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(t.x << 16);
    x[1] = __uint_as_float(t.x & 0xffff0000u);
    x[2] = __uint_as_float(t.y << 16);
    x[3] = __uint_as_float(t.y & 0xffff0000u);
  }
  __device__ static __forceinline__ void st4(bf16_t* p, const float (&x)[4]) {
    uint2 t;
    t.x = static_cast<uint32_t>(f32_to_bf16(x[0])) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
    t.y = static_cast<uint32_t>(f32_to_bf16(x[2])) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
    *reinterpret_cast<uint2*>(p) = t;
  }
};

// Load n consecutive elements (n a multiple of 4) as floats.
template <typename T, int N>
__device__ __forceinline__ void ld_vec(const T* p, float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    float t[4];
    io<T>::ld4(p + i, t);
    x[i] = t[0]; x[i + 1] = t[1]; x[i + 2] = t[2]; x[i + 3] = t[3];
  }
}

// Recurrent state rows stream through once per call: non-temporal 16-byte
// accesses
typedef __attribute__((ext_vector_type(4))) float nt4;
__device__ __forceinline__ void ld4_stream(const float* p, float (&x)[4]) {
  const nt4 v = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(p));
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void st4_stream(float* p, const float (&x)[4]) {
  const nt4 v = {x[0], x[1], x[2], x[3]};
  __builtin_nontemporal_store(v, reinterpret_cast<nt4*>(p));
}

// sigmoid and SiLU from the hardware base-2 exponential and reciprocal (each
// about one unit in the last place); a large negative argument gives
// exp2 = inf, reciprocal 0, so SiLU tends to (-)0 and sigmoid to 0.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
__device__ __forceinline__ float silu_fast(float x) { return x * sigmoid_fast(x); }

// Sum over the lanes that differ only in bits >= log2(FIRST) of the lane id,
// without the LDS crossbar: inside a row of 16 lanes by DPP moves (quad
// permutations for lane bits 0 and 1, row rotations by 4 and 8 for bits 2
// and 3: after x += ror4(x) and x += ror8(x) every lane holds the sum of the
// four lanes i, i +- 4, i +- 8 of its row that agree in bits 0 and 1), then
// across rows by the gfx950 permlane swaps (rows 2r and 2r+1, then the two
// halves of the wave; each swap of x with itself hands every lane the value
// of its partner, and the sum is symmetric).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int FIRST>
__device__ __forceinline__ float wave_sum_from(float x) {
  static_assert(FIRST == 1 || FIRST == 2 || FIRST == 4 || FIRST == 8 || FIRST == 16 || FIRST == 32 ||
                FIRST == 64, "a power of two up to 64");
  if constexpr (FIRST <= 1) x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (FIRST <= 2) x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (FIRST <= 4) x += dpp_mov<0x124>(x);  // row_ror:4
  if constexpr (FIRST <= 8) x += dpp_mov<0x128>(x);  // row_ror:8
  if constexpr (FIRST <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (FIRST <= 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Sum of x over aligned groups of NL adjacent lanes (NL = 2 .. 32, a power of
// two; every lane of a group active).  Inside a row of 16 lanes on DPP moves:
// the two quad permutations pair lanes 1 and 2 apart, then the half-row
// mirror joins the two (now uniform) quads of each 8 lanes and the row mirror
// the two halves; a 32-lane group adds the neighbouring row by the permlane
// swap of rows 2r and 2r + 1.
template <int NL>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(NL == 2 || NL == 4 || NL == 8 || NL == 16 || NL == 32, "group of 2..32 lanes");
  x += dpp_mov<0xB1>(x);                          // quad_perm [1, 0, 3, 2]
  if constexpr (NL > 2) x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  if constexpr (NL > 4) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (NL > 8) x += dpp_mov<0x140>(x);   // row_mirror
  if constexpr (NL > 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// State slices through a buffer resource: one whose size is 0 makes every
// load return 0, so a slice with no source needs no branch and its loads are
// issued on every path (which keeps the compiler's load-counter waits exact).
constexpr int kBufWord3 = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)
constexpr int kBufNonTemporal = 2;

// A buffer resource from values that are the same on every lane, held in
// scalar registers (the compiler cannot always prove that by itself).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* ua = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ua, 0, __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}

// 16 bytes of a state slice through a buffer resource (non-temporal; 0 when
// the resource has size 0), whole offset in the vector offset
__device__ __forceinline__ void ld4_rsrc(__amdgpu_buffer_rsrc_t r, int voff, float (&x)[4]) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kBufNonTemporal);
  x[0] = __uint_as_float(v[0]); x[1] = __uint_as_float(v[1]);
  x[2] = __uint_as_float(v[2]); x[3] = __uint_as_float(v[3]);
}

// 16 bytes of a state slice through a buffer resource (non-temporal; dropped
// when the resource has size 0).  The whole offset goes in the vector
// offset and the scalar offset is the constant 0: with a scalar register
// there, the compiler inserts no wait before a vector write to the store's
// data registers, and measured stores then took some lanes' first dword
// from the next value written to that register.
__device__ __forceinline__ void st4_rsrc(__amdgpu_buffer_rsrc_t r, int voff, int off, const float (&x)[4]) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff + off, 0, kBufNonTemporal);
}

// Gated RMS norm of one output vector of D channels held 4 per lane by
// D / 4 consecutive lanes (sum of squares across them by butterfly
// shuffles): o <- o / sqrt(mean o^2 + eps) * weight * sigmoid(gate).
template <int D, typename Tin>
__device__ __forceinline__ void gate_norm4(float (&o)[4], const Tin* gate, const Tin* weight, float eps) {
  float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
  for (int m = 1; m < D / 4; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float inv = 1.f / sqrtf(ss * (1.f / D) + eps);
  float z[4], w[4];
  io<Tin>::ld4(gate, z);
  io<Tin>::ld4(weight, w);
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = o[c] * inv * w[c] * sigmoid_fast(z[c]);
}

}  // namespace kda
