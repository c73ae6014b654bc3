// Internal helpers shared by the H2O kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

// Storage tag for bfloat16 elements (raw 16-bit patterns).
struct bf16 {
  uint16_t bits;
};

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;  // elements per 16-byte chunk
  static constexpr int kBytes = 4;
  // 16 raw bytes -> 4 floats
  __device__ static inline void unpack(const uint4& raw, float* x) {
    x[0] = __uint_as_float(raw.x);
    x[1] = __uint_as_float(raw.y);
    x[2] = __uint_as_float(raw.z);
    x[3] = __uint_as_float(raw.w);
  }
};

template <>
struct Elem<bf16> {
  static constexpr int kPer16B = 8;
  static constexpr int kBytes = 2;
  // 16 raw bytes -> 8 floats; element 2i is the low half of word i.
  __device__ static inline void unpack(const uint4& raw, float* x) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Storage tag for E4M3 cache codes (OCP 8-bit float: bias 7, max 448, no inf).
struct e4m3 {
  uint8_t bits;
};

template <>
struct Elem<e4m3> {
  static constexpr int kPer16B = 16;
  static constexpr int kBytes = 1;
  // 16 codes -> 16 floats (exact); byte 0 of word i is element 4i.
  __device__ static inline void unpack(const uint4& raw, float* x) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      x[4 * i] = lo.x;
      x[4 * i + 1] = lo.y;
      x[4 * i + 2] = hi.x;
      x[4 * i + 3] = hi.y;
    }
  }
};

// Four floats already scaled into [-464, 464) -> four E4M3 codes, nearest
// even.  Values in (448, 464) round to 448 under that rule; clamping them
// first gives the same code on every path.
__device__ inline uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 16-byte load with the non-temporal hint: data read once per kernel
// should not displace reusable lines from the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// Streaming 16-byte store with the non-temporal hint.
__device__ inline void store16_nt(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

// DPP lane permutations (row = 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140; // lane i <- lane 15-i within a row
constexpr int kDppHalfMirror = 0x141;// lane i <- lane 7-i within each half row

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Every lane l gets its own value of x and lane l ^ 16's (pair16) or lane
// l ^ 32's (pair32), in an order that depends on the lane: gfx950's
// v_permlane16_swap / v_permlane32_swap exchange rows between two copies of x
// in the vector ALU, where a shuffle (ds_bpermute) takes an LDS round trip.
// Symmetric operations of the pair (sum, min, max) need not know the order.
struct LanePair {
  uint32_t a, b;
};
__device__ inline LanePair pair16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return {r[0], r[1]};
}
__device__ inline LanePair pair32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}
template <bool k32>
__device__ inline float sum_pair(float x) {
  const LanePair p = k32 ? pair32(__float_as_uint(x)) : pair16(__float_as_uint(x));
  return __uint_as_float(p.a) + __uint_as_float(p.b);
}
template <bool k32>
__device__ inline float max_pair(float x) {
  const LanePair p = k32 ? pair32(__float_as_uint(x)) : pair16(__float_as_uint(x));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}

// Sum over aligned groups of G consecutive lanes; every lane of a group gets the total.
template <int G>
__device__ inline float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (G >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (G >= 32) x = sum_pair<false>(x);
  if constexpr (G >= 64) x = sum_pair<true>(x);
  return x;
}

// Maximum over aligned groups of G consecutive lanes (G <= 16).
template <int G>
__device__ inline float group_max(float x) {
  static_assert(G == 4 || G == 8 || G == 16, "group size");
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  if constexpr (G >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (G >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

// One E4M3 cache row chunk: 16 input values of a row whose absolute maximum
// over all its lanes is amax -> 16 codes; the row scale is amax / 448.
__device__ inline uint4 quantize16_e4m3(const float* x, float amax) {
  const float inv = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack4_e4m3(x[4 * i] * inv, x[4 * i + 1] * inv, x[4 * i + 2] * inv, x[4 * i + 3] * inv);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace h2o
