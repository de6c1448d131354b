// Device-side building blocks shared by the prefill and decode kernels (gfx950).
//
// Matrix-core layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (32 x 16, M x K): lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]
//   B operand (16 x 32, K x N): lane l holds B[8*(l/32) .. +7][l % 32]
//   C/D (32 x 32 float):        lane l, register j holds
//                               C[8*(j/4) + 4*(l/32) + (j%4)][l % 32]
// Scores are computed transposed, S^T = K Q^T (keys on M, query rows on N), so
// one lane owns one query row: row statistics are per-lane scalars and the
// other half-wave (lane ^ 32) holds the rest of that row's keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Both halves of the wave end up holding op(x[lane], x[lane ^ 32]).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight floats to bf16, round to nearest even (the gfx950 conversion).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}

// 16-byte loads of eight bf16 values; fp32 sources are read as two 16-byte
// loads and rounded on the way.
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <typename T> struct In;
template <> struct In<__bf16> {
  // raw holds 8 bf16
  struct Raw { u32x4 v; };
  __device__ __forceinline__ static Raw load(const __bf16* p) { return Raw{load16(p)}; }
  __device__ __forceinline__ static Raw zero() { return Raw{u32x4{0, 0, 0, 0}}; }
  __device__ __forceinline__ static u32x4 pack(const Raw& r) { return r.v; }
};
template <> struct In<float> {
  struct Raw { f32x4 a, b; };
  __device__ __forceinline__ static Raw load(const float* p) {
    return Raw{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
  }
  __device__ __forceinline__ static Raw zero() { return Raw{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ __forceinline__ static u32x4 pack(const Raw& r) {
    float f[8] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3]};
    bf16x8 h = to_bf16x8(f);
    return __builtin_bit_cast(u32x4, h);
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): together about 16
// significant bits of each float32 value.
__device__ __forceinline__ void split_hi_lo(const In<float>::Raw& r, bf16x8& hi, bf16x8& lo) {
  float f[8] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3]};
  hi = to_bf16x8(f);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] -= (float)hi[i];
  lo = to_bf16x8(f);
}
__device__ __forceinline__ void split_hi_lo(const In<__bf16>::Raw& r, bf16x8& hi, bf16x8& lo) {
  hi = as_bf16x8(r.v);
  lo = bf16x8{};
}

// Key order inside a 32-key block: the A-operand row m of S^T = K Q^T reads key
// sigma(m), sigma swapping bits 2 and 3 of m. Then accumulator register j of
// half h holds key 16*(j/8) + 8*h + (j%8): eight consecutive keys per 16-key
// chunk, which is exactly the B-operand layout P^T needs for O^T = V^T P^T.
__device__ __forceinline__ int sigma32(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
__device__ __forceinline__ int acc_key(int j, int half) { return 16 * (j >> 3) + 8 * half + (j & 7); }

// LDS layouts (bf16 elements, 16-byte chunks swizzled by XOR so that the
// matrix-core fragment reads are bank-conflict free):
//   K tile  [keys][D]: chunk c of key r stored at chunk c ^ kswz(r)
//   Vt tile [D][keys]: chunk c (8 keys) of row d stored at c ^ vswz(d)
__device__ __forceinline__ int kswz(int r) { return (r & 3) | ((r >> 1) & 4); }
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

}  // namespace fa
