// Shared device/host helpers of the hybrid-head mixer library (gfx950 only).
//
// Element types.  A layer has a storage type for its boundary (x, y, weights)
// and an activation type for everything it produces internally and exchanges
// with its KV-sharing partner:
//   fp32 layers:  storage fp32, activations fp32;
//   bf16 layers:  storage bf16, activations fp16 (11-bit significand; fp16 MFMA
//                 runs at the bf16 rate on gfx950), accumulation and SSM state fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymba {

typedef __bf16 bf16_t;
typedef _Float16 half_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));   // four bf16 bit patterns (MFMA x8 operand)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- 16-bit pairs packed in a 32-bit word -------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// two floats -> packed pair, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Pair helpers selected by element type.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  __device__ static __forceinline__ float lo(uint32_t w) { return bf16lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return bf16hi(w); }
  __device__ static __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
template <> struct Pair<half_t> {
  __device__ static __forceinline__ float lo(uint32_t w) { return f16lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return f16hi(w); }
  __device__ static __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};

// Scalar load/store with conversion to/from fp32.
template <typename T> struct Elem {
  __device__ static __forceinline__ float load(const T* p) { return static_cast<float>(*p); }
  __device__ static __forceinline__ void store(T* p, float v) { *p = static_cast<T>(v); }
};

// 16 bytes of a storage type <-> floats (8 for 16-bit types, 4 for fp32).
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // non-temporal forms (nt cache policy) for data read or written once
  __device__ static __forceinline__ void load_nt(const float* p, float (&v)[4]) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  }
  __device__ static __forceinline__ void store_nt(float* p, const float (&v)[4]) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  }
};
template <typename T> struct Vec16H {   // 16-bit element types
  static constexpr int n = 8;
  __device__ static __forceinline__ void load(const T* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    v[0] = Pair<T>::lo(x.x); v[1] = Pair<T>::hi(x.x); v[2] = Pair<T>::lo(x.y); v[3] = Pair<T>::hi(x.y);
    v[4] = Pair<T>::lo(x.z); v[5] = Pair<T>::hi(x.z); v[6] = Pair<T>::lo(x.w); v[7] = Pair<T>::hi(x.w);
  }
  __device__ static __forceinline__ void store(T* p, const float (&v)[8]) {
    uint4 x;
    x.x = Pair<T>::pack(v[0], v[1]); x.y = Pair<T>::pack(v[2], v[3]);
    x.z = Pair<T>::pack(v[4], v[5]); x.w = Pair<T>::pack(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = x;
  }
  __device__ static __forceinline__ void load_nt(const T* p, float (&v)[8]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v[0] = Pair<T>::lo(x[0]); v[1] = Pair<T>::hi(x[0]); v[2] = Pair<T>::lo(x[1]); v[3] = Pair<T>::hi(x[1]);
    v[4] = Pair<T>::lo(x[2]); v[5] = Pair<T>::hi(x[2]); v[6] = Pair<T>::lo(x[3]); v[7] = Pair<T>::hi(x[3]);
  }
  __device__ static __forceinline__ void store_nt(T* p, const float (&v)[8]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x{Pair<T>::pack(v[0], v[1]), Pair<T>::pack(v[2], v[3]),
                  Pair<T>::pack(v[4], v[5]), Pair<T>::pack(v[6], v[7])};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
  }
};
template <> struct Vec16<bf16_t> : Vec16H<bf16_t> {};
template <> struct Vec16<half_t> : Vec16H<half_t> {};

// exp2 / log2 on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + e^{-|x|}), via exp2/log2.
__device__ __forceinline__ float softplus_f(float x) {
  float t = fast_exp2(-fabsf(x) * kLog2e);
  return fmaxf(x, 0.f) + kLn2 * fast_log2(1.f + t);
}

// z * sigmoid(z)
__device__ __forceinline__ float silu_f(float z) {
  return z / (1.f + fast_exp2(-z * kLog2e));
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace hymba
