// Shared pieces of the MFMA attention kernels (prefill and decode): LDS row
// strides of K and V rows (head dim 64, fp16), the fp16 MFMA and pair-sum
// operations, 16-byte chunk loads and stores, the transposed V read
// (ds_read_b64_tr_b16, the A operand of the P.V product) and the cross-lane
// max/sum of the 32x32 layout.
#pragma once

#include <type_traits>

#include "common.h"

namespace hymba {
namespace attn {

constexpr int kHd = 64;          // head dim of the MFMA kernel
constexpr int kQB = 32;          // queries per wave (one MFMA column block)
constexpr int kKT = 64;          // keys per decode tile
constexpr int kKStr = kHd + 8;   // LDS row stride (16-bit words) of K rows: 144 B
// LDS row strides of V rows.  With 32x32 fragments a transposed read's two 16-lane groups
// take 4 rows at dims d and d + 16; a 192 B stride would make that conflict-free at 33% more
// LDS per stage, but the prefill kernel measured faster with K's 144 B stride and some 2-way
// conflicts.  With 16x16 fragments (decode) a read's groups take 8 consecutive rows at the
// same dims: 160 B puts them 40 banks apart.
constexpr int kVStr = kKStr;         // 144 B, the prefill stages (32x32 fragments)
constexpr int kVStr16 = kHd + 16;    // 160 B, the decode tile step (16x16 fragments)
constexpr float kLazyLog2 = 8.f;   // rescale threshold of the decode tile's online softmax (log2 units)

struct __align__(16) U4 { uint32_t x, y, z, w; };

template <typename ET> struct Op;
template <> struct Op<half_t> {
  typedef f16x8_t vec;
  __device__ static __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // c + the two 16-bit values of w (v_dot2c_f32_f16 against (1, 1): exact products, fp32 sum)
  __device__ static __forceinline__ float add_pair(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), f16x2_t{1, 1}, c, false);
  }
};
template <typename ET>
__device__ __forceinline__ typename Op<ET>::vec as_vec(U4 v) { return __builtin_bit_cast(typename Op<ET>::vec, v); }

__device__ __forceinline__ U4 masked_load(const void* p, bool keep) {
  const U4 x = *reinterpret_cast<const U4*>(p);
  U4 r;
  r.x = keep ? x.x : 0u;
  r.y = keep ? x.y : 0u;
  r.z = keep ? x.z : 0u;
  r.w = keep ? x.w : 0u;
  return r;
}

// chunks it + 128 j (j < 4) of a tile: row (it >> 3) + 16 j, dims 8 (it & 7) + 0..7.  Stored
// field by field: a plain struct copy from the fetch registers to LDS stays a memory-to-memory
// copy that the compiler routes through scratch.
__device__ __forceinline__ void chunk_store(const U4 (&r)[4], uint16_t* base, int str, int it) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(base + ((it >> 3) + 16 * j) * str + (it & 7) * 8) =
        make_uint4(r[j].x, r[j].y, r[j].z, r[j].w);
}

// 4 keys x 1 dim of a V tile [key][dim] (row stride vstr) per lane, transposed by the LDS: the
// 16 lanes of a group read 4 rows x 16 dims (lane j: row j / 4, dims 4 (j % 4) + 0..3 from p)
// and lane i receives dim i of the 4 rows, keys in order.
__device__ __forceinline__ uint2 v_tr4(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) v4s*)(const_cast<uint16_t*>(p))));
}

// x combined with the same register of lane l ^ 32 (v_permlane32_swap with
// both operands x: the two results are the low half and the high half
// broadcast to both halves, so any symmetric op of them is the xor-32 reduction).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max of three.  Plain fmaxf, which the compiler turns into v_max3_f32 after quieting inputs it
// cannot prove canonical: an inline-asm v_max3_f32 would be invisible to the hazard recognizer,
// which then inserts no wait states between an MFMA writing the scores and the asm reading them.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

}  // namespace attn
}  // namespace hymba
