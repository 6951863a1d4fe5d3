// Tile machinery of the MFMA attention kernels (prefill and decode): 64-key
// tiles of K and V rows in LDS, and one wave's online-softmax step over a tile
// for 32 query columns with v_mfma_f32_32x32x16_{f16,bf16}.  V is stored as it
// comes (key rows) and read back transposed by ds_read_b64_tr_b16 as the A
// operand of the P.V product.
//
// Scores are computed transposed (S^T = K Q^T) so each lane owns one query
// column and 16 keys of a 32-key block: the softmax max needs one exchange
// with lane l^32, and the probabilities feed the P.V product as the B operand
// without any cross-lane movement.
#pragma once

#include <type_traits>

#include "common.h"

namespace hymba {
namespace attn {

constexpr int kHd = 64;          // head dim of the MFMA kernel
constexpr int kQB = 32;          // queries per wave (one MFMA column block)
constexpr int kKT = 64;          // keys per tile
constexpr int kKStr = kHd + 8;   // LDS row stride (16-bit words) of K tiles: 144 B
// LDS row strides of V tiles.  With 32x32 fragments a transposed read's two 16-lane groups
// take 4 rows at dims d and d + 16; a 192 B stride would make that conflict-free, but the
// prefill stage then needs 43 KB instead of 37 KB per workgroup, and the kernel measured
// faster with K's 144 B stride and some 2-way conflicts.  With 16x16 fragments (decode) a
// read's groups take 8 consecutive rows at the same dims: 160 B puts them 40 banks apart.
constexpr int kVStr = kKStr;         // 144 B, the prefill tile step (32x32 fragments)
constexpr int kVStr16 = kHd + 16;    // 160 B, the decode tile step (16x16 fragments)
constexpr float kLazyLog2 = 8.f;   // rescale threshold of the decode tile's online softmax (log2 units)

struct __align__(16) U4 { uint32_t x, y, z, w; };

template <typename ET> struct Op;
template <> struct Op<half_t> {
  typedef f16x8_t vec;
  typedef f16x4_t vec4;
  __device__ static __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x16_t mfma8(vec4 a, vec4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c, 0, 0, 0);
  }
  // c + the two 16-bit values of w (v_dot2c_f32_f16 against (1, 1): exact products, fp32 sum)
  __device__ static __forceinline__ float add_pair(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), f16x2_t{1, 1}, c, false);
  }
};
template <> struct Op<bf16_t> {
  typedef bf16x8_t vec;
  typedef s16x4_t vec4;
  __device__ static __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x16_t mfma8(vec4 a, vec4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float add_pair(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), bf16x2_t{1, 1}, c, false);
  }
};
template <typename ET>
__device__ __forceinline__ typename Op<ET>::vec as_vec(U4 v) { return __builtin_bit_cast(typename Op<ET>::vec, v); }

// 16-bit elements stored as raw 16-bit words; a double-buffered stage of 64-key tiles
struct AttnSmem {
  uint16_t kw[2][kKT * kKStr];        // K tiles [key][dim]
  uint16_t vw[2][kKT * kVStr];        // V tiles [key][dim]
};

// Cooperative load of a 64-key tile spread over the workgroup's 256 threads,
// four 16-byte loads each: threads [0, 128) own K chunks tid + 128 j (j < 4)
// of the tile's 512 (64 rows x 8 chunks), threads [128, 256) the same chunks
// of V.  Rows beyond `nvalid` (>= 1) read a clamped, valid row and are
// zero-filled by value.

__device__ __forceinline__ uint32_t u4_get(const U4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

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

// item < 128: K chunks into ks; item >= 128: the same chunks of V into vs (a branch, not a
// pointer select: the item is wave-uniform in K/V at every call)
__device__ __forceinline__ void item_store(const U4 (&r)[4], uint16_t* ks, uint16_t* vs, int vstr, int key_off,
                                           int item) {
  if (item < 128) chunk_store(r, ks + key_off * kKStr, kKStr, item);
  else chunk_store(r, vs + key_off * vstr, vstr, item - 128);
}

// 4 keys x 1 dim of a V tile [key][dim] (row stride vstr) per lane, transposed by the LDS: the
// 16 lanes of a group read 4 rows x 16 dims (lane j: row j / 4, dims 4 (j % 4) + 0..3 from p)
// and lane i receives dim i of the 4 rows, keys in order.
__device__ __forceinline__ uint2 v_tr4(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) v4s*)(const_cast<uint16_t*>(p))));
}

// The calling thread's item (tid < 256) of the tile whose first row is at
// kbase / vbase (row stride ld elements, 32-bit offsets).  Full tiles load
// without any clamping; only a tile with nvalid < 64 valid rows takes the
// clamped, zero-filling path.
struct TileRegs {
  U4 r[4];
};

template <typename ET>
__device__ __forceinline__ void tile_fetch(TileRegs& t, const ET* __restrict__ kbase,
                                           const ET* __restrict__ vbase, int ld, int nvalid, int tid) {
  const bool is_k = tid < 128;                       // waves 0-1: K chunks; waves 2-3: V chunks
  const ET* base = is_k ? kbase : vbase;
  const int it = tid & 127;
  const int row0 = it >> 3;
  constexpr int rstep = 16;
  const int col = (it & 7) * 8;
  if (nvalid >= kKT) {
    const char* b = reinterpret_cast<const char*>(base);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = static_cast<uint32_t>(((row0 + rstep * j) * ld + col) * (int)sizeof(ET));
      t.r[j] = *reinterpret_cast<const U4*>(b + off);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + rstep * j;
      t.r[j] = masked_load(base + (int64_t)min(row, nvalid - 1) * ld + col, row < nvalid);
    }
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& t, uint16_t* ks, uint16_t* vs, int tid) {
  item_store(t.r, ks, vs, kVStr, 0, tid);
}

// Online-softmax state of one wave (32 query columns).  Each query keeps a
// reference max m (raw score units) that its 16-bit type represents exactly.
// The score chain of a tile starts with one 32x32x8 MFMA step that adds -m to
// every score (A = all ones, B = -m in the first k slot of the query's lane
// < 32), so a probability costs one multiply by the scale and one exp2, with
// no subtraction and no per-tile max.  The reference only moves when a tile
// would give some lane of the wave a probability sum above kGrowSum: that
// tile's scores are then recomputed without the bias, the tile max is taken,
// and the accumulators are rescaled.  Every probability of an accepted tile is
// therefore at most kGrowSum, far below the 16-bit P's overflow.  The first
// tile always takes that path, and so does every tile of a wave in which some
// query's max has left the 16-bit range (|m| > kRefMax, only reachable with
// fp16): that wave keeps m in fp32 and subtracts it per score from then on.
constexpr float kGrowSum = 4096.f;
constexpr float kRefMax = 6.0e4f;   // largest reference magnitude kept as a 16-bit value

struct WaveState {
  f32x16_t acc[2];    // O^T blocks: dims [0,32) and [32,64), column = query
  float m;            // reference max of the lane's query, raw score units (-inf until a key is visible)
  float l;            // partial row sum over this lane's keys, relative to m
  uint32_t bias;      // 16-bit pair (-m, 0) in lanes < 32, zero in lanes >= 32
  bool exact;         // wave-uniform: some query's max left the 16-bit range, m is plain fp32
};

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

// Mask of a tile: key j is kept iff lo_key <= j < hi_key and, for tq >= 0 (a
// real query tq), j <= tq and (win <= 0 or j > tq - win).  Register r of block
// kb holds key key0 + 4 half + off with off = 32 kb + 8 (r/4) + r%4 (< 64); the
// lane's visible offsets form one range [a, b), kept as a 64-bit mask, so each
// score costs a bit extract and a bit select.
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[2], int half, int key0, int lo_key, int hi_key, int tq,
                                          int win) {
  int lo = lo_key, hi = hi_key;
  if (tq >= 0) {
    hi = min(hi, tq + 1);
    if (win > 0) lo = max(lo, tq - win + 1);
  }
  const int base = key0 + 4 * half;
  const int a = min(max(lo - base, 0), 64), b = min(max(hi - base, 0), 64);
  const uint64_t below_b = b >= 64 ? ~0ull : (1ull << b) - 1;
  const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1;
  const uint64_t keep = below_b & ~below_a;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint32_t word = static_cast<uint32_t>(keep >> (32 * kb));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bit = 8 * (r >> 2) + (r & 3);
      const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(word << (31 - bit)) >> 31);
      s[kb][r] = __uint_as_float((__float_as_uint(s[kb][r]) & m) | (0xff800000u & ~m));   // -inf: exp2 gives 0
    }
  }
}

// One 64-key tile: S^T = K Q^T (minus the reference), online softmax,
// O^T += V^T P^T.  ks: [64][kKStr] K rows; vs: [64][vstr] V rows; key0: first
// key index of the tile in the mask's coordinates; sc: log2(e)/sqrt(hd), applied
// in fp32 to the biased scores (P = 2^(sc (s - m))); `first`: the wave's first tile.
template <typename ET>
__device__ __forceinline__ void attend_tile(WaveState& st, const typename Op<ET>::vec (&qf)[4],
                                            const uint16_t* ks, const uint16_t* vs, int vstr, float sc, int lane,
                                            int key0, int lo_key, int hi_key, int tq, int win, bool mask,
                                            bool first) {
  typedef typename Op<ET>::vec4 V4;
  const int col = lane & 31, half = lane >> 5;
  const uint32_t one2 = Pair<ET>::pack(1.f, 1.f);
  const V4 ones = __builtin_bit_cast(V4, make_uint2(one2, one2));
  f32x16_t s[2];
  auto scores = [&](auto biased) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t* krow = ks + (kb * 32 + col) * kKStr + half * 8;
      f32x16_t c = f32x16_t{};
      if constexpr (decltype(biased)::value) c = Op<ET>::mfma8(ones, __builtin_bit_cast(V4, make_uint2(st.bias, 0u)), c);
#pragma unroll
      for (int st4 = 0; st4 < 4; ++st4) {
        const auto a = as_vec<ET>(*reinterpret_cast<const U4*>(krow + st4 * 16));
        c = Op<ET>::mfma(a, qf[st4], c);
      }
      s[kb] = c;
    }
    if (mask) mask_tile(s, half, key0, lo_key, hi_key, tq, win);
  };
  // P^T as 16-bit pairs (B fragments of the P.V steps) and this lane's sum of them
  U4 pw[4];
  float psum;
  auto probs = [&](float sub) {
    const float off = -sub * sc;   // P = 2^(sc (s - sub)) as one FMA per score (one multiply for sub = 0)
    psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(s[kb][hh * 8 + j], sc, off));
        U4 w;
        w.x = Pair<ET>::pack(p[0], p[1]);
        w.y = Pair<ET>::pack(p[2], p[3]);
        w.z = Pair<ET>::pack(p[4], p[5]);
        w.w = Pair<ET>::pack(p[6], p[7]);
        psum = Op<ET>::add_pair(w.x, psum);
        psum = Op<ET>::add_pair(w.y, psum);
        psum = Op<ET>::add_pair(w.z, psum);
        psum = Op<ET>::add_pair(w.w, psum);
        pw[kb * 2 + hh] = w;
      }
  };
  bool slow = first || __builtin_amdgcn_readfirstlane(st.exact);
  if (!slow) {
    scores(std::true_type{});
    probs(0.f);
    slow = __builtin_amdgcn_ballot_w64(psum > kGrowSum) != 0;
  }
  if (slow) {
    scores(std::false_type{});
    float mt = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mt = max3f(mt, s[0][r], s[0][r + 1]);
    mt = max3f(mt, s[0][15], s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) mt = max3f(mt, s[1][r], s[1][r + 1]);
    mt = fmaxf(mt, s[1][15]);
    mt = max_xor32(mt);
    // the new reference: the larger of the old one and the tile max, rounded to the 16-bit type
    // unless some query's max is out of its range (then fp32, for the rest of the wave's tiles)
    float mnew = fmaxf(st.m, mt);
    if (__builtin_amdgcn_ballot_w64(mnew != -INFINITY && fabsf(mnew) > kRefMax) != 0) st.exact = true;
    if (!st.exact && mnew != -INFINITY) mnew = Pair<ET>::lo(Pair<ET>::pack(mnew, 0.f));
    const bool none = mnew == -INFINITY;              // no visible key yet: nothing to rescale
    if (!first) {   // the first tile has nothing accumulated yet
      const float alpha = none ? 1.f : fast_exp2((st.m - mnew) * sc);
      st.l *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[db][r] *= alpha;
    }
    st.m = mnew;
    st.bias = half ? 0u : Pair<ET>::pack(-mnew, 0.f);
    probs(none ? 0.f : mnew);
  }
  st.l += psum;
  // O^T[dim][q] += sum_k V^T[dim][k] P^T[k][q]; PV k-step s covers tile keys
  // [16 s, 16 s + 16); k-index 8 h + j <-> key 16 s + 8 (j/4) + 4 h + j%4.  The A
  // fragment (lane l: dim 32 db + l % 32) comes from two transposed reads of 4 keys:
  // lane group g = l / 16 reads rows 16 s + 4 h (+ 8) + (l % 16) / 4 at dims
  // 32 db + 16 (g % 2) + 4 (l % 4).
  const uint16_t* vlane = vs + (4 * half + ((lane & 15) >> 2)) * vstr + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const uint2 lo = v_tr4(vlane + 16 * s4 * vstr + 32 * db);
      const uint2 hi = v_tr4(vlane + (16 * s4 + 8) * vstr + 32 * db);
      U4 w = {lo.x, lo.y, hi.x, hi.y};
      st.acc[db] = Op<ET>::mfma(as_vec<ET>(w), as_vec<ET>(pw[s4]), st.acc[db]);
    }
  }
}

}  // namespace attn
}  // namespace hymba
