// Many-row projection GEMM on the matrix cores (gfx950):
//
//   Y[m, n] = sum_k X[m, k] W[n, k]          X [M, K], W [N, K] (both K-contiguous, 16-bit)
//
// with fp32 accumulation, Y rounded once to its 16-bit type, and optionally a column range
// [c0, c1) also written in fp32 from the accumulator.  These are the layer's shared input
// projection, its attention lift W_O and its output projection (Hymba summary, "A Fused
// Hybrid-Head Module", Eq. 3: one shared projection feeds both head groups; W_O and the output
// projection are the linear maps on either side of the fused sum), the O(T D^2) part of a
// layer (Griffin summary, "Training speed on longer sequences").
//
// Work split.  A workgroup of four waves owns a 256 x 256 output tile and walks K in 64-wide
// steps.  Each step's X and W slices (256 rows x 128 bytes each) go global -> registers ->
// LDS (two stages, one barrier per step), loaded through buffer resources two steps ahead
// into two register sets.  Wave (wm, wn) owns the 128 x 128 quarter at rows 128 wm, columns
// 128 wn: 4 x 4 blocks of v_mfma_f32_32x32x16 with W rows as the A operand and X rows as the
// B operand, so the accumulator gives each lane one row m of Y and four consecutive columns n
// per register quad.  The epilogue rounds each quarter through LDS and stores whole 256-byte
// row pieces; the fp32 copy goes straight from the accumulator (16 bytes per lane).
//
// LDS rows are 64 elements (128 bytes) with the 16-byte chunks of row r permuted by
// c -> c ^ ((r / 2) % 8): the stores (8 lanes per row) and the fragment reads (lane l: row
// l % 32, elements 8 (l / 32) + 0..7 of a 16-wide k slice) both touch 64 distinct banks per
// 16 lanes.
//
// Tile order.  Workgroups are dealt to the 8 XCDs round robin; workgroup g runs tile
// (g % 8) * (tiles / 8) + g / 8, so each XCD takes one contiguous range of the tile order,
// and that order sweeps the column tiles of 2 row tiles at a time: the X rows and W rows that
// an XCD's resident workgroups read at one time are shared through its L2.
//
// Measured on the 8K input projection (131072 x 11232 x 1600): 4.4 ms, 0.43 of the bf16 MFMA
// peak, against 3.5 ms for hipBLASLt.  The same kernel without the global loads and LDS stores
// of later steps runs at 0.68: the LDS stores of the staged steps, not the products or the
// fragment reads, bound it.
#include <algorithm>

#include "common.h"
#include "gemm_blaslt.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStr = kBK;                  // LDS row stride, 16-bit elements (128 bytes, swizzled)
constexpr int kRowsPerPass = 256 / 8;      // rows one 16-byte load per thread covers
constexpr int kPasses = kBM / kRowsPerPass;   // 8 loads per operand per thread and step
constexpr int kGroupM = 2;                 // row tiles per sweep of the column tiles (2, 4, 8 measured)

struct __align__(16) Chunk { uint32_t x, y, z, w; };

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  __device__ static __forceinline__ f32x16_t run(Chunk a, Chunk b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
};
template <> struct Mfma<half_t> {
  __device__ static __forceinline__ f32x16_t run(Chunk a, Chunk b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                  c, 0, 0, 0);
  }
};

template <typename OT> struct Out4;
template <> struct Out4<half_t> {
  __device__ static __forceinline__ uint2 pack(float a, float b, float c, float d) {
    return make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
  }
};
template <> struct Out4<bf16_t> {
  __device__ static __forceinline__ uint2 pack(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
};

struct Stage {
  uint16_t x[kBM * kStr];
  uint16_t w[kBN * kStr];
};
constexpr int kEp = 128 + 8;   // epilogue LDS row stride (elements) of a wave's 128 x 128 block
constexpr int kSmemBytes = 2 * (int)sizeof(Stage) > 4 * 128 * kEp * 2 ? 2 * (int)sizeof(Stage) : 4 * 128 * kEp * 2;

// LDS position of 16-byte chunk c (0..7) of stage row r: chunk c ^ ((r / 2) % 8) of the row.
// A store of 8 lanes per row puts two consecutive rows (the 16 lanes the LDS serves together)
// on all 64 banks once; a fragment read of one chunk of rows r..r+15 does too.
__device__ __forceinline__ int swz(int r, int c) { return r * kStr + ((c ^ ((r >> 1) & 7)) << 3); }

// Buffer resource over `bytes` bytes from p (gfx9: stride 0, byte range; a read whose offset
// is past the range returns 0), built from wave-uniform values so that it lives in scalar
// registers.  readfirstlane returns a signed int: each half of the address goes through
// uint32_t before widening.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int64_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  const uint64_t u = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < INT32_MAX ? bytes : INT32_MAX));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, n, 0x00020000);
}

constexpr uint32_t kPastRange = 0x80000000u;   // a vector offset past every resource's range

// The 16-byte chunks of one K step this thread loads: rows (tid / 8) + 32 p of the tile,
// elements 8 (tid % 8) + 0..7 of the step.  Each operand's resource covers only the tile's rows
// that exist, so rows past M or N read 0; a chunk past K takes an offset past the range and
// reads 0 too.  The per-lane offset is one register per operand; the pass and the step go in
// the scalar offset.
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t rs_x, __amdgpu_buffer_rsrc_t rs_w, uint32_t vx,
                                          uint32_t vw, int sx, int sw, int k0, bool in_k, Chunk (&rx)[kPasses],
                                          Chunk (&rw)[kPasses]) {
  const uint32_t ox = in_k ? vx : kPastRange, ow = in_k ? vw : kPastRange;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    rx[p] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(rs_x, ox, p * sx + 2 * k0, 0));
    rw[p] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(rs_w, ow, p * sw + 2 * k0, 0));
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ void store_step(Stage& st, int tid, const Chunk (&rx)[kPasses], const Chunk (&rw)[kPasses]) {
  const int o = swz(tid >> 3, tid & 7);   // rows 32 p further keep the same swizzle
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    *reinterpret_cast<uint4*>(&st.x[o + kRowsPerPass * p * kStr]) = make_uint4(rx[p].x, rx[p].y, rx[p].z, rx[p].w);
    *reinterpret_cast<uint4*>(&st.w[o + kRowsPerPass * p * kStr]) = make_uint4(rw[p].x, rw[p].y, rw[p].z, rw[p].w);
  }
}

// The A (W rows) and B (X rows) fragments of one 16-wide k slice of a stage.
struct Frags { Chunk a[4], b[4]; };

// Fragment reads in the order the products of slice_slots first use them.
// wrow, xrow: the lane's slice-0 chunk positions (swz of its rows, chunk lane / 32); chunk
// 2 kk + lane / 32 of the same row is at position ^ (16 kk) (the row base has no low bits set).
__device__ __forceinline__ void read_frags(const Stage& st, int wrow, int xrow, int kk, Frags& f) {
  auto ra = [&](int i) { f.a[i] = *reinterpret_cast<const Chunk*>(&st.w[(wrow ^ (16 * kk)) + i * 32 * kStr]); };
  auto rb = [&](int j) { f.b[j] = *reinterpret_cast<const Chunk*>(&st.x[(xrow ^ (16 * kk)) + j * 32 * kStr]); };
  ra(0); rb(0); rb(1); ra(1); rb(2); ra(2); rb(3); ra(3);
}

// One k slice as 16 issue slots, each pinned in order by a scheduling barrier: slot q issues
// product q in growing-square order (the k-th fragment read of a slice is first needed by
// product 1, 2, 3, 5, 7, 10, 13 for k = 1..8, so the last reads have the most time to land), then (READ) on even q the (q/2)-th fragment read of
// the next slice into nf, (STORE) the q-th chunk of the prefetched step into stage ws, and
// (LOAD) the q-th global load of a later step.  Chunks are stored in the order they were
// loaded, so the wait before each store covers only the loads issued before it, and every
// wait has the products already issued in flight behind it.
struct Loads {
  __amdgpu_buffer_rsrc_t rs_x, rs_w;
  uint32_t ox, ow;   // per-lane offsets (past the range for a chunk past K)
  int sx, sw, k0;    // pass strides and the step's first element
};

template <typename AT, bool READ, int STORE, bool LOAD>
__device__ __forceinline__ void slice_slots(const Frags& f, f32x16_t (&acc)[4][4], const Stage& rs, int wrow,
                                            int xrow, int kk, Frags& nf, Stage& ws, int tid, Chunk (&rx)[kPasses],
                                            Chunk (&rw)[kPasses], const Loads& ld) {
  constexpr int kOrder[16][2] = {{0, 0}, {0, 1}, {1, 0}, {1, 1}, {0, 2}, {1, 2}, {2, 0}, {2, 1},
                                 {2, 2}, {0, 3}, {1, 3}, {2, 3}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
  constexpr int kRead[8][2] = {{0, 0}, {1, 0}, {1, 1}, {0, 1}, {1, 2}, {0, 2}, {1, 3}, {0, 3}};   // (is_b, idx)
  const int o = swz(tid >> 3, tid & 7);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = kOrder[q][0], j = kOrder[q][1];
    acc[i][j] = Mfma<AT>::run(f.a[i], f.b[j], acc[i][j]);
    if constexpr (READ) {
      if (q % 2 == 0) {
        const int b = kRead[q / 2][0], x = kRead[q / 2][1];
        if (b) nf.b[x] = *reinterpret_cast<const Chunk*>(&rs.x[(xrow ^ (16 * kk)) + x * 32 * kStr]);
        else nf.a[x] = *reinterpret_cast<const Chunk*>(&rs.w[(wrow ^ (16 * kk)) + x * 32 * kStr]);
      }
    }
    if constexpr (STORE > 0) {
      if (q % 2 == 0) {   // chunk 8 (STORE - 1) + q / 2 of the prefetched step: x and w alternate
        const int qq = (STORE - 1) * 8 + q / 2, p = qq / 2;
        if (qq % 2 == 0)
          *reinterpret_cast<uint4*>(&ws.x[o + kRowsPerPass * p * kStr]) = make_uint4(rx[p].x, rx[p].y, rx[p].z, rx[p].w);
        else
          *reinterpret_cast<uint4*>(&ws.w[o + kRowsPerPass * p * kStr]) = make_uint4(rw[p].x, rw[p].y, rw[p].z, rw[p].w);
      }
    }
    if constexpr (LOAD) {
      const int p = q / 2;
      if (q % 2 == 0)
        rx[p] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(ld.rs_x, ld.ox, p * ld.sx + 2 * ld.k0, 0));
      else
        rw[p] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(ld.rs_w, ld.ow, p * ld.sw + 2 * ld.k0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename AT, typename OT>
__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(MfmaGemmArgs a) {
  __shared__ __align__(16) char smem[kSmemBytes];
  Stage* lds = reinterpret_cast<Stage*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // tile of this workgroup
  const int tiles_m = static_cast<int>(ceil_div(a.M, kBM)), tiles_n = static_cast<int>(ceil_div(a.N, kBN));
  const int tiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int tm = first_m + (t % per_group) % gm, tn = (t % per_group) / gm;
  const int64_t m0 = (int64_t)tm * kBM;
  const int n0 = tn * kBN;

  // this thread's load offsets: row (tid / 8) of the tile, elements 8 (tid % 8) of a step
  const int kc = (tid & 7) * 8;
  const auto rs_x = tile_rsrc(static_cast<const AT*>(a.x) + m0 * a.ldx, min<int64_t>(a.M - m0, kBM) * a.ldx * 2);
  const auto rs_w = tile_rsrc(static_cast<const AT*>(a.w) + (int64_t)n0 * a.ldw,
                              (int64_t)min(a.N - n0, kBN) * a.ldw * 2);
  const uint32_t vx = static_cast<uint32_t>(((tid >> 3) * a.ldx + kc) * 2);
  const uint32_t vw = static_cast<uint32_t>(((tid >> 3) * a.ldw + kc) * 2);
  const int sx = static_cast<int>(kRowsPerPass * a.ldx * 2), sw = static_cast<int>(kRowsPerPass * a.ldw * 2);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  // Pipeline per K step s (stage s % 2 in LDS; the chunks of steps s + 1 and s + 2 in two
  // register sets, set (s + 1) % 2 holding step s + 1):
  //   slice 0: products beside the fragment reads of the next slice;
  //   slices 1, 2: products beside the reads of the next slice and the stores of step s + 1 to
  //     the other stage (free: every wave passed the previous barrier after its last read of it);
  //   barrier;
  //   slice 3: products beside the reads of step s + 1's slice 0 and the global loads of
  //     step s + 3 into the set just stored.
  // A load is thus issued seven slices before its store.  The last steps store and load too
  // (a stage nobody reads, a clamped valid step), so that the loop body has no branches.
  const int wrow = swz(wn * 128 + (lane & 31), lane >> 5);
  const int xrow = swz(wm * 128 + (lane & 31), lane >> 5);
  Chunk rxa[kPasses], rwa[kPasses], rxb[kPasses], rwb[kPasses];
  Frags f0, f1;
  const int steps = static_cast<int>(ceil_div(a.K, kBK));
  auto loads_of = [&](int st) {
    const int k0 = min(st, steps - 1) * kBK;
    const bool in_k = k0 + kc < a.K;
    return Loads{rs_x, rs_w, in_k ? vx : kPastRange, in_k ? vw : kPastRange, sx, sw, k0};
  };
  auto load_set = [&](int st, Chunk (&rx)[kPasses], Chunk (&rw)[kPasses]) {
    const Loads l = loads_of(st);
    load_step(l.rs_x, l.rs_w, vx, vw, sx, sw, l.k0, l.k0 + kc < a.K, rx, rw);
  };
  load_set(0, rxa, rwa);
  store_step(lds[0], tid, rxa, rwa);
  load_set(1, rxb, rwb);
  load_set(2, rxa, rwa);
  __syncthreads();
  read_frags(lds[0], wrow, xrow, 0, f0);
  // one step; (rx, rw) holds step s + 1 and is refilled with step s + 3
  auto step = [&](int s, Chunk (&rx)[kPasses], Chunk (&rw)[kPasses]) {
    const Stage& st = lds[s & 1];
    Stage& nx = lds[(s + 1) & 1];
    const Loads ld = loads_of(s + 3);
    slice_slots<AT, true, 0, false>(f0, acc, st, wrow, xrow, 1, f1, nx, tid, rx, rw, ld);
    slice_slots<AT, true, 1, false>(f1, acc, st, wrow, xrow, 2, f0, nx, tid, rx, rw, ld);
    slice_slots<AT, true, 2, false>(f0, acc, st, wrow, xrow, 3, f1, nx, tid, rx, rw, ld);
    __syncthreads();
    slice_slots<AT, true, 0, true>(f1, acc, nx, wrow, xrow, 0, f0, nx, tid, rx, rw, ld);
  };
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, rxb, rwb);
    step(s + 1, rxa, rwa);
  }
  if (s < steps) step(s, rxb, rwb);

  // Epilogue.  acc[i][j] register 4 g + q is Y[m, n] at m = m0 + 128 wm + 32 j + lane % 32,
  // n = n0 + 128 wn + 32 i + 8 g + 4 (lane / 32) + q.  Each wave rounds its 128 x 128 quarter
  // into its own LDS block (rows of 128 + 8 elements), then stores it row by row: 16 lanes
  // write one row's 256 contiguous bytes.  The fp32 copy of the columns [c0, c1) goes straight
  // from the accumulator (16 bytes per lane).
  __syncthreads();   // the last fragment reads of every wave have landed: the stages are free
  uint16_t* ep = reinterpret_cast<uint16_t*>(smem) + wave * 128 * kEp;
  const int frow = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16_t& c = acc[i][j];
        *reinterpret_cast<uint2*>(ep + (32 * j + frow) * kEp + 32 * i + 8 * g + 4 * (lane >> 5)) =
            Out4<OT>::pack(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
      }
  if (a.y32 && n0 + wn * 128 < a.c1 && n0 + wn * 128 + 128 > a.c0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 128 + j * 32 + frow;
      if (m >= a.M) continue;
      float* brow = a.y32 + m * a.ldy32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
          const f32x16_t& c = acc[i][j];
          if (n >= a.c0 && n < a.c1)
            *reinterpret_cast<float4*>(brow + (n - a.c0)) =
                make_float4(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
        }
    }
  }
  __syncthreads();   // each wave reads back only its own block; the barrier orders the LDS writes
  OT* Y = static_cast<OT*>(a.y);
  const int rr = lane >> 4, cc = (lane & 15) * 8;
  const int n = n0 + wn * 128 + cc;
  const bool wide = (a.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(a.y) % 16) == 0;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int r = it * 4 + rr;
    const int64_t m = m0 + wm * 128 + r;
    if (m >= a.M || n >= a.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(ep + r * kEp + cc);
    OT* dst = Y + m * a.ldy + n;
    if (wide && n + 8 <= a.N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {   // 8-byte pieces (rows only 8-byte aligned, or the last 4 columns of N)
      *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
      if (n + 8 <= a.N) *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
    }
  }
}

template <typename AT, typename OT>
hipError_t launch(const MfmaGemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!mfma_gemm_shape_ok(a)) return hipErrorInvalidValue;
  const int64_t tiles = ceil_div(a.M, kBM) * ceil_div(a.N, kBN);
  hipLaunchKernelGGL((gemm_mfma_kernel<AT, OT>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool mfma_gemm_shape_ok(const MfmaGemmArgs& a) {
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; };
  if (a.K <= 0 || a.K % 8 || a.N % 4 || a.ldx % 8 || a.ldw % 8 || a.ldy % 4) return false;
  if (!al(a.x, 16) || !al(a.w, 16) || !al(a.y, 8)) return false;
  if (a.ldx < a.K || a.ldw < a.K || a.ldy < a.N) return false;
  if (ceil_div(a.M, kBM) * ceil_div(a.N, kBN) > 0x7fffffff) return false;
  if (a.y32) {
    if (a.c0 % 4 || a.c1 % 4 || a.c0 < 0 || a.c1 > a.N || a.c0 > a.c1 || a.ldy32 % 4 || a.ldy32 < a.c1 - a.c0)
      return false;
    if (!al(a.y32, 16)) return false;
  }
  return true;
}

hipError_t launch_mfma_gemm(const MfmaGemmArgs& a, int in_type, int out_type, hipStream_t s) {
  if (in_type == GT_BF16 && out_type == GT_F16) return launch<bf16_t, half_t>(a, s);
  if (in_type == GT_BF16 && out_type == GT_BF16) return launch<bf16_t, bf16_t>(a, s);
  if (in_type == GT_F16 && out_type == GT_F16) return launch<half_t, half_t>(a, s);
  if (in_type == GT_F16 && out_type == GT_BF16) return launch<half_t, bf16_t>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace hymba
