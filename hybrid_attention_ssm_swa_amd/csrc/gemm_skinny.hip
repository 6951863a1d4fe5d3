// Weight-streaming GEMM for few rows (decode): Y[M, N] = X[M, K] . W[N, K]^T with
// 16-bit operands and fp32 accumulation on v_mfma_f32_32x32x16_{f16,bf16}.
//
// At M ~ 128 the product moves W (N*K 16-bit words) through the chip once against
// 2*M*N*K flops, and what limits it is how fast each CU takes data in (measured on
// MI355X: ~25-40 GB/s per CU from HBM, ~80 GB/s from L2 when neighbours share the
// lines).  So the design keeps the bytes per CU low and a lot of them in flight:
//  * a workgroup of 8 waves owns F (64 or 32) output features x 32 rows over the whole
//    of K: K is never split across workgroups, so there are no partial sums in memory
//    and no second kernel;
//  * the row blocks of one feature tile get consecutive slots on one XCD (workgroups
//    are dealt to the 8 XCDs round-robin), so W comes from HBM once and from that XCD's
//    L2 for the other row blocks; X (M x K, small) stays in L2;
//  * K is walked in phases of 512: each phase's W and X tiles are loaded coalesced (a
//    wave's 64 lanes read one 1 KB row segment) into registers two phases ahead, then
//    staged in LDS (row stride 1040 B: the MFMA operand reads are conflict-free);
//  * in a phase wave w multiplies the 64-k chunk w; at the end the 8 waves'
//    accumulators are added in wave order through LDS (deterministic);
//  * the product is computed transposed, C = W . X^T, so a lane holds 4 consecutive
//    features of one row per register group.
// An optional fp32 copy of the output columns [c0, c1) goes to y32 (the decode path's
// B/C columns, which the scan reads in fp32).  X may be bf16 with W fp16: it is
// converted on its way into LDS (exact in range).
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

#ifndef HYMBA_RW_WAVES
#define HYMBA_RW_WAVES 8
#endif
#ifndef HYMBA_RW_PHASE_K
#define HYMBA_RW_PHASE_K 512
#endif
#ifndef HYMBA_RW_DEPTH
#define HYMBA_RW_DEPTH 2
#endif
constexpr int kRwR = 32;                   // rows per workgroup
constexpr int kRwWaves = HYMBA_RW_WAVES;
constexpr int kRwThreads = 64 * kRwWaves;
constexpr int kRwPhaseK = HYMBA_RW_PHASE_K;   // k per phase
constexpr int kRwDepth = HYMBA_RW_DEPTH;      // phases in flight
constexpr int kRwStr = kRwPhaseK + 8;      // LDS row stride in 16-bit words (conflict-free MFMA reads)
constexpr int kRwSegs = kRwPhaseK / 8;     // 16-byte segments of a row's phase
constexpr int kRwChunks = kRwPhaseK / 64 / kRwWaves;   // 64-k chunks per wave and phase
static_assert(kRwChunks >= 1 && kRwThreads % kRwSegs == 0, "phase shape");
constexpr int kRwMaxUnrolled = 8;          // K walks of up to this many phases are unrolled

struct __align__(16) Q4 { uint32_t x, y, z, w; };

// cache policy of the weight loads: the default (allocate).  A decode step re-reads every weight,
// and with the K/V caches read non-temporally the weights stay in the 256 MB MALL from one step to
// the next (non-temporal weight loads measured 1.5 % slower per decode pair step).
constexpr int kWeightCachePolicy = 0;

// v if keep, else zeros: per 32-bit word (a select of the whole struct is lowered through
// scratch memory)
__device__ __forceinline__ Q4 keep_or_zero(bool keep, Q4 v) {
  Q4 r;
  r.x = keep ? v.x : 0u;
  r.y = keep ? v.y : 0u;
  r.z = keep ? v.z : 0u;
  r.w = keep ? v.w : 0u;
  return r;
}

template <typename WT> struct Mfma;
template <> struct Mfma<half_t> {
  __device__ static __forceinline__ f32x16_t run(Q4 a, Q4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
};
template <> struct Mfma<bf16_t> {
  __device__ static __forceinline__ f32x16_t run(Q4 a, Q4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
};

// 8 elements of X's type -> 8 elements of W's type
template <typename XT, typename WT> struct ToW {
  __device__ static __forceinline__ Q4 run(Q4 v) { return v; }
};
template <> struct ToW<bf16_t, half_t> {
  __device__ static __forceinline__ Q4 run(Q4 v) {
    Q4 r;
    r.x = pack_f16x2(bf16lo(v.x), bf16hi(v.x));
    r.y = pack_f16x2(bf16lo(v.y), bf16hi(v.y));
    r.z = pack_f16x2(bf16lo(v.z), bf16hi(v.z));
    r.w = pack_f16x2(bf16lo(v.w), bf16hi(v.w));
    return r;
  }
};

template <typename OT> struct Out4;
template <> struct Out4<half_t> {
  __device__ static __forceinline__ void store(half_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
  }
};
template <> struct Out4<bf16_t> {
  __device__ static __forceinline__ void store(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
};
template <> struct Out4<float> {
  __device__ static __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

// Buffer resource (gfx9: stride 0, byte range; reads whose vector offset is past the range
// return 0) built from wave-uniform values, so that its loads need no per-lane loop.
// readfirstlane returns a signed int: each half goes through uint32_t before widening, or a low
// word with bit 31 set would sign-extend into the high word and wreck the base address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int64_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  const uint64_t u = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < INT32_MAX ? bytes : INT32_MAX));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, n, 0x00020000);
}

// Loads of one phase: LW segments of W's tile rows and LX of X's, 16 bytes each.
template <int F>
struct RwPhase {
  static constexpr int LW = F * kRwSegs / kRwThreads;
  static constexpr int LX = kRwR * kRwSegs / kRwThreads;
  Q4 r[LW + LX];
};

// Workgroup i: XCD i % 8, slot i / 8 on it; slot -> (feature tile 8 (slot / rbs) + xcd,
// row block slot % rbs).
// NPH > 0: the K walk has exactly NPH phases and is unrolled (straight-line code, so each wait
// covers just the oldest register set); NPH == 0: a loop for any K (it drains all loads in flight
// every three phases, which the compiler's waits at the loop head force).
template <typename WT, typename XT, typename OT, int F, int NPH>
__global__ __launch_bounds__(kRwThreads) void rows_gemm_kernel(SkinnyArgs<WT, XT, OT> a, int tiles, int rbs) {
  constexpr int LW = RwPhase<F>::LW, LX = RwPhase<F>::LX, FB = F / 32;
  // staging: W rows [0, F), then X rows [F, F + 32); afterwards the waves' accumulators
  constexpr int kStage = (F + kRwR) * kRwStr, kRed = kRwWaves * FB * 4 * 64 * 8;
  __shared__ __align__(16) uint16_t lds[kStage > kRed ? kStage : kRed];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int tile = xcd + 8 * (slot / rbs), rb = slot % rbs;
  if (tile >= tiles) return;   // uniform over the workgroup
  const int f0 = tile * F, m0 = rb * kRwR;
  const int nph = NPH > 0 ? NPH : static_cast<int>(ceil_div(a.K, kRwPhaseK));
  // Buffer resources with the whole byte offset in the per-lane offset (range-checked): rows
  // past N (M) are clamped to N (M), i.e. wholly past the range, and read as zeros.  Phases past
  // the end load through a zero-length resource: no memory access, zeros.
  const auto rs_w = uniform_rsrc(a.w, int64_t(a.N) * a.ldw * 2);
  const auto rs_x = uniform_rsrc(a.x, int64_t(a.M) * a.ldx * 2);
  const auto rs_0 = uniform_rsrc(a.w, 0);
  // the thread's segments: row tid / kRwSegs + q * (threads / kRwSegs), 16 bytes at k 8 * seg
  constexpr int kRowStep = kRwThreads / kRwSegs;
  const int row0 = tid / kRwSegs, seg = tid % kRwSegs;
  uint32_t vw[LW], vx[LX];
#pragma unroll
  for (int q = 0; q < LW; ++q)
    vw[q] = static_cast<uint32_t>(((int64_t)min(f0 + row0 + kRowStep * q, a.N) * a.ldw + 8 * seg) * 2);
#pragma unroll
  for (int q = 0; q < LX; ++q)
    vx[q] = static_cast<uint32_t>(((int64_t)min(m0 + row0 + kRowStep * q, a.M) * a.ldx + 8 * seg) * 2);
  auto issue = [&](RwPhase<F>& ph, int p) {
    const bool live = p < nph;   // uniform
    const auto rw = live ? rs_w : rs_0;
    const auto rx = live ? rs_x : rs_0;
    const uint32_t kb = live ? static_cast<uint32_t>(p) * kRwPhaseK * 2 : 0u;
#pragma unroll
    for (int q = 0; q < LW; ++q)
      ph.r[q] = __builtin_bit_cast(Q4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw[q] + kb, 0, kWeightCachePolicy));
#pragma unroll
    for (int q = 0; q < LX; ++q)
      ph.r[LW + q] = __builtin_bit_cast(Q4, __builtin_amdgcn_raw_buffer_load_b128(rx, vx[q] + kb, 0, 0));
    // keep the phases' loads in phase order: a wait for the oldest set then leaves the later
    // ones in flight
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x16_t acc[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) acc[fb] = f32x16_t{};
  auto consume = [&](const RwPhase<F>& ph, int p) {
    const int k0 = p * kRwPhaseK;
    const bool kin = k0 + 8 * seg < a.K;   // K % 8 == 0: a 16-byte segment is wholly in or out
    __syncthreads();   // every wave is done with the previous phase's tiles
#pragma unroll
    for (int q = 0; q < LW; ++q)
      *reinterpret_cast<Q4*>(&lds[(row0 + kRowStep * q) * kRwStr + 8 * seg]) = keep_or_zero(kin, ph.r[q]);
#pragma unroll
    for (int q = 0; q < LX; ++q)
      *reinterpret_cast<Q4*>(&lds[(F + row0 + kRowStep * q) * kRwStr + 8 * seg]) =
          keep_or_zero(kin, ToW<XT, WT>::run(ph.r[LW + q]));
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kRwChunks; ++c) {
      const int ch = w + kRwWaves * c;   // the wave's 64-k chunk of the phase
      if (k0 + 64 * ch >= a.K) break;     // uniform
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = 64 * ch + 16 * s + 8 * (lane >> 5);
        const Q4 xb = *reinterpret_cast<const Q4*>(&lds[(F + (lane & 31)) * kRwStr + kk]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          const Q4 wa = *reinterpret_cast<const Q4*>(&lds[(32 * fb + (lane & 31)) * kRwStr + kk]);
          acc[fb] = Mfma<WT>::run(wa, xb, acc[fb]);
        }
      }
    }
  };
  // kRwDepth phases in flight: the register sets rotate with the phase index
  if constexpr (NPH > 0) {
    RwPhase<F> r[kRwDepth];
#pragma unroll
    for (int p = 0; p < kRwDepth && p < NPH; ++p) issue(r[p], p);
#pragma unroll
    for (int p = 0; p < NPH; ++p) {
      consume(r[p % kRwDepth], p);
      if (p + kRwDepth < NPH) issue(r[p % kRwDepth], p + kRwDepth);
    }
  } else {
    RwPhase<F> r0, r1, r2;
    issue(r0, 0);
    issue(r1, 1);
    issue(r2, 2);
    for (int p = 0; p < nph; p += 3) {
      consume(r0, p);
      issue(r0, p + 3);
      if (p + 1 >= nph) break;
      consume(r1, p + 1);
      issue(r1, p + 4);
      if (p + 2 >= nph) break;
      consume(r2, p + 2);
      issue(r2, p + 5);
    }
  }

  // sum of the 8 waves' accumulators, in wave order: float4 (w, fb, g, lane) in LDS
  __syncthreads();
  float4* red = reinterpret_cast<float4*>(lds);
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      red[((w * FB + fb) * 4 + g) * 64 + lane] =
          make_float4(acc[fb][4 * g], acc[fb][4 * g + 1], acc[fb][4 * g + 2], acc[fb][4 * g + 3]);
  __syncthreads();
  for (int j = tid; j < FB * 256; j += kRwThreads) {
    const int ln = j & 63, g = (j >> 6) & 3, fb = j >> 8;
    float4 s4 = red[j];
#pragma unroll
    for (int ww = 1; ww < kRwWaves; ++ww) {
      const float4 v = red[ww * FB * 256 + j];
      s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
    }
    // float4 (fb, g, ln): row m0 + ln % 32, features f0 + 32 fb + 8 g + 4 (ln / 32) + 0..3
    const int m = m0 + (ln & 31), f = f0 + 32 * fb + 8 * g + 4 * (ln >> 5);
    if (m >= a.M || f >= a.N) continue;   // N % 4 == 0: a group is wholly in or out
    Out4<OT>::store(a.y + (int64_t)m * a.ldy + f, s4.x, s4.y, s4.z, s4.w);
    if (a.y32 && f >= a.c0 && f < a.c1)   // c0, c1 multiples of 4
      Out4<float>::store(a.y32 + (int64_t)m * a.ldy32 + (f - a.c0), s4.x, s4.y, s4.z, s4.w);
  }
}

template <typename WT, typename XT, typename OT, int F>
void rows_launch(int64_t nph, dim3 grid, hipStream_t s, const SkinnyArgs<WT, XT, OT>& a, int tiles, int rbs) {
  const dim3 block(kRwThreads);
#define HYMBA_RW_CASE(n)                                                                              \
  case n:                                                                                             \
    if constexpr (n <= kRwMaxUnrolled) {                                                              \
      hipLaunchKernelGGL((rows_gemm_kernel<WT, XT, OT, F, n>), grid, block, 0, s, a, tiles, rbs);     \
      return;                                                                                         \
    }                                                                                                 \
    break;
  switch (nph) {
    HYMBA_RW_CASE(1) HYMBA_RW_CASE(2) HYMBA_RW_CASE(3) HYMBA_RW_CASE(4)
    HYMBA_RW_CASE(5) HYMBA_RW_CASE(6) HYMBA_RW_CASE(7) HYMBA_RW_CASE(8)
    HYMBA_RW_CASE(9) HYMBA_RW_CASE(10) HYMBA_RW_CASE(11) HYMBA_RW_CASE(12)
    HYMBA_RW_CASE(13) HYMBA_RW_CASE(14) HYMBA_RW_CASE(15) HYMBA_RW_CASE(16)
    default: break;
  }
#undef HYMBA_RW_CASE
  hipLaunchKernelGGL((rows_gemm_kernel<WT, XT, OT, F, 0>), grid, block, 0, s, a, tiles, rbs);
}

template <typename WT, typename XT, typename OT>
hipError_t rows_dispatch(const SkinnyArgs<WT, XT, OT>& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.N % 4 || a.K % 8 || a.K <= 0 || a.ldw % 8 || a.ldx % 8 || a.ldy % 4 || a.c0 % 4 || a.c1 % 4 ||
      (a.y32 && a.ldy32 % 4))
    return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(a.w) % 16 || reinterpret_cast<uintptr_t>(a.x) % 16 ||
      reinterpret_cast<uintptr_t>(a.y) % 16 || reinterpret_cast<uintptr_t>(a.y32) % 16)
    return hipErrorInvalidValue;
  // buffer offsets are 32-bit: the clamped row (N, M) plus the last phase's reach stays below 2 GiB
  const int64_t reach = ceil_div(a.K, kRwPhaseK) * kRwPhaseK * 2;
  if (((int64_t)a.N + 1) * a.ldw * 2 + reach >= INT32_MAX || ((int64_t)a.M + 1) * a.ldx * 2 + reach >= INT32_MAX)
    return hipErrorInvalidValue;
  const int F = skinny_plan(a.M, a.N, a.K).F;
  const int tiles = static_cast<int>(ceil_div(a.N, F)), rbs = static_cast<int>(ceil_div(a.M, kRwR));
  const int64_t groups = 8 * ceil_div(tiles, 8) * rbs;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups)), block(kRwThreads);
  const int64_t nph = ceil_div(a.K, kRwPhaseK);
  if (F == 64) rows_launch<WT, XT, OT, 64>(nph, grid, s, a, tiles, rbs);
  else rows_launch<WT, XT, OT, 32>(nph, grid, s, a, tiles, rbs);
  return hipGetLastError();
}

}  // namespace

// Feature tile: 64 when that gives at least 128 workgroups, else 32 (twice the workgroups, X
// read twice as often).
#ifndef HYMBA_RW_F64_MIN_GROUPS
#define HYMBA_RW_F64_MIN_GROUPS 128
#endif
SkinnyPlan skinny_plan(int M, int N, int K) {
  (void)K;
  SkinnyPlan p;
  p.F = ceil_div(N, 64) * ceil_div(M, kRwR) >= HYMBA_RW_F64_MIN_GROUPS ? 64 : 32;
  return p;
}

hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, half_t>& a, hipStream_t s) { return rows_dispatch(a, s); }
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, bf16_t, half_t>& a, hipStream_t s) { return rows_dispatch(a, s); }
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, bf16_t>& a, hipStream_t s) { return rows_dispatch(a, s); }
hipError_t launch_skinny_gemm(const SkinnyArgs<bf16_t, bf16_t, bf16_t>& a, hipStream_t s) { return rows_dispatch(a, s); }

}  // namespace hymba
