// hipBLASLt plans for the three projections of the mixer (shared input
// projection, attention W_O, output projection).  Row-major Y = X W^T is the
// column-major product Y^T = W^T-op(A = W) x X: A = W with op T (K-contiguous),
// B = X with op N, both K-contiguous ("TN"), the layout MFMA GEMMs prefer.
// Plans (descriptors + algorithm) are cached per device and shape.  The
// algorithm is the fastest of hipBLASLt's heuristic candidates -- for GEMMs of
// more than ~50 GFLOP also of the library's other kernels with the same macro
// tile as its top picks -- timed once on the first call's own operands and
// stream (skipped while the stream is being captured, or when the environment
// sets HYMBA_GEMM_TUNE=0: then the first heuristic candidate is taken).  Real
// operands matter: these GEMMs run power-limited, and bit toggling in the
// data moves the clock.
#include "gemm_blaslt.h"
#include "kernels.h"

#include <hipblaslt/hipblaslt.h>
#include <hipblaslt/hipblaslt-ext.hpp>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

namespace hymba {

namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
};

using Key = std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, size_t>;

hipDataType dt_of(GemmType t) { return t == GT_F16 ? HIP_R_16F : t == GT_BF16 ? HIP_R_16BF : HIP_R_32F; }

struct State {
  std::mutex mu;
  std::map<int, hipblasLtHandle_t> handles;
  std::map<Key, Plan> plans;
};

State& state() {
  static State* s = new State();   // lives until process exit (handles are per device)
  return *s;
}

bool env_flag(const char* name, bool dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::strcmp(v, "0") != 0;
}

// Mean milliseconds of `reps` runs of one candidate (after one untimed run), or a negative value if
// it fails.  With `spin_us` > 0 a wait kernel of that length runs first, so that the timed calls are
// all queued before the first starts and run back to back: for a few-microsecond GEMM the
// library's host time per call (~17 us) is longer than the kernel, and without the wait the
// candidates would all time at the host's pace.
float time_candidate(hipblasLtHandle_t handle, const Plan& p, const hipblasLtMatmulAlgo_t& algo, const void* W,
                     const void* X, void* Y, void* ws, size_t ws_bytes, hipStream_t s, int reps, int spin_us) {
  const float alpha = 1.f, beta = 0.f;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) { hipEventDestroy(e0); return -1.f; }
  float ms = -1.f;
  bool ok = hipblasLtMatmul(handle, p.desc, &alpha, W, p.la, X, p.lb, &beta, Y, p.lc, Y, p.lc, &algo, ws,
                            ws_bytes, s) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && (spin_us <= 0 || launch_spin(spin_us, s) == hipSuccess);
  ok = ok && hipEventRecord(e0, s) == hipSuccess;
  for (int r = 0; ok && r < reps; ++r)
    ok = hipblasLtMatmul(handle, p.desc, &alpha, W, p.la, X, p.lb, &beta, Y, p.lc, Y, p.lc, &algo, ws, ws_bytes,
                         s) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
  if (ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess) ms /= reps;
  else ms = -1.f;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ms;
}

// Macro-tile tag ("MT256x256x64") of a kernel name, or "".
std::string macro_tile(const std::string& name) {
  const size_t a = name.find("_MT");
  if (a == std::string::npos) return "";
  const size_t b = name.find('_', a + 3);
  return name.substr(a + 1, b == std::string::npos ? std::string::npos : b - a - 1);
}

// Appends up to 48 supported algorithms whose macro tile matches one of the top three heuristic
// candidates' (hipBLASLt's heuristic ranks few of each tile's variants).
void add_same_tile_algos(hipblasLtHandle_t handle, const Plan& p, GemmType in_type, GemmType out_type,
                         hipblasLtMatmulHeuristicResult_t* res, int n, size_t ws_bytes,
                         std::vector<hipblasLtMatmulAlgo_t>& cand) {
  std::vector<std::string> tiles;
  for (int i = 0; i < n && i < 3; ++i) {
    const std::string t = macro_tile(hipblaslt_ext::getKernelNameFromAlgo(handle, res[i].algo));
    if (!t.empty()) tiles.push_back(t);
  }
  if (tiles.empty()) return;
  std::vector<hipblasLtMatmulHeuristicResult_t> all;
  if (hipblaslt_ext::getAllAlgos(handle, hipblaslt_ext::GemmType::HIPBLASLT_GEMM, HIPBLAS_OP_T, HIPBLAS_OP_N,
                                 dt_of(in_type), dt_of(in_type), dt_of(out_type), dt_of(out_type),
                                 HIPBLAS_COMPUTE_32F, all) != HIPBLAS_STATUS_SUCCESS)
    return;
  const float alpha = 1.f, beta = 0.f;
  int added = 0;
  for (auto& r : all) {
    if (added >= 48) break;
    const std::string t = macro_tile(hipblaslt_ext::getKernelNameFromAlgo(handle, r.algo));
    if (std::find(tiles.begin(), tiles.end(), t) == tiles.end()) continue;
    const int idx = hipblaslt_ext::getIndexFromAlgo(r.algo);
    bool dup = false;
    for (auto& c : cand) dup = dup || hipblaslt_ext::getIndexFromAlgo(c) == idx;
    if (dup) continue;
    size_t need = 0;
    if (hipblaslt_ext::matmulIsAlgoSupported(handle, p.desc, &alpha, p.la, p.lb, &beta, p.lc, p.lc, r.algo, need) !=
            HIPBLAS_STATUS_SUCCESS ||
        need > ws_bytes)
      continue;
    cand.push_back(r.algo);
    ++added;
  }
}

}  // namespace

int gemm_16(GemmType in_type, GemmType out_type, const void* X, int64_t ldx, const void* W, int64_t ldw,
            void* Y, int64_t ldy, int64_t rows, int64_t out, int64_t in, void* ws, size_t ws_bytes,
            hipStream_t s, const char** err) {
  if (rows <= 0 || out <= 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { *err = "hipGetDevice failed"; return -5; }
  State& st = state();
  Plan plan;
  hipblasLtHandle_t handle;
  {
    std::lock_guard<std::mutex> lock(st.mu);
    auto hit = st.handles.find(dev);
    if (hit == st.handles.end()) {
      hipblasLtHandle_t h;
      if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtCreate failed"; return -5; }
      hit = st.handles.emplace(dev, h).first;
    }
    handle = hit->second;
    const Key key{dev, static_cast<int>(in_type), static_cast<int>(out_type), rows, out, in, ldx, ldw, ldy, ws_bytes};
    auto it = st.plans.find(key);
    if (it == st.plans.end()) {
      Plan p;
      hipblasOperation_t opA = HIPBLAS_OP_T, opB = HIPBLAS_OP_N;
      bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
      ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opA, sizeof(opA)) == HIPBLAS_STATUS_SUCCESS;
      ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opB, sizeof(opB)) == HIPBLAS_STATUS_SUCCESS;
      // A: W stored [out, in] row-major = column-major (in x out), ld = ldw
      ok = ok && hipblasLtMatrixLayoutCreate(&p.la, dt_of(in_type), in, out, ldw) == HIPBLAS_STATUS_SUCCESS;
      // B: X stored [rows, in] row-major = column-major (in x rows), ld = ldx
      ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, dt_of(in_type), in, rows, ldx) == HIPBLAS_STATUS_SUCCESS;
      // C/D: Y stored [rows, out] row-major = column-major (out x rows), ld = ldy
      ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, dt_of(out_type), out, rows, ldy) == HIPBLAS_STATUS_SUCCESS;
      if (!ok) { *err = "hipBLASLt descriptor creation failed"; return -5; }
      hipblasLtMatmulPreference_t pref;
      uint64_t wsb = ws_bytes;
      hipblasLtMatmulPreferenceCreate(&pref);
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
      constexpr int kCand = 16;
      hipblasLtMatmulHeuristicResult_t res[kCand];
      int n = 0;
      const hipblasStatus_t hs = hipblasLtMatmulAlgoGetHeuristic(handle, p.desc, p.la, p.lb, p.lc, p.lc,
                                                                 pref, kCand, res, &n);
      hipblasLtMatmulPreferenceDestroy(pref);
      if (hs != HIPBLAS_STATUS_SUCCESS || n == 0) {
        *err = "hipBLASLt found no algorithm for this GEMM shape";
        return -2;
      }
      std::vector<hipblasLtMatmulAlgo_t> cand;
      for (int i = 0; i < n; ++i)
        if (res[i].workspaceSize <= ws_bytes) cand.push_back(res[i].algo);
      if (cand.empty()) {
        *err = "hipBLASLt found no algorithm within the workspace";
        return -2;
      }
      int best = 0;
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cap) != hipSuccess) cap = hipStreamCaptureStatusActive;
      if (cap == hipStreamCaptureStatusNone && env_flag("HYMBA_GEMM_TUNE", true)) {
        if (2.0 * rows * out * in > 5e10) add_same_tile_algos(handle, p, in_type, out_type, res, n, ws_bytes, cand);
        const bool log = env_flag("HYMBA_GEMM_TUNE_LOG", false);
        // a few-microsecond GEMM (a decode step's projection) is timed over more runs: two runs
        // of ~20 us each left the choice to timer noise
        const int reps = 2.0 * rows * out * in < 1e11 ? 12 : 2;
        float best_ms = -1.f;
        for (size_t i = 0; cand.size() > 1 && i < cand.size(); ++i) {
          const float ms = time_candidate(handle, p, cand[i], W, X, Y, ws, ws_bytes, s, reps,
                                          reps > 2 ? 40 * reps : 0);
          if (log)
            std::fprintf(stderr, "[hymba gemm] rows %lld out %lld in %lld candidate %zu: %.4f ms\n",
                         (long long)rows, (long long)out, (long long)in, i, ms);
          if (ms > 0.f && (best_ms < 0.f || ms < best_ms)) { best_ms = ms; best = static_cast<int>(i); }
        }
      }
      p.algo = cand[best];
      it = st.plans.emplace(key, p).first;
    }
    plan = it->second;
  }
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t rs = hipblasLtMatmul(handle, plan.desc, &alpha, W, plan.la, X, plan.lb, &beta, Y,
                                             plan.lc, Y, plan.lc, &plan.algo, ws, ws_bytes, s);
  if (rs != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtMatmul failed"; return -5; }
  return 0;
}

}  // namespace hymba
