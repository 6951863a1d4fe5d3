// Projection GEMMs through hipBLASLt: Y[rows, out] = X[rows, in] . W[out, in]^T
// with 16-bit inputs, fp32 accumulation and the requested output type.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hymba {

// Returns 0 on success; on failure a negative status and a message in *err.
enum GemmType { GT_F16 = 0, GT_BF16 = 1, GT_F32 = 2 };

int gemm_16(GemmType in_type, GemmType out_type, const void* X, int64_t ldx, const void* W, int64_t ldw,
            void* Y, int64_t ldy, int64_t rows, int64_t out, int64_t in, void* ws, size_t ws_bytes,
            hipStream_t s, const char** err);

constexpr size_t kGemmWorkspaceBytes = size_t(64) << 20;

}  // namespace hymba
