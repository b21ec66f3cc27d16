// bf16 GEMM with both operands contraction-contiguous, for the merge's
// backward (the merge forward's kernel with a row pitch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

// out[M, N] (bf16, row pitch N) = a[M, Kc] bt[N, Kc]^T with fp32
// accumulation; a and bt row-major with row pitch Kc.  Kc % 128 == 0, and
// each operand must span at most 2^31 - 16 bytes.
hipError_t launch_gemm_nt_bf16(const uint16_t* a, const uint16_t* bt, uint16_t* out, long long M,
                               long long Kc, int N, hipStream_t s);

}  // namespace vdn
