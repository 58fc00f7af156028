// qgemv_launch.h -- internal launchers (host side), one per kernel family.
// Arguments have already been validated by qgemv_api.cpp; each launcher picks
// a launch geometry, enqueues one kernel on `stream` and returns the HIP status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

hipError_t launch_int4_gemv(const uint16_t* x, int64_t ldx, const uint8_t* w,
                            const uint16_t* scales, const uint8_t* zp, void* y,
                            int64_t ldy, int y_type, int M, int N, int K,
                            int block_size, hipStream_t stream);

hipError_t launch_q4k_gemv(const float* x, int64_t ldx, const uint8_t* w,
                           const float* dsc, float* y, int64_t ldy, int M, int N,
                           int K, hipStream_t stream);

hipError_t launch_q4k_build_plane(const uint8_t* w, float* dsc, int N, int K,
                                  hipStream_t stream);

hipError_t launch_bf16_gemv(const uint16_t* x, int64_t ldx, const uint16_t* w,
                            int64_t ldw, void* y, int64_t ldy, int y_type, int M,
                            int N, int K, hipStream_t stream);

// LDS budget per workgroup for staged activations (bytes).
constexpr int kLdsBudget = 64 * 1024;

}  // namespace qg
