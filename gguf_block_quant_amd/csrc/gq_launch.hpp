// gq_launch.hpp -- internal launchers called by the C ABI layer (gq_abi.cpp)
// after it has validated every argument. Each returns the hipGetLastError()
// status of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int64_t kMaxK = 32768;          // every compute entry point
constexpr int64_t kMaxRows = int64_t(1) << 30;

hipError_t launch_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* qs,
                       uint16_t* d, hipStream_t stream);

hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                hipStream_t stream);

hipError_t launch_qmv_f32(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                          const float* x, float* y, hipStream_t stream);

hipError_t launch_qmv_q8(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                         const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                         hipStream_t stream);

hipError_t launch_ffn_gate_up(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs,
                              const uint16_t* u_d, int64_t n_ff, int64_t k, const float* x,
                              float* h, hipStream_t stream);

hipError_t launch_tile_q4_0(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, int m,
                            const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                            hipStream_t stream);

}  // namespace gq
