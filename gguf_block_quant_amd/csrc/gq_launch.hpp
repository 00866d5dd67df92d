// gq_launch.hpp -- internal launchers called by the C ABI layer (gq_abi.cpp)
// after it has validated every argument. Each returns the hipGetLastError()
// status of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace gq {

// Launch through hipLaunchKernel so the returned status belongs to this
// launch alone (a triple-chevron launch is only observable through
// hipGetLastError, which also reports errors left behind by other callers).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<std::decay_t<KArgs>...> vals(static_cast<std::decay_t<KArgs>>(args)...);
    void* ptrs[sizeof...(KArgs)];
    std::apply([&ptrs](auto&... v) {
        size_t i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

constexpr int64_t kMaxK = 32768;          // every compute entry point
constexpr int64_t kMaxRows = int64_t(1) << 30;

hipError_t launch_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* qs,
                       uint16_t* d, hipStream_t stream);

hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                hipStream_t stream);

constexpr size_t kArgmaxWorkspaceBytes = 16384;  // >= 8 bytes x the largest matvec grid

hipError_t launch_qmv_f32(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                          const float* x, const float* norm_w, float norm_eps, const float* residual,
                          float* y, hipStream_t stream);

hipError_t launch_qmv_argmax(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                             const float* x, const float* norm_w, float norm_eps, float softcap,
                             float* y, void* workspace, int32_t* index, float* value, hipStream_t stream);

// The same with the first stage's keys in a library-held device array
// (no workspace argument, nothing allocated).
hipError_t launch_qmv_argmax_noalloc(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                                     const float* x, const float* norm_w, float norm_eps, float softcap,
                                     float* y, int32_t* index, float* value, hipStream_t stream);

hipError_t launch_qmv_q8(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                         const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                         hipStream_t stream);

hipError_t launch_qmv_q8x(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                          int8_t* xq_out, uint16_t* xd_out, float* y, int32_t* blockdots, hipStream_t stream);

hipError_t launch_ffn_gate_up(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs,
                              const uint16_t* u_d, int64_t n_ff, int64_t k, const float* x,
                              const float* norm_w, float norm_eps, float* h, hipStream_t stream);

// K-quant super-blocks (Q4_K = 12, Q6_K = 14; 256 elements, k % 256 == 0)
size_t kq_layout(int type, int64_t n, int64_t k, size_t* offsets /* [4] or NULL */);
hipError_t launch_kq_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* packed,
                          hipStream_t stream);
hipError_t launch_qmv_kq(int type, const uint8_t* packed, int64_t n, int64_t k, const float* x, float* y,
                         hipStream_t stream);

hipError_t launch_tile_q4_0(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, int m,
                            const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                            hipStream_t stream);

}  // namespace gq
