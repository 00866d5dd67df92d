// read_stream.hip -- measurement helper for the benchmark, not part of
// libgq: the read-stream ceiling of the device, i.e. how fast plain 16-byte
// non-temporal loads can pull a buffer from HBM when nothing is done with
// the bytes but an XOR. The quantised matvecs are read streams with a
// little arithmetic on top, so their bandwidth is judged against this.
// Two access shapes, since which one is faster depends on the grid:
//  0: every lane strides over the buffer by the grid's thread count,
//     8 independent loads in flight per lane;
//  1: every wave reads 8 KiB contiguous chunks (8 loads of 1 KiB), the
//     chunks strided over the grid's waves.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kWave = 64;

__global__ __launch_bounds__(kThreads) void lane_stride_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               uint32_t* __restrict__ out) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    // full rounds: every index i + u * stride < n16
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kThreads) void wave_chunk_kernel(const u32x4* __restrict__ p, size_t n16,
                                                              uint32_t* __restrict__ out) {
    constexpr size_t kChunk = kUnroll * kWave;      // 16-byte pieces per chunk
    const int lane = threadIdx.x % kWave;
    const size_t waves = static_cast<size_t>(gridDim.x) * (kThreads / kWave);
    const size_t chunks = n16 / kChunk;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t c = static_cast<size_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave; c < chunks;
         c += waves) {
        const u32x4* q = p + c * kChunk + lane;
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(q + u * kWave);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    // the tail past the last whole chunk, one piece per thread of the grid
    for (size_t i = chunks * kChunk + static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * kThreads)
        acc ^= __builtin_nontemporal_load(p + i);
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// XOR-reduce `bytes` (a multiple of 16, p 16-byte aligned) with `grid`
// workgroups of 256 threads in access shape `pattern` (0 or 1); out
// receives grid * 256 uint32 words. Returns 0 on success, 1 on bad
// arguments, 2 on a failed launch.
int gqb_read_stream(const void* p, size_t bytes, uint32_t* out, int grid, int pattern, void* stream) {
    if (p == nullptr || out == nullptr || grid < 1 || bytes % 16 != 0 || (pattern != 0 && pattern != 1) ||
        (reinterpret_cast<uintptr_t>(p) & 15) != 0)
        return 1;
    const u32x4* q = static_cast<const u32x4*>(p);
    size_t n16 = bytes / 16;
    void* args[] = {&q, &n16, &out};
    const void* kernel = pattern == 0 ? reinterpret_cast<const void*>(lane_stride_kernel)
                                      : reinterpret_cast<const void*>(wave_chunk_kernel);
    return hipLaunchKernel(kernel, dim3(grid), dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? 0
               : 2;
}

}  // extern "C"
