// gq_misc.hip -- load-time weight pack and the Q8_0 activation quantiser.
#include "gq_device.hpp"
#include "gq_launch.hpp"

namespace gq {

// ---------------------------------------------------------------------------
// Pack: GGUF blocks (34 B Q8_0 / 18 B Q4_0, any byte alignment) -> quants
// qs (16-B aligned rows) and scales d. One thread per block; byte loads
// because a block's start is only 2-byte aligned at best. Pure byte moves.
// The idea of a kernel-layout weight pack derived from the canonical file
// comes from the Gemma-4-E2B raw-Metal port page ("Architecture", pack
// bullet) and the Gem native architecture page ("M4 Max operating
// assumptions", packed sidecar).
// ---------------------------------------------------------------------------
template <int TYPE>
__global__ __launch_bounds__(kBlockThreads)
void pack_kernel(const uint8_t* __restrict__ blocks, int64_t nblocks, uint8_t* __restrict__ qs,
                 uint16_t* __restrict__ d) {
    constexpr int BB = (TYPE == kTypeQ8_0) ? 34 : 18;
    constexpr int QB = BB - 2;                       // quant bytes per block
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    const uint8_t* src = blocks + i * BB;
    d[i] = static_cast<uint16_t>(src[0] | (src[1] << 8));
    uint32_t w[QB / 4];
#pragma unroll
    for (int j = 0; j < QB / 4; ++j)
        w[j] = static_cast<uint32_t>(src[2 + 4 * j]) | (static_cast<uint32_t>(src[3 + 4 * j]) << 8) |
               (static_cast<uint32_t>(src[4 + 4 * j]) << 16) | (static_cast<uint32_t>(src[5 + 4 * j]) << 24);
    uint4* dst = reinterpret_cast<uint4*>(qs + i * QB);  // row bytes are multiples of 16
#pragma unroll
    for (int j = 0; j < QB / 16; ++j) dst[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
}

hipError_t launch_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* qs,
                       uint16_t* d, hipStream_t stream) {
    const int64_t nblocks = n * (k / 32);
    const int64_t grid = (nblocks + kBlockThreads - 1) / kBlockThreads;
    const dim3 g(static_cast<unsigned>(grid)), b(kBlockThreads);
    if (type == kTypeQ8_0) return launch_kernel(pack_kernel<kTypeQ8_0>, g, b, stream, blocks, nblocks, qs, d);
    return launch_kernel(pack_kernel<kTypeQ4_0>, g, b, stream, blocks, nblocks, qs, d);
}

// ---------------------------------------------------------------------------
// Q8_0 activation quantiser (quantize_q8_0_lane4 in gq_device.hpp holds the
// arithmetic). Eight lanes share a block, four elements each: one 16-byte
// load per lane, the block's amax by a max over the eight lanes with DPP
// (max is exact, so the order does not matter), four divides per lane, one
// 4-byte store per lane (a wave writes 256 contiguous code bytes) and the
// scale from the block's first lane. The blocks of all m rows are one flat
// sequence (x, xq and xd are contiguous row after row).
// ---------------------------------------------------------------------------
constexpr int kQuantLanesPerBlock = 8;

__global__ __launch_bounds__(kBlockThreads)
void quantize_q8_0_kernel(const float* __restrict__ x, int64_t nblocks, int8_t* __restrict__ xq,
                          uint16_t* __restrict__ xd) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t blk = t / kQuantLanesPerBlock;
    // the grid is whole waves and a block's eight lanes sit in one aligned
    // group of a wave, so a group is either entirely in range or entirely out
    if (blk >= nblocks) return;
    const float4 v = reinterpret_cast<const float4*>(x)[t];
    uint16_t hb;
    const uint32_t w = quantize_q8_0_lane4(v, hb);
    if ((t & (kQuantLanesPerBlock - 1)) == 0) xd[blk] = hb;
    reinterpret_cast<uint32_t*>(xq)[t] = w;
}

hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                hipStream_t stream) {
    const int64_t threads = m * (k / 32) * kQuantLanesPerBlock;
    const int64_t grid = (threads + kBlockThreads - 1) / kBlockThreads;
    return launch_kernel(quantize_q8_0_kernel, dim3(static_cast<unsigned>(grid)), dim3(kBlockThreads), stream,
                         x, m * (k / 32), xq, xd);
}

}  // namespace gq
