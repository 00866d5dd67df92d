// gq_tile.hip -- small-M prefill tile: Q4_0 weights [n][k] against M = 8,
// 16 or 32 Q8_0 activation rows, on the int8 matrix cores.
//
// Prompt evaluation running tiles of up to 32 tokens through each projection
// is the Gem native architecture page's prefill tile ("Ownership
// boundaries", profiling bullet) and the raw-Metal port page's M = 8/16
// widenings ("Batched prefill"); here the tile is a real int8 contraction,
// so it goes to MFMA, while the M = 1 path stays a streaming matvec.
//
// One v_mfma_i32_16x16x32_i8 covers exactly one 32-element block (K = 32),
// so every MFMA result is a per-block integer dot S[n][m] -- exact, and
// separable from the per-block scales. The fp32 epilogue then adds
// dw[n][b] * dx[m][b] * S into the accumulators.
//
// Operand layout (gfx950 MFMA 16x16x32 int8; lane l, s = l / 16):
//   A (weights, 16 rows x 32 k): lane holds row l % 16, k = 8s .. 8s+7;
//   B (activations, 32 k x 16 cols): lane holds col l % 16, k = 8s .. 8s+7;
//   D (16 x 16 int32): lane holds rows 4s .. 4s+3 of col l % 16.
// Q4_0 byte j of a block holds elements j (low nibble) and j+16 (high), so
// k = 8s..8s+7 is bytes 8(s&1)..+7, low nibbles for s < 2, high for s >= 2.
//
// Work split: a wave owns 16 weight rows (one A tile) and 1/4 of the blocks
// of k; the four waves of a workgroup cover all of k for the same rows and
// add their fp32 partials through LDS in slice order (deterministic).
#include "gq_device.hpp"
#include "gq_launch.hpp"

namespace gq {

typedef int int32x4_t __attribute__((ext_vector_type(4)));

namespace {

// 8 unsigned nibbles (two dwords of bytes 0..15) -> 8 signed bytes (q - 8):
// (q + 120) ^ 0x80 per byte is q - 8 in two's complement; q + 120 <= 135
// never carries into the next byte.
__device__ __forceinline__ uint32_t nib_to_s8(uint32_t v) {
    return (v + 0x78787878u) ^ 0x80808080u;
}

template <int MT>   // number of 16-column activation tiles (M = 16 * MT, M = 8 uses MT = 1)
__global__ __launch_bounds__(kBlockThreads)
void tile_kernel(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int n, int nb,
                 int m, const int8_t* __restrict__ xq, const uint16_t* __restrict__ xd,
                 float* __restrict__ y, int32_t* __restrict__ blockdots) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int s = lane >> 4;                  // k group
    const int c = lane & 15;                  // A row / B col / D col within tile
    const int n0 = blockIdx.x * 16;
    const int64_t k = static_cast<int64_t>(nb) * 32;
    const int row_bytes = nb * 16;

    // this wave's slice of blocks
    const int b_begin = static_cast<int>((static_cast<int64_t>(nb) * wave) / kWavesPerBlock);
    const int b_end = static_cast<int>((static_cast<int64_t>(nb) * (wave + 1)) / kWavesPerBlock);

    const int arow = min(n0 + c, n - 1);                  // A operand row (clamped, masked later)
    const uint8_t* arow_ptr = qs + static_cast<int64_t>(arow) * row_bytes + 8 * (s & 1);
    const int ashift = (s >> 1) * 4;
    int drow[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) drow[v] = min(n0 + 4 * s + v, n - 1);

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = 0.f;

#pragma unroll 2
    for (int b = b_begin; b < b_end; ++b) {
        const uint2 wq = *reinterpret_cast<const uint2*>(arow_ptr + 16 * b);
        const uint32_t a0 = nib_to_s8((wq.x >> ashift) & 0x0F0F0F0Fu);
        const uint32_t a1 = nib_to_s8((wq.y >> ashift) & 0x0F0F0F0Fu);
        const long a = static_cast<long>((static_cast<uint64_t>(a1) << 32) | a0);
        float dw[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) dw[v] = half_bits_to_float(d[static_cast<int64_t>(drow[v]) * nb + b]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int mcol = 16 * t + c;
            long bop = 0;
            float dx = 0.f;
            if (mcol < m) {
                bop = *reinterpret_cast<const long*>(xq + static_cast<int64_t>(mcol) * k + 32 * b + 8 * s);
                dx = half_bits_to_float(xd[static_cast<int64_t>(mcol) * nb + b]);
            }
            const int32x4_t zero = {0, 0, 0, 0};
            const int32x4_t S = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bop, zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(dw[v] * dx, static_cast<float>(S[v]), acc[t][v]);
            if (blockdots != nullptr && mcol < m) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = n0 + 4 * s + v;
                    if (row < n)
                        blockdots[(static_cast<int64_t>(mcol) * n + row) * nb + b] = S[v];
                }
            }
        }
    }

    __shared__ float part[kWavesPerBlock][MT][4][kWave];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wave][t][v][lane] = acc[t][v];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int mcol = 16 * t + c;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float tot = part[0][t][v][lane];
#pragma unroll
                for (int w = 1; w < kWavesPerBlock; ++w) tot += part[w][t][v][lane];
                const int row = n0 + 4 * s + v;
                if (mcol < m && row < n) y[static_cast<int64_t>(mcol) * n + row] = tot;
            }
        }
    }
}

}  // namespace

hipError_t launch_tile_q4_0(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, int m,
                            const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                            hipStream_t stream) {
    const int grid = static_cast<int>((n + 15) / 16);
    const int nb = static_cast<int>(k / 32);
    if (m <= 16)
        return launch_kernel(tile_kernel<1>, dim3(grid), dim3(kBlockThreads), stream, qs, d,
                             static_cast<int>(n), nb, m, xq, xd, y, blockdots);
    return launch_kernel(tile_kernel<2>, dim3(grid), dim3(kBlockThreads), stream, qs, d,
                         static_cast<int>(n), nb, m, xq, xd, y, blockdots);
}

}  // namespace gq
