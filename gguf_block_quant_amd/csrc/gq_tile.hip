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
// so every MFMA result is a per-block integer dot S[m][n] -- exact, and
// separable from the per-block scales. The fp32 epilogue then adds
// dx[m][b] * dw[n][b] * S into the accumulators.
//
// Operand layout (gfx950 MFMA 16x16x32 int8; lane l, s = l / 16, c = l % 16):
//   A (activations, 16 rows x 32 k): lane holds row c, k = 8s .. 8s+7;
//   B (weights, 32 k x 16 cols):     lane holds col c, k = 8s .. 8s+7;
//   D (16 x 16 int32):               lane holds rows 4s .. 4s+3 of col c.
// Q4_0 byte j of a block holds elements j (low nibble) and j+16 (high), so
// k = 8s..8s+7 is bytes 8(s&1)..+7, low nibbles for s < 2, high for s >= 2.
//
// Work split: a workgroup owns 16 weight rows and walks k in chunks of
// kChunk blocks (32 for one activation tile, 16 for two). Each chunk's
// weight rows, activation codes and both scale sets are staged in LDS with
// contiguous 16-byte global loads (the weight rows stream from HBM in
// 512- or 256-byte runs per row; the activations are
// shared by every workgroup and come from L2), while the registers already
// hold the next chunk's loads. The eight waves split the chunk's blocks;
// their fp32 partials meet in LDS and are added in wave order (deterministic).
// LDS rows are padded so the MFMA fragment reads are bank-conflict free.
#include "gq_device.hpp"
#include "gq_launch.hpp"

namespace gq {

typedef int int32x4_t __attribute__((ext_vector_type(4)));

namespace {

#ifndef GQ_TILE_CHUNK1
#define GQ_TILE_CHUNK1 32
#endif
#ifndef GQ_TILE_THREADS1
#define GQ_TILE_THREADS1 512     // workgroup size for one activation tile (8 waves, measured)
#endif
#ifndef GQ_TILE_THREADS2
#define GQ_TILE_THREADS2 512     // ... and for two (measured)
#endif
#ifndef GQ_TILE_CHUNK2
#define GQ_TILE_CHUNK2 16        // two row tiles: shorter chunks keep the LDS and registers in budget (measured)
#endif
#ifndef GQ_TILE_DEPTH1
#define GQ_TILE_DEPTH1 1         // chunks whose global loads are in flight at once (one activation tile; measured)
#endif
#ifndef GQ_TILE_DEPTH2
#define GQ_TILE_DEPTH2 1         // ... (two activation tiles; measured)
#endif
#ifndef GQ_TILE_WPAD1
#define GQ_TILE_WPAD1 16         // LDS row padding (bytes) of the staged weights, one activation tile
#endif
#ifndef GQ_TILE_XPAD1
#define GQ_TILE_XPAD1 32         // ... of the staged activation codes
#endif
#ifndef GQ_TILE_WPAD2
#define GQ_TILE_WPAD2 16         // ... weights, two activation tiles
#endif
#ifndef GQ_TILE_XPAD2
#define GQ_TILE_XPAD2 16         // ... activation codes, two activation tiles (32 measured 3 % slower)
#endif
constexpr int kRows = 16;                          // weight rows per workgroup
// Blocks per k chunk, and the LDS pitches that follow from it: a staged row
// is padded by an odd number of 16-byte units or by 32 bytes (an activation
// row CH * 32 + 32 for one tile, CH * 32 + 16 for two; a weight row
// CH * 16 + 16), so the fragment reads of the 16 rows spread over the banks
// (a pad of 64 bytes made the two-tile kernel 25 % slower).
template <int MT> struct Tiling {
    static constexpr int kChunk = MT == 1 ? GQ_TILE_CHUNK1 : GQ_TILE_CHUNK2;
    static constexpr int kThreads = MT == 1 ? GQ_TILE_THREADS1 : GQ_TILE_THREADS2;
    static constexpr int kWaves = kThreads / kWave;
    static constexpr int kWPitch = kChunk * 16 + (MT == 1 ? GQ_TILE_WPAD1 : GQ_TILE_WPAD2);
    static constexpr int kXPitch = kChunk * 32 + (MT == 1 ? GQ_TILE_XPAD1 : GQ_TILE_XPAD2);
    static constexpr int kWavePart = kChunk / kWaves;            // blocks per wave per chunk
    static constexpr int kDepth = MT == 1 ? GQ_TILE_DEPTH1 : GQ_TILE_DEPTH2;
};
#ifndef GQ_TILE_BATCH
#define GQ_TILE_BATCH 8
#endif
#ifndef GQ_TILE_BATCH2
#define GQ_TILE_BATCH2 4
#endif
#ifndef GQ_TILE_PAIR_BATCH
#define GQ_TILE_PAIR_BATCH 4     // block pairs whose MFMAs issue before their epilogues (M <= 8)
#endif
#ifndef GQ_TILE_EARLY_PAIR
#define GQ_TILE_EARLY_PAIR 1     // paired blocks: next chunk's loads before the barrier after the LDS store
#endif
#ifndef GQ_TILE_EARLY
#define GQ_TILE_EARLY 0          // ... the other tiles
#endif
#ifndef GQ_TILE_PAIRS
#define GQ_TILE_PAIRS 1          // M <= 8 takes the paired-block MFMA
#endif
#ifndef GQ_TILE_JB_UNROLL
#define GQ_TILE_JB_UNROLL 1
#endif
// blocks whose MFMAs issue before their epilogues (smaller for two row tiles,
// whose batches carry twice the scales and results)
template <int MT> struct Batch { static constexpr int value = MT == 1 ? GQ_TILE_BATCH : GQ_TILE_BATCH2; };
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// 8 unsigned nibbles (4 bytes) -> 8 signed bytes q - 8:
// (q + 120) ^ 0x80 per byte is q - 8 in two's complement; q + 120 <= 135
// never carries into the next byte.
__device__ __forceinline__ uint32_t nib_to_s8(uint32_t v) {
    return (v + 0x78787878u) ^ 0x80808080u;
}

template <int MR, int CH, int T>
struct Stage {                                      // one chunk's global loads, in registers
    // pieces of the chunk, and per thread (rounded up; threads past the
    // total skip the last round)
    static constexpr int kW = kRows * CH, kX = MR * CH * 2, kDX = MR * CH, kDW = kRows * CH;
    static constexpr int WV = (kW + T - 1) / T;     // 16-B weight pieces / thread
    static constexpr int XV = (kX + T - 1) / T;     // 16-B activation pieces / thread
    static constexpr int DXV = (kDX + T - 1) / T;   // activation scales / thread
    static constexpr int DWV = (kDW + T - 1) / T;   // weight scales / thread
    uint4 w[WV];
    uint4 x[XV];
    uint16_t dx[DXV];
    uint16_t dw[DWV];
};

// One chunk's global loads into registers (cn >= 1 blocks of it exist).
// Every thread issues every load of its pieces, straight-line: a piece that
// does not exist (past the end of k, past the m activation rows, past the
// piece count) reads a clamped, valid neighbour instead -- one that another
// lane reads anyway -- and is zeroed when it is written to LDS. Addresses are
// a workgroup-uniform base plus a 32-bit lane offset (one VGPR each).
template <int MR, int CH, int T>
__device__ __forceinline__ void stage_load(Stage<MR, CH, T>& st, int tid, int cb, int cn, int rmax, int nb, int m,
                                           int k, const uint8_t* wbase, const uint16_t* dbase, const int8_t* xq,
                                           const uint16_t* xd) {
    using S = Stage<MR, CH, T>;
    const int row_bytes = nb * 16;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < S::WV; ++i) {
        const int e = min(tid + i * T, S::kW - 1);
        const int row = min(e / CH, rmax), b = min(e % CH, cn - 1);    // a row's pieces are consecutive
        const uint32_t off = static_cast<uint32_t>(row * row_bytes + (cb + b) * 16);
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wbase + off));
        st.w[i] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int i = 0; i < S::XV; ++i) {
        const int e = min(tid + i * T, S::kX - 1);
        const int row = min(e / (2 * CH), m - 1), piece = min(e % (2 * CH), 2 * cn - 1);
        const uint32_t off = static_cast<uint32_t>(row * k + cb * 32 + piece * 16);
        st.x[i] = *reinterpret_cast<const uint4*>(xq + off);
    }
#pragma unroll
    for (int i = 0; i < S::DXV; ++i) {
        const int e = min(tid + i * T, S::kDX - 1);
        const int b = min(e / MR, cn - 1), row = min(e % MR, m - 1);
        st.dx[i] = xd[static_cast<uint32_t>(row * nb + cb + b)];
    }
#pragma unroll
    for (int i = 0; i < S::DWV; ++i) {
        const int e = min(tid + i * T, S::kDW - 1);
        const int b = min(e / kRows, cn - 1), row = min(e % kRows, rmax);
        st.dw[i] = dbase[static_cast<uint32_t>(row * nb + cb + b)];
    }
}

// Registers -> LDS for a chunk of cn blocks. Every loaded piece is written
// as it is (the clamped loads hold valid neighbours); then the scales of
// blocks past cn are overwritten with zeros, so those blocks add exactly 0.
// Pieces past the matrix rows or the m activation rows only produce results
// that are never stored, so they need no clearing. (A select between a
// loaded value and zero compiled to a branch that waited for that load
// inside it, one piece at a time.) Pieces past the count are not written.
template <int MR, int CH, int T>
__device__ __forceinline__ void stage_store(const Stage<MR, CH, T>& st, int tid, int cn, int m, uint8_t* ws,
                                            int wpitch, int8_t* xs, int xpitch, float* dxs, float* dws) {
    using S = Stage<MR, CH, T>;
    (void)m;
#pragma unroll
    for (int i = 0; i < S::WV; ++i) {
        const int e = tid + i * T;
        if (S::kW % T != 0 && e >= S::kW) break;
        *reinterpret_cast<uint4*>(&ws[(e / CH) * wpitch + (e % CH) * 16]) = st.w[i];
    }
#pragma unroll
    for (int i = 0; i < S::XV; ++i) {
        const int e = tid + i * T;
        if (S::kX % T != 0 && e >= S::kX) break;
        *reinterpret_cast<uint4*>(&xs[(e / (2 * CH)) * xpitch + (e % (2 * CH)) * 16]) = st.x[i];
    }
#pragma unroll
    for (int i = 0; i < S::DXV; ++i) {
        const int e = tid + i * T;
        if (S::kDX % T != 0 && e >= S::kDX) break;
        dxs[e] = half_bits_to_float(st.dx[i]);                     // [b][row], row-major
    }
#pragma unroll
    for (int i = 0; i < S::DWV; ++i) {
        const int e = tid + i * T;
        if (S::kDW % T != 0 && e >= S::kDW) break;
        dws[e] = half_bits_to_float(st.dw[i]);                     // [b][row], row-major
    }
    if (cn < CH) {                                                  // the last, ragged chunk only
#pragma unroll
        for (int i = 0; i < S::DXV; ++i) {
            const int e = tid + i * T;
            if (S::kDX % T != 0 && e >= S::kDX) break;
            if (e / MR >= cn) dxs[e] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < S::DWV; ++i) {
            const int e = tid + i * T;
            if (S::kDW % T != 0 && e >= S::kDW) break;
            if (e / kRows >= cn) dws[e] = 0.f;
        }
    }
}

// MT activation tiles of 16 rows (M <= 16 -> 1; M <= 32 -> 2). PAIR (M <= 8
// only, MT = 1): one v_mfma_i32_16x16x64_i8 covers two consecutive blocks --
// its 16 A rows are the <= 8 activation rows twice, the first copy holding
// block b in the k positions where B holds block b's weights and zeros where
// B holds block b+1's, the second copy the other way round -- so D rows 0..7
// are S for block b and rows 8..15 S for block b+1, and no MFMA row or
// epilogue lane is spent on padding.
template <int MT, bool PAIR>
__global__ __launch_bounds__(Tiling<MT>::kThreads)
void tile_kernel(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int n, int nb,
                 int m, const int8_t* __restrict__ xq, const uint16_t* __restrict__ xd,
                 float* __restrict__ y, int32_t* __restrict__ blockdots) {
    static_assert(!PAIR || MT == 1, "paired blocks are for M <= 8");
    constexpr int MR = PAIR ? 8 : 16 * MT;
    constexpr int kChunk = Tiling<MT>::kChunk;
    constexpr int kWPitch = Tiling<MT>::kWPitch;
    constexpr int kXPitch = Tiling<MT>::kXPitch;
    constexpr int kWavePart = Tiling<MT>::kWavePart;
    constexpr int kThreads = Tiling<MT>::kThreads;
    constexpr int kWaves = Tiling<MT>::kWaves;
    using St = Stage<MR, kChunk, kThreads>;
    __shared__ __align__(16) uint8_t ws[kRows][kWPitch];
    __shared__ __align__(16) int8_t xs[MR][kXPitch];
    __shared__ __align__(16) float dxs[kChunk][MR];
    __shared__ __align__(16) float dws[kChunk][kRows];
    __shared__ __align__(16) float part[kWaves][MT][4][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int s = lane >> 4;
    const int c = lane & 15;
    const int n0 = blockIdx.x * kRows;
    __builtin_assume(nb >= 1);                      // k >= 32: the chunk loop runs at least once
    const int64_t k = static_cast<int64_t>(nb) * 32;
    const int ashift = (s >> 1) * 4;

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = 0.f;

    // kDepth chunks' loads are in flight at once: chunk c's registers are
    // refilled with chunk c + kDepth as soon as they are in LDS
    constexpr int kDepth = Tiling<MT>::kDepth;
    St st[kDepth];
    // the workgroup's rows: base addresses, and the last row inside the matrix
    const uint8_t* wbase = qs + static_cast<int64_t>(n0) * (nb * 16);
    const uint16_t* dbase = d + static_cast<int64_t>(n0) * nb;
    const int rmax = n - 1 - n0;
#pragma unroll
    for (int dd = 0; dd < kDepth; ++dd) {
        if (dd == 0 || dd * kChunk < nb)
            stage_load<MR, kChunk, kThreads>(st[dd], tid, dd * kChunk, min(kChunk, nb - dd * kChunk), rmax, nb, m,
                                             static_cast<int>(k), wbase, dbase, xq, xd);
        // chunk by chunk, in the loop's order: the wait for chunk 0 must not
        // include chunk 1's loads on the way into the loop either
        __builtin_amdgcn_sched_barrier(0);
    }

    for (int cb0 = 0; cb0 < nb; cb0 += kDepth * kChunk) {
#pragma unroll
    for (int dd = 0; dd < kDepth; ++dd) {
        const int cb = cb0 + dd * kChunk;
        if (cb >= nb) break;
        const int cn = min(kChunk, nb - cb);
        stage_store<MR, kChunk, kThreads>(st[dd], tid, cn, m, &ws[0][0], kWPitch, &xs[0][0], kXPitch, &dxs[0][0],
                                          &dws[0][0]);
        // the next chunk's loads: for paired blocks they go out before the
        // barrier (they overlap the other waves' stores; M = 8: 4.98 -> 4.74
        // us), otherwise after it (measured faster there)
        constexpr bool kEarly = PAIR ? GQ_TILE_EARLY_PAIR : GQ_TILE_EARLY;
        if constexpr (!kEarly) __syncthreads();
        {
            const int nx = cb + kDepth * kChunk;
            if (nx < nb)
                stage_load<MR, kChunk, kThreads>(st[dd], tid, nx, min(kChunk, nb - nx), rmax, nb, m,
                                                 static_cast<int>(k), wbase, dbase, xq, xd);
        }
        if constexpr (kEarly) __syncthreads();

        // this wave's blocks of the chunk, kBatch at a time: the batch's
        // scales are read from LDS first, then its MFMAs are issued, then
        // their epilogues run (LDS and MFMA latency hide behind the batch).
        // Blocks past the end of k need no branch: both their staged scales
        // are zero, so they add exactly 0.
        const int b0 = wave * kWavePart;
        if constexpr (PAIR) {
            // lane (s, c): block bl + (s >> 1) of weight row c, nibble half s & 1
            // (elements 16 (s & 1) .. +15); activation row c & 7 of the same
            // block where the copy matches (c < 8 with s < 2, c >= 8 with s >= 2),
            // zeros elsewhere. D value v of lane (s, c): activation row
            // 4 (s & 1) + v, weight row c, block bl + (s >> 1).
            constexpr int kPairs = cmin(GQ_TILE_PAIR_BATCH, kWavePart / 2);
            static_assert(kWavePart % (2 * kPairs) == 0, "a wave's blocks of a chunk must be whole pair batches");
            const int half = s >> 1;
            const bool live = (c < 8) == (half == 0);
            const int nshift = (s & 1) * 4;
#pragma unroll GQ_TILE_JB_UNROLL
            for (int jb = 0; jb < kWavePart; jb += 2 * kPairs) {
                int32x4_t S[kPairs];
                float dwv[kPairs];
                float4 dxv[kPairs];
#pragma unroll
                for (int j = 0; j < kPairs; ++j) {
                    const int bl = b0 + jb + 2 * j + half;
                    dwv[j] = dws[bl][c];
                    dxv[j] = *reinterpret_cast<const float4*>(&dxs[bl][4 * (s & 1)]);
                }
#pragma unroll
                for (int j = 0; j < kPairs; ++j) {
                    const int bl = b0 + jb + 2 * j + half;
                    const uint4 wq = *reinterpret_cast<const uint4*>(&ws[c][bl * 16]);
                    typedef int int32x4v __attribute__((ext_vector_type(4)));
                    const int32x4v bop = {static_cast<int>(nib_to_s8((wq.x >> nshift) & 0x0F0F0F0Fu)),
                                          static_cast<int>(nib_to_s8((wq.y >> nshift) & 0x0F0F0F0Fu)),
                                          static_cast<int>(nib_to_s8((wq.z >> nshift) & 0x0F0F0F0Fu)),
                                          static_cast<int>(nib_to_s8((wq.w >> nshift) & 0x0F0F0F0Fu))};
                    const uint4 xa = *reinterpret_cast<const uint4*>(&xs[c & 7][bl * 32 + 16 * (s & 1)]);
                    const int32x4v aop = {live ? static_cast<int>(xa.x) : 0, live ? static_cast<int>(xa.y) : 0,
                                          live ? static_cast<int>(xa.z) : 0, live ? static_cast<int>(xa.w) : 0};
                    const int32x4_t zero = {0, 0, 0, 0};
                    S[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, zero, 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < kPairs; ++j) {
                    const float dx[4] = {dxv[j].x, dxv[j].y, dxv[j].z, dxv[j].w};
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[0][v] = fmaf(dwv[j] * dx[v], static_cast<float>(S[j][v]), acc[0][v]);
                }
                if (blockdots != nullptr) {
                    const int col = n0 + c;
#pragma unroll
                    for (int j = 0; j < kPairs; ++j) {
                        const int bl = b0 + jb + 2 * j + half;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int mrow = 4 * (s & 1) + v;
                            if (bl < cn && mrow < m && col < n)
                                blockdots[(static_cast<int64_t>(mrow) * n + col) * nb + cb + bl] = S[j][v];
                        }
                    }
                }
            }
        } else {
            constexpr int kBatch = cmin(Batch<MT>::value, kWavePart);
            static_assert(kWavePart % kBatch == 0, "a wave's blocks of a chunk must be whole batches");
#pragma unroll GQ_TILE_JB_UNROLL
            for (int jb = 0; jb < kWavePart; jb += kBatch) {
                int32x4_t S[kBatch][MT];
                float dwv[kBatch];
                float4 dxv[kBatch][MT];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int bl = b0 + jb + j;
                    dwv[j] = dws[bl][c];
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        dxv[j][t] = *reinterpret_cast<const float4*>(&dxs[bl][16 * t + 4 * s]);
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int bl = b0 + jb + j;
                    const uint2 wq = *reinterpret_cast<const uint2*>(&ws[c][bl * 16 + 8 * (s & 1)]);
                    const uint32_t lo = nib_to_s8((wq.x >> ashift) & 0x0F0F0F0Fu);
                    const uint32_t hi = nib_to_s8((wq.y >> ashift) & 0x0F0F0F0Fu);
                    const long bop = static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const long aop = *reinterpret_cast<const long*>(&xs[16 * t + c][bl * 32 + 8 * s]);
                        const int32x4_t zero = {0, 0, 0, 0};
                        S[j][t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, zero, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const float dx[4] = {dxv[j][t].x, dxv[j][t].y, dxv[j][t].z, dxv[j][t].w};
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[t][v] = fmaf(dwv[j] * dx[v], static_cast<float>(S[j][t][v]), acc[t][v]);
                    }
                }
                if (blockdots != nullptr) {
                    const int col = n0 + c;
#pragma unroll
                    for (int j = 0; j < kBatch; ++j) {
                        const int bl = b0 + jb + j;
#pragma unroll
                        for (int t = 0; t < MT; ++t)
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int mrow = 16 * t + 4 * s + v;
                                if (bl < cn && mrow < m && col < n)
                                    blockdots[(static_cast<int64_t>(mrow) * n + col) * nb + cb + bl] = S[j][t][v];
                            }
                    }
                }
            }
        }
        __syncthreads();   // LDS is rewritten by the next chunk
    }
    }

    // add the waves' partials in wave order (and, for paired blocks, the
    // two lane halves holding even and odd blocks) and store
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wave][t][v][lane] = acc[t][v];
    __syncthreads();
    if constexpr (PAIR) {
        if (tid < 2 * 4 * 16) {                      // 8 activation rows x 16 weight rows
            const int l = tid % 32;                  // lane of the even-block half: s = l / 16 in {0, 1}
            const int v = tid / 32;
            float tot = part[0][0][v][l] + part[0][0][v][l + 32];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) tot += part[w][0][v][l] + part[w][0][v][l + 32];
            const int mrow = 4 * (l >> 4) + v;
            const int col = n0 + (l & 15);
            if (mrow < m && col < n) y[static_cast<int64_t>(mrow) * n + col] = tot;
        }
    } else {
        for (int e = tid; e < MT * 4 * kWave; e += kThreads) {
            const int l = e % kWave;
            const int v = (e / kWave) % 4;
            const int t = e / (kWave * 4);
            float tot = part[0][t][v][l];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) tot += part[w][t][v][l];
            const int mrow = 16 * t + 4 * (l >> 4) + v;
            const int col = n0 + (l & 15);
            if (mrow < m && col < n) y[static_cast<int64_t>(mrow) * n + col] = tot;
        }
    }
}

}  // namespace

hipError_t launch_tile_q4_0(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, int m,
                            const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                            hipStream_t stream) {
    const int grid = static_cast<int>((n + kRows - 1) / kRows);
    const int nb = static_cast<int>(k / 32);
    if (GQ_TILE_PAIRS && m <= 8)
        return launch_kernel(tile_kernel<1, true>, dim3(grid), dim3(Tiling<1>::kThreads), stream, qs, d,
                             static_cast<int>(n), nb, m, xq, xd, y, blockdots);
    if (m <= 16)
        return launch_kernel(tile_kernel<1, false>, dim3(grid), dim3(Tiling<1>::kThreads), stream, qs, d,
                             static_cast<int>(n), nb, m, xq, xd, y, blockdots);
    return launch_kernel(tile_kernel<2, false>, dim3(grid), dim3(Tiling<2>::kThreads), stream, qs, d,
                         static_cast<int>(n), nb, m, xq, xd, y, blockdots);
}

}  // namespace gq
