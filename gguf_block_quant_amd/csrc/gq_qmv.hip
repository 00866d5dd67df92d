// gq_qmv.hip -- M = 1 decode kernels: Q8_0 / Q4_0 matvec with fp32 or
// Q8_0-quantised activations, and the fused gate+up GELU FFN pass.
//
// Decomposition (gfx950, wave64):
//  * A "unit" is 16 bytes of packed quants: one global_load_dwordx4 per lane.
//    For Q8_0 that is half a block (16 elements), for Q4_0 one whole block
//    (32 elements). Lane l of a wave owns units l, l+64, ... of its K-slice,
//    so each load instruction reads 1 KiB of one row contiguously.
//  * The activation values a lane needs for its units are loaded once into
//    VGPRs and reused for every row the wave streams; for k <= 8192 the
//    workgroup first stages all of x in LDS (one read of x per workgroup).
//  * A wave streams R rows per step (R x NI independent 16-byte loads in
//    flight per lane), dequantises and dot-reduces in registers, and sums
//    the lanes of all the group's rows at once with lane-half and row swaps
//    and DPP (wave_sum4_rows), fixed order, no atomics. The next row
//    group's loads go out after the current group's dot, into the same
//    registers.
//  * Long rows (large k) are split over WS waves of the workgroup; their
//    partial sums meet in LDS and are added in slice order.
//  * The grid is persistent: at most the resident workgroups, striding over
//    the row groups, so each wave amortises its activation load over many
//    rows.
// The decode projection being a weight-streaming matvec, and the lesson that
// an M == 1 product wants its own kernel rather than a tiled GEMM, follow the
// SafeC Gemma 4 DESIGN_NOTES page ("A dedicated GEMV kernel for the M==1
// decode step") and the Gemma-4-E2B raw-Metal port page ("Why this exists").
#include <atomic>
#include <mutex>
#include <type_traits>

#include "gq_device.hpp"
#include "gq_launch.hpp"

#ifndef GQ_QMV_MAX_GRID
#define GQ_QMV_MAX_GRID 1280   // workgroups of 4 waves (5 per CU on 256 CUs; the vocabulary head, measured)
#endif
#ifndef GQ_QMV_R_SHORT
#define GQ_QMV_R_SHORT 1         // rows per wave step for shorter un-split matrices
#endif
#ifndef GQ_QMV_R_FFN
#define GQ_QMV_R_FFN 2           // rows per wave step of the gate+up pass (each a gate and an up row)
#endif
#ifndef GQ_QMV_SPLIT_SUBS
#define GQ_QMV_SPLIT_SUBS 1      // row groups per workgroup when rows are split over 4 waves (at most 16 waves)
#endif
#ifndef GQ_QMV_STAGE_WS
#define GQ_QMV_STAGE_WS 4        // largest K split whose workgroups stage x in LDS (all of x: k <= 8192)
#endif
#ifndef GQ_QMV_WAVES1
#define GQ_QMV_WAVES1 4        // waves per workgroup for un-split rows (they share one LDS copy of x)
#endif
#ifndef GQ_QMV_WAVES1_TALL
#define GQ_QMV_WAVES1_TALL 4   // ... for tall matrices at R_TALL rows per step (2 and 8 measured slower)
#endif
#ifndef GQ_QMV_WAVES1_SHORT
#define GQ_QMV_WAVES1_SHORT 8  // ... for shorter matvecs at R_SHORT rows per step (measured)
#endif
#ifndef GQ_QMV_WAVES1_Q8X
#define GQ_QMV_WAVES1_Q8X 8    // ... for the integer path quantising x in its prologue (measured)
#endif
#ifndef GQ_QMV_R_Q8X
#define GQ_QMV_R_Q8X 1         // rows per wave step of the integer path quantising x in its prologue (measured)
#endif
#ifndef GQ_QMV_R_TALL
#define GQ_QMV_R_TALL 4        // rows per wave step for tall un-split matrices
#endif
#ifndef GQ_QMV_TALL_MIN_BYTES
#define GQ_QMV_TALL_MIN_BYTES (16 << 20)   // fp32-x matvecs with at least this many quant bytes take R_TALL rows
#endif                                      // per step (measured: Q8_0 from 8192 x 2048, Q4_0 from 16384 x 2048)
#ifndef GQ_QMV_TALL_MIN_BYTES_Q8
#define GQ_QMV_TALL_MIN_BYTES_Q8 (32 << 20)  // ... pre-quantised x from this many (measured: Q8_0 16384 x 2048
#endif                                        // 8.23 -> 7.74 us, 8192 x 2048 slower)
#ifndef GQ_QMV_TALL_MIN_N
#define GQ_QMV_TALL_MIN_N 65536  // ... the other un-split paths (gate+up, x quantised in the kernel) from this many rows
#endif
#ifndef GQ_QMV_R_SPLIT
#define GQ_QMV_R_SPLIT 4         // rows per wave step when a row is split over 4 or 8 waves
#endif
#ifndef GQ_QMV_NT
#define GQ_QMV_NT 1            // non-temporal loads for the quant stream (read once)
#endif

namespace gq {

enum Mode { kF32 = 0, kQ8X = 1, kFFN = 2 };

template <int TYPE> struct Fmt;
template <> struct Fmt<kTypeQ8_0> {
    static constexpr int kElemsPerUnit = 16;
    static constexpr int kUnitToBlockShift = 1;
};
template <> struct Fmt<kTypeQ4_0> {
    static constexpr int kElemsPerUnit = 32;
    static constexpr int kUnitToBlockShift = 0;
};

struct QmvParams {
    const uint8_t* qs;      // packed quants [n][row_bytes]
    const uint16_t* d;      // scales [n][nb]
    const uint8_t* qs2;     // FFN: up-matrix quants
    const uint16_t* d2;     // FFN: up-matrix scales
    const float* x;         // fp32 activations [k]
    const int8_t* xq;       // Q8_0 activation codes [k]
    const uint16_t* xd;     // Q8_0 activation scales [k/32]
    float* y;               // output [n]
    int32_t* blockdots;     // optional S [n][nb]
    const float* norm_w;    // optional RMSNorm weight [k] (prologue on x)
    const float* residual;  // optional residual [n] added to the output
    unsigned long long* part;  // optional argmax partials [gridDim.x]
    int8_t* xq_out;         // integer path quantising x itself: optional codes out [k]
    uint16_t* xd_out;       // ... and scales out [k/32] (written by workgroup 0)
    float norm_eps;
    double inv_k;           // 1 / k (the RMSNorm mean's divisor)
    float softcap;          // > 0: output = softcap * tanh(output / softcap)
    int n;
    int k;
    int units;              // 16-byte units per row
    int nb;                 // blocks per row
    int row_groups;         // ceil(n / R)
};

// Order-preserving 64-bit key of (value, row) for a greedy argmax: a larger
// value gives a larger key, and for equal values the lower row does; -0 is
// folded into +0 and NaN ranks below every number. 0 means "no row".
__device__ __forceinline__ unsigned long long argmax_key(float v, int row) {
    uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    if (v != v) u = 0u;
    return (static_cast<unsigned long long>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(row));
}

// fp32-activation dot of one unit against the lane's activation registers.
template <int TYPE>
__device__ __forceinline__ float unit_dot_f32(const uint4 q, const float* xr) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float p = 0.0f;
    if constexpr (TYPE == kTypeQ8_0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                p = fmaf(static_cast<float>(static_cast<int8_t>(w[j] >> (8 * b))), xr[4 * j + b], p);
    } else {
        // Two nibbles at bits 0..3 and 16..19, OR-ed under the binary16
        // exponent of 1024 (0x6400), are the half2 (1024 + q_a, 1024 + q_b);
        // one packed fp16 add of -1032 leaves q - 8 exactly, and
        // v_fma_mix_f32 multiplies that half by the fp32 activation with a
        // single rounding -- the same value as an fp32 FMA on (float)(q - 8).
        // The high nibbles are taken in place (bits 4..7 and 20..23), which
        // gives 1024 + 16 q; adding -1152 leaves 16 (q - 8), still exact in
        // binary16, accumulated separately and scaled by 1/16 (exact) at the
        // end. Two masks share one shift per word instead of three shifts.
        typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
        const half2_t off_lo = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
        const half2_t off_hi = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
        // keep the exponent pattern in a VGPR: gfx9 VOP3 takes no literal, and
        // with one register operand the mask-and-or is a single v_and_or_b32
        uint32_t magic = 0x64006400u;
        asm volatile("" : "+v"(magic));
        float ph = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t v = w[j];
            const uint32_t v8 = v >> 8;
            const half2_t lo02 = __builtin_bit_cast(half2_t, (v & 0x000F000Fu) | magic) + off_lo;
            const half2_t lo13 = __builtin_bit_cast(half2_t, (v8 & 0x000F000Fu) | magic) + off_lo;
            const half2_t hi02 = __builtin_bit_cast(half2_t, (v & 0x00F000F0u) | magic) + off_hi;
            const half2_t hi13 = __builtin_bit_cast(half2_t, (v8 & 0x00F000F0u) | magic) + off_hi;
            // element order: 4j+b (low nibble of byte b), then 16+4j+b (its high nibble)
            p = fmaf(static_cast<float>(lo02.x), xr[4 * j + 0], p);
            ph = fmaf(static_cast<float>(hi02.x), xr[16 + 4 * j + 0], ph);
            p = fmaf(static_cast<float>(lo13.x), xr[4 * j + 1], p);
            ph = fmaf(static_cast<float>(hi13.x), xr[16 + 4 * j + 1], ph);
            p = fmaf(static_cast<float>(lo02.y), xr[4 * j + 2], p);
            ph = fmaf(static_cast<float>(hi02.y), xr[16 + 4 * j + 2], ph);
            p = fmaf(static_cast<float>(lo13.y), xr[4 * j + 3], p);
            ph = fmaf(static_cast<float>(hi13.y), xr[16 + 4 * j + 3], ph);
        }
        p = fmaf(ph, 0.0625f, p);
    }
    return p;
}

// Exact int32 dot of one unit against the lane's Q8_0 activation codes.
// Q4_0: the unsigned nibbles (0..15, valid positive int8) are dotted and the
// -8 offset is taken out with the exact integer sum of the codes, sx.
template <int TYPE>
__device__ __forceinline__ int unit_dot_q8(const uint4 q, const uint32_t* xr, int sx) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    int s = 0;
    if constexpr (TYPE == kTypeQ8_0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s = dot4(w[j], xr[j], s);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s = dot4(w[j] & 0x0F0F0F0Fu, xr[j], s);               // elements 4j..4j+3
            s = dot4((w[j] >> 4) & 0x0F0F0F0Fu, xr[4 + j], s);    // elements 16+4j..
        }
        s -= 8 * sx;
    }
    return s;
}

// Waves per workgroup for a K split over WS waves: at least 4; split rows
// put GQ_QMV_SPLIT_SUBS row groups in one workgroup while that stays within
// 16 waves (measured: with x staged in LDS, one 4-row group per 4-wave
// workgroup is the fastest for the 2048 x 8192 down projection).
// Un-split rows take GQ_QMV_WAVES1 waves (the vocabulary head, the gate+up
// pass), except shorter matvecs at R_SHORT rows per step and the integer
// path with the quantiser folded in, whose workgroups each quantise all of x
// first: there more waves share the staging or quantiser prologue
// (GQ_QMV_WAVES1_SHORT, GQ_QMV_WAVES1_Q8X; measured).
template <int WS, int MODE, bool FOLD, int R> struct Waves {
    static constexpr int value =
        WS == 1 ? ((MODE == kQ8X && FOLD)                    ? GQ_QMV_WAVES1_Q8X
                   : (MODE != kFFN && R == GQ_QMV_R_SHORT) ? GQ_QMV_WAVES1_SHORT
                   : (R == GQ_QMV_R_TALL)                  ? GQ_QMV_WAVES1_TALL
                                                           : GQ_QMV_WAVES1)
                : (WS < 4 ? 4 : (WS * GQ_QMV_SPLIT_SUBS > 16 ? WS : WS * GQ_QMV_SPLIT_SUBS));
};

// FOLD selects the variant with the optional RMSNorm prologue and the
// residual / soft-cap / argmax epilogue (runtime flags in QmvParams); the
// plain variant carries none of that code, so its register budget is
// untouched.
template <int TYPE, int MODE, int NI, int WS, int R, bool FOLD>
__global__ __launch_bounds__((Waves<WS, MODE, FOLD, R>::value * kWave))
void qmv_kernel(const QmvParams p) {
    constexpr int EPU = Fmt<TYPE>::kElemsPerUnit;
    constexpr int SH = Fmt<TYPE>::kUnitToBlockShift;
    constexpr int WAVES = Waves<WS, MODE, FOLD, R>::value;
    constexpr int SUBS = WAVES / WS;                // independent row groups per workgroup
    constexpr int NMAT = (MODE == kFFN) ? 2 : 1;
    const int lane = threadIdx.x & (kWave - 1);
    // Instantiations for tall matrices (R_TALL rows per step at WS = 1: fp32
    // x from 16 MiB of quants, pre-quantised x from 32 MiB, the other paths
    // from 65536 rows): each wave walks many row groups. These keep the wave
    // index in a scalar register (the row arithmetic and each row's base
    // address are then scalar), one scale per 32-bit register, and the
    // pinned loop below; so do the gate+up pass and split rows. Measured on
    // MI355X: the vocabulary head, the FFN and the down projection gain from
    // the pinned loop, the un-split one-group matvecs (2048 x 2048) do not.
    constexpr bool kManyGroups = (WS == 1 && R == GQ_QMV_R_TALL);
    constexpr bool kPinned = kManyGroups || MODE == kFFN || WS > 1;
    // The plain split-row kernels (2 to 8 waves per row) take the scalar wave
    // index too (measured: down projection 2048 x 8192 4.25 -> 4.07 us,
    // 2048 x 16384 7.77 -> 7.64 us); the 16-wave split, the folded variants
    // and the un-split gate+up pass measured slower with it (11.6 -> 11.75,
    // 2048 x 2048 RMSNorm 3.18 -> 3.36, gate+up 5.3 -> 5.5 us).
    constexpr bool kScalarWave = kManyGroups || (WS > 1 && WS < 16 && !FOLD);
    const int wave = kScalarWave ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave)
                                 : static_cast<int>(threadIdx.x) / kWave;
    const int slice = wave % WS;
    const int sub = wave / WS;
    const int row_bytes = p.units * 16;
    // fp32 activations are staged through LDS (below) for un-split rows and
    // for rows split over up to GQ_QMV_STAGE_WS waves (all of x, which the
    // workgroup's row groups share)
    constexpr bool kStage = (MODE != kQ8X) && (WS <= GQ_QMV_STAGE_WS);
    constexpr int kPitch = EPU + 4;
    constexpr int kThreads = WAVES * kWave;
    // float4s of x per thread when staging; the LDS copy is padded to whole
    // rounds of the workgroup so every thread writes its slots unconditionally
    constexpr int kStageF4 = kStage ? (WS * NI * kWave * EPU / 4 + kThreads - 1) / kThreads : 0;
    constexpr int kStageUnits = kStage ? (kStageF4 * kThreads * 4 + EPU - 1) / EPU : 1;
    static_assert(!kStage || kStageUnits >= WS * NI * kWave, "every lane's unit has a staged slot");
    __shared__ float xstage[kStage ? kStageUnits * kPitch : 1];
    // integer path with the quantiser folded in: the workgroup's Q8_0 codes
    // (4 per word) and binary16 scales of all of x
    constexpr bool kQuantX = (MODE == kQ8X) && FOLD;
    constexpr int kQuantF4 = kQuantX ? (WS * NI * kWave * EPU / 4 + kThreads - 1) / kThreads : 0;
    constexpr int kQxWords = kQuantX ? kQuantF4 * kThreads : 1;       // whole rounds, as above
    __shared__ uint32_t qx_s[kQxWords];
    __shared__ uint16_t qd_s[kQuantX ? kQxWords / 8 : 1];
    __shared__ double nss[WAVES];
    __shared__ int nfl[WAVES];      // per wave: 1 = some |x w| above 2^40, 2 = some at or above 2^-40

    // ---- this lane's units ------------------------------------------------
    int unit[NI];
    bool uvalid[NI];
    uint32_t uload[NI];     // clamped unit index (lanes past a short row)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        unit[i] = (slice * NI + i) * kWave + lane;
        uvalid[i] = unit[i] < p.units;
        uload[i] = static_cast<uint32_t>(min(unit[i], p.units - 1));
    }

    // Quant chunks and scales of one row group, for every unit of the lane.
    // Lanes past the end of a short row load a clamped (valid) unit and
    // contribute nothing: their activations are zero and their scale is
    // masked to zero below, so no load sits behind a divergent branch.
    uint4 q[NI][NMAT][R];
    // (two 16-bit scales packed into one register would make the compiler
    // wait for their loads right where the next group's are issued; the
    // other instantiations keep 16-bit scales, measured faster for them)
    using ScaleT = std::conditional_t<kManyGroups, uint32_t, uint16_t>;
    ScaleT db[NI][NMAT][R];
    // The gate+up pass and split rows read their scales with non-temporal
    // loads, like the quants (measured: gate+up 5.59 -> 5.37 us, down 4.41
    // -> 4.29 us); the other paths keep cached scale loads (for the vocab
    // head non-temporal ones re-fetched 0.5 % of its bytes from HBM and
    // gained nothing in the step; the 2048 x 2048 matvecs did not change).
    auto load_scale = [](const uint16_t* a) -> uint16_t {
        if constexpr (MODE == kFFN || WS > 1) return __builtin_nontemporal_load(a);
        else return *a;
    };
    // split rows issue a group's scales before its quants (measured: the
    // down projection 4.53 -> 4.41 us with the staging below; the compiler
    // waits for the scales early, and then that wait covers no quant load)
    constexpr bool kScalesFirst = WS > 1;
    auto load_group = [&](uint4 (&qd)[NI][NMAT][R], ScaleT (&dd)[NI][NMAT][R], int r0) {
        if constexpr (kScalesFirst) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const uint16_t* dm = (m == 0) ? p.d : p.d2;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
                        dd[i][m][r] = load_scale(dm + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.nb) +
                                                 (uload[i] >> SH));
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint8_t* qsm = (m == 0) ? p.qs : p.qs2;
                const uint16_t* dm = (m == 0) ? p.d : p.d2;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    // rows past n re-read row n-1 (in bounds); their results are discarded
                    const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
                    const uint8_t* src = qsm + static_cast<uint64_t>(row) * static_cast<uint32_t>(row_bytes) +
                                         uload[i] * 16u;
#if GQ_QMV_NT
                    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
                    qd[i][m][r] = make_uint4(t.x, t.y, t.z, t.w);
#else
                    qd[i][m][r] = *reinterpret_cast<const uint4*>(src);
#endif
                    if constexpr (!kScalesFirst)
                        dd[i][m][r] = load_scale(dm + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.nb) +
                                                 (uload[i] >> SH));
                }
            }
    };

    // Loads of the activations that the workgroup stages (fp32 x, and the
    // RMSNorm weight; or x for the folded quantiser) go out first, then the
    // first row group's weights: loads complete in issue order, so waiting
    // for the activations (an L2 hit) does not wait for the weights (HBM),
    // and the staging overlaps the weights' flight.
    bool norm = false;
    if constexpr (MODE != kQ8X && FOLD) norm = p.norm_w != nullptr;
    const int nf4 = p.k >> 2;
    constexpr int kPreF4 = kStageF4 > kQuantF4 ? kStageF4 : kQuantF4;    // at most one is nonzero
    float4 xpre[kPreF4 > 0 ? kPreF4 : 1];
    float4 gpre[(kStage && FOLD) ? kStageF4 : 1];
    if constexpr (kPreF4 > 0) {
        // unconditional (clamped) loads: straight-line code lets the wait
        // before the LDS writes count only these loads
#pragma unroll
        for (int u = 0; u < kPreF4; ++u) {
            const int j = min(static_cast<int>(threadIdx.x) + u * kThreads, nf4 - 1);
            xpre[u] = reinterpret_cast<const float4*>(p.x)[j];
        }
        if constexpr (kStage && FOLD) {
            const float4* g4 = reinterpret_cast<const float4*>(norm ? p.norm_w : p.x);
#pragma unroll
            for (int u = 0; u < kStageF4; ++u) {
                const int j = min(static_cast<int>(threadIdx.x) + u * kThreads, nf4 - 1);
                gpre[u] = g4[j];
            }
        }
    }

    // The other paths read their lane's activation slice straight into
    // registers; those loads go out before the weights as well (clamped
    // units, masked below), so the first row's dot waits for its own loads
    // rather than for the whole group.
    constexpr bool kDirect = !kStage && !kQuantX;
    constexpr bool kDirectF = kDirect && MODE != kQ8X;
    constexpr bool kDirectQ = kDirect && MODE == kQ8X;
    float4 xd4[kDirectF ? NI : 1][kDirectF ? EPU / 4 : 1];
    float4 gd4[(kDirectF && FOLD) ? NI : 1][(kDirectF && FOLD) ? EPU / 4 : 1];
    uint4 xq4[kDirectQ ? NI : 1][kDirectQ ? EPU / 16 : 1];
    uint16_t xdb[NI];
    if constexpr (kDirectF) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int v = 0; v < EPU / 4; ++v) xd4[i][v] = reinterpret_cast<const float4*>(p.x + uload[i] * EPU)[v];
        if constexpr (FOLD) {
            const float* gsrc = norm ? p.norm_w : p.x;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int v = 0; v < EPU / 4; ++v)
                    gd4[i][v] = reinterpret_cast<const float4*>(gsrc + uload[i] * EPU)[v];
        }
    }
    if constexpr (kDirectQ) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int v = 0; v < EPU / 16; ++v) xq4[i][v] = reinterpret_cast<const uint4*>(p.xq + uload[i] * EPU)[v];
            xdb[i] = p.xd[uload[i] >> SH];
        }
    }

    // (the grid never exceeds the row-group iterations, so every workgroup's
    // first group exists; the load is unconditional, which also keeps the
    // activation waits above exact)
    // keep the scheduler from hoisting the weight loads above the activation
    // loads (the point of the order above)
    // The row group's NMAT * R sums are reduced over the wave together
    // (wave_sum4_rows): four of them leave 16-lane row q holding value
    // ((q & 1) << 1) | (q >> 1), value v being acc[v / R][v % R]. So the
    // lane that finishes a row is lane 16 q for four rows (and for the
    // gate+up pass at 4 row pairs, which reduces gates and ups separately);
    // lane 32 r for the gate+up pass at 2 row pairs (a row swap pairs each
    // gate with its up); lane 0 for one row; and lane r of slice 0 for split
    // rows, which add the slices' sums in LDS.
    constexpr int kV = NMAT * R;
    static_assert(kV == 1 || kV == 4 || (kV == 8 && NMAT == 2), "1, 4 or 2 x 4 sums per row group");
    auto lane_row = [&](int l) -> int {
        if constexpr (WS > 1) return l % R;
        else if constexpr (kV == 1) return 0;
        else if constexpr (kV == 4 && NMAT == 2) return l >> 5;
        else return (((l >> 4) & 1) << 1) | (l >> 5);
    };
    // The residual of the row this lane finishes goes out just before its
    // row group's weights: loads complete in issue order, so the wait for
    // the weights covers it (issued after them, it had held up every dot).
    // The load is unconditional -- without a residual it reads (and ignores)
    // x[0], which every workgroup reads anyway (y[0] if there were no x): a
    // load on one path only makes the compiler count the loads before it for
    // the shorter path, so the prologue's wait for x would also have waited
    // for the residual (2048 x 2048 RMSNorm + residual 3.12 -> 2.6 us).
    // (A dummy read of y's own rows measured 0.25 us slower.)
    float resv = 0.f, resv_next = 0.f;
    auto load_res = [&](float& dst, int r0) {
        if constexpr (FOLD) {
            const float* src = p.residual != nullptr ? p.residual + min(r0 + lane_row(lane), p.n - 1)
                                                     : (p.x != nullptr ? p.x : p.y);
            dst = *src;
        }
    };

    __builtin_amdgcn_sched_barrier(0);
    int it = blockIdx.x;
    load_res(resv, (it * SUBS + sub) * R);
    load_group(q, db, (it * SUBS + sub) * R);

    // ---- activation registers for this lane's units ----------------------
    // Optional RMSNorm prologue (SafeC Gemma 4 DESIGN_NOTES page, "RMSNorm"):
    // x <- x * (mean(x^2) + eps)^-1/2 * w, the weight multiplying directly.
    // The sum of squares of the raw x is taken in fp64 (x^2 of any finite
    // fp32 value is exact there, and k <= 32768 such terms can neither
    // overflow nor underflow to zero unless x is zero), and the scale
    // inv = (sum / k + eps)^-1/2 stays in fp64; w is folded into the staged
    // activations and inv into each lane's activation registers (an fp64
    // product rounded once to fp32) before any dot, so the dot products run
    // on the normalised activations, |x_i * inv| <= sqrt(k), for any finite
    // x -- no fp32 overflow of the sum or of the scale.
    float xr[(MODE == kQ8X) ? 1 : NI][(MODE == kQ8X) ? 1 : EPU];
    uint32_t xqr[(MODE == kQ8X) ? NI : 1][(MODE == kQ8X) ? EPU / 4 : 1];
    float dxr[NI];
    int sxr[NI];
    double ss = 0.0;
    // inv = (sum / k + eps)^(-1/2): the hardware reciprocal square root (good
    // to about 2^-24) and one Newton step in fp64 (to about 2^-47; the
    // callers round to fp32). The divide and correctly rounded square root
    // of 1/sqrt(sum/k + eps) cost every wave a long fp64 sequence, about a
    // microsecond for the 2 x 8192 x 2048 FFN's 16 waves per CU. The mean is
    // 0 (x all zero with eps 0: inv = +Inf, as 1/sqrt(0)) or at least 2^-313
    // (the square of the smallest fp32 subnormal over k <= 32768), far from
    // the fp64 subnormals where the approximation weakens.
    auto norm_scale = [&](double sum) {
        const double a = fma(sum, p.inv_k, static_cast<double>(p.norm_eps));
        const double y0 = __builtin_amdgcn_rsq(a);
        const double h = a * y0;
        const double y1 = fma(0.5 * y0, fma(-h, y0, 1.0), y0);
        return (a > 0.0 && a < __builtin_inf()) ? y1 : y0;
    };
    auto scaled = [](float v, double s) { return static_cast<float>(static_cast<double>(v) * s); };
    // RMSNorm: when the largest |x_i w_i| lies in [2^-40, 2^40] (the usual
    // case; uniform over the launch, decided from two wave ballots), the dots
    // run on x w as staged and each finished row is multiplied by inv in fp64
    // (rounded once) -- no dot can overflow there (|y| <= k 65504 127 2^40)
    // and the largest products stay far above fp32's underflow. Outside that
    // range the activations are scaled by inv before the dots, as an fp64
    // product rounded once, which keeps every dot in range for any finite x.
    float mxl = 0.f;                 // this thread's max |x w|
    bool post = false;               // scale the finished rows by post_inv
    double post_inv = 1.0;
    constexpr float kPostLo = 0x1p-40f, kPostHi = 0x1p40f;
    if constexpr (kStage) {
        // Un-split rows: every wave of the workgroup needs all of x, so the
        // workgroup reads it (and w) from memory once into LDS, padded to a
        // pitch of EPU + 4 floats per unit so the lanes' 16-byte reads of
        // consecutive units do not collide in a bank, and the waves copy
        // their slices from there. Without this each wave re-reads the same
        // few KiB, which for short matrices is more traffic than the weights.
        // Slots past k get zeros (lanes past a short row read them). The
        // loaded values are written unconditionally (the clamped loads are
        // valid memory) and the padding slots overwritten with zeros after:
        // a select on a loaded value turns into a branch that waits for the
        // load inside it, one float4 at a time.
        // (measured: the split-row kernels, with several float4s per thread,
        // gain from this; the un-split ones keep the select)
        constexpr bool kZeroPass = WS > 1;
#pragma unroll
        for (int u = 0; u < kStageF4; ++u) {
            const int j = threadIdx.x + u * kThreads;
            float4 t = kZeroPass ? xpre[u] : (j < nf4 ? xpre[u] : make_float4(0.f, 0.f, 0.f, 0.f));
            if constexpr (FOLD) {
                if (norm) {
                    const float4 g = gpre[u];
                    double q = static_cast<double>(t.x) * static_cast<double>(t.x);
                    q = fma(static_cast<double>(t.y), static_cast<double>(t.y), q);
                    q = fma(static_cast<double>(t.z), static_cast<double>(t.z), q);
                    q = fma(static_cast<double>(t.w), static_cast<double>(t.w), q);
                    if constexpr (kZeroPass) ss += j < nf4 ? q : 0.0;
                    else ss += q;                // t is zero past k
                    t.x *= g.x; t.y *= g.y; t.z *= g.z; t.w *= g.w;
                    const float m4 = fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w)));
                    if constexpr (kZeroPass) mxl = j < nf4 ? fmaxf(mxl, m4) : mxl;
                    else mxl = fmaxf(mxl, m4);
                }
            }
            const int e = j << 2;
            *reinterpret_cast<float4*>(&xstage[(e / EPU) * kPitch + (e % EPU)]) = t;
        }
        if constexpr (kZeroPass) {
#pragma unroll
            for (int u = 0; u < kStageF4; ++u) {
                const int j = threadIdx.x + u * kThreads;
                const int e = j << 2;
                if (j >= nf4)
                    *reinterpret_cast<float4*>(&xstage[(e / EPU) * kPitch + (e % EPU)]) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if constexpr (FOLD) {
            if (norm) {
                ss = wave_sum_f64_all(ss);
                const int fl = range_flags(mxl, kPostLo, kPostHi);
                if (lane == 0) {
                    nss[wave] = ss;
                    nfl[wave] = fl;
                }
            }
        }
        __syncthreads();
        double inv = 1.0;
        if constexpr (FOLD) {
            if (norm) {
                double t = nss[0];
                int fl = nfl[0];
#pragma unroll
                for (int w = 1; w < WAVES; ++w) {
                    t += nss[w];
                    fl |= nfl[w];
                }
                inv = norm_scale(t);
                post = fl == 2;             // the largest |x w| within [2^-40, 2^40]
                if (post) {
                    post_inv = inv;
                    inv = 1.0;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            // the lane's own (unclamped) unit: the slots of units past the row
            // hold zeros, so a lane past a short row needs no select here
            const float* xs = &xstage[unit[i] * kPitch];
#pragma unroll
            for (int v = 0; v < EPU / 4; ++v) {
                const float4 t = *reinterpret_cast<const float4*>(xs + 4 * v);
                xr[i][4 * v + 0] = t.x; xr[i][4 * v + 1] = t.y;
                xr[i][4 * v + 2] = t.z; xr[i][4 * v + 3] = t.w;
            }
            dxr[i] = 0.f; sxr[i] = 0;
        }
        // the scale on the activations (the rare path) after all the LDS
        // reads: a branch per read made each wait for its own LDS round trip
        if constexpr (FOLD) {
            if (norm && !post) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int e = 0; e < EPU; ++e) xr[i][e] = scaled(xr[i][e], inv);
            }
        }
    } else {
        if constexpr (kQuantX) {
            // The quantiser as a prologue: every workgroup quantises all of x
            // (k floats, eight lanes per 32-block, the same arithmetic as the
            // standalone quantiser) into LDS, so no separate launch is needed;
            // workgroup 0 also writes the codes and scales out if asked.
            // every lane quantises (zeros past k, into padding slots that are
            // never read); only the codes of x itself are written out
#pragma unroll
            for (int u = 0; u < kQuantF4; ++u) {
                const int j = threadIdx.x + u * kThreads;
                uint16_t hb;
                const uint32_t w =
                    quantize_q8_0_lane4(j < nf4 ? xpre[u] : make_float4(0.f, 0.f, 0.f, 0.f), hb);
                qx_s[j] = w;
                if ((j & 7) == 0) qd_s[j >> 3] = hb;
                if (blockIdx.x == 0 && p.xq_out != nullptr && j < nf4) {
                    reinterpret_cast<uint32_t*>(p.xq_out)[j] = w;
                    if ((j & 7) == 0) p.xd_out[j >> 3] = hb;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if constexpr (MODE != kQ8X) {
#pragma unroll
                for (int v = 0; v < EPU / 4; ++v) {
                    const float4 t = uvalid[i] ? xd4[i][v] : make_float4(0.f, 0.f, 0.f, 0.f);
                    xr[i][4 * v + 0] = t.x; xr[i][4 * v + 1] = t.y;
                    xr[i][4 * v + 2] = t.z; xr[i][4 * v + 3] = t.w;
                }
                dxr[i] = 0.f; sxr[i] = 0;
            } else {
                if constexpr (kQuantX) {
                    const uint4* xs = reinterpret_cast<const uint4*>(&qx_s[uload[i] * (EPU / 4)]);
#pragma unroll
                    for (int v = 0; v < EPU / 16; ++v) {
                        const uint4 t = uvalid[i] ? xs[v] : make_uint4(0u, 0u, 0u, 0u);
                        xqr[i][4 * v + 0] = t.x; xqr[i][4 * v + 1] = t.y;
                        xqr[i][4 * v + 2] = t.z; xqr[i][4 * v + 3] = t.w;
                    }
                    dxr[i] = uvalid[i] ? half_bits_to_float(qd_s[uload[i] >> SH]) : 0.f;
                } else {
#pragma unroll
                    for (int v = 0; v < EPU / 16; ++v) {
                        const uint4 t = uvalid[i] ? xq4[i][v] : make_uint4(0u, 0u, 0u, 0u);
                        xqr[i][4 * v + 0] = t.x; xqr[i][4 * v + 1] = t.y;
                        xqr[i][4 * v + 2] = t.z; xqr[i][4 * v + 3] = t.w;
                    }
                    dxr[i] = uvalid[i] ? half_bits_to_float(xdb[i]) : 0.f;
                }
                int sx = 0;
                if constexpr (TYPE == kTypeQ4_0) {
#pragma unroll
                    for (int v = 0; v < EPU / 4; ++v) sx = dot4(xqr[i][v], 0x01010101u, sx);
                }
                sxr[i] = sx;
            }
        }
        // split rows: the WS waves of a row group hold all of x between them,
        // so the sum of squares is a wave sum plus an LDS sum over the slices
        // in fixed order
        if constexpr (MODE != kQ8X && FOLD) {
            if (norm) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
#pragma unroll
                    for (int v = 0; v < EPU / 4; ++v) {
                        const float4 g = gd4[i][v];
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            ss = fma(static_cast<double>(xr[i][4 * v + c]), static_cast<double>(xr[i][4 * v + c]), ss);
                        xr[i][4 * v + 0] *= g.x; xr[i][4 * v + 1] *= g.y;
                        xr[i][4 * v + 2] *= g.z; xr[i][4 * v + 3] *= g.w;
#pragma unroll
                        for (int c = 0; c < 4; ++c) mxl = fmaxf(mxl, fabsf(xr[i][4 * v + c]));   // zero past k
                    }
                }
                ss = wave_sum_f64_all(ss);
                const int fl0 = range_flags(mxl, kPostLo, kPostHi);
                if (lane == 0) {
                    nss[wave] = ss;
                    nfl[wave] = fl0;
                }
                __syncthreads();
                double t = nss[sub * WS];
                int fl = nfl[sub * WS];
#pragma unroll
                for (int sl = 1; sl < WS; ++sl) {
                    t += nss[sub * WS + sl];
                    fl |= nfl[sub * WS + sl];
                }
                const double inv = norm_scale(t);
                post = fl == 2;             // the largest |x w| within [2^-40, 2^40]
                if (post) {
                    post_inv = inv;
                } else {
#pragma unroll
                    for (int i = 0; i < NI; ++i)
#pragma unroll
                        for (int e = 0; e < EPU; ++e) xr[i][e] = scaled(xr[i][e], inv);
                }
            }
        }
    }

    // ---- epilogue of one finished row: residual, soft cap, store, argmax --
    unsigned long long best = 0ull;
    auto post_scale = [&](float v) {
        if constexpr (FOLD) return post ? scaled(v, post_inv) : v;
        else return v;
    };
    auto emit = [&](int row, float v) {
        if constexpr (FOLD) {
            (void)row;
            if (p.residual != nullptr) v += resv;
            if (p.softcap > 0.0f) v = p.softcap * tanhf(v / p.softcap);
        }
        p.y[row] = v;
        if constexpr (FOLD) {
            const unsigned long long key = argmax_key(v, row);
            best = key > best ? key : best;
        }
    };

    // ---- one row group: the dot over this lane's units ------------------
    auto dot_group = [&](const uint4 (&qd)[NI][NMAT][R], const ScaleT (&dd)[NI][NMAT][R], int r0,
                         float (&acc)[NMAT][R]) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    // the scale bits pass through an opaque statement here, at
                    // their use: otherwise the compiler unpacks or masks them
                    // right after the staging, waiting there for every load
                    uint32_t dbits = dd[i][m][r];
                    asm volatile("" : "+v"(dbits));
                    if constexpr (MODE != kQ8X) {
                        // the binary16 scale enters the FMA as it is
                        // (v_fma_mix_f32: the same single rounding as after
                        // an exact conversion); lanes past the row take +0
                        uint32_t hb = uvalid[i] ? dbits : 0u;
                        asm volatile("" : "+v"(hb));     // keeps the select on the bits
                        acc[m][r] = fmaf(half_bits_to_float(static_cast<uint16_t>(hb)),
                                         unit_dot_f32<TYPE>(qd[i][m][r], xr[i]), acc[m][r]);
                    } else {
                        const float dw = uvalid[i] ? half_bits_to_float(static_cast<uint16_t>(dbits)) : 0.f;
                        int s = unit_dot_q8<TYPE>(qd[i][m][r], xqr[i], sxr[i]);
                        if constexpr (TYPE == kTypeQ8_0) {
                            // a block is two adjacent lanes' units: S_b = s(2t) + s(2t+1)
                            s += dpp_i32<kDppQuadSwap1>(s);
                        }
                        const bool owner = (TYPE == kTypeQ4_0) || ((lane & 1) == 0);
                        const int row = r0 + r;
                        if (p.blockdots != nullptr && owner && uvalid[i] && row < p.n)
                            p.blockdots[static_cast<int64_t>(row) * p.nb + (unit[i] >> SH)] = s;
                        const float sc = dw * dxr[i];          // exact: 11-bit x 11-bit
                        acc[m][r] = owner ? fmaf(sc, static_cast<float>(s), acc[m][r]) : acc[m][r];
                    }
                }
        }
    };

    // ---- cross-lane and cross-wave reduction, epilogue and store --------
    __shared__ float lpart[WAVES][NMAT][R];
    auto finish_group = [&](float (&acc)[NMAT][R], int r0) {
        float t0, t1 = 0.f;
        if constexpr (kV == 1) {
            t0 = wave_sum_swapped(acc[0][0]);
        } else if constexpr (kV == 4) {
            t0 = wave_sum4_rows(acc[0][0], acc[1 / R][1 % R], acc[2 / R][2 % R], acc[3 / R][3 % R]);
        } else {
            t0 = wave_sum4_rows(acc[0][0], acc[0][1 % R], acc[0][2 % R], acc[0][3 % R]);
            t1 = wave_sum4_rows(acc[NMAT - 1][0], acc[NMAT - 1][1 % R], acc[NMAT - 1][2 % R], acc[NMAT - 1][3 % R]);
        }
        const int q = lane >> 4;
        const int vq = ((q & 1) << 1) | (q >> 1);     // the value row q holds

        if constexpr (WS == 1) {
            // The rows' epilogues -- GELU, soft cap, argmax key -- run side
            // by side in their finishing lanes.
            if constexpr (kV == 4 && NMAT == 2) {
                // rows hold g0, u0, g1, u1: one row swap gives lanes 0..31
                // (g0, u0) and lanes 32..63 (g1, u1)
                const f32x2_t gu = swap_rows(t0, t0);
                if ((lane & 31) == 0) {
                    const int row = r0 + (lane >> 5);
                    if (row < p.n) emit(row, gelu_tanh(post_scale(gu.x)) * post_scale(gu.y));
                }
            } else if constexpr (kV == 8) {
                if ((lane & 15) == 0) {
                    const int row = r0 + vq;
                    if (row < p.n) emit(row, gelu_tanh(post_scale(t0)) * post_scale(t1));
                }
            } else if ((lane & 15) == 0 && (kV == 4 || lane == 0)) {
                const int row = r0 + (kV == 1 ? 0 : vq);
                if (row < p.n) emit(row, post_scale(t0));
            }
        } else {
            if ((lane & 15) == 0 && (kV != 1 || lane == 0)) {
                if constexpr (kV == 1) {
                    lpart[wave][0][0] = t0;
                } else if constexpr (kV == 4) {
                    lpart[wave][vq / R][vq % R] = t0;
                } else {
                    lpart[wave][0][vq] = t0;
                    lpart[wave][NMAT - 1][vq] = t1;
                }
            }
            __syncthreads();
            if (slice == 0 && lane < R) {
                const int row = r0 + lane;
                float tot[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    float t = lpart[wave][m][lane];
#pragma unroll
                    for (int s = 1; s < WS; ++s) t += lpart[wave + s][m][lane];
                    tot[m] = post_scale(t);
                }
                if (row < p.n) {
                    if constexpr (MODE == kFFN)
                        emit(row, gelu_tanh(tot[0]) * tot[1]);
                    else
                        emit(row, tot[0]);
                }
            }
            __syncthreads();
        }
    };

    // ---- the workgroup's row groups, gridDim.x apart ----------------------
    // The grid never exceeds the groups, so the first one exists; the loop
    // condition is uniform over the workgroup, so every wave reaches the
    // barriers in finish_group. One register set: the next group's loads are
    // issued after this group's dot (its quants are dead by then) and fly
    // during the reduction and the stores.
    if constexpr (kPinned) {
        for (;;) {
            const int r0 = (it * SUBS + sub) * R;
            const int itn = it + gridDim.x;
            const bool more = itn * SUBS < p.row_groups;
            float acc[NMAT][R];
            dot_group(q, db, r0, acc);
            // pin the order: the dot is finished (its results pass through
            // an opaque statement) before a memory barrier the next loads
            // cannot be hoisted over -- otherwise they go out first into a
            // second register set, and the loop copies one set into the other
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[m][r]));
            asm volatile("" ::: "memory");
            if (more) {
                load_res(resv_next, (itn * SUBS + sub) * R);
                load_group(q, db, (itn * SUBS + sub) * R);
            }
            finish_group(acc, r0);
            if (!more) break;
            resv = resv_next;
            it = itn;
        }
    } else {
        // (the compiler is free to hoist the next group's loads here)
        for (; it * SUBS < p.row_groups; it += gridDim.x) {
            const int r0 = (it * SUBS + sub) * R;
            const int itn = it + gridDim.x;
            float acc[NMAT][R];
            dot_group(q, db, r0, acc);
            if (itn * SUBS < p.row_groups) {
                load_res(resv_next, (itn * SUBS + sub) * R);
                load_group(q, db, (itn * SUBS + sub) * R);
            }
            finish_group(acc, r0);
            resv = resv_next;
        }
    }

    // ---- argmax partial of this workgroup (a maximum: exact in any order) --
    if (FOLD && p.part != nullptr) {
        __shared__ unsigned long long keys[WAVES];
        const unsigned long long wb = wave_max_u64(best);
        if (lane == 0) keys[threadIdx.x / kWave] = wb;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long b = keys[0];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) b = keys[w] > b ? keys[w] : b;
            p.part[blockIdx.x] = b;
        }
    }
}

// Second stage of the argmax: one workgroup folds the per-workgroup keys
// (1 <= nparts <= kArgmaxParts). Each thread issues all of its loads before
// it waits (indexes past nparts re-read the last key, which changes no
// maximum), then the waves fold their lanes and thread 0 the waves.
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxParts = static_cast<int>(kArgmaxWorkspaceBytes / sizeof(unsigned long long));
constexpr int kArgmaxPer = (kArgmaxParts + kArgmaxThreads - 1) / kArgmaxThreads;
__global__ __launch_bounds__(kArgmaxThreads)
void argmax_reduce_kernel(const unsigned long long* __restrict__ part, int nparts, int32_t* __restrict__ index,
                          float* __restrict__ value) {
    unsigned long long kv[kArgmaxPer];
#pragma unroll
    for (int j = 0; j < kArgmaxPer; ++j) kv[j] = part[min(static_cast<int>(threadIdx.x) + j * kArgmaxThreads, nparts - 1)];
    unsigned long long b = kv[0];
#pragma unroll
    for (int j = 1; j < kArgmaxPer; ++j) b = kv[j] > b ? kv[j] : b;
    b = wave_max_u64(b);
    __shared__ unsigned long long keys[kArgmaxThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) keys[threadIdx.x / kWave] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kArgmaxThreads / kWave; ++w) b = keys[w] > b ? keys[w] : b;
        const unsigned long long k = b;
        const uint32_t hi = static_cast<uint32_t>(k >> 32);
        const uint32_t u = (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi;
        *index = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));
        *value = hi == 0u ? __builtin_nanf("") : __builtin_bit_cast(float, u);
    }
}

// ---------------------------------------------------------------------------
// Host-side launch: pick the K split (WS) and units per lane (NI) from k.
// ---------------------------------------------------------------------------

namespace {

constexpr int kMaxGrid = GQ_QMV_MAX_GRID;
// the argmax first stage writes one 8-byte key per workgroup (its grid is
// also capped to the workspace at launch)
static_assert(sizeof(unsigned long long) * kMaxGrid <= kArgmaxWorkspaceBytes, "argmax workspace too small");

// Compute units of the current device, queried once per device.
inline int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Workgroups of one kernel that can be resident on a CU at once: a property
// of that kernel's code object (registers, LDS, workgroup size). The caller
// keeps the answer in a function-local static of its own instantiation, so
// every kernel variant has its own (one query per variant per process).
template <typename K>
int occupancy_per_cu(K kernel, int threads) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, threads, 0) != hipSuccess || b < 1) b = 1;
    return b;
}

template <int TYPE, int MODE, int NI, int WS, int R, bool FOLD>
hipError_t launch_variant(QmvParams p, hipStream_t stream, int* grid_out) {
    constexpr int WAVES = Waves<WS, MODE, FOLD, R>::value;
    constexpr int SUBS = WAVES / WS;
    p.row_groups = (p.n + R - 1) / R;
    const int64_t iters = (static_cast<int64_t>(p.row_groups) + SUBS - 1) / SUBS;
    const auto kernel = qmv_kernel<TYPE, MODE, NI, WS, R, FOLD>;
    // resident workgroups: the persistent grid is never larger, so no
    // workgroup waits for a second dispatch round (one static per variant)
    static const int per_cu = occupancy_per_cu(kernel, WAVES * kWave);
    int64_t cap = static_cast<int64_t>(per_cu) * device_cus();
    const int64_t max_grid = kMaxGrid * 4 / WAVES;
    cap = cap < max_grid ? cap : max_grid;
    // the argmax first stage writes one 8-byte key per workgroup
    const int64_t max_parts = static_cast<int64_t>(kArgmaxWorkspaceBytes / sizeof(unsigned long long));
    if (p.part != nullptr && cap > max_parts) cap = max_parts;
    const int grid = static_cast<int>(iters < cap ? iters : cap);
    if (grid_out != nullptr) *grid_out = grid;
    return launch_kernel(kernel, dim3(grid), dim3(WAVES * kWave), stream, p);
}

template <int TYPE, int MODE, int NI, int WS, int R>
hipError_t launch_rows(QmvParams p, hipStream_t stream, int* grid_out) {
    // the folded variant: the fp32 prologue/epilogue folds, or (integer path)
    // the activation quantiser as a prologue
    const bool fold = p.norm_w != nullptr || p.residual != nullptr || p.softcap > 0.0f || p.part != nullptr ||
                      (MODE == kQ8X && p.x != nullptr);
    if (fold) return launch_variant<TYPE, MODE, NI, WS, R, true>(p, stream, grid_out);
    return launch_variant<TYPE, MODE, NI, WS, R, false>(p, stream, grid_out);
}

// Rows per wave step (measured on MI355X): rows split over 4 or 8 waves
// stream 4 rows at a time; very tall matrices take 4 (each wave loops over
// many groups); the gate+up pass takes 2 row pairs; shorter matvecs, and the
// integer path quantising x in its prologue, take 1 row at 8 waves per
// workgroup, so more waves share the dequantisation work.
template <int TYPE, int MODE, int NI, int WS>
hipError_t launch_cfg(QmvParams p, hipStream_t stream, int* grid_out) {
    if constexpr (Waves<WS, MODE, false, GQ_QMV_R_SPLIT>::value >= 16) {
        // 1024-thread workgroups cap a lane at 128 VGPRs: 4 rows (2 row pairs
        // for the gate+up FFN) fit unspilled
        return launch_rows<TYPE, MODE, NI, WS, (MODE == kFFN ? 2 : 4)>(p, stream, grid_out);
    } else if constexpr (WS >= 4) {
        return launch_rows<TYPE, MODE, NI, WS, GQ_QMV_R_SPLIT>(p, stream, grid_out);
    } else {
        const int64_t quant_bytes = static_cast<int64_t>(p.n) * p.units * 16;
        const bool tall = MODE == kF32                        ? quant_bytes >= GQ_QMV_TALL_MIN_BYTES
                          : (MODE == kQ8X && p.x == nullptr) ? quant_bytes >= GQ_QMV_TALL_MIN_BYTES_Q8
                                                             : p.n >= GQ_QMV_TALL_MIN_N;
        if (tall) return launch_rows<TYPE, MODE, NI, WS, GQ_QMV_R_TALL>(p, stream, grid_out);
        if constexpr (MODE == kQ8X) {
            if (p.x != nullptr) return launch_rows<TYPE, MODE, NI, WS, GQ_QMV_R_Q8X>(p, stream, grid_out);
        }
        return launch_rows<TYPE, MODE, NI, WS, (MODE == kFFN ? GQ_QMV_R_FFN : GQ_QMV_R_SHORT)>(p, stream, grid_out);
    }
}

// units per lane needed when the row is split over ws waves
inline int units_per_lane(int units, int ws) {
    const int per_wave = (units + ws - 1) / ws;
    return (per_wave + kWave - 1) / kWave;
}

template <int TYPE, int MODE>
hipError_t dispatch(QmvParams p, hipStream_t stream, int* grid_out = nullptr) {
    // The lane's activation slice stays at <= 32 values in VGPRs (Q8_0: two
    // units, Q4_0: one unit); longer rows are split over more waves.
    constexpr int kNiMax = (TYPE == kTypeQ8_0) ? 2 : 1;
    if (units_per_lane(p.units, 1) == 1) return launch_cfg<TYPE, MODE, 1, 1>(p, stream, grid_out);
    if (units_per_lane(p.units, 1) <= kNiMax) return launch_cfg<TYPE, MODE, kNiMax, 1>(p, stream, grid_out);
    if (units_per_lane(p.units, 2) <= kNiMax) return launch_cfg<TYPE, MODE, kNiMax, 2>(p, stream, grid_out);
    if (units_per_lane(p.units, 4) <= kNiMax) return launch_cfg<TYPE, MODE, kNiMax, 4>(p, stream, grid_out);
    if (units_per_lane(p.units, 8) <= kNiMax) return launch_cfg<TYPE, MODE, kNiMax, 8>(p, stream, grid_out);
    if (units_per_lane(p.units, 16) <= kNiMax) return launch_cfg<TYPE, MODE, kNiMax, 16>(p, stream, grid_out);
    return hipErrorInvalidValue;    // beyond the documented maximum k (32768)
}

QmvParams base_params(const void* qs, const uint16_t* d, int64_t n, int64_t k, int bytes_per_32) {
    QmvParams p{};
    p.qs = static_cast<const uint8_t*>(qs);
    p.d = d;
    p.n = static_cast<int>(n);
    p.units = static_cast<int>(k / 32 * bytes_per_32 / 16);
    p.nb = static_cast<int>(k / 32);
    p.k = static_cast<int>(k);
    p.inv_k = 1.0 / static_cast<double>(k);
    return p;
}

}  // namespace

hipError_t launch_qmv_f32(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                          const float* x, const float* norm_w, float norm_eps, const float* residual,
                          float* y, hipStream_t stream) {
    QmvParams p = base_params(qs, d, n, k, type == kTypeQ8_0 ? 32 : 16);
    p.x = x; p.y = y; p.norm_w = norm_w; p.norm_eps = norm_eps; p.residual = residual;
    return type == kTypeQ8_0 ? dispatch<kTypeQ8_0, kF32>(p, stream) : dispatch<kTypeQ4_0, kF32>(p, stream);
}

hipError_t launch_qmv_argmax(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                             const float* x, const float* norm_w, float norm_eps, float softcap,
                             float* y, void* workspace, int32_t* index, float* value, hipStream_t stream) {
    QmvParams p = base_params(qs, d, n, k, type == kTypeQ8_0 ? 32 : 16);
    p.x = x; p.y = y; p.norm_w = norm_w; p.norm_eps = norm_eps; p.softcap = softcap;
    p.part = static_cast<unsigned long long*>(workspace);
    int grid = 0;
    hipError_t e = type == kTypeQ8_0 ? dispatch<kTypeQ8_0, kF32>(p, stream, &grid)
                                     : dispatch<kTypeQ4_0, kF32>(p, stream, &grid);
    if (e != hipSuccess) return e;
    return launch_kernel(argmax_reduce_kernel, dim3(1), dim3(kArgmaxThreads), stream,
                         static_cast<const unsigned long long*>(workspace), grid, index, value);
}

// ---- the argmax's partials in library-held device memory -----------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the first stage's per-workgroup keys go to this file-scope array
// instead of a caller workspace. Its size is the workspace size, which the
// first stage's grid never exceeds (the grid is capped at it at launch). Each
// device holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device
// (the array's name on the host is a stand-in, not a device address). The
// stages write every key they read, so no part of it needs clearing; calls
// that overlap on one device share it and race.
static __device__ __align__(256) unsigned long long scratch[kArgmaxWorkspaceBytes / sizeof(unsigned long long)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];     // per device, set once under the mutex

// This device's address of `scratch`, looked up on the first call on the
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_qmv_argmax_noalloc(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                                     const float* x, const float* norm_w, float norm_eps, float softcap,
                                     float* y, int32_t* index, float* value, hipStream_t stream) {
    static_assert(sizeof(scratch) == kArgmaxWorkspaceBytes, "scratch holds one workspace");
    void* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_qmv_argmax(type, qs, d, n, k, x, norm_w, norm_eps, softcap, y, ws, index, value, stream);
}

hipError_t launch_qmv_q8(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k,
                         const int8_t* xq, const uint16_t* xd, float* y, int32_t* blockdots,
                         hipStream_t stream) {
    if (type == kTypeQ8_0) {
        QmvParams p = base_params(qs, d, n, k, 32);
        p.xq = xq; p.xd = xd; p.y = y; p.blockdots = blockdots;
        return dispatch<kTypeQ8_0, kQ8X>(p, stream);
    }
    QmvParams p = base_params(qs, d, n, k, 16);
    p.xq = xq; p.xd = xd; p.y = y; p.blockdots = blockdots;
    return dispatch<kTypeQ4_0, kQ8X>(p, stream);
}

hipError_t launch_qmv_q8x(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                          int8_t* xq_out, uint16_t* xd_out, float* y, int32_t* blockdots, hipStream_t stream) {
    QmvParams p = base_params(qs, d, n, k, type == kTypeQ8_0 ? 32 : 16);
    p.x = x; p.xq_out = xq_out; p.xd_out = xd_out; p.y = y; p.blockdots = blockdots;
    return type == kTypeQ8_0 ? dispatch<kTypeQ8_0, kQ8X>(p, stream) : dispatch<kTypeQ4_0, kQ8X>(p, stream);
}

hipError_t launch_ffn_gate_up(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs,
                              const uint16_t* u_d, int64_t n_ff, int64_t k, const float* x,
                              const float* norm_w, float norm_eps, float* h, hipStream_t stream) {
    QmvParams p = base_params(g_qs, g_d, n_ff, k, 16);
    p.qs2 = u_qs; p.d2 = u_d; p.x = x; p.y = h; p.norm_w = norm_w; p.norm_eps = norm_eps;
    return dispatch<kTypeQ4_0, kFFN>(p, stream);
}

}  // namespace gq
