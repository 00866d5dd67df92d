// gq_device.hpp -- device-side helpers shared by the libgq kernels (gfx950,
// wave64). Nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;   // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlockThreads / kWave;

constexpr int kTypeQ4_0 = 2;
constexpr int kTypeQ8_0 = 8;

// binary16 bits -> fp32 (exact; v_cvt_f32_f16 keeps fp16 subnormals).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// DPP move of a 32-bit value within a row of 16 lanes (all lanes valid for
// the quad_perm and mirror patterns used here).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15 - i within 16

// Sum of v over the 64 lanes of the wave, returned in every lane. The order
// is fixed (butterfly inside each 16-lane row, then rows 0+1 and 2+3), so the
// result is bitwise reproducible and identical in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// gfx950 lane swaps: v_permlane32_swap_b32 exchanges the upper 32 lanes of
// a with the lower 32 lanes of b, v_permlane16_swap_b32 the odd 16-lane rows
// of a with the even rows of b; each returns both registers. The returned
// pair is reinterpreted as a whole: a bit cast of one element of the
// returned integer vector has compiled to a read of its first element.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2_t swap_halves(float a, float b) {
    return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                                         __builtin_bit_cast(uint32_t, b), false, false));
}
__device__ __forceinline__ f32x2_t swap_rows(float a, float b) {
    return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                                         __builtin_bit_cast(uint32_t, b), false, false));
}
// Lane i plus lane i + 32: lanes 0..31 receive a's sums, lanes 32..63 b's.
__device__ __forceinline__ float fold_halves(float a, float b) {
    const f32x2_t t = swap_halves(a, b);
    return t.x + t.y;
}
// Row 2j plus row 2j + 1 (rows of 16 lanes): rows 0 and 2 receive a's sums
// (of rows 0 + 1 and 2 + 3), rows 1 and 3 b's.
__device__ __forceinline__ float fold_rows(float a, float b) {
    const f32x2_t t = swap_rows(a, b);
    return t.x + t.y;
}
// Sum over the 16 lanes of each row, identical in every lane of the row.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    return v;
}
// Four sums over the 64 lanes at once, transposed: every lane of row q
// receives the sum of value ((q & 1) << 1) | (q >> 1) of (a0, a1, a2, a3),
// i.e. rows 0..3 hold the sums of a0, a2, a1, a3 -- two lane-half swaps,
// one row swap and four DPP adds where four separate sums take 16 DPP adds
// and 16 lane reads. Every value is summed in the same fixed order (lanes
// i + i+32, then rows 0+1 / 2+3, then the butterfly in the row), so the
// result is reproducible.
__device__ __forceinline__ float wave_sum4_rows(float a0, float a1, float a2, float a3) {
    return row_sum(fold_rows(fold_halves(a0, a1), fold_halves(a2, a3)));
}
// One sum over the 64 lanes in the same order, in every lane.
__device__ __forceinline__ float wave_sum_swapped(float a) {
    const float h = fold_halves(a, a);
    return row_sum(fold_rows(h, h));
}

// One DPP move of a double: its two 32-bit halves with the same control.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false));
    const uint32_t hi =
        static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false));
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
// The sum of v over the 64 lanes, in every lane, with no lane reads: a
// lane-half swap and a row swap (each moving the two 32-bit halves of the
// value) add the four rows' lanes pairwise, then four DPP steps add the 16
// lanes of a row. Every lane holds the same bits.
__device__ __forceinline__ double join_f64(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64_all(double v) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    const u32x2_t l32 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(
        static_cast<uint32_t>(b), static_cast<uint32_t>(b), false, false));
    const u32x2_t h32 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(
        static_cast<uint32_t>(b >> 32), static_cast<uint32_t>(b >> 32), false, false));
    v = join_f64(l32.x, h32.x) + join_f64(l32.y, h32.y);
    b = __builtin_bit_cast(uint64_t, v);
    const u32x2_t l16 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(
        static_cast<uint32_t>(b), static_cast<uint32_t>(b), false, false));
    const u32x2_t h16 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(
        static_cast<uint32_t>(b >> 32), static_cast<uint32_t>(b >> 32), false, false));
    v = join_f64(l16.x, h16.x) + join_f64(l16.y, h16.y);
    v += dpp_f64<kDppQuadSwap1>(v);
    v += dpp_f64<kDppQuadSwap2>(v);
    v += dpp_f64<kDppRowHalfMirror>(v);
    v += dpp_f64<kDppRowMirror>(v);
    return v;
}

// The largest of v over the 64 lanes, in every lane (64-bit keys, moved as
// two 32-bit halves per step).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
        const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Where the largest of v over the 64 lanes falls against [lo, hi], without
// finding it: bit 0 set if some lane's v is above hi, bit 1 if some lane's v
// is at or above lo (two ballots). The largest lies within [lo, hi] exactly
// when the result is 2. (v is a lane's own maximum, NaN-free as fmaxf makes it.)
__device__ __forceinline__ int range_flags(float v, float lo, float hi) {
    const unsigned long long above = __ballot(v > hi);
    const unsigned long long reach = __ballot(v >= lo);
    return (above != 0ull ? 1 : 0) | (reach != 0ull ? 2 : 0);
}

// Exact int8x4 dot product with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Tanh-form GELU, G(t) = 0.5 t (1 + tanh(z)), z = sqrt(2/pi) (t + 0.044715 t^3),
// evaluated as t / (1 + exp(-2 z)) (the same function: 0.5 (1 + tanh z) is
// the logistic function of 2z). For large positive z the exponential
// underflows to 0 and G -> t; for large negative z it overflows to +inf and
// G -> -0, so finite t never produces NaN.
__device__ __forceinline__ float gelu_tanh(float t) {
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    const float z = c * fmaf(0.044715f * t, t * t, t);
    // exp(-2 z) as the hardware base-2 exponential of -2 z log2(e), and the
    // hardware reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each): relative
    // error about (4 |z| + 7) 2^-24 for G(t) u, inside (8 + 10 |z|) 2^-24,
    // and 15 instructions fewer than expf and an IEEE divide per row pair.
    // z -> -inf gives 1 + e = inf and t * 0 = -0; z -> +inf gives t.
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * z);
    return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- Q8_0 activation quantiser, eight lanes per 32-element block ---------
// Each lane holds four consecutive elements of one block and the block's
// eight lanes are an aligned group of a wave (all active). Returns the
// lane's four codes packed little-endian and sets the block's binary16
// scale bits: amax (fp32, exact) -> d = binary16(amax / 127) (fp32 divide,
// round to nearest even) -> q = clamp(round half away(x / d), -127, 127)
// with the divide in fp32 by the rounded d; q = 0 when d == 0 (the
// activation quantiser of the jouleclaw-loader-gguf BENCHMARKS page, "Matmul
// throughput -- Q8_0 scalar vs NEON", taken per GGUF 32-element block). The
// same code serves the standalone quantiser and the prologue of the fused
// integer-path matvec, so both give identical codes.
__device__ __forceinline__ uint32_t quantize_q8_0_lane4(const float4 v, uint16_t& scale_bits) {
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, dpp_f32<kDppQuadSwap1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppQuadSwap2>(amax));
    amax = fmaxf(amax, dpp_f32<kDppRowHalfMirror>(amax));
    const uint16_t hb = float_to_half_bits(amax / 127.0f);
    const float dh = half_bits_to_float(hb);
    scale_bits = hb;
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int q = 0;
        if (dh != 0.0f) {
            float r = roundf(e[b] / dh);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q = static_cast<int>(r);
        }
        w |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * b);
    }
    return w;
}

}  // namespace gq
