// gq_kquant.hip -- M = 1 decode matvec over K-quant super-blocks (Q4_K, Q5_K
// and Q6_K, 256 elements each) with fp32 activations, and their load-time
// pack.
//
// What is computed follows the jouleclaw-loader-gguf BENCHMARKS page: "Q4_K
// matmul" works on 32-element sub-blocks, each with a scale and a minimum,
// w = d_sub q - m_sub, and splits the sum as d_sub sum(a q) - m_sub sum(a);
// "Q5_K + Q6_K matmul" takes one high bit per element for Q5_K, and two high
// bits and a signed -32 offset for Q6_K. The super-block byte layout (not
// printed on the pages) is the GGUF one:
//   Q4_K (144 B): binary16 d, binary16 dmin, 12 bytes of packed 6-bit
//     sub-block scales sc_j and minimums m_j, 128 quant bytes; quant byte
//     32g + l holds element 64g + l (low nibble) and 64g + 32 + l (high);
//     element e of sub-block j = e / 32 is d sc_j q - dmin m_j.
//   Q5_K (176 B): d, dmin and the 12 scale bytes as Q4_K, qh[32], 128 quant
//     bytes as Q4_K; the fifth bit of element 64g + l is bit 2g of qh byte
//     l (l < 32), that of 64g + 32 + l bit 2g + 1; q in 0..31.
//   Q6_K (210 B): ql[128] (low four bits), qh[64] (high two bits), int8
//     scales[16], binary16 d; element e is d scales[e / 16] (q - 32).
//
// Packed layout (gq_kq_pack; sections 256-byte aligned). Every value is
// kept bit for bit; only the places of the scale and high-bit fields change,
// so that a lane finds its own fields in one load with no unpacking:
//   Q4_K: qs [n][k/2] (the quant bytes of each super-block in order), then
//         hdr [n][k/256][16]: d, dmin, then for each 64-element chunk g
//         (sub-blocks 2g and 2g + 1) the 24-bit field sc_2g | sc_2g+1 << 6 |
//         m_2g << 12 | m_2g+1 << 18 in bytes 4 + 3g .. 6 + 3g.
//   Q5_K: qs and hdr as Q4_K, then fifth [n][k/32]: one 32-bit word per
//         16-byte quant unit holding the fifth bits of its 32 elements
//         (layout at kq5_lo_pos).
//   Q6_K: ql [n][k/2] (as in the super-block); qh [n][k/4]: for each 16-byte
//         unit of ql (below), 8 bytes holding the high two bits of its 32
//         elements (layout at qh_fields); sc [n][k/16]: for each unit, its two
//         int8 scales (low run, high run); d [n][k/256] binary16.
// Decomposition: lane l of a wave owns unit l of its slice of the row (16
// bytes = 32 elements, in two runs of 16 that share a sub-block scale each:
//   Q4_K / Q5_K unit u of a super-block: runs 64(u/2) + 16(u%2) (low
//     nibbles, sub-block u & 6) and that + 32 (high nibbles, sub-block
//     (u & 6) + 1);
//   Q6_K unit 4h + j: runs 128h + 16j (scale 8h + j) and that + 64 (scale
//     8h + j + 4), the high bits from the unit's own 8 packed qh bytes).
// The lane's 32 activations stay in VGPRs for every row it streams. Rows
// longer than 2048 elements are split over WS waves whose partial sums meet
// in LDS in slice order; waves stream R rows per step; sums over lanes use
// lane-half and row swaps and DPP (wave_sum4_rows; at other step sizes
// wave_sum_last_row), fixed order, no atomics.
#include <atomic>

#include "gq_device.hpp"
#include "gq_launch.hpp"

// Measured on MI355X (fp32 x, k = 2048; 262144 / 8192 rows, and 2048 x 8192):
// 4 rows per step with up to 2048 workgroups: Q4_K 52.2 / 4.5 / 4.7 us with
// the nibbles read as binary16 subnormals (59.0 / 4.7 / 4.8 with the
// normal-range form and its packed add), Q6_K 73.5-73.8 / 5.1 / 5.3 us
// (five waves per SIMD), with the four rows summed over the lanes together (one row
// at a time was 2-3 % slower; with the packed fields read directly; the
// byte-copy layout, unpacking the GGUF fields in the loop, gave 60-62 /
// 5.3 / 5.6 and 82-84 / 6.0-6.2 / 5.5-5.8 us); 2 rows at 1024 workgroups
// were slower; matrices with fewer 4-row groups than the device has SIMDs
// take 2 rows per step instead, so that every SIMD gets a wave (2048 x 2048:
// Q4_K 3.14 -> 2.92 us, Q6_K 3.88 -> 3.27 us; 1 row per step was slower, and
// at 8192 rows and on split rows 4 rows stay faster). Two row groups in
// flight per wave (a second register set)
// measured no better: the loop is bound by its VALU work (for the exact
// nibble dot about 1.6 instructions per element in Q4_K and 2.8 in Q6_K;
// 2.7 and 3.5 per element in all), not by load latency.
#ifndef GQ_KQ_R
#define GQ_KQ_R 4            // rows per wave step
#endif
#ifndef GQ_KQ_R_SHORT
#define GQ_KQ_R_SHORT 2      // rows per wave step for matrices with few rows (below)
#endif
#ifndef GQ_KQ_MAX_GRID
#define GQ_KQ_MAX_GRID 2048  // workgroups of 4 waves at most
#endif

namespace gq {

namespace {

// The sum of v over the 64 lanes of the wave, as wave_sum computes it, but
// complete only in lanes 48..63 (the last row of 16): two DPP row broadcasts
// take the place of the four lane reads. Every row adds
// lane 15 of the row before it (row 0 adds 0), then rows 2 and 3 add lane 31.
// Row 3 ends with (s3 + s2) + (s1 + s0) -- the same additions as wave_sum,
// so the same bits (fp32 addition is commutative); the other rows hold
// partial sums. (Full row masks and zero for missing source lanes let each
// step be one v_add_f32_dpp.)
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
__device__ __forceinline__ float wave_sum_last_row(float v) {
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppRowBcast15,
                                                               0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppRowBcast31,
                                                               0xF, 0xF, true));
    return v;
}

// The sums of a and b over the 64 lanes, complete in lanes 0..31 (a) and
// 32..63 (b): one lane-half swap adds the halves of both, one row swap the
// two rows of each half, four DPP steps the 16 lanes of a row.
__device__ __forceinline__ float wave_sum2_rows(float a, float b) {
    const float h = fold_halves(a, b);
    return row_sum(fold_rows(h, h));
}

constexpr int kTypeQ4_K = 12;
constexpr int kTypeQ5_K = 13;
constexpr int kTypeQ6_K = 14;

inline size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct KqLayout {
    size_t o[4];      // section offsets
    size_t total;
};

}  // namespace

// Section offsets of the packed array of an n x k K-quant matrix.
size_t kq_layout(int type, int64_t n, int64_t k, size_t* offsets) {
    const size_t nn = static_cast<size_t>(n), kk = static_cast<size_t>(k);
    size_t o[4] = {0, 0, 0, 0}, total = 0;
    if (type == kTypeQ4_K) {
        o[1] = round256(nn * kk / 2);
        total = o[1] + nn * (kk / 256) * 16;
    } else if (type == kTypeQ5_K) {
        o[1] = round256(nn * kk / 2);
        o[2] = o[1] + round256(nn * (kk / 256) * 16);
        total = o[2] + nn * (kk / 32) * 4;
    } else {
        o[1] = round256(nn * kk / 2);
        o[2] = o[1] + round256(nn * kk / 4);
        o[3] = o[2] + round256(nn * kk / 16);
        total = o[3] + nn * (kk / 256) * 2;
    }
    if (offsets != nullptr)
        for (int i = 0; i < 4; ++i) offsets[i] = o[i];
    return total;
}

namespace {

// qh_fields: the 8 high-bit bytes of a Q6_K unit are two words, one per pair
// of the unit's 32-bit ql words (2p, 2p + 1). ql word c holds elements
// 4c .. 4c + 3 of both runs (bytes b = 0..3: low nibble -> low run, high
// nibble -> high run). Word c's eight 2-bit fields sit where the fp16
// construction below ORs them in: low-run element 4c + b at bit
// kq6_lo_pos(b) = 4, 6, 20, 22 and high-run element 4c + b at
// kq6_hi_pos(b) = 8, 10, 24, 26 (b = 1 and 3 are brought down by a shift of
// 2, together with their nibbles' shift of 8); word 2p + 1's fields are
// rotated left by 8 into the free bits of the same 32-bit word.
__host__ __device__ constexpr int kq6_lo_pos(int b) { return (b & 2) * 8 + (b & 1) * 2 + 4; }
__host__ __device__ constexpr int kq6_hi_pos(int b) { return kq6_lo_pos(b) + 4; }

// Q5_K fifth bits: one 32-bit word per 16-byte quant unit. Quant word c of
// the unit holds elements 4c .. 4c + 3 of both runs; its eight bits sit
// where the binary16 construction ORs them in -- low-run element 4c + b at
// kq5_lo_pos(b) = 4, 5, 20, 21 and high-run element 4c + b at
// kq5_hi_pos(b) = 8, 9, 24, 25 (b = 1 and 3 brought down by a shift of 1) --
// rotated left by kq5_rot(c) = 0, 2, 8, 10: the four rotated sets are
// disjoint and fill the word, so one rotate gives word c its bits in place.
__host__ __device__ constexpr int kq5_lo_pos(int b) { return (b & 2) * 8 + (b & 1) + 4; }
__host__ __device__ constexpr int kq5_hi_pos(int b) { return kq5_lo_pos(b) + 4; }
__host__ __device__ constexpr int kq5_rot(int c) { return (c & 1) * 2 + (c & 2) * 4; }

// ---------------------------------------------------------------------------
// Pack: one thread per super-block; byte loads (a GGUF block is only
// 2-byte aligned at best), 16-byte stores into the aligned sections.
// ---------------------------------------------------------------------------
template <int TYPE>
__global__ __launch_bounds__(kBlockThreads)
void kq_pack_kernel(const uint8_t* __restrict__ blocks, int64_t nsb_total, uint8_t* __restrict__ out,
                    size_t o1, size_t o2, size_t o3) {
    constexpr int BB = TYPE == kTypeQ4_K ? 144 : (TYPE == kTypeQ5_K ? 176 : 210);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nsb_total) return;
    const uint8_t* src = blocks + i * BB;
    auto word = [&](int off) {
        return static_cast<uint32_t>(src[off]) | (static_cast<uint32_t>(src[off + 1]) << 8) |
               (static_cast<uint32_t>(src[off + 2]) << 16) | (static_cast<uint32_t>(src[off + 3]) << 24);
    };
    auto copy16 = [&](int off, uint8_t* dst) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(word(off), word(off + 4), word(off + 8), word(off + 12));
    };
    if constexpr (TYPE == kTypeQ4_K || TYPE == kTypeQ5_K) {
        // Q5_K: the same header and quant bytes, the quants after its 32
        // fifth-bit bytes
        constexpr int kQs = TYPE == kTypeQ4_K ? 16 : 48;
        uint8_t* qs = out + i * 128;
#pragma unroll
        for (int c = 0; c < 8; ++c) copy16(kQs + 16 * c, qs + 16 * c);
        // the GGUF 6-bit scales and minimums (12 bytes q[0..11] after d and
        // dmin): sub-blocks 0-3 take the low six bits of q[j] (scale) and
        // q[j + 4] (minimum); sub-blocks 4-7 take the nibbles of q[j + 4]
        // (low, high) under the top two bits of q[j - 4] and q[j]
        const uint8_t* q = src + 4;
        uint32_t sc[8], mn[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sc[j] = q[j] & 63u;
            mn[j] = q[j + 4] & 63u;
            sc[j + 4] = (q[j + 8] & 15u) | ((q[j] >> 6) << 4);
            mn[j + 4] = (q[j + 8] >> 4) | ((q[j + 4] >> 6) << 4);
        }
        uint8_t h[16];
        h[0] = src[0]; h[1] = src[1]; h[2] = src[2]; h[3] = src[3];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t f = sc[2 * g] | (sc[2 * g + 1] << 6) | (mn[2 * g] << 12) | (mn[2 * g + 1] << 18);
            h[4 + 3 * g] = static_cast<uint8_t>(f);
            h[5 + 3 * g] = static_cast<uint8_t>(f >> 8);
            h[6 + 3 * g] = static_cast<uint8_t>(f >> 16);
        }
        uint32_t hw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            hw[w] = h[4 * w] | (h[4 * w + 1] << 8) | (h[4 * w + 2] << 16) | (static_cast<uint32_t>(h[4 * w + 3]) << 24);
        *reinterpret_cast<uint4*>(out + o1 + i * 16) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        if constexpr (TYPE == kTypeQ5_K) {
            // unit u = 2 g + t covers quant bytes 32 g + 16 t .. + 15:
            // elements 64 g + 16 t + e (low nibbles) and + 32 (high nibbles),
            // e < 16, whose fifth bits are bits 2 g and 2 g + 1 of GGUF qh
            // byte 16 t + e
            const uint8_t* qhs = src + 16;
            uint32_t* fw = reinterpret_cast<uint32_t*>(out + o2 + i * 32);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int g = u >> 1, t = u & 1;
                uint32_t word = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t f = 0;
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) {
                        const uint32_t qb = qhs[16 * t + 4 * c + bb];
                        f |= ((qb >> (2 * g)) & 1u) << kq5_lo_pos(bb);
                        f |= ((qb >> (2 * g + 1)) & 1u) << kq5_hi_pos(bb);
                    }
                    word |= kq5_rot(c) == 0 ? f : ((f << kq5_rot(c)) | (f >> (32 - kq5_rot(c))));
                }
                fw[u] = word;
            }
        }
    } else {
        uint8_t* ql = out + i * 128;
#pragma unroll
        for (int c = 0; c < 8; ++c) copy16(16 * c, ql + 16 * c);
        // unit u = 4 hh + j covers ql bytes 64 hh + 16 j .. + 15: elements
        // 128 hh + 16 j + e (low nibbles, the low run) and + 64 (high
        // nibbles, the high run), e < 16, whose high bits sit in qh byte
        // 32 hh + 16 (j % 2) + e at bit 2 (j / 2) (low run) and 4 + 2 (j / 2)
        uint32_t* qh = reinterpret_cast<uint32_t*>(out + o1 + i * 64);
        uint16_t* scp = reinterpret_cast<uint16_t*>(out + o2 + i * 16);
        const uint8_t* qhs = src + 128;
        const int8_t* scs = reinterpret_cast<const int8_t*>(src + 192);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int hh = u >> 2, j = u & 3;
            const int sl = 2 * (j >> 1), shi = 4 + 2 * (j >> 1);
            uint32_t field[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t f = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t qb = qhs[32 * hh + 16 * (j & 1) + 4 * c + bb];
                    f |= ((qb >> sl) & 3u) << kq6_lo_pos(bb);
                    f |= ((qb >> shi) & 3u) << kq6_hi_pos(bb);
                }
                field[c] = f;
            }
            qh[2 * u] = field[0] | ((field[1] << 8) | (field[1] >> 24));
            qh[2 * u + 1] = field[2] | ((field[3] << 8) | (field[3] >> 24));
            scp[u] = static_cast<uint16_t>(static_cast<uint8_t>(scs[8 * hh + j]) |
                                           (static_cast<uint16_t>(static_cast<uint8_t>(scs[8 * hh + j + 4])) << 8));
        }
        *reinterpret_cast<uint16_t*>(out + o3 + i * 2) =
            static_cast<uint16_t>(src[208] | (src[209] << 8));
    }
}

struct KqParams {
    const uint8_t* q;       // quant bytes [n][k/2] (Q4_K qs, Q6_K ql)
    const uint8_t* hdr;     // Q4_K, Q5_K: [n][k/256][16] headers
    const uint8_t* qh;      // Q6_K: [n][k/4]
    const int8_t* sc;       // Q6_K: [n][k/16]
    const uint16_t* d;      // Q6_K: [n][k/256]
    const float* x;         // [k]
    float* y;               // [n]
    int n;
    int k;
    int units;              // 16-byte quant units per row (k / 32)
    int row_groups;         // ceil(n / R)
    // (last: placed after hdr it moved the fields the Q4_K kernel reads, and
    // the 8192 x 2048 and 2048 x 8192 Q4_K matvecs took 4.78 / 4.91 us
    // instead of 4.55 / 4.67 with identical kernel code)
    const uint32_t* fifth;  // Q5_K: [n][k/32] fifth-bit words
};

// Waves per workgroup: 4, or WS when a row is split over more waves.
template <int WS> struct KqWaves { static constexpr int value = WS < 4 ? 4 : WS; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr float kTwoM24 = 5.9604644775390625e-08f;   // 2^-24
constexpr float kTwo24 = 16777216.0f;               // 2^24

// Two 4-bit fields of a 32-bit word, held in the low bits of its 16-bit
// halves (mask selects them), read as binary16 numbers with a zero exponent
// field: the subnormals v * 2^-24, exact, with no offset to take out.
// v_fma_mix_f32 multiplies such a half by an fp32 activation with a single
// rounding, as it does a normal one, so each product is the fp32 FMA of
// (float) v scaled by 2^-24 (exact while the result stays above 2^-126; the
// row sums are scaled back by 2^24 at the end).
__device__ __forceinline__ half2_t sub2(uint32_t w, uint32_t mask) {
    return __builtin_bit_cast(half2_t, w & mask);
}

// Five waves per SIMD: the compiler fits the loop in 88 VGPRs (no spills),
// where it would otherwise take 101 and run four (measured: 262144 x 2048
// 58.5 -> 56.5 us, 8192 x 2048 and 2048 x 8192 5.3 -> 5.1 us; six waves
// spill and are slower).
// Q5 (Q5_K): the same kernel with each quant's fifth bit OR-ed in from the
// unit's fifth-bit word (q in 0..31, still a subnormal with no offset).
template <int WS, int R, bool Q5>
__global__ __launch_bounds__(KqWaves<WS>::value * kWave) __attribute__((amdgpu_waves_per_eu(5)))
void qmv_q4_k_kernel(const KqParams p) {
    constexpr int WAVES = KqWaves<WS>::value;
    constexpr int SUBS = WAVES / WS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slice = wave % WS, sub = wave / WS;
    const int unit = slice * kWave + lane;
    const bool valid = unit < p.units;
    const uint32_t uload = static_cast<uint32_t>(min(unit, p.units - 1));
    const int nsb = p.k >> 8;
    const uint32_t sb = uload >> 3, u = uload & 7;

    // this lane's 32 activations: run a (low nibbles) and run b (high)
    const int ea = static_cast<int>(sb) * 256 + 64 * static_cast<int>(u >> 1) + 16 * static_cast<int>(u & 1);
    float xr[32];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 ta = reinterpret_cast<const float4*>(p.x + ea)[v];
        const float4 tb = reinterpret_cast<const float4*>(p.x + ea + 32)[v];
        xr[4 * v + 0] = ta.x; xr[4 * v + 1] = ta.y; xr[4 * v + 2] = ta.z; xr[4 * v + 3] = ta.w;
        xr[16 + 4 * v + 0] = tb.x; xr[16 + 4 * v + 1] = tb.y; xr[16 + 4 * v + 2] = tb.z; xr[16 + 4 * v + 3] = tb.w;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) xr[e] = valid ? xr[e] : 0.f;
    // sums of the two runs, for the minimum terms (dmin m_j sum x)
    float sxa = 0.f, sxb = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        sxa += xr[e];
        sxb += xr[16 + e];
    }
    // the whole row sum is kept at the scale 2^-24 of the subnormal quants
    sxa *= kTwoM24;
    sxb *= kTwoM24;
    // this lane's chunk g = u / 2 (sub-blocks 2g, 2g + 1): its 24-bit field
    // is bytes 3g .. 3g + 2 of the header's last 12, gathered by one byte
    // permute from the word pair (y, z) for g < 2, else (z, w)
    const uint32_t g = u >> 1;
    const bool first_pair = g < 2u;
    const uint32_t fb = first_pair ? 3u * g : 3u * g - 4u;
    const uint32_t psel = fb | ((fb + 1u) << 8) | ((fb + 2u) << 16) | (0x0Cu << 24);    // 0x0C: a zero byte

    __shared__ float lpart[WAVES][R];
    // four rows per step: their sums reduced over the wave together
    // (wave_sum4_rows), 16-lane row q finishing row ((q & 1) << 1) | (q >> 1)
    // of the step
    auto finish4 = [&](const float (&acc)[R], int r0) {
        const float t = wave_sum4_rows(acc[0], acc[1 % R], acc[2 % R], acc[3 % R]);
        const int q = lane >> 4;
        const int vq = ((q & 1) << 1) | (q >> 1);
        if constexpr (WS == 1) {
            if ((lane & 15) == 0 && r0 + vq < p.n) p.y[r0 + vq] = t * kTwo24;
        } else {
            if ((lane & 15) == 0) lpart[wave][vq % R] = t;
            __syncthreads();
            if (slice == 0 && lane < R) {
                float tt = lpart[wave][lane];
#pragma unroll
                for (int sl = 1; sl < WS; ++sl) tt += lpart[wave + sl][lane];
                if (r0 + lane < p.n) p.y[r0 + lane] = tt * kTwo24;
            }
            __syncthreads();
        }
    };
    for (int it = blockIdx.x; it * SUBS < p.row_groups; it += gridDim.x) {
        const int r0 = (it * SUBS + sub) * R;
        uint4 q[R], h[R];
        uint32_t fh[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                p.q + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 2) + uload * 16u));
            q[r] = make_uint4(t.x, t.y, t.z, t.w);
            h[r] = *reinterpret_cast<const uint4*>(p.hdr + (static_cast<uint64_t>(row) * nsb + sb) * 16u);
            if constexpr (Q5)
                fh[r] = __builtin_nontemporal_load(p.fifth + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.units) +
                                                   uload);
            else
                fh[r] = 0u;
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t w[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
            float pa = 0.f, pb = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t v = w[j], v8 = v >> 8;
                half2_t lo02, lo13, hi02, hi13;
                if constexpr (Q5) {
                    // word j's fifth bits, rotated into place: bits 4 and 20
                    // (elements 4j, 4j + 2 of the low run) and 8, 24 (the
                    // high run, nibbles in place); odd elements one bit up
                    const uint32_t hc = kq5_rot(j) == 0 ? fh[r] : __builtin_amdgcn_alignbit(fh[r], fh[r], kq5_rot(j));
                    const uint32_t hc1 = hc >> 1;
                    lo02 = __builtin_bit_cast(half2_t, (hc & 0x00100010u) | (v & 0x000F000Fu));
                    lo13 = __builtin_bit_cast(half2_t, (hc1 & 0x00100010u) | (v8 & 0x000F000Fu));
                    hi02 = __builtin_bit_cast(half2_t, (hc & 0x01000100u) | (v & 0x00F000F0u));     // 16 q
                    hi13 = __builtin_bit_cast(half2_t, (hc1 & 0x01000100u) | (v8 & 0x00F000F0u));
                } else {
                    lo02 = sub2(v, 0x000F000Fu);
                    lo13 = sub2(v8, 0x000F000Fu);
                    hi02 = sub2(v, 0x00F000F0u);     // 16 q
                    hi13 = sub2(v8, 0x00F000F0u);
                }
                pa = fmaf(static_cast<float>(lo02.x), xr[4 * j + 0], pa);
                pb = fmaf(static_cast<float>(hi02.x), xr[16 + 4 * j + 0], pb);
                pa = fmaf(static_cast<float>(lo13.x), xr[4 * j + 1], pa);
                pb = fmaf(static_cast<float>(hi13.x), xr[16 + 4 * j + 1], pb);
                pa = fmaf(static_cast<float>(lo02.y), xr[4 * j + 2], pa);
                pb = fmaf(static_cast<float>(hi02.y), xr[16 + 4 * j + 2], pb);
                pa = fmaf(static_cast<float>(lo13.y), xr[4 * j + 3], pa);
                pb = fmaf(static_cast<float>(hi13.y), xr[16 + 4 * j + 3], pb);
            }
            pb *= 0.0625f;                              // exact
            // the two sub-blocks' 6-bit scales and minimums
            uint32_t hx = h[r].x, hy = h[r].y, hz = h[r].z, hw = h[r].w;
            asm volatile("" : "+v"(hx), "+v"(hy), "+v"(hz), "+v"(hw));
            const uint32_t f = __builtin_amdgcn_perm(first_pair ? hz : hw, first_pair ? hy : hz, psel);
            const float sca = static_cast<float>(f & 63u), scb = static_cast<float>((f >> 6) & 63u);
            const float mna = static_cast<float>((f >> 12) & 63u), mnb = static_cast<float>((f >> 18) & 63u);
            // d and dmin stay binary16: v_fma_mix_f32 takes them as they are
            // (their products with fp32 values round once, as after a conversion)
            const half2_t dh = __builtin_bit_cast(half2_t, valid ? hx : 0u);
            const float t1 = fmaf(scb, pb, sca * pa);
            const float t2 = fmaf(mnb, sxb, mna * sxa);
            const float pm = fmaf(static_cast<float>(dh.y), t2, 0.f);
            acc[r] = fmaf(static_cast<float>(dh.x), t1, -pm);
        }
        if constexpr (R == 4) {
            finish4(acc, r0);
            continue;
        }
        if constexpr (R == 2 && WS == 1) {
            // two rows: lanes 0 and 32 finish rows r0 and r0 + 1
            const float t = wave_sum2_rows(acc[0], acc[1 % R]);
            if ((lane & 31) == 0 && r0 + (lane >> 5) < p.n) p.y[r0 + (lane >> 5)] = t * kTwo24;
            continue;
        }
        // (other step sizes) the row sums are complete in lanes 48..63:
        // lane 64 - R + r stores row r
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum_last_row(acc[r]);
        if constexpr (WS == 1) {
            const int lr = lane - (kWave - R);
            if (lr >= 0) {
                float a = acc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = lr == r ? acc[r] : a;
                if (r0 + lr < p.n) p.y[r0 + lr] = a * kTwo24;
            }
        } else {
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r) lpart[wave][r] = acc[r];
            }
            __syncthreads();
            if (slice == 0 && lane < R) {
                float t = lpart[wave][lane];
#pragma unroll
                for (int s = 1; s < WS; ++s) t += lpart[wave + s][lane];
                if (r0 + lane < p.n) p.y[r0 + lane] = t * kTwo24;
            }
            __syncthreads();
        }
    }
}

// Five waves per SIMD as well (94 VGPRs at four rows per step, no spills;
// measured: 2048 x 2048 3.29 -> 3.10 us, 8192 x 2048 5.32 -> 5.07 us,
// 2048 x 8192 5.47 -> 5.26 us, 262144 x 2048 74.6 -> 73.7 us).
template <int WS, int R>
__global__ __launch_bounds__(KqWaves<WS>::value * kWave) __attribute__((amdgpu_waves_per_eu(5)))
void qmv_q6_k_kernel(const KqParams p) {
    constexpr int WAVES = KqWaves<WS>::value;
    constexpr int SUBS = WAVES / WS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slice = wave % WS, sub = wave / WS;
    const int unit = slice * kWave + lane;
    const bool valid = unit < p.units;
    const uint32_t uload = static_cast<uint32_t>(min(unit, p.units - 1));
    const int nsb = p.k >> 8;
    const uint32_t sb = uload >> 3, hh = (uload >> 2) & 1u, j = uload & 3u;

    // runs: 128h + 16j (scale 8h + j) and 128h + 16j + 64 (scale 8h + j + 4)
    const int el = static_cast<int>(sb) * 256 + 128 * static_cast<int>(hh) + 16 * static_cast<int>(j);
    float xr[32];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 ta = reinterpret_cast<const float4*>(p.x + el)[v];
        const float4 tb = reinterpret_cast<const float4*>(p.x + el + 64)[v];
        xr[4 * v + 0] = ta.x; xr[4 * v + 1] = ta.y; xr[4 * v + 2] = ta.z; xr[4 * v + 3] = ta.w;
        xr[16 + 4 * v + 0] = tb.x; xr[16 + 4 * v + 1] = tb.y; xr[16 + 4 * v + 2] = tb.z; xr[16 + 4 * v + 3] = tb.w;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) xr[e] = valid ? xr[e] : 0.f;

    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));
    // low run: 1024 + q - 1056 = q - 32; high run (in place): 1024 + 16 q - 1536 = 16 (q - 32)
    const half2_t off_lo = {static_cast<_Float16>(-1056.0f), static_cast<_Float16>(-1056.0f)};
    const half2_t off_hi = {static_cast<_Float16>(-1536.0f), static_cast<_Float16>(-1536.0f)};

    __shared__ float lpart[WAVES][R];
    // four rows per step: their sums reduced over the wave together
    // (wave_sum4_rows), 16-lane row q finishing row ((q & 1) << 1) | (q >> 1)
    // of the step
    auto finish4 = [&](const float (&acc)[R], int r0) {
        const float t = wave_sum4_rows(acc[0], acc[1 % R], acc[2 % R], acc[3 % R]);
        const int q = lane >> 4;
        const int vq = ((q & 1) << 1) | (q >> 1);
        if constexpr (WS == 1) {
            if ((lane & 15) == 0 && r0 + vq < p.n) p.y[r0 + vq] = t;
        } else {
            if ((lane & 15) == 0) lpart[wave][vq % R] = t;
            __syncthreads();
            if (slice == 0 && lane < R) {
                float tt = lpart[wave][lane];
#pragma unroll
                for (int sl = 1; sl < WS; ++sl) tt += lpart[wave + sl][lane];
                if (r0 + lane < p.n) p.y[r0 + lane] = tt;
            }
            __syncthreads();
        }
    };
    for (int it = blockIdx.x; it * SUBS < p.row_groups; it += gridDim.x) {
        const int r0 = (it * SUBS + sub) * R;
        uint4 ql[R];
        uint2 qh[R];
        uint16_t scw[R], db[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                p.q + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 2) + uload * 16u));
            ql[r] = make_uint4(t.x, t.y, t.z, t.w);
            qh[r] = *reinterpret_cast<const uint2*>(p.qh + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 4) +
                                                    uload * 8u);
            scw[r] = *reinterpret_cast<const uint16_t*>(p.sc + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 16) +
                                                        uload * 2u);
            db[r] = p.d[static_cast<uint64_t>(row) * nsb + sb];
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t w[4] = {ql[r].x, ql[r].y, ql[r].z, ql[r].w};
            const uint32_t hp[2] = {qh[r].x, qh[r].y};
            float plo = 0.f, phi = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t v = w[c], v8 = v >> 8;
                // the word's high-bit fields: in place for even c, rotated
                // right by 8 for odd c; elements 4c + 1 and 4c + 3 shifted
                // down by 2 together with their nibbles' shift of 8
                const uint32_t hc = (c & 1) ? __builtin_amdgcn_alignbit(hp[c >> 1], hp[c >> 1], 8) : hp[c >> 1];
                const uint32_t hc2 = hc >> 2;
                // low run: nibble at bits 0-3 of each 16-bit half, high bits at 4-5;
                // high run in place: nibble at bits 4-7, high bits at 8-9. The
                // nibble-and-exponent words pass through an opaque statement, so
                // each OR-in of high bits is one v_and_or_b32 (not and, and, or3)
                uint32_t n02 = (v & 0x000F000Fu) | magic, n13 = (v8 & 0x000F000Fu) | magic;
                uint32_t m02 = (v & 0x00F000F0u) | magic, m13 = (v8 & 0x00F000F0u) | magic;
                asm volatile("" : "+v"(n02), "+v"(n13), "+v"(m02), "+v"(m13));
                const half2_t lo02 = __builtin_bit_cast(half2_t, (hc & 0x00300030u) | n02) + off_lo;
                const half2_t lo13 = __builtin_bit_cast(half2_t, (hc2 & 0x00300030u) | n13) + off_lo;
                const half2_t hi02 = __builtin_bit_cast(half2_t, (hc & 0x03000300u) | m02) + off_hi;
                const half2_t hi13 = __builtin_bit_cast(half2_t, (hc2 & 0x03000300u) | m13) + off_hi;
                plo = fmaf(static_cast<float>(lo02.x), xr[4 * c + 0], plo);
                phi = fmaf(static_cast<float>(hi02.x), xr[16 + 4 * c + 0], phi);
                plo = fmaf(static_cast<float>(lo13.x), xr[4 * c + 1], plo);
                phi = fmaf(static_cast<float>(hi13.x), xr[16 + 4 * c + 1], phi);
                plo = fmaf(static_cast<float>(lo02.y), xr[4 * c + 2], plo);
                phi = fmaf(static_cast<float>(hi02.y), xr[16 + 4 * c + 2], phi);
                plo = fmaf(static_cast<float>(lo13.y), xr[4 * c + 3], plo);
                phi = fmaf(static_cast<float>(hi13.y), xr[16 + 4 * c + 3], phi);
            }
            uint32_t s01 = scw[r], dbits = db[r];
            asm volatile("" : "+v"(s01), "+v"(dbits));
            const float sl = static_cast<float>(static_cast<int8_t>(s01 & 0xFFu));
            const float sh = static_cast<float>(static_cast<int8_t>(s01 >> 8));
            const float dd = valid ? half_bits_to_float(static_cast<uint16_t>(dbits)) : 0.f;
            acc[r] = dd * fmaf(sh * 0.0625f, phi, sl * plo);
        }
        if constexpr (R == 4) {
            finish4(acc, r0);
            continue;
        }
        if constexpr (R == 2 && WS == 1) {
            // two rows: lanes 0 and 32 finish rows r0 and r0 + 1
            const float t = wave_sum2_rows(acc[0], acc[1 % R]);
            if ((lane & 31) == 0 && r0 + (lane >> 5) < p.n) p.y[r0 + (lane >> 5)] = t;
            continue;
        }
        // (other step sizes) the row sums are complete in lanes 48..63:
        // lane 64 - R + r stores row r
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum_last_row(acc[r]);
        if constexpr (WS == 1) {
            const int lr = lane - (kWave - R);
            if (lr >= 0) {
                float a = acc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = lr == r ? acc[r] : a;
                if (r0 + lr < p.n) p.y[r0 + lr] = a;
            }
        } else {
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r) lpart[wave][r] = acc[r];
            }
            __syncthreads();
            if (slice == 0 && lane < R) {
                float t = lpart[wave][lane];
#pragma unroll
                for (int s = 1; s < WS; ++s) t += lpart[wave + s][lane];
                if (r0 + lane < p.n) p.y[r0 + lane] = t;
            }
            __syncthreads();
        }
    }
}

// Compute units of the current device, queried once per device.
int kq_device_cus() {
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

template <int TYPE, int WS, int R>
hipError_t launch_ws(KqParams p, hipStream_t stream) {
    constexpr int WAVES = KqWaves<WS>::value;
    constexpr int SUBS = WAVES / WS;
    p.row_groups = (p.n + R - 1) / R;
    const auto kernel = TYPE == kTypeQ4_K ? qmv_q4_k_kernel<WS, R, false>
                        : (TYPE == kTypeQ5_K ? qmv_q4_k_kernel<WS, R, true> : qmv_q6_k_kernel<WS, R>);
    // resident workgroups (one query per kernel variant): the grid strides
    // over the row groups and never needs a second dispatch round
    static const int per_cu = [&] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, WAVES * kWave, 0) != hipSuccess || b < 1) b = 1;
        return b;
    }();
    const int64_t iters = (static_cast<int64_t>(p.row_groups) + SUBS - 1) / SUBS;
    int64_t cap = static_cast<int64_t>(per_cu) * kq_device_cus();
    const int64_t max_grid = static_cast<int64_t>(GQ_KQ_MAX_GRID) * 4 / WAVES;
    cap = cap < max_grid ? cap : max_grid;
    const int grid = static_cast<int>(iters < cap ? iters : cap);
    return launch_kernel(kernel, dim3(grid), dim3(WAVES * kWave), stream, p);
}

// The split of a row over ws waves (<= 16, k <= 32768), and for un-split
// short matrices GQ_KQ_R_SHORT rows per step.
template <int TYPE>
hipError_t launch_type(KqParams p, int ws, bool short_rows, hipStream_t stream) {
    if (ws <= 1) return short_rows ? launch_ws<TYPE, 1, GQ_KQ_R_SHORT>(p, stream) : launch_ws<TYPE, 1, GQ_KQ_R>(p, stream);
    if (ws <= 2) return launch_ws<TYPE, 2, GQ_KQ_R>(p, stream);
    if (ws <= 4) return launch_ws<TYPE, 4, GQ_KQ_R>(p, stream);
    if (ws <= 8) return launch_ws<TYPE, 8, GQ_KQ_R>(p, stream);
    if (ws <= 16) return launch_ws<TYPE, 16, GQ_KQ_R>(p, stream);
    return hipErrorInvalidValue;    // beyond the documented maximum k (32768)
}

}  // namespace

hipError_t launch_kq_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* packed,
                          hipStream_t stream) {
    size_t o[4];
    kq_layout(type, n, k, o);
    const int64_t nsb = n * (k / 256);
    const dim3 g(static_cast<unsigned>((nsb + kBlockThreads - 1) / kBlockThreads)), b(kBlockThreads);
    if (type == kTypeQ4_K) return launch_kernel(kq_pack_kernel<kTypeQ4_K>, g, b, stream, blocks, nsb, packed, o[1], o[2], o[3]);
    if (type == kTypeQ5_K) return launch_kernel(kq_pack_kernel<kTypeQ5_K>, g, b, stream, blocks, nsb, packed, o[1], o[2], o[3]);
    return launch_kernel(kq_pack_kernel<kTypeQ6_K>, g, b, stream, blocks, nsb, packed, o[1], o[2], o[3]);
}

hipError_t launch_qmv_kq(int type, const uint8_t* packed, int64_t n, int64_t k, const float* x, float* y,
                         hipStream_t stream) {
    size_t o[4];
    kq_layout(type, n, k, o);
    KqParams p{};
    p.q = packed;
    if (type == kTypeQ6_K) {
        p.qh = packed + o[1];
        p.sc = reinterpret_cast<const int8_t*>(packed + o[2]);
        p.d = reinterpret_cast<const uint16_t*>(packed + o[3]);
    } else {
        p.hdr = packed + o[1];
        if (type == kTypeQ5_K) p.fifth = reinterpret_cast<const uint32_t*>(packed + o[2]);
    }
    p.x = x;
    p.y = y;
    p.n = static_cast<int>(n);
    p.k = static_cast<int>(k);
    p.units = static_cast<int>(k / 32);
    const int ws = (p.units + kWave - 1) / kWave;          // waves a row is split over
    // un-split rows take GQ_KQ_R_SHORT rows per step when GQ_KQ_R would give
    // fewer row groups (one wave each) than the device has SIMDs
    const bool short_rows = (static_cast<int64_t>(p.n) + GQ_KQ_R - 1) / GQ_KQ_R < 4 * kq_device_cus();
    if (type == kTypeQ4_K) return launch_type<kTypeQ4_K>(p, ws, short_rows, stream);
    if (type == kTypeQ5_K) return launch_type<kTypeQ5_K>(p, ws, short_rows, stream);
    return launch_type<kTypeQ6_K>(p, ws, short_rows, stream);
}

}  // namespace gq
