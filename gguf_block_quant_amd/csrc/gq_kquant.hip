// gq_kquant.hip -- M = 1 decode matvec over K-quant super-blocks (Q4_K and
// Q6_K, 256 elements each) with fp32 activations, and their load-time pack.
//
// What is computed follows the jouleclaw-loader-gguf BENCHMARKS page: "Q4_K
// matmul" works on 32-element sub-blocks, each with a scale and a minimum,
// w = d_sub q - m_sub, and splits the sum as d_sub sum(a q) - m_sub sum(a);
// "Q5_K + Q6_K matmul" takes two high bits per element and a signed -32
// offset for Q6_K. The super-block byte layout (not printed on the pages) is
// the GGUF one:
//   Q4_K (144 B): binary16 d, binary16 dmin, 12 bytes of packed 6-bit
//     sub-block scales sc_j and minimums m_j, 128 quant bytes; quant byte
//     32g + l holds element 64g + l (low nibble) and 64g + 32 + l (high);
//     element e of sub-block j = e / 32 is d sc_j q - dmin m_j.
//   Q6_K (210 B): ql[128] (low four bits), qh[64] (high two bits), int8
//     scales[16], binary16 d; element e is d scales[e / 16] (q - 32).
//
// Packed layout (gq_kq_pack; byte moves only, sections 256-byte aligned):
//   Q4_K: qs [n][k/2] (the quant bytes of each super-block in order), then
//         hdr [n][k/256][16] (d, dmin and the 12 scale bytes).
//   Q6_K: ql [n][k/2], qh [n][k/4], sc [n][k/16] int8, d [n][k/256] binary16.
// A row's quants are then contiguous 16-byte units, one per lane: a wave
// instruction reads 1 KiB of one row, as for Q4_0.
//
// Decomposition: lane l of a wave owns unit l of its slice of the row (16
// bytes = 32 elements, in two runs of 16 that share a sub-block scale each:
//   Q4_K unit u of a super-block: runs 64(u/2) + 16(u%2) (low nibbles,
//     sub-block u & 6) and that + 32 (high nibbles, sub-block (u & 6) + 1);
//   Q6_K unit 4h + j: runs 128h + 16j (scale 8h + j) and that + 64 (scale
//     8h + j + 4), the high bits from qh bytes 32h + 16(j % 2) ..).
// The lane's 32 activations stay in VGPRs for every row it streams. Rows
// longer than 2048 elements are split over WS waves whose partial sums meet
// in LDS in slice order; waves stream R rows per step; sums over lanes use
// DPP (wave_sum), fixed order, no atomics.
#include <atomic>

#include "gq_device.hpp"
#include "gq_launch.hpp"

// Measured on MI355X (fp32 x, k = 2048; 262144 / 8192 rows, and 2048 x 8192):
// 4 rows per step with up to 2048 workgroups: Q4_K 62-64 / 5.3-5.4 / 5.6 us,
// Q6_K 84-88 / 6.0-6.1 / 5.7-5.8 us; 2 rows at 1024 workgroups: 73 / 5.7 /
// 5.8 and 92 / 6.6 / 6.9 us. Two row groups in flight per wave (a second
// register set) measured no better: the loop is bound by its VALU work
// (about 2.1 instructions per element for the exact nibble dot), not by
// load latency.
#ifndef GQ_KQ_R
#define GQ_KQ_R 4            // rows per wave step
#endif
#ifndef GQ_KQ_MAX_GRID
#define GQ_KQ_MAX_GRID 2048  // workgroups of 4 waves at most
#endif

namespace gq {

namespace {

constexpr int kTypeQ4_K = 12;
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

// ---------------------------------------------------------------------------
// Pack: one thread per super-block; byte loads (a GGUF block is only
// 2-byte aligned at best), 16-byte stores into the aligned sections.
// ---------------------------------------------------------------------------
template <int TYPE>
__global__ __launch_bounds__(kBlockThreads)
void kq_pack_kernel(const uint8_t* __restrict__ blocks, int64_t nsb_total, uint8_t* __restrict__ out,
                    size_t o1, size_t o2, size_t o3) {
    constexpr int BB = TYPE == kTypeQ4_K ? 144 : 210;
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
    if constexpr (TYPE == kTypeQ4_K) {
        uint8_t* qs = out + i * 128;
#pragma unroll
        for (int c = 0; c < 8; ++c) copy16(16 + 16 * c, qs + 16 * c);
        copy16(0, out + o1 + i * 16);                       // d, dmin, 12 scale bytes
    } else {
        uint8_t* ql = out + i * 128;
#pragma unroll
        for (int c = 0; c < 8; ++c) copy16(16 * c, ql + 16 * c);
        uint8_t* qh = out + o1 + i * 64;
#pragma unroll
        for (int c = 0; c < 4; ++c) copy16(128 + 16 * c, qh + 16 * c);
        copy16(192, out + o2 + i * 16);                     // 16 int8 scales
        *reinterpret_cast<uint16_t*>(out + o3 + i * 2) =
            static_cast<uint16_t>(src[208] | (src[209] << 8));
    }
}

struct KqParams {
    const uint8_t* q;       // quant bytes [n][k/2] (Q4_K qs, Q6_K ql)
    const uint8_t* hdr;     // Q4_K: [n][k/256][16] headers
    const uint8_t* qh;      // Q6_K: [n][k/4]
    const int8_t* sc;       // Q6_K: [n][k/16]
    const uint16_t* d;      // Q6_K: [n][k/256]
    const float* x;         // [k]
    float* y;               // [n]
    int n;
    int k;
    int units;              // 16-byte quant units per row (k / 32)
    int row_groups;         // ceil(n / R)
};

// Waves per workgroup: 4, or WS when a row is split over more waves.
template <int WS> struct KqWaves { static constexpr int value = WS < 4 ? 4 : WS; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Exact dequantisation of two 4-bit fields of a 32-bit word, held in the
// low bits of its 16-bit halves (mask selects them), through the binary16
// number 1024 + v built by OR-ing them under the exponent pattern in `magic`,
// then one packed add of `off` (exact: every value involved is an integer
// below 2048).
__device__ __forceinline__ half2_t nib2(uint32_t w, uint32_t mask, uint32_t magic, half2_t off) {
    return __builtin_bit_cast(half2_t, (w & mask) | magic) + off;
}

template <int WS, int R>
__global__ __launch_bounds__(KqWaves<WS>::value * kWave)
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
    // which bytes of the 12 hold this lane's two sub-blocks (a = u & 6, b = a + 1)
    const uint32_t jsh = 8u * (u & 2u);            // byte (a & 3) of a scale word
    const bool hi_sub = (u & 4u) != 0;             // sub-blocks 4..7: the split 6-bit encoding

    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));
    const half2_t off_lo = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};

    __shared__ float lpart[WAVES][R];
    for (int it = blockIdx.x; it * SUBS < p.row_groups; it += gridDim.x) {
        const int r0 = (it * SUBS + sub) * R;
        uint4 q[R], h[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                p.q + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 2) + uload * 16u));
            q[r] = make_uint4(t.x, t.y, t.z, t.w);
            h[r] = *reinterpret_cast<const uint4*>(p.hdr + (static_cast<uint64_t>(row) * nsb + sb) * 16u);
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t w[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
            float pa = 0.f, pb = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t v = w[j], v8 = v >> 8;
                const half2_t lo02 = nib2(v, 0x000F000Fu, magic, off_lo);
                const half2_t lo13 = nib2(v8, 0x000F000Fu, magic, off_lo);
                const half2_t hi02 = nib2(v, 0x00F000F0u, magic, off_lo);     // 16 q
                const half2_t hi13 = nib2(v8, 0x00F000F0u, magic, off_lo);
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
            // the two sub-blocks' 6-bit scales and minimums, side by side in
            // the low two bytes of SC and MN
            uint32_t hx = h[r].x, hy = h[r].y, hz = h[r].z, hw = h[r].w;
            asm volatile("" : "+v"(hx), "+v"(hy), "+v"(hz), "+v"(hw));
            const uint32_t Y = hy >> jsh, Z = hz >> jsh, W = hw >> jsh;
            const uint32_t SC = hi_sub ? ((W & 0x0F0Fu) | ((Y >> 2) & 0x3030u)) : (Y & 0x3F3Fu);
            const uint32_t MN = hi_sub ? (((W >> 4) & 0x0F0Fu) | ((Z >> 2) & 0x3030u)) : (Z & 0x3F3Fu);
            const float sca = static_cast<float>(SC & 0xFFu), scb = static_cast<float>((SC >> 8) & 0xFFu);
            const float mna = static_cast<float>(MN & 0xFFu), mnb = static_cast<float>((MN >> 8) & 0xFFu);
            const float dd = valid ? half_bits_to_float(static_cast<uint16_t>(hx & 0xFFFFu)) : 0.f;
            const float dm = valid ? half_bits_to_float(static_cast<uint16_t>(hx >> 16)) : 0.f;
            const float t1 = fmaf(scb, pb, sca * pa);
            const float t2 = fmaf(mnb, sxb, mna * sxa);
            acc[r] = fmaf(dd, t1, -(dm * t2));
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
        if constexpr (WS == 1) {
            if (lane < R) {
                float a = acc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = lane == r ? acc[r] : a;
                if (r0 + lane < p.n) p.y[r0 + lane] = a;
            }
        } else {
            if (lane == 0) {
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

template <int WS, int R>
__global__ __launch_bounds__(KqWaves<WS>::value * kWave)
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
    const uint32_t sh_lo = 2u * (j >> 1);          // bit pair of qh for the low run
    const uint32_t sh_hi = 4u + sh_lo;             // ... and for the high run
    const uint32_t ssh = 8u * j;                   // byte of the scale words

    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));
    // low run: 1024 + q - 1056 = q - 32; high run (in place): 1024 + 16 q - 1536 = 16 (q - 32)
    const half2_t off_lo = {static_cast<_Float16>(-1056.0f), static_cast<_Float16>(-1056.0f)};
    const half2_t off_hi = {static_cast<_Float16>(-1536.0f), static_cast<_Float16>(-1536.0f)};

    __shared__ float lpart[WAVES][R];
    for (int it = blockIdx.x; it * SUBS < p.row_groups; it += gridDim.x) {
        const int r0 = (it * SUBS + sub) * R;
        uint4 ql[R], qh[R];
        uint2 scw[R];
        uint16_t db[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t row = static_cast<uint32_t>(min(r0 + r, p.n - 1));
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                p.q + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 2) + uload * 16u));
            ql[r] = make_uint4(t.x, t.y, t.z, t.w);
            qh[r] = *reinterpret_cast<const uint4*>(p.qh + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 4) +
                                                    sb * 64u + hh * 32u + (j & 1u) * 16u);
            scw[r] = *reinterpret_cast<const uint2*>(p.sc + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.k / 16) +
                                                     sb * 16u + hh * 8u);
            db[r] = p.d[static_cast<uint64_t>(row) * nsb + sb];
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t w[4] = {ql[r].x, ql[r].y, ql[r].z, ql[r].w};
            const uint32_t b[4] = {qh[r].x, qh[r].y, qh[r].z, qh[r].w};
            float plo = 0.f, phi = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t v = w[c], v8 = v >> 8;
                const uint32_t bl = b[c] >> sh_lo, bh = b[c] >> sh_hi;
                // low run: nibble at bits 0-3 of each 16-bit half, high bits to 4-5
                const half2_t lo02 = __builtin_bit_cast(half2_t, ((v & 0x000F000Fu) | magic) |
                                                                     ((bl << 4) & 0x00300030u)) + off_lo;
                const half2_t lo13 = __builtin_bit_cast(half2_t, ((v8 & 0x000F000Fu) | magic) |
                                                                     ((bl >> 4) & 0x00300030u)) + off_lo;
                // high run in place: nibble at bits 4-7, high bits to 8-9
                const half2_t hi02 = __builtin_bit_cast(half2_t, ((v & 0x00F000F0u) | magic) |
                                                                     ((bh << 8) & 0x03000300u)) + off_hi;
                const half2_t hi13 = __builtin_bit_cast(half2_t, ((v8 & 0x00F000F0u) | magic) |
                                                                     (bh & 0x03000300u)) + off_hi;
                plo = fmaf(static_cast<float>(lo02.x), xr[4 * c + 0], plo);
                phi = fmaf(static_cast<float>(hi02.x), xr[16 + 4 * c + 0], phi);
                plo = fmaf(static_cast<float>(lo13.x), xr[4 * c + 1], plo);
                phi = fmaf(static_cast<float>(hi13.x), xr[16 + 4 * c + 1], phi);
                plo = fmaf(static_cast<float>(lo02.y), xr[4 * c + 2], plo);
                phi = fmaf(static_cast<float>(hi02.y), xr[16 + 4 * c + 2], phi);
                plo = fmaf(static_cast<float>(lo13.y), xr[4 * c + 3], plo);
                phi = fmaf(static_cast<float>(hi13.y), xr[16 + 4 * c + 3], phi);
            }
            uint32_t s0 = scw[r].x, s1 = scw[r].y, dbits = db[r];
            asm volatile("" : "+v"(s0), "+v"(s1), "+v"(dbits));
            const float sl = static_cast<float>(static_cast<int8_t>(s0 >> ssh));
            const float sh = static_cast<float>(static_cast<int8_t>(s1 >> ssh));
            const float dd = valid ? half_bits_to_float(static_cast<uint16_t>(dbits)) : 0.f;
            acc[r] = dd * fmaf(sh * 0.0625f, phi, sl * plo);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
        if constexpr (WS == 1) {
            if (lane < R) {
                float a = acc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = lane == r ? acc[r] : a;
                if (r0 + lane < p.n) p.y[r0 + lane] = a;
            }
        } else {
            if (lane == 0) {
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

template <int TYPE, int WS>
hipError_t launch_ws(KqParams p, hipStream_t stream) {
    constexpr int R = GQ_KQ_R;
    constexpr int WAVES = KqWaves<WS>::value;
    constexpr int SUBS = WAVES / WS;
    p.row_groups = (p.n + R - 1) / R;
    const auto kernel = TYPE == kTypeQ4_K ? qmv_q4_k_kernel<WS, R> : qmv_q6_k_kernel<WS, R>;
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

}  // namespace

hipError_t launch_kq_pack(int type, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* packed,
                          hipStream_t stream) {
    size_t o[4];
    kq_layout(type, n, k, o);
    const int64_t nsb = n * (k / 256);
    const dim3 g(static_cast<unsigned>((nsb + kBlockThreads - 1) / kBlockThreads)), b(kBlockThreads);
    if (type == kTypeQ4_K) return launch_kernel(kq_pack_kernel<kTypeQ4_K>, g, b, stream, blocks, nsb, packed, o[1], o[2], o[3]);
    return launch_kernel(kq_pack_kernel<kTypeQ6_K>, g, b, stream, blocks, nsb, packed, o[1], o[2], o[3]);
}

hipError_t launch_qmv_kq(int type, const uint8_t* packed, int64_t n, int64_t k, const float* x, float* y,
                         hipStream_t stream) {
    size_t o[4];
    kq_layout(type, n, k, o);
    KqParams p{};
    p.q = packed;
    p.hdr = packed + o[1];
    p.qh = packed + o[1];
    p.sc = reinterpret_cast<const int8_t*>(packed + o[2]);
    p.d = reinterpret_cast<const uint16_t*>(packed + o[3]);
    p.x = x;
    p.y = y;
    p.n = static_cast<int>(n);
    p.k = static_cast<int>(k);
    p.units = static_cast<int>(k / 32);
    const int ws = (p.units + kWave - 1) / kWave;          // waves a row is split over
    if (type == kTypeQ4_K) {
        if (ws <= 1) return launch_ws<kTypeQ4_K, 1>(p, stream);
        if (ws <= 2) return launch_ws<kTypeQ4_K, 2>(p, stream);
        if (ws <= 4) return launch_ws<kTypeQ4_K, 4>(p, stream);
        if (ws <= 8) return launch_ws<kTypeQ4_K, 8>(p, stream);
        if (ws <= 16) return launch_ws<kTypeQ4_K, 16>(p, stream);
    } else {
        if (ws <= 1) return launch_ws<kTypeQ6_K, 1>(p, stream);
        if (ws <= 2) return launch_ws<kTypeQ6_K, 2>(p, stream);
        if (ws <= 4) return launch_ws<kTypeQ6_K, 4>(p, stream);
        if (ws <= 8) return launch_ws<kTypeQ6_K, 8>(p, stream);
        if (ws <= 16) return launch_ws<kTypeQ6_K, 16>(p, stream);
    }
    return hipErrorInvalidValue;    // beyond the documented maximum k (32768)
}

}  // namespace gq
