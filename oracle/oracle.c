/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for GGUF Q8_0 / Q4_0
 * block-quantised weight x activation products, in fp64. Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may call it; the
 * library's compute path never does. It shares no code, header, table or
 * constant generator with the HIP library: it reads the canonical GGUF
 * block bytes (never the library's packed arrays) and decodes them itself.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (float arithmetic on x86-64 is SSE binary32 with FLT_EVAL_METHOD == 0, so
 * every `float` operation below is one IEEE-754 binary32 operation with
 * round-to-nearest-even).
 *
 * Sources ("page" = one of the web pages the method is taken from):
 *  - Gem native architecture page, "M4 Max operating assumptions": Q4_0 is a
 *    32-element, 18-byte block; Q8_0 is kept for embeddings.
 *  - jouleclaw-loader-gguf BENCHMARKS page, "Matmul throughput -- Q8_0 scalar
 *    vs NEON": Q8_0 weights against int8 activations with an int32 widening
 *    accumulate, the caller picking fp32 activations (quantised first) or
 *    pre-quantised ones.
 *  - SafeC Gemma 4 DESIGN_NOTES page, "Gated FFN" (down(gelu_tanh(gate x) *
 *    up x) and the tanh form of GELU) and "Math primitives" (y = x W^T with
 *    W stored [out][in] row-major).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - block byte layout: fp16 scale d first, then the quants (GGUF order);
 *  - Q4_0 nibble order: byte j of a block holds element j in its low nibble
 *    and element j+16 in its high nibble; value (q - 8) * d;
 *  - activation quantiser: per 32-element block, d = fp16(amax / 127) in
 *    fp32 then round-to-nearest-even to binary16; q = clamp(round-half-away(
 *    x / d), -127, 127) with the division in fp32 by the fp16-rounded scale;
 *    q = 0 when that scale is zero.  Inputs are assumed finite.
 *  - K-quant super-blocks (the jouleclaw-loader-gguf BENCHMARKS page gives
 *    only the arithmetic: "Q4_K matmul", 32-element sub-blocks with a scale
 *    and a minimum, w = d_sub * q - m_sub; "Q5_K + Q6_K matmul", Q6_K with
 *    two high bits per element and a signed -32 offset). The byte layout is
 *    the GGUF one, which the pages do not print: 256 elements per
 *    super-block.
 *      Q4_K, 144 bytes: binary16 d, binary16 dmin, 12 bytes holding eight
 *      6-bit sub-block scales sc_j and eight 6-bit minimums m_j, then 128
 *      bytes of 4-bit quants. For j < 4, sc_j and m_j are the low six bits of
 *      bytes j and j+4 of the 12; for j >= 4 their low four bits come from
 *      byte j+4 (low nibble for sc_j, high nibble for m_j) and their top two
 *      bits from the top two bits of byte j-4 (sc_j) and byte j (m_j). Quant
 *      byte 32g + l (g < 4, l < 32) holds element 64g + l in its low nibble
 *      and element 64g + 32 + l in its high nibble. Element e belongs to
 *      sub-block e / 32 and is d sc_j q_e - dmin m_j.
 *      Q5_K, 176 bytes: binary16 d, binary16 dmin, the same 12 scale and
 *      minimum bytes as Q4_K, 32 bytes qh, then 128 quant bytes laid out as
 *      Q4_K's (low four bits). The fifth bit of element 64g + l (l < 32) is
 *      bit 2g of qh byte l, that of element 64g + 32 + l bit 2g + 1. Element
 *      e belongs to sub-block e / 32 and is d sc_j q_e - dmin m_j, with q_e
 *      in 0..31 (the page's "one high bit per element").
 *      Q6_K, 210 bytes: 128 bytes ql (low four bits), 64 bytes qh (high two
 *      bits), 16 int8 scales, binary16 d. In half h (elements 128h ..
 *      128h + 127; ql bytes 64h.., qh bytes 32h..), for l < 32: ql byte l
 *      gives the low bits of elements l (low nibble) and l + 64 (high
 *      nibble), ql byte l + 32 those of elements l + 32 and l + 96, and qh
 *      byte l the high bits of elements l, l + 32, l + 64, l + 96 in its bit
 *      pairs 0-1, 2-3, 4-5, 6-7 (element numbers relative to the half).
 *      Element e uses scale e / 16 and is d sc (q_e - 32).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <float.h>

#if FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 float evaluation (FLT_EVAL_METHOD == 0)"
#endif

#define OR_QK 32
#define OR_QK_K 256
#define OR_TYPE_Q4_0 2
#define OR_TYPE_Q8_0 8
#define OR_TYPE_Q4_K 12
#define OR_TYPE_Q5_K 13
#define OR_TYPE_Q6_K 14

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> wider types, written out bit by bit.                */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> the exact fp64 value (subnormals, +-0, inf, NaN). */
double or_fp16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal or zero */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* fp32 -> binary16 bits, round to nearest, ties to even. The fp32 value is
 * exact in fp64, so scaling by powers of two and nearbyint() (default
 * rounding mode: nearest-even) give the correctly rounded half. */
uint16_t or_f32_to_fp16_rne(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);
    if (a >= 65520.0)              /* at or past the midpoint above 65504 */
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {             /* subnormal range: multiples of 2^-24 */
        double q = nearbyint(a * 0x1p24);          /* 0..1024; 1024 = min normal */
        return (uint16_t)(sign | (uint16_t)q);
    }
    int E;
    (void)frexp(a, &E);            /* a in [2^(E-1), 2^E) */
    int e = E - 1;
    double s = nearbyint(ldexp(a, 10 - e));        /* in [1024, 2048] */
    if (s == 2048.0) {
        s = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(((e + 15) << 10) | ((int)s - 1024)));
}

/* ------------------------------------------------------------------------ */
/* Block decode.                                                             */
/* ------------------------------------------------------------------------ */

size_t or_block_bytes(int type)
{
    if (type == OR_TYPE_Q8_0) return 34;
    if (type == OR_TYPE_Q4_0) return 18;
    if (type == OR_TYPE_Q4_K) return 144;
    if (type == OR_TYPE_Q5_K) return 176;
    if (type == OR_TYPE_Q6_K) return 210;
    return 0;
}

/* Elements per block: 32, or 256 for the K-quant super-blocks. */
int64_t or_block_elems(int type)
{
    return (type == OR_TYPE_Q4_K || type == OR_TYPE_Q5_K || type == OR_TYPE_Q6_K) ? OR_QK_K : OR_QK;
}

static int is_kquant(int type)
{
    return type == OR_TYPE_Q4_K || type == OR_TYPE_Q5_K || type == OR_TYPE_Q6_K;
}

/* The 6-bit scale and minimum of Q4_K sub-block j from the 12 packed bytes. */
static void q4_k_scale_min(const uint8_t *s12, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s12[j] & 63;
        *m = s12[j + 4] & 63;
    } else {
        *sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
        *m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
    }
}

/* The 256 dequantised values of one K-quant super-block, in fp64. */
static void kblock_values(int type, const uint8_t *blk, double w[OR_QK_K])
{
    if (type == OR_TYPE_Q4_K) {
        double d = or_fp16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        double dmin = or_fp16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
        const uint8_t *s12 = blk + 4, *qs = blk + 16;
        int q[OR_QK_K];
        for (int g = 0; g < 4; ++g)
            for (int l = 0; l < 32; ++l) {
                q[64 * g + l] = qs[32 * g + l] & 15;
                q[64 * g + 32 + l] = qs[32 * g + l] >> 4;
            }
        for (int e = 0; e < OR_QK_K; ++e) {
            int sc, m;
            q4_k_scale_min(s12, e / 32, &sc, &m);
            w[e] = d * (double)sc * (double)q[e] - dmin * (double)m;
        }
    } else if (type == OR_TYPE_Q5_K) {
        double d = or_fp16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        double dmin = or_fp16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
        const uint8_t *s12 = blk + 4, *qh = blk + 16, *qs = blk + 48;
        int q[OR_QK_K];
        for (int g = 0; g < 4; ++g)
            for (int l = 0; l < 32; ++l) {
                q[64 * g + l] = (qs[32 * g + l] & 15) | (((qh[l] >> (2 * g)) & 1) << 4);
                q[64 * g + 32 + l] = (qs[32 * g + l] >> 4) | (((qh[l] >> (2 * g + 1)) & 1) << 4);
            }
        for (int e = 0; e < OR_QK_K; ++e) {
            int sc, m;
            q4_k_scale_min(s12, e / 32, &sc, &m);
            w[e] = d * (double)sc * (double)q[e] - dmin * (double)m;
        }
    } else {
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        double d = or_fp16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
        int q[OR_QK_K];
        for (int h = 0; h < 2; ++h)
            for (int l = 0; l < 32; ++l) {
                const uint8_t *L = ql + 64 * h, *H = qh + 32 * h;
                int *Q = q + 128 * h;
                Q[l] = (L[l] & 15) | (((H[l] >> 0) & 3) << 4);
                Q[l + 32] = (L[l + 32] & 15) | (((H[l] >> 2) & 3) << 4);
                Q[l + 64] = (L[l] >> 4) | (((H[l] >> 4) & 3) << 4);
                Q[l + 96] = (L[l + 32] >> 4) | (((H[l] >> 6) & 3) << 4);
            }
        for (int e = 0; e < OR_QK_K; ++e)
            w[e] = d * (double)sc[e / 16] * (double)(q[e] - 32);
    }
}

/* Integer quant values of one block: Q8_0 q_i, Q4_0 (nibble_i - 8). */
static void block_ints(int type, const uint8_t *blk, int q[OR_QK])
{
    if (type == OR_TYPE_Q8_0) {
        for (int i = 0; i < OR_QK; ++i)
            q[i] = (int)(int8_t)blk[2 + i];
    } else {
        for (int j = 0; j < 16; ++j) {
            q[j] = (int)(blk[2 + j] & 0x0F) - 8;
            q[j + 16] = (int)(blk[2 + j] >> 4) - 8;
        }
    }
}

static double block_scale(const uint8_t *blk)
{
    return or_fp16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Dequantise rows [0, n) of a [n][k/32] block matrix into w[n][k] (fp64,
 * exact: an 11-bit scale times an integer of at most 8 bits). */
int or_dequantize(int type, const uint8_t *blocks, int64_t n, int64_t k, double *w)
{
    size_t bb = or_block_bytes(type);
    if (!bb || k <= 0 || k % or_block_elems(type) || n < 0) return 1;
    if (is_kquant(type)) {
        int64_t nsb = k / OR_QK_K;
        for (int64_t r = 0; r < n; ++r)
            for (int64_t b = 0; b < nsb; ++b)
                kblock_values(type, blocks + (size_t)(r * nsb + b) * bb, w + r * k + b * OR_QK_K);
        return 0;
    }
    int64_t nb = k / OR_QK;
    int q[OR_QK];
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (size_t)(r * nb + b) * bb;
            double d = block_scale(blk);
            block_ints(type, blk, q);
            for (int i = 0; i < OR_QK; ++i)
                w[r * k + b * OR_QK + i] = d * (double)q[i];
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* y = W x with fp64 activations (fp32 inputs widen exactly).                */
/* y[r] = sum_k w[r][k] x[k], k ascending; a[r] = sum_k |w[r][k] x[k]|.      */
/* ------------------------------------------------------------------------ */
int or_matvec(int type, const uint8_t *blocks, int64_t n, int64_t k,
              const double *x, double *y, double *a)
{
    size_t bb = or_block_bytes(type);
    if (!bb || k <= 0 || k % or_block_elems(type) || n < 0) return 1;
    if (is_kquant(type)) {
        int64_t nsb = k / OR_QK_K;
        double w[OR_QK_K];
        for (int64_t r = 0; r < n; ++r) {
            double sum = 0.0, asum = 0.0;
            for (int64_t b = 0; b < nsb; ++b) {
                kblock_values(type, blocks + (size_t)(r * nsb + b) * bb, w);
                for (int i = 0; i < OR_QK_K; ++i) {
                    double p = w[i] * x[b * OR_QK_K + i];
                    sum += p;
                    asum += fabs(p);
                }
            }
            y[r] = sum;
            if (a) a[r] = asum;
        }
        return 0;
    }
    int64_t nb = k / OR_QK;
    int q[OR_QK];
    for (int64_t r = 0; r < n; ++r) {
        double sum = 0.0, asum = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (size_t)(r * nb + b) * bb;
            double d = block_scale(blk);
            block_ints(type, blk, q);
            for (int i = 0; i < OR_QK; ++i) {
                double p = (d * (double)q[i]) * x[b * OR_QK + i];
                sum += p;
                asum += fabs(p);
            }
        }
        y[r] = sum;
        if (a) a[r] = asum;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Q8_0 activation quantiser (an encoding, spelled out step by step).        */
/* x [m][k] fp32 -> xq [m][k] int8, xd [m][k/32] binary16 bits.               */
/* ------------------------------------------------------------------------ */
int or_quantize_q8_0(const float *x, int64_t m, int64_t k, int8_t *xq, uint16_t *xd)
{
    if (k <= 0 || k % OR_QK || m < 0) return 1;
    int64_t nb = k / OR_QK;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * k + b * OR_QK;
            int8_t *qb = xq + r * k + b * OR_QK;
            float amax = 0.0f;                       /* 1: block absolute max */
            for (int i = 0; i < OR_QK; ++i) {
                float v = fabsf(xb[i]);
                if (v > amax) amax = v;
            }
            float d32 = amax / 127.0f;               /* 2: fp32 divide */
            uint16_t h = or_f32_to_fp16_rne(d32);    /* 3: round to binary16 */
            float d16 = (float)or_fp16_to_f64(h);    /*    (exact in fp32) */
            xd[r * nb + b] = h;
            for (int i = 0; i < OR_QK; ++i) {        /* 4: codes */
                int qi = 0;
                if (d16 != 0.0f) {
                    float v = xb[i] / d16;           /* fp32 divide */
                    float rv = roundf(v);            /* half away from zero */
                    if (rv > 127.0f) rv = 127.0f;
                    if (rv < -127.0f) rv = -127.0f;
                    qi = (int)rv;
                }
                qb[i] = (int8_t)qi;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Integer path: weights x Q8_0 activation rows.                              */
/* S[mi][r][b] = sum_i qw[r][b][i] * qx[mi][b][i] exactly (int64, checked to  */
/* fit int32); y[mi][r] = sum_b dw[r][b] dx[mi][b] S (fp64);                  */
/* a[mi][r] = sum_b |dw dx| sum_i |qw qx|.  S, y, a may each be NULL.         */
/* Returns 2 if some S does not fit int32.                                    */
/* ------------------------------------------------------------------------ */
int or_blockdots(int type, const uint8_t *blocks, int64_t n, int64_t k,
                 const int8_t *xq, const uint16_t *xd, int64_t m,
                 int32_t *S, double *y, double *a)
{
    size_t bb = or_block_bytes(type);
    if (!bb || is_kquant(type) || k <= 0 || k % OR_QK || n < 0 || m < 0) return 1;
    int64_t nb = k / OR_QK;
    int q[OR_QK];
    int rc = 0;
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t r = 0; r < n; ++r) {
            double sum = 0.0, asum = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *blk = blocks + (size_t)(r * nb + b) * bb;
                const int8_t *qx = xq + mi * k + b * OR_QK;
                block_ints(type, blk, q);
                int64_t s = 0, sa = 0;
                for (int i = 0; i < OR_QK; ++i) {
                    int64_t p = (int64_t)q[i] * (int64_t)qx[i];
                    s += p;
                    sa += p < 0 ? -p : p;
                }
                if (s > INT32_MAX || s < INT32_MIN) rc = 2;
                double scale = block_scale(blk) * or_fp16_to_f64(xd[mi * nb + b]);
                sum += scale * (double)s;
                asum += fabs(scale) * (double)sa;
                if (S) S[(mi * n + r) * nb + b] = (int32_t)s;
            }
            if (y) y[mi * n + r] = sum;
            if (a) a[mi * n + r] = asum;
        }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* GELU, tanh form (SafeC DESIGN_NOTES page, "Gated FFN"):                    */
/* G(t) = 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))); libm tanh          */
/* saturates to +-1, so finite t gives a finite result.                       */
/* ------------------------------------------------------------------------ */
double or_gelu_tanh(double t)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * t * (1.0 + tanh(c * (t + 0.044715 * t * t * t)));
}

/* Gate/up half of the gated FFN: g = Wg x, u = Wu x (both [n_ff][k]),
 * h = G(g) * u. ag/au are the sum |w x| of each row (may be NULL). */
int or_ffn_gate_up(int type, const uint8_t *gblocks, const uint8_t *ublocks,
                   int64_t n_ff, int64_t k, const double *x,
                   double *g, double *u, double *h, double *ag, double *au)
{
    int rc = or_matvec(type, gblocks, n_ff, k, x, g, ag);
    if (rc) return rc;
    rc = or_matvec(type, ublocks, n_ff, k, x, u, au);
    if (rc) return rc;
    for (int64_t r = 0; r < n_ff; ++r)
        h[r] = or_gelu_tanh(g[r]) * u[r];
    return 0;
}

/* Sampled rows: y[i] = row rows[i] of W times x, for spot checks at sizes
 * where the full product would take too long. */
int or_matvec_rows(int type, const uint8_t *blocks, int64_t n, int64_t k,
                   const int64_t *rows, int64_t nrows, const double *x,
                   double *y, double *a)
{
    size_t bb = or_block_bytes(type);
    if (!bb || k <= 0 || k % or_block_elems(type)) return 1;
    int64_t nb = k / or_block_elems(type);
    for (int64_t i = 0; i < nrows; ++i) {
        if (rows[i] < 0 || rows[i] >= n) return 1;
        const uint8_t *row = blocks + (size_t)(rows[i] * nb) * bb;
        int rc = or_matvec(type, row, 1, k, x, y + i, a ? a + i : NULL);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm (SafeC Gemma 4 DESIGN_NOTES page, "RMSNorm"): out_i = x_i *        */
/* (mean_j x_j^2 + eps)^(-1/2) * w_i, the weight applied directly (no +1);    */
/* w == NULL means w_i = 1. Gemma 4 uses eps = 1e-6 ("Hyperparameters").      */
/* ------------------------------------------------------------------------ */
int or_rmsnorm(const double *x, int64_t k, const double *w, double eps, double *out)
{
    if (k <= 0) return 1;
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)k + eps);
    for (int64_t i = 0; i < k; ++i)
        out[i] = x[i] * inv * (w ? w[i] : 1.0);
    return 0;
}

/* Final-logit soft cap (SafeC DESIGN_NOTES page, "LM head"):                 */
/* cap * tanh(y / cap) for cap > 0; y unchanged for cap == 0.                 */
double or_softcap(double y, double cap)
{
    return cap > 0.0 ? cap * tanh(y / cap) : y;
}

/* Greedy argmax over fp32 values: the largest value wins, ties go to the     */
/* lowest index, NaN ranks below every number (so it wins only if all are     */
/* NaN, and then index 0). Returns the index; n >= 1.                         */
int64_t or_argmax_f32(const float *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i) {
        if (isnan(v[i])) continue;
        if (isnan(v[best]) || v[i] > v[best]) best = i;
    }
    return best;
}
