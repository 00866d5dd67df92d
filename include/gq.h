/*
 * gq.h -- C ABI of libgq: GGUF Q8_0 / Q4_0 block-quantised weight x
 * activation products on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *  - every decode-step projection is a matrix-vector product against
 *    block-quantised weights, and decode is bound by the weight stream
 *    (Gemma-4-E2B raw-Metal port page, "Why this exists (the byte floor ...)";
 *    TensorSharp Gemma 4 page, batched decode section);
 *  - the projection contract is y = W x with W stored [out][in] row-major,
 *    without materialising W^T (SafeC Gemma 4 DESIGN_NOTES page,
 *    "Math primitives implementation status");
 *  - Q4_0 is a 32-element, 18-byte block, Q8_0 is kept as the 8-bit
 *    option (Gem native architecture page, "M4 Max operating assumptions");
 *  - the caller picks an fp32-activation entry or a pre-quantised int8 one
 *    (jouleclaw-loader-gguf BENCHMARKS page, "Matmul throughput -- Q8_0
 *    scalar vs NEON" and "Q8_0 matmul -- NEON direct vs AMX-tiled");
 *  - the gated FFN is down(gelu_tanh(gate x) * up x) (SafeC DESIGN_NOTES,
 *    "Gated FFN"); gate+up fused in one pass (raw-Metal port page,
 *    "Architecture", kernels bullet);
 *  - prompt evaluation runs small-M tiles of up to 32 rows through each
 *    projection (Gem native architecture page, "Ownership boundaries",
 *    Metal/profiling bullets; raw-Metal port page, "Batched prefill").
 *
 * Formats (GGUF, little-endian):
 *  - Q8_0 block, 34 B: binary16 scale d, then int8 q[32]; w_i = d * q_i.
 *  - Q4_0 block, 18 B: binary16 scale d, then 16 bytes; byte j holds
 *    element j in its low nibble and element j+16 in its high nibble;
 *    w_i = d * (nibble_i - 8).
 *  A weight matrix of n rows and k columns is n * k/32 blocks, row-major,
 *  blocks along k.
 *
 * Packed layout (what every compute entry point reads; produced by gq_pack):
 *  - qs: Q8_0 int8 [n][k] (row-major quants); Q4_0 uint8 [n][k/2] (the 16
 *        quant bytes of each block, in GGUF in-block order, blocks along k);
 *  - d : binary16 bits uint16 [n][k/32] (the block scales, row-major).
 *  The pack only moves bytes: the same count as the GGUF blocks, split so
 *  that every 16-byte quant chunk is 16-byte aligned.
 *
 * Conventions for every entry point:
 *  - Pointers named qs, d, x, y, h, xq, xd, blockdots and blocks are DEVICE
 *    pointers on the current HIP device. The caller allocates and frees all
 *    of them; libgq never allocates device memory, frees or synchronises.
 *  - Inputs are read-only. Outputs are fully overwritten.
 *  - stream is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously on that stream.
 *  - Shapes: n >= 1, k >= 32, k % 32 == 0, else GQ_ERR_SHAPE. Each entry
 *    point documents its maximum k (GQ_ERR_UNSUPPORTED beyond it); n (and
 *    m of gq_quantize_q8_0) is limited to 2^30 rows (GQ_ERR_UNSUPPORTED
 *    beyond it).
 *  - Alignment: qs, x, h and xq 16 bytes; d and xd 2 bytes; y and blockdots
 *    4 bytes; else GQ_ERR_ALIGN.
 *  - An output range overlapping any input range gives GQ_ERR_ALIAS.
 *  - Special values: every binary16 scale bit pattern is accepted; +-0 and
 *    subnormal scales are decoded exactly. A row with a non-finite weight
 *    scale (+-Inf, NaN) in any block gets a non-finite output, as the plain
 *    definition sum_c w[r][c] x[c] does (NaN or +-Inf; which of the two is
 *    not specified: the kernels factor the block scale out of its 32
 *    products). Non-finite activations propagate the same way.
 *  - All validation is synchronous and happens before any HIP call: a call
 *    that returns an error has launched nothing and written nothing.
 *  - GQ_ERR_LAUNCH reports a failed kernel launch: the status returned by
 *    hipLaunchKernel for that launch (gq_last_hip_error() gives the HIP
 *    code). Faults inside a kernel are asynchronous and surface at the
 *    caller's next synchronisation.
 *  - No mutable shared state: calls are reentrant and thread-safe. libgq
 *    keeps only read-only caches filled on first use (each device's compute
 *    unit count, each kernel's resident workgroups per compute unit), which
 *    every thread computes identically. Identical inputs give
 *    bitwise-identical outputs (fixed reduction order, no atomics).
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQ_ABI_VERSION 7

enum {
    GQ_OK = 0,
    GQ_ERR_NULL = 1,         /* a required pointer is NULL */
    GQ_ERR_SHAPE = 2,        /* n < 1, k < 32, k % 32 != 0, bad m */
    GQ_ERR_ALIGN = 3,        /* a pointer violates its alignment */
    GQ_ERR_ALIAS = 4,        /* an output overlaps an input */
    GQ_ERR_UNSUPPORTED = 5,  /* unknown type, k or m beyond what is built */
    GQ_ERR_LAUNCH = 6,       /* the kernel launch failed */
    GQ_ERR_VALUE = 7         /* bad eps / soft cap, or workspace too small */
};

enum {
    GQ_TYPE_Q4_0 = 2,        /* GGUF type id of Q4_0 */
    GQ_TYPE_Q8_0 = 8,        /* GGUF type id of Q8_0 */
    GQ_TYPE_Q4_K = 12,       /* GGUF type id of Q4_K (256-element super-blocks) */
    GQ_TYPE_Q5_K = 13,       /* GGUF type id of Q5_K (256-element super-blocks) */
    GQ_TYPE_Q6_K = 14        /* GGUF type id of Q6_K (256-element super-blocks) */
};

/* Version of this header's signatures and of the packed layouts the pack
 * calls write; bumped on any change (7: the K-quant packed layout), so that a
 * caller can probe what the loaded library supports before using it (the
 * capability probe of the TensorSharp Gemma 4 page, batched fused decode
 * section: the managed side queries the native library and keeps older
 * behaviour for what it lacks). */
int gq_abi_version(void);

/* Static, never-NULL description of a status code (for the caller's error
 * messages; same batched fused decode section: failures are reported, not
 * silently routed to another path). */
const char *gq_status_str(int status);

/* The hipError_t value (as int) returned by the calling thread's most recent
 * kernel launch inside libgq: 0 after a successful launch, the HIP error
 * behind a GQ_ERR_LAUNCH otherwise. Thread-local; validation failures do
 * not change it. */
int gq_last_hip_error(void);

/* Bytes of one GGUF block of `type` (34, 18; 144 or 210 for the 256-element
 * K-quant super-blocks), 0 for an unknown type. */
size_t gq_block_bytes(int type);

/* Sizes of the packed arrays for an n x k matrix: qs is n*k (Q8_0) or
 * n*k/2 (Q4_0) bytes, d is n*(k/32)*2 bytes. 0 for invalid arguments. */
size_t gq_packed_qs_bytes(int type, int64_t n, int64_t k);
size_t gq_packed_d_bytes(int64_t n, int64_t k);

/*
 * gq_pack -- split n x k/32 GGUF blocks (device memory, 34 or 18 bytes each,
 * contiguous, any byte alignment) into the packed qs and d arrays above.
 * No value changes. blocks must not overlap qs or d. Any k that is a
 * multiple of 32 is accepted. A one-time, load-time re-layout of each weight
 * into the layout its kernel streams best, derived from the canonical file
 * and moving the same bytes (Gemma-4-E2B raw-Metal port page,
 * "Architecture", pack bullet: every tensor stored in kernel layout; Gem
 * native architecture page, "M4 Max operating assumptions": a packed sidecar
 * reproducibly derived from the canonical GGUF).
 */
int gq_pack(int type, const void *blocks, int64_t n, int64_t k,
            void *qs, uint16_t *d, void *stream);

/*
 * gq_quantize_q8_0 -- quantise m rows of fp32 activations x [m][k] to Q8_0:
 * per 32-element block, amax = max |x_i| (fp32); d = binary16(amax / 127)
 * (fp32 divide, then round to nearest even); q_i = clamp(round half away
 * from zero (x_i / d), -127, 127) with the divide in fp32 by the rounded
 * d, and q_i = 0 when d == 0. Outputs xq int8 [m][k] and xd binary16 bits
 * [m][k/32]. Inputs must be finite. Source: the activation quantiser of the
 * jouleclaw-loader-gguf BENCHMARKS page ("Matmul throughput -- Q8_0 scalar
 * vs NEON"), taken per 32-element block as in the GGUF Q8_0 format.
 * m >= 1; any k that is a multiple of 32.
 */
int gq_quantize_q8_0(const float *x, int64_t m, int64_t k,
                     int8_t *xq, uint16_t *xd, void *stream);

/*
 * gq_qmv_q8_0 / gq_qmv_q4_0 -- decode matvec with fp32 activations:
 * y[r] = sum_c w[r][c] * x[c] for r < n, accumulated in fp32.
 * Accuracy: |y - y_exact| <= 1e-4 * sum_c |w[r][c] x[c]| + 1e-6.
 * qs/d packed as above; x fp32 [k]; y fp32 [n].
 * Maximum k: 32768 (GQ_ERR_UNSUPPORTED beyond it).
 */
int gq_qmv_q8_0(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                const float *x, float *y, void *stream);
int gq_qmv_q4_0(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                const float *x, float *y, void *stream);

/*
 * gq_qmv_q8_0_ex / gq_qmv_q4_0_ex -- the same matvec with the folds that
 * sit on either side of a decode projection (Gemma-4-E2B raw-Metal port page,
 * "Architecture", kernels bullet: rmsnorm prologue and residual epilogue
 * folds; Gem native architecture page, residual epilogues):
 *  - if norm_weight is not NULL, x is first replaced by the Gemma RMSNorm
 *    x * (mean(x^2) + norm_eps)^(-1/2) * norm_weight, with the weight
 *    applied directly (SafeC Gemma 4 DESIGN_NOTES page, "RMSNorm"; Gemma 4
 *    uses norm_eps = 1e-6); norm_weight fp32 [k], 16-byte aligned;
 *    norm_eps >= 0 and finite, else GQ_ERR_VALUE. The sum of squares is
 *    taken in fp64, and the scale (mean + norm_eps)^(-1/2) in fp64 to
 *    within about 1e-14 relative; the scale is applied to each finished row (an fp64
 *    product) when the largest |x[c] * norm_weight[c]| lies in
 *    [2^-40, 2^40], and otherwise to the activations before the products,
 *    so any finite
 *    x is supported as long as every product x[c] * norm_weight[c] is
 *    finite in fp32 (|x w| <= 3.4e38);
 *  - if residual is not NULL, y[r] = residual[r] + (W x)[r]; residual fp32
 *    [n], 4-byte aligned; y may equal residual (in-place accumulate) but
 *    may not overlap it otherwise.
 * With both NULL these are gq_qmv_q8_0 / gq_qmv_q4_0.
 */
int gq_qmv_q8_0_ex(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                   const float *x, const float *norm_weight, float norm_eps,
                   const float *residual, float *y, void *stream);
int gq_qmv_q4_0_ex(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                   const float *x, const float *norm_weight, float norm_eps,
                   const float *residual, float *y, void *stream);

/*
 * gq_qmv_q8_0_argmax / gq_qmv_q4_0_argmax -- the vocabulary head of greedy
 * decode: optional RMSNorm prologue (as in the _ex entries), the matvec,
 * then per row the final-logit soft cap logits[r] = softcap * tanh(y[r] /
 * softcap) (SafeC DESIGN_NOTES page, "LM head"; Gemma 4 uses 30; softcap =
 * 0 leaves y unchanged), all written to logits fp32 [n], and a two-stage
 * on-GPU argmax (raw-Metal port page, "Architecture"): *index receives the
 * row of the largest logit, ties going to the lowest row, NaN ranking below
 * every number; *value receives that logit. workspace is caller-owned
 * device scratch of at least gq_argmax_workspace_bytes() bytes, 8-byte
 * aligned, holding the per-workgroup partials between the two stages; its
 * contents on entry are ignored. softcap must be >= 0 and finite, else
 * GQ_ERR_VALUE (also for a short workspace).
 */
size_t gq_argmax_workspace_bytes(void);
int gq_qmv_q8_0_argmax(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                       const float *x, const float *norm_weight, float norm_eps,
                       float softcap, float *logits, void *workspace,
                       size_t workspace_bytes, int32_t *index, float *value,
                       void *stream);
int gq_qmv_q4_0_argmax(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                       const float *x, const float *norm_weight, float norm_eps,
                       float softcap, float *logits, void *workspace,
                       size_t workspace_bytes, int32_t *index, float *value,
                       void *stream);

/*
 * gq_qmv_q8_0_argmax_noalloc -- gq_qmv_q8_0_argmax for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument; the per-workgroup
 * partials between the two stages live in a library-held device array of
 * gq_argmax_workspace_bytes() bytes (16 KiB) per device, which the first
 * stage's grid never exceeds, so every n is accepted. That array is looked
 * up on the first call on each device and kept until the process ends; the
 * call allocates nothing. Every call on a device shares that device's array:
 * calls that overlap on one device (concurrent streams or threads) race and
 * must be serialised by the caller. Results are bit-identical to
 * gq_qmv_q8_0_argmax's. Arguments, limits and errors as gq_qmv_q8_0_argmax.
 */
int gq_qmv_q8_0_argmax_noalloc(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                               const float *x, const float *norm_weight, float norm_eps,
                               float softcap, float *logits, int32_t *index, float *value,
                               void *stream);

/*
 * gq_qmv_q8_0_q8 / gq_qmv_q4_0_q8 -- decode matvec against one Q8_0
 * activation row (xq int8 [k], xd binary16 bits [k/32]):
 * S[r][b] = sum_i qw[r][b][i] * xq[b][i] computed exactly in int32
 * (qw = q for Q8_0, nibble - 8 for Q4_0), y[r] = sum_b dw[r][b] * dx[b] * S
 * in fp32. If blockdots is not NULL, S is also written to blockdots
 * int32 [n][k/32]. Maximum k as for the fp32 entries.
 */
int gq_qmv_q8_0_q8(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                   const int8_t *xq, const uint16_t *xd, float *y,
                   int32_t *blockdots, void *stream);
int gq_qmv_q4_0_q8(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                   const int8_t *xq, const uint16_t *xd, float *y,
                   int32_t *blockdots, void *stream);

/*
 * gq_qmv_q8_0_q8x / gq_qmv_q4_0_q8x -- the same integer path with the
 * activation quantiser folded in as a prologue: x fp32 [k] is quantised to
 * Q8_0 exactly as gq_quantize_q8_0 does (every workgroup quantises the
 * vector itself, so there is no separate launch and the codes never leave
 * the chip), then S, y and blockdots are as in gq_qmv_*_q8 on those codes,
 * bit for bit. If xq_out and xd_out are given (both or neither, else
 * GQ_ERR_NULL), the codes (int8 [k], 16-byte aligned) and scales (binary16
 * bits [k/32]) are also written there, for later calls on the same
 * activations. Inputs must be finite. Folding the quantiser into its
 * consumer follows the jouleclaw-loader-gguf BENCHMARKS page, where the
 * direct Q8_0 kernel takes fp32 activations and quantises them per call
 * ("Matmul throughput -- Q8_0 scalar vs NEON"). Maximum k: 32768.
 */
int gq_qmv_q8_0_q8x(const int8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                    const float *x, int8_t *xq_out, uint16_t *xd_out, float *y,
                    int32_t *blockdots, void *stream);
int gq_qmv_q4_0_q8x(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k,
                    const float *x, int8_t *xq_out, uint16_t *xd_out, float *y,
                    int32_t *blockdots, void *stream);

/*
 * gq_qffn_gate_up_gelu -- first half of the gated FFN, one pass over both
 * Q4_0 matrices: g = Wg x, u = Wu x (Wg, Wu [n_ff][k] packed), and
 * h[r] = G(g[r]) * u[r] with G the tanh-form GELU
 * G(t) = 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))), evaluated so that
 * it saturates (finite t never gives NaN). x fp32 [k]; h fp32 [n_ff].
 * The down projection is a separate gq_qmv_q4_0(Wd, h) call: every row of
 * it needs all of h. A fused [gate | up] weight is passed as two pointers
 * into it. Maximum k: 32768.
 */
int gq_qffn_gate_up_gelu(const uint8_t *g_qs, const uint16_t *g_d,
                         const uint8_t *u_qs, const uint16_t *u_d,
                         int64_t n_ff, int64_t k, const float *x, float *h,
                         void *stream);

/* The gate+up FFN pass with the pre-FFN RMSNorm folded in as a prologue
 * (norm_weight / norm_eps as in gq_qmv_q4_0_ex; NULL weight = no norm). The
 * residual after the down projection is gq_qmv_q4_0_ex's epilogue. */
int gq_qffn_gate_up_gelu_ex(const uint8_t *g_qs, const uint16_t *g_d,
                            const uint8_t *u_qs, const uint16_t *u_d,
                            int64_t n_ff, int64_t k, const float *x,
                            const float *norm_weight, float norm_eps, float *h,
                            void *stream);

/*
 * gq_qmm_tile_m -- small-M tile, Q4_0 weights [n][k] against m Q8_0
 * activation rows (xq int8 [m][k], xd binary16 bits [m][k/32]):
 * S[mi][r][b] exact in int32, y[mi][r] = sum_b dw[r][b] dx[mi][b] S (fp32),
 * y fp32 [m][n]. blockdots, if not NULL, receives S as int32 [m][n][k/32].
 * m = 8, 16, 32 are the prefill tiles (raw-Metal port page, "Batched
 * prefill"; Gem native architecture page, prefill tile of up to 32 rows);
 * any 1 <= m <= 32 is accepted, which also covers batched decode of m
 * sequences that share every weight read (TensorSharp Gemma 4 page, batched
 * fused decode). m outside [1, 32] gives GQ_ERR_UNSUPPORTED. Maximum k: 32768.
 */
int gq_qmm_tile_m(const uint8_t *qs, const uint16_t *d, int64_t n, int64_t k, int m,
                  const int8_t *xq, const uint16_t *xd, float *y,
                  int32_t *blockdots, void *stream);

/*
 * K-quant super-blocks: Q4_K, Q5_K and Q6_K, 256 elements each (distributed Gemma 4
 * GGUF files are mostly Q4_K_M / UD-Q4_K_XL: TensorSharp Gemma 4 page, model
 * table). The arithmetic is the jouleclaw-loader-gguf BENCHMARKS page's
 * ("Q4_K matmul": 32-element sub-blocks with a 6-bit scale and a 6-bit
 * minimum, w = d sc q - dmin m, summed as d sc sum(x q) - dmin m sum(x);
 * "Q5_K + Q6_K matmul": Q5_K adds one high bit per element to Q4_K's four,
 * w = d sc q - dmin m with q in 0..31; Q6_K has four low bits, two high bits
 * and a signed -32 offset, w = d sc (q - 32) with one int8 scale per 16
 * elements). The
 * GGUF byte layout the pages do not print:
 *  - Q4_K, 144 B: binary16 d, binary16 dmin, 12 bytes of scales/minimums
 *    (for sub-block j < 4: the low six bits of bytes j and j+4; for j >= 4:
 *    the low and high nibble of byte j+4 and the top two bits of bytes j-4
 *    and j), 128 quant bytes (byte 32g + l: element 64g + l in the low
 *    nibble, element 64g + 32 + l in the high one);
 *  - Q5_K, 176 B: d, dmin and the 12 scale/minimum bytes as in Q4_K, qh[32],
 *    then 128 quant bytes as in Q4_K; the fifth bit of element 64g + l
 *    (l < 32) is bit 2g of qh byte l, that of element 64g + 32 + l bit
 *    2g + 1;
 *  - Q6_K, 210 B: ql[128], qh[64], int8 scales[16], binary16 d; in half h
 *    and for l < 32, ql byte 64h + l holds the low bits of elements
 *    128h + l (low nibble) and 128h + l + 64 (high), ql byte 64h + l + 32
 *    those of 128h + l + 32 and 128h + l + 96, and qh byte 32h + l their
 *    high bits in bit pairs 0-1, 2-3, 4-5 and 6-7; element e uses scale e/16.
 * A matrix of n rows and k columns (k % 256 == 0) is n * k/256 super-blocks,
 * row-major.
 *
 * gq_kq_pack splits the GGUF super-blocks (device memory, contiguous, any
 * alignment) into ONE packed device buffer of gq_kq_packed_bytes(type, n, k)
 * bytes, 16-byte aligned, in 256-byte aligned sections (the load-time
 * kernel-layout pack of gq_pack). Every bit of the super-blocks is kept;
 * the scale and high-bit fields are rearranged so that each 16-byte quant
 * unit's own fields can be read with one load and no unpacking:
 *  - Q4_K: quants [n][k/2] (byte copies), then headers [n][k/256][16]: d,
 *    dmin, then for each 64-element chunk g (sub-blocks 2g and 2g+1) the
 *    24-bit field sc_2g | sc_2g+1 << 6 | m_2g << 12 | m_2g+1 << 18 in bytes
 *    4+3g .. 6+3g;
 *  - Q5_K: quants and headers as Q4_K, then fifth bits [n][k/32]: one
 *    little-endian 32-bit word per 16-byte quant unit u = 2g + t of a
 *    super-block (elements 64g + 16t + e, e < 16, and those + 32); quant
 *    word c of the unit holds elements 4c .. 4c+3 of both runs, whose fifth
 *    bits sit at bits 4, 5, 20, 21 (the first run) and 8, 9, 24, 25 (the
 *    second) of a field, rotated left by 0, 2, 8, 10 for c = 0..3 and OR-ed
 *    into the word (the four rotated fields do not overlap);
 *  - Q6_K: ql [n][k/2] (byte copies); qh [n][k/4]: for each 16-byte ql unit
 *    u = 4h + j of a super-block (elements 128h + 16j + e, e < 16, and those
 *    + 64), two little-endian 32-bit words; ql word c of the unit holds
 *    elements 4c .. 4c+3 of both runs, whose 2-bit high parts sit at bits 4,
 *    6, 20, 22 (the first run) and 8, 10, 24, 26 (the second) of a field;
 *    word p holds field 2p as it is and field 2p+1 rotated left by 8;
 *    scales [n][k/16]: per unit, its two int8 scales (8h + j, 8h + j + 4);
 *    d [n][k/256] binary16.
 * gq_kq_packed_bytes returns 0 for an unknown type or invalid shape.
 *
 * gq_qmv_q4_k / gq_qmv_q5_k / gq_qmv_q6_k -- decode matvec on a packed K-quant matrix
 * with fp32 activations: y[r] = sum_c w[r][c] x[c] accumulated in fp32,
 * |y - y_exact| <= 1e-4 * sum_c |w x| + 1e-6. x fp32 [k] (16-byte aligned),
 * y fp32 [n]. k must be a multiple of 256 (else GQ_ERR_SHAPE), at most
 * 32768 (else GQ_ERR_UNSUPPORTED). Special values as for the other matvecs.
 */
size_t gq_kq_packed_bytes(int type, int64_t n, int64_t k);
int gq_kq_pack(int type, const void *blocks, int64_t n, int64_t k, void *packed, void *stream);
int gq_qmv_q4_k(const void *packed, int64_t n, int64_t k, const float *x, float *y, void *stream);
int gq_qmv_q5_k(const void *packed, int64_t n, int64_t k, const float *x, float *y, void *stream);
int gq_qmv_q6_k(const void *packed, int64_t n, int64_t k, const float *x, float *y, void *stream);

/*
 * Decode-step chaining. A decode step is a fixed sequence of many small
 * launches over different weights; replaying it as one recorded unit
 * removes the per-launch host cost and the host round trips between them
 * (raw-Metal port page, "Architecture", host-loop bullet: steps encoded
 * several per command buffer, token dependence kept on the GPU; TensorSharp
 * Gemma 4 page, fused decode: the whole layer stack as one graph dispatch).
 *
 * gq_chain_begin(stream) starts recording on stream: from then until
 * gq_chain_end on the same stream, launches enqueued on it by the calling
 * thread -- libgq entry points and the caller's own kernels alike -- are
 * recorded, not executed, and the entry points still validate and return
 * their status as usual. gq_chain_end(stream, &chain) stops recording and
 * turns the sequence into an executable HIP graph; gq_chain_launch(chain,
 * stream) enqueues one replay of it on any stream of the same device, with
 * the pointers and sizes fixed at recording time (update the buffers' CONTENTS
 * between replays, e.g. a new x, never the pointers). gq_chain_destroy frees
 * it (NULL is a no-op); the caller must not destroy a chain whose replay may
 * still be running. gq_chain_launches reports the kernel launches recorded.
 *
 * The chain object is host memory owned by libgq between gq_chain_end and
 * gq_chain_destroy (the only allocation libgq makes; no device memory).
 * stream must not be NULL (the legacy default stream cannot be recorded):
 * GQ_ERR_VALUE. A HIP failure while recording (e.g. the stream is already
 * recording, or a call that cannot be recorded was made on it) gives
 * GQ_ERR_LAUNCH with gq_last_hip_error() holding the HIP code; a failed
 * gq_chain_end leaves the stream not recording and *chain NULL.
 */
typedef struct gq_chain gq_chain;
int gq_chain_begin(void *stream);
int gq_chain_end(void *stream, gq_chain **chain);
int gq_chain_launch(const gq_chain *chain, void *stream);
int gq_chain_destroy(gq_chain *chain);
size_t gq_chain_launches(const gq_chain *chain);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
