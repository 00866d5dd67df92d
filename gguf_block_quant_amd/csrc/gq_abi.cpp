// gq_abi.cpp -- the extern "C" boundary of libgq (declared in include/gq.h).
// Every entry point validates all of its arguments on the host, before any
// HIP call, then enqueues its kernel(s) on the caller's stream. No device
// allocation, no synchronisation, no global state; the chaining entries own
// one host-side graph object per recorded chain.
#include "../../include/gq.h"

#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "gq_launch.hpp"

namespace {

using gq::kMaxK;
using gq::kMaxRows;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    const void* p;
    size_t bytes;
};

inline bool overlap(Range a, Range b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Any output overlapping any input, or two outputs overlapping each other.
template <size_t NO, size_t NI>
bool any_alias(const Range (&outs)[NO], const Range (&ins)[NI]) {
    for (size_t i = 0; i < NO; ++i) {
        for (size_t j = 0; j < NI; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (size_t j = i + 1; j < NO; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}

inline bool type_ok(int type) { return type == GQ_TYPE_Q4_0 || type == GQ_TYPE_Q8_0; }
inline bool kq_type_ok(int type) { return type == GQ_TYPE_Q4_K || type == GQ_TYPE_Q5_K || type == GQ_TYPE_Q6_K; }

// n x k shape check of the K-quant entry points (whole 256-element super-blocks).
inline int check_kq_shape(int64_t n, int64_t k) {
    if (n < 1 || k < 256 || k % 256 != 0) return GQ_ERR_SHAPE;
    if (n > kMaxRows || k > kMaxK) return GQ_ERR_UNSUPPORTED;
    return GQ_OK;
}

// n x k shape check shared by every entry point.
inline int check_shape(int64_t n, int64_t k) {
    if (n < 1 || k < 32 || k % 32 != 0) return GQ_ERR_SHAPE;
    if (n > kMaxRows) return GQ_ERR_UNSUPPORTED;
    return GQ_OK;
}

inline size_t qs_bytes(int type, int64_t n, int64_t k) {
    return type == GQ_TYPE_Q8_0 ? static_cast<size_t>(n) * static_cast<size_t>(k)
                                : static_cast<size_t>(n) * static_cast<size_t>(k / 2);
}
inline size_t d_bytes(int64_t n, int64_t k) { return static_cast<size_t>(n) * static_cast<size_t>(k / 32) * 2; }

// HIP status of this thread's most recent launch attempt (diagnostics only).
thread_local int t_last_hip_error = 0;

inline int status_of(hipError_t e) {
    t_last_hip_error = static_cast<int>(e);
    return e == hipSuccess ? GQ_OK : GQ_ERR_LAUNCH;
}
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Checks shared by the two matvec families: packed weights, n, k.
int check_weights(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k) {
    if (qs == nullptr || d == nullptr) return GQ_ERR_NULL;
    int st = check_shape(n, k);
    if (st != GQ_OK) return st;
    if (k > kMaxK || !type_ok(type)) return GQ_ERR_UNSUPPORTED;
    if (!aligned(qs, 16) || !aligned(d, 2)) return GQ_ERR_ALIGN;
    return GQ_OK;
}

// Shared checks of the optional prologue / epilogue arguments.
int check_fold(const float* norm_w, float norm_eps, const float* residual) {
    if (norm_w != nullptr && (!aligned(norm_w, 16) || !(norm_eps >= 0.0f) || !(norm_eps < 1e30f)))
        return norm_w != nullptr && !aligned(norm_w, 16) ? GQ_ERR_ALIGN : GQ_ERR_VALUE;
    if (residual != nullptr && !aligned(residual, 4)) return GQ_ERR_ALIGN;
    return GQ_OK;
}

int qmv_f32(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
            const float* norm_w, float norm_eps, const float* residual, float* y, void* stream) {
    if (x == nullptr || y == nullptr) return GQ_ERR_NULL;
    int st = check_weights(type, qs, d, n, k);
    if (st != GQ_OK) return st;
    if (!aligned(x, 16) || !aligned(y, 4)) return GQ_ERR_ALIGN;
    st = check_fold(norm_w, norm_eps, residual);
    if (st != GQ_OK) return st;
    const size_t nb4 = static_cast<size_t>(n) * 4;
    const Range outs[] = {{y, nb4}};
    // y may be the residual itself (in-place accumulate), but no other overlap
    const Range ins[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}, {x, static_cast<size_t>(k) * 4},
                         {norm_w, norm_w ? static_cast<size_t>(k) * 4 : 0},
                         {residual, (residual && residual != y) ? nb4 : 0}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_f32(type, qs, d, n, k, x, norm_w, norm_eps, residual, y,
                                        as_stream(stream)));
}

int qmv_argmax(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
               const float* norm_w, float norm_eps, float softcap, float* logits, void* workspace,
               size_t workspace_bytes, int32_t* index, float* value, void* stream) {
    if (x == nullptr || logits == nullptr || workspace == nullptr || index == nullptr || value == nullptr)
        return GQ_ERR_NULL;
    int st = check_weights(type, qs, d, n, k);
    if (st != GQ_OK) return st;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(workspace, 8) || !aligned(index, 4) ||
        !aligned(value, 4))
        return GQ_ERR_ALIGN;
    st = check_fold(norm_w, norm_eps, nullptr);
    if (st != GQ_OK) return st;
    if (!(softcap >= 0.0f) || !(softcap < 1e30f) || workspace_bytes < gq::kArgmaxWorkspaceBytes) return GQ_ERR_VALUE;
    const Range outs[] = {{logits, static_cast<size_t>(n) * 4}, {workspace, gq::kArgmaxWorkspaceBytes},
                          {index, 4}, {value, 4}};
    const Range ins[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}, {x, static_cast<size_t>(k) * 4},
                         {norm_w, norm_w ? static_cast<size_t>(k) * 4 : 0}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_argmax(type, qs, d, n, k, x, norm_w, norm_eps, softcap, logits, workspace,
                                           index, value, as_stream(stream)));
}

int qmv_argmax_noalloc(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                       const float* norm_w, float norm_eps, float softcap, float* logits, int32_t* index,
                       float* value, void* stream) {
    if (x == nullptr || logits == nullptr || index == nullptr || value == nullptr) return GQ_ERR_NULL;
    int st = check_weights(type, qs, d, n, k);
    if (st != GQ_OK) return st;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(index, 4) || !aligned(value, 4)) return GQ_ERR_ALIGN;
    st = check_fold(norm_w, norm_eps, nullptr);
    if (st != GQ_OK) return st;
    if (!(softcap >= 0.0f) || !(softcap < 1e30f)) return GQ_ERR_VALUE;
    const Range outs[] = {{logits, static_cast<size_t>(n) * 4}, {index, 4}, {value, 4}};
    const Range ins[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}, {x, static_cast<size_t>(k) * 4},
                         {norm_w, norm_w ? static_cast<size_t>(k) * 4 : 0}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_argmax_noalloc(type, qs, d, n, k, x, norm_w, norm_eps, softcap, logits, index,
                                                   value, as_stream(stream)));
}

int qmv_q8(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const int8_t* xq,
           const uint16_t* xd, float* y, int32_t* blockdots, void* stream) {
    if (xq == nullptr || xd == nullptr || y == nullptr) return GQ_ERR_NULL;
    int st = check_weights(type, qs, d, n, k);
    if (st != GQ_OK) return st;
    if (!aligned(xq, 16) || !aligned(xd, 2) || !aligned(y, 4) || !aligned(blockdots, 4)) return GQ_ERR_ALIGN;
    const Range outs[] = {{y, static_cast<size_t>(n) * 4},
                          {blockdots, blockdots ? static_cast<size_t>(n) * static_cast<size_t>(k / 32) * 4 : 0}};
    const Range ins[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}, {xq, static_cast<size_t>(k)},
                         {xd, static_cast<size_t>(k / 32) * 2}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_q8(type, qs, d, n, k, xq, xd, y, blockdots, as_stream(stream)));
}

int qmv_q8x(int type, const void* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
            int8_t* xq_out, uint16_t* xd_out, float* y, int32_t* blockdots, void* stream) {
    if (x == nullptr || y == nullptr || (xq_out == nullptr) != (xd_out == nullptr)) return GQ_ERR_NULL;
    int st = check_weights(type, qs, d, n, k);
    if (st != GQ_OK) return st;
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(blockdots, 4) || !aligned(xq_out, 16) ||
        !aligned(xd_out, 2))
        return GQ_ERR_ALIGN;
    const Range outs[] = {{y, static_cast<size_t>(n) * 4},
                          {blockdots, blockdots ? static_cast<size_t>(n) * static_cast<size_t>(k / 32) * 4 : 0},
                          {xq_out, xq_out ? static_cast<size_t>(k) : 0},
                          {xd_out, xd_out ? static_cast<size_t>(k / 32) * 2 : 0}};
    const Range ins[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}, {x, static_cast<size_t>(k) * 4}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_q8x(type, qs, d, n, k, x, xq_out, xd_out, y, blockdots, as_stream(stream)));
}

}  // namespace

extern "C" {

int gq_abi_version(void) { return GQ_ABI_VERSION; }

int gq_last_hip_error(void) { return t_last_hip_error; }

const char* gq_status_str(int status) {
    switch (status) {
        case GQ_OK: return "ok";
        case GQ_ERR_NULL: return "a required pointer is NULL";
        case GQ_ERR_SHAPE: return "invalid shape (need n >= 1, k >= 32, k % 32 == 0, supported m)";
        case GQ_ERR_ALIGN: return "a pointer is not aligned as required";
        case GQ_ERR_ALIAS: return "an output overlaps an input";
        case GQ_ERR_UNSUPPORTED: return "unsupported type, k, n or m";
        case GQ_ERR_LAUNCH: return "kernel launch failed";
        case GQ_ERR_VALUE: return "invalid scalar argument (eps, soft cap) or workspace too small";
        default: return "unknown status";
    }
}

size_t gq_block_bytes(int type) {
    if (type == GQ_TYPE_Q8_0) return 34;
    if (type == GQ_TYPE_Q4_0) return 18;
    if (type == GQ_TYPE_Q4_K) return 144;
    if (type == GQ_TYPE_Q5_K) return 176;
    if (type == GQ_TYPE_Q6_K) return 210;
    return 0;
}

size_t gq_packed_qs_bytes(int type, int64_t n, int64_t k) {
    if (!type_ok(type) || check_shape(n, k) != GQ_OK) return 0;
    return qs_bytes(type, n, k);
}

size_t gq_packed_d_bytes(int64_t n, int64_t k) {
    if (check_shape(n, k) != GQ_OK) return 0;
    return d_bytes(n, k);
}

int gq_pack(int type, const void* blocks, int64_t n, int64_t k, void* qs, uint16_t* d, void* stream) {
    if (blocks == nullptr || qs == nullptr || d == nullptr) return GQ_ERR_NULL;
    int st = check_shape(n, k);
    if (st != GQ_OK) return st;
    if (!type_ok(type)) return GQ_ERR_UNSUPPORTED;
    if (!aligned(qs, 16) || !aligned(d, 2)) return GQ_ERR_ALIGN;
    const size_t blk_bytes = static_cast<size_t>(n) * static_cast<size_t>(k / 32) * gq_block_bytes(type);
    const Range outs[] = {{qs, qs_bytes(type, n, k)}, {d, d_bytes(n, k)}};
    const Range ins[] = {{blocks, blk_bytes}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_pack(type, static_cast<const uint8_t*>(blocks), n, k,
                                     static_cast<uint8_t*>(qs), d, as_stream(stream)));
}

int gq_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd, void* stream) {
    if (x == nullptr || xq == nullptr || xd == nullptr) return GQ_ERR_NULL;
    int st = check_shape(m, k);
    if (st != GQ_OK) return st;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 2)) return GQ_ERR_ALIGN;
    const Range outs[] = {{xq, static_cast<size_t>(m) * static_cast<size_t>(k)}, {xd, d_bytes(m, k)}};
    const Range ins[] = {{x, static_cast<size_t>(m) * static_cast<size_t>(k) * 4}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_quantize_q8_0(x, m, k, xq, xd, as_stream(stream)));
}

int gq_qmv_q8_0(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x, float* y,
                void* stream) {
    return qmv_f32(GQ_TYPE_Q8_0, qs, d, n, k, x, nullptr, 0.0f, nullptr, y, stream);
}

int gq_qmv_q4_0(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x, float* y,
                void* stream) {
    return qmv_f32(GQ_TYPE_Q4_0, qs, d, n, k, x, nullptr, 0.0f, nullptr, y, stream);
}

int gq_qmv_q8_0_ex(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                   const float* norm_weight, float norm_eps, const float* residual, float* y, void* stream) {
    return qmv_f32(GQ_TYPE_Q8_0, qs, d, n, k, x, norm_weight, norm_eps, residual, y, stream);
}

int gq_qmv_q4_0_ex(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                   const float* norm_weight, float norm_eps, const float* residual, float* y, void* stream) {
    return qmv_f32(GQ_TYPE_Q4_0, qs, d, n, k, x, norm_weight, norm_eps, residual, y, stream);
}

size_t gq_argmax_workspace_bytes(void) { return gq::kArgmaxWorkspaceBytes; }

int gq_qmv_q8_0_argmax(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                       const float* norm_weight, float norm_eps, float softcap, float* logits, void* workspace,
                       size_t workspace_bytes, int32_t* index, float* value, void* stream) {
    return qmv_argmax(GQ_TYPE_Q8_0, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits, workspace,
                      workspace_bytes, index, value, stream);
}

int gq_qmv_q4_0_argmax(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                       const float* norm_weight, float norm_eps, float softcap, float* logits, void* workspace,
                       size_t workspace_bytes, int32_t* index, float* value, void* stream) {
    return qmv_argmax(GQ_TYPE_Q4_0, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits, workspace,
                      workspace_bytes, index, value, stream);
}

int gq_qmv_q8_0_argmax_noalloc(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x,
                               const float* norm_weight, float norm_eps, float softcap, float* logits,
                               int32_t* index, float* value, void* stream) {
    return qmv_argmax_noalloc(GQ_TYPE_Q8_0, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits, index, value,
                              stream);
}

int gq_qmv_q8_0_q8(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const int8_t* xq,
                   const uint16_t* xd, float* y, int32_t* blockdots, void* stream) {
    return qmv_q8(GQ_TYPE_Q8_0, qs, d, n, k, xq, xd, y, blockdots, stream);
}

int gq_qmv_q4_0_q8(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, const int8_t* xq,
                   const uint16_t* xd, float* y, int32_t* blockdots, void* stream) {
    return qmv_q8(GQ_TYPE_Q4_0, qs, d, n, k, xq, xd, y, blockdots, stream);
}

int gq_qmv_q8_0_q8x(const int8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x, int8_t* xq_out,
                    uint16_t* xd_out, float* y, int32_t* blockdots, void* stream) {
    return qmv_q8x(GQ_TYPE_Q8_0, qs, d, n, k, x, xq_out, xd_out, y, blockdots, stream);
}

int gq_qmv_q4_0_q8x(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, const float* x, int8_t* xq_out,
                    uint16_t* xd_out, float* y, int32_t* blockdots, void* stream) {
    return qmv_q8x(GQ_TYPE_Q4_0, qs, d, n, k, x, xq_out, xd_out, y, blockdots, stream);
}

}  // extern "C"

namespace {
int ffn(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs, const uint16_t* u_d, int64_t n_ff,
        int64_t k, const float* x, const float* norm_w, float norm_eps, float* h, void* stream) {
    if (g_qs == nullptr || g_d == nullptr || u_qs == nullptr || u_d == nullptr || x == nullptr ||
        h == nullptr)
        return GQ_ERR_NULL;
    int st = check_shape(n_ff, k);
    if (st != GQ_OK) return st;
    if (k > kMaxK) return GQ_ERR_UNSUPPORTED;
    if (!aligned(g_qs, 16) || !aligned(u_qs, 16) || !aligned(g_d, 2) || !aligned(u_d, 2) ||
        !aligned(x, 16) || !aligned(h, 4))
        return GQ_ERR_ALIGN;
    st = check_fold(norm_w, norm_eps, nullptr);
    if (st != GQ_OK) return st;
    const size_t qb = qs_bytes(GQ_TYPE_Q4_0, n_ff, k), db = d_bytes(n_ff, k);
    const Range outs[] = {{h, static_cast<size_t>(n_ff) * 4}};
    const Range ins[] = {{g_qs, qb}, {g_d, db}, {u_qs, qb}, {u_d, db}, {x, static_cast<size_t>(k) * 4},
                         {norm_w, norm_w ? static_cast<size_t>(k) * 4 : 0}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_ffn_gate_up(g_qs, g_d, u_qs, u_d, n_ff, k, x, norm_w, norm_eps, h,
                                            as_stream(stream)));
}
}  // namespace

extern "C" {

int gq_qffn_gate_up_gelu(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs,
                         const uint16_t* u_d, int64_t n_ff, int64_t k, const float* x, float* h,
                         void* stream) {
    return ffn(g_qs, g_d, u_qs, u_d, n_ff, k, x, nullptr, 0.0f, h, stream);
}

int gq_qffn_gate_up_gelu_ex(const uint8_t* g_qs, const uint16_t* g_d, const uint8_t* u_qs,
                            const uint16_t* u_d, int64_t n_ff, int64_t k, const float* x,
                            const float* norm_weight, float norm_eps, float* h, void* stream) {
    return ffn(g_qs, g_d, u_qs, u_d, n_ff, k, x, norm_weight, norm_eps, h, stream);
}

size_t gq_kq_packed_bytes(int type, int64_t n, int64_t k) {
    if (!kq_type_ok(type) || check_kq_shape(n, k) != GQ_OK) return 0;
    return gq::kq_layout(type, n, k, nullptr);
}

int gq_kq_pack(int type, const void* blocks, int64_t n, int64_t k, void* packed, void* stream) {
    if (blocks == nullptr || packed == nullptr) return GQ_ERR_NULL;
    if (!kq_type_ok(type)) return GQ_ERR_UNSUPPORTED;
    int st = check_kq_shape(n, k);
    if (st != GQ_OK) return st;
    if (!aligned(packed, 16)) return GQ_ERR_ALIGN;
    const size_t bb = gq_block_bytes(type);
    const Range outs[] = {{packed, gq::kq_layout(type, n, k, nullptr)}};
    const Range ins[] = {{blocks, static_cast<size_t>(n) * static_cast<size_t>(k / 256) * bb}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_kq_pack(type, static_cast<const uint8_t*>(blocks), n, k,
                                        static_cast<uint8_t*>(packed), as_stream(stream)));
}

}  // extern "C"

namespace {
int qmv_kq(int type, const void* packed, int64_t n, int64_t k, const float* x, float* y, void* stream) {
    if (packed == nullptr || x == nullptr || y == nullptr) return GQ_ERR_NULL;
    int st = check_kq_shape(n, k);
    if (st != GQ_OK) return st;
    if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4)) return GQ_ERR_ALIGN;
    const Range outs[] = {{y, static_cast<size_t>(n) * 4}};
    const Range ins[] = {{packed, gq::kq_layout(type, n, k, nullptr)}, {x, static_cast<size_t>(k) * 4}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_qmv_kq(type, static_cast<const uint8_t*>(packed), n, k, x, y, as_stream(stream)));
}
}  // namespace

extern "C" {

int gq_qmv_q4_k(const void* packed, int64_t n, int64_t k, const float* x, float* y, void* stream) {
    return qmv_kq(GQ_TYPE_Q4_K, packed, n, k, x, y, stream);
}

int gq_qmv_q5_k(const void* packed, int64_t n, int64_t k, const float* x, float* y, void* stream) {
    return qmv_kq(GQ_TYPE_Q5_K, packed, n, k, x, y, stream);
}

int gq_qmv_q6_k(const void* packed, int64_t n, int64_t k, const float* x, float* y, void* stream) {
    return qmv_kq(GQ_TYPE_Q6_K, packed, n, k, x, y, stream);
}

int gq_qmm_tile_m(const uint8_t* qs, const uint16_t* d, int64_t n, int64_t k, int m, const int8_t* xq,
                  const uint16_t* xd, float* y, int32_t* blockdots, void* stream) {
    if (qs == nullptr || d == nullptr || xq == nullptr || xd == nullptr || y == nullptr) return GQ_ERR_NULL;
    int st = check_shape(n, k);
    if (st != GQ_OK) return st;
    if (m < 1 || m > 32) return GQ_ERR_UNSUPPORTED;
    if (k > kMaxK) return GQ_ERR_UNSUPPORTED;
    if (!aligned(qs, 16) || !aligned(d, 2) || !aligned(xq, 16) || !aligned(xd, 2) || !aligned(y, 4) ||
        !aligned(blockdots, 4))
        return GQ_ERR_ALIGN;
    const size_t mn = static_cast<size_t>(m) * static_cast<size_t>(n);
    const Range outs[] = {{y, mn * 4}, {blockdots, blockdots ? mn * static_cast<size_t>(k / 32) * 4 : 0}};
    const Range ins[] = {{qs, qs_bytes(GQ_TYPE_Q4_0, n, k)}, {d, d_bytes(n, k)},
                         {xq, static_cast<size_t>(m) * static_cast<size_t>(k)}, {xd, d_bytes(m, k)}};
    if (any_alias(outs, ins)) return GQ_ERR_ALIAS;
    return status_of(gq::launch_tile_q4_0(qs, d, n, k, m, xq, xd, y, blockdots, as_stream(stream)));
}

}  // extern "C"

// ---- decode-step chaining: stream capture into one executable HIP graph ----
struct gq_chain {
    hipGraphExec_t exec;
    size_t launches;     // kernel nodes recorded
};

extern "C" {

int gq_chain_begin(void* stream) {
    if (stream == nullptr) return GQ_ERR_VALUE;
    // relaxed: the caller may interleave its own (unrecorded) host-side HIP
    // calls, e.g. allocations, while the step is being recorded
    return status_of(hipStreamBeginCapture(as_stream(stream), hipStreamCaptureModeRelaxed));
}

int gq_chain_end(void* stream, gq_chain** chain) {
    if (stream == nullptr) return GQ_ERR_VALUE;
    if (chain == nullptr) return GQ_ERR_NULL;
    *chain = nullptr;
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(as_stream(stream), &graph);
    if (e != hipSuccess) {
        if (graph != nullptr) hipGraphDestroy(graph);
        return status_of(e);
    }
    size_t count = 0;
    e = hipGraphGetNodes(graph, nullptr, &count);
    size_t kernels = 0;
    if (e == hipSuccess && count > 0) {
        std::vector<hipGraphNode_t> nodes(count);
        e = hipGraphGetNodes(graph, nodes.data(), &count);
        for (size_t i = 0; e == hipSuccess && i < count; ++i) {
            hipGraphNodeType t;
            e = hipGraphNodeGetType(nodes[i], &t);
            if (e == hipSuccess && t == hipGraphNodeTypeKernel) ++kernels;
        }
    }
    hipGraphExec_t exec = nullptr;
    if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) return status_of(e);
    gq_chain* c = new (std::nothrow) gq_chain{exec, kernels};
    if (c == nullptr) {
        hipGraphExecDestroy(exec);
        return status_of(hipErrorOutOfMemory);
    }
    *chain = c;
    return status_of(hipSuccess);
}

int gq_chain_launch(const gq_chain* chain, void* stream) {
    if (chain == nullptr) return GQ_ERR_NULL;
    return status_of(hipGraphLaunch(chain->exec, as_stream(stream)));
}

int gq_chain_destroy(gq_chain* chain) {
    if (chain == nullptr) return GQ_OK;
    const hipError_t e = hipGraphExecDestroy(chain->exec);
    delete chain;
    return status_of(e);
}

size_t gq_chain_launches(const gq_chain* chain) { return chain == nullptr ? 0 : chain->launches; }

}  // extern "C"
