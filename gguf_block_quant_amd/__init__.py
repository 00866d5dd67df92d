"""gguf_block_quant_amd -- Python binding of libgq (include/gq.h).

Argument marshalling only: every function here checks that its tensors are
device-resident and contiguous, passes their data pointers and the current
(or given) HIP stream to the C ABI entry point of the same name (``gq_``
prefix dropped), and raises ``GQError`` on a non-zero status. All compute
runs in libgq's HIP kernels; there is no fallback. Importing this module
fails loudly when libgq.so has not been built.

The shared library is loaded on first use (so that the build step can run
before it exists); using any entry point without a built libgq.so raises
ImportError.

Tensors are torch tensors (PyTorch supplies device memory and streams).
Binary16 scale arrays are carried as int16/uint16 tensors of raw bits.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

TYPE_Q4_0 = 2
TYPE_Q8_0 = 8
TYPE_Q4_K = 12
TYPE_Q5_K = 13
TYPE_Q6_K = 14

GQ_OK = 0
STATUS_NAMES = {0: "GQ_OK", 1: "GQ_ERR_NULL", 2: "GQ_ERR_SHAPE", 3: "GQ_ERR_ALIGN",
                4: "GQ_ERR_ALIAS", 5: "GQ_ERR_UNSUPPORTED", 6: "GQ_ERR_LAUNCH", 7: "GQ_ERR_VALUE"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float

_SIGS = {
    "gq_abi_version": ([], _I),
    "gq_status_str": ([_I], ctypes.c_char_p),
    "gq_last_hip_error": ([], _I),
    "gq_block_bytes": ([_I], ctypes.c_size_t),
    "gq_packed_qs_bytes": ([_I, _I64, _I64], ctypes.c_size_t),
    "gq_packed_d_bytes": ([_I64, _I64], ctypes.c_size_t),
    "gq_pack": ([_I, _P, _I64, _I64, _P, _P, _P], _I),
    "gq_quantize_q8_0": ([_P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmv_q8_0": ([_P, _P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmv_q4_0": ([_P, _P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmv_q8_0_q8": ([_P, _P, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "gq_qmv_q4_0_q8": ([_P, _P, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "gq_qmv_q8_0_q8x": ([_P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P], _I),
    "gq_qmv_q4_0_q8x": ([_P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P], _I),
    "gq_qffn_gate_up_gelu": ([_P, _P, _P, _P, _I64, _I64, _P, _P, _P], _I),
    "gq_qffn_gate_up_gelu_ex": ([_P, _P, _P, _P, _I64, _I64, _P, _P, _F, _P, _P], _I),
    "gq_qmv_q8_0_ex": ([_P, _P, _I64, _I64, _P, _P, _F, _P, _P, _P], _I),
    "gq_qmv_q4_0_ex": ([_P, _P, _I64, _I64, _P, _P, _F, _P, _P, _P], _I),
    "gq_argmax_workspace_bytes": ([], ctypes.c_size_t),
    "gq_qmv_q8_0_argmax": ([_P, _P, _I64, _I64, _P, _P, _F, _F, _P, _P, ctypes.c_size_t, _P, _P, _P], _I),
    "gq_qmv_q4_0_argmax": ([_P, _P, _I64, _I64, _P, _P, _F, _F, _P, _P, ctypes.c_size_t, _P, _P, _P], _I),
    "gq_qmv_q8_0_argmax_noalloc": ([_P, _P, _I64, _I64, _P, _P, _F, _F, _P, _P, _P, _P], _I),
    "gq_kq_packed_bytes": ([_I, _I64, _I64], ctypes.c_size_t),
    "gq_kq_pack": ([_I, _P, _I64, _I64, _P, _P], _I),
    "gq_qmv_q4_k": ([_P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmv_q5_k": ([_P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmv_q6_k": ([_P, _I64, _I64, _P, _P, _P], _I),
    "gq_qmm_tile_m": ([_P, _P, _I64, _I64, _I, _P, _P, _P, _P, _P], _I),
    "gq_chain_begin": ([_P], _I),
    "gq_chain_end": ([_P, ctypes.POINTER(_P)], _I),
    "gq_chain_launch": ([_P, _P], _I),
    "gq_chain_destroy": ([_P], _I),
    "gq_chain_launches": ([_P], ctypes.c_size_t),
}
_handle = None


def raw():
    """The ctypes handle of libgq, loaded on first use."""
    global _handle
    if _handle is None:
        # libgq must resolve libamdhip64 to the HIP runtime torch already
        # carries (same SONAME), so that device pointers and streams handed
        # over from torch belong to the runtime that launches the kernels.
        # Loading libgq first would pull in a second runtime.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libgq.so is not built (expected at %s); run `python -m gguf_block_quant_amd.build` "
                "or __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _handle = lib
    return _handle


class GQError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        self.hip_error = raw().gq_last_hip_error() if status == 6 else 0
        extra = " [hipError %d]" % self.hip_error if status == 6 else ""
        super().__init__("%s failed: %s (%s)%s" % (fn, STATUS_NAMES.get(status, status),
                                                   status_str(status), extra))


def abi_version() -> int:
    return raw().gq_abi_version()


def status_str(status: int) -> str:
    return raw().gq_status_str(status).decode()


def block_bytes(qtype: int) -> int:
    return raw().gq_block_bytes(qtype)


def packed_qs_bytes(qtype: int, n: int, k: int) -> int:
    return raw().gq_packed_qs_bytes(qtype, n, k)


def packed_d_bytes(n: int, k: int) -> int:
    return raw().gq_packed_d_bytes(n, k)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtypes(kind):
    """Accepted torch dtypes per argument kind."""
    torch = _torch()
    return {
        "f32": (torch.float32,),
        "i8": (torch.int8,),
        "i32": (torch.int32,),
        "h16": (torch.int16, torch.uint16),          # binary16 bit patterns
        "bytes": None,                               # raw bytes: any dtype, sized in bytes
    }[kind]


def _ptr(t, name, kind="bytes", need=0):
    """Device pointer of tensor ``t`` after checking it can hold what the C
    entry point will touch: ``need`` elements of ``kind`` (for "bytes", need
    is a byte count and any dtype is accepted). The C ABI sees only pointers,
    so a short or mistyped buffer would be read or written out of bounds on
    the device; it is refused here with ValueError before any call."""
    if t is None:
        return None
    dts = _dtypes(kind)
    if dts is not None and t.dtype not in dts:
        raise ValueError("%s must have dtype %s, got %s" % (name, " or ".join(str(d) for d in dts), t.dtype))
    have = t.numel() * t.element_size() if dts is None else t.numel()
    need = max(0, int(need))
    if have < need:
        raise ValueError("%s holds %d %s, the call needs %d" % (name, have, "bytes" if dts is None else "elements",
                                                              need))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    p = _TensorPtr(t.data_ptr())
    p.name, p.on_device = name, bool(t.is_cuda)
    return p


class _TensorPtr(ctypes.c_void_p):
    """A tensor's data pointer; _call checks that it is device memory once
    every argument's size and dtype has been checked."""


def _nb(k):
    """Blocks (or block scales) per row of k elements."""
    return max(0, int(k)) // 32


class _CurrentStream:
    """Placeholder for "torch's current stream", resolved by _call after the
    tensor checks (so those run, and fail, without a device)."""


def _stream(stream):
    if stream is None:
        return _CurrentStream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _call(fn, *args):
    for a in args:
        if isinstance(a, _TensorPtr) and not a.on_device:
            raise ValueError("%s must be a device tensor" % a.name)
    args = [ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream) if isinstance(a, _CurrentStream) else a
            for a in args]
    st = getattr(raw(), fn)(*args)
    if st != GQ_OK:
        raise GQError(st, fn)


def _like(ref, shape, dtype):
    torch = _torch()
    return torch.empty(shape, dtype=dtype, device=ref.device)


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
# Each entry point checks its tensors against the sizes its C call will touch
# (_ptr) for shapes the C ABI accepts; for any other shape the sizes are not
# checked (_dims gives zeros) and the C entry point returns its own status.

def _dims(n, k, m=1):
    """(n, k, m) if the C ABI accepts the shape, else (0, 0, 0)."""
    n, k, m = int(n), int(k), int(m)
    if n >= 1 and k >= 32 and k % 32 == 0 and m >= 1:
        return n, k, m
    return 0, 0, 0


def _weights(qtype, qs, d, n, k, names=("qs", "d")):
    n_, k_, _ = _dims(n, k)
    qb = packed_qs_bytes(qtype, n_, k_) if n_ else 0
    return (_ptr(qs, names[0], "bytes", qb), _ptr(d, names[1], "h16", n_ * _nb(k_)))


def pack(qtype, blocks, n, k, qs=None, d=None, stream=None):
    """GGUF blocks (device uint8, n*k/32 blocks) -> packed (qs, d)."""
    torch = _torch()
    if qs is None:
        qs = _like(blocks, (n, k if qtype == TYPE_Q8_0 else k // 2),
                   torch.int8 if qtype == TYPE_Q8_0 else torch.uint8)
    if d is None:
        d = _like(blocks, (n, k // 32), torch.int16)
    n_, k_, _ = _dims(n, k)
    _call("gq_pack", qtype, _ptr(blocks, "blocks", "bytes", n_ * _nb(k_) * block_bytes(qtype)), n, k,
          *_weights(qtype, qs, d, n, k), _stream(stream))
    return qs, d


def quantize_q8_0(x, xq=None, xd=None, stream=None):
    """fp32 x [m][k] (or [k]) -> (xq int8 [m][k], xd binary16 bits [m][k/32])."""
    torch = _torch()
    m, k = (1, x.shape[0]) if x.dim() == 1 else tuple(x.shape)
    if xq is None:
        xq = _like(x, tuple(x.shape), torch.int8)
    if xd is None:
        xd = _like(x, tuple(x.shape[:-1]) + (k // 32,), torch.int16)
    m_, k_, _ = _dims(m, k)
    _call("gq_quantize_q8_0", _ptr(x, "x", "f32", m_ * k_), m, k, _ptr(xq, "xq", "i8", m_ * k_),
          _ptr(xd, "xd", "h16", m_ * _nb(k_)), _stream(stream))
    return xq, xd


def _qmv_f32(fn, qtype, qs, d, n, k, x, y, stream):
    torch = _torch()
    if y is None:
        y = _like(x, (n,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call(fn, *_weights(qtype, qs, d, n, k), n, k, _ptr(x, "x", "f32", k_), _ptr(y, "y", "f32", n_),
          _stream(stream))
    return y


def qmv_q8_0(qs, d, n, k, x, y=None, stream=None):
    return _qmv_f32("gq_qmv_q8_0", TYPE_Q8_0, qs, d, n, k, x, y, stream)


def qmv_q4_0(qs, d, n, k, x, y=None, stream=None):
    return _qmv_f32("gq_qmv_q4_0", TYPE_Q4_0, qs, d, n, k, x, y, stream)


def _qmv_q8(fn, qtype, qs, d, n, k, xq, xd, y, blockdots, stream):
    torch = _torch()
    if y is None:
        y = _like(xq, (n,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call(fn, *_weights(qtype, qs, d, n, k), n, k, _ptr(xq, "xq", "i8", k_), _ptr(xd, "xd", "h16", _nb(k_)),
          _ptr(y, "y", "f32", n_), _ptr(blockdots, "blockdots", "i32", n_ * _nb(k_)), _stream(stream))
    return y


def qmv_q8_0_q8(qs, d, n, k, xq, xd, y=None, blockdots=None, stream=None):
    return _qmv_q8("gq_qmv_q8_0_q8", TYPE_Q8_0, qs, d, n, k, xq, xd, y, blockdots, stream)


def qmv_q4_0_q8(qs, d, n, k, xq, xd, y=None, blockdots=None, stream=None):
    return _qmv_q8("gq_qmv_q4_0_q8", TYPE_Q4_0, qs, d, n, k, xq, xd, y, blockdots, stream)


def _qmv_q8x(fn, qtype, qs, d, n, k, x, y, blockdots, xq_out, xd_out, stream):
    torch = _torch()
    if y is None:
        y = _like(x, (n,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call(fn, *_weights(qtype, qs, d, n, k), n, k, _ptr(x, "x", "f32", k_), _ptr(xq_out, "xq_out", "i8", k_),
          _ptr(xd_out, "xd_out", "h16", _nb(k_)), _ptr(y, "y", "f32", n_),
          _ptr(blockdots, "blockdots", "i32", n_ * _nb(k_)), _stream(stream))
    return y


def qmv_q8_0_q8x(qs, d, n, k, x, y=None, blockdots=None, xq_out=None, xd_out=None, stream=None):
    """Integer path quantising the fp32 x itself (no separate quantise launch)."""
    return _qmv_q8x("gq_qmv_q8_0_q8x", TYPE_Q8_0, qs, d, n, k, x, y, blockdots, xq_out, xd_out, stream)


def qmv_q4_0_q8x(qs, d, n, k, x, y=None, blockdots=None, xq_out=None, xd_out=None, stream=None):
    return _qmv_q8x("gq_qmv_q4_0_q8x", TYPE_Q4_0, qs, d, n, k, x, y, blockdots, xq_out, xd_out, stream)


def qmv_q8_0_ex(qs, d, n, k, x, norm_weight=None, norm_eps=1e-6, residual=None, y=None, stream=None):
    return _qmv_ex("gq_qmv_q8_0_ex", TYPE_Q8_0, qs, d, n, k, x, norm_weight, norm_eps, residual, y, stream)


def qmv_q4_0_ex(qs, d, n, k, x, norm_weight=None, norm_eps=1e-6, residual=None, y=None, stream=None):
    return _qmv_ex("gq_qmv_q4_0_ex", TYPE_Q4_0, qs, d, n, k, x, norm_weight, norm_eps, residual, y, stream)


def _qmv_ex(fn, qtype, qs, d, n, k, x, norm_weight, norm_eps, residual, y, stream):
    torch = _torch()
    if y is None:
        y = _like(x, (n,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call(fn, *_weights(qtype, qs, d, n, k), n, k, _ptr(x, "x", "f32", k_),
          _ptr(norm_weight, "norm_weight", "f32", k_), float(norm_eps), _ptr(residual, "residual", "f32", n_),
          _ptr(y, "y", "f32", n_), _stream(stream))
    return y


def argmax_workspace_bytes() -> int:
    return raw().gq_argmax_workspace_bytes()


def _qmv_argmax(fn, qtype, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits, workspace, index, value,
                stream):
    torch = _torch()
    if logits is None:
        logits = _like(x, (n,), torch.float32)
    if workspace is None:
        workspace = _like(x, (argmax_workspace_bytes(),), torch.uint8)
    if index is None:
        index = _like(x, (1,), torch.int32)
    if value is None:
        value = _like(x, (1,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call(fn, *_weights(qtype, qs, d, n, k), n, k, _ptr(x, "x", "f32", k_),
          _ptr(norm_weight, "norm_weight", "f32", k_), float(norm_eps), float(softcap),
          _ptr(logits, "logits", "f32", n_), _ptr(workspace, "workspace", "bytes", argmax_workspace_bytes()),
          workspace.numel() * workspace.element_size(), _ptr(index, "index", "i32", 1),
          _ptr(value, "value", "f32", 1), _stream(stream))
    return index, value, logits


def qmv_q8_0_argmax(qs, d, n, k, x, norm_weight=None, norm_eps=1e-6, softcap=30.0, logits=None,
                    workspace=None, index=None, value=None, stream=None):
    """Vocabulary head: returns (index int32[1], value fp32[1], logits fp32[n])."""
    return _qmv_argmax("gq_qmv_q8_0_argmax", TYPE_Q8_0, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits,
                       workspace, index, value, stream)


def qmv_q4_0_argmax(qs, d, n, k, x, norm_weight=None, norm_eps=1e-6, softcap=30.0, logits=None,
                    workspace=None, index=None, value=None, stream=None):
    return _qmv_argmax("gq_qmv_q4_0_argmax", TYPE_Q4_0, qs, d, n, k, x, norm_weight, norm_eps, softcap, logits,
                       workspace, index, value, stream)


def qmv_q8_0_argmax_noalloc(qs, d, n, k, x, norm_weight=None, norm_eps=1e-6, softcap=30.0, logits=None,
                            index=None, value=None, stream=None):
    """The vocabulary head without a workspace (library-held device scratch;
    calls overlapping on one device race). Returns (index, value, logits)."""
    torch = _torch()
    if logits is None:
        logits = _like(x, (n,), torch.float32)
    if index is None:
        index = _like(x, (1,), torch.int32)
    if value is None:
        value = _like(x, (1,), torch.float32)
    n_, k_, _ = _dims(n, k)
    _call("gq_qmv_q8_0_argmax_noalloc", *_weights(TYPE_Q8_0, qs, d, n, k), n, k, _ptr(x, "x", "f32", k_),
          _ptr(norm_weight, "norm_weight", "f32", k_), float(norm_eps), float(softcap),
          _ptr(logits, "logits", "f32", n_), _ptr(index, "index", "i32", 1), _ptr(value, "value", "f32", 1),
          _stream(stream))
    return index, value, logits


def kq_packed_bytes(qtype: int, n: int, k: int) -> int:
    return raw().gq_kq_packed_bytes(qtype, n, k)


def _kq_dims(n, k):
    n, k = int(n), int(k)
    return (n, k) if n >= 1 and k >= 256 and k % 256 == 0 else (0, 0)


def kq_pack(qtype, blocks, n, k, packed=None, stream=None):
    """GGUF Q4_K / Q5_K / Q6_K super-blocks (device uint8) -> one packed uint8 buffer."""
    torch = _torch()
    n_, k_ = _kq_dims(n, k)
    need = kq_packed_bytes(qtype, n_, k_) if n_ else 0
    if packed is None:
        packed = _like(blocks, (max(need, 1),), torch.uint8)
    _call("gq_kq_pack", qtype, _ptr(blocks, "blocks", "bytes", n_ * (k_ // 256) * block_bytes(qtype)), n, k,
          _ptr(packed, "packed", "bytes", need), _stream(stream))
    return packed


def _qmv_kq(fn, qtype, packed, n, k, x, y, stream):
    torch = _torch()
    if y is None:
        y = _like(x, (n,), torch.float32)
    n_, k_ = _kq_dims(n, k)
    need = kq_packed_bytes(qtype, n_, k_) if n_ else 0
    _call(fn, _ptr(packed, "packed", "bytes", need), n, k, _ptr(x, "x", "f32", k_), _ptr(y, "y", "f32", n_),
          _stream(stream))
    return y


def qmv_q4_k(packed, n, k, x, y=None, stream=None):
    return _qmv_kq("gq_qmv_q4_k", TYPE_Q4_K, packed, n, k, x, y, stream)


def qmv_q5_k(packed, n, k, x, y=None, stream=None):
    return _qmv_kq("gq_qmv_q5_k", TYPE_Q5_K, packed, n, k, x, y, stream)


def qmv_q6_k(packed, n, k, x, y=None, stream=None):
    return _qmv_kq("gq_qmv_q6_k", TYPE_Q6_K, packed, n, k, x, y, stream)


def _ffn_weights(g_qs, g_d, u_qs, u_d, n_ff, k):
    return (*_weights(TYPE_Q4_0, g_qs, g_d, n_ff, k, ("g_qs", "g_d")),
            *_weights(TYPE_Q4_0, u_qs, u_d, n_ff, k, ("u_qs", "u_d")))


def qffn_gate_up_gelu_ex(g_qs, g_d, u_qs, u_d, n_ff, k, x, norm_weight=None, norm_eps=1e-6, h=None,
                         stream=None):
    torch = _torch()
    if h is None:
        h = _like(x, (n_ff,), torch.float32)
    n_, k_, _ = _dims(n_ff, k)
    _call("gq_qffn_gate_up_gelu_ex", *_ffn_weights(g_qs, g_d, u_qs, u_d, n_ff, k), n_ff, k,
          _ptr(x, "x", "f32", k_), _ptr(norm_weight, "norm_weight", "f32", k_), float(norm_eps),
          _ptr(h, "h", "f32", n_), _stream(stream))
    return h


def qffn_gate_up_gelu(g_qs, g_d, u_qs, u_d, n_ff, k, x, h=None, stream=None):
    torch = _torch()
    if h is None:
        h = _like(x, (n_ff,), torch.float32)
    n_, k_, _ = _dims(n_ff, k)
    _call("gq_qffn_gate_up_gelu", *_ffn_weights(g_qs, g_d, u_qs, u_d, n_ff, k), n_ff, k,
          _ptr(x, "x", "f32", k_), _ptr(h, "h", "f32", n_), _stream(stream))
    return h


def qmm_tile_m(qs, d, n, k, m, xq, xd, y=None, blockdots=None, stream=None):
    torch = _torch()
    if y is None:
        y = _like(xq, (m, n), torch.float32)
    n_, k_, m_ = _dims(n, k, m) if 1 <= int(m) <= 32 else (0, 0, 0)
    _call("gq_qmm_tile_m", *_weights(TYPE_Q4_0, qs, d, n_, k_), n, k, m, _ptr(xq, "xq", "i8", m_ * k_),
          _ptr(xd, "xd", "h16", m_ * _nb(k_)), _ptr(y, "y", "f32", m_ * n_),
          _ptr(blockdots, "blockdots", "i32", m_ * n_ * _nb(k_)), _stream(stream))
    return y


class Chain:
    """A recorded decode step (gq_chain_*). Launches issued on ``stream``
    inside ``with chain:`` are recorded rather than run; ``launch()`` then
    replays the whole sequence as one graph. The stream must not be the
    legacy default stream. Outputs must be allocated before recording and
    kept alive (and their pointers unchanged) for as long as the chain is
    replayed; update inputs in place between replays."""

    def __init__(self, stream=None):
        torch = _torch()
        self._stream_obj = stream if stream is not None else torch.cuda.current_stream()
        self._handle = ctypes.c_void_p()
        self._recording = False

    def __enter__(self):
        _call("gq_chain_begin", _stream(self._stream_obj))
        self._recording = True
        return self

    def __exit__(self, exc_type, exc, tb):
        self._recording = False
        st = raw().gq_chain_end(_stream(self._stream_obj), ctypes.byref(self._handle))
        if st != GQ_OK and exc_type is None:
            raise GQError(st, "gq_chain_end")
        return False

    @property
    def launches(self) -> int:
        return raw().gq_chain_launches(self._handle)

    def launch(self, stream=None):
        if not self._handle:
            raise RuntimeError("chain has not been recorded")
        _call("gq_chain_launch", self._handle, _stream(stream if stream is not None else self._stream_obj))

    def close(self):
        if self._handle:
            h, self._handle = self._handle, ctypes.c_void_p()
            _call("gq_chain_destroy", h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
