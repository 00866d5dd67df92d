"""The C-ABI library on the host, no GPU needed: it loads, exports every
symbol include/gq.h declares, reports sizes, and rejects every invalid
argument combination with the documented status before any HIP call (so no
kernel is ever launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gq.h")

gq = pytest.importorskip("gguf_block_quant_amd")

OK, NULL, SHAPE, ALIGN, ALIAS, UNSUP, VALUE = 0, 1, 2, 3, 4, 5, 7
Q4, Q8 = 2, 8

# Fake, never-dereferenced addresses: every call below fails validation first.
A = 0x10000000          # 256-byte aligned "buffers", far apart
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(gq_\w+)\s*\(", text, re.M)))


def test_header_symbols_all_exported():
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(gq.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    # the binding wraps exactly the declared set
    assert set(names) == set(gq._SIGS)


def test_version_and_status_strings():
    assert gq.abi_version() == 7
    for s in range(8):
        assert gq.status_str(s)
    assert gq.status_str(99) == "unknown status"


def test_sizes():
    assert gq.block_bytes(Q8) == 34 and gq.block_bytes(Q4) == 18 and gq.block_bytes(3) == 0
    assert gq.packed_qs_bytes(Q8, 64, 256) == 64 * 256
    assert gq.packed_qs_bytes(Q4, 2048, 2048) == 2048 * 1024
    assert gq.packed_d_bytes(2048, 2048) == 2048 * 64 * 2
    # packed bytes equal the GGUF block bytes
    assert gq.packed_qs_bytes(Q4, 10, 64) + gq.packed_d_bytes(10, 64) == 10 * 2 * 18
    assert gq.packed_qs_bytes(Q8, 10, 64) + gq.packed_d_bytes(10, 64) == 10 * 2 * 34
    assert gq.packed_qs_bytes(Q8, 10, 33) == 0 and gq.packed_d_bytes(0, 64) == 0


L = gq.raw()  # loads libgq.so


def qmv(fn, qs=A, d=B, n=64, k=256, x=C, y=D):
    return getattr(L, fn)(qs, d, n, k, x, y, None)


@pytest.mark.parametrize("fn", ["gq_qmv_q8_0", "gq_qmv_q4_0"])
def test_qmv_validation(fn):
    assert qmv(fn, qs=None) == NULL
    assert qmv(fn, d=None) == NULL
    assert qmv(fn, x=None) == NULL
    assert qmv(fn, y=None) == NULL
    assert qmv(fn, n=0) == SHAPE
    assert qmv(fn, k=0) == SHAPE
    assert qmv(fn, k=48) == SHAPE
    assert qmv(fn, k=-32) == SHAPE
    assert qmv(fn, k=65536) == UNSUP
    assert qmv(fn, n=(1 << 30) + 1) == UNSUP
    assert qmv(fn, qs=A + 8) == ALIGN
    assert qmv(fn, d=B + 1) == ALIGN
    assert qmv(fn, x=C + 4) == ALIGN
    assert qmv(fn, y=D + 2) == ALIGN
    assert qmv(fn, y=A) == ALIAS              # output over the quants
    assert qmv(fn, y=B + 64) == ALIAS         # output inside the scales
    assert qmv(fn, y=C - 128) == ALIAS        # output running into x


@pytest.mark.parametrize("fn", ["gq_qmv_q8_0_q8", "gq_qmv_q4_0_q8"])
def test_qmv_q8_validation(fn):
    f = getattr(L, fn)
    assert f(A, B, 64, 256, C, None, D, None, None) == NULL
    assert f(A, B, 64, 250, C, E, D, None, None) == SHAPE
    assert f(A, B, 64, 256, C + 8, E, D, None, None) == ALIGN
    assert f(A, B, 64, 256, C, E, D, D + 2, None) == ALIGN
    assert f(A, B, 64, 256, C, E, D, D + 128, None) == ALIAS      # blockdots over y
    assert f(A, B, 64, 256, C, E, D, A + 1024, None) == ALIAS     # blockdots over qs


@pytest.mark.parametrize("fn", ["gq_qmv_q8_0_q8x", "gq_qmv_q4_0_q8x"])
def test_qmv_q8x_validation(fn):
    """(qs, d, n, k, x, xq_out, xd_out, y, blockdots, stream)"""
    f = getattr(L, fn)
    assert f(A, B, 64, 256, None, None, None, D, None, None) == NULL
    assert f(A, B, 64, 256, C, None, None, None, None, None) == NULL
    assert f(A, B, 64, 256, C, E, None, D, None, None) == NULL             # codes out without scales out
    assert f(A, B, 64, 256, C, None, E, D, None, None) == NULL
    assert f(A, B, 64, 250, C, None, None, D, None, None) == SHAPE
    assert f(A, B, 64, 65536, C, None, None, D, None, None) == UNSUP
    assert f(A, B, 64, 256, C + 4, None, None, D, None, None) == ALIGN     # x 16 B
    assert f(A, B, 64, 256, C, E + 8, E + 4096, D, None, None) == ALIGN    # codes out 16 B
    assert f(A, B, 64, 256, C, E, E + 4097, D, None, None) == ALIGN        # scales out 2 B
    assert f(A, B, 64, 256, C, None, None, C + 512, None, None) == ALIAS   # y over x
    assert f(A, B, 64, 256, C, C, E, D, None, None) == ALIAS               # codes out over x
    assert f(A, B, 64, 256, C, E, D, D, None, None) == ALIAS               # scales out over y
    assert f(A, B, 64, 256, C, None, None, D, D + 64, None) == ALIAS       # blockdots over y


def test_ffn_validation():
    f = L.gq_qffn_gate_up_gelu
    assert f(A, B, None, B, 64, 256, C, D, None) == NULL
    assert f(A, B, A, B, 64, 100, C, D, None) == SHAPE
    assert f(A, B, A + 4, B, 64, 256, C, D, None) == ALIGN
    assert f(A, B, C, B, 64, 256, E, B, None) == ALIAS
    assert f(A, B, C, E, 64, 65536, C, D, None) == UNSUP


def test_tile_validation():
    f = L.gq_qmm_tile_m
    assert f(A, B, 64, 256, 0, C, E, D, None, None) == UNSUP
    assert f(A, B, 64, 256, 33, C, E, D, None, None) == UNSUP
    assert f(A, B, 64, 256, -8, C, E, D, None, None) == UNSUP
    assert f(A, B, 64, 256, 16, C, None, D, None, None) == NULL
    assert f(A, B, 64, 0, 16, C, E, D, None, None) == SHAPE
    assert f(A, B, 64, 256, 16, C + 1, E, D, None, None) == ALIGN
    assert f(A, B, 64, 256, 16, C, E, D, D + 4 * 512, None) == ALIAS   # blockdots inside y


def test_pack_and_quantize_validation():
    assert L.gq_pack(3, A, 64, 256, B, C, None) == UNSUP
    assert L.gq_pack(Q8, A, 64, 256, B + 8, C, None) == ALIGN
    assert L.gq_pack(Q8, A, 64, 256, A + 34 * 16, C, None) == ALIAS
    assert L.gq_pack(Q8, None, 64, 256, B, C, None) == NULL
    assert L.gq_quantize_q8_0(A, 2, 100, B, C, None) == SHAPE
    assert L.gq_quantize_q8_0(A + 4, 2, 128, B, C, None) == ALIGN
    assert L.gq_quantize_q8_0(A, 2, 128, A + 16, C, None) == ALIAS


@pytest.mark.parametrize("fn", ["gq_qmv_q8_0_ex", "gq_qmv_q4_0_ex"])
def test_qmv_ex_validation(fn):
    f = getattr(L, fn)
    NW = 0x60000000
    # (qs, d, n, k, x, norm_w, eps, residual, y, stream)
    assert f(A, B, 64, 256, C, NW + 4, 1e-6, None, D, None) == ALIGN      # norm weight 16-B
    assert f(A, B, 64, 256, C, NW, -1.0, None, D, None) == VALUE           # negative eps
    assert f(A, B, 64, 256, C, NW, float("nan"), None, D, None) == VALUE
    assert f(A, B, 64, 256, C, NW, float("inf"), None, D, None) == VALUE
    assert f(A, B, 64, 256, C, None, 1e-6, E + 2, D, None) == ALIGN        # residual 4-B
    assert f(A, B, 64, 256, C, None, 0.0, D + 8, D, None) == ALIAS         # residual overlaps y
    assert f(A, B, 64, 256, C, NW, 1e-6, None, NW + 64, None) == ALIAS     # y over the norm weight
    assert f(A, B, 64, 250, C, NW, 1e-6, None, D, None) == SHAPE


@pytest.mark.parametrize("fn", ["gq_qmv_q8_0_argmax", "gq_qmv_q4_0_argmax"])
def test_argmax_validation(fn):
    f = getattr(L, fn)
    W, I, V = 0x70000000, 0x71000000, 0x72000000
    ws = gq.argmax_workspace_bytes()
    assert ws >= 8 * 1024
    # (qs, d, n, k, x, norm_w, eps, softcap, logits, ws, ws_bytes, index, value, stream)
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, None, ws, I, V, None) == NULL
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, W, ws, None, V, None) == NULL
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, W, ws - 8, I, V, None) == VALUE
    assert f(A, B, 64, 256, C, None, 0.0, -1.0, D, W, ws, I, V, None) == VALUE
    assert f(A, B, 64, 256, C, None, 0.0, float("nan"), D, W, ws, I, V, None) == VALUE
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, W + 4, ws, I, V, None) == ALIGN
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, D + 64, ws, I, V, None) == ALIAS   # workspace over logits
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, W, ws, W + 16, V, None) == ALIAS   # index inside workspace


def test_argmax_noalloc_validation():
    """The allocation-free vocabulary head validates like the workspace one
    (no workspace argument to check)."""
    f = L.gq_qmv_q8_0_argmax_noalloc
    I, V = 0x71000000, 0x72000000
    # (qs, d, n, k, x, norm_w, eps, softcap, logits, index, value, stream)
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, None, I, V, None) == NULL
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, None, V, None) == NULL
    assert f(A, B, 64, 250, C, None, 0.0, 30.0, D, I, V, None) == SHAPE
    assert f(A, B, 64, 65536, C, None, 0.0, 30.0, D, I, V, None) == UNSUP
    assert f(A, B, 64, 256, C, None, 0.0, -1.0, D, I, V, None) == VALUE
    assert f(A, B, 64, 256, C + 4, None, 0.0, 30.0, D, I, V, None) == ALIGN
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, I + 2, V, None) == ALIGN
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, D, D + 16, V, None) == ALIAS     # index over logits
    assert f(A, B, 64, 256, C, None, 0.0, 30.0, C, I, V, None) == ALIAS          # logits over x


def test_kquant_validation():
    """K-quant entry points: whole 256-element super-blocks, k <= 32768."""
    Q4K, Q5K, Q6K = 12, 13, 14
    assert gq.block_bytes(Q4K) == 144 and gq.block_bytes(Q5K) == 176 and gq.block_bytes(Q6K) == 210
    assert gq.kq_packed_bytes(Q4K, 4, 256) == 512 + 4 * 16          # quants, then 16-byte headers
    assert gq.kq_packed_bytes(Q5K, 4, 256) == 512 + 256 + 4 * 32    # + headers padded to 256, fifth-bit words
    assert gq.kq_packed_bytes(Q6K, 4, 256) == 512 + 256 + 256 + 8   # ql, qh, scales (padded to 256), d
    assert gq.kq_packed_bytes(Q4K, 4, 288) == 0 and gq.kq_packed_bytes(Q4_0 := 2, 4, 256) == 0
    for fn in (L.gq_qmv_q4_k, L.gq_qmv_q5_k, L.gq_qmv_q6_k):
        assert fn(None, 4, 256, C, D, None) == NULL
        assert fn(A, 4, 256, None, D, None) == NULL
        assert fn(A, 4, 288, C, D, None) == SHAPE
        assert fn(A, 0, 256, C, D, None) == SHAPE
        assert fn(A, 4, 128, C, D, None) == SHAPE
        assert fn(A, 4, 65536, C, D, None) == UNSUP
        assert fn(A + 8, 4, 256, C, D, None) == ALIGN
        assert fn(A, 4, 256, C + 4, D, None) == ALIGN
        assert fn(A, 4, 256, C, A + 64, None) == ALIAS                       # y inside the packed weights
    f = L.gq_kq_pack
    assert f(Q4K, None, 4, 256, A, None) == NULL
    assert f(2, B, 4, 256, A, None) == UNSUP
    assert f(Q6K, B, 4, 300, A, None) == SHAPE
    assert f(Q6K, B, 4, 256, A + 8, None) == ALIGN
    assert f(Q6K, B, 4, 256, B + 16, None) == ALIAS
    assert f(Q5K, B, 4, 256, B + 16, None) == ALIAS
    assert f(15, B, 4, 256, A, None) == UNSUP                                # Q8_K: not a weight format here


def test_ffn_ex_validation():
    f = L.gq_qffn_gate_up_gelu_ex
    NW = 0x60000000
    assert f(A, B, C, E, 64, 256, D, NW, -1e-6, 0x61000000, None) == VALUE
    assert f(A, B, C, E, 64, 256, D, NW + 8, 1e-6, 0x61000000, None) == ALIGN
    assert f(A, B, C, E, 64, 256, D, NW, 1e-6, NW + 128, None) == ALIAS


def test_chain_validation():
    """Decode-step chaining: argument checks that precede any HIP call."""
    h = ctypes.c_void_p()
    assert L.gq_chain_begin(None) == VALUE                 # the legacy stream cannot be recorded
    assert L.gq_chain_end(None, ctypes.byref(h)) == VALUE
    assert L.gq_chain_end(ctypes.c_void_p(A), None) == NULL
    assert L.gq_chain_launch(None, ctypes.c_void_p(A)) == NULL
    assert L.gq_chain_destroy(None) == OK                  # like free(NULL)
    assert L.gq_chain_launches(None) == 0


def test_product_path_never_loads_the_oracle():
    """The binding and the library are the product: importing the binding
    and loading libgq pull in nothing from oracle/ (a fresh interpreter)."""
    import subprocess
    import sys
    code = ("import sys, gguf_block_quant_amd as gq; gq.raw(); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad; "
            "libs = open('/proc/self/maps').read(); "
            "assert 'liboracle' not in libs and 'oracle.so' not in libs")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
