"""GPU parity: every libgq entry point against the fp64 oracle on the same
seeded inputs. Integer results (packed bytes, quantised codes and scales,
per-block int32 dot sums) must match bit for bit; fp32 results must satisfy
|y - y_ref| <= 1e-4 * sum|w x| + 1e-6 (the method's accuracy contract).
Inputs are canonical GGUF block bytes from ``synth``; the oracle reads those
bytes, the library packs them with its own kernel."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_within, down, packed, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_block_quant_amd as gq  # noqa: E402

Q4, Q8 = gq.TYPE_Q4_0, gq.TYPE_Q8_0


def _qmv(qtype):
    return gq.qmv_q8_0 if qtype == Q8 else gq.qmv_q4_0


def _qmv8(qtype):
    return gq.qmv_q8_0_q8 if qtype == Q8 else gq.qmv_q4_0_q8


# ----------------------------------------------------------------------------
# pack
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("qtype,n,k", [(Q8, 64, 256), (Q4, 33, 96), (Q4, 2048, 2048), (Q8, 7, 32)])
def test_pack_moves_bytes_exactly(qtype, n, k):
    w = synth.weights(np.random.default_rng(1), qtype, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(down(qs).view(np.uint8).reshape(n, -1),
                          np.ascontiguousarray(w["qs"]).view(np.uint8).reshape(n, -1))
    assert np.array_equal(down(d, np.uint16), w["d"])


def test_pack_unaligned_source():
    n, k = 5, 64
    w = synth.q8_0_weights(np.random.default_rng(2), n, k)
    raw = synth.as_bytes(w).reshape(-1)
    buf = up(np.concatenate([np.zeros(3, np.uint8), raw]))
    qs, d = gq.pack(Q8, buf[3:], n, k)
    assert np.array_equal(down(qs).view(np.int8), w["qs"].reshape(n, k))
    assert np.array_equal(down(d, np.uint16), w["d"])


# ----------------------------------------------------------------------------
# fp32-activation matvec
# ----------------------------------------------------------------------------

SHAPES = [
    (Q8, 64, 256),       # the small Q8_0 workload
    (Q4, 2048, 2048),    # the 2048 x 2048 Q4_0 workload
    (Q8, 32768, 2048),   # one GPU's rows of the vocab head split 8 ways
    (Q8, 8192, 2048), (Q8, 8195, 2048),      # 16 MiB of quants: four rows per step (ragged)
    (Q4, 16384, 2048), (Q4, 12288, 2048),    # ... Q4_0 at and below that size
    (Q8, 1, 32), (Q4, 1, 32),                # smallest legal shape
    (Q8, 1001, 96), (Q4, 1001, 160),         # ragged rows, partial wave of units
    (Q8, 300, 1056), (Q4, 300, 3040),        # K not a multiple of a wave's span
    (Q8, 515, 2048), (Q4, 515, 4096),        # K split over 2 waves
    (Q8, 257, 8192), (Q4, 2048, 8192),       # the FFN down-projection width
    (Q8, 64, 32768), (Q4, 64, 32768),        # the maximum K (16-wave split)
    (Q4, 5, 8192), (Q4, 1001, 8192),         # 4-wave split, two row groups per workgroup, ragged
    (Q4, 77, 16384), (Q8, 45, 16384),        # 8-wave split (16-wave workgroups), ragged
]


@pytest.mark.parametrize("qtype,n,k", SHAPES)
def test_qmv_f32(qtype, n, k):
    rng = np.random.default_rng(n * 7 + k)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    qs, d = packed(gq, qtype, w, n, k)
    y = down(_qmv(qtype)(qs, d, n, k, up(x)))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(y, yr, oracle.fp32_path_bound(ar), "qmv type %d %dx%d" % (qtype, n, k))


@pytest.mark.parametrize("qtype", [Q8, Q4])
def test_qmv_exact_power_of_two_case(qtype):
    """Power-of-two scales and small integer activations make every partial
    sum exact in fp32, so the GPU must equal the oracle bit for bit."""
    rng = np.random.default_rng(5)
    n, k = 300, 2048
    w = synth.weights(rng, qtype, n, k)
    e = rng.integers(-10, -6, size=w["d"].shape)
    w["d"] = ((2.0 ** e) * rng.choice([-1.0, 1.0], size=e.shape)).astype(np.float16).view(np.uint16)
    x = rng.integers(-2, 3, size=k).astype(np.float32)
    qs, d = packed(gq, qtype, w, n, k)
    y = down(_qmv(qtype)(qs, d, n, k, up(x)))
    yr, _ = oracle.matvec(qtype, w, n, k, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("qtype", [Q8, Q4])
def test_qmv_one_hot_layout(qtype):
    """x = e_c selects column c: y[r] must equal the dequantised weight w[r][c]
    exactly, for every c of a 2-block row (pins element order and scales)."""
    rng = np.random.default_rng(8)
    n, k = 16, 64
    w = synth.weights(rng, qtype, n, k)
    W = oracle.dequantize(qtype, w, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    X = np.eye(k, dtype=np.float32)
    for c in range(k):
        y = down(_qmv(qtype)(qs, d, n, k, up(X[c])))
        assert np.array_equal(y.astype(np.float64), W[:, c]), c


@pytest.mark.parametrize("qtype", [Q8, Q4])
def test_qmv_large_and_nan_activations(qtype):
    rng = np.random.default_rng(6)
    n, k = 128, 1024
    w = synth.weights(rng, qtype, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    x = (synth.activations(rng, k) * np.float32(1e20)).astype(np.float32)
    y = down(_qmv(qtype)(qs, d, n, k, up(x)))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(y, yr, oracle.fp32_path_bound(ar), "large x")
    x[17] = np.nan
    y = down(_qmv(qtype)(qs, d, n, k, up(x)))
    yr, _ = oracle.matvec(qtype, w, n, k, x)
    assert np.array_equal(np.isnan(y), np.isnan(yr))


@pytest.mark.parametrize("qtype", [Q8, Q4])
def test_qmv_deterministic(qtype):
    rng = np.random.default_rng(9)
    n, k = 4096, 2048
    w = synth.weights(rng, qtype, n, k)
    x = up(synth.activations(rng, k))
    qs, d = packed(gq, qtype, w, n, k)
    a = down(_qmv(qtype)(qs, d, n, k, x))
    b = down(_qmv(qtype)(qs, d, n, k, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_qmv_vocab_full_size_sampled():
    """The Q8_0 vocab projection (262144 x 2048) at full size, as launched by
    the benchmark; the oracle checks 4096 sampled rows plus both ends."""
    wl = synth.workload_vocab()
    n, k, w, x = wl["n"], wl["k"], wl["w"], wl["x"]
    qs, d = packed(gq, Q8, w, n, k)
    y = down(gq.qmv_q8_0(qs, d, n, k, up(x)))
    rows = np.unique(np.concatenate([np.random.default_rng(0).integers(0, n, 4096), [0, 1, n - 2, n - 1]]))
    yr, ar = oracle.matvec_rows(Q8, w, n, k, rows, x)
    check_within(y[rows], yr, oracle.fp32_path_bound(ar), "vocab")
    assert np.all(np.isfinite(y))


# ----------------------------------------------------------------------------
# Q8_0 activation quantiser and the integer path
# ----------------------------------------------------------------------------

def test_quantize_bit_exact():
    rng = np.random.default_rng(10)
    x = synth.activations(rng, (8, 2048))
    x[1] *= np.float32(1e-3)
    x[2] *= np.float32(1e3)
    x[3, :32] = 0
    x[3, 32:64] = np.linspace(-1, 1, 32, dtype=np.float32)
    x[4, :32] = np.float32(1e-9)
    x[4, 32:40] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]
    x[4, 40:64] = 0
    x[5, :32] = np.float32(2e7)
    x[5, 0] = np.float32(-3e7)
    x[6] = rng.uniform(-1, 1, 2048).astype(np.float32) * (10.0 ** rng.integers(-6, 6, 2048)).astype(np.float32)
    xq, xd = gq.quantize_q8_0(up(x))
    rq, rd = oracle.quantize_q8_0(x)
    assert np.array_equal(down(xq), rq)
    assert np.array_equal(down(xd, np.uint16), rd)
    # the 2048-wide workload activation, as a single row
    x1 = synth.workload_q4_0_2048()["x"]
    xq, xd = gq.quantize_q8_0(up(x1))
    rq, rd = oracle.quantize_q8_0(x1)
    assert np.array_equal(down(xq), rq.reshape(-1)) and np.array_equal(down(xd, np.uint16), rd.reshape(-1))


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (5, 1056), (33, 8192), (1, 32768), (257, 64)])
def test_quantize_ragged_shapes(m, k):
    """Block counts that leave part of the last workgroup (and wave) idle."""
    rng = np.random.default_rng(m * 7 + k)
    x = synth.activations(rng, (m, k)) * np.float32(rng.uniform(0.01, 100.0))
    xq, xd = gq.quantize_q8_0(up(x))
    rq, rd = oracle.quantize_q8_0(x)
    assert np.array_equal(down(xq), rq)
    assert np.array_equal(down(xd, np.uint16), rd)


INT_SHAPES = [(Q4, 2048, 2048), (Q8, 64, 256), (Q4, 1, 32), (Q8, 1, 32), (Q4, 999, 96),
              (Q8, 16384, 2048), (Q8, 16387, 2048), (Q4, 32768, 2048), (Q8, 8192, 2048),   # 32 MiB crossover
              (Q8, 777, 1056), (Q4, 300, 8192), (Q8, 300, 8192), (Q4, 33, 32768), (Q4, 77, 16384),
              (Q8, 5, 16384)]


def _qmv8x(qtype):
    return gq.qmv_q8_0_q8x if qtype == Q8 else gq.qmv_q4_0_q8x


@pytest.mark.parametrize("qtype,n,k", INT_SHAPES)
def test_qmv_q8x_equals_quantise_then_q8(qtype, n, k):
    """The fused quantiser prologue gives the standalone quantiser's codes and
    the same block dots and outputs bit for bit, and matches the oracle."""
    rng = np.random.default_rng(3 * n + k)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k) * np.float32(rng.uniform(0.1, 10.0))
    qs, d = packed(gq, qtype, w, n, k)
    xg = up(x)
    xq, xd = gq.quantize_q8_0(xg)
    bd_ref = torch.empty((n, k // 32), dtype=torch.int32, device="cuda")
    y_ref = down(_qmv8(qtype)(qs, d, n, k, xq, xd, blockdots=bd_ref))
    bd = torch.full((n, k // 32), 7, dtype=torch.int32, device="cuda")
    xq_out = torch.full((k,), 99, dtype=torch.int8, device="cuda")
    xd_out = torch.zeros((k // 32,), dtype=torch.int16, device="cuda")
    y = down(_qmv8x(qtype)(qs, d, n, k, xg, blockdots=bd, xq_out=xq_out, xd_out=xd_out))
    assert np.array_equal(down(xq_out), down(xq)) and np.array_equal(down(xd_out), down(xd))
    assert np.array_equal(down(bd), down(bd_ref))
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
    # without the optional outputs
    y2 = down(_qmv8x(qtype)(qs, d, n, k, xg))
    assert np.array_equal(y2.view(np.uint32), y_ref.view(np.uint32))
    rq, rd = oracle.quantize_q8_0(x)
    S, yr, ar = oracle.blockdots(qtype, w, n, k, rq, rd)
    assert np.array_equal(down(bd), S[0])
    check_within(y, yr[0], oracle.fp32_path_bound(ar[0]), "fused int path")


@pytest.mark.parametrize("qtype,n,k", INT_SHAPES)
def test_qmv_q8_block_dots_exact(qtype, n, k):
    rng = np.random.default_rng(n + k)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    qs, d = packed(gq, qtype, w, n, k)
    xq, xd = gq.quantize_q8_0(up(x))
    bd = torch.full((n, k // 32), 123456789, dtype=torch.int32, device="cuda")
    y = down(_qmv8(qtype)(qs, d, n, k, xq, xd, blockdots=bd))
    rq, rd = oracle.quantize_q8_0(x)
    S, yr, ar = oracle.blockdots(qtype, w, n, k, rq, rd)
    assert np.array_equal(down(bd), S[0])
    check_within(y, yr[0], oracle.fp32_path_bound(ar[0]), "int path")
    # without the block-dot output the result is the same
    y2 = down(_qmv8(qtype)(qs, d, n, k, xq, xd))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_qmv_q8_extreme_codes():
    """Q8_0 weights of -128 against codes of -127: the largest block sum."""
    n, k = 4, 64
    w = np.zeros((n, k // 32), dtype=synth.Q8_0_BLOCK)
    w["qs"] = -128
    w["d"] = 0x3C00
    xq = np.full(k, -127, np.int8)
    xd = np.full(k // 32, 0x3C00, np.uint16)
    qs, d = packed(gq, Q8, w, n, k)
    bd = torch.empty((n, k // 32), dtype=torch.int32, device="cuda")
    y = down(gq.qmv_q8_0_q8(qs, d, n, k, up(xq), up(xd), blockdots=bd))
    assert np.all(down(bd) == 32 * 128 * 127)
    assert np.all(y == 2 * 32 * 128 * 127)


# ----------------------------------------------------------------------------
# fused gate+up GELU FFN, then the down projection
# ----------------------------------------------------------------------------

def _ffn_case(n_ff, k, seed):
    wl = synth.workload_ffn(seed=seed, n_ff=n_ff, k=k)
    g = packed(gq, Q4, wl["wg"], n_ff, k)
    u = packed(gq, Q4, wl["wu"], n_ff, k)
    dn = packed(gq, Q4, wl["wd"], k, n_ff)
    x = wl["x"]
    h = gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x))
    y = gq.qmv_q4_0(dn[0], dn[1], k, n_ff, h)
    return wl, down(h), down(y)


@pytest.mark.parametrize("n_ff,k", [(8192, 2048), (1024, 2048),   # the FFN; one GPU's share of 8
                                    (1056, 96), (64, 32), (224, 8192), (96, 16384)])
def test_ffn_stage_by_stage(n_ff, k):
    wl, h, y = _ffn_case(n_ff, k, seed=0)
    ref = oracle.ffn_gate_up(Q4, wl["wg"], wl["wu"], n_ff, k, wl["x"])
    # (i) h against the fp64 h with the propagated bound
    check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]), "h")
    # (ii) down projection of the GPU's own h
    yr, ar = oracle.matvec(Q4, wl["wd"], k, n_ff, h)
    check_within(y, yr, oracle.fp32_path_bound(ar), "down(h_gpu)")
    # (iii) end to end against W_d h_ref
    hb = oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"])
    Wd = np.abs(oracle.dequantize(Q4, wl["wd"], k, n_ff))
    ye, ae = oracle.matvec(Q4, wl["wd"], k, n_ff, ref["h"])
    check_within(y, ye, Wd @ hb + oracle.fp32_path_bound(ae), "end to end")


@pytest.mark.parametrize("n_ff,k", [(1001, 2048), (77, 8192), (45, 16384), (3, 32768), (65539, 2048)])
def test_ffn_gate_up_ragged_rows(n_ff, k):
    """Gate+up alone at row counts that leave row groups (and, for split
    rows, the second row group of a workgroup) partly or wholly past the end;
    65539 rows take the tall shape (four row pairs per wave step, their gate
    and up sums reduced as two transposed sets of four)."""
    rng = np.random.default_rng(n_ff + k)
    wg = synth.q4_0_weights(rng, n_ff, k)
    wu = synth.q4_0_weights(rng, n_ff, k)
    x = synth.activations(rng, k)
    g = packed(gq, Q4, wg, n_ff, k)
    u = packed(gq, Q4, wu, n_ff, k)
    h = down(gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x)))
    ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, x)
    check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]), "h")


def test_ffn_gelu_on_exact_inputs():
    """One nonzero weight per row with power-of-two scales makes g and u
    exact on the GPU, isolating the GELU epilogue. Includes the pages'
    large-gate regression (gate = up = 30 -> 900)."""
    n_ff, k = 64, 64
    rng = np.random.default_rng(12)
    x = np.zeros(k, np.float32)
    x[:32] = (np.round(rng.standard_normal(32) * 256) / 256).astype(np.float32)  # <= 11 bits: products exact
    x[5] = 3.0
    wg = np.zeros((n_ff, 2), dtype=synth.Q4_0_BLOCK)
    wu = np.zeros((n_ff, 2), dtype=synth.Q4_0_BLOCK)
    wg["qs"] = 0x88
    wu["qs"] = 0x88
    wg["d"] = 0x4000          # 2.0
    wu["d"] = 0x4000
    for r in range(n_ff):
        j = (r * 7) % 16
        if r == 0:
            wg["qs"][r, 0, 5] = 0x80 | 13       # element 5: 2 * (13 - 8) * 3 = 30
            wu["qs"][r, 0, 5] = 0x80 | 13
            continue
        wg["qs"][r, 0, j] = 0x80 | (r % 16)
        wu["qs"][r, 0, (j + 3) % 16] = 0x80 | ((r * 5) % 16)
    g = packed(gq, Q4, wg, n_ff, k)
    u = packed(gq, Q4, wu, n_ff, k)
    h = down(gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x))).astype(np.float64)
    ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, x)
    assert h[0] == 900.0
    gz = np.sqrt(2 / np.pi) * (ref["g"] + 0.044715 * ref["g"] ** 3)
    bound = np.abs(ref["h"]) * (8.0 + 10.0 * np.abs(gz)) * 2.0 ** -24 + 1e-30
    check_within(h, ref["h"], bound, "gelu epilogue")


def test_ffn_large_gate_no_nan():
    n_ff, k = 16, 32
    wg = np.zeros((n_ff, 1), dtype=synth.Q4_0_BLOCK)
    wg["qs"] = 0xFF
    wg["d"] = (np.linspace(-30000, 30000, n_ff) / 7 / 32).astype(np.float16).view(np.uint16).reshape(n_ff, 1)
    wu = wg.copy()
    x = np.ones(k, np.float32)
    g = packed(gq, Q4, wg, n_ff, k)
    u = packed(gq, Q4, wu, n_ff, k)
    h = down(gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x)))
    assert np.all(np.isfinite(h))
    ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, x)
    check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]), "big g")


# ----------------------------------------------------------------------------
# small-M prefill tile
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("m", [8, 16, 32, 4])
def test_tile_workload(m):
    """The prefill workload at full size (M = 4 is the batched-decode launch:
    the first four rows of the M = 8 activations)."""
    wl = synth.workload_tile()
    n, k, w = wl["n"], wl["k"], wl["w"]
    xq, xd = wl["acts"][m] if m in wl["acts"] else (wl["acts"][8][0][:m].copy(), wl["acts"][8][1][:m].copy())
    qs, d = packed(gq, Q4, w, n, k)
    bd = torch.full((m, n, k // 32), -7, dtype=torch.int32, device="cuda")
    y = down(gq.qmm_tile_m(qs, d, n, k, m, up(xq), up(xd), blockdots=bd))
    S, yr, ar = oracle.blockdots(Q4, w, n, k, xq, xd)
    assert np.array_equal(down(bd), S)
    check_within(y, yr, oracle.fp32_path_bound(ar), "tile m=%d" % m)
    # each tile row agrees with the M = 1 integer path on that row
    y1 = down(gq.qmv_q4_0_q8(qs, d, n, k, up(xq[m - 1]), up(xd[m - 1])))
    check_within(y[m - 1], yr[m - 1], oracle.fp32_path_bound(ar[m - 1]), "tile last row")
    check_within(y1, yr[m - 1], oracle.fp32_path_bound(ar[m - 1]), "m=1 path on last row")


@pytest.mark.parametrize("m,n,k", [(8, 1000, 96), (16, 17, 32), (32, 100, 1056), (32, 64, 8192),
                                   (1, 300, 2048), (2, 513, 512), (3, 64, 96), (5, 129, 1024),
                                   (7, 2048, 2048), (12, 80, 256), (20, 48, 320), (31, 33, 4096),
                                   (24, 40, 544), (17, 16, 32768)])
def test_tile_ragged(m, n, k):
    rng = np.random.default_rng(m * n + k)
    w = synth.q4_0_weights(rng, n, k)
    xq, xd = synth.q8_0_activations(rng, m, k)
    qs, d = packed(gq, Q4, w, n, k)
    bd = torch.empty((m, n, k // 32), dtype=torch.int32, device="cuda")
    y = down(gq.qmm_tile_m(qs, d, n, k, m, up(xq), up(xd), blockdots=bd))
    S, yr, ar = oracle.blockdots(Q4, w, n, k, xq, xd)
    assert np.array_equal(down(bd), S)
    check_within(y, yr, oracle.fp32_path_bound(ar), "tile ragged")


def test_tile_deterministic_and_blockdots_optional():
    wl = synth.workload_tile(n=2048, k=2048, ms=(32,))
    xq, xd = wl["acts"][32]
    qs, d = packed(gq, Q4, wl["w"], 2048, 2048)
    a = down(gq.qmm_tile_m(qs, d, 2048, 2048, 32, up(xq), up(xd)))
    b = down(gq.qmm_tile_m(qs, d, 2048, 2048, 32, up(xq), up(xd),
                           blockdots=torch.empty((32, 2048, 64), dtype=torch.int32, device="cuda")))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ----------------------------------------------------------------------------
# binding-level argument errors on real device tensors (nothing launched)
# ----------------------------------------------------------------------------

def test_binding_rejects_misaligned_and_host_tensors():
    n, k = 64, 256
    w = synth.q8_0_weights(np.random.default_rng(0), n, k)
    qs, d = packed(gq, Q8, w, n, k)
    x = torch.zeros(k + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(gq.GQError) as e:
        gq.qmv_q8_0(qs, d, n, k, x[1:])
    assert e.value.status == 3
    with pytest.raises(ValueError):
        gq.qmv_q8_0(qs, d, n, k, torch.zeros(k))
    with pytest.raises(gq.GQError) as e:
        gq.qmm_tile_m(qs, d, n, k, 33, torch.zeros((33, k), dtype=torch.int8, device="cuda"),
                      torch.zeros((33, k // 32), dtype=torch.int16, device="cuda"))
    assert e.value.status == 5
