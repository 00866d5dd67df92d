"""GPU parity of the K-quant path (Q4_K, Q5_K, Q6_K super-blocks of 256 elements):
the load-time pack lays out every byte as specified, and the fp32-activation matvec
matches the fp64 oracle (which reads the canonical GGUF super-block bytes)
within |y - y_ref| <= 1e-4 sum|w x| + 1e-6 at every dispatch shape, bit for
bit on one-hot and exact-arithmetic inputs, with special scale values, and
reproducibly."""
import numpy as np
import pytest

import oracle
import synth
import kq_layout_model as kq_model
from gpu_util import check_special, check_within, down, packed_kq, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_block_quant_amd as gq  # noqa: E402

Q4K, Q5K, Q6K = gq.TYPE_Q4_K, gq.TYPE_Q5_K, gq.TYPE_Q6_K
KQ = [Q4K, Q5K, Q6K]


def _fn(qtype):
    return {Q4K: gq.qmv_q4_k, Q5K: gq.qmv_q5_k, Q6K: gq.qmv_q6_k}[qtype]


@pytest.mark.parametrize("qtype,n,k", [(Q4K, 7, 256), (Q4K, 33, 2048), (Q5K, 7, 256), (Q5K, 33, 2304),
                                       (Q6K, 7, 256), (Q6K, 33, 4352)])
def test_kq_pack_lays_out_every_byte(qtype, n, k):
    # the packed sections are the layout's lossless rearrangement of the GGUF
    # bits (modelled on the host; the model is pinned by test_kq_layout.py)
    w = synth.weights(np.random.default_rng(n + k), qtype, n, k)
    p = down(packed_kq(gq, qtype, w, n, k))
    assert p.size >= gq.kq_packed_bytes(qtype, n, k)
    nsb = k // 256
    r256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    if qtype in (Q4K, Q5K):
        qs = p[: n * k // 2].reshape(n, nsb, 128)
        o1 = r256(n * k // 2)
        hdr = p[o1: o1 + n * nsb * 16].reshape(n, nsb, 16)
        assert np.array_equal(qs, w["qs"])
        assert np.array_equal(hdr, kq_model.q4_k_header(w))
        if qtype == Q5K:
            o2 = o1 + r256(n * nsb * 16)
            assert p.size == o2 + n * k // 8
            assert np.array_equal(p[o2: o2 + n * k // 8].copy().view("<u4").reshape(n, nsb, 8),
                                  kq_model.q5_k_fifth_words(w))
    else:
        o1 = r256(n * k // 2)
        o2 = o1 + r256(n * k // 4)
        o3 = o2 + r256(n * k // 16)
        assert np.array_equal(p[: n * k // 2].reshape(n, nsb, 128), w["ql"])
        assert np.array_equal(p[o1: o1 + n * k // 4].copy().view("<u4").reshape(n, nsb, 8, 2),
                              kq_model.q6_k_high_words(w))
        assert np.array_equal(p[o2: o2 + n * k // 16].view(np.int8).reshape(n, nsb, 8, 2),
                              kq_model.q6_k_unit_scales(w))
        assert np.array_equal(p[o3: o3 + n * nsb * 2].view(np.uint16).reshape(n, nsb), w["d"])


# shapes: one wave per row (k <= 2048; k = 256 uses 8 lanes), rows split over
# 2, 4, 8 and 16 waves (a last partial wave), ragged row counts (two rows per
# wave step), the 2048 x 2048 and 8192 x 2048 decode shapes
SHAPES = [(2048, 2048), (8192, 2048), (1, 256), (3, 768), (1001, 1536), (515, 2304), (300, 4096),
          (77, 8192), (45, 11776), (64, 16384), (17, 32768), (4096, 2048), (4099, 1792)]


@pytest.mark.parametrize("qtype", KQ)
@pytest.mark.parametrize("n,k", SHAPES)
def test_qmv_kq(qtype, n, k):
    rng = np.random.default_rng(3 * n + k + qtype)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    p = packed_kq(gq, qtype, w, n, k)
    y = down(_fn(qtype)(p, n, k, up(x)))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(y, yr, oracle.fp32_path_bound(ar), "type %d %dx%d" % (qtype, n, k))


@pytest.mark.parametrize("qtype", KQ)
def test_qmv_kq_one_hot_layout(qtype):
    """x = e_c selects column c: y[r] must be the dequantised weight w[r][c]
    rounded once to fp32, for every c of a two-super-block row."""
    rng = np.random.default_rng(40 + qtype)
    n, k = 24, 512
    w = synth.weights(rng, qtype, n, k)
    W = oracle.dequantize(qtype, w, n, k)
    p = packed_kq(gq, qtype, w, n, k)
    X = np.eye(k, dtype=np.float32)
    for c in range(k):
        y = down(_fn(qtype)(p, n, k, up(X[c])))
        assert np.array_equal(y, W[:, c].astype(np.float32)), c


@pytest.mark.parametrize("qtype", KQ)
def test_qmv_kq_exact_power_of_two_case(qtype):
    """Power-of-two super-block scales and small integer activations keep
    every partial sum exact in fp32: the GPU must equal the oracle bitwise."""
    rng = np.random.default_rng(50 + qtype)
    n, k = 300, 2048
    w = synth.weights(rng, qtype, n, k)
    pw = lambda shape: (2.0 ** rng.integers(-10, -6, size=shape)).astype(np.float16).view(np.uint16)  # noqa: E731
    w["d"] = pw(w["d"].shape)
    if qtype in (Q4K, Q5K):
        w["dmin"] = pw(w["dmin"].shape)
    x = rng.integers(-2, 3, size=k).astype(np.float32)
    p = packed_kq(gq, qtype, w, n, k)
    y = down(_fn(qtype)(p, n, k, up(x)))
    yr, _ = oracle.matvec(qtype, w, n, k, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("qtype", KQ)
@pytest.mark.parametrize("n,k", [(2048, 2048), (77, 8192), (17, 32768)])
def test_qmv_kq_special_scales(qtype, n, k):
    rng = np.random.default_rng(60 + n + qtype)
    w = synth.weights(rng, qtype, n, k)
    fields = ["d", "dmin"] if qtype in (Q4K, Q5K) else ["d"]
    finite = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x8200, 0x7BFF, 0xFBFF], np.uint16)
    for f in fields:
        mask = rng.random(w[f].shape) < 0.1
        w[f][mask] = rng.choice(finite, size=int(mask.sum()))
    nonfinite = [0x7C00, 0xFC00, 0x7E00, 0xFE01]
    for r in range(0, n, 5):
        w[fields[r % len(fields)]][r, rng.integers(0, k // 256)] = nonfinite[r % 4]
    x = synth.activations(rng, k)
    p = packed_kq(gq, qtype, w, n, k)
    y = down(_fn(qtype)(p, n, k, up(x)))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    assert (~np.isfinite(yr)).sum() > 0
    check_special(y, yr, ar, "type %d %dx%d special" % (qtype, n, k))


@pytest.mark.parametrize("qtype", KQ)
def test_qmv_kq_deterministic_and_large_x(qtype):
    rng = np.random.default_rng(70 + qtype)
    n, k = 4096, 4096
    w = synth.weights(rng, qtype, n, k)
    p = packed_kq(gq, qtype, w, n, k)
    x = (synth.activations(rng, k) * np.float32(1e20)).astype(np.float32)
    y1 = down(_fn(qtype)(p, n, k, up(x)))
    y2 = down(_fn(qtype)(p, n, k, up(x)))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(y1, yr, oracle.fp32_path_bound(ar), "large x")


@pytest.mark.parametrize("qtype", KQ)
@pytest.mark.parametrize("scale", [1e-30, 1e-36])
def test_qmv_kq_tiny_x(qtype, scale):
    """Activations near the bottom of the fp32 range (products below 2^-126
    at 1e-36): the contract still holds and nothing turns non-finite."""
    rng = np.random.default_rng(80 + qtype)
    n, k = 512, 2048
    w = synth.weights(rng, qtype, n, k)
    p = packed_kq(gq, qtype, w, n, k)
    x = (synth.activations(rng, k).astype(np.float64) * scale).astype(np.float32)
    y = down(_fn(qtype)(p, n, k, up(x)))
    assert np.isfinite(y).all()
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(y, yr, oracle.fp32_path_bound(ar), "tiny x %g" % scale)


@pytest.mark.parametrize("qtype", KQ)
def test_qmv_kq_full_size_sampled_rows(qtype):
    """The tall launch shape the benchmark times (262144 x 2048, each wave
    walking many row groups), plus a ragged 3-row tail: sampled rows -- the
    first and last groups, both sides of every 4-row group boundary in a
    stretch, and random rows -- against the oracle row by row."""
    rng = np.random.default_rng(90 + qtype)
    n, k = 262147, 2048
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    p = packed_kq(gq, qtype, w, n, k)
    y = down(_fn(qtype)(p, n, k, up(x)))
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(n - 16, n), np.arange(131064, 131080),
                                     rng.integers(0, n, 200)]))
    yr, ar = oracle.matvec_rows(qtype, w, n, k, rows, x)
    check_within(y[rows], yr, oracle.fp32_path_bound(ar), "type %d full size" % qtype)
    assert np.isfinite(y).all()


def test_kq_binding_errors():
    x = torch.zeros(256, dtype=torch.float32, device="cuda")
    p = torch.zeros(gq.kq_packed_bytes(Q4K, 4, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(gq.GQError):
        gq.qmv_q4_k(p, 4, 288, torch.zeros(288, dtype=torch.float32, device="cuda"))   # not whole super-blocks
    with pytest.raises(ValueError):
        gq.qmv_q4_k(p[:-1], 4, 256, x)
    assert gq.kq_packed_bytes(Q4K, 4, 288) == 0 and gq.kq_packed_bytes(2, 4, 256) == 0
