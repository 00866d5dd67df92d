"""Pins for the fp64 oracle: each test checks the oracle against something
other than itself -- a value printed on the pages, a closed form, an
invariant, a library routine the case reduces to, or exact brute force on a
tiny input -- so that a dropped term, a wrong sign, a swapped nibble or a
transposed index fails at least one of them. CPU only."""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import synth


# ----------------------------------------------------------------------------
# binary16 decode / encode against numpy's float16 (a library routine)
# ----------------------------------------------------------------------------

def test_fp16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.fp16_to_f64_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, oracle.fp16_to_f64(0x8000)) == -1.0


def _enc_ref(vals32):
    with np.errstate(over="ignore"):
        return vals32.astype(np.float16).view(np.uint16)


def test_fp16_encode_rounding_midpoints_vs_numpy():
    """Every positive finite half, the fp32 midpoints between neighbouring
    halves (exact ties) and the fp32 values one ulp either side of them."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mid = ((v + nxt) / 2).astype(np.float32)          # exact: 12 significant bits
    assert np.array_equal(mid.astype(np.float64), (v + nxt) / 2)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    cand = np.concatenate([v.astype(np.float32), mid, below, above])
    cand = np.concatenate([cand, -cand])
    ref = _enc_ref(cand)
    f = oracle.lib().or_f32_to_fp16_rne
    got = np.array([f(float(c)) for c in cand], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (cand[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_fp16_encode_random_bits_vs_numpy():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # bias half the sample into the binary16 range, where rounding decides
    small = (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-9, 5, 100_000)).astype(np.float32)
    cand = np.concatenate([vals, small, np.array([65504, 65519.996, 65520, 1e-8, 2.0**-25,
                                                  3 * 2.0**-26, 0.0], np.float32)])
    ref = _enc_ref(cand)
    f = oracle.lib().or_f32_to_fp16_rne
    got = np.array([f(float(c)) for c in cand], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# Block layout: one-hot probes on hand-built blocks
# ----------------------------------------------------------------------------

ONE = 0x3C00   # binary16 1.0
TWO = 0x4000   # binary16 2.0


def _q8_block(d_bits, qs):
    b = bytearray([d_bits & 0xFF, d_bits >> 8])
    b += bytes(np.asarray(qs, dtype=np.int8).view(np.uint8))
    assert len(b) == 34
    return b


def _q4_block(d_bits, lo, hi):
    """lo[j] -> low nibble of quant byte j, hi[j] -> its high nibble."""
    b = bytearray([d_bits & 0xFF, d_bits >> 8])
    b += bytes(((int(h) & 15) << 4) | (int(l) & 15) for l, h in zip(lo, hi))
    assert len(b) == 18
    return b


def _rows(blocks_bytes_per_row):
    return np.frombuffer(b"".join(bytes(b) for row in blocks_bytes_per_row for b in row),
                         dtype=np.uint8)


def test_block_geometry_matches_pages(golden):
    g = golden("block_geometry.txt")
    assert oracle.lib().or_block_bytes(oracle.TYPE_Q4_0) == int(g["q4_0_bytes"])
    assert oracle.lib().or_block_bytes(oracle.TYPE_Q8_0) == int(g["q8_0_bytes"])
    assert synth.Q4_0_BLOCK.itemsize == int(g["q4_0_bytes"])
    assert synth.Q8_0_BLOCK.itemsize == int(g["q8_0_bytes"])


def test_one_hot_q8_0_layout():
    # row 0: q_i = i - 16 with d = 1; row 1: q_i = 3*(15 - i) clipped, d = 2
    k = 64
    r0 = [_q8_block(ONE, [i - 16 for i in range(32)]), _q8_block(ONE, [i + 40 for i in range(32)])]
    r1 = [_q8_block(TWO, [max(-127, 3 * (15 - i)) for i in range(32)]),
          _q8_block(TWO, [-(i + 1) for i in range(32)])]
    blocks = _rows([r0, r1])
    expect = np.zeros((2, k))
    expect[0, :32] = [i - 16 for i in range(32)]
    expect[0, 32:] = [i + 40 for i in range(32)]
    expect[1, :32] = [2 * max(-127, 3 * (15 - i)) for i in range(32)]
    expect[1, 32:] = [-2 * (i + 1) for i in range(32)]
    for kk in range(k):
        x = np.zeros(k)
        x[kk] = 1.0
        y, a = oracle.matvec(oracle.TYPE_Q8_0, blocks, 2, k, x)
        assert y[0] == expect[0, kk] and y[1] == expect[1, kk], kk
        assert np.array_equal(a, np.abs(expect[:, kk]))


def test_one_hot_q4_0_layout():
    # row 0: low nibble of byte j = j, high nibble = 15 - j   (d = 1)
    #   -> element j = j - 8, element j + 16 = 7 - j
    # row 1: low = (3j) mod 16, high = (5j + 1) mod 16       (d = 2)
    k = 32
    lo0, hi0 = list(range(16)), [15 - j for j in range(16)]
    lo1, hi1 = [(3 * j) % 16 for j in range(16)], [(5 * j + 1) % 16 for j in range(16)]
    blocks = _rows([[_q4_block(ONE, lo0, hi0)], [_q4_block(TWO, lo1, hi1)]])
    e0 = [j - 8 for j in range(16)] + [7 - j for j in range(16)]
    e1 = [2 * (l - 8) for l in lo1] + [2 * (h - 8) for h in hi1]
    for kk in range(k):
        x = np.zeros(k)
        x[kk] = 1.0
        y, _ = oracle.matvec(oracle.TYPE_Q4_0, blocks, 2, k, x)
        assert y[0] == e0[kk] and y[1] == e1[kk], kk


def test_every_nibble_at_every_position_brute_force():
    """16 structured patterns: nibble at position i is (i + p) mod 16."""
    for p in range(16):
        lo = [(j + p) % 16 for j in range(16)]
        hi = [(j + 16 + p) % 16 for j in range(16)]
        blocks = _rows([[_q4_block(ONE, lo, hi)]])
        w = oracle.dequantize(oracle.TYPE_Q4_0, blocks, 1, 32)
        assert list(w[0]) == [float(((i + p) % 16) - 8) for i in range(32)]


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("k", [32, 256, 2048])
def test_closed_form_q4_0_all_eight_is_zero(k):
    nb = k // 32
    blocks = _rows([[_q4_block(0x2E66, [8] * 16, [8] * 16) for _ in range(nb)]])
    x = np.random.default_rng(0).standard_normal(k)
    y, a = oracle.matvec(oracle.TYPE_Q4_0, blocks, 1, k, x)
    assert y[0] == 0.0 and a[0] == 0.0


@pytest.mark.parametrize("k", [32, 64, 8192])
def test_closed_form_q4_0_fifteen_ones(k):
    nb = k // 32
    blocks = _rows([[_q4_block(ONE, [15] * 16, [15] * 16) for _ in range(nb)]])
    y, a = oracle.matvec(oracle.TYPE_Q4_0, blocks, 1, k, np.ones(k))
    assert y[0] == 7.0 * k and a[0] == 7.0 * k


def test_closed_form_q8_0_constant():
    k = 512
    half = 0x3800  # binary16 0.5
    blocks = _rows([[_q8_block(half, [1] * 32) for _ in range(k // 32)],
                    [_q8_block(half, [-127] * 32) for _ in range(k // 32)]])
    y, _ = oracle.matvec(oracle.TYPE_Q8_0, blocks, 2, k, np.ones(k))
    assert y[0] == k / 2 and y[1] == -127 * k / 2
    # alternating x cancels exactly
    x = np.tile([1.0, -1.0], k // 2)
    y, a = oracle.matvec(oracle.TYPE_Q8_0, blocks, 2, k, x)
    assert y[0] == 0.0 and a[0] == k / 2


# ----------------------------------------------------------------------------
# Exact arithmetic brute force (Python integers / Fractions) on small inputs
# ----------------------------------------------------------------------------

def _decode_fraction(qtype, blk):
    """Independent decode of one block into exact Fractions."""
    blk = [int(v) for v in blk]
    d_bits = blk[0] | (blk[1] << 8)
    e = (d_bits >> 10) & 31
    m = d_bits & 1023
    assert e not in (0, 31)
    d = Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))
    if d_bits >> 15:
        d = -d
    if qtype == oracle.TYPE_Q8_0:
        q = [b - 256 if b > 127 else b for b in blk[2:34]]
    else:
        q = [(blk[2 + j] & 15) - 8 for j in range(16)] + [(blk[2 + j] >> 4) - 8 for j in range(16)]
    return [d * qi for qi in q]


@pytest.mark.parametrize("qtype", [oracle.TYPE_Q8_0, oracle.TYPE_Q4_0])
def test_exact_power_of_two_scales_and_integer_x(qtype):
    rng = np.random.default_rng(7)
    n, k = 3, 96
    w = synth.weights(rng, qtype, n, k)
    # power-of-two scales 2^-7 .. 2^-10, random signs
    exps = rng.integers(-10, -6, size=w["d"].shape)
    d = (2.0 ** exps) * rng.choice([-1.0, 1.0], size=exps.shape)
    w["d"] = d.astype(np.float16).view(np.uint16)
    x = rng.integers(-2, 3, size=k).astype(np.float64)
    raw = synth.as_bytes(w)
    bb = oracle.lib().or_block_bytes(qtype)
    y, a = oracle.matvec(qtype, w, n, k, x)
    for r in range(n):
        exact = Fraction(0)
        aexact = Fraction(0)
        for b in range(k // 32):
            vals = _decode_fraction(qtype, raw[r, b * bb:(b + 1) * bb])
            for i, v in enumerate(vals):
                exact += v * int(x[b * 32 + i])
                aexact += abs(v * int(x[b * 32 + i]))
        assert Fraction(y[r]) == exact
        assert Fraction(a[r]) == aexact


@pytest.mark.parametrize("qtype", [oracle.TYPE_Q8_0, oracle.TYPE_Q4_0])
def test_random_rows_within_fp64_rounding_of_exact(qtype):
    rng = np.random.default_rng(11)
    n, k = 2, 64
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    raw = synth.as_bytes(w)
    bb = oracle.lib().or_block_bytes(qtype)
    y, a = oracle.matvec(qtype, w, n, k, x)
    for r in range(n):
        exact = sum(v * Fraction(float(x[b * 32 + i]))
                    for b in range(k // 32)
                    for i, v in enumerate(_decode_fraction(qtype, raw[r, b * bb:(b + 1) * bb])))
        assert abs(Fraction(y[r]) - exact) <= Fraction(k * 2.0**-52) * Fraction(a[r])


# ----------------------------------------------------------------------------
# A second, independent decode (numpy, vectorised) as a library cross-check
# ----------------------------------------------------------------------------

def _numpy_dequant(qtype, blocks):
    d = blocks["d"].view(np.float16).astype(np.float64)
    if qtype == oracle.TYPE_Q8_0:
        q = blocks["qs"].astype(np.float64)
    else:
        qs = blocks["qs"]
        q = np.concatenate([(qs & 15), (qs >> 4)], axis=-1).astype(np.float64) - 8.0
    return (d[..., None] * q).reshape(blocks.shape[0], -1)


@pytest.mark.parametrize("qtype,n,k", [(oracle.TYPE_Q8_0, 64, 256), (oracle.TYPE_Q4_0, 40, 2048),
                                       (oracle.TYPE_Q4_0, 5, 8192)])
def test_numpy_decode_and_matmul_agree(qtype, n, k):
    rng = np.random.default_rng(3)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    W = _numpy_dequant(qtype, w)
    assert np.array_equal(oracle.dequantize(qtype, w, n, k), W)
    y, a = oracle.matvec(qtype, w, n, k, x)
    yr = W @ x.astype(np.float64)
    assert np.all(np.abs(y - yr) <= 1e-12 * np.abs(W * x).sum(axis=1))
    assert np.allclose(a, np.abs(W * x).sum(axis=1), rtol=1e-12, atol=0)
    ys, as_ = oracle.matvec_rows(qtype, w, n, k, [n - 1, 0], x)
    assert ys[0] == y[n - 1] and ys[1] == y[0] and as_[0] == a[n - 1]


# ----------------------------------------------------------------------------
# Q8_0 activation quantiser
# ----------------------------------------------------------------------------

def _numpy_quantize(x):
    """Same steps as the reading of the quantiser, written with numpy float32
    operations and an explicit half-away-from-zero rounding in float64."""
    x = np.asarray(x, np.float32).reshape(-1, 32)
    amax = np.abs(x).max(axis=1)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / d32[:, None]).astype(np.float64)
    r = np.trunc(v + np.copysign(0.5, v))
    r = np.where(d32[:, None] == 0, 0.0, np.clip(r, -127, 127))
    return r.astype(np.int8).reshape(-1), d16.view(np.uint16)


def test_quantizer_matches_numpy_and_bounds():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 2048)).astype(np.float32)
    x[0] *= 1e-3
    x[1] *= 300.0
    x[2, :32] = 0.0
    xq, xd = oracle.quantize_q8_0(x)
    rq, rd = _numpy_quantize(x)
    assert np.array_equal(xd.reshape(-1), rd)
    assert np.array_equal(xq.reshape(-1), rq)
    d = xd.view(np.float16).astype(np.float64)
    deq = xq.astype(np.float64).reshape(6, -1, 32) * d[..., None]
    err = np.abs(deq - x.astype(np.float64).reshape(6, -1, 32))
    assert np.all(err <= d[..., None] / 2)                      # |x - q d| <= d/2
    assert np.all(np.abs(xq.astype(int)) <= 127)
    # the block absolute maximum maps to +-127
    xb = x.reshape(6, -1, 32)
    idx = np.abs(xb).argmax(axis=2)
    qmax = np.take_along_axis(xq.reshape(6, -1, 32).astype(int), idx[..., None], axis=2)[..., 0]
    nz = d > 0
    assert np.all(np.abs(qmax[nz]) == 127)
    assert np.all(xq.reshape(6, -1, 32)[2, 0] == 0) and xd[2, 0] == 0


def test_quantizer_crafted_blocks():
    blocks = []
    blocks.append(np.zeros(32))                                  # all zero
    b = np.zeros(32); b[5] = -3.25; blocks.append(b)             # single nonzero
    b = np.linspace(-1, 1, 32); b[31] = 4.0; blocks.append(b)    # amax last
    b = np.tile([0.7, -0.7], 16); blocks.append(b)               # symmetric
    b = np.arange(32) - 15.5; blocks.append(b)                   # half-integers
    b = np.full(32, 1e-9); blocks.append(b)                      # scale underflows to 0
    b = np.full(32, 2e7); b[0] = -3e7; blocks.append(b)          # scale overflows fp16
    b = np.zeros(32); b[:8] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]
    blocks.append(b)                                             # d = 1: exact ties
    x = np.concatenate(blocks).astype(np.float32)
    xq, xd = oracle.quantize_q8_0(x)
    rq, rd = _numpy_quantize(x)
    assert np.array_equal(xq.reshape(-1), rq) and np.array_equal(xd.reshape(-1), rd)
    q = xq.reshape(-1, 32)
    assert np.all(q[0] == 0) and xd[0, 0] == 0
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1
    assert q[2, 31] == 127
    assert np.all(q[3] == np.tile([127, -127], 16))
    assert np.all(q[4] == -q[4][::-1])                           # odd symmetry
    assert xd[0, 5] == 0 and np.all(q[5] == 0)
    assert xd[0, 6] == 0x7C00 and np.all(q[6] == 0)              # d = inf -> codes 0
    assert xd[0, 7] == 0x3C00                                    # ties round away from 0
    assert list(q[7, :8]) == [127, 3, -3, 1, -1, 2, -2, 127]


def test_quantizer_no_ties_at_seed0_workload():
    """Ties of x/d at half-integers have measure zero for normal x: count the
    elements whose x/d lies within 1e-6 of a half-integer at the 2048-wide
    workload activation and expect none (so rounding mode choice is moot)."""
    wl = synth.workload_q4_0_2048()
    x = wl["x"].reshape(-1, 32)
    xq, xd = oracle.quantize_q8_0(wl["x"])
    d = xd.view(np.float16).astype(np.float32).reshape(-1)
    v = (x / d[:, None]).astype(np.float64)
    frac = np.abs(v - np.floor(v) - 0.5)
    assert np.count_nonzero(frac < 1e-6) == 0


# ----------------------------------------------------------------------------
# Integer path
# ----------------------------------------------------------------------------

def test_int_product_table_brute_force():
    """Every weight nibble 0..15 against every activation code -127..127 at
    one position of a Q4_0 block (all other positions zero)."""
    for nib in range(16):
        lo = [8] * 16
        lo[3] = nib
        blocks = _rows([[_q4_block(ONE, lo, [8] * 16)]])
        xq = np.zeros((255, 32), np.int8)
        xq[:, 3] = np.arange(-127, 128)
        xd = np.full((255, 1), ONE, np.uint16)
        S, y, _ = oracle.blockdots(oracle.TYPE_Q4_0, blocks, 1, 32, xq, xd)
        assert np.array_equal(S[:, 0, 0], (nib - 8) * np.arange(-127, 128))
        assert np.array_equal(y[:, 0], (nib - 8) * np.arange(-127, 128).astype(float))


@pytest.mark.parametrize("qtype", [oracle.TYPE_Q8_0, oracle.TYPE_Q4_0])
def test_blockdots_brute_force_small(qtype):
    rng = np.random.default_rng(9)
    n, k, m = 3, 96, 4
    w = synth.weights(rng, qtype, n, k)
    xq, xd = synth.q8_0_activations(rng, m, k)
    raw = synth.as_bytes(w)
    bb = oracle.lib().or_block_bytes(qtype)
    S, y, a = oracle.blockdots(qtype, w, n, k, xq, xd)
    for mi in range(m):
        for r in range(n):
            tot = Fraction(0)
            for b in range(k // 32):
                blk = raw[r, b * bb:(b + 1) * bb]
                dw = _decode_fraction(qtype, blk)          # d * q
                d_bits = int(blk[0]) | (int(blk[1]) << 8)
                dwf = Fraction(float(np.uint16(d_bits).view(np.float16)))
                qw = [v / dwf for v in dw]
                s = sum(int(q) * int(xq[mi, b * 32 + i]) for i, q in enumerate(qw))
                assert S[mi, r, b] == s
                tot += dwf * Fraction(float(np.uint16(xd[mi, b]).view(np.float16))) * s
            assert abs(Fraction(y[mi, r]) - tot) <= Fraction(2.0**-50) * Fraction(a[mi, r])


def test_blockdots_closed_form_sum_of_codes():
    """Q4_0 weights with every nibble 9 (q - 8 = 1) and d = 1: S_b = sum of
    the activation codes of block b."""
    rng = np.random.default_rng(2)
    k = 256
    blocks = _rows([[_q4_block(ONE, [9] * 16, [9] * 16) for _ in range(k // 32)]])
    xq, xd = synth.q8_0_activations(rng, 2, k)
    S, _, _ = oracle.blockdots(oracle.TYPE_Q4_0, blocks, 1, k, xq, xd)
    assert np.array_equal(S[:, 0, :], xq.reshape(2, -1, 32).astype(np.int64).sum(axis=2))


def test_blockdots_q8_0_extreme_fits_int32():
    k = 32
    blocks = _rows([[_q8_block(ONE, [-128] * 32)]])
    xq = np.full((1, 32), -127, np.int8)
    xd = np.full((1, 1), ONE, np.uint16)
    S, y, _ = oracle.blockdots(oracle.TYPE_Q8_0, blocks, 1, k, xq, xd)
    assert S[0, 0, 0] == 32 * 128 * 127 and y[0, 0] == 32 * 128 * 127


# ----------------------------------------------------------------------------
# GELU (tanh form) and the gated FFN
# ----------------------------------------------------------------------------

def test_gelu_page_regression_value(golden):
    g = golden("gelu_large_gate.txt")
    gate, up, h = float(g["gate"]), float(g["up"]), float(g["h"])
    assert oracle.gelu_tanh(gate) * up == h


def test_gelu_against_torch_tanh_gelu():
    torch = pytest.importorskip("torch")
    t = np.concatenate([np.linspace(-12, 12, 4001), [-1.0, 1.0, 0.5, 3.0, 1e-8, -1e-8]])
    ref = torch.nn.functional.gelu(torch.from_numpy(t), approximate="tanh").numpy()
    got = oracle.gelu_tanh_array(t)
    # 1 + tanh(z) cancels for negative t, so both sides carry an absolute
    # error of a few ulp of |t| there; elsewhere they agree to 1e-14 relative
    assert np.all(np.abs(got - ref) <= 1e-14 * np.abs(ref) + 4e-16 * np.abs(t))


def test_gelu_invariants():
    t = np.concatenate([np.linspace(-50, 50, 2001), [1e-3, 1e3, 1e4, -1e4]])
    G = oracle.gelu_tanh_array(t)
    Gm = oracle.gelu_tanh_array(-t)
    assert np.all(np.isfinite(G))
    # G(t) - G(-t) = t for the tanh form (tanh is odd)
    assert np.allclose(G - Gm, t, rtol=1e-15, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(40.0) == 40.0
    neg = oracle.gelu_tanh(-30.0)
    assert neg == 0.0 and math.copysign(1.0, neg) == -1.0
    # Lipschitz constant used by the FFN bound
    tt = np.linspace(-10, 10, 200001)
    GG = oracle.gelu_tanh_array(tt)
    slope = np.abs(np.diff(GG) / np.diff(tt)).max()
    assert 1.12 < slope <= oracle.GELU_LIPSCHITZ


def test_ffn_gate_up_one_hot_rows():
    """Gate row r and up row r each have one nonzero weight, so g and u are
    single products and h = G(g) u can be checked against torch's GELU."""
    torch = pytest.importorskip("torch")
    n_ff, k = 16, 64
    rng = np.random.default_rng(4)
    gb, ub = [], []
    gvals, uvals = [], []
    x = synth.activations(rng, k).astype(np.float64)
    for r in range(n_ff):
        pos_g, pos_u = (3 * r) % k, (5 * r + 1) % k
        rows_g, rows_u = [], []
        for b in range(k // 32):
            lo, hi = [8] * 16, [8] * 16
            if pos_g // 32 == b:
                j = pos_g % 32
                (lo if j < 16 else hi)[j % 16] = r % 16
            rows_g.append(_q4_block(TWO, lo, hi))
            lo, hi = [8] * 16, [8] * 16
            if pos_u // 32 == b:
                j = pos_u % 32
                (lo if j < 16 else hi)[j % 16] = 15 - r % 16
            rows_u.append(_q4_block(ONE, lo, hi))
        gb.append(rows_g)
        ub.append(rows_u)
        gvals.append(2.0 * ((r % 16) - 8) * x[pos_g])
        uvals.append(1.0 * ((15 - r % 16) - 8) * x[pos_u])
    out = oracle.ffn_gate_up(oracle.TYPE_Q4_0, _rows(gb), _rows(ub), n_ff, k, x)
    assert np.array_equal(out["g"], gvals) and np.array_equal(out["u"], uvals)
    ref = torch.nn.functional.gelu(torch.tensor(gvals, dtype=torch.float64), approximate="tanh").numpy()
    assert np.allclose(out["h"], ref * np.array(uvals), rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------
# RMSNorm prologue, soft cap and argmax epilogue
# ----------------------------------------------------------------------------

def test_rmsnorm_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    for k in (32, 2048, 8192):
        x = rng.standard_normal(k) * 3.0
        w = rng.uniform(0.5, 1.5, k)
        got = oracle.rmsnorm(x, w, 1e-6)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (k,), torch.from_numpy(w), eps=1e-6).numpy()
        assert np.allclose(got, ref, rtol=1e-14, atol=0)


def test_rmsnorm_closed_forms():
    # constant input c: every output is c / sqrt(c^2 + eps) (times w)
    for c in (1.0, -2.5, 1e-4):
        got = oracle.rmsnorm(np.full(64, c), None, 1e-6)
        assert np.allclose(got, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    # eps = 0: the output has mean square exactly 1 and is scale invariant
    rng = np.random.default_rng(22)
    x = rng.standard_normal(256)
    a = oracle.rmsnorm(x, None, 0.0)
    b = oracle.rmsnorm(8.0 * x, None, 0.0)
    assert abs(np.mean(a * a) - 1.0) < 1e-14 and np.allclose(a, b, rtol=1e-15)
    # the weight multiplies directly (no 1 + w)
    w = np.zeros(256)
    w[3] = 2.0
    c = oracle.rmsnorm(x, w, 0.0)
    assert np.count_nonzero(c) == 1 and c[3] == pytest.approx(2.0 * a[3], rel=1e-15)


def test_softcap_values():
    y = np.array([0.0, 1e-3, -1e-3, 15.0, -45.0, 1e6, -1e6, 30.0])
    got = oracle.softcap(y, 30.0)
    assert np.allclose(got, 30.0 * np.tanh(y / 30.0), rtol=1e-15, atol=0)
    assert got[5] == 30.0 and got[6] == -30.0                 # saturates, no NaN
    assert np.allclose(oracle.softcap(y, 0.0), y)             # cap 0: identity
    assert np.all(np.diff(oracle.softcap(np.linspace(-100, 100, 1001), 30.0)) >= 0)   # monotone


def test_argmax_rules_brute_force():
    rng = np.random.default_rng(23)
    for _ in range(200):
        v = rng.integers(-3, 4, size=rng.integers(1, 40)).astype(np.float32)   # many ties
        best = max(range(v.size), key=lambda i: (v[i], -i))
        assert oracle.argmax_f32(v) == best
    v = np.array([np.nan, 1.0, 3.0, np.nan, 3.0], np.float32)
    assert oracle.argmax_f32(v) == 2                          # NaN skipped, tie -> lowest
    assert oracle.argmax_f32(np.array([np.nan, np.nan], np.float32)) == 0
    assert oracle.argmax_f32(np.array([-np.inf, -1e30, np.inf], np.float32)) == 2
    big = rng.standard_normal(262144).astype(np.float32)
    assert oracle.argmax_f32(big) == int(np.argmax(big))
