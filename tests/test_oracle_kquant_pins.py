"""Pins for the oracle's K-quant super-block decoders (Q4_K, Q5_K, Q6_K). CPU only.

The pages give the arithmetic of these formats (jouleclaw-loader-gguf
BENCHMARKS page: "Q4_K matmul" with 32-element sub-blocks and the split
d_sub * sum(a q) - m_sub * sum(a); "Q5_K + Q6_K matmul": one high bit per
element for Q5_K, two and a signed -32 offset for Q6_K) but not the byte
layout, which is taken from
the GGUF format (the oracle's header states it). These tests pin the
oracle's decoder to that layout without reusing its code:

* an encoder written here in the opposite direction -- for every element,
  where its bits go -- builds super-blocks from chosen (scales, minimums,
  quants); the oracle must decode them to d sc q - dmin m (Q4_K, Q5_K) or
  d sc (q - 32) (Q6_K) exactly, computed here from the chosen integers;
* brute force over every 6-bit scale/minimum pair of every Q4_K sub-block,
  every 5-bit Q5_K quant and every 6-bit Q6_K quant at every position;
* closed forms (all-zero quants leave only the minimums; q = 32 gives 0);
* a second decoder written with numpy array operations, and the pages'
  algebraic split of the sub-block sum, against the oracle's matvec.

Agreement with GGUF files written by other software depends on the layout
reading and is not pinned by the pages."""
import numpy as np
import pytest

import oracle
import synth

Q4K, Q5K, Q6K = synth.TYPE_Q4_K, synth.TYPE_Q5_K, synth.TYPE_Q6_K


def f16(v):
    """binary16 bits of v (must be exactly representable)."""
    b = np.float16(v)
    assert float(b) == v
    return int(b.view(np.uint16))


def enc_q4_k(d_bits, dmin_bits, sc, m, q):
    """Q4_K super-block bytes from 8 scales, 8 minimums (0..63) and 256
    quants (0..15), placing each field where the layout puts it."""
    b = bytearray(144)
    b[0:2] = int(d_bits).to_bytes(2, "little")
    b[2:4] = int(dmin_bits).to_bytes(2, "little")
    s = bytearray(12)
    for j in range(8):
        if j < 4:
            s[j] |= sc[j]                     # six bits
            s[j + 4] |= m[j]
        else:
            s[j + 4] |= (sc[j] & 15) | ((m[j] & 15) << 4)
            s[j - 4] |= (sc[j] >> 4) << 6     # top two bits
            s[j] |= (m[j] >> 4) << 6
    b[4:16] = s
    for e in range(256):
        g, r = divmod(e, 64)
        if r < 32:
            b[16 + 32 * g + r] |= q[e]
        else:
            b[16 + 32 * g + r - 32] |= q[e] << 4
    return bytes(b)


def enc_q5_k(d_bits, dmin_bits, sc, m, q):
    """Q5_K super-block bytes from 8 scales, 8 minimums (0..63) and 256
    quants (0..31): the Q4_K header and low nibbles, and each quant's fifth
    bit in the 32 qh bytes (element 64g + r: byte r % 32, bit 2g for r < 32,
    2g + 1 otherwise)."""
    q = np.asarray(q)
    b = bytearray(enc_q4_k(d_bits, dmin_bits, sc, m, q & 15))
    qh = bytearray(32)
    for e in range(256):
        g, r = divmod(e, 64)
        qh[r % 32] |= (int(q[e]) >> 4) << (2 * g + r // 32)
    return bytes(b[:16] + qh + b[16:])


def enc_q6_k(d_bits, sc, q):
    """Q6_K super-block bytes from 16 int8 scales and 256 quants (0..63)."""
    b = bytearray(210)
    for e in range(256):
        h, r = divmod(e, 128)
        t, l = divmod(r, 32)
        lo, hi = q[e] & 15, q[e] >> 4
        qlb = 64 * h + l + 32 * (t % 2)
        b[qlb] |= lo if t < 2 else lo << 4
        b[128 + 32 * h + l] |= hi << (2 * t)
    b[192:208] = bytes(np.asarray(sc, dtype=np.int8).view(np.uint8))
    b[208:210] = int(d_bits).to_bytes(2, "little")
    return bytes(b)


def blocks_from(raw):
    return np.frombuffer(b"".join(raw), dtype=np.uint8)


def test_q4_k_encoder_roundtrip_random():
    rng = np.random.default_rng(1)
    raws, expect = [], []
    for _ in range(40):
        d, dmin = rng.choice([0.5, 0.25, 1.0, 2.0, 0.125]), rng.choice([0.5, 0.25, 1.0, 0.0625])
        sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        raws.append(enc_q4_k(f16(d), f16(dmin), sc, m, q))
        expect.append(d * sc[np.arange(256) // 32] * q - dmin * m[np.arange(256) // 32])
    W = oracle.dequantize(Q4K, blocks_from(raws), 40, 256)
    assert np.array_equal(W, np.array(expect, dtype=np.float64))


def test_q6_k_encoder_roundtrip_random():
    rng = np.random.default_rng(2)
    raws, expect = [], []
    for _ in range(40):
        d = rng.choice([0.5, 0.25, 1.0, 2.0, 2.0 ** -14])
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        raws.append(enc_q6_k(f16(d), sc, q))
        expect.append(d * sc[np.arange(256) // 16] * (q - 32))
    W = oracle.dequantize(Q6K, blocks_from(raws), 40, 256)
    assert np.array_equal(W, np.array(expect, dtype=np.float64))


def test_q5_k_encoder_roundtrip_random():
    rng = np.random.default_rng(7)
    raws, expect = [], []
    for _ in range(40):
        d, dmin = rng.choice([0.5, 0.25, 1.0, 2.0, 0.125]), rng.choice([0.5, 0.25, 1.0, 0.0625])
        sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 32, 256)
        raws.append(enc_q5_k(f16(d), f16(dmin), sc, m, q))
        expect.append(d * sc[np.arange(256) // 32] * q - dmin * m[np.arange(256) // 32])
    W = oracle.dequantize(Q5K, blocks_from(raws), 40, 256)
    assert np.array_equal(W, np.array(expect, dtype=np.float64))


def test_q5_k_every_value_at_every_position():
    """Each element takes each 5-bit value in turn, all others 0; sub-block
    scales j + 1 and minimums 0, d = 1: exactly that element reads
    (j + 1) v (a wrong fifth-bit position or sub-block index shows)."""
    sc = np.arange(1, 9)
    for v in range(1, 32):
        raws, expect = [], []
        for e in range(256):
            q = np.zeros(256, int)
            q[e] = v
            raws.append(enc_q5_k(f16(1.0), f16(1.0), sc, np.zeros(8, int), q))
            row = np.zeros(256)
            row[e] = (e // 32 + 1) * v
            expect.append(row)
        W = oracle.dequantize(Q5K, blocks_from(raws), 256, 256)
        assert np.array_equal(W, np.array(expect)), v


def test_q4_k_every_scale_min_pair_of_every_sub_block():
    """All 64 x 64 (scale, minimum) pairs in each of the 8 sub-blocks, with
    every other field zero and all quants 1: the sub-block reads sc - m and
    the rest reads 0 (d = dmin = 1)."""
    vals = np.arange(64)
    for j in range(8):
        raws, expect = [], []
        for a in vals:
            for c in vals:
                sc, m = np.zeros(8, int), np.zeros(8, int)
                sc[j], m[j] = a, c
                raws.append(enc_q4_k(f16(1.0), f16(1.0), sc, m, np.ones(256, int)))
                row = np.zeros(256)
                row[32 * j: 32 * j + 32] = a - c
                expect.append(row)
        W = oracle.dequantize(Q4K, blocks_from(raws), len(raws), 256)
        assert np.array_equal(W, np.array(expect)), j


def test_q4_k_every_nibble_at_every_position():
    """One element at a time takes each value 1..15, all others 0; sub-block
    scale 1, minimum 0, d = 1: exactly that element reads that value."""
    raws, expect = [], []
    for e in range(256):
        for v in (1, 7, 8, 15):
            q = np.zeros(256, int)
            q[e] = v
            raws.append(enc_q4_k(f16(1.0), f16(1.0), np.ones(8, int), np.zeros(8, int), q))
            row = np.zeros(256)
            row[e] = v
            expect.append(row)
    W = oracle.dequantize(Q4K, blocks_from(raws), len(raws), 256)
    assert np.array_equal(W, np.array(expect))


def test_q6_k_every_value_at_every_position():
    """Each element takes each 6-bit value in turn with all others at 32
    (which reads 0); scales = index + 1 so a wrong scale index shows."""
    sc = np.arange(1, 17)
    for v in range(64):
        raws, expect = [], []
        for e in range(256):
            q = np.full(256, 32)
            q[e] = v
            raws.append(enc_q6_k(f16(1.0), sc, q))
            row = np.zeros(256)
            row[e] = (e // 16 + 1) * (v - 32)
            expect.append(row)
        W = oracle.dequantize(Q6K, blocks_from(raws), 256, 256)
        assert np.array_equal(W, np.array(expect)), v


def test_closed_forms():
    rng = np.random.default_rng(3)
    k = 512
    x = rng.standard_normal(k)
    # Q4_K, all quants 0: only the minimums remain, y = -sum_j dmin m_j sum(x_j)
    sc, m = rng.integers(0, 64, (2, 8)), rng.integers(0, 64, (2, 8))
    raw = blocks_from([enc_q4_k(f16(0.5), f16(0.25), sc[i], m[i], np.zeros(256, int)) for i in range(2)])
    y, _ = oracle.matvec(Q4K, raw, 1, k, x)
    xs = x.reshape(16, 32).sum(axis=1)
    assert y[0] == pytest.approx(-0.25 * float((m.reshape(-1) * xs).sum()), rel=1e-13)
    # Q4_K, q = 15, scale 1, minimum 0, d = 1, x = 1: y = 15 k
    raw = blocks_from([enc_q4_k(f16(1.0), f16(3.0), np.ones(8, int), np.zeros(8, int), np.full(256, 15))] * 2)
    y, _ = oracle.matvec(Q4K, raw, 1, k, np.ones(k))
    assert y[0] == 15 * k
    # Q5_K, all quants 0: the same minimum-only sum as Q4_K (same header)
    raw = blocks_from([enc_q5_k(f16(0.5), f16(0.25), sc[i], m[i], np.zeros(256, int)) for i in range(2)])
    y, _ = oracle.matvec(Q5K, raw, 1, k, x)
    assert y[0] == pytest.approx(-0.25 * float((m.reshape(-1) * xs).sum()), rel=1e-13)
    # Q5_K, q = 31, scale 1, minimum 0, d = 1, x = 1: y = 31 k; q = 16 (fifth
    # bit alone) gives 16 k
    for v in (31, 16):
        raw = blocks_from([enc_q5_k(f16(1.0), f16(3.0), np.ones(8, int), np.zeros(8, int), np.full(256, v))] * 2)
        y, _ = oracle.matvec(Q5K, raw, 1, k, np.ones(k))
        assert y[0] == v * k
    # Q6_K, q = 32 everywhere: w = 0 whatever the scales
    raw = blocks_from([enc_q6_k(f16(2.0), rng.integers(-128, 128, 16), np.full(256, 32))] * 2)
    y, a = oracle.matvec(Q6K, raw, 1, k, x)
    assert y[0] == 0.0 and a[0] == 0.0
    # Q6_K, q = 63, scale 1, d = 1, x = 1: y = 31 k; q = 0 gives -32 k
    for v, want in ((63, 31 * k), (0, -32 * k)):
        raw = blocks_from([enc_q6_k(f16(1.0), np.ones(16, int), np.full(256, v))] * 2)
        y, _ = oracle.matvec(Q6K, raw, 1, k, np.ones(k))
        assert y[0] == want


def _numpy_dequant_q4_k(w):
    """A second Q4_K decoder, written with whole-array numpy operations."""
    d = w["d"].view(np.float16).astype(np.float64)[..., None]
    dmin = w["dmin"].view(np.float16).astype(np.float64)[..., None]
    s = w["scales"].astype(np.int64)
    lo_sc, lo_m = s[..., 0:4] & 63, s[..., 4:8] & 63
    hi_sc = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    hi_m = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    sc = np.concatenate([lo_sc, hi_sc], axis=-1)
    m = np.concatenate([lo_m, hi_m], axis=-1)
    qs = w["qs"].astype(np.int64).reshape(w.shape + (4, 32))
    q = np.stack([qs & 15, qs >> 4], axis=-2).reshape(w.shape + (256,))
    sub = np.arange(256) // 32
    vals = d * sc[..., sub] * q - dmin * m[..., sub]
    return vals.reshape(w.shape[0], -1)


def _numpy_dequant_q5_k(w):
    """A second Q5_K decoder: the Q4_K one on the low nibbles, plus 16 times
    each element's fifth bit taken by whole-array shifts."""
    base = w[["d", "dmin", "scales", "qs"]]
    w4 = np.empty(w.shape, dtype=synth.Q4_K_BLOCK)
    for f in ("d", "dmin", "scales", "qs"):
        w4[f] = base[f]
    d = w["d"].view(np.float16).astype(np.float64)[..., None]
    s = w["scales"].astype(np.int64)
    sc = np.concatenate([s[..., 0:4] & 63, (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)], axis=-1)
    qh = w["qh"].astype(np.int64)                                   # (..., 32): byte l
    bits = (qh[..., None, :] >> np.arange(8).reshape(8, 1)) & 1      # (..., 8 bits, 32 l): bit 2g + t
    fifth = bits.reshape(w.shape + (256,))                          # element 64g + 32t + l
    sub = np.arange(256) // 32
    extra = (d * sc[..., sub] * 16 * fifth).reshape(w.shape[0], -1)
    return _numpy_dequant_q4_k(w4) + extra


def _numpy_dequant_q6_k(w):
    d = w["d"].view(np.float16).astype(np.float64)[..., None]
    ql = w["ql"].astype(np.int64).reshape(w.shape + (2, 2, 32))     # half, ql run, l
    qh = w["qh"].astype(np.int64).reshape(w.shape + (2, 1, 32))
    lo = np.concatenate([ql & 15, ql >> 4], axis=-2)                  # runs t = 0, 1 (low), 2, 3 (high)
    hi = (qh >> (2 * np.arange(4)).reshape(4, 1)) & 3
    q = (lo | (hi << 4)).reshape(w.shape + (256,))
    sc = w["scales"].astype(np.int64)[..., np.arange(256) // 16]
    return (d * sc * (q - 32)).reshape(w.shape[0], -1)


@pytest.mark.parametrize("qtype,dec", [(Q4K, _numpy_dequant_q4_k), (Q5K, _numpy_dequant_q5_k),
                                       (Q6K, _numpy_dequant_q6_k)])
def test_numpy_second_decoder_and_matvec(qtype, dec):
    rng = np.random.default_rng(4 + qtype)
    n, k = 37, 1024
    w = synth.weights(rng, qtype, n, k)
    W = dec(w)
    assert np.array_equal(oracle.dequantize(qtype, w, n, k), W)
    x = rng.standard_normal(k)
    y, a = oracle.matvec(qtype, w, n, k, x)
    assert np.allclose(y, W @ x, rtol=1e-12, atol=1e-12 * np.abs(W).sum())
    assert np.allclose(a, np.abs(W * x).sum(axis=1), rtol=1e-12)


def test_q4_k_algebraic_split_of_the_pages():
    """sum(a (d_sub q - m_sub)) = d_sub sum(a q) - m_sub sum(a), sub-block by
    sub-block, computed here from the chosen integers, equals the oracle's
    element-by-element matvec (to fp64 rounding)."""
    rng = np.random.default_rng(5)
    nsb, rows = 4, 6
    k = 256 * nsb
    x = rng.standard_normal(k)
    raws, want = [], []
    for _ in range(rows):
        tot = 0.0
        for s in range(nsb):
            d, dmin = float(np.float16(rng.uniform(1e-4, 3e-4))), float(np.float16(rng.uniform(1e-4, 3e-4)))
            sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 16, 256)
            raws.append(enc_q4_k(f16(d), f16(dmin), sc, m, q))
            xs = x[256 * s: 256 * s + 256].reshape(8, 32)
            qq = q.reshape(8, 32)
            tot += float(((d * sc) * (qq * xs).sum(axis=1) - (dmin * m) * xs.sum(axis=1)).sum())
        want.append(tot)
    y, a = oracle.matvec(Q4K, blocks_from(raws), rows, k, x)
    assert np.allclose(y, want, rtol=0, atol=1e-12 * a.max())


def test_kquant_rejects_partial_super_blocks_and_int_path():
    w = synth.q4_k_weights(np.random.default_rng(6), 2, 256)
    with pytest.raises(RuntimeError):
        oracle.matvec(Q4K, w, 2, 288, np.zeros(288))        # 288 is not a multiple of 256
    with pytest.raises(RuntimeError):
        oracle.blockdots(Q4K, w, 2, 256, np.zeros((1, 256), np.int8), np.zeros((1, 8), np.uint16))
