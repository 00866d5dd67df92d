"""The packed K-quant layout (host-side model, no GPU): super-blocks built by
the independent GGUF encoders of the oracle pins from known scales, minimums
and quants are rearranged as gq_kq_pack lays them out, and the bit recipe the
matvec kernels use to read the packed fields gives back every one of those
values, in every unit and chunk position."""
import numpy as np

import kq_layout_model as model
from test_oracle_kquant_pins import blocks_from, enc_q4_k, enc_q5_k, enc_q6_k, f16

import synth


def test_q4_k_header_fields_read_back_exactly():
    rng = np.random.default_rng(11)
    raw, truth = [], []
    for _ in range(24):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        raw.append(enc_q4_k(f16(0.5), f16(0.25), sc, m, q))
        truth.append((sc, m))
    w = blocks_from(raw).view(synth.Q4_K_BLOCK).reshape(4, 6)
    hdr = model.q4_k_header(w)
    assert np.array_equal(hdr[..., 0:2].copy().view(np.uint16)[..., 0], w["d"])
    assert np.array_equal(hdr[..., 2:4].copy().view(np.uint16)[..., 0], w["dmin"])
    words = hdr.copy().view("<u4")                       # (4, 6, 4)
    for i, (sc, m) in enumerate(truth):
        r, s = divmod(i, 6)
        for g in range(4):
            got = model.q4_k_read_back(words[r, s], g)
            assert got == (sc[2 * g], sc[2 * g + 1], m[2 * g], m[2 * g + 1]), (i, g)


def test_q4_k_header_extreme_fields():
    # every field at 0 and at 63 in turn: no bit of a neighbour leaks in
    for hot in range(16):
        sc = np.zeros(8, np.int64)
        m = np.zeros(8, np.int64)
        (sc if hot < 8 else m)[hot % 8] = 63
        w = blocks_from([enc_q4_k(f16(1.0), f16(1.0), sc, m, np.zeros(256, np.int64))]).view(synth.Q4_K_BLOCK)
        words = model.q4_k_header(w.reshape(1, 1)).copy().view("<u4")[0, 0]
        for g in range(4):
            assert model.q4_k_read_back(words, g) == (sc[2 * g], sc[2 * g + 1], m[2 * g], m[2 * g + 1])


def test_q6_k_high_bits_and_scales_read_back_exactly():
    rng = np.random.default_rng(12)
    raw, truth = [], []
    for _ in range(12):
        q = rng.integers(0, 64, 256)
        sc = rng.integers(-128, 128, 16)
        raw.append(enc_q6_k(f16(0.5), sc, q))
        truth.append((q, sc))
    w = blocks_from(raw).view(synth.Q6_K_BLOCK).reshape(3, 4)
    hw = model.q6_k_high_words(w)
    us = model.q6_k_unit_scales(w)
    for i, (q, sc) in enumerate(truth):
        r, s = divmod(i, 4)
        for u in range(8):
            h, j = divmod(u, 4)
            ql_words = w["ql"][r, s, 64 * h + 16 * j: 64 * h + 16 * j + 16].copy().view("<u4")
            lo, hi = model.q6_k_read_back(ql_words, hw[r, s, u])
            base = 128 * h + 16 * j
            assert np.array_equal(lo, q[base: base + 16]), (i, u)
            assert np.array_equal(hi, q[base + 64: base + 80]), (i, u)
            assert us[r, s, u, 0] == sc[8 * h + j] and us[r, s, u, 1] == sc[8 * h + j + 4]


def test_q6_k_single_high_bit_lands_once():
    # one element at 48 (high bits 3), the rest 0: exactly that element reads back nonzero
    for e in range(256):
        q = np.zeros(256, np.int64)
        q[e] = 48
        w = blocks_from([enc_q6_k(f16(1.0), np.ones(16, np.int64), q)]).view(synth.Q6_K_BLOCK).reshape(1, 1)
        hw = model.q6_k_high_words(w)
        got = np.zeros(256, np.int64)
        for u in range(8):
            h, j = divmod(u, 4)
            ql_words = w["ql"][0, 0, 64 * h + 16 * j: 64 * h + 16 * j + 16].copy().view("<u4")
            lo, hi = model.q6_k_read_back(ql_words, hw[0, 0, u])
            got[128 * h + 16 * j: 128 * h + 16 * j + 16] = lo
            got[128 * h + 16 * j + 64: 128 * h + 16 * j + 80] = hi
        assert np.array_equal(got, q), e


def _q5_k_unit_values(w, r, s_, q_words_of, fifth):
    got = np.zeros(256, np.int64)
    for u in range(8):
        g, t = divmod(u, 2)
        lo, hi = model.q5_k_read_back(q_words_of(u), fifth[r, s_, u])
        got[64 * g + 16 * t: 64 * g + 16 * t + 16] = lo
        got[64 * g + 32 + 16 * t: 64 * g + 32 + 16 * t + 16] = hi
    return got


def test_q5_k_fifth_bits_read_back_exactly():
    rng = np.random.default_rng(13)
    raw, truth = [], []
    for _ in range(12):
        q = rng.integers(0, 32, 256)
        raw.append(enc_q5_k(f16(0.5), f16(0.25), rng.integers(0, 64, 8), rng.integers(0, 64, 8), q))
        truth.append(q)
    w = blocks_from(raw).view(synth.Q5_K_BLOCK).reshape(3, 4)
    fifth = model.q5_k_fifth_words(w)
    for i, q in enumerate(truth):
        r, s_ = divmod(i, 4)
        words = lambda u: w["qs"][r, s_, 16 * u: 16 * u + 16].copy().view("<u4")   # noqa: E731
        assert np.array_equal(_q5_k_unit_values(w, r, s_, words, fifth), q), i
    # the header is the Q4_K one: same packing, same read-back
    hdr = model.q4_k_header(w)
    assert np.array_equal(hdr[..., 0:2].copy().view(np.uint16)[..., 0], w["d"])


def test_q5_k_single_fifth_bit_lands_once():
    # one element at 16 (fifth bit only), the rest 0: exactly that element reads back nonzero
    for e in range(256):
        q = np.zeros(256, np.int64)
        q[e] = 16
        w = blocks_from([enc_q5_k(f16(1.0), f16(1.0), np.ones(8, np.int64), np.zeros(8, np.int64), q)])
        w = w.view(synth.Q5_K_BLOCK).reshape(1, 1)
        fifth = model.q5_k_fifth_words(w)
        words = lambda u: w["qs"][0, 0, 16 * u: 16 * u + 16].copy().view("<u4")   # noqa: E731
        assert np.array_equal(_q5_k_unit_values(w, 0, 0, words, fifth), q), e
