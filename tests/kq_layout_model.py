"""numpy model of the packed K-quant sections that the matvec kernels read
(test infrastructure: the expected output of gq_kq_pack, written from the
layout description in include/gq.h, and the bit recipe the kernels use to
read it back). Every field is a lossless rearrangement of GGUF bits.

Q4_K header (16 bytes per super-block): d, dmin, then for each 64-element
chunk g (sub-blocks 2g, 2g+1) the 24-bit field
sc_2g | sc_2g+1 << 6 | m_2g << 12 | m_2g+1 << 18 in bytes 4+3g .. 6+3g.

Q5_K (qs and header as Q4_K) fifth bits (32 bytes per super-block): one
32-bit word per 16-byte quant unit u (elements 64g + 16t + e, low run, and
+ 32, high run; g = u / 2, t = u % 2, e < 16). Quant word c of the unit
holds elements 4c..4c+3 of both runs; word c's bits sit at 4, 5, 20, 21
(low run, b = 0..3) and 8, 9, 24, 25 (high run), rotated left by 0, 2, 8,
10 for c = 0..3 (the four rotated sets are disjoint and fill the word).

Q6_K high bits (64 bytes per super-block): for each 16-byte ql unit u = 4h+j
(elements 128h + 16j + e, low run, and + 64, high run; e < 16), two 32-bit
words. ql word c of the unit holds elements 4c..4c+3 of both runs; word c's
2-bit fields sit at bits 4, 6, 20, 22 (low run, b = 0..3) and 8, 10, 24, 26
(high run); word 2p holds words 2p's fields in place and word 2p+1's rotated
left by 8. Q6_K scales (16 bytes): per unit, its low-run and high-run int8
scale.
"""
import numpy as np

LO_POS = (4, 6, 20, 22)
HI_POS = (8, 10, 24, 26)
Q5_LO_POS = (4, 5, 20, 21)
Q5_HI_POS = (8, 9, 24, 25)
Q5_ROT = (0, 2, 8, 10)


def q4_k_scale_min(scales):
    """GGUF 12-byte scale field -> (sc, m), each (..., 8) in 0..63."""
    s = scales.astype(np.uint32)
    sc = np.concatenate([s[..., 0:4] & 63, (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)], axis=-1)
    m = np.concatenate([s[..., 4:8] & 63, (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)], axis=-1)
    return sc, m


def q4_k_header(w):
    """Expected packed Q4_K headers, (n, nsb, 16) uint8."""
    sc, m = q4_k_scale_min(w["scales"])
    f = sc[..., 0::2] | (sc[..., 1::2] << 6) | (m[..., 0::2] << 12) | (m[..., 1::2] << 18)   # (n, nsb, 4)
    fb = np.stack([f & 255, (f >> 8) & 255, (f >> 16) & 255], axis=-1).reshape(f.shape[:-1] + (12,))
    hdr = np.empty(w.shape + (16,), np.uint8)
    hdr[..., 0:2] = w["d"][..., None].view(np.uint8).reshape(w.shape + (2,))
    hdr[..., 2:4] = w["dmin"][..., None].view(np.uint8).reshape(w.shape + (2,))
    hdr[..., 4:16] = fb.astype(np.uint8)
    return hdr


def _rotl8(x):
    return ((x << np.uint32(8)) | (x >> np.uint32(24))) & np.uint32(0xFFFFFFFF)


def _rotr8(x):
    return ((x >> np.uint32(8)) | (x << np.uint32(24))) & np.uint32(0xFFFFFFFF)


def _rotl(x, r):
    r %= 32
    return ((x << np.uint32(r)) | (x >> np.uint32((32 - r) % 32))) & np.uint32(0xFFFFFFFF) if r else x


def _rotr(x, r):
    return _rotl(x, 32 - r) if r % 32 else x


def q5_k_fifth_words(w):
    """Expected packed Q5_K fifth-bit words, (n, nsb, 8 units) uint32."""
    qh = w["qh"].astype(np.uint32)
    out = np.zeros(w.shape + (8,), np.uint32)
    for u in range(8):
        g, t = divmod(u, 2)
        word = np.zeros(w.shape, np.uint32)
        for c in range(4):
            f = np.zeros(w.shape, np.uint32)
            for b in range(4):
                qb = qh[..., 16 * t + 4 * c + b]
                f |= ((qb >> np.uint32(2 * g)) & np.uint32(1)) << np.uint32(Q5_LO_POS[b])
                f |= ((qb >> np.uint32(2 * g + 1)) & np.uint32(1)) << np.uint32(Q5_HI_POS[b])
            word |= _rotl(f, Q5_ROT[c])
        out[..., u] = word
    return out


def q5_k_read_back(qs_unit_words, fifth_word):
    """The kernels' recipe, on one unit: quant words (4,) and its fifth-bit
    word -> (low run, high run) 5-bit values, 16 each (the bit patterns the
    kernel reads as binary16 subnormals)."""
    lo, hi = np.zeros(16, np.int64), np.zeros(16, np.int64)
    for c in range(4):
        v = np.uint32(qs_unit_words[c])
        v8 = v >> np.uint32(8)
        hc = _rotr(np.uint32(fifth_word), Q5_ROT[c])
        hc1 = hc >> np.uint32(1)
        for half, sh in ((0, 0), (1, 16)):
            lo[4 * c + 2 * half] = int(((v | 0) >> np.uint32(sh) & np.uint32(0xF)) | ((hc >> np.uint32(sh)) & np.uint32(0x10)))
            lo[4 * c + 2 * half + 1] = int(((v8 >> np.uint32(sh)) & np.uint32(0xF)) | ((hc1 >> np.uint32(sh)) & np.uint32(0x10)))
            hi[4 * c + 2 * half] = int((((v >> np.uint32(sh)) & np.uint32(0xF0)) |
                                        ((hc >> np.uint32(sh)) & np.uint32(0x100))) >> np.uint32(4))
            hi[4 * c + 2 * half + 1] = int((((v8 >> np.uint32(sh)) & np.uint32(0xF0)) |
                                            ((hc1 >> np.uint32(sh)) & np.uint32(0x100))) >> np.uint32(4))
    return lo, hi


def q6_k_high_words(w):
    """Expected packed Q6_K high-bit words, (n, nsb, 8 units, 2) uint32."""
    qh = w["qh"].astype(np.uint32)
    out = np.zeros(w.shape + (8, 2), np.uint32)
    for u in range(8):
        h, j = divmod(u, 4)
        sl, sh = 2 * (j // 2), 4 + 2 * (j // 2)
        fields = []
        for c in range(4):
            f = np.zeros(w.shape, np.uint32)
            for b in range(4):
                qb = qh[..., 32 * h + 16 * (j % 2) + 4 * c + b]
                f |= ((qb >> sl) & 3) << LO_POS[b]
                f |= ((qb >> sh) & 3) << HI_POS[b]
            fields.append(f)
        out[..., u, 0] = fields[0] | _rotl8(fields[1])
        out[..., u, 1] = fields[2] | _rotl8(fields[3])
    return out


def q6_k_unit_scales(w):
    """Expected packed Q6_K scale pairs, (n, nsb, 8 units, 2) int8."""
    s = w["scales"]
    out = np.empty(w.shape + (8, 2), np.int8)
    for u in range(8):
        h, j = divmod(u, 4)
        out[..., u, 0] = s[..., 8 * h + j]
        out[..., u, 1] = s[..., 8 * h + j + 4]
    return out


def q6_k_read_back(ql_unit_words, high_words):
    """The kernels' recipe, on one unit: ql words (4,) and its two high-bit
    words -> (low run, high run) 6-bit values, 16 each."""
    lo, hi = np.zeros(16, np.int64), np.zeros(16, np.int64)
    for c in range(4):
        v = np.uint32(ql_unit_words[c])
        v8 = v >> np.uint32(8)
        hc = np.uint32(high_words[c >> 1])
        if c & 1:
            hc = _rotr8(hc)
        hc2 = hc >> np.uint32(2)
        for half, sh in ((0, 0), (1, 16)):
            # lo02 / lo13: nibble at bits 0-3 of the 16-bit half, high bits at 4-5
            lo[4 * c + 2 * half] = int(((v >> np.uint32(sh)) & np.uint32(15)) | ((hc >> np.uint32(sh)) & np.uint32(0x30)))
            lo[4 * c + 2 * half + 1] = int(((v8 >> np.uint32(sh)) & np.uint32(15)) |
                                           ((hc2 >> np.uint32(sh)) & np.uint32(0x30)))
            # hi02 / hi13: nibble at bits 4-7, high bits at 8-9 (the value times 16)
            hi[4 * c + 2 * half] = int((((v >> np.uint32(sh)) & np.uint32(0xF0)) |
                                        ((hc >> np.uint32(sh)) & np.uint32(0x300))) >> np.uint32(4))
            hi[4 * c + 2 * half + 1] = int((((v8 >> np.uint32(sh)) & np.uint32(0xF0)) |
                                            ((hc2 >> np.uint32(sh)) & np.uint32(0x300))) >> np.uint32(4))
    return lo, hi


def q4_k_read_back(header_words, g):
    """The kernels' recipe: header words (x, y, z, w) and chunk g ->
    (sc_2g, sc_2g+1, m_2g, m_2g+1) via the byte permute of (y, z) or (z, w)."""
    x, y, z, w = (int(t) for t in header_words)
    lo, hi = (y, z) if g < 2 else (z, w)
    fb = 3 * g if g < 2 else 3 * g - 4
    pair = lo | (hi << 32)
    f = (pair >> (8 * fb)) & 0xFFFFFF
    return f & 63, (f >> 6) & 63, (f >> 12) & 63, (f >> 18) & 63
