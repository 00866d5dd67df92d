"""GPU parity at special values, on every dispatch path of every kernel
family: weight scales that are +-0, binary16 subnormals, the largest finite
binary16, +-Inf and NaN; zero activation scales (all-zero activation blocks,
and pre-quantised blocks whose scale is 0); and the RMSNorm prologue at the
edges of the fp32 range.

What is compared (the plain definition y = sum_c w[r][c] x[c], computed by
the fp64 oracle from the same GGUF bytes):
  * finite oracle rows: the GPU value within the accuracy contract
    |y - y_ref| <= 1e-4 sum|w x| + 1e-6 (integer block sums bit for bit);
  * non-finite oracle rows (a non-finite scale in the row): the GPU value is
    non-finite too, and where both are infinite they have the same sign.
    Which of NaN and Inf is not fixed: a block whose scale is Inf gives NaN in
    the plain definition as soon as one of its 32 products is Inf * 0, while
    the kernels multiply the scale into the block's summed products."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_special, check_within, down, packed, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_block_quant_amd as gq  # noqa: E402

Q4, Q8 = gq.TYPE_Q4_0, gq.TYPE_Q8_0

FINITE_SPECIAL = [0x0000, 0x8000,            # +0, -0
                  0x0001, 0x8001, 0x03FF,    # subnormals: smallest, its negative, largest
                  0x8200, 0x0400,            # a negative subnormal; the smallest normal
                  0x7BFF, 0xFBFF]            # +-65504, the largest finite
NONFINITE = [0x7C00, 0xFC00, 0x7E00, 0xFE01]  # +Inf, -Inf, quiet NaN, a negative NaN


def plant(rng, w, patterns, frac):
    """Overwrite a fraction of the blocks' scale bits with the given
    patterns (input construction only: the bytes both sides read)."""
    d = w["d"]
    mask = rng.random(d.shape) < frac
    d[mask] = rng.choice(np.array(patterns, dtype=np.uint16), size=int(mask.sum()))
    return w


def plant_rows(rng, w, patterns, rows):
    """Non-finite scales in one block of each of the given rows only."""
    nb = w["d"].shape[1]
    for r in rows:
        w["d"][r, rng.integers(0, nb)] = patterns[r % len(patterns)]
    return w


def special_weights(qtype, n, k, seed, nonfinite_rows=True):
    rng = np.random.default_rng(seed)
    w = synth.weights(rng, qtype, n, k)
    plant(rng, w, FINITE_SPECIAL, 0.05)
    # a few whole rows of zero scales, and of subnormal ones
    w["d"][min(3, n - 1)] = 0x0000
    w["d"][min(5, n - 1)] = 0x0001
    if nonfinite_rows:
        plant_rows(rng, w, NONFINITE, range(0, n, 7))
    return w, rng


# every dispatch path of the fp32 matvec: one row per wave step at 8 waves
# (2048 x 2048), four rows per step (tall), rows split over 2 / 4 waves with
# x staged, over 8 / 16 waves with x in registers
F32_SHAPES = [(Q4, 2048, 2048), (Q8, 1001, 96), (Q8, 8195, 2048), (Q4, 16384, 2048),
              (Q8, 515, 2048), (Q4, 300, 4096), (Q4, 1001, 8192), (Q8, 257, 8192),
              (Q4, 77, 16384), (Q8, 64, 32768)]


@pytest.mark.parametrize("qtype,n,k", F32_SHAPES)
def test_fp32_matvec_special_scales(qtype, n, k):
    w, rng = special_weights(qtype, n, k, n + 3 * k)
    x = synth.activations(rng, k)
    qs, d = packed(gq, qtype, w, n, k)
    fn = gq.qmv_q8_0 if qtype == Q8 else gq.qmv_q4_0
    y = down(fn(qs, d, n, k, up(x)))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    assert np.isfinite(yr).sum() > 0 and (~np.isfinite(yr)).sum() > 0
    check_special(y, yr, ar, "qmv type %d %dx%d" % (qtype, n, k))


INT_SHAPES = [(Q4, 2048, 2048), (Q8, 1001, 96), (Q8, 16384, 2048), (Q4, 515, 4096),
              (Q4, 1001, 8192), (Q8, 45, 16384), (Q4, 64, 32768)]


@pytest.mark.parametrize("qtype,n,k", INT_SHAPES)
def test_int_matvec_special_scales_and_zero_activation_blocks(qtype, n, k):
    """Pre-quantised activations with some block scales 0 (codes nonzero),
    and the fused-quantiser path on x with all-zero blocks (scale 0, codes
    0): block sums S bit for bit, y within the bound where finite."""
    w, rng = special_weights(qtype, n, k, 5 * n + k)
    nb = k // 32
    qs, d = packed(gq, qtype, w, n, k)
    xq, xd = synth.q8_0_activations(rng, 1, k)
    xd[0, rng.random(nb) < 0.2] = 0x0000
    xd[0, 0] = 0x8000
    bd = torch.empty((n, nb), dtype=torch.int32, device="cuda")
    fn8 = gq.qmv_q8_0_q8 if qtype == Q8 else gq.qmv_q4_0_q8
    y = down(fn8(qs, d, n, k, up(xq[0]), up(xd[0]), blockdots=bd))
    S, yr, ar = oracle.blockdots(qtype, w, n, k, xq, xd)
    assert np.array_equal(down(bd), S[0])
    check_special(y, yr[0], ar[0], "int path type %d %dx%d" % (qtype, n, k))

    x = synth.activations(rng, k)
    x[: 32] = 0.0
    x.reshape(nb, 32)[rng.random(nb) < 0.2] = 0.0
    rq, rd = oracle.quantize_q8_0(x)
    assert (rd == 0).sum() >= 1
    fn8x = gq.qmv_q8_0_q8x if qtype == Q8 else gq.qmv_q4_0_q8x
    xq_out = torch.empty(k, dtype=torch.int8, device="cuda")
    xd_out = torch.empty(nb, dtype=torch.int16, device="cuda")
    y = down(fn8x(qs, d, n, k, up(x), blockdots=bd, xq_out=xq_out, xd_out=xd_out))
    assert np.array_equal(down(xq_out), rq[0]) and np.array_equal(down(xd_out, np.uint16), rd[0])
    S, yr, ar = oracle.blockdots(qtype, w, n, k, rq, rd)
    assert np.array_equal(down(bd), S[0])
    check_special(y, yr[0], ar[0], "fused-quantiser path type %d %dx%d" % (qtype, n, k))


@pytest.mark.parametrize("n_ff,k", [(8192, 2048), (1056, 8192), (320, 16384)])
def test_ffn_special_scales(n_ff, k):
    """Gate and up matrices with special scales: h finite exactly where the
    oracle's is, and within the propagated bound there; then the down
    projection with special (finite and non-finite) scales on a finite h."""
    wg, rng = special_weights(Q4, n_ff, k, n_ff + k)
    wu, _ = special_weights(Q4, n_ff, k, n_ff + k + 1)
    x = synth.activations(rng, k)
    g = packed(gq, Q4, wg, n_ff, k)
    u = packed(gq, Q4, wu, n_ff, k)
    h = down(gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x)))
    ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, x)
    fin = np.isfinite(ref["h"])
    assert np.array_equal(np.isfinite(h), fin), "finiteness of h"
    assert (~fin).sum() > 0
    hb = oracle.ffn_h_bound(ref["g"][fin], ref["u"][fin], ref["ag"][fin], ref["au"][fin], ref["h"][fin])
    check_within(h[fin], ref["h"][fin], hb, "ffn h")

    wd, _ = special_weights(Q4, k, n_ff, n_ff + k + 2)
    hf = np.where(np.isfinite(h), h, 0.0).astype(np.float32)
    dq = packed(gq, Q4, wd, k, n_ff)
    y = down(gq.qmv_q4_0(dq[0], dq[1], k, n_ff, up(hf)))
    yr, ar = oracle.matvec(Q4, wd, k, n_ff, hf)
    check_special(y, yr, ar, "ffn down")


@pytest.mark.parametrize("m", [1, 4, 8, 16, 32])
def test_tile_special_scales(m):
    n, k = 515, 2048
    w, rng = special_weights(Q4, n, k, 100 + m)
    qs, d = packed(gq, Q4, w, n, k)
    xq, xd = synth.q8_0_activations(rng, m, k)
    xd[rng.random(xd.shape) < 0.1] = 0x0000
    xq[m - 1, :64] = 0
    xd[m - 1, :2] = 0x0000                              # all-zero blocks of the last row
    bd = torch.empty((m, n, k // 32), dtype=torch.int32, device="cuda")
    y = down(gq.qmm_tile_m(qs, d, n, k, m, up(xq), up(xd), blockdots=bd))
    S, yr, ar = oracle.blockdots(Q4, w, n, k, xq, xd)
    assert np.array_equal(down(bd), S)
    check_special(y, yr, ar, "tile m=%d" % m)


# ----------------------------------------------------------------------------
# RMSNorm prologue at the edges of the fp32 range
# ----------------------------------------------------------------------------

FOLD_SHAPES = [(Q8, 300, 2048), (Q4, 2048, 2048), (Q4, 515, 8192), (Q8, 45, 16384), (Q4, 64, 32768)]


def _norm_cases(rng, k):
    base = synth.activations(rng, k)
    huge = (base * np.float32(1e36)).astype(np.float32)       # sum of squares ~ 1e75: past fp32
    edge = base.copy()
    edge[k // 3] = np.float32(3.0e38)                           # one element near the fp32 maximum
    tiny = (base * np.float32(1e-30)).astype(np.float32)       # squares ~ 1e-60: below fp32
    return [("huge", huge, 1e-6), ("edge", edge, 1e-6), ("tiny eps=0", tiny, 0.0), ("normal", base, 1e-6)]


@pytest.mark.parametrize("qtype,n,k", FOLD_SHAPES)
def test_rmsnorm_fold_full_fp32_range(qtype, n, k):
    rng = np.random.default_rng(n + k)
    w = synth.weights(rng, qtype, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    g = rng.uniform(0.5, 1.0, k).astype(np.float32)            # |x g| stays finite for |x| <= 3.4e38
    fn = gq.qmv_q8_0_ex if qtype == Q8 else gq.qmv_q4_0_ex
    for name, x, eps in _norm_cases(rng, k):
        y = down(fn(qs, d, n, k, up(x), norm_weight=up(g), norm_eps=eps))
        xn = oracle.rmsnorm(x, g, eps)
        yr, ar = oracle.matvec(qtype, w, n, k, xn)
        assert np.all(np.isfinite(yr))
        check_within(y, yr, oracle.fp32_path_bound(ar), "rmsnorm %s type %d %dx%d" % (name, qtype, n, k))


def _boundary_cases(rng, k):
    """x and g whose largest |x g| sits exactly on, or one ulp outside, the
    ends of the range where the fold scales the finished rows (2^-40, 2^40);
    outside it the activations are scaled first. Both must match the oracle."""
    out = []
    j = k // 5
    for edge in (2.0 ** 40, 2.0 ** -40):
        for name, v in (("at", edge), ("outside", np.nextafter(np.float32(edge), np.float32(np.inf if edge > 1 else 0)))):
            g = rng.uniform(0.5, 1.0, k).astype(np.float32)
            g[j] = 1.0
            base = synth.activations(rng, k)
            x = (base * np.float32(edge / 2 / np.abs(base).max())).astype(np.float32)   # |x g| <= edge / 2
            x[j] = np.float32(v)
            out.append(("%s %g" % (name, edge), x, g))
    return out


@pytest.mark.parametrize("qtype,n,k", [(Q4, 2048, 2048), (Q8, 515, 8192), (Q4, 64, 32768)])
def test_rmsnorm_fold_scaling_path_boundary(qtype, n, k):
    rng = np.random.default_rng(7 * n + k)
    w = synth.weights(rng, qtype, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    fn = gq.qmv_q8_0_ex if qtype == Q8 else gq.qmv_q4_0_ex
    for name, x, g in _boundary_cases(rng, k):
        y = down(fn(qs, d, n, k, up(x), norm_weight=up(g), norm_eps=1e-6))
        yr, ar = oracle.matvec(qtype, w, n, k, oracle.rmsnorm(x, g, 1e-6))
        check_within(y, yr, oracle.fp32_path_bound(ar), "rmsnorm boundary %s type %d %dx%d" % (name, qtype, n, k))


def test_rmsnorm_fold_ffn_scaling_path_boundary():
    n_ff, k = 1024, 2048
    rng = np.random.default_rng(17)
    wg, wu = synth.q4_0_weights(rng, n_ff, k), synth.q4_0_weights(rng, n_ff, k)
    gw, uw = packed(gq, Q4, wg, n_ff, k), packed(gq, Q4, wu, n_ff, k)
    for name, x, g in _boundary_cases(rng, k):
        h = down(gq.qffn_gate_up_gelu_ex(gw[0], gw[1], uw[0], uw[1], n_ff, k, up(x), norm_weight=up(g),
                                         norm_eps=1e-6))
        ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, oracle.rmsnorm(x, g, 1e-6))
        check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]),
                     "ffn rmsnorm boundary " + name)


@pytest.mark.parametrize("n_ff,k", [(1024, 2048), (300, 8192)])
def test_rmsnorm_fold_ffn_and_vocab_head_full_range(n_ff, k):
    rng = np.random.default_rng(3 * n_ff + k)
    wg, wu = synth.q4_0_weights(rng, n_ff, k), synth.q4_0_weights(rng, n_ff, k)
    gw, uw = packed(gq, Q4, wg, n_ff, k), packed(gq, Q4, wu, n_ff, k)
    g = rng.uniform(0.5, 1.0, k).astype(np.float32)
    wv = synth.q8_0_weights(rng, 4096, k)
    vq = packed(gq, Q8, wv, 4096, k)
    for name, x, eps in _norm_cases(rng, k):
        xn = oracle.rmsnorm(x, g, eps)
        h = down(gq.qffn_gate_up_gelu_ex(gw[0], gw[1], uw[0], uw[1], n_ff, k, up(x), norm_weight=up(g),
                                         norm_eps=eps))
        ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, xn)
        check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]),
                     "ffn rmsnorm " + name)
        idx, val, logits = gq.qmv_q8_0_argmax(vq[0], vq[1], 4096, k, up(x), norm_weight=up(g), norm_eps=eps,
                                              softcap=30.0)
        lg = down(logits)
        yr, ar = oracle.matvec(Q8, wv, 4096, k, xn)
        check_within(lg, oracle.softcap(yr, 30.0), oracle.fp32_path_bound(ar) + 1e-5, "head rmsnorm " + name)
        assert int(down(idx)[0]) == oracle.argmax_f32(lg)
