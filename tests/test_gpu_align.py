"""GPU: every kernel family at the smallest alignments the C header allows
(scales and activation scales 2-byte aligned, outputs 4-byte aligned) gives
the same bits as the same call on 256-byte aligned buffers, and matches the
fp64 oracle. Offsets come from views one element into a larger buffer."""
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


def shifted(t):
    """A copy of t whose data starts one element past a 256-byte boundary."""
    flat = t.reshape(-1)
    big = torch.empty(flat.numel() + 1, dtype=t.dtype, device=t.device)
    v = big[1:]
    v.copy_(flat)
    return v


def out_shifted(numel, dtype=torch.float32):
    big = torch.full((numel + 1,), float("nan"), dtype=dtype, device="cuda")
    return big[1:]


@pytest.mark.parametrize("qtype,n,k", [(Q8, 65536, 256),     # tall: four rows per wave step
                                       (Q4, 2048, 2048),     # rows in one wave
                                       (Q4, 300, 8192),      # rows split over waves, x staged
                                       (Q8, 64, 32768)])     # the widest split
def test_fp32_matvec_at_minimum_alignment(qtype, n, k):
    rng = np.random.default_rng(n + k)
    w = synth.q8_0_weights(rng, n, k) if qtype == Q8 else synth.q4_0_weights(rng, n, k)
    x = rng.standard_normal(k).astype(np.float32)
    qs, d = packed(gq, qtype, w, n, k)
    fn = gq.qmv_q8_0 if qtype == Q8 else gq.qmv_q4_0
    ref = down(fn(qs, d, n, k, up(x)))
    ds = shifted(d)
    assert ds.data_ptr() % 4 == 2
    y = out_shifted(n)
    assert y.data_ptr() % 8 == 4
    got = down(fn(qs, ds, n, k, up(x), y=y))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(got, yr, oracle.fp32_path_bound(ar), "shifted scales")


@pytest.mark.parametrize("qtype,n,k", [(Q4, 2048, 2048), (Q8, 65536, 256)])
def test_int_matvec_at_minimum_alignment(qtype, n, k):
    rng = np.random.default_rng(7 * n + k)
    w = synth.q8_0_weights(rng, n, k) if qtype == Q8 else synth.q4_0_weights(rng, n, k)
    xq, xd = synth.q8_0_activations(rng, 1, k)
    qs, d = packed(gq, qtype, w, n, k)
    fn = gq.qmv_q8_0_q8 if qtype == Q8 else gq.qmv_q4_0_q8
    ref = down(fn(qs, d, n, k, up(xq[0]), up(xd[0])))
    got = down(fn(qs, shifted(d), n, k, up(xq[0]), shifted(up(xd[0])), y=out_shifted(n)))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_ffn_and_tile_at_minimum_alignment():
    rng = np.random.default_rng(11)
    n_ff, k = 1024, 2048
    wg = synth.q4_0_weights(rng, n_ff, k)
    wu = synth.q4_0_weights(rng, n_ff, k)
    x = rng.standard_normal(k).astype(np.float32)
    g = packed(gq, Q4, wg, n_ff, k)
    u = packed(gq, Q4, wu, n_ff, k)
    ref = down(gq.qffn_gate_up_gelu(g[0], g[1], u[0], u[1], n_ff, k, up(x)))
    got = down(gq.qffn_gate_up_gelu(g[0], shifted(g[1]), u[0], shifted(u[1]), n_ff, k, up(x),
                                    h=out_shifted(n_ff)))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))

    m, n = 16, 512
    w = synth.q4_0_weights(rng, n, k)
    xq, xd = synth.q8_0_activations(rng, m, k)
    qs, d = packed(gq, Q4, w, n, k)
    ref = down(gq.qmm_tile_m(qs, d, n, k, m, up(xq), up(xd)))
    got = down(gq.qmm_tile_m(qs, shifted(d), n, k, m, up(xq), shifted(up(xd)), y=out_shifted(m * n)))
    assert np.array_equal(got.reshape(m, n).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("qtype", [gq.TYPE_Q4_K, gq.TYPE_Q6_K])
def test_kquant_at_minimum_alignment(qtype):
    """K-quant matvec with the packed weights and x 16 bytes past a 256-byte
    boundary and y 4 bytes past one: the same bits as aligned buffers."""
    rng = np.random.default_rng(13 + qtype)
    n, k = 1001, 4096
    w = synth.weights(rng, qtype, n, k)
    x = rng.standard_normal(k).astype(np.float32)
    p = gq.kq_pack(qtype, up(synth.as_bytes(w).reshape(-1)), n, k)
    fn = gq.qmv_q4_k if qtype == gq.TYPE_Q4_K else gq.qmv_q6_k
    ref = down(fn(p, n, k, up(x)))
    pb = torch.empty(p.numel() + 16, dtype=torch.uint8, device="cuda")
    ps = pb[16:]
    ps.copy_(p)
    xb = torch.empty(k + 4, dtype=torch.float32, device="cuda")
    xs = xb[4:]
    xs.copy_(up(x))
    assert ps.data_ptr() % 256 == 16 and xs.data_ptr() % 256 == 16
    y = out_shifted(n)
    got = down(fn(ps, n, k, xs, y=y))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    check_within(got, yr, oracle.fp32_path_bound(ar), "shifted k-quant")
