"""GPU: the allocation-free vocabulary head (gq_qmv_q8_0_argmax_noalloc),
called through the C ABI, gives the same logits, index and value as
gq_qmv_q8_0_argmax with a caller workspace, bit for bit, on two calls in a
row (the second on a smaller input, so the library-held partials still hold
the first call's keys when it starts), and matches the fp64 oracle."""
import ctypes

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

Q8 = gq.TYPE_Q8_0


def _noalloc_c(qs, d, n, k, x, g, eps, cap):
    """Call the entry point through the C ABI with raw pointers."""
    logits = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    index = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    value = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    st = gq.raw().gq_qmv_q8_0_argmax_noalloc(P(qs), P(d), n, k, P(x), P(g), ctypes.c_float(eps),
                                             ctypes.c_float(cap), P(logits), P(index), P(value),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, gq.status_str(st)
    return index, value, logits


@pytest.mark.parametrize("with_norm", [False, True])
def test_noalloc_matches_workspace_entry_two_calls(with_norm):
    rng = np.random.default_rng(31 + with_norm)
    cases = [(131072, 2048, 30.0), (3001, 1024, 0.0)]      # second call smaller
    for n, k, cap in cases:
        w = synth.q8_0_weights(rng, n, k, dist="normal40")
        x = synth.activations(rng, k)
        g = rng.uniform(0.5, 1.5, k).astype(np.float32) if with_norm else None
        qs, d = packed(gq, Q8, w, n, k)
        xt, gt = up(x), (up(g) if g is not None else None)
        i0, v0, l0 = _noalloc_c(qs, d, n, k, xt, gt, 1e-6, cap)
        i1, v1, l1 = gq.qmv_q8_0_argmax(qs, d, n, k, xt, norm_weight=gt, norm_eps=1e-6, softcap=cap)
        torch.cuda.synchronize()
        a0, a1 = down(l0), down(l1)
        assert np.array_equal(a0.view(np.uint32), a1.view(np.uint32)), (n, k)
        assert int(down(i0)[0]) == int(down(i1)[0]) == oracle.argmax_f32(a0), (n, k)
        assert down(v0).view(np.uint32)[0] == down(v1).view(np.uint32)[0]
        assert down(v0)[0] == a0[int(down(i0)[0])]
        rows = np.unique(np.concatenate([rng.integers(0, n, 64), [0, n - 1, int(down(i0)[0])]]))
        xn = oracle.rmsnorm(x, g, 1e-6) if with_norm else x
        yr, ar = oracle.matvec_rows(Q8, w, n, k, rows, xn)
        check_within(a0[rows], oracle.softcap(yr, cap), oracle.fp32_path_bound(ar) + 1e-5, "noalloc head")
