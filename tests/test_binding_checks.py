"""The Python binding refuses tensors that are too short or of the wrong
dtype before calling the C ABI (which only sees pointers, so such a buffer
would be read or written out of bounds on the device). Host only: the size
and dtype checks run before the device check, so CPU tensors exercise them
and a correctly sized CPU tensor gets as far as "must be a device tensor"."""
import pytest

torch = pytest.importorskip("torch")
gq = pytest.importorskip("gguf_block_quant_amd")

N, K = 64, 256
NB = K // 32


def t(n, dtype=torch.float32):
    return torch.zeros(n, dtype=dtype)


def weights(qtype=gq.TYPE_Q8_0, n=N, k=K):
    qb = n * k if qtype == gq.TYPE_Q8_0 else n * k // 2
    return t(qb, torch.int8 if qtype == gq.TYPE_Q8_0 else torch.uint8), t(n * (k // 32), torch.int16)


def refused(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_correct_sizes_reach_the_device_check():
    qs, d = weights()
    refused("must be a device tensor", gq.qmv_q8_0, qs, d, N, K, t(K), y=t(N))


@pytest.mark.parametrize("qtype,fn", [(gq.TYPE_Q8_0, gq.qmv_q8_0), (gq.TYPE_Q4_0, gq.qmv_q4_0)])
def test_qmv_short_and_mistyped(qtype, fn):
    qs, d = weights(qtype)
    refused("x holds", fn, qs, d, N, K, t(K - 1), y=t(N))
    refused("y holds", fn, qs, d, N, K, t(K), y=t(N - 1))
    refused("qs holds", fn, qs[:-1], d, N, K, t(K), y=t(N))
    refused("d holds", fn, qs, d[:-1], N, K, t(K), y=t(N))
    refused("x must have dtype", fn, qs, d, N, K, t(K, torch.float64), y=t(N))
    refused("y must have dtype", fn, qs, d, N, K, t(K), y=t(N, torch.float16))
    refused("d must have dtype", fn, qs, d.float(), N, K, t(K), y=t(N))


def test_q8_paths():
    qs, d = weights(gq.TYPE_Q4_0)
    xq, xd = t(K, torch.int8), t(NB, torch.int16)
    refused("xq holds", gq.qmv_q4_0_q8, qs, d, N, K, xq[:-1], xd, y=t(N))
    refused("xd holds", gq.qmv_q4_0_q8, qs, d, N, K, xq, xd[:-1], y=t(N))
    refused("xq must have dtype", gq.qmv_q4_0_q8, qs, d, N, K, xq.to(torch.uint8), xd, y=t(N))
    refused("blockdots holds", gq.qmv_q4_0_q8, qs, d, N, K, xq, xd, y=t(N), blockdots=t(N * NB - 1, torch.int32))
    refused("blockdots must have dtype", gq.qmv_q4_0_q8, qs, d, N, K, xq, xd, y=t(N),
            blockdots=t(N * NB, torch.float32))
    refused("xq_out holds", gq.qmv_q4_0_q8x, qs, d, N, K, t(K), y=t(N), xq_out=xq[:-1], xd_out=xd)
    refused("xd_out holds", gq.qmv_q4_0_q8x, qs, d, N, K, t(K), y=t(N), xq_out=xq, xd_out=xd[:-1])


def test_folds_and_argmax():
    qs, d = weights()
    refused("norm_weight holds", gq.qmv_q8_0_ex, qs, d, N, K, t(K), norm_weight=t(K - 4), y=t(N))
    refused("residual holds", gq.qmv_q8_0_ex, qs, d, N, K, t(K), residual=t(N - 1), y=t(N))
    ws = t(gq.argmax_workspace_bytes(), torch.uint8)
    refused("workspace holds", gq.qmv_q8_0_argmax, qs, d, N, K, t(K), logits=t(N), workspace=ws[:-8],
            index=t(1, torch.int32), value=t(1))
    refused("index must have dtype", gq.qmv_q8_0_argmax, qs, d, N, K, t(K), logits=t(N), workspace=ws,
            index=t(1, torch.int64), value=t(1))
    refused("logits holds", gq.qmv_q8_0_argmax, qs, d, N, K, t(K), logits=t(N - 1), workspace=ws,
            index=t(1, torch.int32), value=t(1))


def test_ffn_tile_pack_quantize():
    qs, d = weights(gq.TYPE_Q4_0)
    refused("u_qs holds", gq.qffn_gate_up_gelu, qs, d, qs[:-1], d, N, K, t(K), h=t(N))
    refused("h holds", gq.qffn_gate_up_gelu, qs, d, qs, d, N, K, t(K), h=t(N - 1))
    m = 8
    refused("xq holds", gq.qmm_tile_m, qs, d, N, K, m, t(m * K - 1, torch.int8), t(m * NB, torch.int16),
            y=t(m * N))
    refused("y holds", gq.qmm_tile_m, qs, d, N, K, m, t(m * K, torch.int8), t(m * NB, torch.int16),
            y=t(m * N - 1))
    blocks = t(N * NB * 18 - 1, torch.uint8)
    refused("blocks holds", gq.pack, gq.TYPE_Q4_0, blocks, N, K, qs=qs, d=d)
    refused("xq holds", gq.quantize_q8_0, t(K), xq=t(K - 1, torch.int8), xd=t(NB, torch.int16))
