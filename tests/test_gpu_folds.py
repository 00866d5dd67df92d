"""GPU parity for the folds around a decode projection: the RMSNorm prologue,
the residual epilogue, and the vocabulary head's soft cap + greedy argmax,
each against the fp64 oracle on seeded inputs."""
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
EPS = 1e-6


def _ex(qtype):
    return gq.qmv_q8_0_ex if qtype == Q8 else gq.qmv_q4_0_ex


def _case(qtype, n, k, seed):
    rng = np.random.default_rng(seed)
    w = synth.weights(rng, qtype, n, k)
    x = (synth.activations(rng, k) * np.float32(3.0)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, k).astype(np.float32)
    res = synth.activations(rng, n)
    return w, x, g, res


FOLD_SHAPES = [(Q8, 64, 256), (Q4, 2048, 2048), (Q4, 2048, 8192), (Q8, 300, 1056), (Q4, 64, 32768),
               (Q8, 515, 4096), (Q4, 1, 32), (Q4, 1001, 8192), (Q8, 77, 16384)]
# at least 16 MiB of quants: four rows per wave step, rows finished on separate lanes (ragged last group)
TALL_FOLD_SHAPES = [(Q8, 8195, 2048), (Q4, 16385, 2048)]


@pytest.mark.parametrize("qtype,n,k", FOLD_SHAPES + TALL_FOLD_SHAPES)
def test_rmsnorm_prologue(qtype, n, k):
    w, x, g, _ = _case(qtype, n, k, n + k)
    qs, d = packed(gq, qtype, w, n, k)
    y = down(_ex(qtype)(qs, d, n, k, up(x), norm_weight=up(g), norm_eps=EPS))
    xn = oracle.rmsnorm(x, g, EPS)
    yr, ar = oracle.matvec(qtype, w, n, k, xn)
    check_within(y, yr, oracle.fp32_path_bound(ar), "rmsnorm prologue")


@pytest.mark.parametrize("qtype,n,k", FOLD_SHAPES[:4] + TALL_FOLD_SHAPES)
def test_residual_epilogue_and_in_place(qtype, n, k):
    w, x, g, res = _case(qtype, n, k, 3 * n + k)
    qs, d = packed(gq, qtype, w, n, k)
    yr, ar = oracle.matvec(qtype, w, n, k, x)
    bound = oracle.fp32_path_bound(ar) + 1e-6 * np.abs(res)
    y = down(_ex(qtype)(qs, d, n, k, up(x), residual=up(res)))
    check_within(y, res.astype(np.float64) + yr, bound, "residual")
    # in place: y is the residual buffer
    acc = up(res)
    _ex(qtype)(qs, d, n, k, up(x), residual=acc, y=acc)
    assert np.array_equal(down(acc).view(np.uint32), y.view(np.uint32))
    # both folds together, and the plain entry is the _ex entry with no folds
    y2 = down(_ex(qtype)(qs, d, n, k, up(x), norm_weight=up(g), norm_eps=EPS, residual=up(res)))
    yr2, ar2 = oracle.matvec(qtype, w, n, k, oracle.rmsnorm(x, g, EPS))
    check_within(y2, res.astype(np.float64) + yr2, oracle.fp32_path_bound(ar2) + 1e-6 * np.abs(res), "both")
    plain = gq.qmv_q8_0 if qtype == Q8 else gq.qmv_q4_0
    assert np.array_equal(down(plain(qs, d, n, k, up(x))).view(np.uint32),
                          down(_ex(qtype)(qs, d, n, k, up(x))).view(np.uint32))


@pytest.mark.parametrize("n_ff,k", [(8192, 2048), (1056, 8192), (65539, 2048)])   # the last: tall shape
def test_ffn_rmsnorm_prologue(n_ff, k):
    # gate, up and x only (no down matrix: n_ff need not be a whole number of blocks)
    rng = np.random.default_rng(5)
    wg = synth.q4_0_weights(rng, n_ff, k)
    wu = synth.q4_0_weights(rng, n_ff, k)
    x = synth.activations(rng, k)
    gw = np.random.default_rng(6).uniform(0.5, 1.5, k).astype(np.float32)
    gt = packed(gq, Q4, wg, n_ff, k)
    ut = packed(gq, Q4, wu, n_ff, k)
    h = down(gq.qffn_gate_up_gelu_ex(gt[0], gt[1], ut[0], ut[1], n_ff, k, up(x), norm_weight=up(gw), norm_eps=EPS))
    ref = oracle.ffn_gate_up(Q4, wg, wu, n_ff, k, oracle.rmsnorm(x, gw, EPS))
    check_within(h, ref["h"], oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]), "ffn norm")


def _argmax(qtype):
    return gq.qmv_q8_0_argmax if qtype == Q8 else gq.qmv_q4_0_argmax


def test_vocab_head_full_size():
    """The Q8_0 vocabulary projection with the soft cap and greedy argmax, at
    262144 x 2048: logits within the bound (tanh is 1-Lipschitz, so the cap
    does not widen it), the index exactly the argmax of the GPU's own logits,
    and a valid argmax of the exact logits."""
    wl = synth.workload_vocab()
    n, k, w, x = wl["n"], wl["k"], wl["w"], wl["x"]
    qs, d = packed(gq, Q8, w, n, k)
    idx, val, logits = _argmax(Q8)(qs, d, n, k, up(x), softcap=30.0)
    lg = down(logits)
    i, v = int(down(idx)[0]), float(down(val)[0])
    yr, ar = oracle.matvec(Q8, w, n, k, x)
    lr = 30.0 * np.tanh(yr / 30.0)
    bound = oracle.fp32_path_bound(ar) + 4 * np.spacing(np.float32(30.0))
    check_within(lg, lr, bound, "capped logits")
    assert i == oracle.argmax_f32(lg) and v == lg[i]
    assert lr[i] >= lr.max() - 2 * bound.max()
    # no cap: the logits are the plain matvec bit for bit
    _, _, raw = _argmax(Q8)(qs, d, n, k, up(x), softcap=0.0)
    assert np.array_equal(down(raw).view(np.uint32), down(gq.qmv_q8_0(qs, d, n, k, up(x))).view(np.uint32))


@pytest.mark.parametrize("qtype,n,k", [(Q8, 5000, 256), (Q4, 3000, 2048), (Q4, 700, 8192), (Q8, 1, 32),
                                       (Q8, 8195, 2048)])
def test_argmax_ties_go_to_lowest_row(qtype, n, k):
    rng = np.random.default_rng(n)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    yr, _ = oracle.matvec(qtype, w, n, k, x)
    src = int(np.argmax(yr))
    top = sorted({src, 0, n - 1, n // 2})
    for r in top:
        w[r] = w[src]                                      # identical rows -> identical logits
    qs, d = packed(gq, qtype, w, n, k)
    idx, val, logits = _argmax(qtype)(qs, d, n, k, up(x), softcap=30.0)
    lg = down(logits)
    i = int(down(idx)[0])
    assert i == oracle.argmax_f32(lg)
    assert all(lg[r] == lg[top[0]] for r in top)
    assert i == top[0] and float(down(val)[0]) == lg[i]


def test_argmax_nan_and_norm():
    n, k = 4096, 2048
    w, x, g, _ = _case(Q8, n, k, 11)
    qs, d = packed(gq, Q8, w, n, k)
    xn = x.copy()
    xn[7] = np.nan
    idx, val, logits = _argmax(Q8)(qs, d, n, k, up(xn), softcap=30.0)
    assert int(down(idx)[0]) == 0 and np.isnan(down(val)[0]) and np.all(np.isnan(down(logits)))
    # with the final norm folded in
    idx, val, logits = _argmax(Q8)(qs, d, n, k, up(x), norm_weight=up(g), norm_eps=EPS, softcap=30.0)
    lg = down(logits)
    yr, ar = oracle.matvec(Q8, w, n, k, oracle.rmsnorm(x, g, EPS))
    check_within(lg, 30.0 * np.tanh(yr / 30.0), oracle.fp32_path_bound(ar) + 1e-5, "norm + cap")
    assert int(down(idx)[0]) == oracle.argmax_f32(lg)


@pytest.mark.parametrize("qtype,n,k", [(Q8, 262144, 256), (Q4, 300000, 64)])
def test_argmax_stays_inside_its_workspace(qtype, n, k):
    """The first stage writes one key per workgroup into the caller's
    workspace: at the largest grid (a tall matrix) every write stays inside
    gq_argmax_workspace_bytes(); the bytes after it are untouched."""
    rng = np.random.default_rng(n + k)
    w = synth.weights(rng, qtype, n, k)
    x = synth.activations(rng, k)
    qs, d = packed(gq, qtype, w, n, k)
    wsb = gq.argmax_workspace_bytes()
    buf = torch.full((wsb + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    ws = buf[:wsb]
    idx, val, logits = _argmax(qtype)(qs, d, n, k, up(x), softcap=0.0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(buf[wsb:] == 0xAB).item()
    lg = down(logits)
    assert int(down(idx)[0]) == oracle.argmax_f32(lg)


@pytest.mark.parametrize("qtype,n,k", [(Q8, 262144, 2048), (Q4, 5000, 1024), (Q8, 7, 64)])
def test_argmax_calls_in_a_row_share_one_workspace(qtype, n, k):
    """One workspace, many calls in a row with new activations: every call's
    index and value are those of its own logits, never a stale partial."""
    rng = np.random.default_rng(3 * n + k)
    w = synth.weights(rng, qtype, n, k)
    qs, d = packed(gq, qtype, w, n, k)
    ws = torch.full((gq.argmax_workspace_bytes(),), 0xFF, dtype=torch.uint8, device="cuda")
    for call in range(6):
        x = synth.activations(rng, k)
        idx, val, logits = _argmax(qtype)(qs, d, n, k, up(x), softcap=30.0 if call % 2 else 0.0, workspace=ws)
        lg = down(logits)
        i = int(down(idx)[0])
        assert i == oracle.argmax_f32(lg), call
        assert down(val).view(np.uint32)[0] == lg.view(np.uint32)[i]
