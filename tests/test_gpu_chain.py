"""Decode-step chaining (gq_chain_*): a step of several entry points is
recorded once on a side stream and replayed as one graph. Every replay is
compared bit for bit with the same sequence run eagerly on the same buffers
(the kernels are deterministic, so a correct replay is identical), with the
program's own eager work and synchronisations between replays, and the
first replay is also checked against the fp64 oracle."""
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


class DecodeStep:
    """quantize -> int-path projection -> norm + gate/up GELU -> down with the
    residual -> norm + vocabulary head with soft cap and argmax."""

    def __init__(self, k=2048, n_q=1024, n_ff=4096, n_vocab=8192, seed=21):
        rng = np.random.default_rng(seed)
        self.k, self.n_q, self.n_ff, self.n_vocab = k, n_q, n_ff, n_vocab
        self.host = {
            "wq": synth.q4_0_weights(rng, n_q, k),
            "wg": synth.q4_0_weights(rng, n_ff, k),
            "wu": synth.q4_0_weights(rng, n_ff, k),
            "wd": synth.q4_0_weights(rng, k, n_ff),
            "wv": synth.q8_0_weights(rng, n_vocab, k),
            "g1": rng.uniform(0.5, 1.5, k).astype(np.float32),
            "g2": rng.uniform(0.5, 1.5, k).astype(np.float32),
        }
        h = self.host
        self.wq = packed(gq, Q4, h["wq"], n_q, k)
        self.wg = packed(gq, Q4, h["wg"], n_ff, k)
        self.wu = packed(gq, Q4, h["wu"], n_ff, k)
        self.wd = packed(gq, Q4, h["wd"], k, n_ff)
        self.wv = packed(gq, Q8, h["wv"], n_vocab, k)
        self.g1, self.g2 = up(h["g1"]), up(h["g2"])
        dev = torch.device("cuda:0")
        f32 = dict(dtype=torch.float32, device=dev)
        self.x = torch.zeros(k, **f32)
        self.xq = torch.empty(k, dtype=torch.int8, device=dev)
        self.xd = torch.empty(k // 32, dtype=torch.int16, device=dev)
        self.yq = torch.empty(n_q, **f32)
        self.hh = torch.empty(n_ff, **f32)
        self.y = torch.empty(k, **f32)
        self.logits = torch.empty(n_vocab, **f32)
        self.ws = torch.empty(gq.argmax_workspace_bytes(), dtype=torch.uint8, device=dev)
        self.idx = torch.empty(1, dtype=torch.int32, device=dev)
        self.val = torch.empty(1, **f32)

    def enqueue(self, s):
        k = self.k
        gq.quantize_q8_0(self.x, xq=self.xq, xd=self.xd, stream=s)
        gq.qmv_q4_0_q8(*self.wq, self.n_q, k, self.xq, self.xd, y=self.yq, stream=s)
        gq.qffn_gate_up_gelu_ex(*self.wg, *self.wu, self.n_ff, k, self.x, norm_weight=self.g1, norm_eps=EPS,
                                h=self.hh, stream=s)
        gq.qmv_q4_0_ex(*self.wd, k, self.n_ff, self.hh, residual=self.x, y=self.y, stream=s)
        gq.qmv_q8_0_argmax(*self.wv, self.n_vocab, k, self.y, norm_weight=self.g2, norm_eps=EPS, softcap=30.0,
                           logits=self.logits, workspace=self.ws, index=self.idx, value=self.val, stream=s)

    def outputs(self):
        return {name: down(getattr(self, name)).copy() for name in
                ("xq", "xd", "yq", "hh", "y", "logits", "idx", "val")}


def _bitwise_equal(a, b):
    assert a.keys() == b.keys()
    for name in a:
        assert np.array_equal(a[name].view(np.uint8), b[name].view(np.uint8)), name


def test_chained_decode_step_replays_match_eager():
    step = DecodeStep()
    s = torch.cuda.Stream()
    rng = np.random.default_rng(5)
    xs = [synth.activations(rng, step.k) for _ in range(4)]
    torch.cuda.synchronize()                # packing ran on the default stream
    with torch.cuda.stream(s):
        step.x.copy_(up(xs[0]))
        step.enqueue(s)                     # eager once (first-call set-up happens outside recording)
        s.synchronize()
        chain = gq.Chain(s)
        with chain:
            step.enqueue(s)
        assert chain.launches == 6          # quantize, q8 matvec, FFN, down, vocab matvec + argmax reduce
        for i, xv in enumerate(xs):
            step.x.copy_(up(xv))
            chain.launch(s)
            s.synchronize()
            replay = step.outputs()
            step.enqueue(s)                 # the same step, eagerly, same buffers
            s.synchronize()
            _bitwise_equal(replay, step.outputs())
            if i == 0:
                h = step.host
                ref = oracle.ffn_gate_up(Q4, h["wg"], h["wu"], step.n_ff, step.k, oracle.rmsnorm(xv, h["g1"], EPS))
                check_within(replay["hh"], ref["h"],
                             oracle.ffn_h_bound(ref["g"], ref["u"], ref["ag"], ref["au"], ref["h"]), "chained h")
                rq, rd = oracle.quantize_q8_0(xv)
                assert np.array_equal(replay["xq"].reshape(-1), rq.reshape(-1))
                yr, ar = oracle.matvec(Q4, h["wd"], step.k, step.n_ff, replay["hh"])
                check_within(replay["y"], xv.astype(np.float64) + yr,
                             oracle.fp32_path_bound(ar) + 1e-6 * np.abs(xv), "chained down + residual")
                assert int(replay["idx"][0]) == oracle.argmax_f32(replay["logits"])
        chain.close()


def test_chained_prefill_tiles():
    rng = np.random.default_rng(8)
    n, k = 4096, 2048
    w = synth.q4_0_weights(rng, n, k)
    qs, d = packed(gq, Q4, w, n, k)
    s = torch.cuda.Stream()
    dev = torch.device("cuda:0")
    ms = (8, 16, 32, 5)
    xf = {m: torch.zeros((m, k), dtype=torch.float32, device=dev) for m in ms}
    xq = {m: torch.empty((m, k), dtype=torch.int8, device=dev) for m in ms}
    xd = {m: torch.empty((m, k // 32), dtype=torch.int16, device=dev) for m in ms}
    y = {m: torch.empty((m, n), dtype=torch.float32, device=dev) for m in ms}

    def enqueue():
        for m in ms:
            gq.quantize_q8_0(xf[m], xq=xq[m], xd=xd[m], stream=s)
            gq.qmm_tile_m(qs, d, n, k, m, xq[m], xd[m], y=y[m], stream=s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        enqueue()
        s.synchronize()
        chain = gq.Chain(s)
        with chain:
            enqueue()
        assert chain.launches == 2 * len(ms)
        for rep in range(3):
            for m in ms:
                xf[m].copy_(up(synth.activations(rng, (m, k))))
            chain.launch(s)
            s.synchronize()
            got = {m: down(y[m]).copy() for m in ms}
            enqueue()
            s.synchronize()
            for m in ms:
                assert np.array_equal(got[m].view(np.uint32), down(y[m]).view(np.uint32)), (rep, m)
            if rep == 0:
                for m in (5, 32):
                    rq, rd = oracle.quantize_q8_0(down(xf[m]))
                    _, yr, ar = oracle.blockdots(Q4, w, n, k, rq, rd, want_s=False)
                    check_within(got[m], yr, oracle.fp32_path_bound(ar), "chained tile m=%d" % m)
        chain.close()


def test_chain_records_nothing_for_a_rejected_call():
    """Validation still runs while recording: a bad call raises and adds no
    launch to the chain."""
    rng = np.random.default_rng(9)
    n, k = 256, 512
    w = synth.q4_0_weights(rng, n, k)
    qs, d = packed(gq, Q4, w, n, k)
    x = up(synth.activations(rng, k))
    y = torch.empty(n, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gq.qmv_q4_0(qs, d, n, k, x, y=y, stream=s)
        s.synchronize()
        chain = gq.Chain(s)
        with chain:
            with pytest.raises(gq.GQError):
                gq.qmv_q4_0(qs, d, n, k + 1, x, y=y, stream=s)
            gq.qmv_q4_0(qs, d, n, k, x, y=y, stream=s)
        assert chain.launches == 1
        y.zero_()
        chain.launch(s)
        s.synchronize()
        yr, ar = oracle.matvec(Q4, w, n, k, down(x))
        check_within(down(y), yr, oracle.fp32_path_bound(ar), "chained single matvec")
        chain.close()


def test_chained_kquant_matvecs():
    """Q4_K, Q5_K and Q6_K matvecs recorded in one chain, replayed with new
    activations: every replay bit-equal to eager calls, and within the bound
    of the oracle."""
    rng = np.random.default_rng(12)
    n, k = 3000, 2304
    s = torch.cuda.Stream()
    ws = {}
    for qtype in (gq.TYPE_Q4_K, gq.TYPE_Q5_K, gq.TYPE_Q6_K):
        w = synth.weights(rng, qtype, n, k)
        ws[qtype] = (w, gq.kq_pack(qtype, up(synth.as_bytes(w).reshape(-1)), n, k))
    x = torch.zeros(k, dtype=torch.float32, device="cuda:0")
    y = {q: torch.empty(n, dtype=torch.float32, device="cuda:0") for q in ws}
    fns = {gq.TYPE_Q4_K: gq.qmv_q4_k, gq.TYPE_Q5_K: gq.qmv_q5_k, gq.TYPE_Q6_K: gq.qmv_q6_k}

    def enqueue():
        for q, (_, p) in ws.items():
            fns[q](p, n, k, x, y=y[q], stream=s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        enqueue()
        s.synchronize()
        chain = gq.Chain(s)
        with chain:
            enqueue()
        assert chain.launches == 3
        for rep in range(3):
            xv = synth.activations(rng, k)
            x.copy_(up(xv))
            chain.launch(s)
            s.synchronize()
            got = {q: down(y[q]).copy() for q in ws}
            enqueue()
            s.synchronize()
            for q in ws:
                assert np.array_equal(got[q].view(np.uint32), down(y[q]).view(np.uint32)), (rep, q)
                if rep == 0:
                    yr, ar = oracle.matvec(q, ws[q][0], n, k, xv)
                    check_within(got[q], yr, oracle.fp32_path_bound(ar), "chained k-quant %d" % q)
        chain.close()
