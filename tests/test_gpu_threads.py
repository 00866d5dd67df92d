"""The library is reentrant: host threads calling entry points at the same
time, each on its own stream, get exactly the results of the same calls made
one after another (the binding releases the interpreter lock for the C call,
so validation, the per-kernel occupancy set-up and the launches overlap)."""
import threading

import numpy as np
import pytest

import synth
from gpu_util import down, packed, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_block_quant_amd as gq  # noqa: E402

Q4, Q8 = gq.TYPE_Q4_0, gq.TYPE_Q8_0


def test_concurrent_host_threads_match_serial_calls():
    rng = np.random.default_rng(31)
    cases = []
    for i, (qtype, n, k) in enumerate([(Q8, 3000, 2048), (Q4, 2048, 8192), (Q4, 4096, 2048), (Q8, 512, 32768)]):
        w = synth.weights(rng, qtype, n, k)
        qs, d = packed(gq, qtype, w, n, k)
        x = up(synth.activations(rng, k))
        cases.append((qtype, n, k, qs, d, x))
    wt = synth.q4_0_weights(rng, 1024, 2048)
    tqs, td = packed(gq, Q4, wt, 1024, 2048)
    txq, txd = synth.q8_0_activations(rng, 8, 2048)
    txq, txd = up(txq), up(txd)
    kq = {}
    for qtype in (gq.TYPE_Q4_K, gq.TYPE_Q6_K):
        wk = synth.weights(rng, qtype, 2048, 4096)
        kq[qtype] = gq.kq_pack(qtype, up(synth.as_bytes(wk).reshape(-1)), 2048, 4096)
    kx = up(synth.activations(rng, 4096))
    torch.cuda.synchronize()

    def run(case_id, stream, out):
        qtype, n, k, qs, d, x = cases[case_id]
        fn = gq.qmv_q8_0 if qtype == Q8 else gq.qmv_q4_0
        fx = gq.qmv_q8_0_q8x if qtype == Q8 else gq.qmv_q4_0_q8x
        for rep in range(10):
            out.append(fn(qs, d, n, k, x, stream=stream))
            out.append(fx(qs, d, n, k, x, stream=stream))
            out.append(gq.qmm_tile_m(tqs, td, 1024, 2048, 8, txq, txd, stream=stream))
            out.append(gq.qmv_q4_k(kq[gq.TYPE_Q4_K], 2048, 4096, kx, stream=stream))
            out.append(gq.qmv_q6_k(kq[gq.TYPE_Q6_K], 2048, 4096, kx, stream=stream))

    # serial reference on the default stream
    ref = []
    for cid in range(len(cases)):
        r = []
        run(cid, torch.cuda.current_stream(), r)
        ref.append(r)
    torch.cuda.synchronize()
    ref = [[down(t).copy() for t in r] for r in ref]

    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[] for _ in cases]
    errors = []

    def worker(cid):
        try:
            run(cid, streams[cid], outs[cid])
        except Exception as e:      # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(cid,)) for cid in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for cid in range(len(cases)):
        assert len(outs[cid]) == len(ref[cid])
        for a, b in zip(outs[cid], ref[cid]):
            assert np.array_equal(down(a).view(np.uint32), b.view(np.uint32)), cid
