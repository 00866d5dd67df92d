"""Seeded generators: determinism, shapes and the value distributions the
workloads call for. CPU only."""
import numpy as np

import synth


def test_workloads_are_deterministic_and_shaped():
    a = synth.workload_q4_0_2048()
    b = synth.workload_q4_0_2048()
    assert np.array_equal(synth.as_bytes(a["w"]), synth.as_bytes(b["w"]))
    assert np.array_equal(a["x"], b["x"])
    assert a["w"].shape == (2048, 64) and synth.as_bytes(a["w"]).shape == (2048, 64 * 18)
    c = synth.workload_q8_0_small()
    assert synth.as_bytes(c["w"]).shape == (64, 8 * 34) and c["x"].dtype == np.float32


def test_value_distributions():
    w = synth.workload_q8_0_small()["w"]
    q = w["qs"].astype(int)
    assert q.min() >= -127 and q.max() <= 127 and q.min() < -120 and q.max() > 120
    d = w["d"].view(np.float16).astype(float)
    assert d.min() >= 1e-3 - 1e-6 and d.max() <= 1e-2 + 1e-5
    w4 = synth.workload_q4_0_2048()["w"]
    nib = np.concatenate([w4["qs"] & 15, w4["qs"] >> 4]).reshape(-1)
    counts = np.bincount(nib, minlength=16)
    assert counts.size == 16 and counts.min() > 0.9 * counts.mean()
    rng = np.random.default_rng(0)
    v = synth.q8_0_weights(rng, 64, 2048, dist="normal40", chunk_rows=16)
    qs = v["qs"].astype(float)
    assert 36 < qs.std() < 42 and qs.min() >= -127 and qs.max() <= 127


def test_tile_workload_draw_order():
    t = synth.workload_tile(n=64, k=256)
    assert set(t["acts"]) == {8, 16, 32}
    xq, xd = t["acts"][16]
    assert xq.shape == (16, 256) and xd.shape == (16, 8)
    # a shorter M list draws the same prefix of the stream
    t2 = synth.workload_tile(n=64, k=256, ms=(8,))
    assert np.array_equal(t2["acts"][8][0], t["acts"][8][0])
