"""Helpers for the GPU parity tests: move numpy inputs to the device and pack
GGUF block bytes with the library's own pack kernel."""
import numpy as np

import synth


def torch_mod():
    import torch
    return torch


def dev():
    return torch_mod().device("cuda:0")


def up(a):
    """numpy -> device tensor (uint16 scale bits travel as int16)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def down(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def packed(gq, qtype, blocks, n, k):
    """Upload canonical GGUF block bytes and pack them on the device."""
    raw = up(synth.as_bytes(blocks).reshape(-1))
    qs, d = gq.pack(qtype, raw, n, k)
    return qs, d


def check_within(y, y_ref, bound, what):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, "%s: %d of %d outside tolerance; first %s: got %r ref %r bound %r" % (
        what, bad.size, y.size, bad[:3], y.reshape(-1)[bad[:3]], np.asarray(y_ref).reshape(-1)[bad[:3]],
        np.asarray(bound).reshape(-1)[bad[:3]])


def packed_kq(gq, qtype, blocks, n, k):
    """Upload canonical GGUF K-quant super-blocks and pack them on the device."""
    raw = up(synth.as_bytes(blocks).reshape(-1))
    return gq.kq_pack(qtype, raw, n, k)


def check_special(y, yr, ar, what):
    """Finite oracle values: within the fp32-path bound. Non-finite ones (a
    non-finite scale in the row): the GPU value is non-finite too, and where
    both are infinite they have the same sign."""
    import oracle
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    yr = np.asarray(yr, dtype=np.float64).reshape(-1)
    ar = np.asarray(ar, dtype=np.float64).reshape(-1)
    fin_r, fin_g = np.isfinite(yr), np.isfinite(y)
    bad = np.nonzero(fin_r != fin_g)[0]
    assert bad.size == 0, "%s: finiteness differs at %s: got %r ref %r" % (what, bad[:5], y[bad[:5]], yr[bad[:5]])
    inf = np.isinf(y) & np.isinf(yr)
    assert np.array_equal(np.sign(y[inf]), np.sign(yr[inf])), what + ": sign of Inf"
    check_within(y[fin_r], yr[fin_r], oracle.fp32_path_bound(ar[fin_r]), what)
