"""The seeded generators (CPU): one request generated on its own is
bit-identical to its rows in the whole batch, and the varlen batch's
calibrated structure keeps the spread of keep ratios it was calibrated for
(measured with the oracle)."""
import numpy as np

import oracle
import synth


def test_request_alone_matches_batch_rows():
    wl = synth.tiny((300, 0, 129, 77), hq=8, hkv=2, d=64, seed=3)
    cu, q, k = synth.make_qk(wl)
    for r in range(wl.num_reqs):
        qr, kr = synth.make_request_qk(wl, r)
        assert np.array_equal(qr, q[cu[r]:cu[r + 1]]) and np.array_equal(kr, k[cu[r]:cu[r + 1]]), r


def test_varlen_batch_keep_ratios_span_the_range():
    wl = synth.llama_varlen4()
    cu, q, k = synth.make_qk(wl)
    sel = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    ratios = [int(sel["kept"][r]) / int(cu[r + 1] - cu[r]) for r in range(wl.num_reqs)]
    assert abs(ratios[0] - 0.10) < 0.02 and abs(ratios[1] - 0.35) < 0.03 and abs(ratios[2] - 0.60) < 0.03, ratios
    assert abs(ratios[3] - 0.90) < 0.02, ratios
