"""One drop layer driven from plain C (tests/c_driver.c, run as a child
process with only the HIP runtime and libuniprefill.so loaded): the C ABI on
its own, against the CPU oracle.  Inputs come from synth/, expected values
from oracle/; block scores within the parity tolerance, keep flags within
the threshold rule, and compaction, index map, offsets, metadata and the
Eq. 8 scatter-back bit-exact given the GPU's own mask."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT
from gpu_helpers import check_masks, check_scores

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(ROOT, "tests", "c_driver")
MAGIC = 0x31435055
MAX_DROPS = 2
CASES = {
    "two_requests_d64": lambda: synth.tiny((500, 260), hq=4, hkv=2, d=64, G=32, A=8, n=16, p=0.95, seed=3),
    "four_requests_d128": lambda: synth.tiny((3000, 1500, 64, 1), hq=8, hkv=2, d=128, G=64, A=16, n=32,
                                             p=0.9, seed=11, kind="hot", hot=4, hot_lambda=6.0),
    "one_request_d256": lambda: synth.tiny((2600,), hq=4, hkv=2, d=256, G=128, A=32, n=64, p=0.98, seed=7),
}


def write_input(path, wl, cu, q, k, hidden, layer, num_layers, seq_lens):
    T = int(cu[-1])
    rb = hidden.shape[1] * hidden.itemsize
    hdr = np.array([MAGIC, wl.num_reqs, T, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, rb, layer, num_layers],
                   dtype=np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.float64(wl.p).tobytes())
        f.write(np.asarray(cu, np.int32).tobytes())
        f.write(np.asarray(seq_lens, np.int32).tobytes())
        f.write(np.ascontiguousarray(q).tobytes())
        f.write(np.ascontiguousarray(k).tobytes())
        f.write(np.ascontiguousarray(hidden).tobytes())


def read_output(path, R, T, rb, num_layers):
    raw = open(path, "rb").read()
    pos = 0

    def take(dtype, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=pos)
        pos += a.nbytes
        return a

    out = {"status": take(np.int32, 4)}
    mb = int(take(np.int64, 1)[0])
    out["scores"] = take(np.float32, mb)
    out["block_offsets"] = take(np.int32, R + 1)
    out["keep_block"] = take(np.uint8, mb)
    out["mask"] = take(np.uint8, T)
    out["kept"] = take(np.int32, R)
    out["cu_out"] = take(np.int32, R + 1)
    out["index_out"] = take(np.int32, T)
    out["hidden_out"] = take(np.uint8, T * rb).reshape(T, rb)
    out["seq_lens"] = take(np.int32, R)
    out["num_actual"] = int(take(np.int32, 1)[0])
    out["drop_count"] = take(np.int32, R)
    out["drop_layer"] = take(np.int32, R * MAX_DROPS).reshape(R, MAX_DROPS)
    out["drop_len"] = take(np.int32, R * MAX_DROPS).reshape(R, MAX_DROPS)
    out["seqused_base"] = take(np.int32, R * num_layers).reshape(num_layers, R)
    out["full"] = take(np.uint8, T * rb).reshape(T, rb)
    assert pos == len(raw)
    return out


@pytest.mark.parametrize("case", sorted(CASES))
def test_c_driver_matches_oracle(case, tmp_path):
    if not os.path.exists(DRIVER):
        pytest.fail("tests/c_driver is not built (run __graft_entry__.build() or tests/build_c_driver.py)")
    print(f"[c_driver] {case}", flush=True)
    wl = CASES[case]()
    cu, q, k = synth.make_qk(wl)
    R, T = wl.num_reqs, int(cu[-1])
    hidden = synth.hidden_words(np.arange(T), 64)          # 256-byte rows
    rb = hidden.shape[1] * 4
    layer, num_layers = 2, 5
    seq_lens = (np.diff(cu) + np.arange(R) * 7).astype(np.int32)   # some prior context
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    write_input(fin, wl, cu, q, k, hidden, layer, num_layers, seq_lens)
    p = subprocess.run([DRIVER, fin, fout], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, (p.returncode, p.stdout, p.stderr)
    got = read_output(fout, R, T, rb, num_layers)
    assert list(got["status"]) == [0, 0, 0, 0]

    ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    nbt = int(ref["block_offsets"][-1])
    assert np.array_equal(got["block_offsets"], ref["block_offsets"])
    check_scores(got["scores"][:nbt], ref["b64"], ref["block_offsets"])
    check_masks(ref, got["keep_block"][:nbt], got["mask"], got["kept"], cu, wl)

    # compaction of the GPU's own mask, bit-exact
    hid_bytes = hidden.view(np.uint8).reshape(T, rb)
    (rows,), index_out, cu_out = oracle.compact(got["mask"], cu, [hid_bytes])
    K = len(index_out)
    assert np.array_equal(got["cu_out"], cu_out)
    assert np.array_equal(got["index_out"][:K], index_out)
    assert np.array_equal(got["hidden_out"][:K], rows)

    # metadata after the drop at `layer`
    st, nat = oracle.update_metadata(oracle.MetadataState.fresh(seq_lens), layer, cu, cu_out)
    assert np.array_equal(got["seq_lens"], st.seq_lens) and got["num_actual"] == nat
    assert (got["drop_count"] == 1).all()
    assert (got["drop_layer"][:, 0] == layer).all() and (got["drop_layer"][:, 1] == -1).all()
    assert np.array_equal(got["drop_len"][:, 0], st.seq_lens) and (got["drop_len"][:, 1] == -1).all()
    for lp in range(num_layers):
        want = st.seq_lens if lp > layer else seq_lens
        assert np.array_equal(got["seqused_base"][lp], want), lp

    # Eq. 8: kept rows carried back, every other row untouched (0xEE)
    full_ref = oracle.scatter_back(np.full((T, rb), 0xEE, np.uint8), rows, index_out, K)
    assert np.array_equal(got["full"], full_ref)
