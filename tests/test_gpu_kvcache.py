"""GPU parity of the Eq. 16 slot mapping and the paged KV-cache write against
the CPU oracle: bit-exact slots and cache contents on seeded inputs, from the
hand-worked fixture up to the 16 x 128K serving batch (sampled requests
checked one by one, properties checked for all)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import ROOT
from gpu_helpers import dev

tlb = pytest.importorskip("token_level_block_amd")

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def gpu_slots(table, B, cu, seq_lens, max_tokens, width=None):
    table = np.asarray(table, dtype=np.int32)
    R = len(cu) - 1
    width = table.shape[1] if width is None else width
    t = dev(table) if table.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((max(max_tokens, 1),), 7777, dtype=torch.int64, device="cuda")
    seq = np.asarray(seq_lens, np.int32) if len(seq_lens) else np.zeros(1, np.int32)
    tlb.slot_mapping(t, table.shape[1] if table.ndim == 2 else 0, width, B, dev(np.asarray(cu, np.int32)),
                     dev(seq), R, max_tokens, out)
    torch.cuda.synchronize()
    return out[:max_tokens].cpu().numpy()


def random_case(rng, R, B, width, neg_frac=0.0, short_table=False):
    kept = rng.integers(0, 4 * B + 9, size=R)
    kept[rng.random(R) < 0.2] = 0
    ctx = rng.integers(0, 3 * B + 5, size=R)
    cu = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    seq = (ctx + kept).astype(np.int32)
    need = int(((seq + B - 1) // B).max()) if R else 0
    w = max(1, need - 1) if short_table else max(width, need)
    table = rng.permutation(R * w + 17)[: R * w].reshape(R, w).astype(np.int32)
    table[rng.random(table.shape) < neg_frac] = -1
    return cu, seq, table


def test_slot_fixture_through_gpu():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "eq16_slot_example.json")))
    s = gpu_slots(g["block_table"], g["B"], g["cu_seqlens"], g["seq_lens"], g["max_tokens"])
    assert list(s) == g["slots"]


@pytest.mark.parametrize("seed,R,B,neg,short", [
    (0, 1, 16, 0.0, False), (1, 5, 16, 0.0, False), (2, 8, 1, 0.0, False), (3, 7, 5, 0.1, False),
    (4, 6, 64, 0.0, True), (5, 12, 16, 0.05, True), (6, 3, 3, 0.0, False), (7, 0, 16, 0.0, False)])
def test_slot_mapping_matches_oracle(seed, R, B, neg, short):
    rng = np.random.default_rng(seed)
    cu, seq, table = random_case(rng, R, B, width=6, neg_frac=neg, short_table=short)
    T = int(cu[-1])
    mt = T + 37
    ref = oracle.slot_mapping(table, B, cu, seq, mt) if R else np.full(mt, -1)
    got = gpu_slots(table, B, cu, seq, mt) if R else gpu_slots(np.zeros((0, 0)), B, cu, seq, mt, width=0)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]


def test_slot_mapping_narrower_width_than_stride():
    """Only the first max_blocks_per_req columns of each table row are used."""
    rng = np.random.default_rng(9)
    cu, seq, table = random_case(rng, 4, 8, width=10)
    w = 3
    ref = oracle.slot_mapping(table[:, :w], 8, cu, seq)
    got = gpu_slots(table, 8, cu, seq, int(cu[-1]), width=w)
    assert np.array_equal(got, ref)


def write_case(rng, rows, rb, nslots, strided, with_value):
    words = rb // 4
    stride_words = words + (8 if strided else 0)
    key = rng.integers(0, 2 ** 32, size=(rows, stride_words), dtype=np.uint64).astype(np.uint32)
    val = rng.integers(0, 2 ** 32, size=(rows, stride_words), dtype=np.uint64).astype(np.uint32)
    slots = rng.permutation(nslots + 24)[:rows].astype(np.int64) - 12   # some negative, some past the cache
    return key, val, slots, stride_words


@pytest.mark.parametrize("rb,strided,with_value", [
    (4, False, True), (12, True, True), (16, False, True), (2048, False, True), (2048, True, True),
    (4096, False, False), (2064, False, True), (1024, True, False), (8208, False, True), (8192, True, True)])
def test_kv_write_matches_oracle(rb, strided, with_value):
    rng = np.random.default_rng(rb + strided)
    rows, nslots = 300, 512
    key, val, slots, sw = write_case(rng, rows, rb, nslots, strided, with_value)
    count = rows - 11
    cu = np.array([0, 100, 100, count], dtype=np.int32)
    words = rb // 4
    kc0 = np.full((nslots, words), 0xDEADBEEF, dtype=np.uint32)
    vc0 = np.full((nslots, words), 0x0BADF00D, dtype=np.uint32)
    ref_k, ref_v = oracle.write_kv_cache(kc0, vc0 if with_value else None, slots, key[:, :words],
                                         val[:, :words], count)
    kd, vd = dev(key.view(np.int32)), dev(val.view(np.int32))
    kcd, vcd = dev(kc0.view(np.int32)), dev(vc0.view(np.int32))
    tlb.write_kv_cache(kd, sw * 4, vd if with_value else None, sw * 4, rb, dev(slots), dev(cu), 3, rows,
                       kcd, vcd if with_value else None, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(kcd.cpu().numpy().view(np.uint32), ref_k)
    if with_value:
        assert np.array_equal(vcd.cpu().numpy().view(np.uint32), ref_v)
    else:
        assert np.array_equal(vcd.cpu().numpy().view(np.uint32), vc0)


def test_slots_and_cache_128k_layer():
    """The 128K LLaMA layer after a 40 % keep: 52608 retained rows, KV block
    size 16, K and V rows of 8 heads x 128 bf16 (2 KiB), a shuffled block
    table; slots bit-exact, every written cache row equal to its K/V row and
    every other row untouched."""
    rng = np.random.default_rng(128)
    kept, B, rb = 52608, 16, 2048
    cu = np.array([0, kept], dtype=np.int32)
    seq = np.array([kept], dtype=np.int32)
    nblk = kept // B + 40
    table = rng.permutation(nblk)[None, :].astype(np.int32)
    ref = oracle.slot_mapping(table, B, cu, seq, kept + 5)
    got = gpu_slots(table, B, cu, seq, kept + 5)
    assert np.array_equal(got, ref)
    key = torch.randint(-2 ** 31, 2 ** 31 - 1, (kept, rb // 4), dtype=torch.int32, device="cuda")
    val = torch.randint(-2 ** 31, 2 ** 31 - 1, (kept, rb // 4), dtype=torch.int32, device="cuda")
    kc = torch.full((nblk * B, rb // 4), -3, dtype=torch.int32, device="cuda")
    vc = torch.full_like(kc, -4)
    sl = dev(ref)
    tlb.write_kv_cache(key, rb, val, rb, rb, sl, dev(cu), 1, kept + 5, kc, vc, nblk * B)
    torch.cuda.synchronize()
    s = sl[:kept]
    assert torch.equal(kc[s], key) and torch.equal(vc[s], val)
    untouched = torch.ones(nblk * B, dtype=torch.bool, device="cuda")
    untouched[s] = False
    assert bool((kc[untouched] == -3).all()) and bool((vc[untouched] == -4).all())


@pytest.mark.timeout(600)
def test_slots_serving_16x128k():
    """16 requests of the serving batch after a drop (retained lengths from
    the batch's keep ratios, prior context on some), KV block size 16 and a
    separate table per request, two layers with different tables (as a
    global and a sliding-window layer would have): two sampled requests per
    layer through the oracle one by one; for all rows, slots are unique,
    sit at offset p mod B of the block the table names, and the cache write
    lands every K row at its slot."""
    rng = np.random.default_rng(4)
    R, B = 16, 16
    rho = rng.uniform(0.2, 0.9, size=R)
    kept = np.round(rho * 131072).astype(np.int64)
    ctx = np.where(rng.random(R) < 0.3, rng.integers(0, 4096, size=R), 0)
    cu = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    seq = (ctx + kept).astype(np.int32)
    T = int(cu[-1])
    width = int(((seq + B - 1) // B).max())
    for layer, samples in ((0, (2, 11)), (1, (5, 15))):
        table = rng.permutation(R * width).reshape(R, width).astype(np.int32)
        got = gpu_slots(table, B, cu, seq, T)
        for r in samples:
            ref = oracle.slot_mapping(table[r:r + 1], B, [0, int(kept[r])], seq[r:r + 1])
            assert np.array_equal(got[cu[r]:cu[r + 1]], ref), (layer, r)
        assert (got >= 0).all()
        assert len(np.unique(got)) == T
        p = np.concatenate([ctx[r] + np.arange(kept[r]) for r in range(R)])
        owner = np.repeat(np.arange(R), kept)
        assert np.array_equal(got % B, p % B)
        assert np.array_equal(got // B, table[owner, p // B])
        say(f"  layer {layer}: {T} slots checked")
    # cache write of 4-word rows (the full 2 KiB rows would need 2 x 4.6 GB)
    key = torch.arange(T, dtype=torch.int32, device="cuda")[:, None].repeat(1, 4)
    kc = torch.full((R * width * B, 4), -1, dtype=torch.int32, device="cuda")
    sl = dev(got)
    tlb.write_kv_cache(key, 16, None, 0, 16, sl, dev(cu), R, T, kc, None, R * width * B)
    torch.cuda.synchronize()
    assert torch.equal(kc[sl], key)
    assert int((kc[:, 0] >= 0).sum().item()) == T
