"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input comes from the seeded generators in synth/ (or is drawn here from
a seeded NumPy generator); every expected value comes from oracle/.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import token_level_block_amd as tlb  # noqa: E402
from token_level_block_amd.runner import CompactBuffers, MetadataBuffers, SelectBuffers, run_scatter_back  # noqa: E402

from gpu_helpers import check_masks, check_scores, dev, upload_qk  # noqa: E402
from oracle_pool import OraclePool  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_select(wl, cu, q, k, max_tokens=None, scale=0.0, bufs=None):
    T = int(cu[-1])
    max_tokens = T if max_tokens is None else max_tokens
    if bufs is None:
        prm = tlb.make_params(wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p, softmax_scale=scale)
        bufs = SelectBuffers.allocate(prm, wl.num_reqs, max_tokens)
    bufs.keep_mask.fill_(0xAB)
    cu_d, qd, kd = upload_qk(wl, cu, q, k)
    bufs.run(qd, kd, cu_d)
    torch.cuda.synchronize()
    offs = bufs.block_offsets[: wl.num_reqs + 1].cpu().numpy()
    nbt = int(offs[-1])
    return dict(
        offs=offs,
        b=bufs.block_scores[:nbt].cpu().numpy(),
        keep=bufs.keep_block[:nbt].cpu().numpy(),
        mask=bufs.keep_mask[:T].cpu().numpy(),
        kept=bufs.kept[: wl.num_reqs].cpu().numpy(),
        bufs=bufs,
    )


def check_select(wl, label=""):
    say(f"[select] {label} {wl.name} lengths={wl.lengths[:6]} hq={wl.hq} hkv={wl.hkv} d={wl.d} G={wl.G} "
        f"A={wl.A} n={wl.n} p={wl.p}")
    cu, q, k = synth.make_qk(wl)
    ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    got = run_select(wl, cu, q, k)
    assert np.array_equal(got["offs"], ref["block_offsets"])
    check_scores(got["b"], ref["b64"], ref["block_offsets"])
    mism = check_masks(ref, got["keep"], got["mask"], got["kept"], cu, wl)
    return ref, got, mism


TINY_CASES = [
    # lengths, hq, hkv, d, G, A, n, p, kind
    ((40,), 4, 2, 64, 32, 8, 8, 0.9, "hot"),
    ((1, 5, 33, 64, 65, 100), 4, 1, 64, 32, 4, 8, 0.95, "hot"),
    ((0, 300, 0, 129), 8, 2, 128, 32, 16, 16, 0.99, "powerlaw"),
    ((2500,), 8, 2, 128, 64, 128, 128, 0.99, "powerlaw"),
    ((1100, 3000, 77), 4, 4, 128, 64, 32, 100, 0.9, "hot"),
    ((5000,), 16, 2, 256, 128, 128, 128, 0.99, "powerlaw"),
    ((700, 1500), 16, 8, 256, 32, 64, 64, 0.98, "hot"),
    ((96, 128, 200), 2, 2, 64, 96, 0, 1, 1.0, "powerlaw"),
    ((4096,), 32, 8, 128, 64, 128, 128, 0.99, "hot"),
    ((70,) * 16, 4, 2, 64, 32, 8, 8, 0.9, "powerlaw"),
    ((3000,), 4, 2, 128, 64, 128, 256, 0.99, "powerlaw"),    # 512 queries per KV head: one slice
    ((3000, 700), 8, 2, 128, 64, 128, 256, 0.99, "powerlaw"),  # 1024 queries per KV head: two slices
    # 63 requests: the most whose offsets the score kernel derives itself (one per lane)
    ((0,) + (33,) * 30 + (0,) + (70,) * 31, 4, 2, 64, 32, 8, 8, 0.9, "powerlaw"),
    # 70 requests: offsets from the prep kernel
    ((33,) * 40 + (0,) * 10 + (130,) * 20, 4, 2, 64, 32, 8, 8, 0.9, "powerlaw"),
]


@pytest.mark.parametrize("idx", range(len(TINY_CASES)), ids=[f"t{i}" for i in range(len(TINY_CASES))])
def test_select_small_shapes(idx):
    lengths, hq, hkv, d, G, A, n, p, kind = TINY_CASES[idx]
    wl = synth.tiny(lengths, hq=hq, hkv=hkv, d=d, G=G, A=A, n=n, p=p, seed=100 + idx,
                    kind=kind, hot=3, hot_lambda=6.0, c=1.5)
    check_select(wl)


@pytest.mark.parametrize("lengths", [(500, 0, 300), (33,) * 40 + (0,) * 10 + (130,) * 20],
                         ids=["offsets_in_score_kernel", "offsets_from_prep"])
def test_select_stream_with_leading_gap(lengths):
    """Requests that start past token 0 (cu_seqlens[0] = 100): both ways of
    forming the offsets (in the score kernel for a few requests, the prep
    kernel for many) select from the right rows and leave the tokens before
    the first request untouched."""
    gap = 100
    wl = synth.tiny(lengths, hq=4, hkv=2, d=64, G=32, A=8, n=8, p=0.9, seed=41, kind="powerlaw", c=1.5)
    cu, q, k = synth.make_qk(wl)
    rng = np.random.default_rng(42)
    pad_q = rng.integers(-2 ** 15, 2 ** 15, size=(gap,) + q.shape[1:]).astype(np.int16).view(q.dtype)
    pad_k = rng.integers(-2 ** 15, 2 ** 15, size=(gap,) + k.shape[1:]).astype(np.int16).view(k.dtype)
    q2, k2 = np.concatenate([pad_q, q]), np.concatenate([pad_k, k])
    cu2 = (cu + gap).astype(np.int32)
    ref = oracle.select(q2, k2, cu2, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    got = run_select(wl, cu2, q2, k2)
    assert np.array_equal(got["offs"], ref["block_offsets"])
    check_scores(got["b"], ref["b64"], ref["block_offsets"])
    assert (got["mask"][:gap] == 0xAB).all()
    check_masks(ref, got["keep"], got["mask"], got["kept"], cu2, wl)


def random_case(seed):
    """A seeded random small workload: 1 to 70 requests (some empty, lengths
    ragged around and between the sink, window and block sizes), any head
    dimension, GQA ratio, block size, sink count, window and p."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([32, 64, 96, 128]))
    n = int(rng.choice([1, 8, 32, 64, 100, 128]))
    A = int(rng.choice([0, 4, 64, 128]))
    p = float(rng.choice([0.5, 0.9, 0.95, 0.98, 0.99, 1.0]))
    R = int(rng.choice([1, 2, 3, 5, 16, 40, 63, 64, 70]))
    budget = 24000 // max(1, hq * n // 64)          # keep the oracle's work to a second or two
    lengths = []
    for _ in range(R):
        u = rng.random()
        L = 0 if u < 0.08 else int(rng.integers(1, 2 * G + n + A + 2)) if u < 0.4 else int(rng.integers(1, 4000))
        lengths.append(L)
    while sum(lengths) > budget and max(lengths) > 1:
        i = int(np.argmax(lengths))
        lengths[i] //= 2
    kind = str(rng.choice(["hot", "powerlaw"]))
    return synth.tiny(tuple(lengths), hq=hq, hkv=hkv, d=d, G=G, A=A, n=n, p=p, seed=2000 + seed, kind=kind,
                      hot=int(rng.integers(1, 6)), hot_lambda=float(rng.uniform(3.0, 8.0)),
                      c=float(rng.uniform(0.8, 1.8)))


@pytest.mark.parametrize("seed", range(20), ids=[f"r{i}" for i in range(20)])
def test_select_random_shapes(seed):
    check_select(random_case(seed), label=f"random {seed}")


# window-query tiles that straddle two query heads (n = 100), pad past the last
# query, or hold rows past a short request's window: the per-row path of the
# score kernel's staged query loads, at d = 128 with eight waves of two tiles
# and at d = 256 with eight waves of one tile
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (16, 8, 256)], ids=["d128_two_tiles", "d256_one_tile"])
def test_select_query_tiles_straddle_heads(hq, hkv, d):
    wl = synth.tiny((3000, 57, 1200, 99), hq=hq, hkv=hkv, d=d, G=64, A=64, n=100, p=0.95, seed=51,
                    kind="powerlaw", c=1.4)
    ref, got, mism = check_select(wl, label=f"straddle d={d}")
    say(f"  kept={got['kept'].tolist()} mismatched={mism}")


def test_select_repeatable():
    wl = synth.tiny((3000, 900), hq=8, hkv=2, d=128, G=64, A=128, n=128, p=0.99, seed=7, kind="powerlaw", c=1.4)
    cu, q, k = synth.make_qk(wl)
    a = run_select(wl, cu, q, k)
    b = run_select(wl, cu, q, k)
    for key in ("b", "keep", "mask", "kept"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["b"].view(np.uint32), b["b"].view(np.uint32))


def test_select_softmax_scale_override():
    """The ABI's softmax_scale replaces 1/sqrt(d) inside the softmax (UniPrefill
    Sec. 3.2 Eq. 2 prints 1/sqrt(d); the override serves other scalings)."""
    wl = synth.tiny((1500, 333), hq=8, hkv=2, d=128, G=64, A=64, n=64, p=0.95, seed=21, kind="hot", hot=3,
                    hot_lambda=6.0)
    cu, q, k = synth.make_qk(wl)
    for scale in (0.03, 0.25):
        say(f"[scale] {scale}")
        ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p, scale=scale)
        got = run_select(wl, cu, q, k, scale=scale)
        check_scores(got["b"], ref["b64"], ref["block_offsets"])
        check_masks(ref, got["keep"], got["mask"], got["kept"], cu, wl)


def test_select_reuses_buffers_for_a_smaller_batch():
    """One set of buffers and workspace serves a long batch and then a shorter
    one: the second call's results depend on nothing the first left behind."""
    big = synth.tiny((4000, 2500), hq=8, hkv=2, d=128, G=64, A=64, n=64, p=0.99, seed=31, kind="powerlaw", c=1.5)
    small = synth.tiny((700, 65), hq=8, hkv=2, d=128, G=64, A=64, n=64, p=0.99, seed=32, kind="hot", hot=2,
                       hot_lambda=6.0)
    cu_b, q_b, k_b = synth.make_qk(big)
    cu_s, q_s, k_s = synth.make_qk(small)
    prm = tlb.make_params(big.hq, big.hkv, big.d, big.G, big.A, big.n, big.p)
    bufs = SelectBuffers.allocate(prm, 2, int(cu_b[-1]))
    first = run_select(big, cu_b, q_b, k_b, bufs=bufs)
    second = run_select(small, cu_s, q_s, k_s, bufs=bufs)
    for wl, cu, q, k, got in ((big, cu_b, q_b, k_b, first), (small, cu_s, q_s, k_s, second)):
        ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
        assert np.array_equal(got["offs"], ref["block_offsets"])
        check_scores(got["b"], ref["b64"], ref["block_offsets"])
        check_masks(ref, got["keep"], got["mask"], got["kept"], cu, wl)


def test_select_max_tokens_larger_than_stream():
    wl = synth.tiny((500, 260), hq=4, hkv=2, d=64, G=32, A=8, n=16, p=0.95, seed=3)
    cu, q, k = synth.make_qk(wl)
    ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    got = run_select(wl, cu, q, k, max_tokens=int(cu[-1]) + 1000)
    check_scores(got["b"], ref["b64"], ref["block_offsets"])
    check_masks(ref, got["keep"], got["mask"], got["kept"], cu, wl)


# ---------------------------------------------------------------------------
# top-p from given scores: bit-exact
# ---------------------------------------------------------------------------
def _scores_case(seed, lengths, G, kinds):
    rng = np.random.default_rng(seed)
    nbs = [-(-L // G) for L in lengths]
    parts = []
    for r, nb in enumerate(nbs):
        parts.append(synth.random_scores(rng, nb, kinds[r % len(kinds)]))
    return np.concatenate(parts) if parts else np.zeros(0, np.float32)


@pytest.mark.parametrize("seed,lengths,G,A,n,p,kinds", [
    (0, (1000, 64, 1, 0, 4096), 64, 128, 128, 0.99, ("lognormal", "ties", "sparse", "pareto")),
    (1, (777, 3333), 7, 5, 9, 0.9, ("ties", "lognormal")),
    (2, (131072,), 64, 128, 128, 0.99, ("pareto",)),
    (3, (65536,), 32, 128, 128, 0.98, ("lognormal",)),
    (4, (5000, 6000, 7000), 128, 0, 1, 1.0, ("sparse", "ties", "lognormal")),
    (5, tuple([300] * 16), 16, 16, 16, 0.5, ("ties", "lognormal", "pareto", "sparse")),
    # more blocks than the kernel keeps in LDS (4096): keys re-read from the scores
    (6, (300000, 5, 262208), 32, 16, 64, 0.95, ("lognormal", "ties", "ties")),
    (7, (262208, 262144), 64, 128, 128, 0.99, ("pareto", "sparse")),
    # all scores equal: the keys differ only in the block index
    (8, (131072, 640, 64), 64, 128, 128, 0.99, ("constant",)),
])
def test_topp_scores_in_bit_exact(seed, lengths, G, A, n, p, kinds):
    say(f"[topp] seed={seed} lengths={lengths[:5]} G={G} p={p}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    sc = _scores_case(seed, lengths, G, kinds)
    if seed == 0:   # values that carry no mass: zeros, -0, negatives, inf, nan
        sc[3] = 0.0
        sc[4] = -0.0
        sc[5] = -2.5
        sc[16] = np.inf
        sc[17] = np.nan
    R = len(lengths)
    ref = oracle.select(None, None, cu, 1, 1, 1, G, A, n, p, scores_in=sc)
    prm = tlb.make_params(1, 1, 1, G, A, n, p, scores_in=True)
    bufs = SelectBuffers.allocate(prm, R, T)
    bufs.block_scores.fill_(-1)
    bufs.run(None, None, dev(cu), scores_in=dev(sc))
    torch.cuda.synchronize()
    nbt = len(sc)
    assert np.array_equal(bufs.block_offsets[: R + 1].cpu().numpy(), ref["block_offsets"])
    assert np.array_equal(bufs.keep_block[:nbt].cpu().numpy(), ref["keep_block"])
    assert np.array_equal(bufs.keep_mask[:T].cpu().numpy(), ref["mask"])
    assert np.array_equal(bufs.kept[:R].cpu().numpy(), ref["kept"])
    assert np.array_equal(bufs.block_scores[:nbt].cpu().numpy().view(np.uint32), sc.view(np.uint32))


def test_topp_fixture_through_gpu():
    from pins import load_golden
    g = load_golden("expand_hand_example.json")
    sc = np.array(g["scores_times_64"], np.float32) / 64
    cu = np.array([0, g["N"]], np.int32)
    prm = tlb.make_params(1, 1, 1, g["G"], g["A"], g["n"], g["p"], scores_in=True)
    bufs = SelectBuffers.allocate(prm, 1, g["N"])
    bufs.run(None, None, dev(cu), scores_in=dev(sc))
    torch.cuda.synchronize()
    assert bufs.keep_mask[: g["N"]].cpu().tolist() == g["mask"]
    assert int(bufs.kept[0]) == g["kept_tokens"]


def test_select_two_request_fixture_through_gpu():
    """The hand-worked two-request fixture that pins oracle.select (stream
    offset 5, a request no longer than A + n) through the C ABI from its fp32
    scores: offsets, flags, mask placement and kept counts as worked by hand."""
    from pins import load_golden
    g = load_golden("select_two_requests.json")
    c = g["scores_in"]
    sc = np.array(c["scores_times_64"], np.float32) / np.float32(64)
    cu = np.array(g["cu_seqlens"], np.int32)
    T = int(cu[-1])
    prm = tlb.make_params(1, 1, 1, g["G"], g["A"], g["n"], c["p"], scores_in=True)
    bufs = SelectBuffers.allocate(prm, 2, T)
    bufs.keep_mask.fill_(0xAB)
    bufs.run(None, None, dev(cu), scores_in=dev(sc))
    torch.cuda.synchronize()
    assert bufs.block_offsets[:3].cpu().tolist() == g["block_offsets"]
    assert bufs.keep_block[:8].cpu().tolist() == c["keep_block"]
    # tokens before the first request belong to no request: left untouched
    assert bufs.keep_mask[:5].cpu().tolist() == [0xAB] * 5
    assert bufs.keep_mask[5:T].cpu().tolist() == c["mask"][5:]
    assert bufs.kept[:2].cpu().tolist() == c["kept"]


# ---------------------------------------------------------------------------
# compaction, scatter-back, metadata: bit-exact
# ---------------------------------------------------------------------------
COMPACT_CASES = [
    (0, (5000, 0, 3000, 9000), 0.4, (8192, 12, 4)),
    (1, (1, 2, 3), 0.5, (16,)),
    (2, (131072,), 0.4, (8192,)),
    (3, tuple([4100] * 5), 0.9, (7680, 4096)),
    (4, (300, 0), 0.0, (32,)),
    (5, (70000,), 1.0, (4,)),
    (6, (777, 0, 1234), 0.5, (36, 48, 100, 16)),   # wide unaligned rows, 3-unit rows, narrow aligned rows
    # max_tokens = 131072 exactly: the largest stream ranked in one launch (case 2 takes the
    # count + rank path, its max_tokens being 37 past 131072)
    (7, (100000, 31035), 0.3, (8192, 4)),
    # more requests than the one-launch rank kernel's threads (the stream length and
    # the new offsets are then formed by the whole workgroup), below and above 131072 tokens
    (8, (3, 0, 17) * 500, 0.5, (16, 4)),
    (9, (100,) * 1400, 0.3, (32,)),
]


@pytest.mark.parametrize("seed,lengths,rho,row_bytes", COMPACT_CASES)
def test_compact_and_scatter_bit_exact(seed, lengths, rho, row_bytes):
    say(f"[compact] seed={seed} lengths={lengths[:5]} rho={rho} row_bytes={row_bytes}")
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    R = len(lengths)
    max_tokens = T + 37
    mask = np.zeros(max_tokens, np.uint8)
    mask[:T] = (rng.random(T) < rho).astype(np.uint8) * rng.integers(1, 256, T).astype(np.uint8)
    mask[T:] = 1          # beyond the stream: must be ignored
    bufs_h = [rng.integers(0, 2 ** 32, size=(max_tokens, rb // 4), dtype=np.uint64).astype(np.uint32)
              for rb in row_bytes]
    index_in = rng.permutation(10 * max_tokens)[:max_tokens].astype(np.int32)
    for use_index in (False, True):
        outs, idx, cu_out = oracle.compact(mask, cu, bufs_h, index_in if use_index else None)
        src = [dev(b.view(np.int32)) for b in bufs_h]
        dst = [torch.full_like(s, -7) for s in src]
        cb = CompactBuffers.allocate(R, max_tokens)
        cb.index_out.fill_(-5)
        cb.run(dev(mask), dev(cu), src, dst, index_in=dev(index_in) if use_index else None)
        torch.cuda.synchronize()
        K = len(idx)
        assert np.array_equal(cb.cu_out[: R + 1].cpu().numpy(), cu_out)
        assert np.array_equal(cb.index_out[:K].cpu().numpy(), idx)
        assert (cb.index_out[K:max_tokens].cpu().numpy() == -5).all()
        for o, d in zip(outs, dst):
            got = d[:K].cpu().numpy().view(np.uint32)
            assert np.array_equal(got, o)
            assert (d[K:].cpu().numpy() == -7).all()
        if not use_index:
            # Eq. 8: scatter processed rows (x + 1) back into the full buffers
            for b, (o, d) in enumerate(zip(outs, dst)):
                proc = (o.astype(np.uint64) + 1).astype(np.uint32)
                want = oracle.scatter_back(bufs_h[b], proc, idx, K)
                full = dev(bufs_h[b].view(np.int32))
                run_scatter_back(dev(proc.view(np.int32)) if K else torch.zeros((1, proc.shape[1]), dtype=torch.int32, device="cuda"),
                                 cb.index_out, cb.cu_out, R, max_tokens, full)
                torch.cuda.synchronize()
                assert np.array_equal(full.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("seed", range(12), ids=[f"r{i}" for i in range(12)])
def test_compact_and_scatter_random(seed):
    """Seeded random compactions: 1 to 70 requests (some empty), keep ratios
    from 0 to 1 (block-structured or per token), one to four buffers with rows
    of 4 bytes to 8 KiB (16-byte multiples and not), max_tokens at or past the
    stream (around the one-launch rank limit too), with and without an index
    map; bit-exact against the oracle, then the Eq. 8 scatter back."""
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.choice([1, 2, 5, 16, 63, 70]))
    big = seed % 4 == 0
    lengths = [0 if rng.random() < 0.1 else int(rng.integers(1, (131072 // R) if big else 3000)) for _ in range(R)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    max_tokens = T + int(rng.choice([0, 1, 37, 4096]))
    rho = float(rng.choice([0.0, 0.05, 0.4, 0.9, 1.0]))
    if rng.random() < 0.5:
        blk = (rng.random(T // 64 + 1) < rho).astype(np.uint8)
        m = blk[np.arange(T) // 64]
    else:
        m = (rng.random(T) < rho).astype(np.uint8)
    mask = np.zeros(max_tokens, np.uint8)
    mask[:T] = m * rng.integers(1, 256, T).astype(np.uint8)
    mask[T:] = 1
    nbuf = int(rng.integers(1, 5))
    row_bytes = tuple(int(rng.choice([4, 8, 12, 16, 32, 36, 48, 64, 100, 2048, 7680, 8192])) for _ in range(nbuf))
    if big:
        row_bytes = tuple(min(rb, 2048) for rb in row_bytes)   # keep the host copies small
    say(f"[compact-rand] seed={seed} R={R} T={T} max_tokens={max_tokens} rho={rho} rows={row_bytes}")
    bufs_h = [rng.integers(0, 2 ** 32, size=(max_tokens, rb // 4), dtype=np.uint64).astype(np.uint32)
              for rb in row_bytes]
    use_index = bool(rng.random() < 0.5)
    index_in = rng.permutation(4 * max_tokens + 1)[:max_tokens].astype(np.int32) if use_index else None
    outs, idx, cu_out = oracle.compact(mask, cu, bufs_h, index_in)
    src = [dev(b.view(np.int32)) for b in bufs_h]
    dst = [torch.full_like(t, -7) for t in src]
    cb = CompactBuffers.allocate(R, max_tokens)
    cb.run(dev(mask), dev(cu), src, dst, index_in=dev(index_in) if use_index else None)
    torch.cuda.synchronize()
    K = len(idx)
    assert np.array_equal(cb.cu_out[: R + 1].cpu().numpy(), cu_out)
    assert np.array_equal(cb.index_out[:K].cpu().numpy(), idx)
    for o, d in zip(outs, dst):
        assert np.array_equal(d[:K].cpu().numpy().view(np.uint32), o)
        assert (d[K:].cpu().numpy() == -7).all()
    if not use_index and K:
        b = int(rng.integers(0, nbuf))
        proc = (outs[b].astype(np.uint64) + 1).astype(np.uint32)
        want = oracle.scatter_back(bufs_h[b], proc, idx, K)
        full = dev(bufs_h[b].view(np.int32))
        run_scatter_back(dev(proc.view(np.int32)), cb.index_out, cb.cu_out, R, max_tokens, full)
        torch.cuda.synchronize()
        assert np.array_equal(full.cpu().numpy().view(np.uint32), want)


def test_compact_twice_composes_index():
    rng = np.random.default_rng(11)
    lengths = (6000, 2500, 9000)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    H = rng.integers(0, 2 ** 32, size=(T, 8), dtype=np.uint64).astype(np.uint32)
    m1 = (rng.random(T) < 0.6).astype(np.uint8)
    (h1,), i1, cu1 = oracle.compact(m1, cu, [H])
    m2 = (rng.random(len(i1)) < 0.5).astype(np.uint8)
    (h2,), i2, cu2 = oracle.compact(m2, cu1, [h1], index_in=i1)
    Hd = dev(H.view(np.int32))
    d1 = torch.empty_like(Hd)
    c1 = CompactBuffers.allocate(3, T)
    c1.run(dev(m1), dev(cu), [Hd], [d1])
    d2 = torch.empty_like(Hd)
    c2 = CompactBuffers.allocate(3, T)
    m2d = torch.zeros(T, dtype=torch.uint8, device="cuda")
    m2d[: len(m2)] = dev(m2)
    c2.run(m2d, c1.cu_out, [d1], [d2], index_in=c1.index_out)
    torch.cuda.synchronize()
    K = len(i2)
    assert np.array_equal(c2.index_out[:K].cpu().numpy(), i2)
    assert np.array_equal(c2.cu_out.cpu().numpy(), cu2)
    assert np.array_equal(d2[:K].cpu().numpy().view(np.uint32), h2)


def test_metadata_and_eq17():
    rng = np.random.default_rng(5)
    R, L, max_drops = 6, 32, 3
    lens = rng.integers(50, 400, R)
    ctx = rng.integers(0, 30, R)
    orig = lens + ctx
    st = oracle.MetadataState.fresh(orig)
    mb = MetadataBuffers.allocate(orig, L, max_drops)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layers = [3, 9, 17, 25]      # one more drop than the history can hold
    for layer in layers:
        cur = np.diff(cu)
        kept = np.array([int(rng.integers(0, c + 1)) for c in cur])
        cu_new = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
        st, nat = oracle.update_metadata(st, layer, cu, cu_new)
        mb.run(layer, dev(cu), dev(cu_new))
        torch.cuda.synchronize()
        assert int(mb.num_actual_tokens[0]) == nat
        assert np.array_equal(mb.seq_lens.cpu().numpy(), st.seq_lens)
        cu = cu_new
    assert np.array_equal(mb.drop_count.cpu().numpy(), np.full(R, len(layers)))
    dl = mb.drop_layer.cpu().numpy().reshape(R, max_drops)
    dn = mb.drop_len.cpu().numpy().reshape(R, max_drops)
    for r in range(R):
        assert [(int(a), int(b)) for a, b in zip(dl[r], dn[r])] == st.history[r][:max_drops]
    base = mb.seqused_base.cpu().numpy().reshape(L, R)
    kv_len = orig + rng.integers(0, 20, R)
    for lp in range(L):
        for r in range(R):
            want = oracle.seqused_eq17(st.history[r], lp, int(orig[r]), int(kv_len[r]))
            assert int(base[lp, r]) + int(kv_len[r] - orig[r]) == want, (lp, r)


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------
def test_llama_4k_single_request():
    ref, got, mism = check_select(synth.llama_4k())
    say(f"  kept={got['kept'].tolist()} mismatched blocks={mism}")


def test_llama_varlen_batch():
    ref, got, mism = check_select(synth.llama_varlen4())
    say(f"  kept={got['kept'].tolist()} of {list(synth.llama_varlen4().lengths)} mismatched={mism}")


@pytest.mark.parametrize("model", ["qwen_next", "gemma3"])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_hybrid_64k(model, G):
    wl = synth.hybrid_64k(model, G, p=0.98 if model == "gemma3" else 0.99)
    ref, got, mism = check_select(wl)
    say(f"  kept={got['kept'].tolist()} mismatched={mism}")


def test_llama_128k_end_to_end():
    """Select, compact hidden rows, patch metadata, scatter back: the bench's
    workload at full size, checked against the oracle."""
    wl = synth.llama_128k()
    ref, got, mism = check_select(wl)
    cu = wl.cu_seqlens()
    T = int(cu[-1])
    mask_ref = ref["mask"]
    _, idx_ref, cu_out_ref = oracle.compact(mask_ref, cu, [])
    nwords = wl.hidden // 2
    hidden = synth.hidden_words_torch(0, T, nwords, "cuda")
    out = torch.empty_like(hidden)
    cb = CompactBuffers.allocate(1, T)
    cb.run(dev(mask_ref), dev(cu), [hidden], [out])
    torch.cuda.synchronize()
    K = len(idx_ref)
    assert np.array_equal(cb.index_out[:K].cpu().numpy(), idx_ref)
    assert np.array_equal(cb.cu_out.cpu().numpy(), cu_out_ref)
    # compacted rows equal the index-encoded rows of the oracle's kept tokens
    for a in range(0, K, 8192):
        z = min(K, a + 8192)
        want = torch.from_numpy(synth.hidden_words(idx_ref[a:z], nwords).view(np.int32)).cuda()
        assert torch.equal(out[a:z], want)
    # Eq. 8 with processed = compacted + 1 on kept rows
    full = hidden.clone()
    run_scatter_back(out[:K] + 1, cb.index_out, cb.cu_out, 1, T, full)
    torch.cuda.synchronize()
    keep = torch.from_numpy(mask_ref.astype(bool)).cuda()
    assert torch.equal(full[~keep], hidden[~keep])
    assert torch.equal(full[keep], hidden[keep] + 1)
    say(f"  kept tokens={int(got['kept'][0])} ({got['kept'][0] / T:.3f}) blocks kept="
        f"{int(got['keep'].sum())}/{len(got['keep'])} mismatched={mism}")


# ---------------------------------------------------------------------------
# serving-scale batch: 16 requests x 131072 tokens, two drop layers
# ---------------------------------------------------------------------------
def _upload_hidden(T, nwords):
    hid = torch.empty((T, nwords), dtype=torch.int32, device="cuda")
    step = 1 << 16
    for a in range(0, T, step):
        z = min(T, a + step)
        hid[a:z] = synth.hidden_words_torch(a, z - a, nwords, "cuda")
    return hid


def _serving_select(wl):
    """Selection of one serving layer on the GPU, with the invariants checked
    for every request on the GPU's own scores: each window row's softmax sums
    to one, Eq. 6 in aggregated form, and the mask and kept count follow the
    keep flags with the sinks and window forced."""
    cu, q, k = synth.make_qk(wl)
    say(f"  generated {wl.name}: T={int(cu[-1])}")
    got = run_select(wl, cu, q, k)
    del q, k
    offs = got["offs"]
    b = got["b"].astype(np.float64)
    keep = got["keep"].astype(bool)
    mask = got["mask"]
    for r in range(wl.num_reqs):
        a, z = int(offs[r]), int(offs[r + 1])
        N = int(cu[r + 1] - cu[r])
        ne = min(wl.n, N)
        assert abs(b[a:z].sum() * wl.G * ne - wl.hq * ne) <= 1e-4 * wl.hq * ne, r
        tot = b[a:z].sum()
        assert b[a:z][~keep[a:z]].sum() <= (1 - wl.p) * tot * (1 + 1e-6), r
        i = np.arange(N)
        want = (keep[a:z][i // wl.G] | (i < wl.A) | (i >= N - wl.n)).astype(np.uint8)
        assert np.array_equal(mask[cu[r]:cu[r + 1]], want), r
        assert int(got["kept"][r]) == int(want.sum()), r
    return cu, got


def _against_oracle(wl, got, futures):
    """Scores of every request within tolerance of the oracle, and keep flags
    equal but for blocks at the top-p threshold (the end-to-end rule)."""
    from gpu_helpers import allowed_mismatch
    offs = got["offs"]
    keep = got["keep"].astype(bool)
    total_diff = 0
    for r in range(wl.num_reqs):
        b_ref = futures[r].result()
        a, z = int(offs[r]), int(offs[r + 1])
        assert z - a == len(b_ref), r
        check_scores(got["b"][a:z], b_ref, np.array([0, z - a]))
        b32 = b_ref.astype(np.float32)
        keep_ref = oracle.top_p_select(b32, wl.p)
        diff = np.nonzero(keep_ref != keep[a:z])[0]
        if len(diff):
            assert allowed_mismatch(b32, keep_ref, wl.p)[diff].all(), (r, diff[:10])
        total_diff += len(diff)
    say(f"  {wl.name}: all {wl.num_reqs} requests agree with the oracle; {total_diff} blocks at the threshold")


@pytest.mark.timeout(1800)
def test_serving_16x128k_two_layers():
    """Two drop layers in a row on 16 x 131072 packed tokens (cumulative
    reading of UniPrefill Sec. 3.4 Eq. 8 / Sec. 3.5 drop history):
      * layer 0 selects on the full stream; layer 1 selects on the GPU's own
        compacted stream (its lengths are layer 0's kept counts, its offsets
        layer 0's cu_seqlens_out, fresh seeded Q and K of those lengths);
      * every request of both layers against the oracle (scores 1e-3, keep
        flags up to threshold ties);
      * the 16 GiB hidden rows compacted at layer 0 and, with layer 0's index
        map as index_in, again at layer 1: the composed index map equals layer
        0's map at layer 1's kept positions, and every gathered row is the
        index-encoded original;
      * Eq. 8 at both layers into the one full-length buffer: each original
        row ends as its original value plus the number of layers it survived
        (processing adds 1 per layer), dropped rows keeping the value they
        had when dropped;
      * seq_lens, drop history and the Eq. 17 table after both drops."""
    wl0 = synth.serving_16x128k(layer=0)
    R = wl0.num_reqs
    with OraclePool(16) as pool:
        fut0 = pool.submit(wl0, range(R))
        cu0, got0 = _serving_select(wl0)
        T0 = int(cu0[-1])
        nwords = wl0.hidden // 2
        hidden = _upload_hidden(T0, nwords)
        out0 = torch.empty_like(hidden)
        cb0 = CompactBuffers.allocate(R, T0)
        cb0.run(got0["bufs"].keep_mask, dev(cu0), [hidden], [out0])
        torch.cuda.synchronize()
        cu_out0 = cb0.cu_out.cpu().numpy()
        K0 = int(cu_out0[-1])
        assert np.array_equal(np.diff(cu_out0), got0["kept"])
        idx0 = cb0.index_out[:K0]
        assert bool((idx0[1:] > idx0[:-1]).all())
        assert torch.equal(torch.nonzero(got0["bufs"].keep_mask[:T0]).flatten().to(torch.int32), idx0)
        step = 1 << 16
        for a in range(0, K0, step):
            z = min(K0, a + step)
            assert torch.equal(out0[a:z], synth.hidden_words_torch_at(idx0[a:z], nwords)), a
        out0[:K0] += 1           # the sublayers between the two drops

        # layer 1: selection on the compacted stream the GPU produced
        lengths1 = tuple(int(x) for x in np.diff(cu_out0))
        wl1 = synth.serving_16x128k(lengths=lengths1, layer=1)
        fut1 = pool.submit(wl1, range(R))
        cu1, got1 = _serving_select(wl1)
        assert np.array_equal(cu1, cu_out0)
        out1 = torch.empty((K0, nwords), dtype=torch.int32, device="cuda")
        cb1 = CompactBuffers.allocate(R, K0)
        cb1.run(got1["bufs"].keep_mask, dev(cu1), [out0[:K0]], [out1], index_in=cb0.index_out)
        torch.cuda.synchronize()
        cu_out1 = cb1.cu_out.cpu().numpy()
        K1 = int(cu_out1[-1])
        assert np.array_equal(np.diff(cu_out1), got1["kept"])
        pos1 = torch.nonzero(got1["bufs"].keep_mask[:K0]).flatten()
        idx1 = cb1.index_out[:K1]
        assert torch.equal(idx1, idx0[pos1])        # the index map composes
        for a in range(0, K1, step):
            z = min(K1, a + step)
            assert torch.equal(out1[a:z], synth.hidden_words_torch_at(idx1[a:z], nwords) + 1), a
        out1[:K1] += 1           # the sublayers after the second drop

        # Eq. 8 at both layers, into the full-length state
        run_scatter_back(out0, cb0.index_out, cb0.cu_out, R, T0, hidden)
        run_scatter_back(out1, cb1.index_out, cb1.cu_out, R, K0, hidden)
        torch.cuda.synchronize()
        survived = torch.zeros(T0, dtype=torch.int32, device="cuda")
        survived[idx0.long()] += 1
        survived[idx1.long()] += 1
        for a in range(0, T0, step):
            z = min(T0, a + step)
            want = synth.hidden_words_torch(a, z - a, nwords, "cuda") + survived[a:z, None]
            assert torch.equal(hidden[a:z], want), a
        del hidden, out0, out1
        torch.cuda.empty_cache()

        # metadata after both drops (layers 3 and 11 of 32)
        L = 32
        mb = MetadataBuffers.allocate(np.diff(cu0), L, 4)
        mb.run(3, dev(cu0), cb0.cu_out)
        mb.run(11, dev(cu1), cb1.cu_out)
        torch.cuda.synchronize()
        kept0 = got0["kept"].astype(np.int64)
        kept1 = got1["kept"].astype(np.int64)
        orig = np.diff(cu0).astype(np.int64)
        assert np.array_equal(mb.seq_lens.cpu().numpy(), kept1)
        assert np.array_equal(mb.drop_count.cpu().numpy(), np.full(R, 2))
        dl = mb.drop_layer.cpu().numpy().reshape(R, 4)
        dn = mb.drop_len.cpu().numpy().reshape(R, 4)
        assert (dl[:, 0] == 3).all() and (dl[:, 1] == 11).all()
        assert np.array_equal(dn[:, 0], kept0) and np.array_equal(dn[:, 1], kept1)
        base = mb.seqused_base.cpu().numpy().reshape(L, R)
        for lp in range(L):
            want = orig if lp <= 3 else (kept0 if lp <= 11 else kept1)
            assert np.array_equal(base[lp], want), lp

        _against_oracle(wl0, got0, fut0)
        _against_oracle(wl1, got1, fut1)
    say(f"  layer0 kept {int(kept0.sum())}/{T0}, layer1 kept {int(kept1.sum())}/{K0}")


# ---------------------------------------------------------------------------
# window sizes of the paper's ablation (n = 32 and n = 512; Table 4)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [32, 512])
def test_window_ablation_128k(n):
    """The 131072-token LLaMA-shaped request of the benchmark at the ablation's
    window sizes, in the launch shape the benchmark's sweep times (n = 512:
    four query slices per key chunk)."""
    from dataclasses import replace
    wl = replace(synth.llama_128k(), n=n, name=f"llama8b_128k_n{n}")
    ref, got, mism = check_select(wl)
    say(f"  n={n}: kept={got['kept'].tolist()} of 131072, mismatched={mism}")


@pytest.mark.parametrize("n", [32, 512])
def test_window_ablation_sizes(n):
    wl = synth.with_structures(
        synth.Workload(f"llama8b_16k_n{n}", (16384, 3000), n=n, seed=21, **synth.LLAMA_8B),
        [synth.RequestStructure("powerlaw", c=synth.POWERLAW_C)] * 2)
    ref, got, mism = check_select(wl)
    say(f"  n={n}: kept={got['kept'].tolist()} mismatched={mism}")


# ---------------------------------------------------------------------------
# Q and K as views into one fused QKV projection buffer (the layout serving
# stacks hand over): row strides larger than Hq*d and Hkv*d
# ---------------------------------------------------------------------------
def test_select_fused_qkv_views():
    wl = synth.tiny((700, 1500, 90), hq=8, hkv=2, d=128, G=64, A=64, n=64, p=0.95, seed=17,
                    kind="hot", hot=3, hot_lambda=6.0)
    cu, q, k = synth.make_qk(wl)
    T = int(cu[-1])
    ref_contig = run_select(wl, cu, q, k)
    width = (wl.hq + 2 * wl.hkv) * wl.d
    qkv = torch.full((T, width), 0x7F80, dtype=torch.int16, device="cuda")   # bf16 +inf outside Q and K
    cu_d, qd, kd = upload_qk(wl, cu, q, k)
    qkv[:, : wl.hq * wl.d] = qd.reshape(T, -1)
    qkv[:, wl.hq * wl.d: (wl.hq + wl.hkv) * wl.d] = kd.reshape(T, -1)
    qv = qkv[:, : wl.hq * wl.d]
    kv = qkv[:, wl.hq * wl.d: (wl.hq + wl.hkv) * wl.d]
    assert qv.stride(0) == width and kv.stride(0) == width
    prm = tlb.make_params(wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    bufs = SelectBuffers.allocate(prm, wl.num_reqs, T)
    bufs.run(qv, kv, cu_d)
    torch.cuda.synchronize()
    nbt = int(ref_contig["offs"][-1])
    assert np.array_equal(bufs.block_scores[:nbt].cpu().numpy(), ref_contig["b"])
    assert np.array_equal(bufs.keep_mask[:T].cpu().numpy(), ref_contig["mask"])
    assert np.array_equal(bufs.kept[: wl.num_reqs].cpu().numpy(), ref_contig["kept"])
    ref = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    check_scores(ref_contig["b"], ref["b64"], ref["block_offsets"])
