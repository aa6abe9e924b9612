"""Checks that pin the CPU oracle to the UniPrefill paper (arXiv 2605.06221).

Each check takes the implementation under test as a namespace `impl` with the
oracle's function names, so the same checks run against the oracle (they
must pass) and against deliberately broken copies of it in
test_oracle_mutations.py (each copy must fail at least one check).  None of
the checks retypes the oracle's formula: they compare it with hand-worked
fixtures, closed forms, brute force, library routines and invariants.
"""
from __future__ import annotations

from fractions import Fraction
import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_bits(x):
    """float -> bf16 bits by truncation-free RNE via float32 (test helper)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Scores (Eq. 2-4)
# ---------------------------------------------------------------------------
def check_uniform_fixture(impl):
    """Q = 0 hand example (N=8, n=2, G=4, one head)."""
    g = load_golden("uniform_closed_form.json")
    N, n, G = g["N"], g["n"], g["G"]
    q = np.zeros((N, 1, 16), np.uint16)
    k = bf16_bits(np.random.default_rng(0).standard_normal((N, 1, 16)))
    b, o = impl.request_block_scores(q, k, 0, N, 1, 1, 16, G, n)
    assert np.allclose(o * 56, g["importance_times_56"], rtol=0, atol=1e-12), o * 56
    assert np.allclose(b * 112, g["block_scores_times_112"], rtol=0, atol=1e-12), b * 112


def check_uniform_closed_form(impl):
    """Q = 0 closed form on ragged shapes: o_i = Hq * sum_{j >= max(i, N-n_eff)} 1/(j+1)."""
    rng = np.random.default_rng(1)
    for (N, n, G, hq, hkv) in [(37, 5, 8, 4, 2), (5, 8, 4, 2, 1), (64, 16, 16, 3, 1), (1, 4, 4, 2, 2)]:
        d = 8
        q = np.zeros((N + 3, hq, d), np.uint16)
        k = bf16_bits(rng.standard_normal((N + 3, hkv, d)))
        b, o = impl.request_block_scores(q, k, 3, N, hq, hkv, d, G, n)
        ne = min(n, N)
        exp_o = np.array([hq * sum(Fraction(1, j + 1) for j in range(max(i, N - ne), N))
                          for i in range(N)], dtype=object)
        assert np.allclose(o, exp_o.astype(float), rtol=1e-12, atol=0), (N, n, o, exp_o)
        nb = -(-N // G)
        exp_b = [float(sum(exp_o[g * G: min(N, (g + 1) * G)]) / (G * ne)) for g in range(nb)]
        assert np.allclose(b, exp_b, rtol=1e-12, atol=0), (N, n, G, b, exp_b)


def _torch_reference_o(q, k, start, N, hq, hkv, d, n, scale):
    import torch
    ne = min(n, N)
    o = torch.zeros(N, dtype=torch.float64)
    for h in range(hq):
        kv = h // (hq // hkv)
        Q = torch.from_numpy(bits_to_f64(q[start + N - ne: start + N, h]))
        K = torch.from_numpy(bits_to_f64(k[start: start + N, kv]))
        for t in range(ne):
            pos = N - ne + t
            logits = (K[: pos + 1] @ Q[t]) * scale
            o[: pos + 1] += torch.softmax(logits, dim=0)
    return o.numpy()


def check_vs_torch_softmax(impl):
    """Random tiny shapes against torch.softmax (float64, CPU), row by row."""
    rng = np.random.default_rng(2)
    for (N, n, G, hq, hkv, d) in [(29, 6, 8, 4, 2, 16), (16, 16, 4, 2, 2, 8), (40, 7, 16, 6, 3, 32)]:
        q = bf16_bits(rng.standard_normal((N + 5, hq, d)) * 1.5)
        k = bf16_bits(rng.standard_normal((N + 5, hkv, d)) * 1.5)
        scale = 1.0 / math.sqrt(d)
        b, o = impl.request_block_scores(q, k, 2, N, hq, hkv, d, G, n)
        ref = _torch_reference_o(q, k, 2, N, hq, hkv, d, n, scale)
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)
        # explicit scale override
        b2, o2 = impl.request_block_scores(q, k, 2, N, hq, hkv, d, G, n, scale=0.3)
        ref2 = _torch_reference_o(q, k, 2, N, hq, hkv, d, n, 0.3)
        assert np.allclose(o2, ref2, rtol=1e-12, atol=1e-14)


def check_mass_invariant(impl):
    """Every window row sums to one: sum_g b_g * G * n_eff = Hq * n_eff."""
    rng = np.random.default_rng(3)
    for (N, n, G, hq, hkv, d) in [(100, 8, 16, 8, 2, 16), (7, 16, 4, 2, 1, 8)]:
        q = bf16_bits(rng.standard_normal((N, hq, d)) * 3)
        k = bf16_bits(rng.standard_normal((N, hkv, d)) * 3)
        b, _ = impl.request_block_scores(q, k, 0, N, hq, hkv, d, G, n)
        ne = min(n, N)
        assert abs(b.sum() * G * ne - hq * ne) < 1e-12 * hq * ne


def check_gqa_invariance(impl):
    """Replicating each KV head over its query group (so Hkv = Hq) changes nothing."""
    rng = np.random.default_rng(4)
    N, n, G, hq, hkv, d = 50, 9, 8, 8, 2, 16
    q = bf16_bits(rng.standard_normal((N, hq, d)) * 2)
    k = bf16_bits(rng.standard_normal((N, hkv, d)) * 2)
    group = hq // hkv
    k_full = np.repeat(k, group, axis=1)     # head h gets kv head h // group
    b1, _ = impl.request_block_scores(q, k, 0, N, hq, hkv, d, G, n)
    b2, _ = impl.request_block_scores(q, k_full, 0, N, hq, hq, d, G, n)
    assert np.allclose(b1, b2, rtol=1e-13, atol=0)


def check_spike(impl):
    """One key with a +50 logit for every window row takes almost all mass."""
    N, n, G, hq, d = 64, 8, 8, 2, 16
    q = np.zeros((N, hq, d), np.float64)
    q[:, :, 0] = 1.0
    k = np.zeros((N, 1, d), np.float64)
    k[19, 0, 0] = 50.0 * math.sqrt(d)
    b, o = impl.request_block_scores(bf16_bits(q), bf16_bits(k), 0, N, hq, 1, d, G, n)
    assert b[19 // G] * G * n > 0.999999 * hq * n
    assert o[19] > 0.999999 * hq * n


def check_packing_independence(impl):
    """Blocks are anchored at each request's start: a packed batch scores each
    request exactly as alone."""
    rng = np.random.default_rng(5)
    hq, hkv, d, G, n = 4, 2, 16, 8, 6
    lens = [13, 1, 30, 8]
    T = sum(lens)
    q = bf16_bits(rng.standard_normal((T, hq, d)) * 2)
    k = bf16_bits(rng.standard_normal((T, hkv, d)) * 2)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    b, offs = impl.block_scores(q, k, cu, hq, hkv, d, G, n)
    for r, N in enumerate(lens):
        s = cu[r]
        br, _ = impl.request_block_scores(q[s: s + N].copy(), k[s: s + N].copy(), 0, N, hq, hkv, d, G, n)
        assert np.array_equal(b[offs[r]: offs[r + 1]], br)
        assert offs[r + 1] - offs[r] == -(-N // G)


def check_causal(impl):
    """A key after a window row's own position gets none of that row's mass."""
    N, n, G, d = 16, 4, 4, 8
    q = np.zeros((N, 1, d))
    q[:, 0, 0] = 1.0
    k = np.zeros((N, 1, d))
    k[N - 1, 0, 0] = 30.0 * math.sqrt(d)      # huge logit on the very last key
    b, o = impl.request_block_scores(bf16_bits(q), bf16_bits(k), 0, N, 1, 1, d, G, n)
    # only the last window row can see key N-1; the other rows spread uniformly
    rows = [N - n + t for t in range(n)]
    exp_o0 = sum(1.0 / (j + 1) for j in rows[:-1])
    assert abs(o[0] - exp_o0) < 1e-9, (o[0], exp_o0)
    assert abs(o[N - 1] - 1.0) < 1e-9


SCORE_CHECKS = [check_uniform_fixture, check_uniform_closed_form, check_vs_torch_softmax,
                check_mass_invariant, check_gqa_invariance, check_spike,
                check_packing_independence, check_causal]


# ---------------------------------------------------------------------------
# Top-p (Eq. 5, Eq. 14) and expansion
# ---------------------------------------------------------------------------
def check_topp_fixture(impl):
    g = load_golden("topp_hand_example.json")
    b = np.array(g["scores_times_64"], dtype=np.float32) / 64
    keep = impl.top_p_select(b, g["p"])
    assert sorted(np.nonzero(keep)[0].tolist()) == g["kept_blocks"]
    order = np.argsort(impl.pack_keys(b))[::-1]
    assert order.tolist() == g["descending_order"]


def _brute_min_card(b, p):
    """Smallest number of blocks whose exact mass reaches p times the total."""
    fr = [Fraction(float(x)) for x in b]
    tot = sum(fr)
    pf = Fraction(p)
    for size in range(1, len(b) + 1):
        best = sum(sorted(fr, reverse=True)[:size])
        if best >= pf * tot:
            return size
    return len(b)


def check_topp_bruteforce(impl):
    """|S| equals the minimum cardinality over all subsets (nb <= 9), and S is
    the top-|S| prefix in packed-key order."""
    rng = np.random.default_rng(6)
    for trial in range(300):
        nb = int(rng.integers(1, 10))
        b = (rng.random(nb) ** 3).astype(np.float32)
        p = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99]))
        keep = impl.top_p_select(b, p)
        kmin = _brute_min_card(b, p)
        assert keep.sum() == kmin, (b, p, keep, kmin)
        # the minimal set is a prefix of the descending packed order
        order = np.argsort(impl.pack_keys(b))[::-1]
        assert set(np.nonzero(keep)[0]) == set(order[: kmin].tolist())
        # exhaustive: no smaller subset of any kind reaches p (tiny nb only)
        if nb <= 6 and kmin > 1:
            fr = [Fraction(float(x)) for x in b]
            tot = sum(fr)
            for sub in itertools.combinations(range(nb), kmin - 1):
                assert sum(fr[i] for i in sub) < Fraction(p) * tot


def check_eq6_and_minimality(impl):
    """Dropped mass <= (1-p) of the total (Eq. 6, aggregated form), and
    removing the last kept block falls short of p."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        nb = int(rng.integers(2, 300))
        b = np.exp(rng.standard_normal(nb) * 3).astype(np.float32)
        p = float(rng.uniform(0.5, 0.999))
        keep = impl.top_p_select(b, p)
        bf = b.astype(np.float64)
        tot = bf.sum()
        slack = nb * 2.0 ** -50 * bf.max()
        assert bf[~keep].sum() <= (1 - p) * tot + slack
        kept_sorted = np.sort(bf[keep])
        assert bf[keep].sum() - kept_sorted[0] < p * tot + slack


def check_phi(impl):
    """phi is strictly monotone over float32 (incl. +-0, subnormals, +-inf) and
    packing round-trips."""
    rng = np.random.default_rng(8)
    special = np.array([-np.inf, -3.4e38, -1.0, -1e-40, -0.0, 0.0, 1e-45, 1e-40, 1.0, 3.4e38, np.inf],
                       dtype=np.float32)
    x = np.concatenate([special, (rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000)).astype(np.float32)])
    ph = impl.phi(x).astype(np.int64)
    xf = x.astype(np.float64)
    order = np.lexsort((np.signbit(x).astype(int) * -1, xf))   # by value, -0 before +0
    ph_sorted = ph[order]
    assert np.all(np.diff(ph_sorted) >= 0)
    assert impl.phi(np.array([-0.0], np.float32))[0] < impl.phi(np.array([0.0], np.float32))[0]
    keys = impl.pack_keys(x)
    assert np.array_equal((keys >> np.uint64(32)).astype(np.uint32), impl.phi(x))
    assert np.array_equal((keys & np.uint64(0xFFFFFFFF)).astype(np.int64), np.arange(len(x)))


def check_topp_edges(impl):
    """p = 1 keeps every positive block and drops zero ones; an all-zero vector
    keeps one block (k* >= 1); larger p never keeps fewer blocks."""
    b = np.array([0.0, 2.0, 0.0, 1.0, 3.0], np.float32)
    assert np.nonzero(impl.top_p_select(b, 1.0))[0].tolist() == [1, 3, 4]
    z = np.zeros(5, np.float32)
    assert np.nonzero(impl.top_p_select(z, 0.99))[0].tolist() == [4]
    rng = np.random.default_rng(9)
    for _ in range(50):
        b = np.exp(rng.standard_normal(64) * 2).astype(np.float32)
        prev = None
        for p in [0.3, 0.6, 0.9, 0.99, 1.0]:
            k = impl.top_p_select(b, p)
            if prev is not None:
                assert np.all(k >= prev)
            prev = k


def check_expand_fixture(impl):
    g = load_golden("expand_hand_example.json")
    b = np.array(g["scores_times_64"], dtype=np.float32) / 64
    kb = impl.top_p_select(b, g["p"])
    m = impl.expand_mask(kb, g["N"], g["G"], g["A"], g["n"])
    assert m.tolist() == g["mask"]
    assert int(m.sum()) == g["kept_tokens"]


def check_expand_invariants(impl):
    rng = np.random.default_rng(10)
    for _ in range(100):
        N = int(rng.integers(1, 300))
        G = int(rng.integers(1, 40))
        A = int(rng.integers(0, 50))
        n = int(rng.integers(1, 50))
        nb = -(-N // G)
        kb = rng.random(nb) < 0.3
        m = impl.expand_mask(kb, N, G, A, n)
        i = np.arange(N)
        assert np.all(m[i < A] == 1) and np.all(m[i >= N - n] == 1)
        free = (i >= A) & (i < N - n)
        assert np.array_equal(m[free].astype(bool), kb[i[free] // G])


def f32_nearest_even(fr):
    """float32 nearest to the exact rational fr, ties to the even significand
    (a test helper: RNE from the exact value, not through float64).  Also
    returns whether fr lies within 1e-12 (relative) of a rounding midpoint,
    where an inexact float64 intermediate could round the other way."""
    x = np.float32(float(fr))
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    dist = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(dist)
    near = [c for c, dd in zip(cands, dist) if dd == best]
    if len(near) > 1:
        near = [c for c in near if int(np.array(c, np.float32).view(np.uint32)) % 2 == 0]
    lo = max(c for c in cands if Fraction(float(c)) <= fr)
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
    return np.float32(near[0]), abs(fr - mid) <= Fraction(1, 10 ** 12) * abs(fr)


def _select_fixture_common(res, g, case):
    """Outputs of select shared by both modes of the two-request fixture."""
    T = g["cu_seqlens"][-1]
    assert np.asarray(res["block_offsets"]).tolist() == g["block_offsets"], res["block_offsets"]
    assert np.asarray(res["keep_block"]).astype(int).tolist() == case["keep_block"], res["keep_block"]
    mask = np.asarray(res["mask"])
    assert mask.dtype == np.uint8 and len(mask) == T
    assert mask.tolist() == case["mask"], mask.tolist()
    assert np.asarray(res["kept"]).tolist() == case["kept"], res["kept"]


def check_select_scores_in(impl):
    """select() from given fp32 scores on two packed requests, the first at a
    nonzero stream offset, the second no longer than A + n: per-request block
    offsets (ceil(N/G), the second block partial), top-p per request, the
    expanded mask placed at each request's stream offset, and kept counts that
    include the forced sink and window tokens."""
    g = load_golden("select_two_requests.json")
    c = g["scores_in"]
    b = np.array(c["scores_times_64"], dtype=np.float32) / np.float32(64)
    res = impl.select(None, None, np.array(g["cu_seqlens"], np.int32), 1, 1, 8, g["G"], g["A"], g["n"],
                      c["p"], scores_in=b)
    _select_fixture_common(res, g, c)
    b32 = np.asarray(res["b32"])
    assert b32.dtype == np.float32 and np.array_equal(b32.view(np.uint32), b.view(np.uint32))


def check_select_q_zero(impl):
    """select() end to end with Q = 0 (closed-form uniform softmax) on the same
    two packed requests: fp64 block scores equal the hand-worked fractions,
    the fp32 scores handed to top-p are their round-to-nearest-even values,
    and equal scores are ranked larger block index first."""
    g = load_golden("select_two_requests.json")
    c = g["q_zero"]
    cu = np.array(g["cu_seqlens"], np.int32)
    T = int(cu[-1])
    hq, hkv, d = c["num_heads_q"], c["num_heads_kv"], c["head_dim"]
    q = np.zeros((T, hq, d), np.uint16)
    k = bf16_bits(np.random.default_rng(40).standard_normal((T, hkv, d)) * 2.0)
    res = impl.select(q, k, cu, hq, hkv, d, g["G"], g["A"], g["n"], c["p"])
    _select_fixture_common(res, g, c)
    exact = [Fraction(s) / c["scale_denominator"] for s in c["block_sums"]]
    b64 = np.asarray(res["b64"], dtype=np.float64)
    assert np.allclose(b64, [float(x) for x in exact], rtol=1e-14, atol=0), b64
    b32 = np.asarray(res["b32"])
    assert b32.dtype == np.float32, b32.dtype
    for i, x in enumerate(exact):
        want, near_mid = f32_nearest_even(x)
        assert not near_mid, "fixture value too close to a float32 rounding midpoint"
        assert b32[i].view(np.uint32) == want.view(np.uint32), (i, b32[i], want)


SELECT_CHECKS = [check_select_scores_in, check_select_q_zero]


TOPP_CHECKS = [check_topp_fixture, check_topp_bruteforce, check_eq6_and_minimality,
               check_phi, check_topp_edges, check_expand_fixture, check_expand_invariants]


# ---------------------------------------------------------------------------
# Compaction, carry-forward (Eq. 7-8) and metadata (Eq. 17)
# ---------------------------------------------------------------------------
def check_compact_roundtrip(impl):
    """compact then scatter-back with identity sublayers returns the input
    exactly; with f(x) = x + 1 exactly the kept rows change."""
    rng = np.random.default_rng(11)
    for _ in range(30):
        lens = rng.integers(0, 50, size=int(rng.integers(1, 6)))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
        mask = (rng.random(T) < 0.4).astype(np.uint8)
        H = rng.integers(0, 2 ** 31, size=(T, 5), dtype=np.int64)
        (out,), idx, cu_out = impl.compact(mask, cu, [H])
        assert np.array_equal(out, H[mask.astype(bool)])
        assert np.all(np.diff(idx) > 0)
        assert cu_out[-1] == mask.sum() and np.all(np.diff(cu_out) >= 0)
        for r in range(len(lens)):
            assert cu_out[r + 1] - cu_out[r] == mask[cu[r]: cu[r + 1]].sum()
        back = impl.scatter_back(H, out, idx, len(idx))
        assert np.array_equal(back, H)
        back2 = impl.scatter_back(H, out + 1, idx, len(idx))
        changed = np.any(back2 != H, axis=1)
        assert np.array_equal(changed, mask.astype(bool))


def check_compact_composition(impl):
    """A second drop on the compacted stream maps back through the first
    index map to the original rows."""
    rng = np.random.default_rng(12)
    lens = [40, 25, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    H = np.arange(T * 3).reshape(T, 3)
    m1 = (rng.random(T) < 0.6).astype(np.uint8)
    (h1,), i1, cu1 = impl.compact(m1, cu, [H])
    m2 = (rng.random(int(cu1[-1])) < 0.5).astype(np.uint8)
    (h2,), i2, cu2 = impl.compact(m2, cu1, [h1], index_in=i1)
    assert np.array_equal(H[i2], h2)
    keep_both = np.zeros(T, bool)
    keep_both[np.nonzero(m1)[0][m2.astype(bool)]] = True
    assert np.array_equal(i2, np.nonzero(keep_both)[0])


def check_eq17_fixture(impl):
    g = load_golden("eq17_example.json")
    st = impl.MetadataState.fresh([g["orig_len"]])
    cu_old = np.array([0, g["orig_len"]])
    for layer, kept in g["drops"]:
        cu_new = np.array([0, kept])
        st, nat = impl.update_metadata(st, layer, cu_old, cu_new)
        assert nat == kept
        cu_old = cu_new
    for lp, want in g["seqused_by_layer"].items():
        got = impl.seqused_eq17(st.history[0], int(lp), g["orig_len"], g["kv_len"])
        assert got == want, (lp, got, want)


def check_metadata_conservation(impl):
    """seq_lens drop by exactly the dropped count; prior context is kept."""
    rng = np.random.default_rng(13)
    lens = rng.integers(1, 100, size=6)
    ctx = rng.integers(0, 50, size=6)
    cu = np.concatenate([[0], np.cumsum(lens)])
    kept = np.array([int(rng.integers(0, L + 1)) for L in lens])
    cu_new = np.concatenate([[0], np.cumsum(kept)])
    st = impl.MetadataState.fresh(lens + ctx)
    st2, nat = impl.update_metadata(st, 3, cu, cu_new)
    assert np.array_equal(st2.seq_lens, ctx + kept)
    assert nat == kept.sum()
    assert all(h == [(3, int(ctx[r] + kept[r]))] for r, h in enumerate(st2.history))


COMPACT_CHECKS = [check_compact_roundtrip, check_compact_composition,
                  check_eq17_fixture, check_metadata_conservation]


# ---------------------------------------------------------------------------
# Per-layer KV cache slots (Eq. 16) and the paged-cache write
# ---------------------------------------------------------------------------
def check_slot_fixture(impl):
    g = load_golden("eq16_slot_example.json")
    pos = impl.retained_positions(g["cu_seqlens"], g["seq_lens"])
    assert list(pos) == g["positions"]
    s = impl.slot_mapping(g["block_table"], g["B"], g["cu_seqlens"], g["seq_lens"], g["max_tokens"])
    assert list(s) == g["slots"], list(s)


def _random_slot_case(rng, R, B, width, contiguous):
    kept = rng.integers(0, 3 * B + 5, size=R)
    ctx = rng.integers(0, 2 * B + 3, size=R)
    cu = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    seq = ctx + kept
    if contiguous:
        base = rng.integers(0, 1000, size=R)
        table = base[:, None] + np.arange(width)[None, :]
    else:
        table = rng.permutation(R * width).reshape(R, width)
    return kept, ctx, cu, seq, table


def check_slot_closed_form(impl):
    """With a contiguous table row (entries base_r, base_r + 1, ...), block
    column times B plus the offset inside the block is just p: the slot is
    base_r * B + p."""
    rng = np.random.default_rng(21)
    for B in (1, 3, 4, 16):
        kept, ctx, cu, seq, table = _random_slot_case(rng, 5, B, width=64, contiguous=True)
        s = impl.slot_mapping(table, B, cu, seq)
        for r in range(5):
            p = ctx[r] + np.arange(kept[r])
            assert np.array_equal(s[cu[r]: cu[r + 1]], table[r, 0] * B + p)


def check_slot_structure(impl):
    """Disjoint tables: valid slots are distinct, sit in the table's block for
    column floor(p/B) at offset p mod B, and exactly the positions past the
    table's width get -1."""
    rng = np.random.default_rng(22)
    for B, width in ((4, 3), (5, 6), (16, 2)):
        kept, ctx, cu, seq, table = _random_slot_case(rng, 6, B, width, contiguous=False)
        s = impl.slot_mapping(table, B, cu, seq, int(cu[-1]) + 7)
        assert np.all(s[int(cu[-1]):] == -1)
        valid = s[s >= 0]
        assert len(np.unique(valid)) == len(valid)
        for r in range(6):
            p = ctx[r] + np.arange(kept[r])
            sr = s[cu[r]: cu[r + 1]]
            inside = p // B < width
            assert np.array_equal(sr >= 0, inside)
            assert np.array_equal(sr[inside] % B, p[inside] % B)
            assert np.array_equal(sr[inside] // B, table[r, p[inside] // B])


def check_slot_eq17_consistency(impl):
    """After a drop, the positions a later layer writes are exactly the
    seqused of Eq. 17 entries of its cache (the tokens cached before this
    chunk, then the retained ones): Eq. 16 and Eq. 17 agree."""
    rng = np.random.default_rng(23)
    lens = rng.integers(1, 90, size=5)
    prior = rng.integers(0, 40, size=5)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    mask = (rng.random(int(cu[-1])) < 0.5).astype(np.uint8)
    _, _, cu_out = impl.compact(mask, cu)
    st = impl.MetadataState.fresh(lens + prior)
    st, _ = impl.update_metadata(st, 6, cu, cu_out)
    pos = impl.retained_positions(cu_out, st.seq_lens)
    for r in range(5):
        used = impl.seqused_eq17(st.history[r], 7, int(lens[r] + prior[r]), int(lens[r] + prior[r]))
        pr = pos[cu_out[r]: cu_out[r + 1]]
        assert np.array_equal(pr, np.arange(prior[r], used))


def check_kv_write(impl):
    """Every row with a slot lands in that cache row, rows past `count` and
    rows without a slot write nothing, and every other cache row keeps its
    value."""
    rng = np.random.default_rng(24)
    rows, width, nslots = 40, 6, 64
    key = rng.integers(0, 2 ** 31, size=(rows, width), dtype=np.int64)
    val = key + 7
    slots = rng.permutation(nslots + 20)[:rows] - 10        # some negative, some past the cache
    kc0 = np.full((nslots, width), -5, dtype=np.int64)
    kc, vc = impl.write_kv_cache(kc0, kc0 - 1, slots, key, val, count=33)
    hit = np.zeros(nslots, bool)
    for i in range(33):
        if 0 <= slots[i] < nslots:
            assert np.array_equal(kc[slots[i]], key[i]) and np.array_equal(vc[slots[i]], val[i])
            hit[slots[i]] = True
    assert np.all(kc[~hit] == -5) and np.all(vc[~hit] == -6)


SLOT_CHECKS = [check_slot_fixture, check_slot_closed_form, check_slot_structure,
               check_slot_eq17_consistency, check_kv_write]

# ---------------------------------------------------------------------------
# A downstream sublayer on the retained set (Eq. 7): the gated FFN
# ---------------------------------------------------------------------------
def check_ffn_fixture(impl):
    g = load_golden("ffn_swiglu_example.json")
    y = impl.ffn_swiglu(bf16_bits(np.array([g["x"]])), bf16_bits(np.array(g["w_gate_up"])),
                        bf16_bits(np.array(g["w_down"])))
    assert np.allclose(y[0], g["y"], rtol=1e-15, atol=0), y
    h = impl.ffn_hidden(bf16_bits(np.array([g["x"]])), bf16_bits(np.array(g["w_gate_up"])))
    assert np.allclose(h[0], g["h"], rtol=1e-15, atol=0), h


def check_ffn_hidden_composes(impl):
    """y is the activation h times the down projection: ffn_swiglu equals
    ffn_hidden @ Wd^T, and h = silu(x Wg^T) * (x Wu^T) channel by channel, so
    a zero up row zeroes its channel and a zero gate row does too (silu(0) = 0)."""
    rng = np.random.default_rng(35)
    rows, D, F = 9, 16, 12
    x, w, wd = _ffn_case(rng, rows, D, F)
    h = impl.ffn_hidden(x, w)
    assert h.shape == (rows, F)
    assert np.allclose(impl.ffn_swiglu(x, w, wd), h @ bits_to_f64(wd).T, rtol=1e-13, atol=1e-15)
    w0 = w.copy()
    w0[F + 3] = 0          # up row of channel 3
    w0[5] = 0              # gate row of channel 5
    h0 = impl.ffn_hidden(x, w0)
    assert np.all(h0[:, 3] == 0) and np.all(h0[:, 5] == 0)
    keep = [c for c in range(F) if c not in (3, 5)]
    assert np.array_equal(h0[:, keep], h[:, keep])


def check_silu(impl):
    """SiLU against torch's own (CPU, float64) and its odd part: silu(z) -
    silu(-z) = z."""
    import torch
    rng = np.random.default_rng(31)
    z = np.concatenate([np.linspace(-40.0, 40.0, 2001), 6.0 * rng.standard_normal(2000)])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    s = impl.silu(z)
    assert np.allclose(s, ref, rtol=1e-14, atol=1e-300)
    assert np.allclose(s - impl.silu(-z), z, rtol=1e-12, atol=1e-12)
    assert impl.silu(np.array([0.0]))[0] == 0.0


def _ffn_case(rng, rows, D, F):
    x = bf16_bits(rng.uniform(-1, 1, size=(rows, D)))
    w = bf16_bits(rng.uniform(-0.1, 0.1, size=(2 * F, D)))
    wd = bf16_bits(rng.uniform(-0.1, 0.1, size=(D, F)))
    return x, w, wd


def check_ffn_saturated_gates(impl):
    """A gate fixed at +30 makes the FFN the plain product 30 (x Wu^T) Wd^T
    (silu(30) = 30 within 1e-11); a gate of -30 silences it."""
    rng = np.random.default_rng(32)
    rows, D, F = 7, 12, 9
    x, w, wd = _ffn_case(rng, rows, D, F)
    x[:, 0] = bf16_bits(np.ones(rows))          # a constant input column drives the gates
    for gate, want_scale in ((30.0, 30.0), (-30.0, 0.0)):
        wg = np.zeros((F, D))
        wg[:, 0] = gate
        ww = w.copy()
        ww[:F] = bf16_bits(wg)
        y = impl.ffn_swiglu(x, ww, wd)
        u = bits_to_f64(x) @ bits_to_f64(w[F:]).T
        ref = want_scale * (u @ bits_to_f64(wd).T)
        assert np.allclose(y, ref, rtol=1e-10, atol=1e-9 * max(1.0, np.abs(ref).max())), gate


def check_ffn_linearity(impl):
    """Linear in the up and down weights (doubling either doubles y exactly);
    not linear in the gate."""
    rng = np.random.default_rng(33)
    rows, D, F = 5, 16, 11
    x, w, wd = _ffn_case(rng, rows, D, F)
    y = impl.ffn_swiglu(x, w, wd)
    w2 = w.copy()
    w2[F:] = bf16_bits(2.0 * bits_to_f64(w[F:]))
    assert np.allclose(impl.ffn_swiglu(x, w2, wd), 2.0 * y, rtol=1e-14, atol=0)
    assert np.allclose(impl.ffn_swiglu(x, w, bf16_bits(2.0 * bits_to_f64(wd))), 2.0 * y, rtol=1e-14, atol=0)
    wg2 = w.copy()
    wg2[:F] = bf16_bits(2.0 * bits_to_f64(w[:F]))
    assert not np.allclose(impl.ffn_swiglu(x, wg2, wd), 2.0 * y, rtol=1e-3)


def check_ffn_rows_independent(impl):
    """Token-wise: the FFN of the retained rows is the retained rows of the FFN
    of the full stream (what lets later sublayers run on the compacted
    stream, Eq. 7)."""
    rng = np.random.default_rng(34)
    x, w, wd = _ffn_case(rng, 40, 16, 24)
    keep = rng.random(40) < 0.4
    assert np.allclose(impl.ffn_swiglu(x[keep], w, wd), impl.ffn_swiglu(x, w, wd)[keep], rtol=1e-13, atol=1e-15)


FFN_CHECKS = [check_ffn_fixture, check_silu, check_ffn_saturated_gates, check_ffn_linearity,
              check_ffn_rows_independent, check_ffn_hidden_composes]

ALL_CHECKS = SCORE_CHECKS + TOPP_CHECKS + SELECT_CHECKS + COMPACT_CHECKS + SLOT_CHECKS + FFN_CHECKS
