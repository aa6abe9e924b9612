"""Helpers for the GPU parity tests: device uploads and the comparison rules.

Comparison rules (UniPrefill selection path vs the CPU oracle):
  * block scores: |gpu - ref| <= 1e-3 |ref| + 1e-30 sum(ref) per request, where
    ref is the oracle's float64 score and the GPU accumulates in fp32 from the
    same bf16 inputs (the absolute floor only matters for blocks whose mass
    underflows fp32);
  * top-p, masks, compaction and metadata: bit-exact when both sides get the
    same fp32 score vector or the same mask;
  * end-to-end masks: a block may differ only if its oracle score is within
    1e-3 of the oracle's last kept score, or the oracle's cumulative mass
    fraction just before or at its rank is within 1e-3 of p.
"""
from __future__ import annotations

import numpy as np
import torch

SCORE_RTOL = 1e-3
SCORE_ATOL_FRAC = 1e-30
NEAR = 1e-3


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload_qk(wl, cu, q, k):
    """Q goes up only for each request's window rows; the rest stays zero."""
    T = int(cu[-1])
    qd = torch.zeros((max(T, 1), wl.hq, wl.d), dtype=torch.int16, device="cuda")
    for r in range(wl.num_reqs):
        s, N = int(cu[r]), int(cu[r + 1] - cu[r])
        ne = min(wl.n, N)
        if ne > 0:
            qd[s + N - ne: s + N] = dev(q[s + N - ne: s + N].view(np.int16))
    kd = dev(k.view(np.int16)) if T > 0 else torch.zeros((1, wl.hkv, wl.d), dtype=torch.int16, device="cuda")
    return dev(cu.astype(np.int32)), qd, kd


def check_scores(b_gpu, b_ref, offs):
    for r in range(len(offs) - 1):
        a, z = int(offs[r]), int(offs[r + 1])
        ref = b_ref[a:z]
        got = b_gpu[a:z].astype(np.float64)
        tol = SCORE_RTOL * np.abs(ref) + SCORE_ATOL_FRAC * ref.sum()
        bad = np.nonzero(np.abs(got - ref) > tol)[0]
        assert len(bad) == 0, (f"request {r}: {len(bad)} block scores out of tolerance; first "
                               f"g={bad[0]} gpu={got[bad[0]]!r} ref={ref[bad[0]]!r}")


def allowed_mismatch(b32, keep_ref, p):
    """Blocks of one request whose keep flag may legitimately differ."""
    nb = len(b32)
    bits = b32.view(np.uint32)
    phi = np.where(bits >> 31, bits ^ np.uint32(0xFFFFFFFF), bits ^ np.uint32(0x80000000)).astype(np.uint64)
    key = (phi << np.uint64(32)) | np.arange(nb, dtype=np.uint64)
    order = np.argsort(key)[::-1]
    bf = np.where(np.isfinite(b32) & (b32 > 0), b32.astype(np.float64), 0.0)
    tot = bf.sum()
    frac = np.cumsum(bf[order]) / tot if tot > 0 else np.ones(nb)
    rank = np.empty(nb, dtype=np.int64)
    rank[order] = np.arange(nb)
    kept_sorted = np.nonzero(keep_ref[order])[0]
    tau = bf[order[kept_sorted[-1]]] if len(kept_sorted) else 0.0
    before = np.where(rank > 0, frac[np.maximum(rank - 1, 0)], 0.0)
    at = frac[rank]
    return (np.abs(bf - tau) <= NEAR * tau) | (np.abs(before - p) <= NEAR) | (np.abs(at - p) <= NEAR)


def check_masks(ref, keep_gpu, mask_gpu, kept_gpu, cu, wl):
    """End-to-end keep flags within the threshold rule; the GPU mask and kept
    counts must agree with the GPU keep flags exactly."""
    offs = ref["block_offsets"]
    mism_total = 0
    for r in range(wl.num_reqs):
        a, z = int(offs[r]), int(offs[r + 1])
        kr = ref["keep_block"][a:z].astype(bool)
        kg = keep_gpu[a:z].astype(bool)
        diff = np.nonzero(kr != kg)[0]
        mism_total += len(diff)
        if len(diff):
            ok = allowed_mismatch(ref["b32"][a:z], kr, wl.p)
            assert ok[diff].all(), f"request {r}: blocks {diff[~ok[diff]][:10]} differ away from the threshold"
        # the GPU's token mask expands the GPU's own keep flags exactly
        s, N = int(cu[r]), int(cu[r + 1] - cu[r])
        i = np.arange(N)
        want = (kg[i // wl.G] | (i < wl.A) | (i >= N - wl.n)).astype(np.uint8) if N else np.zeros(0, np.uint8)
        assert np.array_equal(mask_gpu[s:s + N], want), f"request {r}: mask does not expand keep flags"
        assert int(kept_gpu[r]) == int(want.sum())
        if len(diff) == 0:
            assert int(kept_gpu[r]) == int(ref["kept"][r])
    return mism_total
