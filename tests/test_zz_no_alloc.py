"""up_compact_noalloc (the compaction for callers that cannot allocate) against
up_compact through the C ABI: bit-identical index map, new offsets and
gathered rows, on two calls in a row sharing the per-GPU scratch, the second
with a smaller stream than the first."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import token_level_block_amd as tlb  # noqa: E402
from token_level_block_amd.runner import CompactBuffers  # noqa: E402

from gpu_helpers import dev  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(seed, lengths, rho, row_bytes, slack):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    max_tokens = T + slack
    mask = np.zeros(max_tokens, np.uint8)
    mask[:T] = (rng.random(T) < rho).astype(np.uint8) * rng.integers(1, 256, T).astype(np.uint8)
    mask[T:] = 1          # beyond the stream: must be ignored
    bufs = [rng.integers(0, 2 ** 32, size=(max_tokens, rb // 4), dtype=np.uint64).astype(np.uint32)
            for rb in row_bytes]
    index_in = rng.permutation(10 * max_tokens)[:max_tokens].astype(np.int32)
    return cu, mask, bufs, index_in


def _run_both(cu, mask, bufs, index_in):
    R = len(cu) - 1
    max_tokens = len(mask)
    cu_d, mask_d = dev(cu), dev(mask)
    src = [dev(b.view(np.int32)) for b in bufs]
    idx_d = None if index_in is None else dev(index_in)
    # the existing entry point, with its own workspace
    dst_ref = [torch.full_like(s, -7) for s in src]
    cb = CompactBuffers.allocate(R, max_tokens)
    cb.index_out.fill_(-5)
    cb.run(mask_d, cu_d, src, dst_ref, index_in=idx_d)
    # the allocation-free one: same inputs, outputs of its own
    dst = [torch.full_like(s, -7) for s in src]
    index_out = torch.full((max_tokens,), -5, dtype=torch.int32, device="cuda")
    cu_out = torch.full((R + 1,), -9, dtype=torch.int32, device="cuda")
    rb = [b.shape[1] * 4 for b in bufs]
    tlb.compact_noalloc(mask_d, cu_d, R, max_tokens, src, dst, rb, idx_d, index_out, cu_out)
    torch.cuda.synchronize()
    return cb, dst_ref, dst, index_out, cu_out


def test_compact_noalloc_matches_compact_on_two_calls():
    cases = [
        # longer than 131072 tokens (count + rank path), three buffers, composed index
        dict(seed=1, lengths=(90000, 0, 70000), rho=0.4, row_bytes=(8192, 4, 12), slack=37, use_index=True),
        # then a smaller stream on the same scratch (one-launch rank path), two buffers
        dict(seed=2, lengths=(5000, 3000, 1), rho=0.6, row_bytes=(16, 4096), slack=0, use_index=False),
    ]
    for c in cases:
        say(f"[noalloc] lengths={c['lengths']} rho={c['rho']} row_bytes={c['row_bytes']}")
        cu, mask, bufs, index_in = _case(c["seed"], c["lengths"], c["rho"], c["row_bytes"], c["slack"])
        use = index_in if c["use_index"] else None
        cb, dst_ref, dst, index_out, cu_out = _run_both(cu, mask, bufs, use)
        R = len(cu) - 1
        _, idx, cu_ref = oracle.compact(mask, cu, [], use)
        K = len(idx)
        assert torch.equal(cu_out, cb.cu_out[: R + 1])
        assert np.array_equal(cu_out.cpu().numpy(), cu_ref)
        assert torch.equal(index_out, cb.index_out[: len(mask)])   # kept part and the untouched rest
        assert np.array_equal(index_out[:K].cpu().numpy(), idx)
        for a, b in zip(dst, dst_ref):
            assert torch.equal(a, b)
        say(f"[noalloc] {K} of {int(cu[-1])} rows kept: identical to up_compact")


def test_compact_noalloc_rejects_a_stream_past_its_scratch():
    mask = torch.zeros(16, dtype=torch.uint8, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.zeros(16, dtype=torch.int32, device="cuda")
    st = tlb.compact_noalloc(mask, cu, 1, tlb.COMPACT_NOALLOC_MAX_TOKENS + 1, [], [], [], None, out, cu,
                             raise_on_error=False)
    assert st == tlb.UP_ERR_WORKSPACE
