"""GPU parity of the gated FFN sublayer (UniPrefill Sec. 3.4 Eq. 7: later
sublayers run on the retained rows only) against the CPU oracle, and the
Eq. 7 + Eq. 8 composition on the 128K LLaMA layer: compact the rows, run the
FFN on the retained set, scatter back.

Tolerance, element by element, from the rounding steps of the GPU path (bf16
inputs; products exact in fp32; every sum accumulated in fp32; h = silu(g) * u
formed in fp32 from the fp32 gate and up sums, then rounded to bf16; y
accumulated in fp32 and rounded to bf16).  With u = 2^-8 the unit roundoff of
bf16 and Y, H the oracle's float64 output and activation, output element i of
a row may differ from Y_i by at most
    u |Y_i|                                  rounding of y to bf16,
  + 7 (u / sqrt 3) sqrt(sum_f H_f^2 Wd_if^2)  rounding of each h_f to bf16: F
                                             independent round-to-nearest errors
                                             of at most u |H_f| (standard
                                             deviation u/sqrt 3 relative), taken
                                             at seven standard deviations,
  + 2^-16 sum_f |H_f Wd_if|                  fp32 accumulation of the three
                                             products and the fp32 SiLU: relative
                                             errors of order sqrt(K) 2^-24 < 2^-16
                                             on each term.
Beside the per-element bound, the errors over a whole output, in units of the
standard deviation this model predicts (the two bf16 roundings), must have an
RMS below 1.5: an error that the rounding model does not explain fails even
when each element stays inside its bound.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import dev

tlb = pytest.importorskip("token_level_block_amd")
from token_level_block_amd.runner import CompactBuffers, run_scatter_back  # noqa: E402

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
LAMBDA = 7.0
SLACK_FP32 = 2.0 ** -16
RMS_UNITS = 1.5


def say(*a):
    print(*a, flush=True)


@functools.lru_cache(maxsize=None)
def host_weights(D, F):
    return synth.ffn_weights(D, F)


def bits_dev(bits):
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def gpu_ffn(ffn, x, rows, wg, wd):
    y = torch.empty((max(rows, 1), ffn.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ffn.workspace_bytes(rows), dtype=torch.uint8, device="cuda")
    ffn.forward(x, rows, wg, wd, y, ws)
    torch.cuda.synchronize()
    return y[:rows]


def check_rows(y_gpu, x_bits, wg_bits, wd_bits, where=""):
    """Every element of every given row within the rounding bound; the RMS of
    the errors in predicted standard deviations below RMS_UNITS."""
    H = oracle.ffn_hidden(x_bits, wg_bits)
    wd = oracle.bf16_bits_to_f64(np.asarray(wd_bits))
    Y = H @ wd.T
    got = y_gpu.float().cpu().numpy().astype(np.float64)
    assert got.shape == Y.shape, (got.shape, Y.shape)
    h_sq = np.sqrt((H * H) @ (wd * wd).T)                # sqrt(sum_f H_f^2 Wd_if^2)
    h_abs = np.abs(H) @ np.abs(wd).T                     # sum_f |H_f Wd_if|
    bound = U_BF16 * np.abs(Y) + LAMBDA * (U_BF16 / np.sqrt(3.0)) * h_sq + SLACK_FP32 * h_abs
    err = np.abs(got - Y)
    ratio = err / np.maximum(bound, 1e-300)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio.max() <= 1.0, (where, worst, got[worst], Y[worst], bound[worst])
    sigma = (U_BF16 / np.sqrt(3.0)) * np.sqrt(h_sq ** 2 + Y ** 2)
    rms = float(np.sqrt(np.mean((err / np.maximum(sigma, 1e-300)) ** 2)))
    assert rms <= RMS_UNITS, (where, rms)
    say(f"  {where}: {Y.size} elements, worst error {ratio.max():.3f} of its bound, "
        f"RMS {rms:.3f} predicted standard deviations")
    return Y


# K = D or F: whole 64-element stages, a partial last stage (1000, 200, 584,
# 136, 72, 1096), a single partial stage (8, 16, 24); the narrowest widths (D or
# F = 8); a token tile past a multiple of 256 rows (257); weight panels fewer than 8
# (one XCD walk) and 9 (the shared walk, split unevenly over the XCDs)
@pytest.mark.parametrize("rows,D,F", [(300, 256, 512), (1, 64, 8), (77, 128, 1000), (513, 512, 1536),
                                      (130, 200, 584), (64, 136, 72), (300, 2304, 1096),
                                      (5, 8, 16), (3, 16, 8), (257, 72, 24)])
def test_ffn_small_shapes_all_rows(rows, D, F):
    rng_seed = rows + D + F
    wg = synth.uniform_bf16_bits(11 + rng_seed, 0, 2 * F, D, -4)
    wd = synth.uniform_bf16_bits(12 + rng_seed, 0, D, F, -5)
    x = synth.uniform_bf16_bits(13 + rng_seed, 0, rows, D, 0)
    ffn = tlb.FFN(D, F)
    y = gpu_ffn(ffn, bits_dev(x), rows, bits_dev(wg), bits_dev(wd))
    check_rows(y, x, wg, wd, f"{rows}x{D}x{F}")


# The tile walk's XCD grids over several groups of 8 token panels (11 panels:
# a full group and a partial one): 8 and 16 weight panels in both launches
# (grids of 2 x 4 and 4 x 2 XCDs), and 32 gate/up panels (8 x 1) beside a down
# launch of 4 (fewer than 8: the plain walk).  One row of every token panel,
# every output column: each row
# reads h over all gate/up panels and writes y over all down panels, so every
# tile of both launches is checked.
@pytest.mark.parametrize("D,F", [(2048, 1024), (4096, 2048), (1024, 4096)])
def test_ffn_tile_walk_grids(D, F):
    rows = 2600
    wg = synth.uniform_bf16_bits(61 + D, 0, 2 * F, D, -5)
    wd = synth.uniform_bf16_bits(62 + F, 0, D, F, -5)
    x = synth.uniform_bf16_bits(63, 0, rows, D, 0)
    ffn = tlb.FFN(D, F)
    y = gpu_ffn(ffn, bits_dev(x), rows, bits_dev(wg), bits_dev(wd))
    pick = np.array(sorted({min(rows - 1, 256 * t + (37 * t) % 256) for t in range((rows + 255) // 256)}
                           | {rows - 1}))
    check_rows(y[torch.from_numpy(pick).cuda()], x[pick], wg, wd, f"walk {rows}x{D}x{F}, rows {pick.tolist()}")


def test_ffn_zero_rows_is_a_no_op():
    ffn = tlb.FFN(64, 64)
    y = torch.full((4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ffn.workspace_bytes(0), dtype=torch.uint8, device="cuda")
    assert ffn.forward(y, 0, y, y, y, ws) == tlb.UP_OK
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


@pytest.mark.parametrize("model,rows", [("llama8b", 128), ("gemma3", 97)])
def test_ffn_model_shapes_all_rows(model, rows):
    """LLaMA-3.1-8B (4096 / 14336) and Gemma-3-12B (3840 / 15360) widths:
    every element of every row against the oracle."""
    D = {"llama8b": 4096, "gemma3": 3840}[model]
    F = synth.FFN_INTERMEDIATE[model]
    wg, wd = host_weights(D, F)
    x = synth.ffn_activations(rows, D)
    ffn = tlb.FFN(D, F)
    y = gpu_ffn(ffn, bits_dev(x), rows, bits_dev(wg), bits_dev(wd))
    check_rows(y, x, wg, wd, model)


def test_ffn_rows_are_independent_of_their_tile():
    """The same token rows give bit-identical outputs wherever they sit in the
    batch (first rows of a tile, last rows, a short last tile): nothing in a
    row's arithmetic depends on the other rows."""
    D, F = 512, 1024
    wg = synth.uniform_bf16_bits(41, 0, 2 * F, D, -4)
    wd = synth.uniform_bf16_bits(42, 0, D, F, -5)
    x = synth.uniform_bf16_bits(43, 0, 700, D, 0)
    ffn = tlb.FFN(D, F)
    wgd, wdd = bits_dev(wg), bits_dev(wd)
    full = gpu_ffn(ffn, bits_dev(x), 700, wgd, wdd)
    for lo, hi in [(0, 37), (250, 262), (511, 700), (699, 700)]:
        part = gpu_ffn(ffn, bits_dev(x[lo:hi]), hi - lo, wgd, wdd)
        assert torch.equal(part, full[lo:hi]), (lo, hi)


@pytest.mark.timeout(900)
def test_ffn_on_retained_rows_128k():
    """The 128K LLaMA layer: 131072 activation rows, 40 % of 64-token blocks
    kept.  The FFN on the compacted rows agrees with the FFN of the full
    stream on those rows; after the Eq. 8 scatter the full buffer holds the
    FFN output on kept rows and its old rows elsewhere (bit-exact); sampled
    rows against the oracle."""
    T, D, F, G = 131072, 4096, synth.FFN_INTERMEDIATE["llama8b"], 64
    wg, wd = host_weights(D, F)
    wgd, wdd = bits_dev(wg), bits_dev(wd)
    x = synth.ffn_activations_torch(T, D, "cuda")
    rng = np.random.default_rng(10)
    keep_block = rng.random(T // G) < 0.4
    mask = np.repeat(keep_block, G).astype(np.uint8)
    cu = np.array([0, T], dtype=np.int32)
    cb = CompactBuffers.allocate(1, T)
    xc = torch.empty_like(x)
    cb.run(dev(mask), dev(cu), [x.view(torch.int16)], [xc.view(torch.int16)])
    torch.cuda.synchronize()
    K = int(cb.cu_out[1].item())
    assert K == int(mask.sum())
    ffn = tlb.FFN(D, F)
    y_kept = gpu_ffn(ffn, xc, K, wgd, wdd)
    y_full = gpu_ffn(ffn, x, T, wgd, wdd)
    idx = cb.index_out[:K].to(torch.int64)
    # a row's output does not depend on where it sits in the stream
    assert torch.equal(y_kept, y_full[idx])
    # Eq. 8: the full-length state takes the sublayer's output on kept rows only
    full = x.clone()
    run_scatter_back(y_kept.view(torch.int16), cb.index_out, cb.cu_out, 1, T, full.view(torch.int16))
    torch.cuda.synchronize()
    keep_t = dev(mask).bool()
    assert torch.equal(full[~keep_t], x[~keep_t])
    assert torch.equal(full[idx], y_kept)
    sample = np.sort(rng.choice(np.nonzero(mask)[0], size=64, replace=False))
    xs = np.concatenate([synth.ffn_activations(1, D, row0=int(r)) for r in sample])
    check_rows(full[torch.from_numpy(sample).cuda()], xs, wg, wd, "128k sampled kept rows")
    say(f"  kept {K}/{T} rows; FFN of the compacted rows bit-identical to the full stream's")
