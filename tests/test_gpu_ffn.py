"""GPU parity of the gated FFN sublayer (UniPrefill Sec. 3.4 Eq. 7: later
sublayers run on the retained rows only) against the CPU oracle, and the
Eq. 7 + Eq. 8 composition on the 128K LLaMA layer: compact the rows, run the
FFN on the retained set, scatter back.

Tolerance (floating point, derived from the arithmetic): the GPU multiplies
bf16 inputs exactly and accumulates in fp32, but rounds the gate/up product
and the activation h to bf16 (relative 2^-9 each) and y to bf16.  An error of
a few 2^-9 on each of the F terms of y = h Wd^T, with random signs, gives a
relative L2 error per row of about 5e-3; the bound is 1.5e-2 per row, and no
element may be off by more than 0.05 of its row's rms (about 10 sigma).
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

ROW_REL_L2 = 1.5e-2
ELEM_OF_RMS = 0.05


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
    ref = oracle.ffn_swiglu(x_bits, wg_bits, wd_bits)
    got = y_gpu.float().cpu().numpy().astype(np.float64)
    for i in range(len(ref)):
        rms = np.sqrt(np.mean(ref[i] ** 2))
        rel = np.linalg.norm(got[i] - ref[i]) / np.linalg.norm(ref[i])
        worst = np.abs(got[i] - ref[i]).max() / rms
        assert rel <= ROW_REL_L2 and worst <= ELEM_OF_RMS, (where, i, rel, worst)
    return ref


@pytest.mark.parametrize("rows,D,F", [(300, 256, 512), (1, 64, 8), (77, 128, 1000), (513, 512, 1536)])
def test_ffn_small_shapes_all_rows(rows, D, F):
    rng_seed = rows + D + F
    wg = synth.uniform_bf16_bits(11 + rng_seed, 0, 2 * F, D, -4)
    wd = synth.uniform_bf16_bits(12 + rng_seed, 0, D, F, -5)
    x = synth.uniform_bf16_bits(13 + rng_seed, 0, rows, D, 0)
    ffn = tlb.FFN(D, F)
    y = gpu_ffn(ffn, bits_dev(x), rows, bits_dev(wg), bits_dev(wd))
    check_rows(y, x, wg, wd, f"{rows}x{D}x{F}")


def test_ffn_zero_rows_is_a_no_op():
    ffn = tlb.FFN(64, 64)
    y = torch.full((4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ffn.workspace_bytes(0), dtype=torch.uint8, device="cuda")
    assert ffn.forward(y, 0, y, y, y, ws) == tlb.UP_OK
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


@pytest.mark.parametrize("model,rows", [("llama8b", 777), ("gemma3", 513)])
def test_ffn_model_shapes_sampled_rows(model, rows):
    D = {"llama8b": 4096, "gemma3": 3840}[model]
    F = synth.FFN_INTERMEDIATE[model]
    wg, wd = host_weights(D, F)
    x = synth.ffn_activations(rows, D)
    ffn = tlb.FFN(D, F)
    y = gpu_ffn(ffn, bits_dev(x), rows, bits_dev(wg), bits_dev(wd))
    sample = np.array([0, 1, rows // 3, rows // 2, rows - 2, rows - 1])
    check_rows(y[torch.from_numpy(sample).cuda()], x[sample], wg, wd, model)


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
    a, b = y_kept.float(), y_full[idx].float()
    rel = (a - b).norm(dim=1) / b.norm(dim=1)
    assert float(rel.max()) <= ROW_REL_L2, float(rel.max())
    # Eq. 8: the full-length state takes the sublayer's output on kept rows only
    full = x.clone()
    run_scatter_back(y_kept.view(torch.int16), cb.index_out, cb.cu_out, 1, T, full.view(torch.int16))
    torch.cuda.synchronize()
    keep_t = dev(mask).bool()
    assert torch.equal(full[~keep_t], x[~keep_t])
    assert torch.equal(full[idx], y_kept)
    sample = np.sort(rng.choice(np.nonzero(mask)[0], size=6, replace=False))
    xs = np.concatenate([synth.ffn_activations(1, D, row0=int(r)) for r in sample])
    check_rows(full[torch.from_numpy(sample).cuda()], xs, wg, wd, "128k")
    say(f"  kept {K}/{T} rows; max row rel diff compacted vs full {float(rel.max()):.2e}")
