"""The whole hot-path step (selection, compaction, metadata, Eq. 8 scatter,
Eq. 16 slots and the KV-cache write) captured once in a HIP graph: every
library call only enqueues kernels, so it is capturable.  The graph is
replayed several times, with the program's own eager work and
synchronizations in between, and every replay must reproduce the eager
step's outputs bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import upload_qk

tlb = pytest.importorskip("token_level_block_amd")
from token_level_block_amd.runner import (CompactBuffers, MetadataBuffers, SelectBuffers,  # noqa: E402
                                          run_scatter_back)

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    wl = synth.llama_varlen4()
    cu, q, k = synth.make_qk(wl)
    cu_d, qd, kd = upload_qk(wl, cu, q, k)
    T, R = int(cu[-1]), wl.num_reqs
    nwords = wl.hidden // 2
    hidden = synth.hidden_words_torch(0, T, nwords, "cuda")
    out = torch.empty_like(hidden)
    full = hidden.clone()
    prm = tlb.make_params(wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    sel = SelectBuffers.allocate(prm, R, T)
    cb = CompactBuffers.allocate(R, T)
    B, width = 16, T // 16 + 2
    table = torch.arange(R * width, dtype=torch.int32, device="cuda").flip(0).reshape(R, width).contiguous()
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    rb = wl.hkv * wl.d * 2
    kv = torch.randint(-2 ** 15, 2 ** 15 - 1, (T, rb // 2), dtype=torch.int16, device="cuda")
    kcache = torch.zeros((R * width * B, rb // 2), dtype=torch.int16, device="cuda")

    def step(s, mb):
        sel.run(qd, kd, cu_d, stream=s)
        cb.run(sel.keep_mask, cu_d, [hidden], [out], stream=s)
        mb.run(2, cu_d, cb.cu_out, stream=s)
        run_scatter_back(out, cb.index_out, cb.cu_out, R, T, full, stream=s)
        tlb.slot_mapping(table, width, width, B, cb.cu_out, mb.seq_lens, R, T, slots, stream=s)
        tlb.write_kv_cache(kv, rb, None, 0, rb, slots, cb.cu_out, R, T, kcache, None, R * width * B, stream=s)

    outputs = (sel.keep_mask, sel.kept, sel.block_scores, cb.cu_out, cb.index_out, out, full, slots, kcache)
    cleared = (sel.keep_mask, sel.block_scores, cb.index_out, out, slots, kcache)

    def fresh_metadata():
        return MetadataBuffers.allocate(np.diff(cu), num_layers=8, max_drops=2)

    mb_eager = fresh_metadata()
    for t in cleared:        # entries past the live rows are never written: start them all at zero
        t.zero_()
    step(torch.cuda.current_stream().cuda_stream, mb_eager)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    ref_meta = [t.clone() for t in (mb_eager.seq_lens, mb_eager.num_actual_tokens, mb_eager.seqused_base)]

    mb_graph = fresh_metadata()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side.cuda_stream, fresh_metadata())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream().cuda_stream, mb_graph)
    torch.cuda.synchronize()

    for i in range(4):
        # the program's own eager work between replays
        for t in cleared:
            t.zero_()
        step(torch.cuda.current_stream().cuda_stream, fresh_metadata())
        torch.cuda.synchronize()
        for t in cleared:
            t.zero_()
        for t, v in zip((mb_graph.seq_lens, mb_graph.num_actual_tokens, mb_graph.drop_count,
                         mb_graph.seqused_base),
                        (torch.as_tensor(np.diff(cu), dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                         torch.zeros(R, dtype=torch.int32),
                         torch.as_tensor(np.diff(cu), dtype=torch.int32).repeat(8))):
            t.copy_(v.cuda())
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("keep_mask", "kept", "block_scores", "cu_out", "index_out", "out", "full",
                                    "slots", "kcache"), outputs, ref):
            assert torch.equal(got, want), (i, name)
        for got, want in zip((mb_graph.seq_lens, mb_graph.num_actual_tokens, mb_graph.seqused_base), ref_meta):
            assert torch.equal(got, want), i


def test_ffn_graph_replays_match_eager():
    """The FFN sublayer (its two GEMM launches) captured in a HIP graph: every
    replay, with eager FFN calls on other inputs in between, reproduces the
    eager output bit for bit."""
    rows, D, F = 700, 512, 1536
    wg = synth.uniform_bf16_bits(71, 0, 2 * F, D, -5)
    wd = synth.uniform_bf16_bits(72, 0, D, F, -5)
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    x = to_dev(synth.uniform_bf16_bits(73, 0, rows, D, 0))
    x_other = to_dev(synth.uniform_bf16_bits(74, 0, rows, D, 0))
    wgd, wdd = to_dev(wg), to_dev(wd)
    ffn = tlb.FFN(D, F)
    ws = torch.empty(ffn.workspace_bytes(rows), dtype=torch.uint8, device="cuda")
    y = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    y_other = torch.empty_like(y)
    ffn.forward(x, rows, wgd, wdd, y, ws)
    torch.cuda.synchronize()
    ref = y.clone()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ffn.forward(x, rows, wgd, wdd, y, ws, stream=side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        ffn.forward(x, rows, wgd, wdd, y, ws, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for i in range(4):
        ffn.forward(x_other, rows, wgd, wdd, y_other, ws)   # eager work on the same workspace
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), i
    ffn.close()
