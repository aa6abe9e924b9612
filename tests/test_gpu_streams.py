"""Two independent batches on two streams at once: the library keeps no state
of its own, so calls on disjoint buffers may run concurrently.  Two different
workloads (so that any mixing between them shows) run their whole step
(selection, compaction, metadata, Eq. 8 scatter) on their own streams, both
free-running and phased the way the benchmark pipelines them (each
selection waits for the other batch's), for several rounds; every round's
outputs must equal each batch's single-stream step bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import upload_qk

tlb = pytest.importorskip("token_level_block_amd")
from token_level_block_amd.runner import (CompactBuffers, MetadataBuffers, SelectBuffers,  # noqa: E402
                                          run_scatter_back)

pytestmark = pytest.mark.gpu


class Batch:
    def __init__(self, wl):
        cu, q, k = synth.make_qk(wl)
        self.cu_d, self.qd, self.kd = upload_qk(wl, cu, q, k)
        self.T, self.R = int(cu[-1]), wl.num_reqs
        self.lengths = np.diff(cu)
        self.hidden = synth.hidden_words_torch(0, self.T, wl.hidden // 2, "cuda")
        self.out = torch.zeros_like(self.hidden)
        self.full = self.hidden.clone()
        self.prm = tlb.make_params(wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
        self.sel = SelectBuffers.allocate(self.prm, self.R, self.T)
        self.cb = CompactBuffers.allocate(self.R, self.T)
        self.stream = torch.cuda.Stream()

    def select(self, s):
        self.sel.run(self.qd, self.kd, self.cu_d, stream=s)

    def rest(self, s, mb):
        self.cb.run(self.sel.keep_mask, self.cu_d, [self.hidden], [self.out], stream=s)
        mb.run(1, self.cu_d, self.cb.cu_out, stream=s)
        run_scatter_back(self.out, self.cb.index_out, self.cb.cu_out, self.R, self.T, self.full, stream=s)

    def outputs(self, mb):
        kept = int(self.cb.cu_out[self.R])
        return [t.clone() for t in (self.sel.keep_mask[:self.T], self.sel.kept[:self.R],
                                    self.sel.block_scores[:int(self.sel.block_offsets[self.R])],
                                    self.cb.cu_out, self.cb.index_out[:kept], self.out[:kept], self.full,
                                    mb.seq_lens, mb.drop_count)]

    def metadata(self):
        return MetadataBuffers.allocate(self.lengths, num_layers=4, max_drops=2)


@pytest.mark.parametrize("phased", [False, True], ids=["free", "phased"])
def test_two_batches_on_two_streams_match_one_stream(phased):
    print(f"[streams] phased={phased}", file=sys.stderr, flush=True)
    batches = [Batch(synth.llama_varlen4()),
               Batch(synth.tiny((3000, 900, 2500), hq=8, hkv=2, d=128, hidden=512, G=64, A=64, n=64, p=0.95,
                                seed=61, kind="powerlaw", c=1.4))]
    main = torch.cuda.current_stream().cuda_stream
    refs = []
    for b in batches:
        mb = b.metadata()
        b.select(main)
        b.rest(main, mb)
        torch.cuda.synchronize()
        refs.append(b.outputs(mb))
    for rnd in range(4):
        mbs = [b.metadata() for b in batches]
        for b in batches:
            b.sel.keep_mask.fill_(0)
            b.out.zero_()
            b.stream.wait_stream(torch.cuda.current_stream())
        done = [torch.cuda.Event(), torch.cuda.Event()]
        for i, b in enumerate(batches):
            if phased and i == 1:
                b.stream.wait_event(done[0])
            b.select(b.stream.cuda_stream)
            done[i].record(b.stream)
            b.rest(b.stream.cuda_stream, mbs[i])
        for b in batches:
            torch.cuda.current_stream().wait_stream(b.stream)
        torch.cuda.synchronize()
        for i, b in enumerate(batches):
            got = b.outputs(mbs[i])
            for j, (x, y) in enumerate(zip(got, refs[i])):
                assert torch.equal(x, y), f"round {rnd}, batch {i}: output {j} differs from its single-stream run"
