#!/usr/bin/env python3
"""Benchmark of the UniPrefill token-selection hot path on one MI355X.

One step = one full-attention layer's pass over the hot path on the resident
workload: up_select_blocks (score GEMM + online softmax + block reduce, top-p,
expansion), up_compact of the hidden rows and token positions,
up_update_metadata, and the Eq. 8 up_scatter_back of the hidden rows.  The
workload is one 131072-token request shaped like a LLaMA-3.1-8B full-attention layer (32 query heads, 8 KV heads, head_dim 128,
hidden 4096, bf16), seeded synthetic data (synth.llama_128k).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "selected+compacted prefill tokens/s at 128K (1 GPU); % MFMA and % HBM roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (the library records
    them on the stream its kernels run on)."""

    def __init__(self):
        # by soname, so the runtime torch (and the library) already loaded is reused
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def new(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(e.value)
        return e.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def cpu_oracle_step(wl, cu, q, k, hidden_host):
    """One step of the same path through the CPU oracle (float64 NumPy)."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    sel = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    (out,), idx, cu_out = oracle.compact(sel["mask"], cu, [hidden_host])
    st = oracle.MetadataState.fresh(np.diff(cu))
    st, nat = oracle.update_metadata(st, 0, cu, cu_out)
    full = oracle.scatter_back(hidden_host, out, idx, len(idx))
    dt = time.perf_counter() - t0
    del full, out
    return dt, sel


SCORE_SOURCES = ("score_plan.h", "score.hip")   # the kernel and the plan that sizes its launch


def score_sources_sha(root):
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(root, "token_level_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(root):
    """HBM bytes per score-kernel launch from the committed counter summary, or
    None when the kernel or its launch configuration has changed since the
    counters were taken."""
    import re
    prof = os.path.join(root, "profiles", "score_kernel_llama8b_128k_hbm.md")
    try:
        text = open(prof).read()
        sha = score_sources_sha(root)
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"score kernel sources sha256 at measurement: `([0-9a-f]+)`", text)
    if not m or not h or h.group(1) != sha:
        return None
    return int(m.group(1))


def measure_peaks(stream, ev):
    """Rates this GPU sustains, from libuppeaks: dense bf16 MFMA on random
    operands with the 32x32x16 instruction (the score kernel's) and the
    16x16x32 one (the FFN GEMM's), in TFLOP/s, and a streaming 1 GiB device
    copy (GB/s, read + write).  Best of three launches after one warm-up each."""
    import torch
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                   "token_level_block_amd", "libuppeaks.so"))
    lib.upk_mfma_out_floats.restype = ctypes.c_int64
    lib.upk_mfma_out_floats.argtypes = [ctypes.c_int32]
    lib.upk_mfma_flops.restype = ctypes.c_double
    lib.upk_mfma_flops.argtypes = [ctypes.c_int32]
    lib.upk_mfma_launch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.upk_mfma16_launch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.upk_copy_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_void_p]

    def best(launch, work):
        rates = []
        for i in range(4):
            a, b = ev.new(), ev.new()
            ev.record(a, stream)
            if launch() != 0:
                raise RuntimeError("peak probe launch failed")
            ev.record(b, stream)
            if i > 0:
                rates.append(work / (ev.ms(a, b) * 1e-3))
        return max(rates)

    blocks = 256 * 8
    out = torch.empty(lib.upk_mfma_out_floats(blocks), dtype=torch.float32, device="cuda")
    mfma = best(lambda: lib.upk_mfma_launch(out.data_ptr(), blocks, stream), lib.upk_mfma_flops(blocks)) / 1e12
    mfma16 = best(lambda: lib.upk_mfma16_launch(out.data_ptr(), blocks, stream), lib.upk_mfma_flops(blocks)) / 1e12
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy = best(lambda: lib.upk_copy_launch(src.data_ptr(), dst.data_ptr(), nbytes, 0, stream),
                2.0 * nbytes) / 1e9
    torch.cuda.synchronize()
    del out, src, dst
    return mfma, mfma16, copy


def time_kv_cache(cu_out, seq_lens, R, kept, wl, stream, ev, reps, B=16):
    """Eq. 16 slot mapping and the paged-cache write of the step's retained
    rows (as the next layer would store them): random K and V rows of Hkv x d
    bf16, KV block size 16, a shuffled block table; the MALL is flushed before
    each timed call."""
    import numpy as np
    import torch
    import token_level_block_amd as tlb
    rb = wl.hkv * wl.d * 2
    width = (kept + B - 1) // B + 1
    rng = np.random.default_rng(wl.seed + 16)
    table = torch.from_numpy(rng.permutation(R * width).astype(np.int32).reshape(R, width)).cuda()
    key = torch.randint(-2 ** 15, 2 ** 15 - 1, (kept, rb // 2), dtype=torch.int16, device="cuda")
    val = torch.randint(-2 ** 15, 2 ** 15 - 1, (kept, rb // 2), dtype=torch.int16, device="cuda")
    kc = torch.empty((R * width * B, rb // 2), dtype=torch.int16, device="cuda")
    vc = torch.empty_like(kc)
    slots = torch.empty(kept, dtype=torch.int64, device="cuda")

    def slot_call():
        tlb.slot_mapping(table, width, width, B, cu_out, seq_lens, R, kept, slots, stream=stream)

    def write_call():
        tlb.write_kv_cache(key, rb, val, rb, rb, slots, cu_out, R, kept, kc, vc, R * width * B, stream=stream)

    # reading 512 MB evicts the 256 MB MALL and leaves no dirty lines behind
    # (a write-based flush would have them written back during the timed call)
    flush = torch.ones(1 << 27, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")

    def mean_us(fn):
        fn()
        marks = [(ev.new(), ev.new()) for _ in range(reps)]
        for a, b in marks:
            torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
            ev.record(a, stream)
            fn()
            ev.record(b, stream)
        return sum(ev.ms(a, b) for a, b in marks) / reps * 1e3

    slot_us = mean_us(slot_call)
    write_us = mean_us(write_call)
    torch.cuda.synchronize()
    nbytes = 2 * 2 * kept * rb + 8 * kept          # K and V rows read and written, slots read
    return {"kernel": "kv_write_kernel", "bound": "hbm", "rows": kept, "row_bytes": rb, "kv_block_size": B,
            "slot_mapping_us": slot_us, "write_us": write_us, "write_gbs": nbytes / (write_us * 1e-6) / 1e9,
            "peak": PEAK_HBM_GBS, "unit": "GB/s"}


def time_ffn(keep_mask, cu_d, R, T, kept, wl, stream, ev, reps=3):
    """Eq. 7 / Eq. 10 in practice: the layer's gated FFN (LLaMA-3.1-8B widths,
    seeded synthetic weights and activations) on the retained rows against
    the same FFN on the full stream."""
    import torch
    import synth
    import token_level_block_amd as tlb
    from token_level_block_amd.runner import CompactBuffers
    D = wl.hidden
    F = synth.FFN_INTERMEDIATE["llama8b"]
    wg, wd = synth.ffn_weights_torch(D, F, "cuda")
    x = synth.ffn_activations_torch(T, D, "cuda")
    xc = torch.empty_like(x)
    cb = CompactBuffers.allocate(R, T)
    cb.run(keep_mask, cu_d, [x.view(torch.int16)], [xc.view(torch.int16)], stream=stream)
    ffn = tlb.FFN(D, F)
    ws = torch.empty(ffn.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)

    def mean_ms(inp, rows):
        ffn.forward(inp, rows, wg, wd, y, ws, stream=stream)
        marks = [(ev.new(), ev.new()) for _ in range(reps)]
        for a, b in marks:
            ev.record(a, stream)
            ffn.forward(inp, rows, wg, wd, y, ws, stream=stream)
            ev.record(b, stream)
        return sum(ev.ms(a, b) for a, b in marks) / reps

    ms_full = mean_ms(x, T)
    ms_kept = mean_ms(xc, kept)
    torch.cuda.synchronize()
    ffn.close()
    flops = lambda rows: 6.0 * rows * D * F
    return {"hidden": D, "intermediate": F, "rows_full": T, "rows_kept": kept,
            "ms_full": ms_full, "ms_kept": ms_kept,
            "tflops_full": flops(T) / (ms_full * 1e-3) / 1e12, "tflops_kept": flops(kept) / (ms_kept * 1e-3) / 1e12,
            "saving_measured": 1.0 - ms_kept / ms_full, "saving_eq10": 1.0 - kept / T,
            "gemms": "ffn_gemm_kernel: bf16 MFMA 16x16x32, fp32 accumulate; SwiGLU fused into the gate/up epilogue"}


def vendor_ffn(rows, reps=3):
    """Context for the FFN GEMM: torch's bf16 F.linear (the vendor GEMM library)
    on the same products, 131072 rows of LLaMA-3.1-8B widths and the same
    seeded tensors as the ffn_eq7 record.  The gate/up product is written
    whole ([rows, 2F], no SwiGLU); the down product reads the h that the
    library's own gate/up launch leaves in its workspace.  The library's two
    launches run first on the same tensors, so a kernel trace of this mode
    holds both side by side.  Not part of the default run."""
    import torch
    import torch.nn.functional as Fn
    import synth
    import token_level_block_amd as tlb
    D = 4096
    F = synth.FFN_INTERMEDIATE["llama8b"]
    wg, wd = synth.ffn_weights_torch(D, F, "cuda")
    x = synth.ffn_activations_torch(rows, D, "cuda")
    y = torch.empty_like(x)
    ffn = tlb.FFN(D, F)
    ws = torch.empty(ffn.workspace_bytes(rows), dtype=torch.uint8, device="cuda")
    h = ws[: rows * F * 2].view(torch.bfloat16).view(rows, F)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def mean_ms(fn):
        fn()
        torch.cuda.synchronize()
        marks = [(ev(), ev()) for _ in range(reps)]
        for a, b in marks:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in marks) / reps

    ours = mean_ms(lambda: ffn.forward(x, rows, wg, wd, y, ws))
    gu = mean_ms(lambda: Fn.linear(x, wg))
    dn = mean_ms(lambda: Fn.linear(h, wd))
    ffn.close()
    fl = lambda n_out, k: 2.0 * rows * n_out * k
    return {"rows": rows, "hidden": D, "intermediate": F,
            "library_ffn_ms": ours, "library_ffn_tflops": 6.0 * rows * D * F / (ours * 1e-3) / 1e12,
            "vendor_gate_up_ms": gu, "vendor_gate_up_tflops": fl(2 * F, D) / (gu * 1e-3) / 1e12,
            "vendor_down_ms": dn, "vendor_down_tflops": fl(D, F) / (dn * 1e-3) / 1e12,
            "note": "vendor gate/up writes the [rows, 2F] product without SwiGLU; per-kernel times "
                    "come from a kernel trace of this mode"}


def ratio(a, b):
    return None if b is None else a / b


def run_sweep(args, ev, stream):
    """The step on every workload shape of the parity suite (short to long
    contexts, one to sixteen requests); prints one JSON line with a record per
    workload.  Not the benchmark line: the 128K request is the measured
    configuration."""
    import torch
    import synth
    from dataclasses import replace
    base = synth.llama_128k()
    wls = [synth.llama_4k(), synth.llama_varlen4(),
           *(synth.hybrid_64k("qwen_next", G) for G in (32, 64, 128)),
           *(synth.hybrid_64k("gemma3", G, p=0.98) for G in (32, 64, 128)),
           base,
           # the window ablation of UniPrefill Table 4 at 128K: n = 32 and 512
           *(replace(base, n=n, name=f"llama8b_128k_n{n}") for n in (32, 512)),
           synth.serving_16x128k(),
           # the second drop layer of the serving batch: a selection on the compacted stream
           synth.serving_16x128k(lengths=synth.serving_16x128k_layer1_lengths(), layer=1)]
    records = []
    for wl in wls:
        log(f"[sweep] {wl.name}: {wl.num_reqs} request(s), {sum(wl.lengths)} tokens")
        m = measure_step(wl, args.steps, args.warmup, ev, stream)
        T = m["T"]
        flops = sum(2.0 * min(wl.n, L) * wl.hq * wl.d * L for L in wl.lengths)
        rec = {"workload": wl.name, "requests": m["R"], "tokens": T, "kept": m["kept"],
               "num_heads_q": wl.hq, "num_heads_kv": wl.hkv, "head_dim": wl.d, "hidden": wl.hidden,
               "G": wl.G, "n": wl.n, "p": wl.p, "ms_per_step": m["ms_per_step"],
               "launch": "hip_graph" if m["ms_graph"] is not None else "eager",
               "tokens_per_s": T / (m["ms_per_step"] * 1e-3),
               "breakdown_ms": {"select": m["select_ms"], "score_kernel": m["score_ms"],
                                "compact": m["compact_ms"], "metadata": m["meta_ms"],
                                "scatter_back": m["scatter_ms"]},
               "score_tflops": flops / (m["score_ms"] * 1e-3) / 1e12}
        log(f"[sweep] {wl.name}: {rec['ms_per_step']:.3f} ms/step ({rec['launch']}), "
            f"{rec['tokens_per_s'] / 1e6:.1f} M tokens/s, score {m['score_ms'] * 1e3:.1f} us "
            f"({rec['score_tflops']:.0f} TFLOP/s), kept {m['kept']}/{T}")
        records.append(rec)
        del m
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": records}), flush=True)


def select_compact_hbm(wl, m):
    """The select + compact HBM figure of one measured step: algorithmic bytes
    (kept hidden rows and positions read and written, index map, token mask,
    block scores and flags) over the time of the kernels that move them (select
    and compact without the score GEMM, whose time is the MFMA roofline's)."""
    kept, T, row_bytes = m["kept"], m["T"], wl.hidden * 2
    nbytes = 2 * kept * row_bytes + 2 * 4 * kept + 4 * kept + T + 5 * m["nblocks"]
    ms = m["select_ms"] - m["score_ms"] + m["compact_ms"]
    return nbytes, ms, nbytes / (ms * 1e-3) / 1e9


def config_record(label, wl, m, note=None):
    """One record of the default line's `configs` array."""
    T = m["T"]
    flops = sum(2.0 * min(wl.n, L) * wl.hq * wl.d * L for L in wl.lengths)
    score_tflops = flops / (m["score_ms"] * 1e-3) / 1e12
    nbytes, sc_ms, sc_gbs = select_compact_hbm(wl, m)
    rec = {"config": label, "workload": wl.name, "requests": m["R"], "tokens": T,
           "num_heads_q": wl.hq, "num_heads_kv": wl.hkv, "head_dim": wl.d, "hidden": wl.hidden,
           "G": wl.G, "A": wl.A, "n": wl.n, "p": wl.p,
           "ms_per_step": m["ms_per_step"], "launch": "hip_graph" if m["ms_graph"] is not None else "eager",
           "tokens_per_s": T / (m["ms_per_step"] * 1e-3),
           "ms_per_step_mall_flushed": m["ms_flushed"],
           "tokens_per_s_mall_flushed": T / (m["ms_flushed"] * 1e-3),
           "breakdown_ms": {"select": m["select_ms"], "score_kernel": m["score_ms"], "compact": m["compact_ms"],
                            "metadata": m["meta_ms"], "scatter_back": m["scatter_ms"]},
           "score_tflops": score_tflops, "score_frac": score_tflops / PEAK_BF16_TFLOPS,
           "select_compact_gbs": sc_gbs, "select_compact_frac": sc_gbs / PEAK_HBM_GBS,
           "select_compact_bytes": nbytes,
           "keep_ratio": m["kept"] / T,
           "keep_ratio_per_request": [round(k / L, 4) if L else None for k, L in zip(m["kept_per_req"], wl.lengths)]}
    if note:
        rec["note"] = note
    return rec


def run_configs(steps, warmup, ev, stream):
    """Every workload of the benchmark's configuration list except the
    headline's 128K request: the 4K request, the 4-request varlen batch, the
    Qwen3-Next- and Gemma-3-shaped 64K layers at G = 32 / 64 / 128 (and Gemma
    at p = 0.98, the paper's Gemma setting), and both drop layers of the
    16 x 128K serving batch."""
    import torch
    import synth
    items = [("0", synth.llama_4k(), None), ("1", synth.llama_varlen4(), None)]
    items += [(f"3a_G{G}", synth.hybrid_64k("qwen_next", G), None) for G in (32, 64, 128)]
    items += [(f"3b_G{G}", synth.hybrid_64k("gemma3", G), None) for G in (32, 64, 128)]
    items += [("3b_G64_p0.98", synth.hybrid_64k("gemma3", 64, p=0.98), None)]
    items += [("4_layer0", synth.serving_16x128k(layer=0), None),
              ("4_layer1", synth.serving_16x128k(lengths=synth.serving_16x128k_layer1_lengths(), layer=1),
               "second selection on a compacted stream: the lengths are the tokens of the first layer's "
               "planted hot blocks plus its sink and window blocks (the GPU's own layer-0 kept counts "
               "drive it in the parity test)")]
    out = []
    for label, wl, note in items:
        t0 = time.perf_counter()
        m = measure_step(wl, steps, warmup, ev, stream)
        rec = config_record(label, wl, m, note)
        rec["setup_and_timing_s"] = round(time.perf_counter() - t0, 1)
        log(f"[configs] {label} {wl.name}: {rec['ms_per_step']:.3f} ms/step ({rec['ms_per_step_mall_flushed']:.3f} "
            f"flushed), score {rec['score_tflops']:.0f} TFLOP/s ({rec['score_frac']:.3f}), select+compact "
            f"{rec['select_compact_gbs']:.0f} GB/s ({rec['select_compact_frac']:.3f}), keep {rec['keep_ratio']:.3f}")
        out.append(rec)
        del m
        torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name (first /proc/cpuinfo entry), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    """Threads NumPy's BLAS may use: the OpenBLAS / OpenMP setting, else the core count."""
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit():
            return int(v)
    return len(os.sched_getaffinity(0))


def threads_used():
    n = len(os.sched_getaffinity(0))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit():
            n = min(n, int(v))
    return n


def measure_step(wl, steps, warmup, ev, stream, pipelined=False):
    """Set up one workload (seeded inputs resident in HBM) and time the step:
    eager, eager with per-phase events (breakdown), and replayed from a HIP
    graph after three bit-exact checks against the eager step.  With
    `pipelined`, also two independent batches in flight on two streams (see
    measure_two_in_flight)."""
    import numpy as np
    import torch
    import synth
    import token_level_block_amd as tlb
    from token_level_block_amd.runner import CompactBuffers, MetadataBuffers, SelectBuffers, run_scatter_back

    class _A:
        pass
    args = _A()
    args.steps, args.warmup = steps, warmup
    log(f"[bench] generating {wl.name}: lengths={wl.lengths} hq={wl.hq} hkv={wl.hkv} d={wl.d} D={wl.hidden}")
    cu, q, k = synth.make_qk(wl)
    T = int(cu[-1])
    R = wl.num_reqs
    nwords = wl.hidden // 2
    cu_d = torch.from_numpy(cu).cuda()
    qd = torch.zeros((T, wl.hq, wl.d), dtype=torch.int16, device="cuda")
    for r in range(R):
        s, N = int(cu[r]), int(cu[r + 1] - cu[r])
        ne = min(wl.n, N)
        qd[s + N - ne: s + N] = torch.from_numpy(q[s + N - ne: s + N].view(np.int16)).cuda()
    kd = torch.from_numpy(k.view(np.int16)).cuda()
    hidden = synth.hidden_words_torch(0, T, nwords, "cuda")
    out = torch.empty_like(hidden)
    full = hidden.clone()
    # token positions (RoPE) move with the hidden rows: position within the request
    owner = torch.repeat_interleave(torch.arange(R, device="cuda"), cu_d[1:].long() - cu_d[:-1].long())
    pos = (torch.arange(T, device="cuda") - cu_d[:-1].long()[owner]).to(torch.int32)
    pos_out = torch.empty_like(pos)

    prm = tlb.make_params(wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    sel = SelectBuffers.allocate(prm, R, T)
    cb = CompactBuffers.allocate(R, T)
    mb = MetadataBuffers.allocate(np.diff(cu), num_layers=32, max_drops=4)

    def step(s, marks=None):
        if marks is not None:
            ev.record(marks["t0"], s)
        sel.run(qd, kd, cu_d, stream=s, score_events=None if marks is None else marks["score"])
        if marks is not None:
            ev.record(marks["t1"], s)
        cb.run(sel.keep_mask, cu_d, [hidden, pos], [out, pos_out], stream=s)
        if marks is not None:
            ev.record(marks["t2"], s)
        mb.run(0, cu_d, cb.cu_out, stream=s)
        if marks is not None:
            ev.record(marks["t3"], s)
        run_scatter_back(out, cb.index_out, cb.cu_out, R, T, full, stream=s)
        if marks is not None:
            ev.record(marks["t4"], s)

    def timed(run_one):
        start, stop = ev.new(), ev.new()
        torch.cuda.synchronize()
        ev.record(start, stream)
        for _ in range(args.steps):
            run_one()
        ev.record(stop, stream)
        torch.cuda.synchronize()
        return ev.ms(start, stop) / args.steps

    for _ in range(args.warmup):
        step(stream)
    # K plain steps (launched one call at a time) ...
    ms_eager = timed(lambda: step(stream))
    # the live part of every output (entries past the kept rows are never written)
    kept_now = int(cb.cu_out[R].item())

    def live():
        return (sel.keep_mask[:T], sel.kept[:R], cb.cu_out, cb.index_out[:kept_now], out[:kept_now],
                pos_out[:kept_now], full)
    ref_out = [t.clone() for t in live()]
    # ... K more with events between the phases, for the per-kernel breakdown
    marks = [dict(score=(ev.new(), ev.new()), t0=ev.new(), t1=ev.new(), t2=ev.new(), t3=ev.new(), t4=ev.new())
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(stream, marks[i])
    torch.cuda.synchronize()

    # two batches in flight on two streams; before any graph capture, since in
    # a process that has captured and replayed a HIP graph the two streams were
    # measured to run one after the other (0.46 against 0.36 ms per batch)
    two = None
    if pipelined:
        two = measure_two_in_flight(args.steps, ev, stream, ref_out, kept_now, R, T, prm, cu_d, qd, kd, hidden, pos,
                                    mb_lengths=np.diff(cu), first=(sel, cb, mb, out, pos_out, full))

    # ... and the same step captured once in a HIP graph and replayed K times
    # (every call only enqueues kernels, so the whole step is capturable); each
    # of three checked replays must reproduce the eager step's outputs bit for bit
    ms_graph, graph_note = None, None
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for _ in range(3):
            for t in (sel.keep_mask, out, pos_out):
                t.zero_()
            step(stream)                 # eager work between replays
            for t in (sel.keep_mask, out, pos_out):
                t.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(live(), ref_out)):
                raise RuntimeError("a graph replay differs from the eager step")
        ms_graph = timed(graph.replay)
    except Exception as e:       # report the eager figure only
        graph_note = f"graph replay not used: {e}"
        log(f"[bench] {graph_note}")
    ms_per_step = ms_graph if ms_graph is not None else ms_eager

    # the same step with the 256 MB MALL flushed before each one: a 512 MB
    # read (no dirty lines left to write back inside the timed step), then the
    # step between two events; the median over K steps
    flush = torch.ones(1 << 27, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    run_one = graph.replay if ms_graph is not None else (lambda: step(stream))
    fmarks = [(ev.new(), ev.new()) for _ in range(args.steps)]
    for a, b in fmarks:
        torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
        ev.record(a, stream)
        run_one()
        ev.record(b, stream)
    torch.cuda.synchronize()
    flushed = sorted(ev.ms(a, b) for a, b in fmarks)
    ms_flushed = flushed[len(flushed) // 2]
    del flush, sink

    def mean(a, b):
        return sum(ev.ms(m[a], m[b]) for m in marks) / len(marks)

    score_ms = sum(ev.ms(*m["score"]) for m in marks) / len(marks)
    select_ms = mean("t0", "t1")
    compact_ms = mean("t1", "t2")
    meta_ms = mean("t2", "t3")
    scatter_ms = mean("t3", "t4")

    kept = int(sel.kept[:R].sum().item())
    if two is not None:
        two["ms_one_stream"] = ms_per_step
        two["speedup"] = ms_per_step / two["ms_per_batch"]
    kept_per_req = sel.kept[:R].cpu().tolist()
    nblocks = int(sel.block_offsets[R].item())
    return dict(wl=wl, T=T, R=R, kept=kept, cu=cu, q=q, k=k, cu_d=cu_d, sel=sel, cb=cb, nwords=nwords,
                kept_per_req=kept_per_req, nblocks=nblocks, ms_flushed=ms_flushed,
                ms_eager=ms_eager, ms_graph=ms_graph, graph_note=graph_note, ms_per_step=ms_per_step,
                score_ms=score_ms, select_ms=select_ms, compact_ms=compact_ms, meta_ms=meta_ms,
                scatter_ms=scatter_ms, two=two, release=lambda: None)


def measure_two_in_flight(steps, ev, stream, ref_out, kept_now, R, T, prm, cu_d, qd, kd, hidden, pos,
                          mb_lengths, first):
    """Throughput with two independent batches of the same workload in flight,
    each with its own buffers and stream (default priority).  The score GEMM is
    bound by the matrix core and VALU and reads 0.27 GB, the row copies by HBM
    (1.7 GB), so each batch's selection waits for the other's: the score
    kernels alternate and each one runs beside the other batch's copies.
    Eager launches (the GPU stays busy well past the launch cost).  Both
    batches' outputs must equal the single-stream step's bit for bit."""
    import torch
    from token_level_block_amd.runner import CompactBuffers, MetadataBuffers, SelectBuffers, run_scatter_back

    sel2 = SelectBuffers.allocate(prm, R, T)
    cb2 = CompactBuffers.allocate(R, T)
    mb2 = MetadataBuffers.allocate(mb_lengths, num_layers=32, max_drops=4)
    out2, pos_out2 = torch.empty_like(first[3]), torch.empty_like(first[4])
    full2 = hidden.clone()
    sets = [first, (sel2, cb2, mb2, out2, pos_out2, full2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    done = [torch.cuda.Event(), torch.cuda.Event()]   # each batch's selection finished

    def rounds(n):
        cur = torch.cuda.current_stream()
        for st in streams:
            st.wait_stream(cur)
        for i in range(n):
            for b in (0, 1):
                sel, cb, mb, out, pos_out, full = sets[b]
                st = streams[b]
                if i > 0 or b == 1:
                    st.wait_event(done[1 - b])   # the other batch's selection
                h = st.cuda_stream
                sel.run(qd, kd, cu_d, stream=h)
                done[b].record(st)
                cb.run(sel.keep_mask, cu_d, [hidden, pos], [out, pos_out], stream=h)
                mb.run(0, cu_d, cb.cu_out, stream=h)
                run_scatter_back(out, cb.index_out, cb.cu_out, R, T, full, stream=h)
        for st in streams:
            cur.wait_stream(st)

    # new streams run slowly for their first few milliseconds of work (measured:
    # the first 20 rounds at 0.57-0.62 ms per batch, later ones at 0.36-0.39)
    rounds(max(steps, 20))
    torch.cuda.synchronize()
    start, stop = ev.new(), ev.new()
    ev.record(start, stream)
    rounds(steps)
    ev.record(stop, stream)
    ms = ev.ms(start, stop) / (2 * steps)
    torch.cuda.synchronize()
    same = True
    for sel, cb, mb, out, pos_out, full in sets:
        got = (sel.keep_mask[:T], sel.kept[:R], cb.cu_out, cb.index_out[:kept_now], out[:kept_now],
               pos_out[:kept_now], full)
        same = same and all(torch.equal(a, b) for a, b in zip(got, ref_out))
    del sel2, cb2, mb2, out2, pos_out2, full2
    torch.cuda.empty_cache()
    if not same:
        raise RuntimeError("a batch run beside another differs from the single-stream step")
    return {"batches_in_flight": 2, "streams": 2, "ms_per_batch": ms, "tokens_per_s": T / (ms * 1e-3),
            "outputs_bit_exact": True, "launch": "eager",
            "schedule": "each batch's selection waits for the other's, so each score GEMM runs beside "
                        "the other batch's row copies"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step only: skip the next-row extras (Eq. 16 slots and KV write, the FFN) "
                         "and the measured peaks (for short profiled runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records (configs 0, 1, 3, 4) of the default line")
    ap.add_argument("--sweep", action="store_true",
                    help="time the step on every workload shape (4K to 16 x 128K) instead of the benchmark line")
    ap.add_argument("--two-in-flight", action="store_true",
                    help="also time two independent batches in flight on two streams (two_batches_in_flight); "
                         "off by default so that a kernel trace of the default run holds only serial launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM byte counters)")
    ap.add_argument("--vendor-ffn", action="store_true",
                    help="only time the FFN on 131072 rows beside torch's bf16 F.linear on the same products "
                         "(context for the FFN GEMM; prints one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU hot path only; --gpus {args.gpus} is not supported "
              "(nothing in this path spans GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import token_level_block_amd as tlb
    from token_level_block_amd.runner import CompactBuffers, MetadataBuffers, SelectBuffers, run_scatter_back

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {src.numel() * 4} bytes three times")
        return

    if args.vendor_ffn:
        print(json.dumps(vendor_ffn(131072)), flush=True)
        return

    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    if args.sweep:
        run_sweep(args, ev, stream)
        return
    wl = synth.llama_128k()
    m = measure_step(wl, args.steps, args.warmup, ev, stream, pipelined=args.two_in_flight)
    T, R, kept, cu, q, k, cu_d, sel, cb, nwords = (m[x] for x in ("T", "R", "kept", "cu", "q", "k", "cu_d", "sel",
                                                                    "cb", "nwords"))
    ms_eager, ms_graph, graph_note, ms_per_step = m["ms_eager"], m["ms_graph"], m["graph_note"], m["ms_per_step"]
    score_ms, select_ms, compact_ms = m["score_ms"], m["select_ms"], m["compact_ms"]
    meta_ms, scatter_ms = m["meta_ms"], m["scatter_ms"]
    keep_ratio = kept / T
    tokens_per_s = T / (ms_per_step * 1e-3)
    sel_compact_tps = T / ((select_ms + compact_ms + meta_ms) * 1e-3)

    flops = 2.0 * wl.n * wl.hq * wl.d * T
    score_tflops = flops / (score_ms * 1e-3) / 1e12
    row_bytes = wl.hidden * 2
    compact_bytes = 2 * kept * row_bytes + 2 * 4 * kept + 4 * kept + T   # hidden and position rows, index map, mask
    compact_gbs = compact_bytes / (compact_ms * 1e-3) / 1e9
    scatter_bytes = 2 * kept * row_bytes + 4 * kept
    scatter_gbs = scatter_bytes / (scatter_ms * 1e-3) / 1e9
    log(f"[bench] eager {ms_eager:.3f} ms/step, graph replay "
        f"{'-' if ms_graph is None else f'{ms_graph:.3f}'} ms/step")
    log(f"[bench] {ms_per_step:.3f} ms/step  select {select_ms:.3f} (score {score_ms:.3f}) compact "
        f"{compact_ms:.3f} metadata {meta_ms:.3f} scatter {scatter_ms:.3f}  kept {kept}/{T}")
    # select + compact as HBM work: kept rows read and written, index map, token
    # mask, block scores and flags, over the time of the kernels that move them
    # (select and compact without the score GEMM, whose K reads and time are
    # counted under the MFMA roofline); and, for the whole select + compact, the
    # same bytes plus the score GEMM's K and window-query reads over the whole time
    sc_bytes, sc_ms, sc_gbs = select_compact_hbm(wl, m)
    qk_bytes = 2 * T * wl.hkv * wl.d + 2 * R * min(wl.n, T) * wl.hq * wl.d
    all_gbs = (sc_bytes + qk_bytes) / ((select_ms + compact_ms) * 1e-3) / 1e9
    torch.cuda.empty_cache()
    kv = ffn = None
    mfma_peak = mfma16_peak = copy_peak = None
    if not args.step_only:
        # the timed steps re-applied the same drop, so take the patched lengths of a
        # single drop on a fresh prefill: the retained counts
        retained = (cb.cu_out[1:R + 1] - cb.cu_out[:R]).to(torch.int32).contiguous()
        kv = time_kv_cache(cb.cu_out, retained, R, kept, wl, stream, ev, args.steps)
        log(f"[bench] Eq. 16 slot mapping {kv['slot_mapping_us']:.1f} us, KV-cache write {kv['write_us']:.1f} us "
            f"({kv['write_gbs']:.0f} GB/s) for {kept} retained rows")
        ffn = time_ffn(sel.keep_mask, cu_d, R, T, kept, wl, stream, ev)
        log(f"[bench] FFN on {kept} retained rows {ffn['ms_kept']:.2f} ms vs {T} rows {ffn['ms_full']:.2f} ms: "
            f"saving {ffn['saving_measured']:.3f} (Eq. 10: {ffn['saving_eq10']:.3f})")
        mfma_peak, mfma16_peak, copy_peak = measure_peaks(stream, ev)
        kv["frac"] = kv["write_gbs"] / PEAK_HBM_GBS
        kv["frac_measured"] = kv["write_gbs"] / copy_peak
        # the FFN GEMMs against the dense bf16 peak and the measured rate of
        # their own instruction (16x16x32)
        ffn.update(peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", bound="mfma",
                   frac_full=ffn["tflops_full"] / PEAK_BF16_TFLOPS, frac_kept=ffn["tflops_kept"] / PEAK_BF16_TFLOPS,
                   measured_peak=mfma16_peak,
                   frac_measured_full=ffn["tflops_full"] / mfma16_peak,
                   frac_measured_kept=ffn["tflops_kept"] / mfma16_peak)
        log(f"[bench] measured peaks: bf16 MFMA {mfma_peak:.0f} TFLOP/s (32x32x16) and {mfma16_peak:.0f} TFLOP/s "
            f"(16x16x32), random operands; copy {copy_peak:.0f} GB/s")
    configs = None
    if not (args.step_only or args.no_configs):
        configs = run_configs(args.steps, args.warmup, ev, stream)
    ev.close()

    cpu = None
    if not args.no_cpu_baseline:
        # whole steps of the same workload until at least 10 s of wall time (at
        # most 8 steps); the rate is over all of them
        log("[bench] timing the CPU oracle on full steps of the same workload")
        hidden_host = synth.hidden_words(np.arange(T), nwords)
        steps, wall = 0, 0.0
        cpu0 = time.process_time()
        while steps < 8 and (steps == 0 or wall < 10.0):
            dt, _ = cpu_oracle_step(wl, cu, q, k, hidden_host)
            steps += 1
            wall += dt
            log(f"[bench] oracle step {steps}: {dt:.2f} s")
        cpu_s = time.process_time() - cpu0
        cpu = {"value": steps * T / wall, "unit": "tokens/s", "cores": threads_used(), "kind": "oracle",
               "sample": f"{steps} full steps (select, compact, metadata, scatter-back) of the {T}-token "
                         f"request, {wall:.1f} s wall, {cpu_s:.0f} s of CPU time",
               "cpu_model": cpu_model(), "blas_threads": blas_threads()}
        log(f"[bench] oracle: {steps} steps in {wall:.2f} s -> {steps * T / wall:.0f} tokens/s")

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": R, "tokens": T, "num_heads_q": wl.hq,
                   "num_heads_kv": wl.hkv, "head_dim": wl.d, "hidden": wl.hidden, "G": wl.G, "A": wl.A,
                   "n": wl.n, "p": wl.p, "keep_ratio": round(keep_ratio, 4)},
        "roofline": {"bound": "mfma", "kernel": "score_kernel<128>", "achieved": score_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": score_tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__))),
                     "measured_peak": mfma_peak, "frac_measured": ratio(score_tflops, mfma_peak)},
        "roofline_compact": {"bound": "hbm", "kernel": "up_compact", "achieved": compact_gbs,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": compact_gbs / PEAK_HBM_GBS,
                             "measured_peak": copy_peak, "frac_measured": ratio(compact_gbs, copy_peak)},
        "roofline_scatter": {"bound": "hbm", "kernel": "up_scatter_back", "achieved": scatter_gbs,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": scatter_gbs / PEAK_HBM_GBS,
                             "measured_peak": copy_peak, "frac_measured": ratio(scatter_gbs, copy_peak)},
        "hbm_select_compact": {"achieved": sc_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": sc_gbs / PEAK_HBM_GBS, "measured_peak": copy_peak,
                               "frac_measured": ratio(sc_gbs, copy_peak), "bytes": sc_bytes, "ms": sc_ms,
                               "over": "select + compact kernels except the score GEMM"},
        "hbm_select_compact_with_score": {"achieved": all_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                          "frac": all_gbs / PEAK_HBM_GBS, "bytes": sc_bytes + qk_bytes,
                                          "ms": select_ms + compact_ms,
                                          "over": "all of select + compact, K and window-query reads included"},
        "kv_cache_eq16": kv,
        "ffn_eq7": ffn,
        "measured_peaks": {"bf16_mfma_tflops": mfma_peak, "bf16_mfma16_tflops": mfma16_peak, "copy_gbs": copy_peak,
                           "how": "libuppeaks: random-operand bf16 MFMA loops at 2 waves/SIMD, "
                                  "32x32x16 (bf16_mfma_tflops) and 16x16x32 (bf16_mfma16_tflops); "
                                  "1 GiB streaming copy, one 16-byte unit per thread in one pass, "
                                  "read + write bytes"},
        "ms_per_step_mall_flushed": m["ms_flushed"],
        "configs": configs,
        "launch": "hip_graph" if ms_graph is not None else f"eager ({graph_note})",
        "ms_per_step_eager": ms_eager,
        "ms_per_step_graph": ms_graph,
        "breakdown_ms": {"select": select_ms, "score_kernel": score_ms, "compact": compact_ms,
                         "metadata": meta_ms, "scatter_back": scatter_ms},
        "select_compact_tokens_per_s": sel_compact_tps,
        # with --two-in-flight: the same workload with two batches in flight (not `value`:
        # that is one batch at a time)
        "two_batches_in_flight": m["two"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
