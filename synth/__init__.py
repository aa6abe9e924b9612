"""Seeded synthetic workloads for the UniPrefill token-selection path.

This module is shared by the CPU oracle's tests and by the GPU tests and
benchmark.  It holds none of the method's arithmetic: no logits, no softmax,
no block scores, no selection and no compaction.  It only draws seeded random
numbers, rounds them to bf16, and writes index-encoded bit patterns for the
hidden rows that compaction moves.

Shapes follow the full-attention layers of the three model families the
UniPrefill paper (arXiv 2605.06221, Sec. 4.1) evaluates on; the paper prints
no head counts, so those come from the public model cards:

  * LLaMA-3.1-8B:   32 query heads, 8 KV heads, head_dim 128, hidden 4096
  * Qwen3-Next-like: 16 query heads, 2 KV heads, head_dim 256, hidden 2048
  * Gemma-3-12B:    16 query heads, 8 KV heads, head_dim 256, hidden 3840

The paper measures on RULER prompts of 4K-128K tokens.  RULER is not used
here: these generators stand in for the shape of such prompts (lengths,
packing, a few strongly attended token blocks among many weak ones), not for
any of its items.

Generator recipe (per request r and KV head j, each from its own stream):
  u      = a random unit vector in R^d              (the "mean query direction")
  q[t,h] = P x + gamma * u,  x ~ N(0,1)^d             for the last min(n, N_r) rows
  k[i]   = N(0,1)^d + (sqrt(d)/gamma) * lam[i] * u   for every token of the request
where P removes the component along u.  A window query's scaled logit
against key i then has mean lam[i] and a background spread of about one unit
for every window row alike.  (Without P, the query noise along u would scale
each row's alignment by 1 + (x.u)/gamma; the few rows where that factor is
near zero spread their attention evenly and, at p = 0.99, force most blocks to
be kept whatever the structure.)  lam[i] = 3 for the first 128 tokens of
a request (attention sinks, A tokens in general) and otherwise the value of
the structure block (64 tokens) that holds i.  Every draw is made in float64,
rounded to float32 and
then to bf16 with round-to-nearest-even.  Query rows outside each request's
window are never read by the method and are left zero.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
import os

import numpy as np

GAMMA = 2.0          # query alignment with u
SINK_LAMBDA = 3.0    # alignment of the first A keys of each request (sinks)
STRUCT_BLOCK = 64    # granularity of the generator's hot/cold structure

# Calibrated generator constants (see tests/golden/calibrate_generator.py,
# which bisects them against the oracle's keep ratio at p = 0.99).
POWERLAW_C = 1.4590  # keeps 40.1% of the 2048 blocks of the 128K request at p = 0.99
# hot-block alignment of each request of the varlen batch: the requests keep
# 9.4%, 34.4%, 60.2% and 90.6% of their tokens (the last: 25 hot blocks of its
# 28 non-forced ones, the 3 others dropped)
HOT_LAMBDA_VARLEN = (8.0, 6.9462, 6.2224, 8.0)

LLAMA_8B = dict(hq=32, hkv=8, d=128, hidden=4096)
QWEN_NEXT = dict(hq=16, hkv=2, d=256, hidden=2048)
GEMMA3_12B = dict(hq=16, hkv=8, d=256, hidden=3840)


@dataclass(frozen=True)
class RequestStructure:
    """How the key alignments lam[] of one request are drawn.

    kind == "hot":      `hot` random non-forced 64-token blocks get lam = hot_lambda,
                        the other blocks lam = 0.
    kind == "powerlaw": every 64-token block gets lam = c * ln(P), P ~ Pareto(1),
                        i.e. c times a unit exponential draw.
    """
    kind: str
    hot: int = 0
    hot_lambda: float = 0.0
    c: float = 0.0


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple
    hq: int
    hkv: int
    d: int
    hidden: int
    G: int = 64
    A: int = 128
    n: int = 128
    p: float = 0.99
    seed: int = 0
    structures: tuple = field(default_factory=tuple)
    struct_block: int = STRUCT_BLOCK

    @property
    def num_reqs(self) -> int:
        return len(self.lengths)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(len(self.lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.lengths, dtype=np.int64))
        return cu


def _nonforced_blocks(N: int, A: int, n: int, sb: int) -> np.ndarray:
    """Structure blocks that hold neither sink nor window tokens."""
    nb = -(-N // sb)
    g = np.arange(nb)
    lo = g * sb
    hi = np.minimum(lo + sb, N)
    ok = (lo >= A) & (hi <= N - n)
    return g[ok]


def block_lambdas(wl: Workload, r: int) -> np.ndarray:
    """Per-structure-block alignment lam for request r (float64, one per block)."""
    N = int(wl.lengths[r])
    nb = -(-N // wl.struct_block)
    st = wl.structures[r]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, r, 0xB10C])))
    lam = np.zeros(nb, dtype=np.float64)
    if st.kind == "hot":
        cand = _nonforced_blocks(N, wl.A, wl.n, wl.struct_block)
        h = min(int(st.hot), len(cand))
        if h > 0:
            pick = rng.choice(cand, size=h, replace=False)
            lam[pick] = st.hot_lambda
    elif st.kind == "powerlaw":
        lam[:] = st.c * rng.exponential(1.0, size=nb)
    elif st.kind == "none":
        pass
    else:
        raise ValueError(f"unknown structure kind {st.kind!r}")
    return lam


def token_lambdas(wl: Workload, r: int) -> np.ndarray:
    N = int(wl.lengths[r])
    lam = np.repeat(block_lambdas(wl, r), wl.struct_block)[:N].copy()
    lam[: min(wl.A, N)] = SINK_LAMBDA
    return lam


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 bits (RNE), as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + bias) >> 16).astype(np.uint16)


def _stream(wl: Workload, r: int, j: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, r, j, tag])))


def _fill_request_head(wl, r, j, s, lam, q, k):
    N = int(wl.lengths[r])
    d = wl.d
    rng = _stream(wl, r, j, 0x5EED)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    group = wl.hq // wl.hkv
    ne = min(wl.n, N)
    if ne > 0:
        for hh in range(group):
            h = j * group + hh
            x = rng.standard_normal((ne, d))
            x -= (x @ u)[:, None] * u[None, :]
            x += GAMMA * u
            q[s + N - ne: s + N, h, :] = f64_to_bf16_bits(x)
    # keys in chunks to bound the float64 temporaries
    step = 1 << 15
    for a in range(0, N, step):
        b = min(N, a + step)
        y = rng.standard_normal((b - a, d))
        y += (math.sqrt(d) / GAMMA) * lam[a:b, None] * u[None, :]
        k[s + a: s + b, j, :] = f64_to_bf16_bits(y)


def make_qk(wl: Workload, workers: int | None = None):
    """Return (cu_seqlens int32 [R+1], q uint16 [T,Hq,d], k uint16 [T,Hkv,d]).

    q and k hold bf16 bit patterns.  q is allocated with np.zeros, so the
    untouched non-window rows cost no physical memory.
    """
    cu = wl.cu_seqlens()
    T = int(cu[-1])
    q = np.zeros((T, wl.hq, wl.d), dtype=np.uint16)
    k = np.zeros((T, wl.hkv, wl.d), dtype=np.uint16)
    jobs = []
    for r in range(wl.num_reqs):
        lam = token_lambdas(wl, r)
        for j in range(wl.hkv):
            jobs.append((r, j, int(cu[r]), lam))
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers <= 1 or len(jobs) == 1:
        for r, j, s, lam in jobs:
            _fill_request_head(wl, r, j, s, lam, q, k)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda a: _fill_request_head(wl, a[0], a[1], a[2], a[3], q, k), jobs))
    return cu, q, k


def make_request_qk(wl: Workload, r: int):
    """Request r of make_qk(wl) on its own: (q uint16 [N_r, Hq, d], k uint16
    [N_r, Hkv, d]), bit-identical to rows cu[r] .. cu[r+1]-1 of make_qk's
    arrays (each request and KV head draws from its own stream)."""
    N = int(wl.lengths[r])
    q = np.zeros((N, wl.hq, wl.d), dtype=np.uint16)
    k = np.zeros((N, wl.hkv, wl.d), dtype=np.uint16)
    lam = token_lambdas(wl, r)
    for j in range(wl.hkv):
        _fill_request_head(wl, r, j, 0, lam, q, k)
    return q, k


def random_scores(rng: np.random.Generator, nb: int, kind: str = "lognormal") -> np.ndarray:
    """Non-negative fp32 block-score vectors for feeding selection directly."""
    if kind == "lognormal":
        x = np.exp(rng.standard_normal(nb) * 2.0)
    elif kind == "ties":
        x = rng.integers(0, 4, size=nb).astype(np.float64)
    elif kind == "sparse":
        x = np.where(rng.random(nb) < 0.05, rng.random(nb) * 100.0, rng.random(nb) * 1e-3)
    elif kind == "pareto":
        x = rng.pareto(1.0, size=nb)
    elif kind == "constant":
        x = np.full(nb, 0.25)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


# ---------------------------------------------------------------------------
# Index-encoded hidden rows.  Word j (4 bytes) of row i holds
#     (i * 0x9E3779B1 + j * 0x7F4A7C15 + 0x632BE5AB) mod 2**32.
# The multiplier of i is odd, so rows differ from one another in every word,
# and the j term makes a shifted or misaligned copy visible as well.
# ---------------------------------------------------------------------------
_MI = 0x9E3779B1
_MJ = 0x7F4A7C15
_C0 = 0x632BE5AB


def hidden_words(rows: np.ndarray, nwords: int) -> np.ndarray:
    """uint32 [len(rows), nwords] contents of the given hidden rows."""
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(nwords, dtype=np.uint64)[None, :]
    v = (i * np.uint64(_MI) + j * np.uint64(_MJ) + np.uint64(_C0)) & np.uint64(0xFFFFFFFF)
    return v.astype(np.uint32)


def hidden_words_torch(row0: int, nrows: int, nwords: int, device):
    """Same pattern as hidden_words for rows [row0, row0+nrows), as a torch int32 tensor."""
    import torch
    return hidden_words_torch_at(torch.arange(row0, row0 + nrows, dtype=torch.int64, device=device), nwords)


def hidden_words_torch_at(rows, nwords: int):
    """Same pattern as hidden_words for the rows listed in a torch tensor."""
    import torch
    i = rows.to(torch.int64)[:, None]
    j = torch.arange(nwords, dtype=torch.int64, device=rows.device)[None, :]
    v = (i * _MI + j * _MJ + _C0) & 0xFFFFFFFF
    v = torch.where(v >= 2 ** 31, v - 2 ** 32, v)
    return v.to(torch.int32)


# ---------------------------------------------------------------------------
# Dense bf16 tensors for the downstream FFN sublayer: element (i, j) of tensor
# `tag` (row-major, ncols columns) is a fixed function of (tag, i*ncols + j):
# the murmur3 32-bit finalizer of the counter (mod 2^32) plus tag * 0x9E3779B1,
# whose top 24 bits k give the value (k - 2^23) / 2^23 * 2^scale_log2 (uniform
# on [-2^s, 2^s), exact in float32), rounded to bf16 (round to nearest even).
# Any row range can be generated on its own, on the host or on a device, with
# the same bits.
# ---------------------------------------------------------------------------
FFN_INTERMEDIATE = {"llama8b": 14336, "gemma3": 15360}
_TAGMUL = 0x9E3779B1
_FM1, _FM2 = 0x85EBCA6B, 0xC2B2AE35
_M32 = 0xFFFFFFFF


def uniform_bf16_bits(tag: int, row0: int, nrows: int, ncols: int, scale_log2: int) -> np.ndarray:
    """uint16 [nrows, ncols]: rows row0 .. row0+nrows-1 of tensor `tag`, on
    the host (computed with torch on the CPU, the same code as on a device)."""
    import torch
    t = uniform_bf16_torch(tag, row0, nrows, ncols, scale_log2, "cpu")
    return t.view(torch.int16).numpy().view(np.uint16)


def uniform_bf16_torch(tag: int, row0: int, nrows: int, ncols: int, scale_log2: int, device,
                       chunk_rows: int = 4096):
    """Same values as uniform_bf16_bits, as a torch bfloat16 tensor on `device`."""
    import torch
    out = torch.empty((nrows, ncols), dtype=torch.bfloat16, device=device)
    col = torch.arange(ncols, dtype=torch.int64, device=device)[None, :]
    base = (tag * _TAGMUL) & _M32
    for a in range(0, nrows, chunk_rows):
        z = min(nrows, a + chunk_rows)
        rows = torch.arange(row0 + a, row0 + z, dtype=torch.int64, device=device)[:, None]
        h = (rows * ncols + col + base) & _M32
        h ^= h >> 16
        h = (h * _FM1) & _M32
        h ^= h >> 13
        h = (h * _FM2) & _M32
        h ^= h >> 16
        k = (h >> 8) - (1 << 23)
        out[a:z] = (k.to(torch.float32) * (2.0 ** (scale_log2 - 23))).to(torch.bfloat16)
    return out


def ffn_weights(D: int, F: int, seed: int = 7):
    """(w_gate_up [2F, D], w_down [D, F]) bf16 bits; entries uniform with
    scale 2^-6, so a unit-range activation row gives gate and up values of
    order 0.3 and outputs of order 0.1."""
    return (uniform_bf16_bits(2 * seed + 1, 0, 2 * F, D, -6),
            uniform_bf16_bits(2 * seed + 2, 0, D, F, -6))


def ffn_weights_torch(D: int, F: int, device, seed: int = 7):
    """ffn_weights as bfloat16 tensors on `device`."""
    return (uniform_bf16_torch(2 * seed + 1, 0, 2 * F, D, -6, device),
            uniform_bf16_torch(2 * seed + 2, 0, D, F, -6, device))


def ffn_activations(rows: int, D: int, seed: int = 7, row0: int = 0):
    """bf16 bits [rows, D], entries uniform on [-1, 1)."""
    return uniform_bf16_bits(2 * seed + 3, row0, rows, D, 0)


def ffn_activations_torch(rows: int, D: int, device, seed: int = 7, row0: int = 0):
    return uniform_bf16_torch(2 * seed + 3, row0, rows, D, 0, device)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------
def llama_4k(seed: int = 0) -> Workload:
    return Workload("llama8b_4k", (4096,), seed=seed,
                    structures=(RequestStructure("hot", hot=6, hot_lambda=2.0),), **LLAMA_8B)


def llama_varlen4(seed: int = 1, hot_lambda=None) -> Workload:
    """hot_lambda: one alignment for all four requests, or one per request."""
    lam = HOT_LAMBDA_VARLEN if hot_lambda is None else hot_lambda
    lams = tuple(lam) if isinstance(lam, (tuple, list)) else (float(lam),) * 4
    hots = (2, 8, 20, 25)
    return Workload("llama8b_varlen4", (4096, 8192, 16384, 2048), seed=seed,
                    structures=tuple(RequestStructure("hot", hot=h, hot_lambda=l) for h, l in zip(hots, lams)),
                    **LLAMA_8B)


def llama_128k(seed: int = 2, c: float | None = None, N: int = 131072) -> Workload:
    cc = POWERLAW_C if c is None else c
    return Workload("llama8b_128k", (N,), seed=seed,
                    structures=(RequestStructure("powerlaw", c=cc),), **LLAMA_8B)


def hybrid_64k(model: str, G: int, seed: int = 3, p: float = 0.99) -> Workload:
    shape = {"qwen_next": QWEN_NEXT, "gemma3": GEMMA3_12B}[model]
    return Workload(f"{model}_64k_G{G}", (65536,), G=G, p=p, seed=seed,
                    structures=(RequestStructure("powerlaw", c=POWERLAW_C),), **shape)


def serving_16x128k_keep_ratios(seed: int = 4, layer: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, 0xC0F4])))
    return rng.uniform(0.2, 0.9, size=16)


def serving_16x128k(seed: int = 4, lengths=None, layer: int = 0) -> Workload:
    """16 requests of 128K tokens; layer 1 is the second selection on the
    compacted stream, with fresh draws (seed + 1000) and fresh keep ratios."""
    if lengths is None:
        lengths = (131072,) * 16
    rho = serving_16x128k_keep_ratios(seed, layer)
    structs = []
    for r, N in enumerate(lengths):
        nbg = -(-int(N) // STRUCT_BLOCK)
        h = max(0, int(round(rho[r] * nbg)) - 4)
        structs.append(RequestStructure("hot", hot=h, hot_lambda=8.0))
    return Workload(f"llama8b_16x128k_layer{layer}", tuple(int(x) for x in lengths),
                    seed=seed + 1000 * layer, structures=tuple(structs), **LLAMA_8B)


def serving_16x128k_layer1_lengths(seed: int = 4) -> tuple:
    """Lengths of the second selection's stream: the tokens of the hot blocks the
    first layer's generator planted plus the two sink and two window blocks."""
    wl0 = serving_16x128k(seed)
    out = []
    for N, st in zip(wl0.lengths, wl0.structures):
        out.append(int(min(N, (st.hot + 4) * STRUCT_BLOCK)))
    return tuple(out)


def tiny(lengths, hq=4, hkv=2, d=64, hidden=64, G=8, A=8, n=8, p=0.9, seed=0,
         kind="hot", hot=2, hot_lambda=4.0, c=1.0) -> Workload:
    """Small workloads for tests: several tiles, ragged tails, short requests."""
    st = RequestStructure(kind, hot=hot, hot_lambda=hot_lambda, c=c)
    return Workload(f"tiny_{seed}", tuple(int(x) for x in lengths), hq=hq, hkv=hkv, d=d,
                    hidden=hidden, G=G, A=A, n=n, p=p, seed=seed,
                    structures=tuple(st for _ in lengths), struct_block=G)


def with_structures(wl: Workload, structures) -> Workload:
    return replace(wl, structures=tuple(structures))
