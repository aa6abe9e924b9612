"""Plain NumPy float64 restatement of UniPrefill's token-selection path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product.  No blocking, fusion or
reordering beyond what each definition states; library routines (matmul,
argsort, cumsum) serve as single steps.

Source: "UniPrefill: Universal Long-Context Prefill Acceleration via
Block-wise Dynamic Sparsification" (arXiv 2605.06221), cited below as
"UniPrefill" with its section and equation numbers.

Readings of points the paper leaves open (each is also listed in the design
notes of the repository):
  * Query-head aggregation is a SUM over heads (Sec. 3.5, the block-reduce
    kernel contracts over heads; Eq. 15 adds per-rank partials).
  * GQA: query head h reads KV head floor(h * Hkv / Hq).
  * Softmax scale 1/sqrt(d) (Eq. 2) unless the caller overrides it.
  * Window row t (absolute position N - n_eff + t) sees keys <= its own
    position (causal masking, Sec. 3.5 "Kernel design").
  * n_eff = min(n, N); the 1/G of Eq. 4 is kept for a partial last block.
  * Top-p ties: the packed key of Eq. 14 ranks equal scores by the larger
    block index first.
  * The cumulative sum of Eq. 5 is taken in exact integers: scores are
    scaled by a power of two and floored (see top_p_select).
  * Forced sink/window tokens are OR-ed in after top-p; they do not change
    the top-p budget.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Importance estimation: UniPrefill Sec. 3.2, Eq. 2-4; Sec. 3.5 Eq. 13
# ---------------------------------------------------------------------------
def token_importance(q_bits, k_bits, start: int, N: int, hq: int, hkv: int, d: int,
                     n: int, scale: float | None = None) -> np.ndarray:
    """o_i = sum over query heads h and window rows j of A[h, j, i]  (float64 [N]).

    A[h, j, :] is the full-sequence softmax of row j's scaled logits
    (Eq. 2), for the last n_eff = min(n, N) rows of the request (Eq. 3),
    with causal masking of keys after the row's own position.
    """
    if N <= 0:
        return np.zeros(0, dtype=np.float64)
    ne = min(n, N)
    sc = 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)
    keys = np.arange(N)
    rowpos = (N - ne) + np.arange(ne)               # position of each window row
    future = keys[None, :] > rowpos[:, None]        # causal mask [ne, N]
    o = np.zeros(N, dtype=np.float64)
    for h in range(hq):
        kv = (h * hkv) // hq
        Qw = bf16_bits_to_f64(q_bits[start + N - ne: start + N, h, :])   # [ne, d]
        Kr = bf16_bits_to_f64(k_bits[start: start + N, kv, :])           # [N, d]
        Z = (Qw @ Kr.T) * sc                                             # [ne, N]
        Z[future] = -np.inf
        Z -= Z.max(axis=1, keepdims=True)
        E = np.exp(Z)
        A = E / E.sum(axis=1, keepdims=True)        # textbook row softmax
        o += A.sum(axis=0)
    return o


def request_block_scores(q_bits, k_bits, start: int, N: int, hq: int, hkv: int, d: int,
                         G: int, n: int, scale: float | None = None):
    """Block scores b_g of Eq. 4 for one request (float64 [ceil(N/G)]), and o.

    Blocks are anchored at the request's first token; the last one may be
    partial and is still divided by G.
    """
    o = token_importance(q_bits, k_bits, start, N, hq, hkv, d, n, scale)
    if N <= 0:
        return np.zeros(0, dtype=np.float64), o
    ne = min(n, N)
    nb = -(-N // G)
    b = np.zeros(nb, dtype=np.float64)
    for g in range(nb):
        b[g] = o[g * G: min((g + 1) * G, N)].sum() / (G * ne)
    return b, o


def block_scores(q_bits, k_bits, cu_seqlens, hq: int, hkv: int, d: int, G: int, n: int,
                 scale: float | None = None):
    """Eq. 4 over a cu_seqlens-packed batch.

    Returns (b float64 [sum nb_r], block_offsets int64 [R+1]).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    R = len(cu) - 1
    parts, offs = [], [0]
    for r in range(R):
        N = int(cu[r + 1] - cu[r])
        b, _ = request_block_scores(q_bits, k_bits, int(cu[r]), N, hq, hkv, d, G, n, scale)
        parts.append(b)
        offs.append(offs[-1] + len(b))
    b = np.concatenate(parts) if parts else np.zeros(0)
    return b, np.asarray(offs, dtype=np.int64)


# ---------------------------------------------------------------------------
# Top-p selection: UniPrefill Sec. 3.3 Eq. 5; Sec. 3.5 Eq. 14
# ---------------------------------------------------------------------------
def phi(b32: np.ndarray) -> np.ndarray:
    """Monotone map of Eq. 14 from float32 to uint32, decided by the sign bit."""
    bits = np.ascontiguousarray(b32, dtype=np.float32).view(np.uint32)
    negative = (bits >> np.uint32(31)) == 1
    return np.where(negative, bits ^ np.uint32(0xFFFFFFFF),
                    bits ^ np.uint32(0x80000000)).astype(np.uint32)


def pack_keys(b32: np.ndarray) -> np.ndarray:
    """packed_g = (phi(b_g) << 32) | g, as uint64 (Eq. 14)."""
    g = np.arange(len(b32), dtype=np.uint64)
    return (phi(b32).astype(np.uint64) << np.uint64(32)) | g


def top_p_select(b32: np.ndarray, p: float) -> np.ndarray:
    """Keep flags (bool [nb]) of the minimal top-p block set of Eq. 5.

    1. pi = blocks in descending order of their packed key (Eq. 14).
    2. The cumulative sum is taken on exact integers:
         e     = binary exponent of the largest positive score (max = m 2^e, m in [0.5,1)),
         shift = 52 - ceil(log2 nb) - e,
         q_g   = floor(b_g 2^shift)  for b_g > 0 and finite, else 0,
       so every q_g and their total T fit in 52 bits.
    3. thr = p * T as one float64 multiply; k* is the first k (k >= 1) with
       q_pi(1) + ... + q_pi(k) >= thr; the kept set is pi(1..k*).
    """
    b32 = np.ascontiguousarray(b32, dtype=np.float32)
    nb = len(b32)
    keep = np.zeros(nb, dtype=bool)
    if nb == 0:
        return keep
    order = np.argsort(pack_keys(b32), kind="stable")[::-1]
    bf = b32.astype(np.float64)
    usable = np.isfinite(bf) & (bf > 0)
    e = int(np.frexp(bf[usable].max())[1]) if usable.any() else 0
    shift = 52 - (nb - 1).bit_length() - e
    qv = np.zeros(nb, dtype=np.int64)
    qv[usable] = np.floor(np.ldexp(bf[usable], shift)).astype(np.int64)
    total = int(qv.sum())
    thr = float(p) * float(total)
    csum = np.cumsum(qv[order])
    hit = np.nonzero(csum.astype(np.float64) >= thr)[0]
    kstar = int(hit[0]) + 1 if len(hit) else nb
    keep[order[:kstar]] = True
    return keep


def expand_mask(keep_block: np.ndarray, N: int, G: int, A: int, n: int) -> np.ndarray:
    """Token mask M (uint8 [N]): its block's keep flag, or a sink (i < A), or
    in the query window (i >= N - n).  UniPrefill Sec. 3.3 and Sec. 3.5."""
    i = np.arange(N)
    m = keep_block[i // G] | (i < A) | (i >= N - n)
    return m.astype(np.uint8)


def select(q_bits, k_bits, cu_seqlens, hq, hkv, d, G, A, n, p, scale=None, scores_in=None):
    """The whole selection: Eq. 4 scores, fp32 rounding, Eq. 5 top-p, expansion.

    With scores_in (float32 [sum nb_r]) the scoring step is skipped.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    R = len(cu) - 1
    if scores_in is None:
        b64, offs = block_scores(q_bits, k_bits, cu, hq, hkv, d, G, n, scale)
        b32 = b64.astype(np.float32)            # round to nearest even
    else:
        offs = [0]
        for r in range(R):
            offs.append(offs[-1] + (-(-int(cu[r + 1] - cu[r]) // G)))
        offs = np.asarray(offs, dtype=np.int64)
        b64 = None
        b32 = np.ascontiguousarray(scores_in, dtype=np.float32)
    T = int(cu[-1])
    mask = np.zeros(T, dtype=np.uint8)
    keep_block = np.zeros(len(b32), dtype=np.uint8)
    kept = np.zeros(R, dtype=np.int32)
    for r in range(R):
        N = int(cu[r + 1] - cu[r])
        kb = top_p_select(b32[offs[r]: offs[r + 1]], p)
        keep_block[offs[r]: offs[r + 1]] = kb
        m = expand_mask(kb, N, G, A, n)
        mask[cu[r]: cu[r + 1]] = m
        kept[r] = int(m.sum())
    return dict(b64=b64, b32=b32, block_offsets=offs, keep_block=keep_block,
                mask=mask, kept=kept)


# ---------------------------------------------------------------------------
# Compaction and carry-forward: UniPrefill Sec. 3.4 Eq. 7-8; Sec. 3.5
# ---------------------------------------------------------------------------
def compact(mask, cu_seqlens, buffers=(), index_in=None):
    """Keep the rows whose mask is set, in their original order.

    Returns (outs, index_out, cu_out): the gathered rows of every buffer,
    index_out[k] = index_in[i_k] (or i_k itself) for the k-th kept token i_k,
    and cu_out[r] = number of kept tokens before request r's first token.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    keep = np.asarray(mask[:T]).astype(bool)
    idx = np.nonzero(keep)[0]
    src_index = np.arange(T) if index_in is None else np.asarray(index_in)[:T]
    index_out = src_index[idx].astype(np.int32)
    before = np.concatenate([[0], np.cumsum(keep)])
    cu_out = before[cu].astype(np.int32)
    outs = [np.asarray(buf)[:T][idx] for buf in buffers]
    return outs, index_out, cu_out


def scatter_back(full, compacted, index_map, count: int):
    """Eq. 8: rows listed in index_map take the processed state; every other
    row of the full-length buffer keeps its earlier value."""
    out = np.array(full, copy=True)
    out[np.asarray(index_map[:count], dtype=np.int64)] = np.asarray(compacted)[:count]
    return out


# ---------------------------------------------------------------------------
# Metadata and drop history: UniPrefill Sec. 3.5 ("vLLM scheduler
# integration"), Eq. 17
# ---------------------------------------------------------------------------
@dataclass
class MetadataState:
    seq_lens: np.ndarray
    history: list = field(default_factory=list)   # per request: [(layer, retained_len), ...]

    @staticmethod
    def fresh(seq_lens):
        s = np.asarray(seq_lens, dtype=np.int64).copy()
        return MetadataState(s, [[] for _ in range(len(s))])


def update_metadata(state: MetadataState, layer: int, cu_old, cu_new):
    """Patch seq_lens and num_actual_tokens after a drop at `layer` and record
    (layer, retained length) in each request's drop history."""
    cu_old = np.asarray(cu_old, dtype=np.int64)
    cu_new = np.asarray(cu_new, dtype=np.int64)
    R = len(cu_old) - 1
    seq = state.seq_lens.copy()
    hist = [list(h) for h in state.history]
    for r in range(R):
        dropped = (cu_old[r + 1] - cu_old[r]) - (cu_new[r + 1] - cu_new[r])
        seq[r] = seq[r] - dropped
        hist[r].append((int(layer), int(seq[r])))
    return MetadataState(seq, hist), int(cu_new[R])


def seqused_eq17(history_r, layer_prime: int, orig_len: int, kv_len: int) -> int:
    """seqused of request r at layer l' (Eq. 17): the retained length after the
    last drop at a layer strictly before l', plus the tokens appended since
    prefill; with no such drop, the original length plus those tokens."""
    before = [(l, s) for (l, s) in history_r if l < layer_prime]
    base = max(before)[1] if before else orig_len
    return int(base + (kv_len - orig_len))


# ---------------------------------------------------------------------------
# Per-layer KV cache slots and the paged-cache write: UniPrefill Sec. 3.5
# ("vLLM scheduler integration"), Eq. 16
# ---------------------------------------------------------------------------
def retained_positions(cu_seqlens, seq_lens):
    """Logical position p_i of every row of the (compacted) token stream.

    Reading of p_i in Eq. 16: a layer after a drop caches only the retained
    tokens, densely (its KV length is the retained length, Eq. 17), so the
    k-th retained token of request r sits at p = (seq_lens[r] - kept_r) + k,
    where seq_lens[r] - kept_r counts the request's tokens already cached
    before this prefill chunk (zero for a fresh prefill).  seq_lens are the
    patched lengths after the drop."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    pos = np.empty(int(cu[-1]), dtype=np.int64)
    for r in range(len(cu) - 1):
        kept = int(cu[r + 1] - cu[r])
        pos[cu[r]: cu[r + 1]] = (sl[r] - kept) + np.arange(kept)
    return pos


def slot_mapping(block_table, B: int, cu_seqlens, seq_lens, max_tokens=None):
    """Eq. 16: slot_i = block_table[r_i, floor(p_i / B)] * B + (p_i mod B).

    One slot per row of the stream, padded with -1 up to max_tokens.  A row
    whose position falls outside the table (p < 0, or floor(p / B) beyond the
    table's width) or whose table entry is negative gets -1: no slot."""
    table = np.asarray(block_table, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    width = table.shape[1] if table.ndim == 2 else 0
    slots = np.full(T if max_tokens is None else int(max_tokens), -1, dtype=np.int64)
    pos = retained_positions(cu, seq_lens)
    for r in range(len(cu) - 1):
        for i in range(int(cu[r]), int(cu[r + 1])):
            p = int(pos[i])
            if p < 0 or p // B >= width:
                continue
            phys = int(table[r, p // B])
            if phys >= 0:
                slots[i] = phys * B + p % B
    return slots


def write_kv_cache(key_cache, value_cache, slots, key, value, count: int):
    """Rows i < count of key and value go to cache row slots[i] (slot-major
    cache: [num_blocks * B, row]); rows without a slot (negative, or past the
    cache) are not written.  Returns the new caches."""
    kc = np.array(key_cache, copy=True)
    vc = None if value_cache is None else np.array(value_cache, copy=True)
    for i in range(int(count)):
        s = int(slots[i])
        if 0 <= s < len(kc):
            kc[s] = key[i]
            if vc is not None:
                vc[s] = value[i]
    return kc, vc


# ---------------------------------------------------------------------------
# A downstream sublayer on the retained set: UniPrefill Sec. 3.4 Eq. 7 (each
# sublayer after a drop maps only the retained rows) and Eq. 9-10 (the saved
# cost is the dropped share of every later sublayer's O(N d^2))
# ---------------------------------------------------------------------------
def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def ffn_hidden(x_bits, w_gate_up_bits):
    """The gated FFN's activation, token by token: g = x Wg^T, u = x Wu^T,
    h = silu(g) * u.  x [rows, D], w_gate_up [2F, D] (gate rows first, then
    up rows), bf16 bit patterns; float64 [rows, F]."""
    x = bf16_bits_to_f64(np.asarray(x_bits))
    w = bf16_bits_to_f64(np.asarray(w_gate_up_bits))
    F = w.shape[0] // 2
    g = x @ w[:F].T
    u = x @ w[F:].T
    return silu(g) * u


def ffn_swiglu(x_bits, w_gate_up_bits, w_down_bits):
    """Gated FFN of the LLaMA family (SwiGLU), token by token:
        y = h Wd^T with h = silu(x Wg^T) * (x Wu^T) (ffn_hidden),
    w_down [D, F] bf16 bit patterns; float64 throughout."""
    wd = bf16_bits_to_f64(np.asarray(w_down_bits))
    return ffn_hidden(x_bits, w_gate_up_bits) @ wd.T
