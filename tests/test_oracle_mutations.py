"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them.  This shows the pins are strong enough to tie the
oracle to the paper: a dropped term, a wrong sign or index, or a transposed
operand anywhere in it fails at least one check.  Everything runs on the CPU;
the oracle itself is never modified."""
from __future__ import annotations

import math
import types

import numpy as np
import pytest

import oracle
import pins
from oracle import uniprefill_oracle as U


def _namespace(**over):
    ns = types.SimpleNamespace(**{name: getattr(U, name) for name in dir(U) if not name.startswith("_")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _importance_variant(head_mean=False, causal=True, gqa="floor", scale_one=False, transpose_rows=False):
    def token_importance(q_bits, k_bits, start, N, hq, hkv, d, n, scale=None):
        if N <= 0:
            return np.zeros(0)
        ne = min(n, N)
        sc = 1.0 if scale_one else (1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale))
        keys = np.arange(N)
        rowpos = (N - ne) + np.arange(ne)
        if transpose_rows:
            rowpos = rowpos[::-1]
        future = keys[None, :] > rowpos[:, None]
        o = np.zeros(N)
        for h in range(hq):
            kv = (h * hkv) // hq if gqa == "floor" else h % hkv
            Qw = U.bf16_bits_to_f64(q_bits[start + N - ne: start + N, h, :])
            Kr = U.bf16_bits_to_f64(k_bits[start: start + N, kv, :])
            Z = (Qw @ Kr.T) * sc
            if causal:
                Z[future] = -np.inf
            Z -= Z.max(axis=1, keepdims=True)
            E = np.exp(Z)
            o += (E / E.sum(axis=1, keepdims=True)).sum(axis=0)
        return o / hq if head_mean else o
    return token_importance


def _scores_variant(ti, partial_true_len=False, use_n=False):
    def request_block_scores(q_bits, k_bits, start, N, hq, hkv, d, G, n, scale=None):
        o = ti(q_bits, k_bits, start, N, hq, hkv, d, n, scale)
        if N <= 0:
            return np.zeros(0), o
        ne = n if use_n else min(n, N)
        nb = -(-N // G)
        b = np.zeros(nb)
        for g in range(nb):
            seg = o[g * G: min((g + 1) * G, N)]
            b[g] = seg.sum() / ((len(seg) if partial_true_len else G) * ne)
        return b, o

    def block_scores(q_bits, k_bits, cu_seqlens, hq, hkv, d, G, n, scale=None):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        parts, offs = [], [0]
        for r in range(len(cu) - 1):
            b, _ = request_block_scores(q_bits, k_bits, int(cu[r]), int(cu[r + 1] - cu[r]), hq, hkv, d, G, n, scale)
            parts.append(b)
            offs.append(offs[-1] + len(b))
        return np.concatenate(parts), np.asarray(offs)
    return request_block_scores, block_scores


def _scoring_mutant(ti_kw=None, **sc_kw):
    ti = _importance_variant(**(ti_kw or {}))
    rbs, bs = _scores_variant(ti, **sc_kw)
    return _namespace(token_importance=ti, request_block_scores=rbs, block_scores=bs)


def _topp_variant(tie="larger_first", exclusive=False, ascending=False, float_sum=False):
    def pack_keys(b32):
        g = np.arange(len(b32), dtype=np.uint64)
        if tie == "smaller_first":
            g = np.uint64(len(b32) - 1) - g if len(b32) else g
        return (U.phi(b32).astype(np.uint64) << np.uint64(32)) | g

    def top_p_select(b32, p):
        b32 = np.ascontiguousarray(b32, dtype=np.float32)
        nb = len(b32)
        keep = np.zeros(nb, bool)
        if nb == 0:
            return keep
        order = np.argsort(pack_keys(b32), kind="stable")
        if not ascending:
            order = order[::-1]
        bf = b32.astype(np.float64)
        if float_sum:          # mass taken as the count of blocks, not their scores
            cs = np.cumsum(np.ones(nb))
            thr = p * nb
        else:
            cs = np.cumsum(bf[order])
            thr = p * bf.sum()
        hit = np.nonzero(cs >= thr)[0]
        kstar = int(hit[0]) + 1 if len(hit) else nb
        if exclusive:
            kstar -= 1
        keep[order[:kstar]] = True
        return keep
    return _namespace(pack_keys=pack_keys, top_p_select=top_p_select)


def _phi_ge_zero(b32):
    x = np.ascontiguousarray(b32, dtype=np.float32)
    bits = x.view(np.uint32)
    return np.where(x >= 0, bits ^ np.uint32(0x80000000), bits ^ np.uint32(0xFFFFFFFF)).astype(np.uint32)


def _expand_no_window(keep_block, N, G, A, n):
    i = np.arange(N)
    return (keep_block[i // G] | (i < A)).astype(np.uint8)


def _expand_off_by_one(keep_block, N, G, A, n):
    i = np.arange(N)
    return (keep_block[i // G] | (i <= A) | (i > N - n)).astype(np.uint8)


def _compact_no_compose(mask, cu_seqlens, buffers=(), index_in=None):
    return U.compact(mask, cu_seqlens, buffers, None)


def _compact_cu_inclusive(mask, cu_seqlens, buffers=(), index_in=None):
    outs, idx, cu_out = U.compact(mask, cu_seqlens, buffers, index_in)
    cu = np.asarray(cu_seqlens)
    m = np.asarray(mask).astype(np.int64)
    cu_out = np.array([m[: min(c + 1, len(m))].sum() for c in cu], dtype=np.int32)
    return outs, idx, cu_out


def _seqused_le(history_r, layer_prime, orig_len, kv_len):
    before = [(l, s) for (l, s) in history_r if l <= layer_prime]
    base = max(before)[1] if before else orig_len
    return int(base + (kv_len - orig_len))


def _seqused_first(history_r, layer_prime, orig_len, kv_len):
    before = [(l, s) for (l, s) in history_r if l < layer_prime]
    base = min(before)[1] if before else orig_len
    return int(base + (kv_len - orig_len))


def _update_sets_kept(state, layer, cu_old, cu_new):
    cu_new = np.asarray(cu_new)
    seq = np.diff(cu_new).astype(np.int64)
    hist = [list(h) + [(int(layer), int(seq[r]))] for r, h in enumerate(state.history)]
    return U.MetadataState(seq, hist), int(cu_new[-1])


def _scatter_all(full, compacted, index_map, count):
    out = np.array(full, copy=True)
    n = min(len(out), len(compacted))
    out[:n] = np.asarray(compacted)[:n]
    return out


def _slot_variant(positions="dense", swap_div_mod=False):
    def retained_positions(cu_seqlens, seq_lens):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        sl = np.asarray(seq_lens, dtype=np.int64)
        pos = np.empty(int(cu[-1]), dtype=np.int64)
        for r in range(len(cu) - 1):
            kept = int(cu[r + 1] - cu[r])
            ctx = {"dense": sl[r] - kept, "no_context": 0, "context_plus_one": sl[r] - kept + 1}[positions]
            pos[cu[r]: cu[r + 1]] = ctx + np.arange(kept)
        return pos

    def slot_mapping(block_table, B, cu_seqlens, seq_lens, max_tokens=None):
        table = np.asarray(block_table, dtype=np.int64)
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        width = table.shape[1]
        slots = np.full(int(cu[-1]) if max_tokens is None else int(max_tokens), -1, dtype=np.int64)
        pos = retained_positions(cu, seq_lens)
        for r in range(len(cu) - 1):
            for i in range(int(cu[r]), int(cu[r + 1])):
                p = int(pos[i])
                col, off = (p % B, p // B) if swap_div_mod else (p // B, p % B)
                if p < 0 or col >= width:
                    continue
                phys = int(table[r, col])
                if phys >= 0:
                    slots[i] = phys * B + off
        return slots
    return _namespace(retained_positions=retained_positions, slot_mapping=slot_mapping)


def _kv_write_all_rows(key_cache, value_cache, slots, key, value, count):
    return U.write_kv_cache(key_cache, value_cache, slots, key, value, len(slots))


def _ffn_variant(act="silu", swap=False, no_up=False):
    def ffn_swiglu(x_bits, w_gate_up_bits, w_down_bits):
        x = U.bf16_bits_to_f64(np.asarray(x_bits))
        w = U.bf16_bits_to_f64(np.asarray(w_gate_up_bits))
        wd = U.bf16_bits_to_f64(np.asarray(w_down_bits))
        F = w.shape[0] // 2
        g, u = x @ w[:F].T, x @ w[F:].T
        if swap:
            g, u = u, g
        a = {"silu": U.silu, "relu": lambda z: np.maximum(z, 0.0), "sigmoid": lambda z: 1.0 / (1.0 + np.exp(-z))}[act](g)
        h = a if no_up else a * u
        return h @ wd.T
    return ffn_swiglu


def _bf16_round(x):
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (((b + (((b >> 16) & 1) + 0x7FFF)) >> 16) << 16).astype(np.uint32).view(np.float32)


def _select_variant(mask_at_block_offsets=False, kept_before_forcing=False, rounding="f32",
                    offsets="ceil", batch_topp=False):
    """select() with one planted mistake: the mask written at the block offsets
    instead of the stream offsets, kept counted from the top-p blocks before
    the sinks and window are forced, the scores left in float64 or rounded to
    bf16, block offsets by floor division or one too many per request, or
    top-p taken over the whole batch instead of each request."""
    def select(q_bits, k_bits, cu_seqlens, hq, hkv, d, G, A, n, p, scale=None, scores_in=None):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        R = len(cu) - 1
        if scores_in is None:
            b64, _ = U.block_scores(q_bits, k_bits, cu, hq, hkv, d, G, n, scale)
            b32 = {"f32": b64.astype(np.float32), "none": b64, "bf16": _bf16_round(b64)}[rounding]
        else:
            b64, b32 = None, np.ascontiguousarray(scores_in, dtype=np.float32)
        offs = [0]
        for r in range(R):
            N = int(cu[r + 1] - cu[r])
            nb = {"ceil": -(-N // G), "floor": N // G, "plus_one": N // G + 1}[offsets]
            offs.append(offs[-1] + nb)
        offs = np.asarray(offs, dtype=np.int64)
        T = int(cu[-1])
        mask = np.zeros(T, dtype=np.uint8)
        keep_block = np.zeros(len(b32), dtype=np.uint8)
        kept = np.zeros(R, dtype=np.int32)
        whole = U.top_p_select(b32, p) if batch_topp else None
        for r in range(R):
            N = int(cu[r + 1] - cu[r])
            kb = whole[offs[r]: offs[r + 1]] if batch_topp else U.top_p_select(b32[offs[r]: offs[r + 1]], p)
            keep_block[offs[r]: offs[r + 1]] = kb
            # a request's flags padded or cut to its true block count, so a
            # wrong offset shows in the outputs rather than as a crash
            kbx = np.zeros(-(-N // G), dtype=bool)
            kbx[: min(len(kb), len(kbx))] = np.asarray(kb[: len(kbx)], dtype=bool)
            m = U.expand_mask(kbx, N, G, A, n)
            at = int(offs[r]) if mask_at_block_offsets else int(cu[r])
            mask[at: at + N] = m[: max(0, min(N, T - at))]
            kept[r] = int(sum(min(G, N - g * G) for g in np.nonzero(kbx)[0])) if kept_before_forcing else int(m.sum())
        return dict(b64=b64, b32=b32, block_offsets=offs, keep_block=keep_block, mask=mask, kept=kept)
    return select


def _hidden_variant(swap=False, relu=False):
    def ffn_hidden(x_bits, w_gate_up_bits):
        x = U.bf16_bits_to_f64(np.asarray(x_bits))
        w = U.bf16_bits_to_f64(np.asarray(w_gate_up_bits))
        F = w.shape[0] // 2
        g, u = x @ w[:F].T, x @ w[F:].T
        if swap:
            g, u = u, g
        return (np.maximum(g, 0.0) if relu else U.silu(g)) * u
    return ffn_hidden


def _silu_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


MUTANTS = {
    "head_mean": _scoring_mutant(ti_kw=dict(head_mean=True)),
    "no_causal_mask": _scoring_mutant(ti_kw=dict(causal=False)),
    "gqa_modulo": _scoring_mutant(ti_kw=dict(gqa="mod")),
    "scale_missing": _scoring_mutant(ti_kw=dict(scale_one=True)),
    "window_rows_reversed": _scoring_mutant(ti_kw=dict(transpose_rows=True)),
    "partial_block_true_len": _scoring_mutant(partial_true_len=True),
    "n_instead_of_n_eff": _scoring_mutant(use_n=True),
    "tie_smaller_index_first": _topp_variant(tie="smaller_first"),
    "kstar_exclusive": _topp_variant(exclusive=True),
    "ascending_sort": _topp_variant(ascending=True),
    "count_not_mass": _topp_variant(float_sum=True),
    "phi_by_value": _namespace(phi=_phi_ge_zero),
    "expand_no_window": _namespace(expand_mask=_expand_no_window),
    "expand_off_by_one": _namespace(expand_mask=_expand_off_by_one),
    "compact_no_compose": _namespace(compact=_compact_no_compose),
    "cu_out_inclusive": _namespace(compact=_compact_cu_inclusive),
    "scatter_everything": _namespace(scatter_back=_scatter_all),
    "eq17_le": _namespace(seqused_eq17=_seqused_le),
    "eq17_first_drop": _namespace(seqused_eq17=_seqused_first),
    "seq_lens_set_to_kept": _namespace(update_metadata=_update_sets_kept),
    "slot_without_context": _slot_variant(positions="no_context"),
    "slot_context_off_by_one": _slot_variant(positions="context_plus_one"),
    "slot_div_mod_swapped": _slot_variant(swap_div_mod=True),
    "kv_write_ignores_count": _namespace(write_kv_cache=_kv_write_all_rows),
    "ffn_gate_up_swapped": _namespace(ffn_swiglu=_ffn_variant(swap=True)),
    "ffn_relu_gate": _namespace(ffn_swiglu=_ffn_variant(act="relu")),
    "ffn_sigmoid_gate": _namespace(ffn_swiglu=_ffn_variant(act="sigmoid")),
    "ffn_no_up_projection": _namespace(ffn_swiglu=_ffn_variant(no_up=True)),
    "silu_is_sigmoid": _namespace(silu=_silu_sigmoid),
    "ffn_hidden_gate_up_swapped": _namespace(ffn_hidden=_hidden_variant(swap=True)),
    "ffn_hidden_relu_gate": _namespace(ffn_hidden=_hidden_variant(relu=True)),
    "select_mask_at_block_offsets": _namespace(select=_select_variant(mask_at_block_offsets=True)),
    "select_kept_before_forcing": _namespace(select=_select_variant(kept_before_forcing=True)),
    "select_scores_unrounded": _namespace(select=_select_variant(rounding="none")),
    "select_scores_bf16": _namespace(select=_select_variant(rounding="bf16")),
    "select_offsets_floor": _namespace(select=_select_variant(offsets="floor")),
    "select_offsets_plus_one": _namespace(select=_select_variant(offsets="plus_one")),
    "select_topp_over_batch": _namespace(select=_select_variant(batch_topp=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    impl = MUTANTS[name]
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failures.append(check.__name__)
        except Exception as e:  # a crash is also a catch, but say which
            failures.append(f"{check.__name__}:{type(e).__name__}")
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_namespace_passes():
    impl = _namespace()
    for check in pins.ALL_CHECKS:
        check(impl)
    assert impl.top_p_select is oracle.top_p_select
