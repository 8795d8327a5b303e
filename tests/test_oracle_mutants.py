"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Every mutant replaces one oracle function for the duration of a test; the pin
suite of test_oracle_pins.py must then fail somewhere.  This shows the pins are
strong enough that a dropped term, a wrong sign or index, or a transposed
operand in the oracle cannot go unnoticed.
"""
import numpy as np
import pytest

import oracle
from oracle import core as OA, masks as M, paged as OP, blockmask as OB, backward as OBW
import test_oracle_pins as P
import test_oracle_backward as PB
import test_oracle_score_mods as PS
from oracle import score_mods as OSM

PINS = [
    lambda: [P.pin_brute(c) for c in P.BRUTE_CASES],
    P.pin_sdpa_causal, P.pin_sdpa_window_docs, P.pin_sdpa_block, P.pin_sdpa_tiles_gqa,
    P.pin_sdpa_decode_paged, P.pin_probs_sum_to_one, P.pin_constant_v, P.pin_one_visible_key,
    P.pin_q0_counts, P.pin_identities, P.pin_split_combine, P.pin_paged_equals_contiguous,
    P.pin_blockmask_classes, P.test_hand_worked_golden, P.test_brute_force_paged_two_splits,
] + PB.BWD_PINS + PS.SCORE_PINS


def _caught():
    for pin in PINS:
        try:
            pin()
        except Exception:
            return True
    return False


def _scores_no_scale(q_rows, k, scale):
    return np.asarray(q_rows, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T


def _softmax_lse_no_max(s, visible):
    p, lse = _orig_softmax(s, visible)
    s2 = np.where(visible, s, -np.inf)
    m = np.max(s2, axis=-1)
    return p, np.where(np.isfinite(m), lse - m, lse)


def _softmax_sign(s, visible):
    return _orig_softmax(-s, visible)


def _causal_off_by_one(Nq, Nk):
    def mod(b, h, q_idx, kv_idx):
        return np.asarray(kv_idx) < np.asarray(q_idx) + (Nk - Nq)
    return mod


def _causal_top_left(Nq, Nk):
    def mod(b, h, q_idx, kv_idx):
        return np.asarray(kv_idx) <= np.asarray(q_idx)
    return mod


def _window_exclusive(left, right, Nq, Nk):
    def mod(b, h, q_idx, kv_idx):
        p = np.asarray(q_idx) + (Nk - Nq)
        k = np.asarray(kv_idx)
        return (k > p - left) & (k <= p + right)
    return mod


def _block_causal_strict(bs, Nq, Nk):
    def mod(b, h, q_idx, kv_idx):
        p = np.asarray(q_idx) + (Nk - Nq)
        return (np.asarray(kv_idx) // bs) < (p // bs) + (np.asarray(kv_idx) % bs == 0)
    return mod


def _combine_unweighted(o_parts, lse_parts, axis=0):
    o, lse = _orig_combine(o_parts, lse_parts, axis)
    return np.mean(np.asarray(o_parts), axis=axis), lse


def _gather_swapped(pool, block_table, b, seq_len):
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    P = pool.shape[1]
    j = np.arange(seq_len)
    rows = pool[bt[b, j % bt.shape[1]], (j // P) % P]
    return np.transpose(rows, (1, 0, 2))


def _blockmask_full_masked(tile_map, tile, partial_mod):
    def mod(b, h, q_idx, kv_idx):
        tm = np.asarray(tile_map)
        tm = tm if tm.ndim == 2 else tm[0, 0]
        st = tm[np.asarray(q_idx) // tile, np.asarray(kv_idx) // tile]
        return (st >= 1) & partial_mod(b, h, q_idx, kv_idx)
    return mod


_orig_softmax = OA.masked_softmax
_orig_combine = OA.combine


def _attention_rows_gqa_modulo(q, k, v, scale, mask_mod, b, hq, rows):
    Hkv = k.shape[1]
    kk = np.asarray(k)[:, [hq % Hkv] * k.shape[1]]
    vv = np.asarray(v)[:, [hq % Hkv] * k.shape[1]]
    G = q.shape[1] // Hkv
    return _orig_rows(q, kk, vv, scale, mask_mod, b, (hq % Hkv) * G, rows)


def _attention_rows_kv_swapped(q, k, v, scale, mask_mod, b, hq, rows):
    return _orig_rows(q, v, k, scale, mask_mod, b, hq, rows)


_orig_rows = OA.attention_rows
_orig_bwd_rows = OBW.bwd_rows


def _softmax_grad_no_delta(p, dp):
    return p * dp


def _softmax_grad_delta_sign(p, dp):
    return p * (dp + np.sum(p * dp, axis=-1, keepdims=True))


def _bwd_rows_dk_unscaled(q, k, v, do, scale, mask_mod, b, hq, rows):
    dq, dk, dv, p, ds = _orig_bwd_rows(q, k, v, do, scale, mask_mod, b, hq, rows)
    return dq, dk / scale, dv, p, ds


def _bwd_rows_dq_uses_v(q, k, v, do, scale, mask_mod, b, hq, rows):
    dq, dk, dv, p, ds = _orig_bwd_rows(q, k, v, do, scale, mask_mod, b, hq, rows)
    kvh = hq // (q.shape[1] // k.shape[1])
    return scale * (ds @ np.asarray(v[b, kvh], dtype=np.float64)), dk, dv, p, ds


def _bwd_rows_dv_from_o(q, k, v, do, scale, mask_mod, b, hq, rows):
    dq, dk, dv, p, ds = _orig_bwd_rows(q, k, v, do, scale, mask_mod, b, hq, rows)
    kvh = hq // (q.shape[1] // k.shape[1])
    return dq, dk, p.T @ (p @ np.asarray(v[b, kvh], dtype=np.float64)), p, ds


def _bwd_rows_gqa_modulo(q, k, v, do, scale, mask_mod, b, hq, rows):
    Hkv = k.shape[1]
    G = q.shape[1] // Hkv
    kk = np.repeat(np.asarray(k)[:, [hq % Hkv]], Hkv, axis=1)
    vv = np.repeat(np.asarray(v)[:, [hq % Hkv]], Hkv, axis=1)
    kvh = hq // G
    kk[:, kvh], vv[:, kvh] = np.asarray(k)[:, hq % Hkv], np.asarray(v)[:, hq % Hkv]
    return _orig_bwd_rows(q, kk, vv, do, scale, mask_mod, b, hq, rows)

def _alibi_sign(slopes, Nq, Nk):
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score - sl[h] * (np.asarray(kv_idx) - (np.asarray(q_idx) + (Nk - Nq)))
    return OSM._additive(mod)


def _alibi_sym_no_abs(slopes, Nq, Nk):
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score - sl[h] * (np.asarray(kv_idx) - (np.asarray(q_idx) + (Nk - Nq)))
    return OSM._additive(mod)


def _alibi_top_left(slopes, Nq, Nk):
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score + sl[h] * (np.asarray(kv_idx) - np.asarray(q_idx))
    return OSM._additive(mod)


def _rel_bias_unclamped_offset(table, R, Nq, Nk):
    tb = np.asarray(table, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        d = np.asarray(kv_idx) - (np.asarray(q_idx) + (Nk - Nq))
        return score + tb[h][np.clip(d + R, 0, 2 * R - 1)]
    return OSM._additive(mod)


def _rel_bias_reversed(table, R, Nq, Nk):
    tb = np.asarray(table, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        d = np.asarray(q_idx) + (Nk - Nq) - np.asarray(kv_idx)
        return score + tb[h][np.clip(d, -R, R) + R]
    return OSM._additive(mod)


def _softcap_no_jacobian(cap):
    m = _orig_softcap(cap)
    m.dscore = lambda score, b, h, q_idx, kv_idx: np.ones_like(np.asarray(score, dtype=np.float64))
    return m


def _softcap_jacobian_sign(cap):
    m = _orig_softcap(cap)

    def dscore(score, b, h, q_idx, kv_idx):
        t = np.tanh(np.asarray(score, dtype=np.float64) / cap)
        return 1.0 + t * t
    m.dscore = dscore
    return m


def _softcap_no_cap_factor(cap):
    def mod(score, b, h, q_idx, kv_idx):
        return np.tanh(np.asarray(score, dtype=np.float64) / cap)

    def dscore(score, b, h, q_idx, kv_idx):
        t = np.tanh(np.asarray(score, dtype=np.float64) / cap)
        return (1.0 - t * t) / cap
    mod.dscore = dscore
    return mod


_orig_softcap = OSM.softcap



_orig_document = M.document
_orig_key_range = M.key_range
_orig_classify = OB.classify
_orig_tile_lists = OB.tile_lists


def _document_shifted(doc_lengths_per_batch, Nq, Nk):
    """Document boundaries one token late (the first document one token longer)."""
    lens = [[l[0] + 1, *l[1:-1], l[-1] - 1] if len(l) > 1 else list(l) for l in doc_lengths_per_batch]
    return _orig_document(lens, Nq, Nk)


def _key_range_inclusive(lo, hi):
    def mod(b, h, q_idx, kv_idx):
        k = np.asarray(kv_idx)
        return np.broadcast_to((k >= lo) & (k <= hi), np.broadcast(np.asarray(q_idx), k).shape)
    return mod


def _classify_partial_as_full(mask_mod, b, h, Nq, Nk, tile):
    c = _orig_classify(mask_mod, b, h, Nq, Nk, tile)
    c[c == OB.PARTIAL] = OB.FULL
    return c


def _classify_padded_tiles(mask_mod, b, h, Nq, Nk, tile):
    """Pairs past the sequence ends counted as hidden pairs of the tile."""
    nqt, nkt = -(-Nq // tile), -(-Nk // tile)
    out = np.zeros((nqt, nkt), dtype=np.uint8)
    for i in range(nqt):
        rows = np.arange(i * tile, (i + 1) * tile)
        dm = np.zeros((tile, nkt * tile), dtype=bool)
        dm[rows < Nq, :Nk] = M.dense(mask_mod, b, h, Nq, Nk, rows[rows < Nq])
        for j in range(nkt):
            blk = dm[:, j * tile:(j + 1) * tile]
            out[i, j] = OB.EMPTY if not blk.any() else (OB.FULL if blk.all() else OB.PARTIAL)
    return out


def _tile_lists_classes_swapped(classes):
    pn, pi, fn, fi = _orig_tile_lists(classes)
    return fn, fi, pn, pi



_orig_window = M.window
_orig_and = M.and_
_orig_smod_combine = OSM.combine


def _window_top_left(left, right, Nq, Nk):
    """Window positions not aligned to the end of the key sequence when Nq != Nk."""
    return _orig_window(left, right, Nk, Nk)


def _and_as_or(*mods):
    def mod(b, h, q_idx, kv_idx):
        out = None
        for m in mods:
            r = m(b, h, q_idx, kv_idx)
            out = r if out is None else (out | r)
        return out
    return mod


def _softmax_empty_rows_lse_zero(s, visible):
    p, lse = _orig_softmax(s, visible)
    return p, np.where(np.isfinite(lse), lse, 0.0)


def _smod_combine_reversed(*mods):
    """The score changes applied in reverse order (the soft-cap after the additive terms)."""
    return _orig_smod_combine(*reversed(mods))


_orig_blockmask = M.blockmask


def _blockmask_first_map_only(tile_map, tile, partial_mod):
    """Per-(batch, head) tile maps read as the map of batch 0, head 0."""
    tm = np.asarray(tile_map)
    return _orig_blockmask(tm if tm.ndim == 2 else tm[0, 0], tile, partial_mod)


MUTANTS = {
    "scale_dropped": (OA, "scores", _scores_no_scale),
    "lse_without_max": (OA, "masked_softmax", _softmax_lse_no_max),
    "score_sign": (OA, "masked_softmax", _softmax_sign),
    "causal_off_by_one": (M, "causal", _causal_off_by_one),
    "causal_top_left": (M, "causal", _causal_top_left),
    "window_exclusive": (M, "window", _window_exclusive),
    "block_causal_wrong": (M, "block_causal", _block_causal_strict),
    "combine_unweighted": (OA, "combine", _combine_unweighted),
    "paged_index_swapped": (OP, "gather", _gather_swapped),
    "blockmask_full_tiles_masked": (M, "blockmask", _blockmask_full_masked),
    "gqa_modulo_mapping": (OA, "attention_rows", _attention_rows_gqa_modulo),
    "k_v_transposed": (OA, "attention_rows", _attention_rows_kv_swapped),
    "bwd_delta_dropped": (OBW, "softmax_grad", _softmax_grad_no_delta),
    "bwd_delta_sign": (OBW, "softmax_grad", _softmax_grad_delta_sign),
    "bwd_dk_unscaled": (OBW, "bwd_rows", _bwd_rows_dk_unscaled),
    "bwd_dq_uses_v": (OBW, "bwd_rows", _bwd_rows_dq_uses_v),
    "bwd_dv_from_o": (OBW, "bwd_rows", _bwd_rows_dv_from_o),
    "bwd_gqa_modulo_mapping": (OBW, "bwd_rows", _bwd_rows_gqa_modulo),
    "alibi_sign": (OSM, "alibi", _alibi_sign),
    "alibi_sym_without_abs": (OSM, "alibi_sym", _alibi_sym_no_abs),
    "alibi_top_left": (OSM, "alibi", _alibi_top_left),
    "rel_bias_clamp_off_by_one": (OSM, "rel_bias", _rel_bias_unclamped_offset),
    "rel_bias_reversed_distance": (OSM, "rel_bias", _rel_bias_reversed),
    "softcap_jacobian_dropped": (OSM, "softcap", _softcap_no_jacobian),
    "softcap_jacobian_sign": (OSM, "softcap", _softcap_jacobian_sign),
    "softcap_cap_factor_dropped": (OSM, "softcap", _softcap_no_cap_factor),
    "document_boundary_shifted": (M, "document", _document_shifted),
    "key_range_inclusive_end": (M, "key_range", _key_range_inclusive),
    "tile_class_partial_as_full": (OB, "classify", _classify_partial_as_full),
    "tile_class_padded_tail": (OB, "classify", _classify_padded_tiles),
    "tile_lists_classes_swapped": (OB, "tile_lists", _tile_lists_classes_swapped),
    "window_top_left": (M, "window", _window_top_left),
    "mask_and_as_or": (M, "and_", _and_as_or),
    "empty_row_lse_zero": (OA, "masked_softmax", _softmax_empty_rows_lse_zero),
    "score_mod_order_reversed": (OSM, "combine", _smod_combine_reversed),
    "blockmask_first_map_only": (M, "blockmask", _blockmask_first_map_only),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, repl = MUTANTS[name]
    monkeypatch.setattr(mod, attr, repl)
    # functions re-exported at package level are patched too
    if hasattr(oracle, attr) and mod is OA:
        monkeypatch.setattr(oracle, attr, repl)
    assert _caught(), f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_all_pins():
    assert not _caught()
