"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each."""

import math

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention, front, obstruction, paging, rope

_orig_rotate = rope.rotate
_orig_thetas = rope.thetas
_orig_matrix = rope.rotation_matrix
_orig_materialised = attention.materialised
_orig_values = attention.materialise_values
_orig_keys = attention.materialise_keys
_orig_visible = attention._visible
_orig_slot = paging.slot
_orig_fold = front.fold_query_weights
_orig_components = obstruction.frequency_components
_orig_family = obstruction.family
_orig_span = obstruction.span


def _clockwise_rotate(x, positions, base=10000.0):
    return _orig_rotate(x, -np.asarray(positions), base)


def _clockwise_matrix(p, d, base=10000.0):
    return _orig_matrix(-p, d, base)


def _half_split_rotate(x, positions, base=10000.0):
    # "rotate-half" pairing (j, j + d/2) instead of (2j, 2j+1)
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.empty(d, dtype=int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y = _orig_rotate(x[..., perm], positions, base)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _wrong_thetas(d, base=10000.0):
    return np.power(np.float64(base), -np.arange(d // 2, dtype=np.float64) / d)


def _keys_without_rope(c, kr, w_uk, key_pos, base=10000.0):
    k = _orig_keys(c, kr, w_uk, key_pos, base)
    k[..., w_uk.shape[1]:] = 0.0
    return k


def _per_head_keys_take_head0(c, kr, w_uk, key_pos, base=10000.0):
    # per-head position keys read as head 0's key for every head
    kr = np.asarray(kr)
    if kr.ndim == 3:
        kr = np.repeat(kr[:, :1, :], kr.shape[1], axis=1)
    return _orig_keys(c, kr, w_uk, key_pos, base)


def _keys_unrotated(c, kr, w_uk, key_pos, base=10000.0):
    return _orig_keys(c, kr, w_uk, np.zeros_like(np.asarray(key_pos)), base)


def _values_from_uk(c, w_uv):
    return _orig_values(c, w_uv[:, ::-1, :])  # wrong row order of W_UV (a transposed-index slip)


def _strict_causal(q_pos, key_pos, causal):
    if causal:
        return key_pos[None, :] < np.asarray(q_pos)[:, None]
    return _orig_visible(q_pos, key_pos, causal)


def _materialised_no_scale(*a, **k):
    if len(a) > 7:
        a = a[:7] + (1.0,) + a[8:]
    else:
        k["scale"] = 1.0
    return _orig_materialised(*a, **k)


def _materialised_scales_swapped(*a, position_scale=None, **k):
    # the two factors applied to the wrong channels
    if position_scale is None:
        return _orig_materialised(*a, **k)
    a = list(a)
    a[7], position_scale = position_scale, a[7]
    return _orig_materialised(*a, position_scale=position_scale, **k)


def _materialised_query_unrotated(qc, qr, q_pos, *a, **k):
    return _orig_materialised(qc, qr, np.zeros_like(np.asarray(q_pos)), *a, **k)


_orig_decode_batch = attention.decode_batch
_orig_prefill_batch = attention.prefill_batch


def _decode_query_one_late(seq_lens, c_rows, kr_rows, row_offsets, qc, qr, *a, **k):
    # the query placed at T_b (one past its own token) instead of T_b - 1
    lens = np.asarray(seq_lens)
    out = []
    for b in range(len(lens)):
        t, r0 = int(lens[b]), int(row_offsets[b])
        out.append(attention.materialised(qc[b:b + 1], qr[b:b + 1], np.array([t]), c_rows[r0:r0 + t],
                                          kr_rows[r0:r0 + t], *a[:3]))
    return {key: np.concatenate([r[key] for r in out]) for key in ("o", "obar", "lse")}


def _decode_rows_shifted(seq_lens, c_rows, kr_rows, row_offsets, *a, **k):
    # every sequence reads its rows one further on (an offset slip)
    offs = np.minimum(np.asarray(row_offsets) + 1, len(c_rows) - np.asarray(seq_lens))
    return _orig_decode_batch(seq_lens, c_rows, kr_rows, np.maximum(offs, 0), *a, **k)


def _prefill_not_causal(cu_q, q_start, *a, **k):
    # every chunk query sees its whole chunk (start positions taken as one chunk later)
    return _orig_prefill_batch(cu_q, np.asarray(q_start) + 1, *a, **k)


def _bad_slot(table, seq, pos, ps):
    return int(table[seq, pos // ps]) * ps + pos // ps


def _kv_latent_transposed(h, w_dkv):
    # the weight read as [in, out]: only survives where it is square
    w = np.asarray(w_dkv, np.float64)
    return np.asarray(h, np.float64)[:, : w.shape[0]] @ w[:, : w.shape[0]]


def _fold_wrong_side(w_uq, w_uk):
    # W_UQ^T W_UK contracted over the wrong index pair (d_q with d_c swapped)
    f = _orig_fold(w_uq, w_uk)
    return f[:, ::-1, :]


def _query_skips_latent(cq, w_uq):
    # the content query taken without its up-projection's head split
    w = np.asarray(w_uq, np.float64)
    return np.einsum("hdq,nq->nhd", w[::-1], np.asarray(cq, np.float64))


def _position_query_from_content(cq, w_qr):
    return np.einsum("hrq,nq->nhr", np.asarray(w_qr, np.float64), np.asarray(cq, np.float64)) * 0.0


def _components_sine_flipped(w_qr, w_ukr):
    # J taken as the clockwise quarter turn
    mc, ms = _orig_components(w_qr, w_ukr)
    return mc, -ms


def _family_ignores_shift(w_qr, w_ukr, deltas, base=10000.0):
    return _orig_family(w_qr, w_ukr, np.zeros(len(deltas)), base)


def _family_half_the_pairs(w_qr, w_ukr, deltas, base=10000.0):
    # only the first half of the rotated dimensions carried into the family
    h = max(2, (np.asarray(w_qr).shape[0] // 4) * 2)
    return _orig_family(np.asarray(w_qr)[:h], np.asarray(w_ukr)[:h], deltas, base)


def _family_reversed_shift(w_qr, w_ukr, deltas, base=10000.0):
    # delta taken as query position minus key position
    return _orig_family(w_qr, w_ukr, -np.asarray(deltas), base)


def _span_absolute_cliff(fam, cliff=1e-10):
    rows = np.asarray(fam, np.float64).reshape(len(fam), -1)
    sv = np.linalg.svd(rows, compute_uv=False)
    rank = int(np.sum(sv > cliff))
    return rank, sv, float(sv[rank] / sv[0]) if 0 < rank < sv.size else 0.0


def _dc_first_member(fam):
    fam = np.asarray(fam, np.float64)
    m = fam[0]
    return m, float(np.sum((fam - m) ** 2) / np.sum(fam * fam))


MUTATIONS = {
    "rope_clockwise": [(rope, "rotate", _clockwise_rotate), (rope, "rotation_matrix", _clockwise_matrix)],
    "rope_half_split_pairs": [(rope, "rotate", _half_split_rotate)],
    "rope_theta_exponent": [(rope, "thetas", _wrong_thetas)],
    "keys_drop_rope_term": [(attention, "materialise_keys", _keys_without_rope)],
    "per_head_keys_head0_only": [(attention, "materialise_keys", _per_head_keys_take_head0)],
    "keys_not_rotated": [(attention, "materialise_keys", _keys_unrotated)],
    "values_wrong_rows": [(attention, "materialise_values", _values_from_uk)],
    "causal_excludes_diagonal": [(attention, "_visible", _strict_causal)],
    "score_scale_dropped": [(attention, "materialised", _materialised_no_scale)],
    "two_scale_swapped": [(attention, "materialised", _materialised_scales_swapped)],
    "query_not_rotated": [(attention, "materialised", _materialised_query_unrotated)],
    "paging_offset_slip": [(paging, "slot", _bad_slot)],
    "decode_query_one_late": [(attention, "decode_batch", _decode_query_one_late)],
    "decode_rows_shifted": [(attention, "decode_batch", _decode_rows_shifted)],
    "prefill_positions_shifted": [(attention, "prefill_batch", _prefill_not_causal)],
    "front_latent_weight_transposed": [(front, "kv_latent", _kv_latent_transposed)],
    "front_fold_wrong_index": [(front, "fold_query_weights", _fold_wrong_side)],
    "front_query_heads_swapped": [(front, "content_query", _query_skips_latent)],
    "front_position_query_dropped": [(front, "position_query", _position_query_from_content)],
    "obstruction_sine_flipped": [(obstruction, "frequency_components", _components_sine_flipped)],
    "obstruction_family_ignores_shift": [(obstruction, "family", _family_ignores_shift)],
    "obstruction_family_reversed_shift": [(obstruction, "family", _family_reversed_shift)],
    "obstruction_family_half_pairs": [(obstruction, "family", _family_half_the_pairs)],
    "obstruction_absolute_cliff": [(obstruction, "span", _span_absolute_cliff)],
    "obstruction_dc_first_member": [(obstruction, "best_single_matrix", _dc_first_member)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    assert pins.failing_pins() == [], "pins must pass on the unmutated oracle"
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    failed = pins.failing_pins()
    assert failed, f"mutation {name} slipped past every pin"
