"""The CPU oracle against its pins (closed forms, invariants, brute force, page figures)."""

import numpy as np
import pytest

import oracle_pins as pins
import synth
from oracle import attention


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def test_absorbed_matches_materialised_tiny_config_shape():
    """At the tiny config's real dims (16 heads, d_c 256, d_r 32) over 300 tokens."""
    case = synth.direct_decode(synth.TINY, "f32", [300], seed=31)
    kw = dict(scale=case.shape.scale)
    m = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                               case.qr, case.w_uk, case.w_uv, evaluate=attention.materialised, **kw)
    a = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                               case.qr, case.w_uk, case.w_uv, evaluate=attention.absorbed, **kw)
    for k in ("o", "obar", "lse"):
        rel = np.max(np.abs(a[k] - m[k])) / np.sqrt(np.mean(m[k] ** 2))
        assert rel <= 1e-12, (k, rel)


def test_config1_scores_have_unit_scale():
    """The tiny fp32 decode config draws h ~ N(0,1), so its scores are O(1), not flat."""
    case = synth.config1()
    r = attention.absorbed(case.qc, case.qr, case.q_pos, case.c_rows, case.kr_rows, case.w_uk,
                           case.w_uv, case.shape.scale)
    # weights are far from uniform: max alpha well above 1/256
    s = r["q_tilde"][0] @ case.c_rows.T
    assert np.std(s * case.shape.scale) > 0.3


def test_prefill_batch_matches_per_sequence_decode():
    case = synth.direct_prefill(synth.TINY, "bf16", [5, 0], [3, 4], seed=37)
    pre = attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets,
                                  case.qc, case.qr, case.w_uk, case.w_uv, case.shape.scale)
    for g in range(int(case.cu_q[-1])):
        b = int(np.searchsorted(case.cu_q, g, side="right") - 1)
        pos = int(case.q_start[b] + g - case.cu_q[b])
        r0 = int(case.row_offsets[b])
        dec = attention.materialised(case.qc[g:g + 1], case.qr[g:g + 1], [pos], case.c_rows[r0:r0 + pos + 1],
                                     case.kr_rows[r0:r0 + pos + 1], case.w_uk, case.w_uv, case.shape.scale)
        for k in ("o", "obar", "lse"):
            assert np.allclose(pre[k][g], dec[k][0], rtol=1e-13, atol=1e-13)
