"""End-to-end GPU parity: decode and prefill through the five C-ABI calls against the oracle.

The oracle's materialised form (K = [W_UK c ; R k^R], V = W_UV c, plain
softmax) is the reference wherever it finishes in seconds; for long sequences
the oracle's absorbed float64 form is used instead (pinned to the
materialised form to 1e-12 by the oracle's own tests).
"""

import numpy as np
import pytest
import torch

import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth
from oracle import attention

pytestmark = pytest.mark.gpu


def oracle_decode(case, seqs=None, evaluate=attention.materialised):
    return attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base, seqs=seqs,
                                  evaluate=evaluate)


def oracle_prefill(case, queries=None, evaluate=attention.materialised):
    return attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                                   case.qr, case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base,
                                   queries=queries, evaluate=evaluate)


# The latent output obar is stored in the input dtype: for bf16 one more RNE
# rounding (<= 2^-8 of an element, i.e. up to ~2e-2 of the row RMS at a row's
# largest element) than the float32 layer output o, so its max bound is 4e-2.
OBAR_BF16_TOL = (4e-2, 5e-3)


def check(got, want, dtype, rows=None, what=""):
    for k in ("o", "obar"):
        g = got[k] if rows is None else got[k][rows]
        tol = OBAR_BF16_TOL if (k == "obar" and dtype == "bf16") else None
        G.assert_close(g, want[k], dtype, f"{what} {k}", tol=tol)
    g = got["lse"] if rows is None else got["lse"][rows]
    G.assert_lse_close(g, want["lse"], dtype, f"{what} lse")


def test_config1_tiny_decode_f32():
    case = synth.config1()
    check(G.run_decode(case), oracle_decode(case), "f32", what="tiny fp32 decode")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_decode_ragged(dtype):
    lens = [1, 63, 64, 65, 300, 1000, 129]
    case = synth.direct_decode(synth.TINY, dtype, lens, seed=41, shuffle=True)
    check(G.run_decode(case), oracle_decode(case), dtype, what="tiny ragged decode")


@pytest.mark.parametrize("split_pages", [None, 1, 3])
def test_dsv2_decode_ragged(split_pages, monkeypatch):
    if split_pages is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", str(split_pages))
    lens = [1, 64, 65, 700, 2048, 130]
    case = synth.direct_decode(synth.DSV2, "bf16", lens, seed=43, shuffle=True)
    check(G.run_decode(case), oracle_decode(case), "bf16", what=f"dsv2 decode split={split_pages}")


def test_decode_empty_sequence():
    lens = [0, 5, 0, 70]
    case = synth.direct_decode(synth.DSV2, "bf16", lens, seed=47)
    got = G.run_decode(case)
    want = oracle_decode(case)
    assert np.all(got["obar"][[0, 2]] == 0) and np.all(np.isneginf(got["lse"][[0, 2]]))
    check(got, want, "bf16", what="decode with empty sequences")


def test_decode_score_overflow_fallback():
    """Scores that climb by far more than 2^64 within one split take the exact two-pass path."""
    case = synth.direct_decode(synth.DSV2, "bf16", [600], seed=53)
    # make later tokens' latents align with the query and grow, so scores rise by tens of nats
    q_t = attention.query_absorption(case.w_uk, case.qc)[0]  # [H, d_c]
    direction = q_t.mean(axis=0)
    direction /= np.linalg.norm(direction)
    grow = np.linspace(0, 60, 600)[:, None]
    case.c_rows = synth.to_storage(case.c_rows + grow * direction[None, :] * 8, "bf16")
    s = case.shape.scale * (q_t @ case.c_rows.T.astype(np.float64))  # content part of the scores [H, T]
    rise_log2 = (s.max(axis=1) - s[:, :32].max(axis=1)) / np.log(2)
    assert rise_log2.max() > 64 + 8, "the case must push some head past the 2^64 headroom"
    got = G.run_decode(case)
    want = oracle_decode(case)
    # Scores here reach ~80 nats; a bf16 q~ perturbs each score by up to ~2^-8 of
    # its largest terms, so this case carries a larger error than unit-scale scores.
    for k in ("o", "obar"):
        G.assert_close(got[k], want[k], "bf16", f"overflow fallback {k}", tol=(8e-2, 1e-2))


def test_decode_bitwise_repeatable_and_page_independent():
    """Same logical cache under three different physical page assignments: identical bits."""
    lens = [257, 1, 4000, 64]
    case = synth.direct_decode(synth.DSV2, "bf16", lens, seed=59, shuffle=False)
    a = G.run_decode(case)
    b = G.run_decode(case)
    for k in ("o", "obar", "lse"):
        assert np.array_equal(a[k], b[k], equal_nan=True), f"run-to-run {k}"
    rng = np.random.default_rng(7)
    for _ in range(2):
        perm = rng.permutation(case.num_pages).astype(np.int32)
        table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
        c = G.run_decode(case, block_table=table)
        for k in ("o", "obar", "lse"):
            assert np.array_equal(a[k], c[k], equal_nan=True), f"page permutation changed {k}"


def test_decode_poison_independent():
    """NaN in unused page slots never reaches the output (zero-filled cache gives the same bits)."""
    lens = [65, 130, 1]
    case = synth.direct_decode(synth.DSV2, "bf16", lens, seed=61, shuffle=True)
    a = G.run_decode(case, cache=G.build_cache(case, fill=float("nan")))
    b = G.run_decode(case, cache=G.build_cache(case, fill=0.0))
    for k in ("o", "obar", "lse"):
        assert np.array_equal(a[k], b[k]), k
        assert np.all(np.isfinite(a[k]))


def test_config2_tiny_prefill_bf16():
    """Tiny causal prefill with the float32 q_lat (two-term scores)."""
    case = synth.config2()
    check(G.run_prefill(case, precise=True), oracle_prefill(case), "bf16", what="tiny causal prefill")


def test_tiny_bf16_query_path():
    """The tiny shape with a bf16 q_lat: one more rounding (of q~) than the default path.
    An exactly rounded float64 emulation of this arithmetic reaches a per-row max
    error of 2.3e-2 on the tiny causal prefill, so the bound here is 4e-2."""
    case = synth.direct_prefill(synth.TINY, "bf16", [0, 30], [200, 64], seed=79)
    got = G.run_prefill(case, precise=False)
    want = oracle_prefill(case)
    G.assert_close(got["o"], want["o"], "bf16", "o", tol=(4e-2, 5e-3))
    dec = synth.direct_decode(synth.TINY, "bf16", [1, 77, 640], seed=83)
    got = G.run_decode(dec, precise=False)
    G.assert_close(got["o"], oracle_decode(dec)["o"], "bf16", "o", tol=(4e-2, 5e-3))


def test_prefill_ragged_chunks():
    for shape in (synth.TINY, synth.DSV2):
        case = synth.direct_prefill(shape, "bf16", [0, 100, 64, 7], [5, 130, 1, 64], seed=67, shuffle=True)
        check(G.run_prefill(case), oracle_prefill(case), "bf16", what=f"prefill n_h={shape.n_heads}")


def test_prefill_f32():
    case = synth.direct_prefill(synth.TINY, "f32", [10, 0], [20, 33], seed=71)
    check(G.run_prefill(case), oracle_prefill(case), "f32", what="prefill f32")


def test_prefill_row_matches_decode_of_prefix():
    """A causal row at position m equals a decode over the prefix 0..m (GPU against GPU)."""
    pre = synth.direct_prefill(synth.DSV2, "bf16", [150], [40], seed=73)
    got = G.run_prefill(pre)
    for j in (0, 17, 39):
        m = 150 + j
        dec = synth.direct_decode(synth.DSV2, "bf16", [m + 1], seed=1)
        dec.c_rows, dec.kr_rows = pre.c_rows[:m + 1], pre.kr_rows[:m + 1]
        dec.qc, dec.qr = pre.qc[j:j + 1], pre.qr[j:j + 1]
        dec.w_uk, dec.w_uv = pre.w_uk, pre.w_uv
        d = G.run_decode(dec)
        for k in ("o", "obar"):
            G.assert_close(got[k][j:j + 1], d[k], "bf16", f"row {j} {k}", tol=OBAR_BF16_TOL if k == "obar" else None)


# ----------------------------------------------------------- full sizes ----

def test_config3_full_decode_sampled():
    case = synth.config3()
    got = G.run_decode(case)
    seqs = [0, 37, 63]
    want = oracle_decode(case, seqs=seqs[:1])
    check(got, want, "bf16", rows=seqs[:1], what="C3 materialised")
    want = oracle_decode(case, seqs=seqs, evaluate=attention.absorbed)
    check(got, want, "bf16", rows=seqs, what="C3 absorbed")
    for k in ("o", "obar", "lse"):
        assert np.all(np.isfinite(got[k]))


def test_config4_full_ragged_decode_sampled():
    case = synth.config4()
    got = G.run_decode(case)
    order = np.argsort(case.seq_lens)
    seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    want = oracle_decode(case, seqs=seqs, evaluate=attention.absorbed)
    check(got, want, "bf16", rows=seqs, what="C4")
    assert np.all(np.isfinite(got["o"]))


def test_config5_full_long_decode_sampled():
    case = synth.config5_decode()
    got = G.run_decode(case)
    want = oracle_decode(case, seqs=[2], evaluate=attention.absorbed)
    check(got, want, "bf16", rows=[2], what="C5 decode")
    assert np.all(np.isfinite(got["o"]))


def test_config5_full_prefill_sampled():
    case = synth.config5_prefill()
    got = G.run_prefill(case)
    queries = [0, 1, 1023, 2046, 2047]
    want = oracle_prefill(case, queries=queries, evaluate=attention.absorbed)
    check(got, want, "bf16", rows=queries, what="C5 prefill")
    assert np.all(np.isfinite(got["o"]))
