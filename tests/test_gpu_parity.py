"""End-to-end GPU parity: decode and prefill through the five C-ABI calls against the oracle.

The oracle's materialised form (K = [W_UK c ; R k^R], V = W_UV c, plain
softmax) is the reference wherever it finishes in seconds; for long sequences
the oracle's absorbed float64 form is used instead (pinned to the
materialised form to 1e-12 by the oracle's own tests).
"""

import numpy as np
import pytest
import torch

import bound_recipes
import cases
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


def check(got, want, dtype, rows=None, what="", name=None):
    """o and obar in the pass metric (tolerances.bound of input `name`; the configured
    bound when name is None), and lse to 2e-2 nats (1e-4 for float32)."""
    for k in ("o", "obar"):
        g = got[k] if rows is None else got[k][rows]
        G.assert_close(g, want[k], dtype, f"{what} {k}", name=name, output=k)
    g = got["lse"] if rows is None else got["lse"][rows]
    G.assert_lse_close(g, want["lse"], dtype, f"{what} lse", name=name)


def test_config1_tiny_decode_f32():
    case = synth.config1()
    check(G.run_decode(case), oracle_decode(case), "f32", what="tiny fp32 decode")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_decode_ragged(dtype):
    case = cases.tiny_decode_ragged(dtype)
    check(G.run_decode(case), oracle_decode(case), dtype, what="tiny ragged decode",
          name=None if dtype == "f32" else "tiny_decode_ragged")


@pytest.mark.parametrize("split_pages", [None, 1, 3])
def test_dsv2_decode_ragged(split_pages, monkeypatch):
    if split_pages is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", str(split_pages))
    case = cases.dsv2_decode_ragged()
    check(G.run_decode(case), oracle_decode(case), "bf16", what=f"dsv2 decode split={split_pages}",
          name="dsv2_decode_ragged")


def test_decode_empty_sequence():
    case = cases.decode_empty()
    got = G.run_decode(case)
    want = oracle_decode(case)
    assert np.all(got["obar"][[0, 2]] == 0) and np.all(np.isneginf(got["lse"][[0, 2]]))
    check(got, want, "bf16", what="decode with empty sequences", name="decode_empty")


def test_decode_score_overflow_fallback():
    """Scores that climb by far more than 2^64 within one split take the exact two-pass path."""
    case = cases.decode_overflow()
    q_t = attention.query_absorption(case.w_uk, case.qc)[0]
    s = case.shape.scale * (q_t @ case.c_rows.T.astype(np.float64))  # content part of the scores [H, T]
    rise_log2 = (s.max(axis=1) - s[:, :32].max(axis=1)) / np.log(2)
    assert rise_log2.max() > 64 + 8, "the case must push some head past the 2^64 headroom"
    check(G.run_decode(case), oracle_decode(case), "bf16", what="overflow fallback", name="decode_overflow")


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
    """Tiny causal prefill in the float32 working precision (two-term q~ and P, float32 obar)."""
    case = synth.config2()
    check(G.run_prefill(case, precise=True), oracle_prefill(case), "bf16", what="tiny causal prefill", name="c2")


def test_tiny_bf16_query_path():
    """The tiny shape in the bf16 working precision: q~, P and obar each rounded to bf16 once."""
    case = cases.tiny_prefill_short()
    got = G.run_prefill(case, precise=False)
    check(got, oracle_prefill(case), "bf16", what="tiny bf16 prefill", name="tiny_bf16_prefill")
    dec = cases.tiny_decode_short()
    check(G.run_decode(dec, precise=False), oracle_decode(dec), "bf16", what="tiny bf16 decode",
          name="tiny_bf16_decode")


@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_prefill_ragged_chunks(shape):
    case = cases.prefill_ragged(shape)
    name = "prefill_ragged_tiny" if shape is synth.TINY else "prefill_ragged_dsv2"
    check(G.run_prefill(case), oracle_prefill(case), "bf16", what=f"prefill n_h={shape.n_heads}", name=name)


def test_prefill_f32():
    case = synth.direct_prefill(synth.TINY, "f32", [10, 0], [20, 33], seed=71)
    check(G.run_prefill(case), oracle_prefill(case), "f32", what="prefill f32")


def test_prefill_row_matches_decode_of_prefix():
    """A causal row at position m equals a decode over the prefix 0..m (GPU against GPU)."""
    pre = cases.prefix_prefill()
    got = G.run_prefill(pre)
    decs = [G.run_decode(cases.prefix_decode(pre, j)) for j in cases.PREFIX_ROWS]
    for k in ("o", "obar"):
        d = np.concatenate([x[k] for x in decs])
        G.assert_close(got[k][cases.PREFIX_ROWS], d, "bf16", f"prefix rows {k}", name="prefix_rows", output=k)


# ----------------------------------------------------------- full sizes ----
# Every sequence of each configured decode workload against the absorbed
# float64 oracle (pinned to the materialised definition to 1e-12), one
# sequence against the materialised definition itself, and 78 queries of the
# prefill chunk (the first and last eight and an even stride across it).

def test_config3_full_decode():
    case = synth.config3()
    got = G.run_decode(case)
    for k in ("o", "obar", "lse"):
        assert np.all(np.isfinite(got[k]))
    check(got, oracle_decode(case, seqs=[37]), "bf16", rows=[37], what="C3 materialised", name="c3")
    check(got, oracle_decode(case, evaluate=attention.absorbed), "bf16", what="C3 all sequences", name="c3")


def test_config4_full_ragged_decode():
    """32 of the 128 sequences, evenly spaced in length order (the shortest and the longest among them)."""
    case = synth.config4()
    got = G.run_decode(case)
    assert np.all(np.isfinite(got["o"]))
    seqs = bound_recipes.c4_sequences(case)
    shortest = seqs[0]
    check(got, oracle_decode(case, seqs=[shortest]), "bf16", rows=[shortest], what="C4 materialised", name="c4")
    check(got, oracle_decode(case, seqs=seqs, evaluate=attention.absorbed), "bf16", rows=seqs,
          what=f"C4 {len(seqs)} sequences", name="c4")


def test_config5_full_long_decode():
    case = synth.config5_decode()
    got = G.run_decode(case)
    assert np.all(np.isfinite(got["o"]))
    check(got, oracle_decode(case, evaluate=attention.absorbed), "bf16", what="C5 decode all sequences", name="c5a")


def test_config5_full_prefill():
    case = synth.config5_prefill()
    got = G.run_prefill(case)
    assert np.all(np.isfinite(got["o"]))
    queries = bound_recipes.c5b_queries()
    want = oracle_prefill(case, queries=queries, evaluate=attention.absorbed)
    check(got, want, "bf16", rows=queries, what=f"C5 prefill {len(queries)} queries", name="c5b")
