"""GPU parity of the materialised-form prefill (mla_prefill_mha) against the oracle.

The oracle's materialised definition (K = [W_UK c ; R k^R], V = W_UV c, plain
softmax) is the reference at small sizes; at the full 2048-after-16384 chunk
sampled queries are checked against the oracle's absorbed float64 form
(pinned to the materialised form to 1e-12 by the oracle's own tests).  This
path rounds the up-projected keys and values, the content query and the
softmax weights to float16; each test is held to the configured bf16 bound,
widened only where the storage-rounding model predicts more for its inputs
(tests/tolerances.py).
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


def oracle_prefill(case, queries=None, evaluate=attention.materialised):
    return attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                                   case.qr, case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base,
                                   queries=queries, evaluate=evaluate)


def check(got, want, rows=None, what="", name=None):
    g = got["o"] if rows is None else got["o"][rows]
    G.assert_close(g, want["o"], "bf16", f"{what} o", name=name)
    g = got["lse"] if rows is None else got["lse"][rows]
    G.assert_lse_close(g, want["lse"], "bf16", f"{what} lse", name=name)


@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_mha_prefill_ragged_chunks(shape):
    """Chunks of 5, 130, 1 and 64 queries after 0, 100, 64 and 7 cached tokens (several key and query blocks,
    ragged tails, a chunk that starts a sequence)."""
    case = cases.prefill_ragged(shape)
    check(G.run_prefill_mha(case), oracle_prefill(case), what=f"materialised prefill n_h={shape.n_heads}",
          name="mha_ragged_tiny" if shape is synth.TINY else "mha_ragged_dsv2")


def test_mha_prefill_long_prefix_and_empty_chunk():
    """A chunk of 300 after 700 cached tokens next to an empty chunk (no queries, keys still up-projected)."""
    case = cases.mha_long_prefix()
    got = G.run_prefill_mha(case)
    check(got, oracle_prefill(case), what="long prefix", name="mha_long_prefix")
    assert np.all(np.isfinite(got["o"]))


def test_mha_prefill_matches_absorbed_path():
    """The two forms of the same chunk agree (each against the other's output) within the sum
    of what the rounding model predicts for each form against the oracle."""
    case = cases.mha_vs_absorbed()
    cache = G.build_cache(case)
    a = G.run_prefill(case, cache=cache)
    m = G.run_prefill_mha(case, cache=cache)
    G.assert_close(m["o"], a["o"], "bf16", "materialised vs absorbed o", name="mha_vs_absorbed")


def test_mha_prefill_bitwise_repeatable():
    case = synth.direct_prefill(synth.DSV2, "bf16", [64, 0], [70, 33], seed=97)
    cache = G.build_cache(case)
    a = G.run_prefill_mha(case, cache=cache)
    b = G.run_prefill_mha(case, cache=cache)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_mha_config2_tiny_prefill():
    case = synth.config2()
    check(G.run_prefill_mha(case), oracle_prefill(case), what="C2 materialised", name="mha_c2")


def test_mha_config5_full_prefill_sampled():
    case = synth.config5_prefill()
    got = G.run_prefill_mha(case)
    queries = bound_recipes.c5b_queries()
    want = oracle_prefill(case, queries=queries, evaluate=attention.absorbed)
    check(got, want, rows=queries, what=f"C5 materialised, {len(queries)} queries", name="c5b_mha")
    assert np.all(np.isfinite(got["o"]))


def test_mha_workspace_is_checked():
    case = synth.direct_prefill(synth.DSV2, "bf16", [10], [20], seed=101)
    dims = G.dims_of(case, precise=False)
    cu, st = torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start)
    need = mla.prefill_mha_workspace_size(dims, cu, st)
    assert need == 2 * 128 * 128 * 128 * 2  # keys and values of 30 positions, padded to 128, float16
    cache = G.build_cache(case)
    step = mla.PrefillStep(dims, cache, cu, st)
    step.mha_workspace = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MLAError):
        step.run_materialised(G.dev(case.qc, torch.bfloat16), G.dev(case.qr, torch.bfloat16),
                              G.dev(case.w_uk, torch.bfloat16), G.dev(case.w_uv, torch.bfloat16))


def test_mha_prefill_flags_float16_overflow():
    """A head whose up-projected keys leave float16 range comes out NaN (never finite and wrong);
    the other heads are untouched, bit for bit."""
    import dataclasses

    case = synth.direct_prefill(synth.TINY, "bf16", [9], [23], seed=131)
    cache = G.build_cache(case)
    base = G.run_prefill_mha(case, cache=cache)
    h = 2
    # scale head h's W_UK so that key 0's largest content-key element is twice float16's overflow point
    k0 = case.w_uk[h] @ case.c_rows[0]
    w_uk = case.w_uk.copy()
    w_uk[h] *= 2 * 65520.0 / np.max(np.abs(k0))
    big = G.run_prefill_mha(dataclasses.replace(case, w_uk=w_uk), cache=cache)
    assert np.all(np.isnan(big["o"][:, h])) and np.all(np.isnan(big["lse"][:, h]))
    others = [i for i in range(case.shape.n_heads) if i != h]
    assert np.array_equal(big["o"][:, others], base["o"][:, others])
    assert np.array_equal(big["lse"][:, others], base["lse"][:, others])
