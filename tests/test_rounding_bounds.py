"""CPU checks of the storage-rounding model and of the GPU tests' bounds.

* The model with every cast switched off is the oracle's absorbed evaluation,
  and each cast is pinned against a library rounding (torch's bf16 cast,
  numpy's float16 cast) and its closed-form error bound.
* Every figure recorded in tests/tolerances.py is what the model gives for
  that test's inputs now (recomputed here; the full-size figures only with
  MLA_FULL_MODEL=1, since they take minutes).
* Every bound a GPU test asserts is at least 1.25 x the model's figure, and
  every bound name a GPU test uses has a figure.
"""

import math
import os
import re

import numpy as np
import pytest
import torch

import bound_recipes
import rounding_model as R
import synth
import tolerances as T
from oracle import attention

HERE = os.path.dirname(os.path.abspath(__file__))


def test_casts_against_library_roundings():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000) * np.exp(rng.uniform(-20, 20, 10000))
    want_bf16 = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(R.bf16(x), want_bf16)
    assert np.array_equal(R.f16(x[:100] * 1e-3), (x[:100] * 1e-3).astype(np.float32).astype(np.float16).astype(np.float64))
    # ties to even: 1 + 2^-8 lies half way between 1 and 1 + 2^-7
    assert R.bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert R.bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # one rounding to 8 significant bits: at most half a spacing, 2^-8 relative; two
    # terms: the lo term's own rounding, at most 2^-16 relative (plus float32's 2^-24)
    y = rng.standard_normal(10000)
    assert np.all(np.abs(R.bf16(y) - y) <= 2.0 ** -8 * np.abs(y) * (1 + 2.0 ** -16))
    assert np.all(np.abs(R.two_term(y) - y) <= (2.0 ** -16 + 2.0 ** -24) * np.abs(y))


def test_scaled_float16_partials():
    """f16q: each group of 128 columns is scaled by 2^-e (e the frexp exponent of its largest
    magnitude), rounded to float16 and scaled back -- checked against numpy's float16 on each
    group one by one, and against float16's error bound relative to the group's largest value."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 256)) * np.exp(rng.uniform(-30, 30, (3, 5, 1)))
    x[0, 0, :128] = 0.0  # an all-zero group stays zero
    got = R.f16_scaled(x)
    for i in range(3):
        for j in range(5):
            for g in range(2):
                v = x[i, j, 128 * g:128 * (g + 1)].astype(np.float32).astype(np.float64)
                mx = np.max(np.abs(v))
                e = math.frexp(mx)[1] if mx > 0 else 0
                want = (v / 2.0 ** e).astype(np.float16).astype(np.float64) * 2.0 ** e
                assert np.array_equal(got[i, j, 128 * g:128 * (g + 1)], want)
                assert np.all(np.abs(want - v) <= 2.0 ** -11 * mx)
    assert np.all(got[0, 0, :128] == 0)


def test_all_partials_stores_a_single_range():
    """all_partials (the fused decode and output absorption): with float32 partials a
    single range is unchanged (obar is float32 either way); with f16q its obar moves by
    at most float16's bound against each 128-column group's largest value, and the
    split ranges, which already went through partials, do not move at all."""
    case = synth.direct_decode(synth.DSV2, "bf16", [40, 130], seed=411)
    base = R.decode_batch(case, **bound_recipes.BF16)
    assert all(np.array_equal(R.decode_batch(case, all_partials=True, **bound_recipes.BF16)[k], base[k])
               for k in base)
    f16q = dict(bound_recipes.BF16, partial="f16q")
    a = R.decode_batch(case, **f16q)
    b = R.decode_batch(case, all_partials=True, **f16q)
    ob, ob0 = b["obar"].reshape(2, -1, 4, 128), a["obar"].reshape(2, -1, 4, 128)
    mx = np.max(np.abs(ob0), axis=-1, keepdims=True)
    assert np.all(np.abs(ob - ob0) <= 2.0 ** -11 * mx) and not np.array_equal(ob, ob0)
    split = R.decode_batch(case, split_keys=64, **f16q)  # 40 keys: one range; 130 keys: three
    fused = R.decode_batch(case, split_keys=64, all_partials=True, **f16q)
    assert np.array_equal(fused["o"][1], split["o"][1]) and not np.array_equal(fused["o"][0], split["o"][0])


@pytest.mark.parametrize("causal", [False, True])
def test_model_without_casts_is_the_oracle(causal):
    case = synth.direct_prefill(synth.TINY, "bf16", [9], [23], seed=3) if causal else \
        synth.direct_decode(synth.TINY, "bf16", [40], seed=3)
    t = int(case.seq_lens[0])
    q_pos = case.q_pos
    exact = dict(q_lat="exact", p="exact", obar="f32", partial="exact", key_cast="exact")
    want = attention.absorbed(case.qc, case.qr, q_pos, case.c_rows[:t], case.kr_rows[:t], case.w_uk, case.w_uv,
                              case.shape.scale, causal=causal)
    for split in (None, 16):
        got = R.absorbed(case.qc, case.qr, q_pos, case.c_rows[:t], case.kr_rows[:t], case.w_uk, case.w_uv,
                         case.shape.scale, causal=causal, split_keys=None if causal else split, **exact)
        for k in ("o", "obar"):
            # obar="f32" and the float32 output cast are the only roundings left
            assert np.max(np.abs(got[k] - want[k])) <= 2.0 ** -23 * np.max(np.abs(want[k])), k
        fin = np.isfinite(want["lse"])
        # splits merge with float32 weights, as the kernels do
        assert np.max(np.abs(got["lse"][fin] - want["lse"][fin])) <= (1e-12 if split is None else 1e-6)
    m = R.materialised(case.qc, case.qr, q_pos, case.c_rows[:t], case.kr_rows[:t], case.w_uk, case.w_uv,
                       case.shape.scale, causal=causal, kv="exact", p="exact", rot="exact")
    assert np.max(np.abs(m["o"] - want["o"])) <= 2.0 ** -23 * np.max(np.abs(want["o"]))


def test_model_casts_move_the_result():
    """Each cast point, switched on alone, changes the output (a dropped cast would not)."""
    case = synth.direct_decode(synth.DSV2, "bf16", [300], seed=9)
    base = dict(q_lat="exact", p="exact", obar="f32", partial="exact", key_cast="exact")
    ref = R.decode_batch(case, **base)["o"]
    for k, v in (("q_lat", "bf16"), ("p", "bf16"), ("obar", "bf16"), ("key_cast", "bf16")):
        got = R.decode_batch(case, **dict(base, **{k: v}))["o"]
        assert np.max(np.abs(got - ref)) > 1e-6 * np.max(np.abs(ref)), k


@pytest.mark.parametrize("name", sorted(T.MODEL))
def test_recorded_figures_match_the_model(name):
    figs = bound_recipes.figure(name)
    assert set(figs) == set(T.MODEL[name]), name
    for out, (fm, fr) in figs.items():
        rm, rr = T.MODEL[name][out]
        print(f"{name}.{out}: model max {fm:.3e} rms {fr:.3e}; bound {T.bound(name, out)}")
        assert math.isclose(fm, rm, rel_tol=0.01) and math.isclose(fr, rr, rel_tol=0.01), (name, out, fm, fr)


@pytest.mark.skipif(os.environ.get("MLA_FULL_MODEL") != "1", reason="full-size figures take minutes: MLA_FULL_MODEL=1")
@pytest.mark.parametrize("name", sorted(T.MODEL_FULL))
def test_recorded_full_size_figures_match_the_model(name):
    figs = bound_recipes.figure(name)
    for out, (fm, fr) in figs.items():
        rm, rr = T.MODEL_FULL[name][out]
        assert math.isclose(fm, rm, rel_tol=0.01) and math.isclose(fr, rr, rel_tol=0.01), (name, out, fm, fr)


def test_bounds_cover_the_model_with_margin():
    for table in (T.MODEL, T.MODEL_FULL):
        for name, outs in table.items():
            for out, (fm, fr) in outs.items():
                bm, br = T.bound(name, out)
                assert bm >= T.CONFIGURED["bf16"][0] and br >= T.CONFIGURED["bf16"][1], (name, out)
                if name in T.CONFIGURED_WORKLOADS and out == "o":
                    # a configured workload: the model must predict a pass of the configured bound
                    assert (bm, br) == T.CONFIGURED["bf16"] and fm < bm and fr < br, (name, fm, fr)
                else:
                    # (the bound is MARGIN x figure rounded up to two digits, with the 1e-9
                    # slack tolerances._up takes against float noise)
                    slack = 1 - 1e-9
                    assert bm >= T.MARGIN * fm * slack and br >= T.MARGIN * fr * slack, (name, out)


def test_every_bound_name_has_a_figure():
    names = set()
    for fn in os.listdir(HERE):
        if fn.startswith("test_gpu_") and fn.endswith(".py"):
            src = open(os.path.join(HERE, fn)).read()
            names |= set(re.findall(r'name="([a-z0-9_]+)"', src))
            names |= {m.replace("{", "").replace("}", "") for m in re.findall(r'f"([a-z0-9_]+)_\{', src)}
    known = set(T.MODEL) | set(T.MODEL_FULL)
    literal = {n for n in names if "_" in n and not n.endswith("_")}
    missing = sorted(n for n in literal if n not in known and not any(k.startswith(n) for k in known))
    assert not missing, missing
