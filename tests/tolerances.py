"""Pass bounds of the GPU parity tests, and the rounding-model figures behind them.

The metric is the one the configured workloads are stated in: over the whole
output o of a test (every query, head and column),

    rel_max = max |o_gpu - o_oracle| / rms(o_oracle)
    rel_rms = rms(o_gpu - o_oracle) / rms(o_oracle),

bounded by 1e-4 for float32 workloads and by 2e-2 (max) and 5e-3 (rms) for
bf16 workloads.  Those bounds hold for every configured workload.

Test inputs outside the configured workloads -- sequences of a handful of
keys, causal chunks that start at position 0 at the DeepSeek-V2 shape, the
two-scale score, layers formed from hidden states -- can need more: rows
averaging few keys are an order of magnitude larger than rows averaging
thousands, so one rounding in such a row is large against the whole output's
RMS.  For every test the storage-rounding model (``rounding_model.py``: the
oracle's float64 arithmetic with a round-to-nearest-even cast at each point
where the library stores or feeds a value at reduced precision) predicts the
error on that test's own inputs.  ``MODEL`` records what
``bound_recipes.py`` prints for it, and ``bound()`` returns the configured
bound, or 1.25 x the model's figure (rounded up to two digits) where that is
larger.  ``test_rounding_bounds.py`` recomputes every figure on the CPU.
lse is held in absolute nats: 2e-2 (max) and 5e-3 (rms) for bf16, widened the
same way where scores are large (a rounding of q~ moves a score of s nats by
up to ~2^-8 s).
"""

from __future__ import annotations

import math

CONFIGURED = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 5e-3)}
# lse (log of the softmax denominator) in absolute nats: max and rms error.
CONFIGURED_LSE = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 5e-3)}
MARGIN = 1.25

# name -> {output: (model rel_max, model rel_rms)}, as `python tests/bound_recipes.py [--full]` prints them.
MODEL = {
    "tiny_decode_ragged": {"o": (2.442e-03, 2.550e-04), "obar": (2.426e-03, 2.591e-04), "lse": (4.902e-04, 1.044e-04)},
    "dsv2_decode_ragged": {"o": (8.224e-03, 6.792e-04), "obar": (7.925e-03, 6.856e-04), "lse": (3.997e-03, 6.345e-04)},
    "decode_proj_many": {"o": (2.960e-02, 2.149e-03), "obar": (3.823e-02, 2.146e-03), "lse": (1.854e-03, 2.952e-04)},
    "decode_empty": {"o": (2.074e-02, 1.650e-03), "obar": (2.642e-02, 1.664e-03), "lse": (2.936e-03, 7.642e-04)},
    "decode_overflow": {"o": (8.885e-03, 6.323e-04), "obar": (9.830e-03, 6.401e-04), "lse": (8.881e-02, 3.187e-02)},
    "tiny_bf16_prefill": {"o": (2.546e-02, 1.906e-03), "obar": (2.161e-02, 1.917e-03), "lse": (4.161e-03, 4.352e-04)},
    "tiny_bf16_decode": {"o": (4.236e-03, 5.110e-04), "obar": (5.469e-03, 5.150e-04), "lse": (2.742e-03, 8.801e-04)},
    "prefill_ragged_dsv2": {"o": (3.140e-02, 1.889e-03), "obar": (3.546e-02, 1.894e-03), "lse": (3.657e-03, 4.324e-04)},
    "prefill_ragged_tiny": {"o": (7.747e-03, 5.379e-04), "obar": (9.251e-03, 5.403e-04), "lse": (1.362e-03, 1.487e-04)},
    "mha_ragged_dsv2": {"o": (2.429e-02, 1.070e-03), "lse": (3.238e-03, 2.963e-04)},
    "mha_ragged_tiny": {"o": (1.039e-02, 8.026e-04), "lse": (1.695e-03, 2.363e-04)},
    "mha_long_prefix": {"o": (1.790e-02, 1.197e-03), "lse": (7.513e-04, 1.432e-04)},
    "mha_vs_absorbed": {"o": (5.288e-02, 3.749e-03)},
    "prefix_rows": {"o": (2.912e-02, 4.723e-03), "obar": (3.691e-02, 4.718e-03)},
    "mha_c2": {"o": (2.139e-02, 8.433e-04), "lse": (2.765e-03, 1.586e-04)},
    "two_scale_decode_tiny": {"o": (7.714e-03, 7.013e-04), "obar": (8.611e-03, 7.025e-04), "lse": (1.752e-03, 4.440e-04)},
    "two_scale_decode_dsv2": {"o": (1.563e-02, 1.212e-03), "obar": (1.971e-02, 1.200e-03), "lse": (6.699e-03, 1.375e-03)},
    "two_scale_prefill_tiny": {"o": (2.564e-02, 1.263e-03), "obar": (2.741e-02, 1.268e-03), "lse": (4.418e-03, 4.807e-04)},
    "two_scale_prefill_dsv2": {"o": (3.981e-02, 2.454e-03), "obar": (5.513e-02, 2.453e-03), "lse": (8.043e-03, 8.663e-04)},
    "two_scale_mha_tiny": {"o": (2.828e-02, 1.844e-03), "lse": (5.723e-03, 8.130e-04)},
    "two_scale_mha_dsv2": {"o": (2.998e-02, 1.780e-03), "lse": (8.377e-03, 7.371e-04)},
    "per_head_f32w": {"o": (2.276e-03, 2.556e-04), "obar": (2.069e-03, 2.541e-04), "lse": (5.217e-04, 1.186e-04)},
    "per_head_bf16": {"o": (6.300e-03, 8.573e-04), "obar": (5.808e-03, 8.576e-04), "lse": (3.576e-03, 6.544e-04)},
    "per_head_two_scale": {"o": (5.978e-03, 9.444e-04), "obar": (6.303e-03, 9.337e-04), "lse": (2.420e-03, 8.889e-04)},
    "front_decode_tiny_unfolded": {"o": (1.106e-02, 1.954e-03), "lse": (6.233e-03, 1.589e-03)},
    "front_decode_tiny_folded": {"o": (1.106e-02, 1.949e-03), "lse": (5.387e-03, 1.444e-03)},
    "front_decode_dsv2_unfolded": {"o": (1.329e-02, 1.799e-03), "lse": (8.815e-03, 1.590e-03)},
    "front_decode_dsv2_folded": {"o": (1.329e-02, 1.798e-03), "lse": (8.503e-03, 1.514e-03)},
    "front_prefill_tiny_unfolded": {"o": (3.455e-02, 3.145e-03), "lse": (6.795e-03, 1.029e-03)},
    "front_prefill_tiny_folded": {"o": (3.652e-02, 3.177e-03), "lse": (8.468e-03, 9.946e-04)},
    "front_prefill_dsv2_unfolded": {"o": (4.095e-02, 3.200e-03), "lse": (1.231e-02, 9.670e-04)},
    "front_prefill_dsv2_folded": {"o": (3.865e-02, 3.188e-03), "lse": (8.899e-03, 9.649e-04)},
    "c2": {"o": (1.768e-02, 5.573e-04), "obar": (1.801e-02, 5.585e-04), "lse": (2.014e-03, 8.533e-05)},
}

# Full-size workloads (minutes of CPU each; `python tests/bound_recipes.py --full`).
MODEL_FULL = {
    "c3": {"o": (1.390e-02, 2.013e-03), "obar": (1.589e-02, 2.014e-03), "lse": (6.640e-04, 1.541e-04)},
    "c4": {"o": (1.883e-02, 1.862e-03), "obar": (2.190e-02, 1.860e-03), "lse": (5.753e-04, 1.501e-04)},
    "c5a": {"o": (7.720e-03, 1.684e-03), "obar": (1.410e-02, 1.673e-03), "lse": (4.514e-04, 1.490e-04)},
    "c5b": {"o": (9.962e-03, 1.779e-03), "obar": (1.792e-02, 1.779e-03), "lse": (6.248e-04, 1.481e-04)},
    "c5b_mha": {"o": (3.202e-03, 4.684e-04), "lse": (5.062e-04, 1.209e-04)},
    "per_head_full": {"o": (2.196e-03, 3.254e-04), "obar": (2.447e-03, 3.261e-04), "lse": (8.292e-05, 1.970e-05)},
}


def _up(x: float) -> float:
    """Round up to two significant digits."""
    if x <= 0:
        return 0.0
    e = math.floor(math.log10(x)) - 1
    return math.ceil(x / 10 ** e - 1e-9) * 10 ** e


def figure(name: str, output: str = "o"):
    fig = (MODEL.get(name) or MODEL_FULL[name])[output]
    return fig


# The configured workloads: their layer output o is held to the configured
# bound itself, never widened (the model's figure must sit below it).
CONFIGURED_WORKLOADS = ("c2", "c3", "c4", "c5a", "c5b")


def bound(name: str | None, output: str = "o", dtype: str = "bf16"):
    """(max, rms) a GPU test holds `output` of input `name` to: the configured bound of
    `dtype`, widened to MARGIN x the model's figure where the model predicts more --
    except for the layer output o of a configured workload, which keeps the configured bound."""
    mx, rms = (CONFIGURED_LSE if output == "lse" else CONFIGURED)[dtype]
    if name is None or (name in CONFIGURED_WORKLOADS and output == "o"):
        return mx, rms
    fm, fr = figure(name, output)
    return max(mx, _up(MARGIN * fm)), max(rms, _up(MARGIN * fr))
