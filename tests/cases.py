"""Named test inputs shared by the GPU parity tests and the CPU check of their bounds.

Each builder returns a ``synth`` case (seeded, synthetic); the GPU test runs
the library on it and the CPU test runs the storage-rounding model on the
very same inputs.  Nothing here computes attention.
"""

from __future__ import annotations

import numpy as np

import synth
from oracle import attention


def tiny_decode_ragged(dtype="bf16"):
    return synth.direct_decode(synth.TINY, dtype, [1, 63, 64, 65, 300, 1000, 129], seed=41, shuffle=True)


def dsv2_decode_ragged():
    return synth.direct_decode(synth.DSV2, "bf16", [1, 64, 65, 700, 2048, 130], seed=43, shuffle=True)


def decode_empty():
    """Empty sequences between short ones (DeepSeek-V2 shape)."""
    return synth.direct_decode(synth.DSV2, "bf16", [0, 5, 0, 70], seed=47)


def decode_proj_many():
    """150 sequences of 0 .. 901 keys (several 64-sequence blocks, a ragged last group
    of 16), shuffled pages: the fused decode and output absorption."""
    lens = [(37 * i) % 900 + (i % 3) for i in range(150)]
    return synth.direct_decode(synth.DSV2, "bf16", lens, seed=313, shuffle=True)


DECODE_PROJ_MANY_ROWS = list(range(0, 150, 7))


def decode_overflow():
    """Scores that climb by far more than 2^64 within one split (DeepSeek-V2 shape, 600 tokens).

    Later tokens' latents are pushed along the mean absorbed query direction,
    so the scores rise by tens of nats over the sequence."""
    case = synth.direct_decode(synth.DSV2, "bf16", [600], seed=53)
    q_t = attention.query_absorption(case.w_uk, case.qc)[0]  # [H, d_c]
    direction = q_t.mean(axis=0)
    direction /= np.linalg.norm(direction)
    grow = np.linspace(0, 60, 600)[:, None]
    case.c_rows = synth.to_storage(case.c_rows + grow * direction[None, :] * 8, "bf16")
    return case


PREFIX_ROWS = [0, 17, 39]


def prefix_prefill():
    """A 40-query chunk after 150 cached tokens (DeepSeek-V2 shape); rows PREFIX_ROWS are
    compared with decodes of their prefixes."""
    return synth.direct_prefill(synth.DSV2, "bf16", [150], [40], seed=73)


def prefix_decode(pre, j):
    """Decode of the prefix 0 .. 150 + j of `pre` with query j of the chunk."""
    m = int(pre.q_start[0]) + j
    dec = synth.direct_decode(synth.DSV2, "bf16", [m + 1], seed=1)
    dec.c_rows, dec.kr_rows = pre.c_rows[:m + 1], pre.kr_rows[:m + 1]
    dec.qc, dec.qr = pre.qc[j:j + 1], pre.qr[j:j + 1]
    dec.w_uk, dec.w_uv = pre.w_uk, pre.w_uv
    return dec


def tiny_prefill_short():
    return synth.direct_prefill(synth.TINY, "bf16", [0, 30], [200, 64], seed=79)


def tiny_decode_short():
    return synth.direct_decode(synth.TINY, "bf16", [1, 77, 640], seed=83)


def prefill_ragged(shape):
    """Chunks of 5, 130, 1 and 64 queries after 0, 100, 64 and 7 cached tokens, shuffled pages."""
    return synth.direct_prefill(shape, "bf16", [0, 100, 64, 7], [5, 130, 1, 64], seed=67, shuffle=True)


def mha_long_prefix():
    return synth.direct_prefill(synth.DSV2, "bf16", [700, 50], [300, 0], seed=83, shuffle=True)


def mha_vs_absorbed():
    return synth.direct_prefill(synth.DSV2, "bf16", [200], [96], seed=89)


def two_scale_decode(shape, dtype):
    return synth.direct_decode(shape, dtype, [1, 64, 65, 700, 129], seed=201, shuffle=True)


def two_scale_prefill(shape):
    return synth.direct_prefill(shape, "bf16", [0, 100, 7], [5, 130, 64], seed=203, shuffle=True)


def two_scale_prefill_materialised(shape):
    return synth.direct_prefill(shape, "bf16", [0, 100, 7], [5, 130, 64], seed=205, shuffle=True)


def per_head_decode():
    return synth.direct_decode(synth.TINY, "bf16", [1, 63, 64, 65, 300, 0, 1000, 129], seed=213, shuffle=True,
                               per_head_rope=True)


def per_head_two_scale():
    return synth.direct_decode(synth.TINY, "bf16", [77, 640, 5], seed=215, shuffle=True, per_head_rope=True)


def per_head_full():
    return synth.direct_decode(synth.TINY, "bf16", [4096] * 64, seed=219, shuffle=True, per_head_rope=True)


# the front of the layer: (shape, d_model, d_qlat) at both shapes
FRONT_SMALL = {"tiny": (synth.TINY, 256, 96), "dsv2": (synth.DSV2, 512, 192)}
FRONT_DECODE_LENS = [130, 1, 64, 200]
FRONT_PREFILL = ([100, 0, 64], [30, 77, 1])  # (prior, new) per sequence


def front_decode(name):
    shape, d_model, d_qlat = FRONT_SMALL[name]
    return synth.front_layer(shape, FRONT_DECODE_LENS, d_model, d_qlat, seed=19, shuffle=True)


def front_prefill(name):
    shape, d_model, d_qlat = FRONT_SMALL[name]
    prior, new = FRONT_PREFILL
    lens = [p_ + n_ for p_, n_ in zip(prior, new)]
    return synth.front_layer(shape, lens, d_model, d_qlat, seed=23, shuffle=True)
