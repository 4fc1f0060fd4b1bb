"""The storage-rounding model evaluated on each GPU test's own inputs (CPU, test infrastructure).

``figure(name)`` returns the model's (max, rms) error against the float64
oracle, in the pass metric (max|err| / rms(want) and rms(err) / rms(want) over
the whole output), for the test input and output that ``name`` stands for.
``tests/tolerances.py`` records these figures next to the bounds the GPU tests
use, and ``test_rounding_bounds.py`` recomputes them.

Run ``python tests/bound_recipes.py [--full]`` to print every figure (the
full-size ones take minutes).
"""

from __future__ import annotations

import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (_HERE, os.path.dirname(_HERE)):
    if _p not in sys.path:
        sys.path.insert(0, _p)

import cases  # noqa: E402
import rounding_model as R  # noqa: E402
import synth  # noqa: E402
from oracle import attention, front  # noqa: E402

# The library's working precisions.  obar and the split partials are float32
# on every path; q~ (with the rotated query) and the softmax weights P are
# bf16, or two-term bf16 splits in the float32 working precision of the
# small shape.
BF16 = dict(q_lat="bf16", p="bf16", obar="f32", partial="f32")
F32W = dict(q_lat="f32", p="two_term", obar="f32", partial="f32")
# The shared-key decode at d_c = 512 in bf16 keeps its split partials as float16
# scaled per 128 columns (the other shapes and working precisions keep float32).
BF16_DC512_DECODE = dict(BF16, partial="f16q")


def _decode_prec(prec, shape):
    return BF16_DC512_DECODE if (prec is BF16 and shape.d_latent == 512) else prec
# Decode splits follow the library's plan, which the model does not know: it
# takes the worst over one range per sequence and splits of 1, 2, 3, 4, 8 and 16
# pages (each split rounds against its own reference maximum).
SPLITS = (None, 64, 128, 192, 256, 512, 1024)


def _oracle_decode(case, evaluate=attention.materialised, seqs=None, position_scale=None, scale=None):
    return attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, case.shape.scale if scale is None else scale,
                                  case.shape.rope_base, seqs=seqs, evaluate=evaluate, position_scale=position_scale)


def _oracle_prefill(case, evaluate=attention.materialised, queries=None, position_scale=None, scale=None):
    return attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                                   case.qr, case.w_uk, case.w_uv, case.shape.scale if scale is None else scale,
                                   case.shape.rope_base, queries=queries, evaluate=evaluate,
                                   position_scale=position_scale)


def _worst(results, want, key):
    err = R.lse_errors if key == "lse" else R.errors
    figs = [err(r[key], want[key]) for r in results]
    return max(f[0] for f in figs), max(f[1] for f in figs)


def _decode_figures(case, prec, want=None, seqs=None, scales=None, fused=False):
    """Worst over the split lengths of the model against the oracle; ``fused``: the
    decode with the merge and output absorption in one launch (every range stored
    as a partial)."""
    prec = _decode_prec(prec, case.shape)
    kw = dict(prec, all_partials=True) if fused else dict(prec)
    if scales is not None:
        kw["position_scale"] = scales[1]
    want = want if want is not None else _oracle_decode(
        case, seqs=seqs, position_scale=None if scales is None else scales[1],
        scale=None if scales is None else scales[0])
    got = []
    for split in SPLITS:
        if scales is not None:  # the model takes one scale argument: rebuild the call
            got.append(_model_decode_scaled(case, scales, split, prec, seqs))
        else:
            got.append(R.decode_batch(case, seqs=seqs, split_keys=split, **kw))
    return {k: _worst(got, want, k) for k in ("o", "obar", "lse")}


def _model_decode_scaled(case, scales, split, prec, seqs=None):
    seqs = range(case.batch) if seqs is None else seqs
    outs = []
    for b in seqs:
        t = int(case.seq_lens[b])
        r0 = int(case.row_offsets[b])
        outs.append(R.absorbed(case.qc[b:b + 1], case.qr[b:b + 1], np.array([t - 1]), case.c_rows[r0:r0 + t],
                               case.kr_rows[r0:r0 + t], case.w_uk, case.w_uv, scales[0], case.shape.rope_base,
                               split_keys=split, position_scale=scales[1], **prec))
    return {k: np.concatenate([r[k] for r in outs], axis=0) for k in ("o", "obar", "lse")}


def _prefill_figures(case, prec, form="absorbed", queries=None, want=None, scales=None):
    kw = dict(prec) if form == "absorbed" else {}
    if scales is not None:
        kw["position_scale"] = scales[1]
    want = want if want is not None else _oracle_prefill(
        case, queries=queries, position_scale=None if scales is None else scales[1],
        scale=None if scales is None else scales[0])
    if scales is not None:
        got = _model_prefill_scaled(case, scales, form, kw, queries)
    else:
        got = R.prefill_batch(case, form=form, queries=queries, **kw)
    return {k: (R.lse_errors if k == "lse" else R.errors)(got[k], want[k]) for k in got if k in ("o", "obar", "lse")}


def _model_prefill_scaled(case, scales, form, kw, queries=None):
    fn = R.absorbed if form == "absorbed" else R.materialised
    want_q = np.arange(case.cu_q[-1]) if queries is None else np.asarray(queries)
    outs = {}
    for b in range(case.batch):
        sel = want_q[(want_q >= case.cu_q[b]) & (want_q < case.cu_q[b + 1])]
        if len(sel) == 0:
            continue
        pos = int(case.q_start[b]) + (sel - case.cu_q[b])
        t = int(pos.max()) + 1
        r0 = int(case.row_offsets[b])
        res = fn(case.qc[sel], case.qr[sel], pos, case.c_rows[r0:r0 + t], case.kr_rows[r0:r0 + t], case.w_uk,
                 case.w_uv, scales[0], case.shape.rope_base, causal=True, **kw)
        for i, g in enumerate(sel):
            outs[int(g)] = {k: res[k][i] for k in res}
    keys = [k for k in next(iter(outs.values())) if k in ("o", "obar", "lse")]
    return {k: np.stack([outs[int(g)][k] for g in want_q]) for k in keys}


def _two_scales(shape):
    return 1.0 / np.sqrt(shape.d_head), 1.0 / np.sqrt(shape.d_rope)


# ---- the front of the layer: the model's inputs carry the front's own roundings

def _front_inputs(fc, rows_q, folded):
    """c, k^R (exact, rotated and rounded by the model), q^C, q^R and q~ as the GPU forms them:
    c = bf16(W_DKV h); c^Q = bf16(W_DQ h); q^C = bf16(W_UQ c^Q); q^R = W_QR c^Q (rotated,
    then rounded by the model); folded: q~ = W_fold c^Q with W_fold = bf16(W_UK^T W_UQ)."""
    c = R.bf16(front.kv_latent(fc.h, fc.w_dkv))
    kr = front.position_key(fc.h, fc.w_kr)
    cq = R.bf16(front.query_latent(fc.h[rows_q], fc.w_dq))
    qr = front.position_query(cq, fc.w_qr)
    if folded:
        w_fold = R.bf16(front.fold_query_weights(fc.w_uq, fc.w_uk))
        return c, kr, None, qr, front.folded_query(cq, w_fold)
    return c, kr, R.bf16(front.content_query(cq, fc.w_uq)), qr, None


def _front_oracle_inputs(fc, rows_q):
    cq = front.query_latent(fc.h[rows_q], fc.w_dq)
    return (front.kv_latent(fc.h, fc.w_dkv), front.position_key(fc.h, fc.w_kr), front.content_query(cq, fc.w_uq),
            front.position_query(cq, fc.w_qr))


def _front_decode_figures(name, folded):
    fc = cases.front_decode(name)
    lens = np.asarray(cases.FRONT_DECODE_LENS, np.int32)
    last = fc.row_offsets + lens - 1
    s = fc.shape
    c, kr, qc, qr, q_t = _front_inputs(fc, last, folded)
    oc, okr, oqc, oqr = _front_oracle_inputs(fc, last)
    want = attention.decode_batch(lens, oc, okr, fc.row_offsets, oqc, oqr, fc.w_uk, fc.w_uv, s.scale)
    got = []
    for split in SPLITS:
        outs = []
        for b in range(len(lens)):
            t, r0 = int(lens[b]), int(fc.row_offsets[b])
            outs.append(R.absorbed(None if folded else qc[b:b + 1], qr[b:b + 1], np.array([t - 1]),
                                   c[r0:r0 + t], kr[r0:r0 + t], fc.w_uk, fc.w_uv, s.scale, s.rope_base,
                                   split_keys=split, q_tilde=None if not folded else q_t[b:b + 1],
                                   **_decode_prec(BF16, s)))
        got.append({k: np.concatenate([r[k] for r in outs], axis=0) for k in ("o", "obar", "lse")})
    return {"o": _worst(got, want, "o"), "lse": _worst(got, want, "lse")}


def _front_prefill_figures(name, folded):
    fc = cases.front_prefill(name)
    prior, new = (np.asarray(x, np.int32) for x in cases.FRONT_PREFILL)
    s = fc.shape
    seqs, pos = fc.kv_seq_pos()
    new_rows = np.nonzero(pos >= prior[seqs])[0]
    c, kr, qc, qr, q_t = _front_inputs(fc, new_rows, folded)
    oc, okr, oqc, oqr = _front_oracle_inputs(fc, new_rows)
    cu_q = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    want = attention.prefill_batch(cu_q, prior, oc, okr, fc.row_offsets, oqc, oqr, fc.w_uk, fc.w_uv, s.scale)
    outs = []
    for b in range(len(prior)):
        n = int(new[b])
        if n == 0:
            continue
        sel = np.arange(cu_q[b], cu_q[b + 1])
        qpos = int(prior[b]) + np.arange(n)
        t, r0 = int(prior[b]) + n, int(fc.row_offsets[b])
        outs.append(R.absorbed(None if folded else qc[sel], qr[sel], qpos, c[r0:r0 + t], kr[r0:r0 + t], fc.w_uk,
                               fc.w_uv, s.scale, s.rope_base, causal=True,
                               q_tilde=None if not folded else q_t[sel], **BF16))
    got = {k: np.concatenate([r[k] for r in outs], axis=0) for k in ("o", "lse")}
    return {"o": R.errors(got["o"], want["o"]), "lse": R.lse_errors(got["lse"], want["lse"])}


def _prefix_rows():
    """GPU prefill rows against GPU decodes of their prefixes: at most the sum of the
    two paths' model errors against the oracle's rows."""
    pre = cases.prefix_prefill()
    rows = cases.PREFIX_ROWS
    want = _oracle_prefill(pre, queries=rows)
    gp = R.prefill_batch(pre, queries=rows, **BF16)
    decs = [cases.prefix_decode(pre, j) for j in rows]
    gd = [{k: np.concatenate([R.decode_batch(d, split_keys=sp, **_decode_prec(BF16, d.shape))[k] for d in decs])
           for k in ("o", "obar")} for sp in SPLITS]
    out = {}
    for k in ("o", "obar"):
        ep = R.errors(gp[k], want[k])
        ed = _worst(gd, want, k)
        out[k] = (ep[0] + ed[0], ep[1] + ed[1])
    return out


def _mha_vs_absorbed():
    """The two GPU prefill forms against each other: at most the sum of their model errors
    against the oracle (each kernel rounds its softmax weights against its own reference
    maximum, so their roundings are not those of one shared model)."""
    case = cases.mha_vs_absorbed()
    want = _oracle_prefill(case)
    ea = R.errors(R.prefill_batch(case, **BF16)["o"], want["o"])
    em = R.errors(R.prefill_batch(case, form="materialised")["o"], want["o"])
    return {"o": (ea[0] + em[0], ea[1] + em[1])}


# Full-size decode splits: the worst over split lengths of 1, 4, 16 and 32
# pages and no split (the plan picks one of these for the workloads here).
FULL_SPLITS = (None, 64, 256, 1024, 2048)


def _full(case_fn, kind, queries=None, seqs=None):
    case = case_fn()
    if kind == "decode":
        seqs = seqs(case) if callable(seqs) else seqs
        want = _oracle_decode(case, evaluate=attention.absorbed, seqs=seqs)
        got = [R.decode_batch(case, seqs=seqs, split_keys=sp, **_decode_prec(BF16, case.shape)) for sp in FULL_SPLITS]
        return {k: _worst(got, want, k) for k in ("o", "obar", "lse")}
    return _prefill_figures(case, BF16, queries=queries,
                            want=_oracle_prefill(case, evaluate=attention.absorbed, queries=queries))


def c4_sequences(case):
    """32 sequences of the ragged workload, evenly spaced in length order: the
    shortest first, the longest last."""
    order = np.argsort(case.seq_lens, kind="stable")
    return [int(order[i]) for i in np.linspace(0, len(order) - 1, 32).round().astype(int)]


def c5b_queries():
    """The queries of the 2048-after-16384 chunk the full-size tests check: the first
    and last eight and an even stride of 64 across the chunk."""
    return np.unique(np.concatenate([np.arange(8), np.arange(2040, 2048),
                                     np.linspace(0, 2047, 64).round().astype(int)]))


RECIPES = {
    "tiny_decode_ragged": lambda: _decode_figures(cases.tiny_decode_ragged(), F32W),
    "dsv2_decode_ragged": lambda: _decode_figures(cases.dsv2_decode_ragged(), BF16),
    "decode_empty": lambda: _decode_figures(cases.decode_empty(), BF16),
    "decode_proj_many": lambda: _decode_figures(cases.decode_proj_many(), BF16, seqs=cases.DECODE_PROJ_MANY_ROWS,
                                                fused=True),
    "decode_overflow": lambda: _decode_figures(cases.decode_overflow(), BF16),
    "tiny_bf16_prefill": lambda: _prefill_figures(cases.tiny_prefill_short(), BF16),
    "tiny_bf16_decode": lambda: _decode_figures(cases.tiny_decode_short(), BF16),
    "prefill_ragged_dsv2": lambda: _prefill_figures(cases.prefill_ragged(synth.DSV2), BF16),
    "prefill_ragged_tiny": lambda: _prefill_figures(cases.prefill_ragged(synth.TINY), F32W),
    "mha_ragged_dsv2": lambda: _prefill_figures(cases.prefill_ragged(synth.DSV2), BF16, form="materialised"),
    "mha_ragged_tiny": lambda: _prefill_figures(cases.prefill_ragged(synth.TINY), BF16, form="materialised"),
    "mha_long_prefix": lambda: _prefill_figures(cases.mha_long_prefix(), BF16, form="materialised"),
    "mha_vs_absorbed": _mha_vs_absorbed,
    "prefix_rows": _prefix_rows,
    "mha_c2": lambda: _prefill_figures(synth.config2(), BF16, form="materialised"),
    "two_scale_decode_tiny": lambda: _decode_figures(cases.two_scale_decode(synth.TINY, "bf16"), F32W,
                                                     scales=_two_scales(synth.TINY)),
    "two_scale_decode_dsv2": lambda: _decode_figures(cases.two_scale_decode(synth.DSV2, "bf16"), BF16,
                                                     scales=_two_scales(synth.DSV2)),
    "two_scale_prefill_tiny": lambda: _prefill_figures(cases.two_scale_prefill(synth.TINY), F32W,
                                                       scales=_two_scales(synth.TINY)),
    "two_scale_prefill_dsv2": lambda: _prefill_figures(cases.two_scale_prefill(synth.DSV2), BF16,
                                                       scales=_two_scales(synth.DSV2)),
    "two_scale_mha_tiny": lambda: _prefill_figures(cases.two_scale_prefill_materialised(synth.TINY), BF16,
                                                   form="materialised", scales=_two_scales(synth.TINY)),
    "two_scale_mha_dsv2": lambda: _prefill_figures(cases.two_scale_prefill_materialised(synth.DSV2), BF16,
                                                   form="materialised", scales=_two_scales(synth.DSV2)),
    "per_head_f32w": lambda: _decode_figures(cases.per_head_decode(), F32W),
    "per_head_bf16": lambda: _decode_figures(cases.per_head_decode(), BF16),
    "per_head_two_scale": lambda: _decode_figures(cases.per_head_two_scale(), F32W,
                                                  scales=_two_scales(synth.TINY)),
    "front_decode_tiny_unfolded": lambda: _front_decode_figures("tiny", False),
    "front_decode_tiny_folded": lambda: _front_decode_figures("tiny", True),
    "front_decode_dsv2_unfolded": lambda: _front_decode_figures("dsv2", False),
    "front_decode_dsv2_folded": lambda: _front_decode_figures("dsv2", True),
    "front_prefill_tiny_unfolded": lambda: _front_prefill_figures("tiny", False),
    "front_prefill_tiny_folded": lambda: _front_prefill_figures("tiny", True),
    "front_prefill_dsv2_unfolded": lambda: _front_prefill_figures("dsv2", False),
    "front_prefill_dsv2_folded": lambda: _front_prefill_figures("dsv2", True),
    "c2": lambda: _prefill_figures(synth.config2(), F32W),
}

# full-size workloads: minutes of CPU each
FULL_RECIPES = {
    "c3": lambda: _full(synth.config3, "decode"),
    "c4": lambda: _full(synth.config4, "decode", seqs=c4_sequences),
    "c5a": lambda: _full(synth.config5_decode, "decode"),
    "c5b": lambda: _full(synth.config5_prefill, "prefill", queries=c5b_queries()),
    "c5b_mha": lambda: _prefill_figures(synth.config5_prefill(), BF16, form="materialised", queries=c5b_queries(),
                                        want=_oracle_prefill(synth.config5_prefill(), evaluate=attention.absorbed,
                                                             queries=c5b_queries())),
    "per_head_full": lambda: _decode_figures(cases.per_head_full(), F32W, seqs=list(range(64)),
                                             want=_oracle_decode(cases.per_head_full(), evaluate=attention.absorbed)),
}


def figure(name: str):
    """{output: (max, rms)} of the model against the oracle for the named test input."""
    fn = RECIPES.get(name) or FULL_RECIPES[name]
    return fn()


if __name__ == "__main__":
    import time

    names = list(RECIPES) + (list(FULL_RECIPES) if "--full" in sys.argv else [])
    only = [a for a in sys.argv[1:] if not a.startswith("--")]
    for name in names:
        if only and name not in only:
            continue
        t0 = time.time()
        figs = figure(name)
        txt = "  ".join(f"{k}: max {v[0]:.3e} rms {v[1]:.3e}" for k, v in figs.items())
        print(f"{name:30s} {txt}   ({time.time() - t0:.1f} s)", flush=True)
