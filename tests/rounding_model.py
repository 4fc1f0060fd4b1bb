"""Storage-rounding model of the library's arithmetic (test infrastructure, CPU only).

The GPU path computes the same attention as the oracle but stores or feeds
some intermediate values at reduced precision.  This module evaluates the
attention in float64 with a round-to-nearest-even cast at each of those
points and nowhere else, so it predicts the error the GPU result should show
against the float64 oracle when every float32 accumulation is taken as exact
(float32 sums over at most a few thousand terms add ~1e-6 relative, two
orders below every bound used here).

It calls only the oracle (``oracle.rope.rotate``, ``oracle.attention``'s
absorption helpers and its materialised definition) and numpy / torch casts.
It shares nothing with the HIP sources and reads no GPU output.  The tests use
it in two ways: a CPU test checks that every bound a GPU test uses is at least
the error this model predicts for that test's inputs, and that the model
with every cast switched off is the oracle's own result.

Rounding points (each a keyword below):

* ``q_lat``  -- the absorbed query q~ = W_UK^T q^C and the rotated query
  R_m q^R as stored in q_lat: "bf16" (one rounding), or "f32" (float32, then
  scored as a two-term bf16 split hi + lo, ~16 significant bits).
* rotated position key R_t k^R_t: always rounded to the cache dtype (bf16)
  when the cache row is written.
* ``p``      -- the softmax weights fed to the weighted sum: "bf16", "f16",
  "two_term" (hi + lo bf16) or "exact".  Each weight is exp(s - m_ref) against
  the same reference maximum the kernel uses (the first 32-key block's
  largest score for the absorbed form, with its overflow fallback; a lazily
  moved running maximum for the materialised form), so the values rounded are
  the kernel's.  The row sum l is always the sum of the unrounded weights
  (float32 in the kernels).
* ``obar``   -- the latent output: "bf16" or "f32".  Decode partials of a
  split sequence are stored as ``partial``: "f32", "bf16", or "f16q" (float16
  with a power-of-two scale per 128 consecutive columns, chosen so that the
  group's largest magnitude lies in [0.5, 1)), and merged with float32
  weights.
* materialised form: K^C = W_UK c and V = W_UV c rounded to ``kv`` ("f16" or
  "bf16"), the content query converted to the same type, the position part
  bf16, the weights P rounded to ``p``.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import attention, rope


# ------------------------------------------------------------------ casts --

def f32(x):
    """Round float64 to float32 (RNE) and return float64."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to float32 then to bfloat16 (RNE both), as a float32 value feeding a bf16 store."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def f16(x):
    """Round to float32 then to float16 (RNE both, subnormals kept)."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def two_term(x):
    """A float32 value fed as hi + lo, hi = bf16(x), lo = bf16(x - hi)."""
    x = f32(x)
    hi = bf16(x)
    return hi + bf16(x - hi)


def f16_scaled(x, group=128):
    """A float32 value stored as float16 after scaling by 2^-e, e the exponent
    (frexp) of the largest magnitude in its group of ``group`` consecutive
    elements of the last axis; scaled back exactly."""
    x = f32(x)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // group, group))
    mx = np.max(np.abs(g), axis=-1, keepdims=True)
    e = np.where(mx > 0, np.frexp(mx)[1], 0)
    return np.ldexp(f16(np.ldexp(g, -e)), e).reshape(x.shape)


_CAST = {"bf16": bf16, "f16": f16, "f32": f32, "two_term": two_term, "f16q": f16_scaled,
         "exact": lambda x: np.asarray(x, np.float64)}


def _q_cast(kind):
    return {"bf16": bf16, "f32": two_term, "exact": _CAST["exact"]}[kind]


# ------------------------------------------------------- absorbed form ----

def absorbed(qc, qr, q_pos, c, kr, w_uk, w_uv, scale, base=10000.0, causal=False, key_offset=0,
             q_lat="bf16", p="bf16", obar="bf16", split_keys=None, partial="bf16", key_cast="bf16",
             position_scale=None, q_tilde=None, all_partials=False):
    """Absorbed attention (q~ . c_t + R_m q^R . R_t k^R_t) with the library's storage roundings.

    Arguments as ``oracle.attention.absorbed`` (kr [T, d_r] shared, or
    [T, H, d_r] one key per head).  ``split_keys`` (decode) cuts the keys into
    consecutive ranges of that many keys, each normalised on its own, stored
    as ``partial`` with its lse and merged in order, as the split decode does;
    None keeps one range.  ``q_tilde`` [N, H, d_c] replaces W_UK^T q^C (a
    query formed elsewhere, e.g. through a folded weight); it is cast like
    q_lat.  ``all_partials`` (the fused decode and output absorption) stores a
    single range as ``partial`` too before obar is formed from it.  Returns
    dict(o, obar, lse).
    """
    qc = np.asarray(qc, np.float64)
    c = np.asarray(c, np.float64)
    q_pos = np.asarray(q_pos)
    key_pos = key_offset + np.arange(c.shape[0])
    qcast = _q_cast(q_lat)
    q_t = qcast(attention.query_absorption(w_uk, qc) if q_tilde is None else q_tilde)  # [N, H, d_c]
    ratio = 1.0 if position_scale is None else position_scale / scale
    q_r = qcast(ratio * rope.rotate(qr, q_pos[:, None], base))             # [N, H, d_r]
    kr = np.asarray(kr, np.float64)
    if kr.ndim == 3:                                                       # one key per head
        k_r = _CAST[key_cast](rope.rotate(kr, key_pos[:, None], base))     # [T, H, d_r]
        pos_dot = np.einsum("nhr,thr->nht", q_r, k_r)
    else:
        k_r = _CAST[key_cast](rope.rotate(kr, key_pos, base))              # [T, d_r]
        pos_dot = q_r @ k_r.T
    s = scale * (q_t @ c.T + pos_dot)                                      # [N, H, T]
    vis = key_pos[None, :] <= q_pos[:, None] if causal else np.ones((len(q_pos), c.shape[0]), bool)
    s = np.where(vis[:, None, :], s, -np.inf)
    n, h = q_t.shape[:2]
    t_all = c.shape[0]
    ranges = [(0, t_all)] if not split_keys or t_all == 0 else \
        [(a, min(t_all, a + split_keys)) for a in range(0, t_all, split_keys)]
    pcast = _CAST[p]
    parts, lses = [], []
    for a, b in ranges:
        sb = s[:, :, a:b]
        m = np.max(sb, axis=-1, keepdims=True) if b > a else np.full((n, h, 1), -np.inf)
        m = np.where(np.isfinite(m), m, 0.0)
        # The kernel's softmax weights are P = exp(s - m_ref): m_ref is the row's largest
        # score in the range's first 32-key block, unless some row's sum of P would pass
        # 2^64 (then its workgroup -- every head of a decode range, or 128 consecutive
        # (query, head) rows of a prefill -- takes the range's true maximum).  The
        # reference changes which values P takes, and so how each rounds.
        m_ref = np.max(sb[:, :, :32], axis=-1, keepdims=True) if b > a else m
        m_ref = np.where(np.isfinite(m_ref), m_ref, m)
        big = np.sum(np.exp(sb - m_ref), axis=-1) > 2.0 ** 64 * 0.999  # [N, H]
        if big.any():
            if causal:
                rows = big.reshape(-1)  # (query, head) rows in order
                blk = np.zeros_like(rows)
                for r0 in range(0, rows.size, 128):
                    blk[r0:r0 + 128] = rows[r0:r0 + 128].any()
                big = blk.reshape(big.shape)
            else:
                big = np.broadcast_to(big.any(axis=1, keepdims=True), big.shape)
            m_ref = np.where(big[..., None], m, m_ref)
        m = m_ref
        e = np.exp(sb - m)
        l_sum = e.sum(axis=-1, keepdims=True)
        num = pcast(e) @ c[a:b]
        with np.errstate(invalid="ignore", divide="ignore"):
            ob = np.where(l_sum > 0, num / np.where(l_sum > 0, l_sum, 1.0), 0.0)
            lse = np.where(l_sum[..., 0] > 0, m[..., 0] + np.log(np.where(l_sum[..., 0] > 0, l_sum[..., 0], 1.0)),
                           -np.inf)
        parts.append(ob)
        lses.append(lse)
    if len(ranges) == 1:
        ob, lse = parts[0], lses[0]
        if all_partials:
            ob = _CAST[partial](ob)
    else:
        pc = _CAST[partial]
        lse_all = np.stack(lses)                                           # [S, N, H]
        mx = np.max(lse_all, axis=0)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        w = f32(np.exp(lse_all - mx))
        wsum = w.sum(axis=0)
        acc = sum(w[i][..., None] * pc(parts[i]) for i in range(len(parts)))
        with np.errstate(invalid="ignore", divide="ignore"):
            ob = np.where(wsum[..., None] > 0, acc / np.where(wsum[..., None] > 0, wsum[..., None], 1.0), 0.0)
            lse = np.where(wsum > 0, mx + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    ob = _CAST[obar](ob)
    o = f32(attention.output_absorption(w_uv, ob))
    return {"o": o, "obar": ob, "lse": lse}


# --------------------------------------------------- materialised form ----

def materialised(qc, qr, q_pos, c, kr, w_uk, w_uv, scale, base=10000.0, causal=False, key_offset=0,
                 kv="f16", p="f16", position_scale=None, rot="bf16"):
    """Materialised attention with the library's roundings: per-head K^C = W_UK c and
    V = W_UV c rounded to ``kv``, the content query converted to ``kv`` (exact
    for bf16 inputs in range), the position part from rotated rows rounded to
    ``rot`` (bf16: the cache row and q_lat's tail), the weights rounded to
    ``p``, float32 output."""
    qc = np.asarray(qc, np.float64)
    c = np.asarray(c, np.float64)
    q_pos = np.asarray(q_pos)
    key_pos = key_offset + np.arange(c.shape[0])
    kcast = _CAST[kv]
    ratio = 1.0 if position_scale is None else position_scale / scale
    k_c = kcast(np.einsum("hdc,tc->htd", np.asarray(w_uk, np.float64), c))  # [H, T, d_h]
    v = kcast(np.einsum("hvc,tc->htv", np.asarray(w_uv, np.float64), c))    # [H, T, d_v]
    q_c = kcast(qc).transpose(1, 0, 2)                                      # [H, N, d_h]
    q_r = _CAST[rot](ratio * rope.rotate(qr, q_pos[:, None], base)).transpose(1, 0, 2)
    k_r = _CAST[rot](rope.rotate(kr, key_pos, base))                        # [T, d_r]
    s = scale * (q_c @ k_c.transpose(0, 2, 1) + q_r @ k_r.T)                # [H, N, T]
    vis = key_pos[None, :] <= q_pos[:, None] if causal else np.ones((len(q_pos), c.shape[0]), bool)
    s = np.where(vis[None], s, -np.inf)
    # The kernel walks 32-key tiles with a running reference: it starts at the first
    # tile's largest score and moves to a tile's largest only when that exceeds it by
    # more than 8 in base 2 (O and the sum are rescaled then, in float32).  Each
    # weight is P = exp(s - reference at its tile), rounded to `p`.
    t_all = s.shape[-1]
    ref = np.full(s.shape[:-1], -np.inf)
    num = np.zeros(s.shape[:-1] + (v.shape[-1],))
    l_sum = np.zeros(s.shape[:-1])
    for t0 in range(0, t_all, 32):
        st = s[..., t0:t0 + 32]
        mt = np.max(st, axis=-1)
        move = mt > ref + 8.0 * math.log(2.0)
        new_ref = np.where(move, mt, ref)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(ref) & move, np.exp(ref - new_ref), np.where(np.isfinite(ref), 1.0, 0.0))
        ref = new_ref
        safe = np.where(np.isfinite(ref), ref, 0.0)
        e = np.exp(st - safe[..., None])
        num = num * alpha[..., None] + _CAST[p](e) @ v[:, t0:t0 + 32]
        l_sum = l_sum * alpha + e.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l_sum[..., None] > 0, num / np.where(l_sum[..., None] > 0, l_sum[..., None], 1.0), 0.0)
        lse = np.where(l_sum > 0, np.where(np.isfinite(ref), ref, 0.0) + np.log(np.where(l_sum > 0, l_sum, 1.0)),
                       -np.inf)
    return {"o": f32(o.transpose(1, 0, 2)), "lse": lse.T}


# ------------------------------------------------------------- batches ----

def decode_batch(case, seqs=None, **kw):
    """The model over a decode case's sequences (query of b at T_b - 1)."""
    seqs = range(case.batch) if seqs is None else seqs
    outs = []
    for b in seqs:
        t = int(case.seq_lens[b])
        r0 = int(case.row_offsets[b])
        outs.append(absorbed(case.qc[b:b + 1], case.qr[b:b + 1], np.array([t - 1]), case.c_rows[r0:r0 + t],
                             case.kr_rows[r0:r0 + t], case.w_uk, case.w_uv, case.shape.scale,
                             case.shape.rope_base, **kw))
    return {k: np.concatenate([r[k] for r in outs], axis=0) for k in ("o", "obar", "lse")}


def prefill_batch(case, form="absorbed", queries=None, **kw):
    """The model over a prefill case (query j of b at q_start[b] + j), in the absorbed
    or the materialised form; ``queries`` lists global query indices."""
    fn = absorbed if form == "absorbed" else materialised
    want = np.arange(case.cu_q[-1]) if queries is None else np.asarray(queries)
    outs = {}
    for b in range(case.batch):
        sel = want[(want >= case.cu_q[b]) & (want < case.cu_q[b + 1])]
        if len(sel) == 0:
            continue
        pos = int(case.q_start[b]) + (sel - case.cu_q[b])
        t = int(pos.max()) + 1
        r0 = int(case.row_offsets[b])
        res = fn(case.qc[sel], case.qr[sel], pos, case.c_rows[r0:r0 + t], case.kr_rows[r0:r0 + t], case.w_uk,
                 case.w_uv, case.shape.scale, case.shape.rope_base, causal=True, **kw)
        for i, g in enumerate(sel):
            outs[int(g)] = {k: res[k][i] for k in res}
    keys = list(next(iter(outs.values())).keys())
    return {k: np.stack([outs[int(g)][k] for g in want]) for k in keys}


def lse_errors(got, want):
    """(max |err|, rms err) of lse in nats over the finite entries (-inf must match)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    if not fin.any():
        return 0.0, 0.0
    err = np.abs(got[fin] - want[fin])
    return float(err.max()), float(np.sqrt(np.mean(err * err)))


def errors(got, want):
    """(max|err| / rms(want), rms(err) / rms(want)) over all elements: the pass metric."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want * want))
    err = got - want
    return float(np.max(np.abs(err)) / rms), float(np.sqrt(np.mean(err * err)) / rms)
