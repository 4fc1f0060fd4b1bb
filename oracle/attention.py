"""MLA attention with decoupled RoPE, float64, three independent evaluations.

The spec is ``materialised``.  It follows the pages' dataflow literally:

* "AI decoupled RoPE MLA" (operatorworld.com), recap section: the cache holds
  only c_t; k_t = W^UK c_t and v_t = W^UV c_t are up-projections of it.
* same page, decoupled-RoPE section: the content channel q^C, k^C = W^UK c_t is
  never rotated; the position channel q^R, k^R (width d_r) is rotated by RoPE;
  the score is the sum of the two channel dot products.
* "Latent Attention Meets RoPE" (sahipadhai.cc), "The fix" section: the score
  is the dot product of the concatenated [content ; position] vectors, and the
  position key k^R is one vector per token shared by every head.
* "Multi-Head Latent Attention" (talalahmed.dev), "Why RoPE makes this harder":
  K = [K^C ; K^R], Q = [Q^C ; Q^R], Q K^T = Q^C K^C^T + Q^R K^R^T; "Why this
  matters on a GPU": softmax and the weighted sum of values are still there.

So for every head i, query n at position m and key t:

    K_i[t] = [ W_UK,i c_t ; R_t k^R_t ]          (d_h + d_r)
    V_i[t] =   W_UV,i c_t                        (d_v)
    Q_i[n] = [ q^C_{n,i} ; R_m q^R_{n,i} ]
    s_t    = scale * Q_i[n] . K_i[t]
    alpha  = softmax over the visible keys, lse = log sum exp(s_t)
    o      = sum_t alpha_t V_i[t]                (the layer output)
    obar   = sum_t alpha_t c_t                   (the latent output)

``absorbed`` is the weight-absorbed twin of the operatorworld.com recap
equations (q~ = W_UK^T q^C; output = W_UV sum_t alpha_t c_t), used only as a
self-check of ``materialised`` (the ropeabsorb README reports the two agree to
2e-13 in float64 but are not bit-identical).

``brute_force`` is the same definition in scalar pure-Python loops, for tiny
cases only.

Readings where the pages are silent (each also used by the GPU path):

* One softmax scale on the summed score by default.  The operatorworld.com
  page's decoupled-RoPE section writes the score with its own factor on each
  channel (content over sqrt(d), position over sqrt(d_r)); every evaluation
  here takes that form when ``position_scale`` is given:
      s_t = scale * (q^C . k^C_t) + position_scale * (R_m q^R . R_t k^R_t).
* Key t sits at position t; a decode query sees keys 0 .. T-1 (its own token
  is already in the cache); a causal query at position m sees keys t <= m.
* A query with no visible key has obar = 0, o = 0 and lse = -inf.
"""

from __future__ import annotations

import math

import numpy as np

from . import rope


def _visible(q_pos: np.ndarray, key_pos: np.ndarray, causal: bool) -> np.ndarray:
    if causal:
        return key_pos[None, :] <= np.asarray(q_pos)[:, None]
    return np.ones((len(q_pos), len(key_pos)), dtype=bool)


def _softmax(s: np.ndarray, visible: np.ndarray):
    """Masked softmax over the last axis.  s [N, H, T], visible [N, T]."""
    s = np.where(visible[:, None, :], s, -np.inf)
    m = s.max(axis=-1, keepdims=True) if s.shape[-1] else np.full(s.shape[:-1] + (1,), -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)
    z = e.sum(axis=-1, keepdims=True)
    alpha = np.where(empty, 0.0, e / np.where(empty, 1.0, z))
    lse = np.where(empty[..., 0], -np.inf, (m_safe + np.log(np.where(empty, 1.0, z)))[..., 0])
    return alpha, lse


def materialise_keys(c, kr, w_uk, key_pos, base=10000.0):
    """K_i[t] = [W_UK,i c_t ; R_{pos t} k^R_t] for every head i.  Returns [T, H, d_h + d_r].

    kr [T, d_r]: one position key per token, the same for every head (the
    decoupled design).  kr [T, H, d_r]: one position key per head and token,
    K_i[t] = [W_UK,i c_t ; R_{pos t} k^R_{t,i}] (the simplified MLA-style
    cache of "Multi-Head Latent Attention", "A concrete size comparison").
    """
    c = np.asarray(c, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    kr = np.asarray(kr, np.float64)
    h, d_h, _ = w_uk.shape
    k_content = (c @ w_uk.reshape(h * d_h, -1).T).reshape(c.shape[0], h, d_h)
    if kr.ndim == 3:
        return np.concatenate([k_content, rope.rotate(kr, np.asarray(key_pos)[:, None], base)], axis=-1)
    k_rope = rope.rotate(kr, np.asarray(key_pos), base)
    return np.concatenate(
        [k_content, np.broadcast_to(k_rope[:, None, :], (c.shape[0], h, k_rope.shape[-1]))], axis=-1)


def materialise_values(c, w_uv):
    """V_i[t] = W_UV,i c_t for every head i.  Returns [T, H, d_v]."""
    c = np.asarray(c, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    h, d_v, _ = w_uv.shape
    return (c @ w_uv.reshape(h * d_v, -1).T).reshape(c.shape[0], h, d_v)


def materialised(qc, qr, q_pos, c, kr, w_uk, w_uv, scale, base=10000.0, causal=False,
                 key_chunk=2048, key_offset=0, position_scale=None):
    """The definition: materialise K and V per head, then plain softmax attention.

    qc [N, H, d_h] and qr [N, H, d_r] (q^R un-rotated), q_pos [N] int;
    c [T, d_c], kr [T, d_r] (k^R un-rotated; key t is at position
    key_offset + t); w_uk [H, d_h, d_c], w_uv [H, d_v, d_c] (weights stored
    [out, in]).  kr may also be [T, H, d_r], one position key per head
    (``materialise_keys``).  With ``position_scale`` the two channels' dot products take
    their own scales (the two-scale score); without it one scale multiplies the
    [content ; position] dot product.  Returns dict(o [N, H, d_v],
    obar [N, H, d_c], lse [N, H]).
    """
    qc = np.asarray(qc, np.float64)
    qr = np.asarray(qr, np.float64)
    c = np.asarray(c, np.float64)
    q_pos = np.asarray(q_pos)
    n, h, _ = qc.shape
    t_all = c.shape[0]
    key_pos = key_offset + np.arange(t_all)
    d_v = np.asarray(w_uv).shape[1]
    q = np.concatenate([qc, rope.rotate(qr, q_pos[:, None], base)], axis=-1)  # [N, H, d_h+d_r]
    q_h = np.ascontiguousarray(q.transpose(1, 0, 2))  # [H, N, D]
    s = np.empty((n, h, t_all), dtype=np.float64)
    for t0 in range(0, t_all, key_chunk):
        t1 = min(t_all, t0 + key_chunk)
        k_full = materialise_keys(c[t0:t1], kr[t0:t1], w_uk, key_pos[t0:t1], base)
        k_h = np.ascontiguousarray(k_full.transpose(1, 2, 0))  # [H, D, Tc]
        if position_scale is None:
            s[:, :, t0:t1] = (scale * (q_h @ k_h)).transpose(1, 0, 2)
        else:
            d_h = qc.shape[2]
            content = q_h[:, :, :d_h] @ k_h[:, :d_h, :]
            position = q_h[:, :, d_h:] @ k_h[:, d_h:, :]
            s[:, :, t0:t1] = (scale * content + position_scale * position).transpose(1, 0, 2)
    alpha, lse = _softmax(s, _visible(q_pos, key_pos, causal))
    o = np.zeros((n, h, d_v), dtype=np.float64)
    for t0 in range(0, t_all, key_chunk):
        t1 = min(t_all, t0 + key_chunk)
        v = materialise_values(c[t0:t1], w_uv)
        o += (alpha[:, :, t0:t1].transpose(1, 0, 2) @ v.transpose(1, 0, 2)).transpose(1, 0, 2)
    obar = alpha @ c  # sum_t alpha_t c_t, [N, H, d_c]
    return {"o": o, "obar": obar, "lse": lse}


def query_absorption(w_uk, qc):
    """q~_{n,i} = W_UK,i^T q^C_{n,i} ("AI decoupled RoPE MLA", recap: merged ahead of the cache).

    w_uk [H, d_h, d_c], qc [N, H, d_h] -> [N, H, d_c]."""
    return np.einsum("hdc,nhd->nhc", np.asarray(w_uk, np.float64), np.asarray(qc, np.float64))


def output_absorption(w_uv, obar):
    """o_{n,i} = W_UV,i obar_{n,i} ("AI decoupled RoPE MLA", recap: W^UV applied after the sum).

    w_uv [H, d_v, d_c], obar [N, H, d_c] -> [N, H, d_v]."""
    return np.einsum("hvc,nhc->nhv", np.asarray(w_uv, np.float64), np.asarray(obar, np.float64))


def absorbed(qc, qr, q_pos, c, kr, w_uk, w_uv, scale, base=10000.0, causal=False, key_offset=0,
             position_scale=None):
    """The weight-absorbed evaluation order (self-check of ``materialised`` only).

    q~ = W_UK^T q^C (per head), s_t = scale (q~ . c_t + R_m q^R . R_t k^R_t)
    (or scale q~ . c_t + position_scale R_m q^R . R_t k^R_t),
    obar = sum_t alpha_t c_t, o = W_UV obar.
    """
    qc = np.asarray(qc, np.float64)
    c = np.asarray(c, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    q_pos = np.asarray(q_pos)
    key_pos = key_offset + np.arange(c.shape[0])
    q_tilde = query_absorption(w_uk, qc)  # W_UK^T q^C
    q_rot = rope.rotate(qr, q_pos[:, None], base)
    kr = np.asarray(kr, np.float64)
    if kr.ndim == 3:  # one position key per head: [T, H, d_r]
        k_rot = rope.rotate(kr, key_pos[:, None], base)
        pos_dot = np.einsum("nhr,thr->nht", q_rot, k_rot)
    else:
        pos_dot = q_rot @ rope.rotate(kr, key_pos, base).T
    if position_scale is None:
        s = scale * (q_tilde @ c.T + pos_dot)
    else:
        s = scale * (q_tilde @ c.T) + position_scale * pos_dot
    alpha, lse = _softmax(s, _visible(q_pos, key_pos, causal))
    obar = alpha @ c
    o = output_absorption(w_uv, obar)
    return {"o": o, "obar": obar, "lse": lse, "q_tilde": q_tilde, "q_rot": q_rot}


def brute_force(qc, qr, q_pos, c, kr, w_uk, w_uv, scale, base=10000.0, causal=False, position_scale=None):
    """Scalar pure-Python loops over the materialised definition (tiny inputs only).

    Uses only ``math`` and Python lists: no numpy arithmetic, no shared helper.
    """
    per_head = np.asarray(kr).ndim == 3  # kr [T, H, d_r]: one position key per head
    qc, qr, c, kr = (np.asarray(a, np.float64).tolist() for a in (qc, qr, c, kr))
    w_uk = np.asarray(w_uk, np.float64).tolist()
    w_uv = np.asarray(w_uv, np.float64).tolist()
    q_pos = [int(p) for p in q_pos]
    n, h = len(qc), len(qc[0])
    d_h, d_r = len(qc[0][0]), len(qr[0][0])
    d_c, d_v, t_all = len(c[0]), len(w_uv[0]), len(c)

    def rot(vec, p):
        out = [0.0] * d_r
        for j in range(d_r // 2):
            a = p * (base ** (-2.0 * j / d_r))
            out[2 * j] = vec[2 * j] * math.cos(a) - vec[2 * j + 1] * math.sin(a)
            out[2 * j + 1] = vec[2 * j] * math.sin(a) + vec[2 * j + 1] * math.cos(a)
        return out

    o = [[[0.0] * d_v for _ in range(h)] for _ in range(n)]
    obar = [[[0.0] * d_c for _ in range(h)] for _ in range(n)]
    lse = [[-math.inf] * h for _ in range(n)]
    for qi in range(n):
        for hi in range(h):
            qrot = rot(qr[qi][hi], q_pos[qi])
            scores = []
            for t in range(t_all):
                if causal and t > q_pos[qi]:
                    continue
                kc = [sum(w_uk[hi][a][b] * c[t][b] for b in range(d_c)) for a in range(d_h)]
                krot = rot(kr[t][hi] if per_head else kr[t], t)
                dot_c = sum(x * y for x, y in zip(qc[qi][hi], kc))
                dot_r = sum(x * y for x, y in zip(qrot, krot))
                if position_scale is None:
                    scores.append((t, scale * (dot_c + dot_r)))
                else:
                    scores.append((t, scale * dot_c + position_scale * dot_r))
            if not scores:
                continue
            mx = max(sv for _, sv in scores)
            z = sum(math.exp(sv - mx) for _, sv in scores)
            lse[qi][hi] = mx + math.log(z)
            for t, sv in scores:
                a = math.exp(sv - mx) / z
                for vi in range(d_v):
                    o[qi][hi][vi] += a * sum(w_uv[hi][vi][b] * c[t][b] for b in range(d_c))
                for b in range(d_c):
                    obar[qi][hi][b] += a * c[t][b]
    return {"o": np.array(o), "obar": np.array(obar), "lse": np.array(lse)}


def decode_batch(seq_lens, c_rows, kr_rows, row_offsets, qc, qr, w_uk, w_uv, scale,
                 base=10000.0, seqs=None, evaluate=materialised, position_scale=None):
    """Decode for a batch: query b sits at position T_b - 1 and sees keys 0 .. T_b - 1.

    c_rows [sum T, d_c] and kr_rows [sum T, d_r] hold each sequence's tokens in
    position order starting at row_offsets[b]; qc [B, H, d_h], qr [B, H, d_r].
    ``seqs`` selects a subset of sequences; results are stacked in that order.
    """
    seqs = range(len(seq_lens)) if seqs is None else seqs
    outs = []
    for b in seqs:
        t = int(seq_lens[b])
        r0 = int(row_offsets[b])
        outs.append(evaluate(qc[b:b + 1], qr[b:b + 1], np.array([t - 1]), c_rows[r0:r0 + t],
                             kr_rows[r0:r0 + t], w_uk, w_uv, scale, base=base, causal=False,
                             position_scale=position_scale))
    return {k: np.concatenate([r[k] for r in outs], axis=0) for k in ("o", "obar", "lse")}


def prefill_batch(cu_q, q_start, c_rows, kr_rows, row_offsets, qc, qr, w_uk, w_uv, scale,
                  base=10000.0, queries=None, evaluate=materialised, position_scale=None):
    """Causal chunked prefill: query j of sequence b sits at position q_start[b] + j.

    c_rows / kr_rows hold positions 0 .. q_start[b] + n_b - 1 of sequence b from
    row_offsets[b].  qc, qr are [sum n_b, H, *].  ``queries`` optionally lists
    global query indices to evaluate (results in that order).
    """
    cu_q = np.asarray(cu_q)
    batch = len(cu_q) - 1
    want = np.arange(cu_q[-1]) if queries is None else np.asarray(queries)
    outs = {}
    for b in range(batch):
        sel = want[(want >= cu_q[b]) & (want < cu_q[b + 1])]
        if len(sel) == 0:
            continue
        pos = int(q_start[b]) + (sel - cu_q[b])
        t = int(pos.max()) + 1
        r0 = int(row_offsets[b])
        res = evaluate(qc[sel], qr[sel], pos, c_rows[r0:r0 + t], kr_rows[r0:r0 + t],
                       w_uk, w_uv, scale, base=base, causal=True, position_scale=position_scale)
        for i, g in enumerate(sel):
            outs[int(g)] = {k: res[k][i] for k in ("o", "obar", "lse")}
    return {k: np.stack([outs[int(g)][k] for g in want]) for k in ("o", "obar", "lse")}
