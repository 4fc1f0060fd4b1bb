"""The front of the layer: latent, query and position projections from the hidden state, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page title / section / equation):
* "AI decoupled RoPE MLA" (operatorworld.com), recap: the latent is the
  down-projection c_t = W^DKV h_t; decoupled-RoPE section: the position
  channel projects k^R_t = W^KR h_t (one per token, shared by the heads) and
  q^R, and only that channel is rotated.
* "Detailed Illustration of the Problem" (notion.site), Step 1: the query
  goes through a compressed query latent c^Q_t = W^DQ h_t and is projected up
  from it, q^pre_t = W^UQ c^Q_t; Step 4: without a rotation between them the
  up-projections fold into one query weight W^{Q'} = (W^UQ)^T W^UK.
* "ropeabsorb" README (github.com/v-code01): the folded and the unfolded
  evaluation orders are one result in exact arithmetic.

Readings (the pages leave them open):
* With the query latent present, both channels of the query come from it:
  q^C_{n,i} = W_UQ,i c^Q_n and q^R_{n,i} = W_QR,i c^Q_n.  (The decoupled
  section writes the channels from h directly; the latent path of Step 1
  sits in front of both.)
* Weights are stored [out, in] (rows are output features): W_DKV [d_c, D],
  W_KR [d_r, D], W_DQ [d_q, D], W_UQ [H, d_h, d_q], W_QR [H, d_r, d_q].
* The folded weight is kept per head as W_fold,i = W_UK,i^T W_UQ,i
  [H, d_c, d_q], so that q~_{n,i} = W_fold,i c^Q_n directly (the transpose
  of the page's W^{Q'}, which multiplies c^Q from the left as a row vector).
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_latent(h, w_dkv):
    """c_n = W_DKV h_n.  h [N, D], w_dkv [d_c, D] -> [N, d_c]."""
    return _f64(h) @ _f64(w_dkv).T


def position_key(h, w_kr):
    """k^R_n = W_KR h_n (un-rotated).  h [N, D], w_kr [d_r, D] -> [N, d_r]."""
    return _f64(h) @ _f64(w_kr).T


def query_latent(h, w_dq):
    """c^Q_n = W_DQ h_n.  h [N, D], w_dq [d_q, D] -> [N, d_q]."""
    return _f64(h) @ _f64(w_dq).T


def content_query(cq, w_uq):
    """q^C_{n,i} = W_UQ,i c^Q_n.  cq [N, d_q], w_uq [H, d_h, d_q] -> [N, H, d_h]."""
    return np.einsum("hdq,nq->nhd", _f64(w_uq), _f64(cq))


def position_query(cq, w_qr):
    """q^R_{n,i} = W_QR,i c^Q_n (un-rotated).  cq [N, d_q], w_qr [H, d_r, d_q] -> [N, H, d_r]."""
    return np.einsum("hrq,nq->nhr", _f64(w_qr), _f64(cq))


def fold_query_weights(w_uq, w_uk):
    """W_fold,i = W_UK,i^T W_UQ,i.  w_uq [H, d_h, d_q], w_uk [H, d_h, d_c] -> [H, d_c, d_q]."""
    return np.einsum("hdc,hdq->hcq", _f64(w_uk), _f64(w_uq))


def folded_query(cq, w_fold):
    """q~_{n,i} = W_fold,i c^Q_n.  cq [N, d_q], w_fold [H, d_c, d_q] -> [N, H, d_c]."""
    return np.einsum("hcq,nq->nhc", _f64(w_fold), _f64(cq))
