"""Why RoPE cannot be absorbed: the position-operator family and its span, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring); also runnable as
``python -m oracle.obstruction`` for a printed report.

Source: "ropeabsorb" README (github.com/v-code01), sections "RoPE spans exactly
d_R dimensions and cannot be folded" and "Partial absorption is impossible".
Routing the rotated key through the latent puts the family
    F_delta = W_QR^T R_delta W_UKR          (delta = key position - query position)
between the query input and the latent; a single absorbing matrix exists only
if F_delta does not depend on delta.  Each 2 x 2 rotation block l (frequency
theta_l) contributes cos(theta_l delta) M_l^c + sin(theta_l delta) M_l^s, so
for L = d_R / 2 distinct nonzero frequencies the family spans exactly 2L = d_R
dimensions; with no rotation it spans one (absorbable); one frequency alone
already spans two.  The best single matrix in least squares is the family's
mean over the shifts (its DC part); the rest is oscillation, and its share of
the energy grows with the range of shifts.  Coupled RoPE (the rotation on the
content channel itself, between W_UQ^T and W_UK) gives the same family over
the whole head width, which is why the content channel is kept unrotated and
the position channel decoupled.

Readings: R_delta is the oracle's rotation (``rope.rotation_matrix``: pairs
(2j, 2j+1), counter-clockwise, theta_j = base^(-2j/d_R)); the family is
sampled at the integer shifts 0 .. window - 1 (or, as an alternative
reading, -(window - 1) .. window - 1); "energy" is the squared
Frobenius norm summed over the shifts.  The page's residual figures (0.69,
0.84, 0.94 for windows of 128, 1024, 4096) come from a setup it does not
state, so this module reports its own and pins none of them (parity
unpinned for those three numbers).
"""

from __future__ import annotations

import numpy as np

from . import rope

# J rotates a pair by +90 degrees: R(a) = cos(a) I + sin(a) J on each 2 x 2 block.
_J = np.array([[0.0, -1.0], [1.0, 0.0]])


def family(w_qr, w_ukr, deltas, base: float = 10000.0) -> np.ndarray:
    """F_delta = W_QR^T R_delta W_UKR for each shift.  w_qr [d_R, d_q], w_ukr [d_R, d_c] -> [n, d_q, d_c]."""
    w_qr = np.asarray(w_qr, np.float64)
    w_ukr = np.asarray(w_ukr, np.float64)
    d_r = w_qr.shape[0]
    return np.stack([w_qr.T @ rope.rotation_matrix(float(d), d_r, base) @ w_ukr for d in deltas])


def coupled_family(w_uq, w_uk, deltas, base: float = 10000.0) -> np.ndarray:
    """Coupled RoPE (the rotation applied to the content query and key themselves, between
    W_UQ^T and W_UK): the operator between the query latent and the latent is
    W_UQ^T R_delta W_UK, the same family with the whole head dimension rotated.
    w_uq [d_h, d_q], w_uk [d_h, d_c] (one head) -> [n, d_q, d_c]."""
    return family(w_uq, w_uk, deltas, base)


def frequency_components(w_qr, w_ukr):
    """(M^c, M^s), each [L, d_q, d_c]: block l's cosine and sine coefficient matrices,
    M_l^c = W_QR,l^T W_UKR,l and M_l^s = W_QR,l^T J W_UKR,l over the pair rows (2l, 2l+1)."""
    w_qr = np.asarray(w_qr, np.float64)
    w_ukr = np.asarray(w_ukr, np.float64)
    half = w_qr.shape[0] // 2
    mc = np.stack([w_qr[2 * l:2 * l + 2].T @ w_ukr[2 * l:2 * l + 2] for l in range(half)])
    ms = np.stack([w_qr[2 * l:2 * l + 2].T @ _J @ w_ukr[2 * l:2 * l + 2] for l in range(half)])
    return mc, ms


def family_from_components(mc, ms, thetas, deltas) -> np.ndarray:
    """sum_l cos(theta_l delta) M_l^c + sin(theta_l delta) M_l^s for each shift."""
    th = np.asarray(thetas, np.float64)
    out = []
    for d in deltas:
        a = th * float(d)
        out.append(np.tensordot(np.cos(a), mc, axes=1) + np.tensordot(np.sin(a), ms, axes=1))
    return np.stack(out)


def span(fam: np.ndarray, cliff: float = 1e-10):
    """(rank, singular values, cliff ratio) of the family's span: the members flattened to
    rows of a matrix; the rank counts singular values above `cliff` times the largest, and
    the ratio is the first singular value past the rank over the largest (the size of the gap)."""
    rows = np.asarray(fam, np.float64).reshape(len(fam), -1)
    sv = np.linalg.svd(rows, compute_uv=False)
    if sv.size == 0 or sv[0] == 0.0:
        return 0, sv, 0.0
    rank = int(np.sum(sv > cliff * sv[0]))
    ratio = float(sv[rank] / sv[0]) if rank < sv.size else 0.0
    return rank, sv, ratio


def best_single_matrix(fam: np.ndarray):
    """(M, residual share): the least-squares constant M = mean over the shifts (the DC part)
    and the share of the family's energy it leaves, sum ||F - M||^2 / sum ||F||^2."""
    fam = np.asarray(fam, np.float64)
    m = fam.mean(axis=0)
    total = float(np.sum(fam * fam))
    resid = float(np.sum((fam - m) ** 2))
    return m, (resid / total if total > 0 else 0.0)


def report(d_r: int = 16, d_q: int = 24, d_c: int = 20, d_h: int = 32, base: float = 10000.0, seed: int = 0,
           windows=(128, 1024, 4096), symmetric: bool = False) -> dict:
    """The page's measurements under this module's readings: the span of the RoPE family, the
    no-RoPE control, a single frequency, coupled RoPE over a d_h-wide head, and the
    best-single-matrix residual per window (shifts 0 .. w-1, or -(w-1) .. w-1 if symmetric)."""
    rng = np.random.default_rng(seed)
    w_qr = rng.standard_normal((d_r, d_q))
    w_ukr = rng.standard_normal((d_r, d_c))
    w_uq = rng.standard_normal((d_h, d_q))
    w_uk = rng.standard_normal((d_h, d_c))
    far = max(windows)
    deltas = np.arange(-(far - 1), far) if symmetric else np.arange(far)
    fam = family(w_qr, w_ukr, deltas, base)
    rank, _, ratio = span(fam)
    no_rope = np.stack([w_qr.T @ w_ukr] * 8)  # R_delta = I at every shift
    one = family(w_qr[:2], w_ukr[:2], np.arange(256), base)
    coupled = span(coupled_family(w_uq, w_uk, np.arange(far), base))[0]

    def window(w):
        return fam[np.abs(deltas) < w]

    residuals = {int(w): best_single_matrix(window(w))[1] for w in windows}
    return {"d_R": d_r, "span_rank": rank, "span_cliff": ratio, "no_rope_rank": span(no_rope)[0],
            "single_frequency_rank": span(one)[0], "d_h": d_h, "coupled_rank": coupled,
            "residual_by_window": residuals}


if __name__ == "__main__":  # pragma: no cover
    r = report()
    print(f"d_R = {r['d_R']}: the family spans {r['span_rank']} dimensions (gap {r['span_cliff']:.1e})")
    print(f"no rotation: rank {r['no_rope_rank']} (absorbable); one frequency: rank {r['single_frequency_rank']}")
    print(f"coupled RoPE over a {r['d_h']}-wide head: rank {r['coupled_rank']} (not absorbable)")
    for sym in (False, True):
        for w, v in report(symmetric=sym)["residual_by_window"].items():
            rng_txt = f"-{w - 1}..{w - 1}" if sym else f"0..{w - 1}"
            print(f"best single matrix over shifts {rng_txt}: residual share {v:.3f}")
