"""Rotary position operator R_p, float64.

Sources (page title / section / equation):

* "Detailed Illustration of the Problem" (notion.site), Step 1 and Step 3: the
  query and key are rotated by a position-indexed operator R^d_{Theta,p}, and
  the product of two rotations obeys R_t^T R_m = R_{m-t}.
* "AI decoupled RoPE MLA" (operatorworld.com), section on the decoupled
  solution: RoPE acts only on the small position channel q^R, k^R of width
  d_r, and R_m^T R_t depends only on t - m.

The pages never define Theta, the pairing or the direction of rotation.  The
readings used here (stated once, used everywhere):

* Theta: theta_j = base^(-2j/d_r), j = 0 .. d_r/2 - 1, base 10000 (the
  RoFormer frequencies).
* Pairing: coordinates (2j, 2j+1) form the j-th 2-D plane.
* Direction: counter-clockwise by +p*theta_j, i.e. (x, y) ->
  (x cos a - y sin a, x sin a + y cos a) with a = p*theta_j.

Parity is pinned by tests against closed forms (R_0 = I, the 2-D rotation
by one radian, orthogonality, the relative property and shift invariance).
"""

from __future__ import annotations

import numpy as np


def thetas(d_rope: int, base: float = 10000.0) -> np.ndarray:
    """Frequencies theta_j = base^(-2j/d_rope), j = 0 .. d_rope/2 - 1 (float64)."""
    if d_rope <= 0 or d_rope % 2:
        raise ValueError("d_rope must be a positive even number")
    j = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / d_rope)


def rotation_matrix(p: float, d_rope: int, base: float = 10000.0) -> np.ndarray:
    """The explicit d_rope x d_rope block-diagonal matrix R_p."""
    r = np.zeros((d_rope, d_rope), dtype=np.float64)
    for j, th in enumerate(thetas(d_rope, base)):
        a = np.float64(p) * th
        c, s = np.cos(a), np.sin(a)
        r[2 * j, 2 * j] = c
        r[2 * j, 2 * j + 1] = -s
        r[2 * j + 1, 2 * j] = s
        r[2 * j + 1, 2 * j + 1] = c
    return r


def rotate(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Apply R_p to the last axis of ``x``.

    ``x`` has shape [..., d_rope]; ``positions`` broadcasts against
    ``x.shape[:-1]``.  The angle p*theta_j is formed in float64 from an
    integer (or float) position and a float64 theta.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[..., None] * thetas(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
