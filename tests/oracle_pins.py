"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, an invariant, a special case that reduces to a library
routine, brute force on a tiny input, or a figure the pages print.  The test
modules call them directly, and the mutation tests plant plausible mistakes
in the oracle and check that at least one pin fails.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import accounting, attention, front, obstruction, paging, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def _small_problem(seed=0, n_heads=3, d_h=8, d_v=6, d_c=12, d_r=8, t=40, n=2):
    rng = np.random.default_rng(seed)
    return dict(
        qc=rng.standard_normal((n, n_heads, d_h)),
        qr=rng.standard_normal((n, n_heads, d_r)),
        c=rng.standard_normal((t, d_c)),
        kr=rng.standard_normal((t, d_r)),
        w_uk=rng.standard_normal((n_heads, d_h, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((n_heads, d_v, d_c)) / math.sqrt(d_c),
        scale=1.0 / math.sqrt(d_h + d_r),
    )


# ---------------------------------------------------------------- RoPE ----

def pin_rope_identity_at_zero():
    """R_0 = I exactly (every angle is 0)."""
    for d in (2, 8, 64):
        assert np.array_equal(rope.rotation_matrix(0, d), np.eye(d))
        x = np.random.default_rng(d).standard_normal(d)
        assert np.array_equal(rope.rotate(x, 0), x)


def pin_rope_closed_form():
    """theta_j = base^(-2j/d): theta_0 = 1 and, for d = 4, theta_1 = 10000^(-1/2) = 0.01.

    With theta_0 = 1 the first plane turns by exactly p radians, counter-
    clockwise: e_0 -> (cos p, sin p), e_1 -> (-sin p, cos p).  Pairs are
    (2j, 2j+1): rotating e_2 in 8 dims moves only coordinates 2 and 3.
    """
    th = rope.thetas(4)
    assert th[0] == 1.0 and abs(th[1] - 0.01) < 1e-17
    th64 = rope.thetas(64)
    assert abs(th64[16] - 0.01) < 1e-17 and abs(th64[31] - 10000.0 ** (-62 / 64)) < 1e-18
    for p in (1, 3, 255):
        got = rope.rotate(np.array([1.0, 0.0]), p)
        assert np.allclose(got, [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
        got = rope.rotate(np.array([0.0, 1.0]), p)
        assert np.allclose(got, [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)
    e2 = np.zeros(8)
    e2[2] = 1.0
    got = rope.rotate(e2, 7)
    a = 7 * 10000.0 ** (-2 / 8)
    want = np.zeros(8)
    want[2], want[3] = math.cos(a), math.sin(a)
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # the vectorised rotation and the explicit matrix agree
    x = np.random.default_rng(1).standard_normal(32)
    for p in (0, 5, 1000, 131071):
        assert np.allclose(rope.rotation_matrix(p, 32) @ x, rope.rotate(x, p), rtol=0, atol=1e-12)


def pin_rope_orthogonal():
    for p in (1, 17, 4095, 131071):
        r = rope.rotation_matrix(p, 64)
        assert np.max(np.abs(r.T @ r - np.eye(64))) < 1e-13


def pin_rope_relative():
    """R_t^T R_m = R_{m-t} (the RoPE relative property)."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        t, m = (int(v) for v in rng.integers(0, 1024, size=2))
        lhs = rope.rotation_matrix(t, 64).T @ rope.rotation_matrix(m, 64)
        assert np.max(np.abs(lhs - rope.rotation_matrix(m - t, 64))) < 1e-12
    p_max = 1 << 17
    bound = 16 * 2.0 ** -52 * p_max
    for _ in range(10):
        t, m = (int(v) for v in rng.integers(0, p_max, size=2))
        lhs = rope.rotation_matrix(t, 64).T @ rope.rotation_matrix(m, 64)
        assert np.max(np.abs(lhs - rope.rotation_matrix(m - t, 64))) < bound


def pin_shift_invariance():
    """Shifting every position by a constant leaves scores, and so outputs, unchanged."""
    pb = _small_problem(seed=3, t=30, n=3)
    q_pos = np.array([29, 10, 20])
    base = attention.materialised(pb["qc"], pb["qr"], q_pos, pb["c"], pb["kr"], pb["w_uk"],
                                  pb["w_uv"], pb["scale"], causal=True)
    for delta in (1, 1000, 1 << 17):
        sh = attention.materialised(pb["qc"], pb["qr"], q_pos + delta, pb["c"], pb["kr"], pb["w_uk"],
                                    pb["w_uv"], pb["scale"], causal=True, key_offset=delta)
        for k in ("o", "obar", "lse"):
            assert _rel(sh[k], base[k]) < 1e-9, (k, delta)
    # and a shift of the query alone does change them (the test can see a mistake)
    moved = attention.materialised(pb["qc"], pb["qr"], q_pos, pb["c"], pb["kr"], pb["w_uk"],
                                   pb["w_uv"], pb["scale"], causal=True, key_offset=1)
    assert _rel(moved["lse"][0], base["lse"][0]) > 1e-6


# ----------------------------------------------------------- attention ----

def pin_absorbed_equals_materialised():
    """Absorption is exact: q~ = W_UK^T q^C and W_UV sum(alpha c) reproduce the definition."""
    for causal in (False, True):
        pb = _small_problem(seed=11, n_heads=4, d_h=16, d_v=16, d_c=32, d_r=8, t=200, n=5)
        q_pos = np.array([199, 150, 3, 0, 120]) if causal else np.full(5, 199)
        m = attention.materialised(pb["qc"], pb["qr"], q_pos, pb["c"], pb["kr"], pb["w_uk"],
                                   pb["w_uv"], pb["scale"], causal=causal, key_chunk=64)
        a = attention.absorbed(pb["qc"], pb["qr"], q_pos, pb["c"], pb["kr"], pb["w_uk"],
                               pb["w_uv"], pb["scale"], causal=causal)
        for k in ("o", "obar", "lse"):
            assert _rel(a[k], m[k]) <= 1e-12, (k, causal, _rel(a[k], m[k]))


def pin_key_rank():
    """The materialised content-key matrix [T x H d_h] has rank exactly d_c (T > d_c)."""
    rng = np.random.default_rng(5)
    t, h, d_h, d_c, d_r = 96, 4, 16, 24, 8
    c = rng.standard_normal((t, d_c))
    kr = rng.standard_normal((t, d_r))
    w_uk = rng.standard_normal((h, d_h, d_c))
    k = attention.materialise_keys(c, kr, w_uk, np.arange(t))
    content = k[:, :, :d_h].reshape(t, h * d_h)
    sv = np.linalg.svd(content, compute_uv=False)
    assert sv[d_c - 1] / sv[0] > 1e-8 and sv[d_c] / sv[0] < 1e-13
    # with the shared position key appended once, the rank is d_c + d_r
    full = np.concatenate([content, k[:, 0, d_h:]], axis=1)
    sv = np.linalg.svd(full, compute_uv=False)
    assert sv[d_c + d_r - 1] / sv[0] > 1e-8 and sv[d_c + d_r] / sv[0] < 1e-13
    # each head's key carries the same rotated k^R
    assert np.array_equal(k[:, 0, d_h:], k[:, h - 1, d_h:])


def pin_brute_force():
    """2 heads x 4 tokens: scalar loops agree with the vectorised definition."""
    rng = np.random.default_rng(13)
    args = dict(qc=rng.standard_normal((2, 2, 2)), qr=rng.standard_normal((2, 2, 2)),
                c=rng.standard_normal((4, 3)), kr=rng.standard_normal((4, 2)),
                w_uk=rng.standard_normal((2, 2, 3)), w_uv=rng.standard_normal((2, 2, 3)), scale=0.7)
    for causal, q_pos in ((False, np.array([3, 3])), (True, np.array([3, 1]))):
        bf = attention.brute_force(args["qc"], args["qr"], q_pos, args["c"], args["kr"], args["w_uk"],
                                   args["w_uv"], args["scale"], causal=causal)
        m = attention.materialised(args["qc"], args["qr"], q_pos, args["c"], args["kr"], args["w_uk"],
                                   args["w_uv"], args["scale"], causal=causal)
        for k in ("o", "obar", "lse"):
            assert _rel(m[k], bf[k]) <= 1e-14, (k, causal)


def pin_special_cases():
    """T = 1 gives obar = c_0 exactly; zero queries give uniform weights; no keys gives 0 / -inf."""
    pb = _small_problem(seed=17, t=1, n=1)
    m = attention.materialised(pb["qc"], pb["qr"], [0], pb["c"], pb["kr"], pb["w_uk"], pb["w_uv"],
                               pb["scale"])
    assert np.array_equal(m["obar"][0, 0], pb["c"][0])
    pb = _small_problem(seed=19, t=33, n=1)
    zq = np.zeros_like(pb["qc"])
    zr = np.zeros_like(pb["qr"])
    m = attention.materialised(zq, zr, [32], pb["c"], pb["kr"], pb["w_uk"], pb["w_uv"], pb["scale"])
    assert _rel(m["obar"][0, 1], pb["c"].mean(axis=0)) < 1e-14
    assert abs(m["lse"][0, 0] - math.log(33)) < 1e-14
    e = attention.materialised(pb["qc"], pb["qr"], [0], pb["c"][:0], pb["kr"][:0], pb["w_uk"],
                               pb["w_uv"], pb["scale"])
    assert np.all(e["obar"] == 0) and np.all(e["o"] == 0) and np.all(np.isneginf(e["lse"]))


def pin_sdpa():
    """Against torch's scaled_dot_product_attention on the CPU in float64.

    No-RoPE control (q^R = 0): textbook MHA with K = W_UK c, V = W_UV c.
    General case: K = [W_UK c ; R_t k^R], Q = [q^C ; R_m q^R], causal mask.
    """
    import torch
    import torch.nn.functional as F

    pb = _small_problem(seed=23, n_heads=4, d_h=16, d_v=12, d_c=20, d_r=8, t=50, n=6)
    q_pos = np.array([49, 40, 7, 0, 25, 49])
    w_uk, w_uv, c = pb["w_uk"], pb["w_uv"], pb["c"]
    k_content = np.stack([c @ w_uk[i].T for i in range(4)])  # [H, T, d_h], written out per head
    v = np.stack([c @ w_uv[i].T for i in range(4)])         # [H, T, d_v]
    # no-RoPE control
    q = np.transpose(pb["qc"], (1, 0, 2))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k_content),
                                         torch.from_numpy(v), scale=pb["scale"]).numpy()
    m = attention.materialised(pb["qc"], np.zeros_like(pb["qr"]), np.full(6, 49), c, pb["kr"] * 0,
                               w_uk, w_uv, pb["scale"])
    assert _rel(m["o"], np.transpose(ref, (1, 0, 2))) < 1e-13
    # general, causal
    qf = np.concatenate([pb["qc"], rope.rotate(pb["qr"], q_pos[:, None])], axis=-1).transpose(1, 0, 2)
    kro = rope.rotate(pb["kr"], np.arange(50))
    kf = np.concatenate([k_content, np.broadcast_to(kro, (4, 50, 8))], axis=-1)
    mask = torch.from_numpy(np.arange(50)[None, :] <= q_pos[:, None])
    ref = F.scaled_dot_product_attention(torch.from_numpy(np.ascontiguousarray(qf)),
                                         torch.from_numpy(np.ascontiguousarray(kf)),
                                         torch.from_numpy(v), attn_mask=mask, scale=pb["scale"]).numpy()
    m = attention.materialised(pb["qc"], pb["qr"], q_pos, c, pb["kr"], w_uk, w_uv, pb["scale"], causal=True)
    assert _rel(m["o"], np.transpose(ref, (1, 0, 2))) < 1e-13


def pin_prefill_is_decode_of_prefix():
    """A causal query at position m equals a decode over keys 0 .. m."""
    pb = _small_problem(seed=29, t=64, n=4)
    q_pos = np.array([0, 17, 40, 63])
    pre = attention.materialised(pb["qc"], pb["qr"], q_pos, pb["c"], pb["kr"], pb["w_uk"], pb["w_uv"],
                                 pb["scale"], causal=True)
    for i, m in enumerate(q_pos):
        dec = attention.materialised(pb["qc"][i:i + 1], pb["qr"][i:i + 1], [m], pb["c"][:m + 1],
                                     pb["kr"][:m + 1], pb["w_uk"], pb["w_uv"], pb["scale"])
        for k in ("o", "obar", "lse"):
            assert _rel(pre[k][i], dec[k][0]) < 1e-13, (k, int(m))


def pin_decode_batch():
    """The batch driver: query b sits at position T_b - 1 and sees that sequence's rows
    row_offsets[b] .. row_offsets[b] + T_b - 1.

    (1) The tiny fp32 decode workload written out: one query at position 255 over
    the keys of positions 0 .. 255, through the definition itself.  (2) A ragged
    batch with non-zero row offsets and an empty sequence, each sequence against
    the pure-Python brute force on its own rows."""
    import synth

    case = synth.config1()
    got = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                 case.w_uk, case.w_uv, case.shape.scale)
    want = attention.materialised(case.qc, case.qr, np.array([255]), case.c_rows[:256], case.kr_rows[:256],
                                  case.w_uk, case.w_uv, case.shape.scale)
    for k in ("o", "obar", "lse"):
        assert np.array_equal(got[k], want[k]), k
    rng = np.random.default_rng(41)
    lens = np.array([3, 1, 0, 5])
    offs = np.array([0, 3, 4, 4])
    n_h, d_h, d_c, d_r, d_v = 2, 2, 3, 4, 2
    c = rng.standard_normal((9, d_c))
    kr = rng.standard_normal((9, d_r))
    qc = rng.standard_normal((4, n_h, d_h))
    qr = rng.standard_normal((4, n_h, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    w_uv = rng.standard_normal((n_h, d_v, d_c))
    got = attention.decode_batch(lens, c, kr, offs, qc, qr, w_uk, w_uv, 0.6)
    for b in range(4):
        t, r0 = int(lens[b]), int(offs[b])
        if t == 0:  # no visible key
            assert np.all(np.isneginf(got["lse"][b])) and np.all(got["obar"][b] == 0) and np.all(got["o"][b] == 0)
            continue
        bf = attention.brute_force(qc[b:b + 1], qr[b:b + 1], [t - 1], c[r0:r0 + t], kr[r0:r0 + t], w_uk, w_uv, 0.6)
        for k in ("o", "obar", "lse"):
            assert np.max(np.abs(got[k][b] - bf[k][0])) <= 1e-13 * max(1.0, np.max(np.abs(bf[k]))), (k, b)


def pin_prefill_batch():
    """The chunk driver: query j of sequence b sits at position q_start[b] + j, is causal,
    and reads that sequence's rows; each query against the brute force on its own rows."""
    rng = np.random.default_rng(43)
    prior, new = np.array([2, 0, 3]), np.array([2, 3, 0])
    lens = prior + new
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    cu_q = np.concatenate([[0], np.cumsum(new)])
    n_h, d_h, d_c, d_r, d_v = 2, 2, 3, 2, 2
    c = rng.standard_normal((int(lens.sum()), d_c))
    kr = rng.standard_normal((int(lens.sum()), d_r))
    qc = rng.standard_normal((int(new.sum()), n_h, d_h))
    qr = rng.standard_normal((int(new.sum()), n_h, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    w_uv = rng.standard_normal((n_h, d_v, d_c))
    got = attention.prefill_batch(cu_q, prior, c, kr, offs, qc, qr, w_uk, w_uv, 0.8)
    for b in range(3):
        for j in range(int(new[b])):
            g = int(cu_q[b]) + j
            m = int(prior[b]) + j
            r0 = int(offs[b])
            bf = attention.brute_force(qc[g:g + 1], qr[g:g + 1], [m], c[r0:r0 + m + 1], kr[r0:r0 + m + 1], w_uk,
                                       w_uv, 0.8)
            for k in ("o", "obar", "lse"):
                assert np.max(np.abs(got[k][g] - bf[k][0])) <= 1e-13 * max(1.0, np.max(np.abs(bf[k]))), (k, g)


# ------------------------------------------------------ paging, figures ----

def pin_paging():
    """Hand-worked example: page size 4, sequence 1 owns physical pages [5, 2]."""
    table = np.array([[0, 3, -1], [5, 2, -1]], dtype=np.int32)
    assert paging.slot(table, 1, 0, 4) == 20
    assert paging.slot(table, 1, 3, 4) == 23
    assert paging.slot(table, 1, 4, 4) == 8
    assert paging.slot(table, 1, 6, 4) == 10
    assert paging.slot(table, 0, 5, 4) == 13
    try:
        paging.slot(table, 0, 9, 4)
    except IndexError:
        pass
    else:
        raise AssertionError("unallocated page must raise")


def pin_page_figures():
    g = json.load(open(GOLDEN))
    f = g["toy_mha_numbers_per_token"]
    assert accounting.mha(f["shape"]["n_heads"], f["shape"]["d_k"], f["shape"]["d_v"]) == f["value"]
    f = g["toy_mla_numbers_per_token_per_head_rope"]
    toy = accounting.mla_per_head_rope(f["shape"]["d_latent"], f["shape"]["n_heads"], f["shape"]["d_rope"])
    assert toy == f["value"]
    assert abs(accounting.reduction(toy, 4096) - g["toy_reduction_about"]["value"]) <= g["toy_reduction_about"]["abs_tol"]
    f = g["dsv2_mha_dims_per_token"]
    mha = accounting.mha(f["shape"]["n_heads"], f["shape"]["d_h"], f["shape"]["d_h"])
    assert mha == f["value"]
    lat = g["dsv2_latent_dims_per_token"]["value"]
    assert abs(mha / lat - g["dsv2_latent_factor_about"]["value"]) <= 1.0
    f = g["dsv2_decoupled_dims_per_token"]
    dec = accounting.mla_shared_rope(f["shape"]["d_latent"], f["shape"]["d_rope"])
    assert dec == f["value"]
    assert abs(mha / dec - g["dsv2_decoupled_fraction_about"]["value"]) <= g["dsv2_decoupled_fraction_about"]["abs_tol"]


# -------------------------------------------------------- front of layer --
# "AI decoupled RoPE MLA", recap (c = W^DKV h) and decoupled-RoPE section
# (k^R = W^KR h); "Detailed Illustration of the Problem", Step 1 (query
# latent c^Q = W^DQ h, q = W^UQ c^Q) and Step 4 (W^{Q'} = (W^UQ)^T W^UK).

def _front_problem(seed=5, n=3, d_model=10, d_q=7, n_heads=2, d_h=4, d_c=6, d_r=4):
    rng = np.random.default_rng(seed)
    return dict(
        h=rng.standard_normal((n, d_model)),
        w_dkv=rng.standard_normal((d_c, d_model)), w_kr=rng.standard_normal((d_r, d_model)),
        w_dq=rng.standard_normal((d_q, d_model)), w_uq=rng.standard_normal((n_heads, d_h, d_q)),
        w_qr=rng.standard_normal((n_heads, d_r, d_q)), w_uk=rng.standard_normal((n_heads, d_h, d_c)),
    )


def pin_front_unit_vectors():
    """h = e_j picks column j of each down-projection exactly (non-square weights, so a
    transposed weight or an input taken from the wrong side fails)."""
    p = _front_problem()
    d_model = p["h"].shape[1]
    for j in (0, 3, d_model - 1):
        e = np.zeros((1, d_model))
        e[0, j] = 1.0
        assert np.array_equal(front.kv_latent(e, p["w_dkv"])[0], p["w_dkv"][:, j])
        assert np.array_equal(front.position_key(e, p["w_kr"])[0], p["w_kr"][:, j])
        assert np.array_equal(front.query_latent(e, p["w_dq"])[0], p["w_dq"][:, j])
    d_q = p["w_dq"].shape[0]
    for j in (0, d_q - 1):
        e = np.zeros((1, d_q))
        e[0, j] = 1.0
        assert np.array_equal(front.content_query(e, p["w_uq"])[0], p["w_uq"][:, :, j])
        assert np.array_equal(front.position_query(e, p["w_qr"])[0], p["w_qr"][:, :, j])


def pin_front_brute_force():
    """Scalar loops over every index equal the vectorised projections and the fold."""
    p = _front_problem(seed=6)
    h, w_dq, w_uq, w_qr, w_uk = p["h"], p["w_dq"], p["w_uq"], p["w_qr"], p["w_uk"]
    n, d_model = h.shape
    d_q = w_dq.shape[0]
    n_heads, d_h, d_c = w_uk.shape
    cq = front.query_latent(h, w_dq)
    for a in range(n):
        for q in range(d_q):
            assert math.isclose(cq[a, q], sum(w_dq[q, k] * h[a, k] for k in range(d_model)), rel_tol=1e-12,
                                abs_tol=1e-12)
    qc = front.content_query(cq, w_uq)
    fold = front.fold_query_weights(w_uq, w_uk)
    for i in range(n_heads):
        for a in range(n):
            for d in range(d_h):
                assert math.isclose(qc[a, i, d], sum(w_uq[i, d, q] * cq[a, q] for q in range(d_q)), rel_tol=1e-12,
                                    abs_tol=1e-12)
        for c in range(d_c):
            for q in range(d_q):
                want = sum(w_uk[i, d, c] * w_uq[i, d, q] for d in range(d_h))
                assert math.isclose(fold[i, c, q], want, rel_tol=1e-12, abs_tol=1e-12)


def pin_fold_equals_absorbed_query():
    """Folding W_UK into the query weight ahead of time gives the absorbed query of the
    unfolded path ("Detailed Illustration of the Problem", Step 4; "ropeabsorb": exact)."""
    p = _front_problem(seed=7, n=5, d_model=16, d_q=9, n_heads=3, d_h=5, d_c=8)
    cq = front.query_latent(p["h"], p["w_dq"])
    via_fold = front.folded_query(cq, front.fold_query_weights(p["w_uq"], p["w_uk"]))
    via_absorb = attention.query_absorption(p["w_uk"], front.content_query(cq, p["w_uq"]))
    assert _rel(via_fold, via_absorb) <= 1e-12


def pin_latent_path_reduces_to_direct_query():
    """With W_DQ = I the latent path is the direct query W_Q h of the tiny configs
    (W_Q [H d_h, D] rows regrouped per head), a plain matrix product."""
    rng = np.random.default_rng(8)
    n, d_model, n_heads, d_h = 4, 12, 3, 4
    h = rng.standard_normal((n, d_model))
    w_q = rng.standard_normal((n_heads * d_h, d_model))
    got = front.content_query(front.query_latent(h, np.eye(d_model)), w_q.reshape(n_heads, d_h, d_model))
    assert _rel(got, (h @ w_q.T).reshape(n, n_heads, d_h)) <= 1e-14


# ------------------------------------------------------ two-scale score ----
# "AI decoupled RoPE MLA", decoupled-RoPE section: each channel's dot product
# takes its own factor, content over sqrt(d) and position over sqrt(d_r).

def pin_two_scale_brute_force():
    """Scalar loops with the two factors equal the vectorised materialised and absorbed forms
    (causal, with a key offset of 0), and equal factors give the one-scale score."""
    p = _small_problem(seed=40, t=12, n=3)
    args = (p["qc"], p["qr"], np.array([3, 7, 11]), p["c"], p["kr"], p["w_uk"], p["w_uv"], 1.0 / math.sqrt(8))
    ps = 1.0 / math.sqrt(8 // 2)
    want = attention.brute_force(*args, causal=True, position_scale=ps)
    for form in (attention.materialised, attention.absorbed):
        got = form(*args, causal=True, position_scale=ps)
        for k in ("o", "obar", "lse"):
            assert _rel(got[k], want[k]) <= 1e-12, (form.__name__, k)
    same = attention.materialised(*args, causal=True, position_scale=args[-1])
    one = attention.materialised(*args, causal=True)
    for k in ("o", "obar", "lse"):
        assert _rel(same[k], one[k]) <= 1e-14


def pin_two_scale_special_cases():
    """With q^R = 0 the position factor has no effect (bitwise); with q^C = 0 the layer is
    textbook attention of the rotated position query over the rotated position keys with
    scale position_scale and values W_UV c (torch's scaled_dot_product_attention, float64)."""
    import torch

    p = _small_problem(seed=41, t=30, n=2)
    pos = np.array([29, 29])
    zr = np.zeros_like(p["qr"])
    a = attention.materialised(p["qc"], zr, pos, p["c"], p["kr"], p["w_uk"], p["w_uv"], 0.3, position_scale=0.05)
    b = attention.materialised(p["qc"], zr, pos, p["c"], p["kr"], p["w_uk"], p["w_uv"], 0.3, position_scale=2.0)
    for k in ("o", "obar", "lse"):
        assert np.array_equal(a[k], b[k])
    zc = np.zeros_like(p["qc"])
    ps = 0.7
    got = attention.materialised(zc, p["qr"], pos, p["c"], p["kr"], p["w_uk"], p["w_uv"], 0.3, position_scale=ps)
    q = torch.from_numpy(rope.rotate(p["qr"], pos[:, None]).transpose(1, 0, 2).copy())  # [H, N, d_r]
    k = torch.from_numpy(rope.rotate(p["kr"], np.arange(30)))[None].expand(q.shape[0], -1, -1)
    v = torch.from_numpy(np.einsum("hvc,tc->htv", p["w_uv"], p["c"]))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=ps).numpy().transpose(1, 0, 2)
    assert _rel(got["o"], ref) <= 1e-12


# ---------------------------------------------------- per-head position keys ----
# "Multi-Head Latent Attention", "A concrete size comparison": the simplified
# MLA-style cache keeps the latent plus one RoPE key per head (256 + 16 x 32).

def pin_per_head_keys_brute_force():
    """Scalar loops over per-head position keys equal the materialised and absorbed forms,
    causal and not, with one scale and with two."""
    p = _small_problem(seed=50, t=14, n=3)
    rng = np.random.default_rng(51)
    kr = rng.standard_normal((14, 3, 8))
    for causal, ps in ((False, None), (True, 0.4)):
        args = (p["qc"], p["qr"], np.array([13, 5, 9]), p["c"], kr, p["w_uk"], p["w_uv"], p["scale"])
        want = attention.brute_force(*args, causal=causal, position_scale=ps)
        for form in (attention.materialised, attention.absorbed):
            got = form(*args, causal=causal, position_scale=ps)
            for k in ("o", "obar", "lse"):
                assert _rel(got[k], want[k]) <= 1e-12, (form.__name__, causal, k)


def pin_per_head_keys_reduce_to_shared():
    """Every head holding the same position key is the shared-key layout; per-head keys that
    differ change only their own head (head 1's key perturbed leaves heads 0 and 2 bitwise)."""
    p = _small_problem(seed=52, t=20, n=2)
    pos = np.array([19, 19])
    args = (p["qc"], p["qr"], pos, p["c"])
    shared = attention.materialised(*args, p["kr"], p["w_uk"], p["w_uv"], p["scale"])
    tiled = np.repeat(p["kr"][:, None, :], 3, axis=1)
    per = attention.materialised(*args, tiled, p["w_uk"], p["w_uv"], p["scale"])
    for k in ("o", "obar", "lse"):
        assert _rel(per[k], shared[k]) <= 1e-14
    moved = tiled.copy()
    moved[:, 1, :] += 1.0
    per2 = attention.materialised(*args, moved, p["w_uk"], p["w_uv"], p["scale"])
    for k in ("o", "obar", "lse"):
        assert np.array_equal(per2[k][:, [0, 2]], per[k][:, [0, 2]])
        assert not np.allclose(per2[k][:, 1], per[k][:, 1])
    assert accounting.mla_per_head_rope(256, 16, 32) == 768


# ------------------------------------------------- the RoPE obstruction ----
# "ropeabsorb" README, "RoPE spans exactly d_R dimensions and cannot be folded"
# and "Partial absorption is impossible".

def _obstruction_weights(seed, d_r, d_q=6, d_c=5):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((d_r, d_q)), rng.standard_normal((d_r, d_c))


def pin_obstruction_one_pair_by_hand():
    """d_R = 2 (theta = 1) expanded by hand: with W_QR rows q0, q1 and W_UKR rows k0, k1,
    F_delta = cos(delta) (q0 k0^T + q1 k1^T) + sin(delta) (q1 k0^T - q0 k1^T).  Both the
    family and its per-frequency decomposition must equal this, entry by entry."""
    w_qr, w_ukr = _obstruction_weights(11, 2)
    q0, q1, k0, k1 = w_qr[0], w_qr[1], w_ukr[0], w_ukr[1]
    deltas = [0, 1, 2, 7, -3]
    fam = obstruction.family(w_qr, w_ukr, deltas)
    mc, ms = obstruction.frequency_components(w_qr, w_ukr)
    via = obstruction.family_from_components(mc, ms, [1.0], deltas)
    for n, d in enumerate(deltas):
        c, s = math.cos(d), math.sin(d)
        for a in range(w_qr.shape[1]):
            for b in range(w_ukr.shape[1]):
                want = c * (q0[a] * k0[b] + q1[a] * k1[b]) + s * (q1[a] * k0[b] - q0[a] * k1[b])
                assert math.isclose(fam[n, a, b], want, rel_tol=1e-12, abs_tol=1e-12)
                assert math.isclose(via[n, a, b], want, rel_tol=1e-12, abs_tol=1e-12)


def pin_obstruction_is_the_rotated_score():
    """The family at delta = t - m is the operator inside the rotated score: for a query input x
    at position m and a key input y at t, (R_m W_QR x) . (R_t W_UKR y) = x^T F_{t-m} y.  The same
    holds for coupled RoPE with W_UQ, W_UK over the whole head, so that family is the coupled one."""
    rng = np.random.default_rng(12)
    for d_r, fam_fn in ((8, obstruction.family), (12, obstruction.coupled_family)):
        w_q, w_k = _obstruction_weights(13 + d_r, d_r)
        for m, t in ((0, 0), (3, 10), (10, 3), (100, 4095)):
            x = rng.standard_normal(w_q.shape[1])
            y = rng.standard_normal(w_k.shape[1])
            want = float(rope.rotate(w_q @ x, m) @ rope.rotate(w_k @ y, t))
            got = float(x @ fam_fn(w_q, w_k, [t - m])[0] @ y)
            assert math.isclose(got, want, rel_tol=1e-11, abs_tol=1e-11), (d_r, m, t, got, want)


def pin_obstruction_decomposition():
    """The family is the sum of its per-frequency cosine and sine parts at RoFormer's
    frequencies, for several d_R and signed shifts."""
    for d_r in (4, 8, 16):
        w_qr, w_ukr = _obstruction_weights(d_r, d_r)
        deltas = np.array([0, 1, 5, 64, 1000, -17])
        mc, ms = obstruction.frequency_components(w_qr, w_ukr)
        th = np.array([10000.0 ** (-2.0 * j / d_r) for j in range(d_r // 2)])
        assert _rel(obstruction.family(w_qr, w_ukr, deltas),
                    obstruction.family_from_components(mc, ms, th, deltas)) <= 1e-12


def pin_obstruction_span():
    """The span over the shifts is exactly d_R = 2L for distinct nonzero frequencies and never
    more, whatever the weights' scale; the no-RoPE control spans 1; equal frequencies (base 1,
    every theta = 1) span 2 however many pairs there are."""
    deltas = np.arange(4096)
    for d_r in (2, 4, 8, 16):
        w_qr, w_ukr = _obstruction_weights(20 + d_r, d_r, d_q=9, d_c=7)
        for scale in (1.0, 1e-14, 1e6):
            rank, _, gap = obstruction.span(obstruction.family(w_qr * scale, w_ukr, deltas))
            assert rank == d_r and gap < 1e-12, (d_r, scale, rank, gap)
        assert obstruction.span(obstruction.family(w_qr, w_ukr, np.zeros(16)))[0] == 1
        assert obstruction.span(obstruction.family(w_qr, w_ukr, deltas[:64], base=1.0))[0] == min(2, d_r)
    w_uq, w_uk = _obstruction_weights(29, 24, d_q=9, d_c=7)
    assert obstruction.span(obstruction.coupled_family(w_uq, w_uk, deltas))[0] == 24


def pin_obstruction_best_single_matrix():
    """The returned constant minimises the summed squared error (a random step away from it
    raises the error, computed member by member); a frequency sampled over whole periods has
    no constant part (share 1); the no-RoPE control is absorbed exactly (share 0); and the
    residual grows with the range of shifts, as the page reports."""
    w_qr, w_ukr = _obstruction_weights(31, 8)
    fam = obstruction.family(w_qr, w_ukr, np.arange(300))
    m, share = obstruction.best_single_matrix(fam)

    def err(x):
        return sum(float(np.sum((f - x) ** 2)) for f in fam)

    total = sum(float(np.sum(f * f)) for f in fam)
    assert math.isclose(share, err(m) / total, rel_tol=1e-12)
    rng = np.random.default_rng(32)
    for _ in range(4):
        e = rng.standard_normal(m.shape)
        assert err(m + 1e-3 * e) > err(m) and err(m - 1e-3 * e) > err(m)
    mc, ms = obstruction.frequency_components(w_qr[:2], w_ukr[:2])
    periodic = obstruction.family_from_components(mc, ms, [2.0 * math.pi / 8.0], np.arange(64))
    assert abs(obstruction.best_single_matrix(periodic)[1] - 1.0) <= 1e-12
    control = obstruction.family(w_qr, w_ukr, np.zeros(5))
    assert obstruction.best_single_matrix(control)[1] <= 1e-28
    r = obstruction.report()["residual_by_window"]
    assert 0.0 < r[128] < r[1024] < r[4096] < 1.0


ALL_PINS = [
    pin_rope_identity_at_zero, pin_rope_closed_form, pin_rope_orthogonal, pin_rope_relative,
    pin_shift_invariance, pin_absorbed_equals_materialised, pin_key_rank, pin_brute_force,
    pin_special_cases, pin_sdpa, pin_prefill_is_decode_of_prefix, pin_paging, pin_page_figures,
    pin_front_unit_vectors, pin_front_brute_force, pin_fold_equals_absorbed_query,
    pin_latent_path_reduces_to_direct_query, pin_obstruction_one_pair_by_hand, pin_obstruction_is_the_rotated_score,
    pin_obstruction_decomposition,
    pin_obstruction_span, pin_obstruction_best_single_matrix, pin_two_scale_brute_force,
    pin_two_scale_special_cases, pin_per_head_keys_brute_force, pin_per_head_keys_reduce_to_shared,
    pin_decode_batch, pin_prefill_batch,
]


def failing_pins():
    """Names of the pins that fail (exceptions other than AssertionError count as failures)."""
    bad = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - a mutation may break a pin in any way
            bad.append(pin.__name__)
    return bad


__all__ = ["ALL_PINS", "failing_pins", "oracle"]
