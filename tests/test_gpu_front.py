"""GPU parity of the front of the layer (mla_kv_project, mla_q_project,
mla_q_project_folded, mla_fold_q_weights) against the float64 oracle.

The oracle forms c = W_DKV h, k^R = W_KR h, c^Q = W_DQ h and the queries in
float64 from the same bf16 inputs; the GPU sums in float32 over K splits and
rounds each output to bf16 once, and rounds the query latent c^Q to bf16 on
the way (a rounding the oracle does not make).  Bounds, elementwise:
* one projection (c, k^R, W_fold): |err| <= 2^-8 |want| + 1e-3 rms(row) --
  one bf16 rounding (2^-9 relative) plus float32 sums;
* outputs behind the rounded c^Q (q^C, q^R, q~): |err| <= 2^-8 |want| +
  2^-8 sum_j |W_ij| |c^Q_j| -- the worst case of rounding every c^Q_j by 2^-9
  (doubled for margin), plus W_fold's own rounding for q~; a rotation mixes a
  pair, so a rotated pair takes the sum of its two bounds.
The layer output o formed from h takes the configured bf16 bound, widened
where the storage-rounding model predicts more: this path also rounds the
cache rows c and R k^R, the query latent c^Q and the content query q^C (or the
folded weight) to bf16, which the model feeds to the attention's own roundings
(tests/tolerances.py, names front_*).
"""

import numpy as np
import pytest
import torch

import cases
import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth
from mla_decoupled_rope_amd import binding as B
from oracle import attention, front, rope

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _dims(shape):
    return mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=BF,
                       softmax_scale=shape.scale, rope_base=shape.rope_base, page_size=shape.page_size,
                       work_dtype=BF)


def _assert_single_rounding(got, want, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    bound = 2.0 ** -8 * np.abs(want) + 1e-3 * rms
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bounds, worst {np.max(np.abs(got - want) / (rms + 1e-30)):.3e}"


def _assert_within(got, want, bound, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bad = err > 2.0 ** -8 * np.abs(want) + bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} out of bounds, worst err/bound {np.max(err / (2.0 ** -8 * np.abs(want) + bound)):.3f}"


def _pair_sum(a):
    """Each element's bound becomes its pair's (2j, 2j+1) total (a rotation mixes the pair)."""
    a = np.asarray(a, np.float64)
    p = a[..., 0::2] + a[..., 1::2]
    out = np.empty_like(a)
    out[..., 0::2] = p
    out[..., 1::2] = p
    return out


def _cache_rows(cache, fc, seqs, pos):
    data = G.to64(cache.data)
    pages = fc.block_table[seqs, pos // fc.shape.page_size]
    return data[pages, pos % fc.shape.page_size]


def _front_case(shape, lens, d_model, d_qlat, seed):
    return synth.front_layer(shape, lens, d_model, d_qlat, seed=seed, shuffle=True)


def _name(shape):
    return "tiny" if shape is synth.TINY else "dsv2"


SMALL = [(synth.TINY, 256, 96), (synth.DSV2, 512, 192)]


@pytest.mark.parametrize("shape,d_model,d_qlat", SMALL, ids=["tiny", "dsv2"])
def test_kv_project_writes_cache_rows(shape, d_model, d_qlat):
    fc = _front_case(shape, [70, 5, 130], d_model, d_qlat, seed=11)
    dims = _dims(shape)
    cache = mla.LatentCache(dims, fc.block_table, fc.num_pages, fill=float("nan"))
    seqs, pos = fc.kv_seq_pos()
    n = len(seqs)
    ws = B.front_workspace(dims, n, d_model)
    B.kv_project(dims, cache.data, cache.block_table, G.dev(fc.h, BF), G.dev(fc.w_dkv, BF), G.dev(fc.w_kr, BF),
                 torch.from_numpy(seqs).cuda(), torch.from_numpy(pos).cuda(), ws)
    torch.cuda.synchronize()
    got = _cache_rows(cache, fc, seqs, pos)
    c = front.kv_latent(fc.h, fc.w_dkv)
    kr = rope.rotate(front.position_key(fc.h, fc.w_kr), pos, shape.rope_base)
    _assert_single_rounding(got[:, : shape.d_latent], c, "latent c")
    _assert_single_rounding(got[:, shape.d_latent:], kr, "rotated k^R")
    # slots past each sequence's end keep their poison
    data = G.to64(cache.data)
    written = np.zeros(data.shape[:2], bool)
    written[fc.block_table[seqs, pos // 64], pos % 64] = True
    assert np.isnan(data[~written]).all()


@pytest.mark.parametrize("shape,d_model,d_qlat", SMALL, ids=["tiny", "dsv2"])
@pytest.mark.parametrize("folded", [False, True], ids=["unfolded", "folded"])
@pytest.mark.parametrize("lens", [[9, 40], [200, 100, 3]], ids=["one-tile", "prefill-sized"])
def test_q_project(shape, d_model, d_qlat, folded, lens):
    """Single- and multi-tile token counts (303 tokens: five 64-token tiles, the last ragged)."""
    fc = _front_case(shape, lens, d_model, d_qlat, seed=13)
    dims = _dims(shape)
    n = fc.h.shape[0]
    q_pos = np.arange(n, dtype=np.int32) * 37 % 5000
    ws = B.front_workspace(dims, n, d_model, d_qlat)
    q_lat = torch.full((n, shape.n_heads, shape.row), float("nan"), dtype=BF, device="cuda")
    cq = front.query_latent(fc.h, fc.w_dq)
    qr = rope.rotate(front.position_query(cq, fc.w_qr), q_pos[:, None], shape.rope_base)
    qr_bound = 2.0 ** -8 * _pair_sum(front.position_query(np.abs(cq), np.abs(fc.w_qr)))
    if folded:
        w_fold = torch.empty((shape.n_heads, shape.d_latent, d_qlat), dtype=BF, device="cuda")
        B.fold_q_weights(dims, G.dev(fc.w_uq, BF), G.dev(fc.w_uk, BF), w_fold)
        B.q_project_folded(dims, G.dev(fc.h, BF), G.dev(fc.w_dq, BF), w_fold, G.dev(fc.w_qr, BF),
                           torch.from_numpy(q_pos).cuda(), q_lat, ws)
        torch.cuda.synchronize()
        w_f = front.fold_query_weights(fc.w_uq, fc.w_uk)
        want = front.folded_query(cq, w_f)
        _assert_within(G.to64(q_lat)[:, :, : shape.d_latent], want,
                       2.0 ** -7 * front.folded_query(np.abs(cq), np.abs(w_f)), "folded q~")
    else:
        q_nope = torch.empty((n, shape.n_heads, shape.d_head), dtype=BF, device="cuda")
        B.q_project(dims, G.dev(fc.h, BF), G.dev(fc.w_dq, BF), G.dev(fc.w_uq, BF), G.dev(fc.w_qr, BF),
                    torch.from_numpy(q_pos).cuda(), q_nope, q_lat, ws)
        torch.cuda.synchronize()
        _assert_within(G.to64(q_nope), front.content_query(cq, fc.w_uq),
                       2.0 ** -8 * front.content_query(np.abs(cq), np.abs(fc.w_uq)), "q^C")
        assert torch.isnan(q_lat[:, :, : shape.d_latent].float()).all(), "the unfolded form leaves q_lat's head alone"
    _assert_within(G.to64(q_lat)[:, :, shape.d_latent:], qr, qr_bound, "rotated q^R")


@pytest.mark.parametrize("shape,d_qlat", [(synth.TINY, 96), (synth.DSV2, 1536)], ids=["tiny", "dsv2"])
def test_fold_q_weights(shape, d_qlat):
    fc = _front_case(shape, [1], 32, d_qlat, seed=17)
    dims = _dims(shape)
    w_fold = torch.empty((shape.n_heads, shape.d_latent, d_qlat), dtype=BF, device="cuda")
    B.fold_q_weights(dims, G.dev(fc.w_uq, BF), G.dev(fc.w_uk, BF), w_fold)
    torch.cuda.synchronize()
    heads = [0, shape.n_heads // 2, shape.n_heads - 1]
    want = front.fold_query_weights(fc.w_uq[heads], fc.w_uk[heads])
    _assert_single_rounding(G.to64(w_fold)[heads], want, "W_fold")


@pytest.mark.parametrize("shape,d_model,d_qlat", SMALL, ids=["tiny", "dsv2"])
@pytest.mark.parametrize("folded", [False, True], ids=["unfolded", "folded"])
def test_layer_decode_from_hidden_state(shape, d_model, d_qlat, folded):
    """Cache rows and queries formed on the GPU from h, then decode and output projection,
    against the materialised float64 definition fed by the oracle's projections of h."""
    lens = cases.FRONT_DECODE_LENS
    fc = cases.front_decode(_name(shape))
    dims = _dims(shape)
    cache = mla.LatentCache(dims, fc.block_table, fc.num_pages, fill=float("nan"))
    seqs, pos = fc.kv_seq_pos()
    n_kv = len(seqs)
    batch = len(lens)
    last = fc.row_offsets + np.asarray(lens) - 1
    ws = B.front_workspace(dims, max(n_kv, batch), d_model, d_qlat)
    h = G.dev(fc.h, BF)
    B.kv_project(dims, cache.data, cache.block_table, h, G.dev(fc.w_dkv, BF), G.dev(fc.w_kr, BF),
                 torch.from_numpy(seqs).cuda(), torch.from_numpy(pos).cuda(), ws)
    lens_h = torch.tensor(lens, dtype=torch.int32)
    q_pos = (lens_h - 1).cuda()
    h_q = h[torch.from_numpy(last).cuda()].contiguous()
    q_lat = torch.empty((batch, shape.n_heads, shape.row), dtype=BF, device="cuda")
    w_uk = G.dev(fc.w_uk, BF)
    if folded:
        w_fold = torch.empty((shape.n_heads, shape.d_latent, d_qlat), dtype=BF, device="cuda")
        B.fold_q_weights(dims, G.dev(fc.w_uq, BF), w_uk, w_fold)
        B.q_project_folded(dims, h_q, G.dev(fc.w_dq, BF), w_fold, G.dev(fc.w_qr, BF), q_pos, q_lat, ws)
    else:
        q_nope = torch.empty((batch, shape.n_heads, shape.d_head), dtype=BF, device="cuda")
        B.q_project(dims, h_q, G.dev(fc.w_dq, BF), G.dev(fc.w_uq, BF), G.dev(fc.w_qr, BF), q_pos, q_nope, q_lat, ws)
        B.absorb_q(dims, q_nope, w_uk, q_lat)
    out_lat = torch.empty((batch, shape.n_heads, shape.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((batch, shape.n_heads), dtype=torch.float32, device="cuda")
    B.decode(dims, cache.data, cache.block_table, q_lat, lens_h.cuda(), lens_h, out_lat, lse,
             B.decode_workspace(dims, lens_h))
    out = torch.empty((batch, shape.n_heads, shape.d_v), dtype=torch.float32, device="cuda")
    B.out_proj(dims, out_lat, G.dev(fc.w_uv, BF), out)
    torch.cuda.synchronize()
    c = front.kv_latent(fc.h, fc.w_dkv)
    kr = front.position_key(fc.h, fc.w_kr)
    cq = front.query_latent(fc.h[last], fc.w_dq)
    qc = front.content_query(cq, fc.w_uq)
    qr = front.position_query(cq, fc.w_qr)
    want = attention.decode_batch(np.asarray(lens, np.int32), c, kr, fc.row_offsets, qc, qr, fc.w_uk, fc.w_uv,
                                  shape.scale)
    name = f"front_decode_{_name(shape)}_{'folded' if folded else 'unfolded'}"
    G.assert_close(G.to64(out), want["o"], "bf16", "layer output o", name=name)
    G.assert_lse_close(G.to64(lse), want["lse"], "bf16", name=name)


def test_front_bitwise_repeatable():
    fc = _front_case(synth.DSV2, [50, 14], 512, 192, seed=23)
    dims = _dims(synth.DSV2)
    n = fc.h.shape[0]
    ws = B.front_workspace(dims, n, 512, 192)
    q_pos = torch.arange(n, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        q_nope = torch.empty((n, 128, 128), dtype=BF, device="cuda")
        q_lat = torch.zeros((n, 128, 576), dtype=BF, device="cuda")
        B.q_project(dims, G.dev(fc.h, BF), G.dev(fc.w_dq, BF), G.dev(fc.w_uq, BF), G.dev(fc.w_qr, BF), q_pos,
                    q_nope, q_lat, ws)
        torch.cuda.synchronize()
        outs.append((q_nope.clone(), q_lat.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_front_full_size_decode_batch():
    """The decode-step shape: 64 tokens, d_model 5120, query latent 1536, n_h 128."""
    shape = synth.DSV2
    fc = _front_case(shape, [1] * 64, 5120, 1536, seed=29)
    dims = _dims(shape)
    n = 64
    pos = (np.arange(n, dtype=np.int32) * 61) % 4096
    # sequence b owns pages 64 b .. 64 b + 63; its token sits at position pos[b]
    cache = mla.LatentCache(dims, np.arange(n * 64, dtype=np.int32).reshape(n, 64), n * 64, fill=float("nan"))
    ws = B.front_workspace(dims, n, 5120, 1536)
    h = G.dev(fc.h, BF)
    seqs = torch.arange(n, dtype=torch.int32, device="cuda")
    B.kv_project(dims, cache.data, cache.block_table, h, G.dev(fc.w_dkv, BF), G.dev(fc.w_kr, BF), seqs,
                 torch.from_numpy(pos).cuda(), ws)
    q_nope = torch.empty((n, 128, 128), dtype=BF, device="cuda")
    q_lat = torch.empty((n, 128, 576), dtype=BF, device="cuda")
    B.q_project(dims, h, G.dev(fc.w_dq, BF), G.dev(fc.w_uq, BF), G.dev(fc.w_qr, BF), torch.from_numpy(pos).cuda(),
                q_nope, q_lat, ws)
    torch.cuda.synchronize()
    page = torch.from_numpy(np.arange(n) * 64 + pos // 64).cuda()
    rows = G.to64(cache.data[page, torch.from_numpy(pos % 64).long().cuda()])
    _assert_single_rounding(rows[:, :512], front.kv_latent(fc.h, fc.w_dkv), "latent c")
    _assert_single_rounding(rows[:, 512:], rope.rotate(front.position_key(fc.h, fc.w_kr), pos), "rotated k^R")
    cq = front.query_latent(fc.h, fc.w_dq)
    _assert_within(G.to64(q_nope), front.content_query(cq, fc.w_uq),
                   2.0 ** -8 * front.content_query(np.abs(cq), np.abs(fc.w_uq)), "q^C")
    _assert_within(G.to64(q_lat)[:, :, 512:], rope.rotate(front.position_query(cq, fc.w_qr), pos[:, None]),
                   2.0 ** -8 * _pair_sum(front.position_query(np.abs(cq), np.abs(fc.w_qr))), "rotated q^R")


@pytest.mark.parametrize("shape,d_model,d_qlat", SMALL, ids=["tiny", "dsv2"])
@pytest.mark.parametrize("folded", [False, True], ids=["unfolded", "folded"])
def test_layer_prefill_from_hidden_state(shape, d_model, d_qlat, folded):
    """Prior tokens' rows written from h, then a causal chunk of each sequence (rows and queries
    from h on the GPU, absorbed prefill, output projection) against the float64 definition."""
    prior, new = cases.FRONT_PREFILL
    fc = cases.front_prefill(_name(shape))
    dims = _dims(shape)
    cache = mla.LatentCache(dims, fc.block_table, fc.num_pages, fill=float("nan"))
    h = G.dev(fc.h, BF)
    seqs, pos = fc.kv_seq_pos()
    is_new = pos >= np.asarray(prior)[seqs]
    old_rows = np.nonzero(~is_new)[0]
    new_rows = np.nonzero(is_new)[0]
    ws = B.front_workspace(dims, len(seqs), d_model, d_qlat)
    if len(old_rows):
        idx = torch.from_numpy(old_rows).cuda()
        B.kv_project(dims, cache.data, cache.block_table, h[idx].contiguous(), G.dev(fc.w_dkv, BF),
                     G.dev(fc.w_kr, BF), torch.from_numpy(seqs[old_rows]).cuda(),
                     torch.from_numpy(pos[old_rows]).cuda(), ws)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(new)]), dtype=torch.int32)
    step = mla.LayerPrefillStep(dims, cache, cu_q, torch.tensor(prior, dtype=torch.int32), d_model, d_qlat, folded)
    w_uk = G.dev(fc.w_uk, BF)
    w_up = G.dev(fc.w_uq, BF)
    if folded:
        w_fold = torch.empty((shape.n_heads, shape.d_latent, d_qlat), dtype=BF, device="cuda")
        B.fold_q_weights(dims, w_up, w_uk, w_fold)
        w_up = w_fold
    out = step.run(h[torch.from_numpy(new_rows).cuda()].contiguous(), G.dev(fc.w_dkv, BF), G.dev(fc.w_kr, BF),
                   G.dev(fc.w_dq, BF), w_up, G.dev(fc.w_qr, BF), w_uk, G.dev(fc.w_uv, BF))
    torch.cuda.synchronize()
    c = front.kv_latent(fc.h, fc.w_dkv)
    kr = front.position_key(fc.h, fc.w_kr)
    cq = front.query_latent(fc.h[new_rows], fc.w_dq)
    qc = front.content_query(cq, fc.w_uq)
    qr = front.position_query(cq, fc.w_qr)
    want = attention.prefill_batch(cu_q.numpy(), np.asarray(prior), c, kr, fc.row_offsets, qc, qr, fc.w_uk,
                                   fc.w_uv, shape.scale)
    name = f"front_prefill_{_name(shape)}_{'folded' if folded else 'unfolded'}"
    G.assert_close(G.to64(out), want["o"], "bf16", "layer prefill output o", name=name)
    G.assert_lse_close(G.to64(step.inner.lse), want["lse"], "bf16", name=name)
