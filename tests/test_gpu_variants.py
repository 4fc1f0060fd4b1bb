"""GPU parity of the score and layout variants the pages state besides the main form.

Two-scale score ("AI decoupled RoPE MLA", decoupled-RoPE section): the content
dot product over sqrt(d_h) plus the position dot product over sqrt(d_r).  The
library reaches it through ``position_scale``: the calls that write the
rotated query multiply it by position_scale / softmax_scale before its one
rounding, and the attention kernels run unchanged.
"""

import math

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


def two_scales(shape):
    return 1.0 / math.sqrt(shape.d_head), 1.0 / math.sqrt(shape.d_rope)


def _check(got, want, dtype, what, name=None):
    for k in ("o", "obar"):
        if k in got:
            G.assert_close(got[k], want[k], dtype, f"{what} {k}", name=name, output=k)
    G.assert_lse_close(got["lse"], want["lse"], dtype, f"{what} lse", name=name)


def _name(shape):
    return "tiny" if shape is synth.TINY else "dsv2"


def _oracle_decode(case, ps):
    sc, pp = ps
    return attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, sc, case.shape.rope_base, position_scale=pp)


def _oracle_prefill(case, ps):
    sc, pp = ps
    return attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                                   case.qr, case.w_uk, case.w_uv, sc, case.shape.rope_base, position_scale=pp)


@pytest.mark.parametrize("shape,dtype", [(synth.TINY, "f32"), (synth.TINY, "bf16"), (synth.DSV2, "bf16")],
                         ids=["tiny-f32", "tiny-bf16", "dsv2-bf16"])
def test_two_scale_decode(shape, dtype):
    case = cases.two_scale_decode(shape, dtype)
    ps = two_scales(shape)
    name = None if dtype == "f32" else f"two_scale_decode_{_name(shape)}"
    _check(G.run_decode(case, scales=ps), _oracle_decode(case, ps), dtype, "two-scale decode", name)


@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_two_scale_prefill(shape):
    case = cases.two_scale_prefill(shape)
    ps = two_scales(shape)
    _check(G.run_prefill(case, scales=ps), _oracle_prefill(case, ps), "bf16", "two-scale prefill",
           f"two_scale_prefill_{_name(shape)}")


@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_two_scale_prefill_materialised(shape):
    case = cases.two_scale_prefill_materialised(shape)
    ps = two_scales(shape)
    _check(G.run_prefill_mha(case, scales=ps), _oracle_prefill(case, ps), "bf16", "two-scale materialised prefill",
           f"two_scale_mha_{_name(shape)}")


def test_two_scale_is_one_scale_when_equal():
    """position_scale == softmax_scale is the one-scale path, bit for bit."""
    case = synth.direct_decode(synth.DSV2, "bf16", [300, 65], seed=207)
    one = G.run_decode(case)
    same = G.run_decode(case, scales=(case.shape.scale, case.shape.scale))
    for k in ("o", "obar", "lse", "q_lat"):
        assert np.array_equal(one[k], same[k]), k


def test_two_scale_query_projection():
    """mla_q_project writes the rotated q^R times position_scale / softmax_scale, one rounding."""
    shape = synth.DSV2
    fc = synth.front_layer(shape, [9, 40], 512, 192, seed=209, shuffle=True)
    sc, pp = two_scales(shape)
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=BF,
                       softmax_scale=sc, position_scale=pp, rope_base=shape.rope_base, work_dtype=BF)
    n = fc.h.shape[0]
    q_pos = np.arange(n, dtype=np.int32) * 37 % 5000
    ws = B.front_workspace(dims, n, 512, 192)
    q_lat = torch.full((n, shape.n_heads, shape.row), float("nan"), dtype=BF, device="cuda")
    q_nope = torch.empty((n, shape.n_heads, shape.d_head), dtype=BF, device="cuda")
    B.q_project(dims, G.dev(fc.h, BF), G.dev(fc.w_dq, BF), G.dev(fc.w_uq, BF), G.dev(fc.w_qr, BF),
                torch.from_numpy(q_pos).cuda(), q_nope, q_lat, ws)
    torch.cuda.synchronize()
    ratio = pp / sc
    cq = front.query_latent(fc.h, fc.w_dq)
    want = ratio * rope.rotate(front.position_query(cq, fc.w_qr), q_pos[:, None], shape.rope_base)
    a = np.abs(front.position_query(np.abs(cq), np.abs(fc.w_qr)))
    bound = ratio * 2.0 ** -8 * (a[..., 0::2] + a[..., 1::2]).repeat(2, axis=-1)
    got = G.to64(q_lat)[:, :, shape.d_latent:]
    err = np.abs(got - want)
    assert (err <= 2.0 ** -8 * np.abs(want) + bound).all(), float(np.max(err / (bound + 1e-30)))


# ---- per-head position keys ("Multi-Head Latent Attention", "A concrete size
# comparison": latent plus one RoPE key per head, 256 + 16 x 32 = 768 per token)

def _per_head_step(case, precise=True, fill=float("nan"), scales=None):
    dims = G.dims_of(case, precise, scales)
    step = mla.PerHeadDecodeStep(dims, case.block_table, case.num_pages, torch.from_numpy(case.seq_lens), fill=fill)
    seqs, pos = case.kv_seq_pos()
    if len(seqs):
        step.write(G.dev(case.c_rows, BF), G.dev(case.kr_rows, BF), torch.from_numpy(seqs).cuda(),
                   torch.from_numpy(pos).cuda())
    return step


def _run_per_head(case, precise=True, scales=None):
    step = _per_head_step(case, precise, scales=scales)
    out = step.run(G.dev(case.qc, BF), G.dev(case.qr, BF), G.dev(case.w_uk, BF), G.dev(case.w_uv, BF))
    torch.cuda.synchronize()
    return {"o": G.to64(out), "obar": G.to64(step.out_latent), "lse": G.to64(step.lse)}, step


def test_per_head_cache_write():
    """Each row is [c | R_t k^R_{t,0} | ... | R_t k^R_{t,15}], rounded once; other slots keep their poison."""
    case = synth.direct_decode(synth.TINY, "bf16", [70, 5, 130], seed=211, shuffle=True, per_head_rope=True)
    step = _per_head_step(case)
    torch.cuda.synchronize()
    seqs, pos = case.kv_seq_pos()
    data = G.to64(step.cache)
    rows = data[case.block_table[seqs, pos // 64], pos % 64]
    s = case.shape
    assert np.array_equal(rows[:, : s.d_latent], case.c_rows)
    want = rope.rotate(case.kr_rows, pos[:, None], s.rope_base).reshape(len(pos), -1)
    err = np.abs(rows[:, s.d_latent:] - want)
    assert (err <= 2.0 ** -8 * np.abs(want) + 1e-30).all(), float(err.max())
    written = np.zeros(data.shape[:2], bool)
    written[case.block_table[seqs, pos // 64], pos % 64] = True
    assert np.isnan(data[~written]).all()


@pytest.mark.parametrize("precise", [True, False], ids=["f32-q", "bf16-q"])
@pytest.mark.parametrize("split_pages", [None, 1, 3])
def test_per_head_decode(precise, split_pages, monkeypatch):
    if split_pages is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", str(split_pages))
    case = cases.per_head_decode()
    got, _ = _run_per_head(case, precise)
    want = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base)
    _check(got, want, "bf16", "per-head decode", "per_head_f32w" if precise else "per_head_bf16")


def test_per_head_decode_two_scale():
    case = cases.per_head_two_scale()
    ps = two_scales(case.shape)
    got, _ = _run_per_head(case, scales=ps)
    want = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, ps[0], case.shape.rope_base, position_scale=ps[1])
    _check(got, want, "bf16", "per-head two-scale", "per_head_two_scale")


def test_per_head_decode_repeatable():
    case = synth.direct_decode(synth.TINY, "bf16", [700, 64, 3000], seed=217, shuffle=True, per_head_rope=True)
    a, step = _run_per_head(case)
    step.attend()
    torch.cuda.synchronize()
    assert np.array_equal(G.to64(step.out_latent), a["obar"]) and np.array_equal(G.to64(step.lse), a["lse"])


def test_per_head_full_size_sampled():
    """64 sequences of 4096 tokens (the bench's per-head workload), every sequence against the oracle."""
    case = cases.per_head_full()
    got, _ = _run_per_head(case)
    want = attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base,
                                  evaluate=attention.absorbed)
    _check(got, want, "bf16", "per-head full size", "per_head_full")


@pytest.mark.parametrize("per_head", [False, True], ids=["shared", "per-head"])
def test_decode_all_sequences_empty(per_head):
    """A batch with no tokens at all: obar = 0 and lse = -inf for every row, with no workspace."""
    case = synth.direct_decode(synth.TINY, "bf16", [0, 0, 0], seed=221, per_head_rope=per_head)
    dims = G.dims_of(case, precise=False)
    lens = torch.from_numpy(case.seq_lens)
    assert mla.decode_workspace_size(dims, lens) == 0
    q_lat = torch.zeros((3, dims.n_heads, dims.row), dtype=BF, device="cuda")
    out = torch.full((3, dims.n_heads, dims.d_latent), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.zeros((3, dims.n_heads), dtype=torch.float32, device="cuda")
    table = torch.from_numpy(case.block_table).cuda()
    if per_head:
        cache = torch.zeros((1, 64, mla.per_head_row(dims)), dtype=BF, device="cuda")
        mla.decode_per_head(dims, cache, table, q_lat, lens.cuda(), lens, out, lse)
    else:
        cache = torch.zeros((1, 64, dims.row), dtype=BF, device="cuda")
        mla.decode(dims, cache, table, q_lat, lens.cuda(), lens, out, lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
