"""Op-level GPU parity: each C-ABI call against the oracle's definition of that step."""

import math

import numpy as np
import pytest
import torch

import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth
from oracle import attention, paging, rope

pytestmark = pytest.mark.gpu

BF16_ULP = 2.0 ** -8  # relative spacing bound of bf16 (one rounding is at most half of it)


@pytest.mark.parametrize("dtype,qdtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_rope_query_rotation(dtype, qdtype, shape):
    """q_lat[..., d_c:] = R_p q^R for positions up to 2^17 - 1 (angles in float64)."""
    rng = np.random.default_rng(11)
    n = 9
    q_r = synth.to_storage(rng.standard_normal((n, shape.n_heads, shape.d_rope)), dtype)
    pos = np.array([0, 1, 2, 255, 4095, 16383, 65536, 131071, 77777], np.int32)
    case_dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q_dt = torch.float32 if qdtype == "f32" else torch.bfloat16
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=case_dt,
                       work_dtype=q_dt)
    q_lat = torch.zeros((n, shape.n_heads, shape.row), dtype=q_dt, device="cuda")
    mla.rope_apply(dims, None, None, q_rope=G.dev(q_r, case_dt), q_pos=torch.from_numpy(pos).cuda(), q_lat=q_lat)
    got = G.to64(q_lat)[..., shape.d_latent:]
    want = rope.rotate(q_r, pos[:, None])
    tol = 1e-6 if qdtype == "f32" else BF16_ULP
    assert np.all(np.abs(got - want) <= tol * np.abs(want) + 1e-30), np.max(np.abs(got - want))
    assert np.all(G.to64(q_lat)[..., :shape.d_latent] == 0), "content columns must be untouched"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_cache_write_paged(dtype):
    """Rows land in block_table[b][p // 64] * 64 + p % 64; the latent is copied bit for bit,
    the position key is rotated to its own position; nothing else is written."""
    shape = synth.DSV2
    lens = [70, 1, 200]
    case = synth.direct_decode(shape, dtype, lens, seed=5, shuffle=True)
    cache = G.build_cache(case)
    torch.cuda.synchronize()
    data = G.to64(cache.data).reshape(-1, shape.row)
    seqs, pos = case.kv_seq_pos()
    slots = paging.slots(case.block_table, seqs, pos, shape.page_size)
    written = np.zeros(len(data), bool)
    written[slots] = True
    assert np.array_equal(data[slots, :shape.d_latent], case.c_rows.astype(np.float64)), "latent copy is not exact"
    want = rope.rotate(case.kr_rows, pos)
    got = data[slots, shape.d_latent:]
    tol = 1e-6 if dtype == "f32" else BF16_ULP
    assert np.all(np.abs(got - want) <= tol * np.abs(want) + 1e-30)
    assert np.all(np.isnan(data[~written])), "rows outside the written slots changed"


def test_rope_cache_write_skips_invalid_rows():
    """Out-of-range sequence, negative position and unallocated pages are skipped."""
    shape = synth.TINY
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope)
    table = np.array([[1, -1], [0, 5]], np.int32)  # page 5 does not exist (2 pages)
    cache = mla.LatentCache(dims, table, 2, fill=float("nan"))
    rng = np.random.default_rng(3)
    c = torch.from_numpy(rng.standard_normal((5, shape.d_latent)).astype(np.float32)).cuda().bfloat16()
    kr = torch.from_numpy(rng.standard_normal((5, shape.d_rope)).astype(np.float32)).cuda().bfloat16()
    seq = torch.tensor([0, 0, 2, 1, 0], dtype=torch.int32).cuda()
    posv = torch.tensor([3, 64, 0, 70, -1], dtype=torch.int32).cuda()
    cache.write(c, kr, seq, posv)
    torch.cuda.synchronize()
    data = G.to64(cache.data).reshape(-1, shape.row)
    ok = ~np.isnan(data).all(axis=1)
    assert ok.sum() == 1 and ok[64 + 3], "only (seq 0, pos 3) -> page 1 row 3 is valid"


@pytest.mark.parametrize("dtype,qdtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("n", [1, 17, 64, 300])
def test_absorb_q(dtype, qdtype, n):
    shape = synth.DSV2 if dtype == "bf16" else synth.TINY
    case = synth.direct_decode(shape, dtype, [1] * n, seed=100 + n)
    dt = G.tdtype(case)
    q_dt = torch.float32 if qdtype == "f32" else torch.bfloat16
    s = case.shape
    dims = mla.MLADims(s.n_heads, s.d_head, s.d_v, s.d_latent, s.d_rope, dtype=dt, work_dtype=q_dt)
    q_lat = torch.full((n, shape.n_heads, shape.row), 7.0, dtype=q_dt, device="cuda")
    mla.absorb_q(dims, G.dev(case.qc, dt), G.dev(case.w_uk, dt), q_lat)
    got = G.to64(q_lat)
    want = attention.query_absorption(case.w_uk, case.qc)
    if qdtype == "f32":  # float32 accumulation of exact bf16 products, no output rounding
        G.assert_close(got[..., :shape.d_latent], want, "f32", "q~")
    else:
        # one RNE rounding of a float32 accumulation, element by element: at most half a
        # spacing of bf16's 8 significant bits (2^-8 |x|), plus the float32 sum's own
        # error (2^-20 of the row's RMS)
        g = got[..., :shape.d_latent]
        rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
        bound = 2.0 ** -8 * np.abs(want) * (1 + 2.0 ** -7) + 2.0 ** -20 * rms
        assert np.all(np.abs(g - want) <= bound), float(np.max(np.abs(g - want) / bound))
    assert np.all(got[..., shape.d_latent:] == 7.0), "rope columns must be untouched"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 31, 64, 257])
def test_out_proj(dtype, n):
    shape = synth.DSV2 if dtype == "bf16" else synth.TINY
    rng = np.random.default_rng(200 + n)
    obar = rng.standard_normal((n, shape.n_heads, shape.d_latent)).astype(np.float32)  # float32 on every path
    w_uv = synth.to_storage(rng.standard_normal((shape.n_heads, shape.d_v, shape.d_latent)) / math.sqrt(shape.d_latent),
                            dtype)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=dt)
    out = torch.empty((n, shape.n_heads, shape.d_v), dtype=torch.float32, device="cuda")
    mla.out_proj(dims, G.dev(obar, torch.float32), G.dev(w_uv, dt), out)
    got = G.to64(out)
    want = attention.output_absorption(w_uv, obar)
    # float32 accumulation, float32 output; with bf16 weights the float32 obar enters as a
    # two-term bf16 split (within 2^-16 of each value): float32-level error on both paths
    G.assert_close(got, want, "f32", "o")


@pytest.mark.parametrize("dtype,qdtype,with_rows", [("bf16", "bf16", True), ("bf16", "f32", True),
                                                      ("bf16", "bf16", False), ("f32", "f32", True)])
@pytest.mark.parametrize("shape", [synth.TINY, synth.DSV2], ids=["tiny", "dsv2"])
def test_rope_absorb_q_is_the_two_calls(dtype, qdtype, with_rows, shape):
    """mla_rope_absorb_q (one launch for bf16) leaves q_lat and the cache bit-identical to
    mla_rope_apply followed by mla_absorb_q, for 300 queries (several token chunks of the
    absorption) and 70 new cache rows."""
    rng = np.random.default_rng(17)
    n, lens = 300, [70, 1, 200]
    case = synth.direct_decode(shape, dtype, lens, seed=19, shuffle=True)
    case_dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q_dt = torch.float32 if qdtype == "f32" else torch.bfloat16
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=case_dt,
                       work_dtype=q_dt)
    q_nope = G.dev(synth.to_storage(rng.standard_normal((n, shape.n_heads, shape.d_head)), dtype), case_dt)
    q_rope = G.dev(synth.to_storage(rng.standard_normal((n, shape.n_heads, shape.d_rope)), dtype), case_dt)
    w_uk = G.dev(case.w_uk, case_dt)
    q_pos = torch.from_numpy(rng.integers(0, 131072, n).astype(np.int32)).cuda()
    seqs, pos = case.kv_seq_pos()
    rows = dict(kv_latent=G.dev(case.c_rows, case_dt), k_rope=G.dev(case.kr_rows, case_dt),
                kv_seq=torch.from_numpy(seqs).cuda(), kv_pos=torch.from_numpy(pos).cuda()) if with_rows else {}
    outs = []
    for fused in (False, True):
        cache = mla.LatentCache(dims, case.block_table, case.num_pages, fill=float("nan"))
        q_lat = torch.full((n, shape.n_heads, shape.row), float("nan"), dtype=q_dt, device="cuda")
        if fused:
            mla.rope_absorb_q(dims, cache.data, cache.block_table, q_nope, w_uk, q_rope, q_pos, q_lat, **rows)
        else:
            mla.rope_apply(dims, cache.data, cache.block_table, q_rope=q_rope, q_pos=q_pos, q_lat=q_lat, **rows)
            mla.absorb_q(dims, q_nope, w_uk, q_lat)
        torch.cuda.synchronize()
        outs.append((q_lat.view(torch.int16 if q_dt == torch.bfloat16 else torch.int32).cpu(),
                     cache.data.view(torch.int16 if case_dt == torch.bfloat16 else torch.int32).cpu()))
    assert torch.equal(outs[0][0], outs[1][0]), "q_lat differs"
    assert torch.equal(outs[0][1], outs[1][1]), "cache differs"
