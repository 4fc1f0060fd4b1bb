"""mla_decode_noalloc (the split partials in the library's fixed device scratch) against
mla_decode with a caller's workspace: the same kernels and plan, so the same bits."""

import numpy as np
import pytest
import torch

import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth

pytestmark = pytest.mark.gpu


def _both(case):
    """(decode with a workspace, decode_noalloc) on one cache: dicts of obar and lse."""
    dims = G.dims_of(case)
    cache = G.build_cache(case)
    lens = torch.from_numpy(case.seq_lens)
    step = mla.DecodeStep(dims, cache, lens)
    dt = G.tdtype(case)
    q_rope, q_nope = G.dev(case.qr, dt), G.dev(case.qc, dt)
    mla.rope_apply(dims, None, None, q_rope=q_rope, q_pos=step.q_pos, q_lat=step.q_lat)
    mla.absorb_q(dims, q_nope, G.dev(case.w_uk, dt), step.q_lat)
    mla.decode(dims, cache.data, cache.block_table, step.q_lat, step.seq_lens, step.seq_lens_host, step.out_latent,
               step.lse, step.workspace)
    out = torch.full_like(step.out_latent, float("nan"))
    lse = torch.full_like(step.lse, float("nan"))
    mla.decode_noalloc(dims, cache.data, cache.block_table, step.q_lat, step.seq_lens, step.seq_lens_host, out, lse)
    torch.cuda.synchronize()
    return ({"obar": G.to64(step.out_latent), "lse": G.to64(step.lse)}, {"obar": G.to64(out), "lse": G.to64(lse)},
            step.workspace)


@pytest.mark.parametrize("shape", [synth.DSV2, synth.TINY], ids=["dsv2", "tiny"])
def test_noalloc_matches_decode_twice_smaller_second(shape):
    """Two calls in a row on one device, the second with a smaller batch: each equals mla_decode bit for bit."""
    first = synth.direct_decode(shape, "bf16", [700, 2048, 130, 1, 4000, 0, 65], seed=301, shuffle=True)
    second = synth.direct_decode(shape, "bf16", [1500, 9], seed=303, shuffle=True)
    for case in (first, second):
        ref, got, ws = _both(case)
        assert ws is not None, "the case must split some sequence (the scratch must be used)"
        for k in ("obar", "lse"):
            assert np.array_equal(ref[k], got[k], equal_nan=False), k
        assert np.all(np.isfinite(got["obar"]))


def test_noalloc_rejects_a_batch_beyond_its_scratch(monkeypatch):
    """64 sequences of 4160 tokens forced into 4-page splits: 1088 items whose partials need
    over 130 MiB, more than the 96 MiB scratch -- an error before any launch."""
    monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", "4")
    case = synth.direct_decode(synth.DSV2, "bf16", [64] * 4, seed=307)
    dims = G.dims_of(case)
    n = 64
    lens_host = torch.full((n,), 4160, dtype=torch.int32)
    assert mla.decode_workspace_size(dims, lens_host) > 96 << 20
    cache = torch.zeros((1, 64, dims.row), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((n, 66), dtype=torch.int32, device="cuda")
    q_lat = torch.zeros((n, dims.n_heads, dims.row), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((n, dims.n_heads, dims.d_latent), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError, match="fixed scratch"):
        mla.decode_noalloc(dims, cache, table, q_lat, lens_host.cuda(), lens_host, out)
    torch.cuda.synchronize()
