"""The debug mode (MLA_DEBUG_VALIDATE=1): paging data the kernels would clamp or skip is
reported as an error before any compute launch, and valid data changes nothing.

Every bad case here runs only the device check (one workgroup reading the block table
and the row lists within their bounds): the error is returned before the attention or
RoPE kernels launch, which the tests confirm by the outputs keeping their poison.
"""

import numpy as np
import pytest
import torch

import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _decode_setup(lens=(700, 64, 1, 2048, 130), seed=331):
    case = synth.direct_decode(synth.DSV2, "bf16", list(lens), seed=seed, shuffle=True)
    dims = G.dims_of(case)
    cache = G.build_cache(case)
    step = mla.DecodeStep(dims, cache, torch.from_numpy(case.seq_lens))
    step.run(G.dev(case.qc, BF), G.dev(case.qr, BF), G.dev(case.w_uk, BF), G.dev(case.w_uv, BF))
    torch.cuda.synchronize()
    return case, dims, cache, step


def test_valid_data_passes_and_changes_nothing(monkeypatch):
    case, dims, cache, step = _decode_setup()
    w_uv = G.dev(case.w_uv, BF)
    want_obar, want_lse = step.out_latent.clone(), step.lse.clone()
    step.attend_proj(w_uv)
    torch.cuda.synchronize()
    want_o = step.out.clone()
    monkeypatch.setenv("MLA_DEBUG_VALIDATE", "1")
    step.out_latent.fill_(float("nan"))
    mla.decode(dims, cache.data, cache.block_table, step.q_lat, step.seq_lens, step.seq_lens_host, step.out_latent,
               step.lse, step.workspace)
    step.out.fill_(float("nan"))
    step.attend_proj(w_uv)
    torch.cuda.synchronize()
    assert torch.equal(step.out_latent, want_obar) and torch.equal(step.lse, want_lse)
    assert torch.equal(step.out, want_o)


def test_bad_page_id_is_reported_before_any_launch(monkeypatch):
    case, dims, cache, step = _decode_setup()
    bad = cache.block_table.clone()
    bad[3, 17] = cache.data.shape[0] + 5  # sequence 3 (2048 tokens) reads page 17
    monkeypatch.setenv("MLA_DEBUG_VALIDATE", "1")
    step.out_latent.fill_(float("nan"))
    with pytest.raises(mla.MLAError, match=r"block_table\[3\]\[17\]"):
        mla.decode(dims, cache.data, bad, step.q_lat, step.seq_lens, step.seq_lens_host, step.out_latent, step.lse,
                   step.workspace)
    step.out.fill_(float("nan"))
    with pytest.raises(mla.MLAError, match=r"block_table\[3\]\[17\]"):
        mla.decode_proj(dims, cache.data, bad, step.q_lat, step.seq_lens, step.seq_lens_host, G.dev(case.w_uv, BF),
                        step.out, step.lse, step.proj_workspace)
    torch.cuda.synchronize()
    assert torch.isnan(step.out_latent).all() and torch.isnan(step.out).all()
    bad[3, 17] = -1
    with pytest.raises(mla.MLAError, match="block_table"):
        mla.decode(dims, cache.data, bad, step.q_lat, step.seq_lens, step.seq_lens_host, step.out_latent, step.lse,
                   step.workspace)


def test_device_lengths_must_match_host_copies(monkeypatch):
    case, dims, cache, step = _decode_setup()
    lens_dev = step.seq_lens.clone()
    lens_dev[2] = 5  # the host plans with 1
    monkeypatch.setenv("MLA_DEBUG_VALIDATE", "1")
    with pytest.raises(mla.MLAError, match="host copies"):
        mla.decode(dims, cache.data, cache.block_table, step.q_lat, lens_dev, step.seq_lens_host, step.out_latent,
                   step.lse, step.workspace)
    lens_dev[2] = 64 * cache.block_table.shape[1] + 1  # beyond the table on the device only
    with pytest.raises(mla.MLAError, match="beyond its block table"):
        mla.decode(dims, cache.data, cache.block_table, step.q_lat, lens_dev, step.seq_lens_host, step.out_latent,
                   step.lse, step.workspace)
    torch.cuda.synchronize()


def test_cache_rows_without_a_page_are_reported(monkeypatch):
    case, dims, cache, step = _decode_setup()
    n = case.batch
    lat = torch.zeros((n, dims.d_latent), dtype=BF, device="cuda")
    kr = torch.zeros((n, dims.d_rope), dtype=BF, device="cuda")
    seq = torch.arange(n, dtype=torch.int32, device="cuda")
    pos = step.q_pos.clone()
    pos[1] = 64 * cache.block_table.shape[1]  # past the block table
    before = cache.data.clone()
    monkeypatch.setenv("MLA_DEBUG_VALIDATE", "1")
    with pytest.raises(mla.MLAError, match=r"cache row 1 \(sequence 1"):
        mla.rope_apply(dims, cache.data, cache.block_table, kv_latent=lat, k_rope=kr, kv_seq=seq, kv_pos=pos)
    q_lat = torch.full_like(step.q_lat, float("nan"))
    with pytest.raises(mla.MLAError, match=r"cache row 1 \(sequence 1"):
        mla.rope_absorb_q(dims, cache.data, cache.block_table, G.dev(case.qc, BF), G.dev(case.w_uk, BF),
                          G.dev(case.qr, BF), step.q_pos, q_lat, lat, kr, seq, pos)
    torch.cuda.synchronize()
    assert torch.equal(cache.data.view(torch.int16), before.view(torch.int16))  # nothing written (NaN-safe compare)
    assert torch.isnan(q_lat).all()


def test_prefill_bad_page_is_reported(monkeypatch):
    case = synth.direct_prefill(synth.DSV2, "bf16", [0, 100, 64, 7], [5, 130, 1, 64], seed=337, shuffle=True)
    dims = G.dims_of(case)
    cache = G.build_cache(case)
    step = mla.PrefillStep(dims, cache, torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start))
    bad = cache.block_table.clone()
    last = int(np.argmax(case.q_start + np.diff(case.cu_q)))
    bad[last, 0] = cache.data.shape[0]
    monkeypatch.setenv("MLA_DEBUG_VALIDATE", "1")
    step.out_latent.fill_(float("nan"))
    with pytest.raises(mla.MLAError, match=rf"block_table\[{last}\]\[0\]"):
        mla.prefill(dims, cache.data, bad, step.q_lat, step.cu_q, step.q_start, step.cu_q_host, step.q_start_host,
                    step.out_latent, step.lse)
    torch.cuda.synchronize()
    assert torch.isnan(step.out_latent).all()
