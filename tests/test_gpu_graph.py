"""Steps replayed as HIP graphs (as bench.py times them) give the eager results, bit for bit.

Each graph is captured once and replayed several times, with eager work on the
same buffers and a synchronisation between replays; every replay is compared
with the eager step.
"""

import numpy as np
import pytest
import torch

import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _replays_match(run, outputs, clobber, replays=3):
    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(replays):
        clobber()  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, outputs):
            assert torch.equal(t, w), f"replay {r} differs from the eager step"


def test_decode_step_graph():
    case = synth.direct_decode(synth.DSV2, "bf16", [700, 64, 1, 2048, 130], seed=231, shuffle=True)
    dims = G.dims_of(case)
    cache = G.build_cache(case)
    step = mla.DecodeStep(dims, cache, torch.from_numpy(case.seq_lens))
    qc, qr, w_uk, w_uv = G.dev(case.qc, BF), G.dev(case.qr, BF), G.dev(case.w_uk, BF), G.dev(case.w_uv, BF)
    last = case.row_offsets + np.maximum(case.seq_lens - 1, 0)
    new_lat, new_kr = G.dev(case.c_rows[last], BF), G.dev(case.kr_rows[last], BF)

    def clobber():
        step.out.fill_(float("nan"))
        step.out_latent.zero_()
        step.lse.fill_(1.0)
        step.q_lat.zero_()

    _replays_match(lambda: step.run(qc, qr, w_uk, w_uv, new_lat, new_kr), [step.out, step.out_latent, step.lse],
                   clobber)


def test_per_head_decode_step_graph():
    case = synth.direct_decode(synth.TINY, "bf16", [700, 64, 1, 3000], seed=233, shuffle=True, per_head_rope=True)
    dims = G.dims_of(case, precise=False)
    step = mla.PerHeadDecodeStep(dims, case.block_table, case.num_pages, torch.from_numpy(case.seq_lens))
    seqs, pos = case.kv_seq_pos()
    step.write(G.dev(case.c_rows, BF), G.dev(case.kr_rows, BF), torch.from_numpy(seqs).cuda(),
               torch.from_numpy(pos).cuda())
    qc, qr, w_uk, w_uv = G.dev(case.qc, BF), G.dev(case.qr, BF), G.dev(case.w_uk, BF), G.dev(case.w_uv, BF)

    def clobber():
        step.out.fill_(float("nan"))
        step.out_latent.zero_()

    _replays_match(lambda: step.run(qc, qr, w_uk, w_uv), [step.out, step.out_latent, step.lse], clobber)


def test_layer_step_from_hidden_state_graph():
    shape = synth.DSV2
    fc = synth.front_layer(shape, [300, 65, 1], 512, 192, seed=235, shuffle=True)
    dims = mla.MLADims(shape.n_heads, shape.d_head, shape.d_v, shape.d_latent, shape.d_rope, dtype=BF,
                       softmax_scale=shape.scale, rope_base=shape.rope_base, work_dtype=BF)
    cache = mla.LatentCache(dims, fc.block_table, fc.num_pages, fill=0.0)
    step = mla.LayerDecodeStep(dims, cache, torch.from_numpy(fc.seq_lens), 512, 192, False)
    w = {k: G.dev(getattr(fc, k), BF) for k in ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv")}
    h = G.dev(fc.h[: len(fc.seq_lens)], BF)

    def run():
        step.run(h, w["w_dkv"], w["w_kr"], w["w_dq"], w["w_uq"], w["w_qr"], w["w_uk"], w["w_uv"])

    def clobber():
        step.inner.out.fill_(float("nan"))
        step.inner.q_lat.zero_()

    _replays_match(run, [step.inner.out, step.inner.out_latent, step.inner.lse], clobber)
