"""Helpers for the GPU tests: move a synth.Case onto the device through the C ABI,
run decode / prefill steps, and compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import mla_decoupled_rope_amd as mla
import tolerances as T


def tdtype(case) -> torch.dtype:
    return torch.float32 if case.dtype == "f32" else torch.bfloat16


def dims_of(case, precise=None, scales=None) -> mla.MLADims:
    """Library dims for a case.  precise=True selects the float32 working
    precision (float32 q_lat, partials and obar; two-term bf16 q~ and P); by
    default the tiny shape takes it and the DeepSeek-V2 shape works in bf16.
    scales = (content, position) gives each part of the score its own factor
    (the two-scale score); None keeps the shape's one scale on the summed score."""
    s = case.shape
    if precise is None:
        precise = s.row <= 288
    qdt = torch.float32 if (case.dtype == "f32" or precise) else torch.bfloat16
    return mla.MLADims(s.n_heads, s.d_head, s.d_v, s.d_latent, s.d_rope, dtype=tdtype(case),
                       softmax_scale=s.scale if scales is None else scales[0],
                       position_scale=None if scales is None else scales[1], rope_base=s.rope_base,
                       page_size=s.page_size, work_dtype=qdt)


def dev(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def build_cache(case, block_table=None, fill=float("nan")) -> mla.LatentCache:
    """Allocate the paged cache (poisoned with `fill`) and write every token row through mla_rope_apply."""
    dims = dims_of(case)
    table = case.block_table if block_table is None else block_table
    cache = mla.LatentCache(dims, table, case.num_pages, fill=fill)
    seqs, pos = case.kv_seq_pos()
    n = len(seqs)
    chunk = 1 << 20
    dt = tdtype(case)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        cache.write(dev(case.c_rows[r0:r1], dt), dev(case.kr_rows[r0:r1], dt),
                    torch.from_numpy(seqs[r0:r1]).to("cuda"), torch.from_numpy(pos[r0:r1]).to("cuda"))
    return cache


def run_decode(case, cache=None, block_table=None, precise=None, scales=None):
    """Full decode step (q^R rotation, absorption, decode, out_proj).  Returns float64 numpy dict."""
    dims = dims_of(case, precise, scales)
    cache = build_cache(case, block_table) if cache is None else cache
    step = mla.DecodeStep(dims, cache, torch.from_numpy(case.seq_lens))
    dt = tdtype(case)
    w_uk, w_uv = dev(case.w_uk, dt), dev(case.w_uv, dt)
    out = step.run(dev(case.qc, dt), dev(case.qr, dt), w_uk, w_uv)
    torch.cuda.synchronize()
    return {"o": to64(out), "obar": to64(step.out_latent), "lse": to64(step.lse), "q_lat": to64(step.q_lat)}


def run_prefill(case, cache=None, precise=None, scales=None):
    dims = dims_of(case, precise, scales)
    cache = build_cache(case) if cache is None else cache
    step = mla.PrefillStep(dims, cache, torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start))
    dt = tdtype(case)
    out = step.run(dev(case.qc, dt), dev(case.qr, dt), dev(case.w_uk, dt), dev(case.w_uv, dt))
    torch.cuda.synchronize()
    return {"o": to64(out), "obar": to64(step.out_latent), "lse": to64(step.lse), "q_lat": to64(step.q_lat)}


def run_prefill_mha(case, cache=None, scales=None):
    """The prefill step in the materialised form (mla_prefill_mha).  Returns float64 numpy dict with o, lse."""
    dims = dims_of(case, precise=False, scales=scales)
    cache = build_cache(case) if cache is None else cache
    step = mla.PrefillStep(dims, cache, torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start))
    dt = tdtype(case)
    out = step.run_materialised(dev(case.qc, dt), dev(case.qr, dt), dev(case.w_uk, dt), dev(case.w_uv, dt))
    torch.cuda.synchronize()
    return {"o": to64(out), "lse": to64(step.lse)}


def rel_errors(got: np.ndarray, want: np.ndarray):
    """(max|err| / rms(want), rms(err) / rms(want)) over the whole output: the pass metric.

    Rows whose reference is all zero (no visible key) must match exactly."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if want.size == 0:
        return 0.0, 0.0
    err = got - want
    row_rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    zero = row_rms[..., 0] == 0
    assert np.all(err[zero] == 0), "rows with no visible key must be exactly zero"
    rms = np.sqrt(np.mean(want * want))
    if rms == 0:
        return 0.0, 0.0
    return float(np.max(np.abs(err)) / rms), float(np.sqrt(np.mean(err * err)) / rms)


def row_rel_max(got, want) -> float:
    """Diagnostic only: the largest per-row max|err| / rms(that row of want)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    row_rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    ok = row_rms[..., 0] > 0
    if not ok.any():
        return 0.0
    return float(np.max(np.abs(got - want)[ok] / row_rms[ok]))


def assert_close(got, want, dtype: str, what: str = "", tol=None, name: str | None = None, output: str = "o"):
    """The pass metric against the bound: `tol` if given, else tolerances.bound(name, output, dtype)
    (the configured bound, widened only where the rounding model predicts more for input `name`)."""
    mx, rms = rel_errors(got, want)
    tmax, trms = tol if tol is not None else T.bound(name, output, dtype)
    model = ""
    if name is not None:
        fm, fr = T.figure(name, output)
        model = f"; model {fm:.3e} / {fr:.3e}"
    print(f"{what}: rel_max {mx:.3e} (<= {tmax:.3g}), rel_rms {rms:.3e} (<= {trms:.3g}), "
          f"row max {row_rel_max(got, want):.3e}{model}", flush=True)
    assert mx <= tmax and rms <= trms, f"{what}: rel_max {mx:.3e} (<= {tmax}), rel_rms {rms:.3e} (<= {trms})"
    return mx, rms


def assert_lse_close(got, want, dtype: str, what: str = "lse", name: str | None = None):
    """lse is float32 on every path: max and rms absolute error in nats against
    tolerances.bound(name, "lse", dtype)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    if not fin.any():
        return
    err = np.abs(got[fin] - want[fin])
    mx, rms = float(err.max()), float(np.sqrt(np.mean(err * err)))
    tmax, trms = T.bound(name, "lse", dtype)
    print(f"{what}: max {mx:.3e} nats (<= {tmax:.3g}), rms {rms:.3e} (<= {trms:.3g})", flush=True)
    assert mx <= tmax and rms <= trms, f"{what}: max abs error {mx:.3e} (<= {tmax}), rms {rms:.3e} (<= {trms})"
