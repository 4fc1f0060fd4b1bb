"""Benchmark: absorbed MLA decode with decoupled RoPE on one MI355X.

One step = one pass of the decode hot path over a batch: RoPE on the new
query's q^R and the new token's cache row with query absorption in one launch
(mla_rope_absorb_q), split attention over the paged latent cache plus the
split merge (mla_decode), output absorption (mla_out_proj).  Default workload:
64 sequences x 4096 cached tokens, n_h = 128, d_c = 512, d_r = 64, bf16, in
64-token pages.  Three identical cache copies are used in rotation so that
the 256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line.  --config selects other workloads for inspection.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "absorbed MLA decode tokens/s + % HBM roofline (n_h=128,d_c=512,d_r=64)"
HBM_PEAK_GBS = 8000.0
QUERY_LATENT = 1536  # the query latent width of the DeepSeek-V2-like layer
BF16_PEAK_TFLOPS = 2500.0
KERNEL_WARMUP_S = 0.05  # untimed lead-in of the kernel-timing loops (not of the steps)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "mla_decoupled_rope_amd", "csrc", "attn_bf16.hip")
MHA_SRC = os.path.join(ROOT, "mla_decoupled_rope_amd", "csrc", "mha.hip")


GEMM_SRC = os.path.join(ROOT, "mla_decoupled_rope_amd", "csrc", "gemm.hip")


def kernel_hash(src=KERNEL_SRC) -> str:
    """sha256[:16] of a kernel source, or of several sources concatenated in order."""
    srcs = [src] if isinstance(src, str) else list(src)
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16]


def decode_bytes(seq_lens, n_heads=128, d_latent=512, d_rope=64, elt=2, q_elt=2) -> int:
    """Algorithmic HBM bytes of one decode call: cache rows (elt bytes an element)
    read once, the query (q_elt bytes) read once, the float32 latent output
    written once, the block table read once."""
    row = (d_latent + d_rope) * elt
    t = np.asarray(seq_lens, np.int64)
    per_q = n_heads * (d_latent + d_rope) * q_elt + n_heads * d_latent * 4
    return int(np.sum(row * t + per_q + 4 * ((t + 63) // 64)))


def decode_proj_bytes(seq_lens, n_heads=128, d_latent=512, d_rope=64, d_v=128, elt=2, q_elt=2) -> int:
    """Algorithmic HBM bytes of one mla_decode_proj call: cache rows (elt bytes an
    element) read once, the query read once, W_UV (elt bytes) read once, the float32
    layer output written once, the block table read once (obar is not an output)."""
    row = (d_latent + d_rope) * elt
    t = np.asarray(seq_lens, np.int64)
    per_q = n_heads * (d_latent + d_rope) * q_elt + n_heads * d_v * 4
    return int(np.sum(row * t + per_q + 4 * ((t + 63) // 64))) + n_heads * d_v * d_latent * elt


def per_head_decode_bytes(seq_lens, n_heads=16, d_latent=256, d_rope=32, q_elt=2, d_v=None) -> int:
    """Algorithmic HBM bytes of one per-head-key decode call: bf16 rows of the latent
    and one position key per head read once, the query read once, the float32
    latent output written once, the block table read once.  With d_v (the fused
    mla_decode_per_head_proj): the float32 layer output in place of the latent
    output, and W_UV (bf16) read once."""
    row = (d_latent + n_heads * d_rope) * 2
    t = np.asarray(seq_lens, np.int64)
    out_w = d_latent if d_v is None else d_v
    per_q = n_heads * (d_latent + d_rope) * q_elt + n_heads * out_w * 4
    w = 0 if d_v is None else n_heads * d_v * d_latent * 2
    return int(np.sum(row * t + per_q + 4 * ((t + 63) // 64))) + w


def prefill_flops(case) -> float:
    """2 * n_h * (576 + 512) per visible (query, key) pair, causal."""
    s = case.shape
    pairs = 0
    for b in range(case.batch):
        n = int(case.cu_q[b + 1] - case.cu_q[b])
        p0 = int(case.q_start[b])
        pairs += n * p0 + n * (n + 1) // 2
    return 2.0 * s.n_heads * (s.row + s.d_latent) * pairs


def prefill_mha_flops(case) -> float:
    """Materialised form: 2 * n_h * (d_h + d_v) * d_c per visible key position for
    the up-projection, plus 2 * n_h * (d_h + d_r + d_v) per visible (query, key)
    pair for the attention."""
    s = case.shape
    pairs = keys = 0
    for b in range(case.batch):
        n = int(case.cu_q[b + 1] - case.cu_q[b])
        p0 = int(case.q_start[b])
        pairs += n * p0 + n * (n + 1) // 2
        keys += p0 + n
    return (2.0 * s.n_heads * (s.d_head + s.d_v) * s.d_latent * keys
            + 2.0 * s.n_heads * (s.d_head + s.d_rope + s.d_v) * pairs)


class DeviceEvents:
    """HIP events on the launch stream, recorded with a device-scope release.

    torch's events take a system-scope release at every record, which writes
    back L2 and stalls the queue for several microseconds around the timed
    call; a device-scope release (hipEventReleaseToDevice) orders the same
    work without that flush.  The events come from the HIP runtime the
    process has loaded (the one torch and libmla share).
    """

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, n: int):
        import ctypes

        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.hip = ctypes.CDLL(path)
        self.ct = ctypes
        self.events = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.RELEASE_TO_DEVICE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(e)
        self.used = 0

    def record(self, stream_handle: int):
        e = self.events[self.used]
        self.used += 1
        if self.hip.hipEventRecord(e, self.ct.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def load_traffic(config_name: str, src: str = KERNEL_SRC):
    """Measured HBM bytes per call, if profiled on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE)).get(config_name)
    if not rec or rec.get("kernel_sha") != kernel_hash(src):
        return None
    return rec.get("bytes_per_launch")


def metric_name(args, case, per_head: bool) -> str:
    """The metric string of a bench line: the headline metric for the 64 x 4096 decode,
    and a name of its own for every other workload and mode."""
    s = case.shape
    shape = f"n_h={s.n_heads},d_c={s.d_latent},d_r={s.d_rope}"
    if per_head:
        return f"MLA decode over per-head position keys tokens/s + % HBM roofline ({shape}, 64 x 4096)"
    if case.kind == "decode":
        what = {"c1": "tiny MLA decode (fp32, 1 x 256)", "c3": None, "c4": "absorbed MLA ragged paged decode "
                "(128 seqs, T ~ U[512, 32768])", "c5a": "absorbed MLA long-context decode (4 x 131072)"}[args.config]
        if args.front != "none":
            return f"MLA decode layer step from hidden states ({args.front} front) tokens/s + % HBM roofline " \
                   f"of mla_decode ({shape})"
        if args.score == "two":
            return f"absorbed MLA decode, two-scale score, tokens/s + % HBM roofline ({shape})"
        return METRIC if what is None else f"{what} tokens/s + % HBM roofline ({shape})"
    what = {"c2": "tiny MLA causal prefill (4 x 1024 from position 0)",
            "c5b": "MLA chunked causal prefill (2048 after 16384)"}[args.config]
    form = "absorbed" if args.prefill_form == "absorbed" else "materialised"
    score = ", two-scale score" if args.score == "two" else ""
    return f"{what}, {form} form{score}, tokens/s + % MFMA roofline ({shape})"


def cpu_baseline(case, budget_s: float = 12.0, form: str = "materialised"):
    """The float64 oracle (the materialised definition, or its absorbed twin) on the host
    cores, on a bounded sample of the same workload: whole decode sequences, or prefill
    queries in blocks of 8 taken evenly across the chunk, until `budget_s` has passed."""
    from threadpoolctl import threadpool_info

    from oracle import attention

    evaluate = attention.materialised if form == "materialised" else attention.absorbed
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    done, t0 = 0, time.perf_counter()
    if case.kind == "decode":
        for b in range(case.batch):
            attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                   case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base, seqs=[b],
                                   evaluate=evaluate)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        what = (f"{form} float64 decode of {done} of {case.batch} sequences "
                f"({int(np.min(case.seq_lens))}..{int(np.max(case.seq_lens))} cached tokens)")
    else:
        n = int(case.cu_q[-1])
        order = np.concatenate([np.arange(i, n, 64) for i in range(64)])  # evenly across the chunk first
        for i in range(0, n, 8):
            attention.prefill_batch(case.cu_q, case.q_start, case.c_rows, case.kr_rows, case.row_offsets, case.qc,
                                    case.qr, case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base,
                                    queries=np.sort(order[i:i + 8]), evaluate=evaluate)
            done += len(order[i:i + 8])
            if time.perf_counter() - t0 > budget_s:
                break
        what = f"{form} float64 causal prefill of {done} of {n} queries, spread evenly over the chunk"
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5a", "c5b"])
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--front", default="none", choices=["none", "unfolded", "folded"],
                    help="decode workloads: start the step from hidden states (d_model 5120, query latent 1536): "
                         "kv_project + q_project + absorb_q (or q_project_folded) + decode + out_proj")
    ap.add_argument("--prefill-form", default="absorbed", choices=["absorbed", "materialised"],
                    help="prefill workloads: absorbed latent attention (mla_prefill) or per-head keys and "
                         "values up-projected first (mla_prefill_mha)")
    ap.add_argument("--score", default="one", choices=["one", "two"],
                    help="one scale on the summed score, or the two-scale score (content over sqrt(d_h), "
                         "position over sqrt(d_r)) through position_scale")
    ap.add_argument("--cache-layout", default="shared", choices=["shared", "per-head"],
                    help="per-head: decode over a cache with one position key per head (16 heads, d_c 256, "
                         "d_r 32, 768-element rows; 64 sequences x 4096 tokens)")
    ap.add_argument("--out-proj", default="fused", choices=["fused", "separate"],
                    help="decode: attention then the split merge and output absorption in one launch "
                         "(mla_decode_proj), or mla_decode + mla_out_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="run one plain 256 MiB copy kernel before timing (HBM counter calibration under rocprofv3)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU sharding of this path is a design note, not a measured mode.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_decoupled_rope_amd as mla
    import synth
    from mla_decoupled_rope_amd import binding as B

    torch.cuda.set_device(0)
    maker = {"c1": synth.config1, "c2": synth.config2, "c3": synth.config3, "c4": synth.config4,
             "c5a": synth.config5_decode, "c5b": synth.config5_prefill}[args.config]
    per_head = args.cache_layout == "per-head"
    if per_head:
        case = synth.direct_decode(synth.TINY, "bf16", [4096] * 64, seed=31, shuffle=True, per_head_rope=True)
        case.note["workload"] = "per-head position keys: 64 x 4096 decode, n_h=16, d_c=256, d_r=32 per head"
    else:
        case = maker()
    s = case.shape
    dt = torch.float32 if case.dtype == "f32" else torch.bfloat16
    scale, position_scale = s.scale, None
    if args.score == "two":
        scale, position_scale = 1.0 / np.sqrt(s.d_head), 1.0 / np.sqrt(s.d_rope)
    # the small shape runs in the float32 working precision (two-term q~ and softmax
    # weights), the path its parity tests hold to the configured bounds
    work = torch.float32 if (dt == torch.float32 or s.row <= 288) and args.prefill_form == "absorbed" else dt
    dims = mla.MLADims(s.n_heads, s.d_head, s.d_v, s.d_latent, s.d_rope, dtype=dt, softmax_scale=scale,
                       position_scale=position_scale, work_dtype=work)
    q_elt = 4 if work == torch.float32 else 2

    def dev(x, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dtype).contiguous()

    seqs, pos = case.kv_seq_pos()
    chunk = 1 << 20
    if per_head:
        ph_steps = [mla.PerHeadDecodeStep(dims, case.block_table, case.num_pages, torch.from_numpy(case.seq_lens))
                    for _ in range(max(1, args.copies))]
        for r0 in range(0, len(seqs), chunk):
            r1 = min(len(seqs), r0 + chunk)
            ph_steps[0].write(dev(case.c_rows[r0:r1]), dev(case.kr_rows[r0:r1]), torch.from_numpy(seqs[r0:r1]).cuda(),
                              torch.from_numpy(pos[r0:r1]).cuda())
        for st in ph_steps[1:]:
            st.cache.copy_(ph_steps[0].cache)
        caches = [st.cache for st in ph_steps]
    else:
        cache0 = mla.LatentCache(dims, case.block_table, case.num_pages)
        for r0 in range(0, len(seqs), chunk):
            r1 = min(len(seqs), r0 + chunk)
            cache0.write(dev(case.c_rows[r0:r1]), dev(case.kr_rows[r0:r1]), torch.from_numpy(seqs[r0:r1]).cuda(),
                         torch.from_numpy(pos[r0:r1]).cuda())
        caches = [cache0]
        for _ in range(1, max(1, args.copies)):
            c = mla.LatentCache(dims, case.block_table, case.num_pages)
            c.data.copy_(cache0.data)
            caches.append(c)
    if args.calibrate:
        # a plain streaming kernel of known size: reads 256 MiB, writes 256 MiB
        cal_src = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")
        cal_dst = torch.empty_like(cal_src)
        torch.neg(cal_src, out=cal_dst)
        torch.cuda.synchronize()
        del cal_src, cal_dst
    w_uk, w_uv = dev(case.w_uk), dev(case.w_uv)
    q_nope, q_rope = dev(case.qc), dev(case.qr)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    events = DeviceEvents(4)
    front_bytes = 0
    fused = args.out_proj == "fused"
    dominant, dominant_name = None, None

    def decode_roofline():
        """(name, algorithmic bytes) of the measured decode call."""
        if fused:
            return ("mla_decode_proj (split attention + merge with output absorption)",
                    decode_proj_bytes(case.seq_lens, s.n_heads, s.d_latent, s.d_rope, s.d_v,
                                      4 if dt == torch.float32 else 2, q_elt))
        return ("mla_decode (split attention + merge)",
                decode_bytes(case.seq_lens, s.n_heads, s.d_latent, s.d_rope, 4 if dt == torch.float32 else 2, q_elt))
    if per_head:
        last = case.row_offsets + np.maximum(case.seq_lens - 1, 0)
        new_lat, new_kr = dev(case.c_rows[last]), dev(case.kr_rows[last])
        kv_seq = torch.arange(case.batch, dtype=torch.int32, device="cuda")

        def call(i):
            if fused:
                ph_steps[i % len(ph_steps)].attend_proj(w_uv)
            else:
                ph_steps[i % len(ph_steps)].attend()

        def step(i):
            st = ph_steps[i % len(ph_steps)]
            st.write(new_lat, new_kr, kv_seq, st.q_pos)
            B.rope_absorb_q(dims, None, None, q_nope, w_uk, q_rope, st.q_pos, st.q_lat)
            call(i)
            if not fused:
                B.out_proj(dims, st.out_latent, w_uv, st.out)
        tokens_per_step = case.batch
        if fused:
            kernel_name = "mla_decode_per_head_proj (split attention + merge with output absorption)"
            algo = per_head_decode_bytes(case.seq_lens, s.n_heads, s.d_latent, s.d_rope, q_elt, d_v=s.d_v)
        else:
            kernel_name = "mla_decode_per_head (split attention + merge)"
            algo = per_head_decode_bytes(case.seq_lens, s.n_heads, s.d_latent, s.d_rope, q_elt)
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
    elif case.kind == "decode" and args.front != "none":
        d_model, d_qlat = s.hidden, QUERY_LATENT
        folded = args.front == "folded"
        fc = synth.front_layer(s, np.ones(case.batch, np.int32), d_model, d_qlat, seed=case.seed + 100, shuffle=False)
        w_dkv, w_kr, w_dq, w_qr = dev(fc.w_dkv), dev(fc.w_kr), dev(fc.w_dq), dev(fc.w_qr)
        w_uk, w_uv = dev(fc.w_uk), dev(fc.w_uv)
        w_up = dev(fc.w_uq)
        if folded:  # weight preparation, once, outside the timed region
            w_fold = torch.empty((s.n_heads, s.d_latent, d_qlat), dtype=dt, device="cuda")
            B.fold_q_weights(dims, w_up, w_uk, w_fold)
            w_up = w_fold
        h_new = dev(fc.h)
        steps = [mla.LayerDecodeStep(dims, c, torch.from_numpy(case.seq_lens), d_model, d_qlat, folded)
                 for c in caches]
        front_bytes = 2 * (w_dkv.numel() + w_kr.numel() + w_dq.numel() + w_qr.numel() + w_up.numel()
                           + (0 if folded else w_uk.numel()))

        def front(i):
            st = steps[i % len(steps)]
            st.kv(h_new, w_dkv, w_kr)
            st.query(h_new, w_dq, w_up, w_qr, w_uk)

        if fused:
            def call(i):
                steps[i % len(steps)].inner.attend_proj(w_uv)

            def step(i):
                front(i)
                call(i)
        else:
            def call(i):
                inner = steps[i % len(steps)].inner
                B.decode(dims, inner.cache.data, inner.cache.block_table, inner.q_lat, inner.seq_lens,
                         inner.seq_lens_host, inner.out_latent, inner.lse, inner.workspace)

            def step(i):
                front(i)
                call(i)
                inner = steps[i % len(steps)].inner
                B.out_proj(dims, inner.out_latent, w_uv, inner.out)
        tokens_per_step = case.batch
        kernel_name, algo = decode_roofline()
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
    elif case.kind == "decode":
        steps = [mla.DecodeStep(dims, c, torch.from_numpy(case.seq_lens)) for c in caches]
        if fused and dt != torch.float32:
            def dominant(i):
                steps[i % len(steps)].attend_split_kv()
            dominant_name = "attn_bf16_kernel (the split attention alone: mla_decode_split_kv)"
        last = case.row_offsets + np.maximum(case.seq_lens - 1, 0)
        new_lat, new_kr = dev(case.c_rows[last]), dev(case.kr_rows[last])

        def call(i):
            st = steps[i % len(steps)]
            if fused:
                st.attend_proj(w_uv)
            else:
                B.decode(dims, st.cache.data, st.cache.block_table, st.q_lat, st.seq_lens, st.seq_lens_host,
                         st.out_latent, st.lse, st.workspace)

        def step(i):
            st = steps[i % len(steps)]
            B.rope_absorb_q(dims, st.cache.data, st.cache.block_table, q_nope, w_uk, q_rope, st.q_pos, st.q_lat,
                            new_lat, new_kr, st.kv_seq, st.q_pos)
            call(i)
            if not fused:
                B.out_proj(dims, st.out_latent, w_uv, st.out)
        tokens_per_step = case.batch
        kernel_name, algo = decode_roofline()
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
    elif args.prefill_form == "materialised":
        steps = [mla.PrefillStep(dims, c, torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start))
                 for c in caches]
        mha_ws = B.prefill_mha_workspace(dims, steps[0].cu_q_host, steps[0].q_start_host)

        def call(i):
            st = steps[i % len(steps)]
            B.prefill_mha(dims, st.cache.data, st.cache.block_table, q_nope, st.q_lat, w_uk, w_uv, st.cu_q,
                          st.q_start, st.cu_q_host, st.q_start_host, st.out, st.lse, mha_ws)

        def step(i):
            st = steps[i % len(steps)]
            B.rope_apply(dims, None, None, q_rope=q_rope, q_pos=st.q_pos, q_lat=st.q_lat)
            call(i)
        tokens_per_step = int(case.cu_q[-1])
        kernel_name = "mla_prefill_mha (key/value up-projection + causal attention)"
        algo = prefill_mha_flops(case)
        bound, unit, peak = "mfma", "TFLOP/s", BF16_PEAK_TFLOPS
    else:
        steps = [mla.PrefillStep(dims, c, torch.from_numpy(case.cu_q), torch.from_numpy(case.q_start))
                 for c in caches]

        def call(i):
            st = steps[i % len(steps)]
            B.prefill(dims, st.cache.data, st.cache.block_table, st.q_lat, st.cu_q, st.q_start, st.cu_q_host,
                      st.q_start_host, st.out_latent, st.lse)

        def step(i):
            st = steps[i % len(steps)]
            B.rope_absorb_q(dims, None, None, q_nope, w_uk, q_rope, st.q_pos, st.q_lat)
            call(i)
            B.out_proj(dims, st.out_latent, w_uv, st.out)
        tokens_per_step = int(case.cu_q[-1])
        kernel_name = "mla_prefill (causal attention)"
        algo = prefill_flops(case)
        bound, unit, peak = "mfma", "TFLOP/s", BF16_PEAK_TFLOPS

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_per_step = el / args.steps * 1e3

    # The measured call alone, after an untimed lead-in, `steps` times back to
    # back on the launch stream between two HIP events: an event recorded between two kernels idles the
    # queue for several microseconds (a kernel trace shows the gap exactly where
    # the event sits), so bracketing each call would time the events too.
    def timed_loop(fn):
        # Untimed first: at least W launches and at least KERNEL_WARMUP_S of them
        # (synchronising every 16 so the host clock follows the GPU), so the
        # kernel is timed at the clock a sustained decode runs at: after an idle
        # host phase the GPU takes tens of milliseconds of load to reach it, and
        # a loop of 20 launches would fall inside that ramp.
        t_w, i = time.perf_counter(), 0
        while i < args.warmup or time.perf_counter() - t_w < KERNEL_WARMUP_S:
            fn(i)
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0 = events.record(sh)
        for i in range(args.steps):
            fn(i)
        e1 = events.record(sh)
        torch.cuda.synchronize()
        return events.elapsed_ms(e0, e1) / args.steps

    kern_ms = timed_loop(call)
    front_ms = timed_loop(front) if args.front != "none" and not per_head and case.kind == "decode" else None
    # The dominant kernel alone, where the measured call has more than one launch:
    # the split attention of the decode call, its partials left for the merge.
    dom_ms = timed_loop(dominant) if dominant is not None else None
    events.close()
    achieved = algo / (kern_ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    call_roofline = None
    if dom_ms is not None:
        call_roofline = {"kernel": kernel_name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                         "frac": achieved / peak, "traffic": None, "algorithmic_per_launch": algo,
                         "avg_launch_ms": kern_ms}
        kernel_name = dominant_name
        algo = decode_bytes(case.seq_lens, s.n_heads, s.d_latent, s.d_rope, 2, q_elt)
        kern_ms = dom_ms
        achieved = algo / (kern_ms * 1e-3) / 1e9
    if per_head:
        ph_src = os.path.join(ROOT, "mla_decoupled_rope_amd", "csrc", "perhead.hip")
        traffic = (load_traffic("per_head_proj", [ph_src, GEMM_SRC]) if fused
                   else load_traffic("per_head", ph_src))
    elif case.kind == "decode" and dom_ms is not None:
        traffic = load_traffic(args.config + "_attn")
        call_roofline["traffic"] = load_traffic(args.config + "_proj", [KERNEL_SRC, GEMM_SRC])
    elif case.kind == "decode" and fused:
        traffic = load_traffic(args.config + "_proj", [KERNEL_SRC, GEMM_SRC])
    elif case.kind == "decode" or args.prefill_form == "absorbed":
        traffic = load_traffic(args.config)
    else:
        traffic = load_traffic(args.config + "_mha", MHA_SRC)
    out = {
        "metric": metric_name(args, case, per_head),
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded N(0,1) latents, keys and queries; weights N(0,1)/sqrt(d_c))",
        "config": {"workload": case.note.get("workload", args.config), "config": args.config,
                   "batch": case.batch, "seq_len": int(np.max(case.seq_lens)), "total_kv_tokens": case.total_tokens,
                   "n_heads": s.n_heads, "d_latent": s.d_latent, "d_rope": s.d_rope, "page_size": s.page_size,
                   "cache_copies": len(caches), "score": "two-scale" if args.score == "two" else "one scale",
                   "cache_layout": args.cache_layout,
                   "step": (("cache_write_per_head + rope_absorb_q + decode_per_head_proj" if fused else
                             "cache_write_per_head + rope_absorb_q + decode_per_head + out_proj") if per_head
                            else "rope_apply + prefill_mha" if case.kind != "decode" and args.prefill_form == "materialised"
                            else (f"kv_project + q_project ({args.front}) + "
                                  + ("decode_proj" if fused else "decode + out_proj")) if args.front != "none"
                            else "rope_absorb_q + decode_proj" if case.kind == "decode" and fused
                            else "rope_absorb_q + decode/prefill + out_proj")},
        "roofline": {"kernel": kernel_name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic, "algorithmic_per_launch": algo,
                     "avg_launch_ms": kern_ms},
    }
    if call_roofline is not None:
        out["roofline_call"] = call_roofline
    if front_ms is not None:
        out["front"] = {"form": args.front, "d_model": s.hidden, "d_qlat": QUERY_LATENT, "avg_ms": front_ms,
                        "weight_bytes": front_bytes, "weight_GBps": front_bytes / (front_ms * 1e-3) / 1e9,
                        "calls": "kv_project + q_project" + (" + absorb_q" if args.front == "unfolded" else "")}
    if not args.no_cpu_baseline and args.front == "none" and not per_head and args.score == "one":
        out["cpu_baseline"] = cpu_baseline(case)
        out["cpu_baseline_absorbed"] = cpu_baseline(case, form="absorbed")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
