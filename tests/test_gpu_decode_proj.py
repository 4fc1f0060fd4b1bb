"""mla_decode_proj -- attention, then the split merge and the output absorption in one
launch -- against the oracle, and against mla_decode + mla_out_proj on the same inputs.

Where a sequence's decode takes several work items the fused merge and projection run
the arithmetic of the two separate calls in the same order, so its output and lse must
equal theirs bit for bit; a sequence of one item goes through its stored partial (float16
scaled per 128 columns at d_c = 512), so its output is held to the oracle's bound only.
"""

import numpy as np
import pytest
import torch

import cases
import gpu_util as G
import mla_decoupled_rope_amd as mla
import synth
from oracle import attention

pytestmark = pytest.mark.gpu


def oracle_decode(case, seqs=None, evaluate=attention.materialised):
    return attention.decode_batch(case.seq_lens, case.c_rows, case.kr_rows, case.row_offsets, case.qc, case.qr,
                                  case.w_uk, case.w_uv, case.shape.scale, case.shape.rope_base, seqs=seqs,
                                  evaluate=evaluate)


def both_paths(case, precise=None):
    """(fused, separate): dicts of o and lse (float64) from one cache and one q_lat."""
    dims = G.dims_of(case, precise)
    cache = G.build_cache(case)
    step = mla.DecodeStep(dims, cache, torch.from_numpy(case.seq_lens))
    dt = G.tdtype(case)
    qc, qr, w_uk, w_uv = G.dev(case.qc, dt), G.dev(case.qr, dt), G.dev(case.w_uk, dt), G.dev(case.w_uv, dt)
    step.run(qc, qr, w_uk, w_uv)
    torch.cuda.synchronize()
    sep = {"o": G.to64(step.out), "lse": G.to64(step.lse)}
    step.out.fill_(float("nan"))
    step.lse.fill_(float("nan"))
    step.attend_proj(w_uv)  # q_lat as the separate path left it
    torch.cuda.synchronize()
    fused = {"o": G.to64(step.out), "lse": G.to64(step.lse)}
    return fused, sep, dims


def items_per_sequence(dims, seq_lens):
    split_pages, _ = mla.decode_plan(dims, torch.from_numpy(np.asarray(seq_lens, np.int32)))
    pages = (np.maximum(np.asarray(seq_lens, np.int64), 0) + 63) // 64
    return (pages + split_pages - 1) // split_pages


def check_against(fused, sep, want, dims, seq_lens, dtype, name, what, rows=None, bitwise_all=False):
    """Bitwise against the separate calls on multi-item (and empty) sequences, every
    sequence when bitwise_all; o and lse against the oracle on `rows`."""
    ns = items_per_sequence(dims, seq_lens)
    same = np.ones(len(ns), bool) if bitwise_all else ns != 1
    for k in ("o", "lse"):
        assert np.array_equal(fused[k][same], sep[k][same]), f"{what}: {k} differs from the two calls"
    print(f"{what}: {int(same.sum())} of {len(ns)} sequences bitwise equal to decode + out_proj", flush=True)
    g = fused if rows is None else {k: fused[k][rows] for k in fused}
    G.assert_close(g["o"], want["o"], dtype, f"{what} o", name=name, output="o")
    G.assert_lse_close(g["lse"], want["lse"], dtype, f"{what} lse", name=name)


def test_decode_proj_tiny_f32():
    """float32 caches: the two calls' kernels with obar in the workspace, bitwise."""
    case = synth.config1()
    fused, sep, dims = both_paths(case)
    check_against(fused, sep, oracle_decode(case), dims, case.seq_lens, "f32", None, "tiny fp32 decode_proj",
                  bitwise_all=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_proj_tiny_ragged(dtype):
    case = cases.tiny_decode_ragged(dtype)
    fused, sep, dims = both_paths(case)
    # the small shape keeps float32 partials: a one-item sequence's obar passes the merge
    # unchanged (weight 1), so every sequence equals the two calls bit for bit
    check_against(fused, sep, oracle_decode(case), dims, case.seq_lens, dtype,
                  None if dtype == "f32" else "tiny_decode_ragged", f"tiny ragged decode_proj {dtype}",
                  bitwise_all=True)


@pytest.mark.parametrize("split_pages", [None, 1, 3, 1000])
def test_decode_proj_dsv2_ragged(split_pages, monkeypatch):
    """Planned splits, forced 1- and 3-page splits, and 1000-page splits (every sequence
    one item: every row passes through its float16 partial)."""
    if split_pages is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", str(split_pages))
    case = cases.dsv2_decode_ragged()
    fused, sep, dims = both_paths(case)
    check_against(fused, sep, oracle_decode(case), dims, case.seq_lens, "bf16", "dsv2_decode_ragged",
                  f"dsv2 decode_proj split={split_pages}")


def fused_in_two_calls(case):
    """(one call, two calls): mla_decode_proj, then mla_decode_split_kv + mla_merge_out_proj on the
    same q_lat, each into freshly poisoned outputs."""
    dims = G.dims_of(case)
    step = mla.DecodeStep(dims, G.build_cache(case), torch.from_numpy(case.seq_lens))
    bf = torch.bfloat16
    w_uv = G.dev(case.w_uv, bf)
    step.run(G.dev(case.qc, bf), G.dev(case.qr, bf), G.dev(case.w_uk, bf), w_uv)
    res = []
    for two in (False, True):
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        if step.proj_workspace is not None:
            step.proj_workspace.fill_(0xFF)  # partials as NaN: a slot left unwritten would show
        if two:
            step.attend_split_kv()
            step.merge_out_proj(w_uv)
        else:
            step.attend_proj(w_uv)
        torch.cuda.synchronize()
        res.append((step.out.clone(), step.lse.clone()))
    return res


@pytest.mark.parametrize("which", ["tiny", "dsv2", "dsv2_split1", "dsv2_one_item", "empty"])
def test_split_kv_then_merge_equals_decode_proj(which, monkeypatch):
    """mla_decode_proj's two launches called one by one give its output and lse bit for bit."""
    forced = {"dsv2_split1": "1", "dsv2_one_item": "1000"}.get(which)
    if forced is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", forced)
    case = {"tiny": lambda: cases.tiny_decode_ragged("bf16"), "empty": cases.decode_empty}.get(
        which, cases.dsv2_decode_ragged)()
    (o1, l1), (o2, l2) = fused_in_two_calls(case)
    print(f"{which}: {case.batch} sequences, lengths {case.seq_lens.min()}..{case.seq_lens.max()}", flush=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert not torch.isnan(o1).any()


def test_decode_proj_empty_sequences():
    case = cases.decode_empty()
    fused, sep, dims = both_paths(case)
    assert np.all(fused["o"][[0, 2]] == 0) and np.all(np.isneginf(fused["lse"][[0, 2]]))
    check_against(fused, sep, oracle_decode(case), dims, case.seq_lens, "bf16", "decode_empty",
                  "decode_proj with empty sequences")


def test_decode_proj_all_empty_batch():
    """No tokens anywhere: no work items and no workspace; o = 0, lse = -inf."""
    case = synth.direct_decode(synth.DSV2, "bf16", [0, 0, 0], seed=311)
    dims = G.dims_of(case)
    bf = torch.bfloat16
    lens = torch.from_numpy(case.seq_lens)
    assert mla.decode_proj_workspace_size(dims, lens) == 0
    q_lat = torch.zeros((3, dims.n_heads, dims.row), dtype=bf, device="cuda")
    out = torch.full((3, dims.n_heads, dims.d_v), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.zeros((3, dims.n_heads), dtype=torch.float32, device="cuda")
    cache = torch.zeros((1, 64, dims.row), dtype=bf, device="cuda")
    table = torch.from_numpy(case.block_table).cuda()
    mla.decode_proj(dims, cache, table, q_lat, lens.cuda(), lens, G.dev(case.w_uv, bf), out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_decode_proj_many_sequences():
    """More than one 64-sequence scan block and a ragged last group of 16; sequences of
    a few keys among them (held to the rounding model's figure for these inputs)."""
    case = cases.decode_proj_many()
    fused, sep, dims = both_paths(case)
    seqs = cases.DECODE_PROJ_MANY_ROWS
    check_against(fused, sep, oracle_decode(case, seqs=seqs, evaluate=attention.absorbed), dims, case.seq_lens,
                  "bf16", "decode_proj_many", "decode_proj 150 sequences", rows=seqs)


def test_decode_proj_graph_replays():
    """The fused step captured as a HIP graph and replayed gives the eager step's bits."""
    case = synth.direct_decode(synth.DSV2, "bf16", [700, 64, 1, 2048, 130], seed=317, shuffle=True)
    dims = G.dims_of(case)
    cache = G.build_cache(case)
    step = mla.DecodeStep(dims, cache, torch.from_numpy(case.seq_lens))
    bf = torch.bfloat16
    qc, qr, w_uk, w_uv = G.dev(case.qc, bf), G.dev(case.qr, bf), G.dev(case.w_uk, bf), G.dev(case.w_uv, bf)
    last = case.row_offsets + np.maximum(case.seq_lens - 1, 0)
    new_lat, new_kr = G.dev(case.c_rows[last], bf), G.dev(case.kr_rows[last], bf)

    def run():
        step.run_fused(qc, qr, w_uk, w_uv, new_lat, new_kr)

    run()
    torch.cuda.synchronize()
    want = [step.out.clone(), step.lse.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        step.out.fill_(float("nan"))
        step.lse.fill_(1.0)
        step.q_lat.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, want[0]) and torch.equal(step.lse, want[1]), f"replay {r} differs"


# --------------------------------------------------------------- full sizes ----

def test_config3_full_decode_proj():
    """64 x 4096: every sequence splits, so the fused output equals the two calls' bit for
    bit, and all sequences meet the absorbed float64 oracle."""
    case = synth.config3()
    fused, sep, dims = both_paths(case)
    assert np.all(items_per_sequence(dims, case.seq_lens) > 1)
    check_against(fused, sep, oracle_decode(case, evaluate=attention.absorbed), dims, case.seq_lens, "bf16", "c3",
                  "C3 decode_proj")


def test_config3_split_kv_then_merge():
    """The launch bench.py times as the dominant kernel (the split attention alone), followed by
    the merge with the output absorption, equals mla_decode_proj bit for bit at 64 x 4096."""
    (o1, l1), (o2, l2) = fused_in_two_calls(synth.config3())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_config4_full_decode_proj():
    case = synth.config4()
    fused, sep, dims = both_paths(case)
    import bound_recipes
    seqs = bound_recipes.c4_sequences(case)
    check_against(fused, sep, oracle_decode(case, seqs=seqs, evaluate=attention.absorbed), dims, case.seq_lens,
                  "bf16", "c4", f"C4 decode_proj {len(seqs)} sequences", rows=seqs)


def test_config5_full_decode_proj():
    case = synth.config5_decode()
    fused, sep, dims = both_paths(case)
    check_against(fused, sep, oracle_decode(case, evaluate=attention.absorbed), dims, case.seq_lens, "bf16", "c5a",
                  "C5 decode_proj")


# ------------------------------------------------------ per-head position keys ----

def per_head_both(case, precise):
    """(fused, separate) over a per-head-key cache: mla_decode_per_head_proj against
    mla_decode_per_head + mla_out_proj on the same q_lat."""
    dims = G.dims_of(case, precise)
    bf = torch.bfloat16
    step = mla.PerHeadDecodeStep(dims, case.block_table, case.num_pages, torch.from_numpy(case.seq_lens),
                                 fill=float("nan"))
    seqs, pos = case.kv_seq_pos()
    step.write(G.dev(case.c_rows, bf), G.dev(case.kr_rows, bf), torch.from_numpy(seqs).cuda(),
               torch.from_numpy(pos).cuda())
    w_uv = G.dev(case.w_uv, bf)
    step.run(G.dev(case.qc, bf), G.dev(case.qr, bf), G.dev(case.w_uk, bf), w_uv)
    torch.cuda.synchronize()
    sep = {"o": G.to64(step.out), "lse": G.to64(step.lse)}
    step.out.fill_(float("nan"))
    step.lse.fill_(float("nan"))
    step.attend_proj(w_uv)
    torch.cuda.synchronize()
    return {"o": G.to64(step.out), "lse": G.to64(step.lse)}, sep, dims


@pytest.mark.parametrize("precise", [True, False], ids=["f32-q", "bf16-q"])
@pytest.mark.parametrize("split_pages", [None, 1, 3])
def test_decode_per_head_proj(precise, split_pages, monkeypatch):
    """float32 partials on this layout: every sequence equals the two calls bit for bit."""
    if split_pages is not None:
        monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", str(split_pages))
    case = cases.per_head_decode()
    fused, sep, dims = per_head_both(case, precise)
    check_against(fused, sep, oracle_decode(case), dims, case.seq_lens, "bf16",
                  "per_head_f32w" if precise else "per_head_bf16", f"per-head decode_proj split={split_pages}",
                  bitwise_all=True)
