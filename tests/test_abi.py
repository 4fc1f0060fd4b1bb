"""CPU-side checks of the C ABI: the library loads, exports what include/mla.h
declares, rejects bad arguments before launching anything, and plans decode
splits deterministically.  No kernel runs here."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import mla_decoupled_rope_amd as mla
from mla_decoupled_rope_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("mla_rope_apply", "mla_absorb_q", "mla_decode", "mla_prefill", "mla_out_proj"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in mla.h but not exported"
    assert set(declared_functions()) == set(B.EXPORTS)


def _dims(**kw):
    base = dict(n_heads=128, d_head=128, d_v=128, d_latent=512, d_rope=64, page_size=64, dtype=B.MLA_BF16,
                work_dtype=B.MLA_BF16, softmax_scale=0.0722, position_scale=0.0722, rope_base=10000.0)
    base.update(kw)
    return B.Dims(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def status_of_decode(d, batch=1, lens=(10,), ws=None, ws_bytes=0, cache_kw=None):
    ck = dict(data=FAKE.value, num_pages=4, block_table=FAKE.value, num_seqs=4, max_pages_per_seq=4)
    ck.update(cache_kw or {})
    cache = B.PagedCache(**ck)
    lens_host = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    return B.LIB.mla_decode(ctypes.byref(d), ctypes.byref(cache), FAKE, FAKE, lens_host, batch, FAKE, None, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("kw, status", [
    (dict(d_rope=63), 1), (dict(n_heads=0), 1), (dict(page_size=32), 2), (dict(dtype=7), 1),
    (dict(softmax_scale=float("nan")), 1), (dict(position_scale=0.0), 1), (dict(position_scale=float("inf")), 1),
    (dict(rope_base=-1.0), 1), (dict(n_heads=64), 2),
    (dict(d_rope=256), 2), (dict(work_dtype=B.MLA_F32), 2), (dict(dtype=B.MLA_F32), 1),
    (dict(work_dtype=5), 1),
])
def test_decode_rejects_bad_dims(kw, status):
    assert status_of_decode(_dims(**kw)) == status
    assert B.LIB.mla_last_error().decode()


def test_decode_rejects_bad_arguments():
    d = _dims()
    assert B.LIB.mla_decode(None, None, None, None, None, 1, None, None, None, 0, None) == 1
    assert status_of_decode(d, batch=-1) == 1
    assert status_of_decode(d, batch=5, lens=(1, 1, 1, 1, 1)) == 1          # more rows than the block table
    assert status_of_decode(d, lens=(300,)) == 1                          # beyond 4 pages of 64
    assert status_of_decode(d, lens=(-3,)) == 1
    assert status_of_decode(d, lens=(5,), cache_kw=dict(num_pages=0)) == 1  # tokens but no pages
    assert status_of_decode(d, batch=0) == 0                              # empty batch: nothing to do


def test_decode_workspace_is_checked(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", "1")
    d = _dims()
    lens = (200,)
    need = B.LIB.mla_decode_workspace_size(ctypes.byref(d), 1, (ctypes.c_int32 * 1)(*lens))
    assert need > 0
    assert status_of_decode(d, lens=lens) == 3
    assert status_of_decode(d, lens=lens, ws=FAKE, ws_bytes=need - 1) == 3
    assert "workspace" in B.LIB.mla_last_error().decode()


def status_of_decode_proj(d, batch=1, lens=(10,), w_uv=FAKE, out=FAKE, ws=None, ws_bytes=0):
    cache = B.PagedCache(data=FAKE.value, num_pages=4, block_table=FAKE.value, num_seqs=4, max_pages_per_seq=4)
    lens_host = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    return B.LIB.mla_decode_proj(ctypes.byref(d), ctypes.byref(cache), FAKE, FAKE, lens_host, batch, w_uv, out,
                                 None, ws, ws_bytes, None)


def test_decode_proj_validates():
    """The fused decode + output absorption runs the checks of both calls before any launch."""
    d = _dims()
    assert status_of_decode_proj(d, w_uv=None) == 1
    assert status_of_decode_proj(d, out=None) == 1
    assert status_of_decode_proj(_dims(d_v=64)) == 2           # the fused kernel covers d_v = 128
    assert status_of_decode_proj(_dims(n_heads=64)) == 2       # shapes decode does not take
    assert status_of_decode_proj(d, batch=5, lens=(1, 1, 1, 1, 1)) == 1
    assert status_of_decode_proj(d, lens=(300,)) == 1
    assert status_of_decode_proj(d, batch=0) == 0
    lens = (200,)
    lens_host = (ctypes.c_int32 * 1)(*lens)
    # a partial slot for every item, so even an unsplit sequence needs workspace
    need = B.LIB.mla_decode_proj_workspace_size(ctypes.byref(d), 1, lens_host)
    assert need > 0 and B.LIB.mla_decode_workspace_size(ctypes.byref(d), 1, lens_host) == 0
    assert status_of_decode_proj(d, lens=lens) == 3
    assert status_of_decode_proj(d, lens=lens, ws=FAKE, ws_bytes=need - 1) == 3
    assert "workspace" in B.LIB.mla_last_error().decode()
    # no tokens anywhere: no items, no workspace
    assert B.LIB.mla_decode_proj_workspace_size(ctypes.byref(d), 2, (ctypes.c_int32 * 2)(0, 0)) == 0
    # float32 caches: obar [batch, H, d_latent] float32 goes through the workspace
    f = _dims(n_heads=16, d_latent=256, d_rope=32, dtype=B.MLA_F32, work_dtype=B.MLA_F32)
    assert B.LIB.mla_decode_proj_workspace_size(ctypes.byref(f), 3, (ctypes.c_int32 * 3)(5, 0, 9)) == 3 * 16 * 256 * 4


def test_split_kv_and_merge_validate():
    """mla_decode_proj's two launches as two calls: each checks its own arguments (and the
    workspace of the fused call) before any launch; float32 caches are refused."""
    d = _dims()
    cache = B.PagedCache(data=FAKE.value, num_pages=4, block_table=FAKE.value, num_seqs=4, max_pages_per_seq=4)

    def split(dd=d, batch=1, lens=(10,), q=FAKE, ws=None, ws_bytes=0):
        lh = (ctypes.c_int32 * max(1, len(lens)))(*lens)
        return B.LIB.mla_decode_split_kv(ctypes.byref(dd), ctypes.byref(cache), q, FAKE, lh, batch, ws, ws_bytes,
                                         None)

    def merge(dd=d, batch=1, lens=(10,), w_uv=FAKE, out=FAKE, ws=None, ws_bytes=0):
        lh = (ctypes.c_int32 * max(1, len(lens)))(*lens)
        return B.LIB.mla_merge_out_proj(ctypes.byref(dd), FAKE, lh, batch, w_uv, out, None, ws, ws_bytes, None)

    assert split(q=None) == 1
    assert split(batch=5, lens=(1, 1, 1, 1, 1)) == 1          # more rows than the block table
    assert split(lens=(300,)) == 1                            # beyond 4 pages of 64
    assert split(_dims(d_v=64)) == 2
    assert split(batch=0) == 0
    assert merge(w_uv=None) == 1 and merge(out=None) == 1
    assert merge(lens=(-1,)) == 1
    assert merge(_dims(n_heads=64)) == 2
    assert merge(batch=0) == 0
    f = _dims(n_heads=16, d_latent=256, d_rope=32, dtype=B.MLA_F32, work_dtype=B.MLA_F32)
    assert split(f) == 2 and merge(f) == 2
    assert "bf16" in B.LIB.mla_last_error().decode()
    lens = (200,)
    need = B.LIB.mla_decode_proj_workspace_size(ctypes.byref(d), 1, (ctypes.c_int32 * 1)(*lens))
    assert need > 0
    for call in (split, merge):
        assert call(lens=lens) == 3
        assert call(lens=lens, ws=FAKE, ws_bytes=need - 1) == 3
        assert "workspace" in B.LIB.mla_last_error().decode()


def test_every_export_has_a_ctypes_signature():
    """Without argtypes ctypes passes a Python int as a C int, truncating 64-bit host
    pointers: every exported function must declare its arguments."""
    for name in B.EXPORTS:
        assert getattr(B.LIB, name).argtypes is not None, f"{name} has no ctypes argtypes"


def test_size_queries_take_host_tensors():
    """The binding's size queries with real (64-bit address) host tensors."""
    dims = mla.MLADims(128, 128, 128, 512, 64, dtype=torch.bfloat16, softmax_scale=0.0722,
                       work_dtype=torch.bfloat16)
    lens = torch.tensor([4096] * 64, dtype=torch.int32)
    plain, fused = B.decode_workspace_size(dims, lens), B.decode_proj_workspace_size(dims, lens)
    assert plain > 0 and fused == plain  # every sequence splits here: the same slots
    short = torch.tensor([10, 20], dtype=torch.int32)  # one item each: no merge
    assert B.decode_workspace_size(dims, short) == 0 < B.decode_proj_workspace_size(dims, short)


def test_other_calls_validate():
    d = _dims()
    assert B.LIB.mla_absorb_q(ctypes.byref(d), None, FAKE, 3, FAKE, None) == 1
    assert B.LIB.mla_absorb_q(ctypes.byref(d), FAKE, FAKE, -1, FAKE, None) == 1
    assert B.LIB.mla_absorb_q(ctypes.byref(_dims(d_head=64)), FAKE, FAKE, 3, FAKE, None) == 2
    assert B.LIB.mla_absorb_q(ctypes.byref(d), None, None, 0, None, None) == 0
    assert B.LIB.mla_out_proj(ctypes.byref(d), FAKE, None, 2, FAKE, None) == 1
    assert B.LIB.mla_out_proj(ctypes.byref(_dims(d_v=100)), FAKE, FAKE, 2, FAKE, None) == 2
    assert B.LIB.mla_rope_apply(ctypes.byref(d), None, None, None, 2, None, None, None, None, None, 0, None) == 1
    assert B.LIB.mla_rope_apply(ctypes.byref(d), None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 1
    # the fused prologue runs the checks of both calls before any launch
    rab = B.LIB.mla_rope_absorb_q
    assert rab(ctypes.byref(d), None, None, FAKE, FAKE, FAKE, 2, FAKE, None, None, None, None, 0, None) == 1  # q_nope
    assert rab(ctypes.byref(d), None, FAKE, FAKE, None, FAKE, 2, FAKE, None, None, None, None, 0, None) == 1  # q_rope
    assert rab(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 1  # cache
    assert rab(ctypes.byref(_dims(d_head=64)), None, FAKE, FAKE, FAKE, FAKE, 2, FAKE, None, None, None, None, 0,
               None) == 2
    assert rab(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, -1, FAKE, None, None, None, None, 0, None) == 1
    assert rab(ctypes.byref(d), None, None, None, None, None, 0, None, None, None, None, None, 0, None) == 0
    cache = B.PagedCache(FAKE.value, 4, FAKE.value, 2, 4)
    cu = (ctypes.c_int32 * 3)(1, 2, 3)
    st = (ctypes.c_int32 * 2)(0, 0)
    assert B.LIB.mla_prefill(ctypes.byref(d), ctypes.byref(cache), FAKE, FAKE, FAKE, cu, st, 2, FAKE, None,
                             None) == 1  # cu_q[0] != 0
    cu = (ctypes.c_int32 * 3)(0, 5, 2)
    assert B.LIB.mla_prefill(ctypes.byref(d), ctypes.byref(cache), FAKE, FAKE, FAKE, cu, st, 2, FAKE, None,
                             None) == 1  # decreasing
    cu = (ctypes.c_int32 * 3)(0, 5, 400)
    assert B.LIB.mla_prefill(ctypes.byref(d), ctypes.byref(cache), FAKE, FAKE, FAKE, cu, st, 2, FAKE, None,
                             None) == 1  # beyond the block table
    assert B.LIB.mla_status_string(3).decode().startswith("workspace")


def test_materialised_prefill_validates():
    d = _dims()
    cache = B.PagedCache(FAKE.value, 4, FAKE.value, 2, 4)
    cu = (ctypes.c_int32 * 3)(0, 5, 9)
    st = (ctypes.c_int32 * 2)(0, 10)

    def call(dims=d, cu=cu, st=st, ws=FAKE, ws_bytes=1 << 40):
        return B.LIB.mla_prefill_mha(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     cu, st, 2, FAKE, None, ws, ws_bytes, None)

    need = B.LIB.mla_prefill_mha_workspace_size(ctypes.byref(d), 2, cu, st)
    assert need == 2 * 128 * (128 + 128) * 128 * 2  # keys 0..4 and 0..13, each range padded to 128, float16
    assert call(ws_bytes=need - 1) == 3
    assert call(ws=None) == 3
    assert call(dims=_dims(d_head=64)) == 2
    assert call(dims=_dims(dtype=0, work_dtype=0)) == 2
    assert call(cu=(ctypes.c_int32 * 3)(1, 5, 9)) == 1  # cu_q[0] != 0
    assert call(cu=(ctypes.c_int32 * 3)(0, 5, 2)) == 1  # decreasing
    assert call(st=(ctypes.c_int32 * 2)(0, 300)) == 1   # beyond the block table (4 pages of 64)
    assert B.LIB.mla_prefill_mha_workspace_size(ctypes.byref(_dims(d_head=64)), 2, cu, st) == 0
    # padded key positions are limited to 2^24 - 128 (32-bit offsets into the transposed values)
    one = (ctypes.c_int32 * 2)(0, 1)
    lim = (1 << 24) - 128
    at_limit = B.LIB.mla_prefill_mha_workspace_size(ctypes.byref(d), 1, one, (ctypes.c_int32 * 1)(lim - 1))
    assert at_limit == 2 * 128 * lim * 128 * 2
    assert B.LIB.mla_prefill_mha_workspace_size(ctypes.byref(d), 1, one, (ctypes.c_int32 * 1)(lim)) == 0


def _plan(lens, dims=None):
    dims = dims or mla.MLADims(128, 128, 128, 512, 64)
    return mla.decode_plan(dims, torch.tensor(lens, dtype=torch.int32))


def test_plan_is_deterministic_and_covers_every_page():
    rng = np.random.default_rng(0)
    for _ in range(20):
        lens = rng.integers(0, 40000, size=int(rng.integers(1, 200))).tolist()
        sp, n = _plan(lens)
        assert (sp, n) == _plan(lens)
        pages = [(t + 63) // 64 for t in lens]
        assert n == sum(p // sp + (p % sp != 0) for p in pages)
        assert sp >= 1


def test_plan_shapes_of_the_named_workloads():
    assert _plan([4096] * 64) == (16, 256)       # 64 x 4096: one split of 16 pages per CU
    assert _plan([131072] * 4) == (32, 256)      # 4 x 131072
    sp, n = _plan([256], mla.MLADims(16, 128, 128, 256, 32, dtype=torch.float32))
    assert n >= 1


def test_plan_env_override(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_SPLIT_PAGES", "3")
    assert _plan([64 * 7, 1, 0]) == (3, 3 + 1)


def test_choose_prefill_form():
    """The per-shape choice between the absorbed and the materialised prefill (host logic only)."""
    dsv2 = mla.MLADims(128, 128, 128, 512, 64)
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32)  # noqa: E731
    # a long chunk: 35.7 M visible pairs over 18,432 keys -> the materialised form
    assert mla.choose_prefill_form(dsv2, i32(0, 2048), i32(16384)) == "materialised"
    # a few queries over a long prefix: forming 100 k keys costs more than it saves
    assert mla.choose_prefill_form(dsv2, i32(0, 4), i32(100000)) == "absorbed"
    # nothing to do, a workspace over the limit, a shape the materialised form does not take
    assert mla.choose_prefill_form(dsv2, i32(0, 0), i32(0)) == "absorbed"
    assert mla.choose_prefill_form(dsv2, i32(0, 2048), i32(16384), workspace_limit=1 << 20) == "absorbed"
    f32 = mla.MLADims(16, 128, 128, 256, 32, dtype=torch.float32)
    assert mla.choose_prefill_form(f32, i32(0, 1024), i32(0)) == "absorbed"


def test_front_projections_validate():
    """The front-of-layer calls: workspace sizing and every rejection, before any launch."""
    d = _dims()
    i32p = ctypes.POINTER(ctypes.c_int32)
    ws_kv = B.LIB.mla_front_workspace_size(ctypes.byref(d), 64, 5120, 0)
    ws_q = B.LIB.mla_front_workspace_size(ctypes.byref(d), 64, 5120, 1536)
    assert 0 < ws_kv < ws_q
    assert ws_q % 256 == 0
    assert B.LIB.mla_front_workspace_size(ctypes.byref(d), 64, 5000, 1536) == 0      # d_model % 32
    assert B.LIB.mla_front_workspace_size(ctypes.byref(d), 64, 5120, 1500) == 0      # d_qlat % 32
    assert B.LIB.mla_front_workspace_size(ctypes.byref(_dims(dtype=0, work_dtype=0)), 64, 5120, 1536) == 0
    cache = B.PagedCache(FAKE.value, 4, FAKE.value, 2, 4)
    seq = ctypes.cast(FAKE, i32p)

    def kv(dims=d, n=64, d_model=5120, h=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return B.LIB.mla_kv_project(ctypes.byref(dims), ctypes.byref(cache), h, n, d_model, FAKE, FAKE, seq, seq,
                                    ws, ws_bytes, None)

    assert kv(n=0) == 0                      # nothing to do, nothing launched
    assert kv(d_model=100) == 1
    assert kv(dims=_dims(dtype=0, work_dtype=0)) == 2
    assert kv(h=None) == 1
    assert kv(h=ctypes.c_void_p(FAKE.value + 2)) == 1  # misaligned
    assert kv(ws_bytes=ws_kv - 1) == 3
    assert kv(ws=None) == 3

    def q(folded=False, n=64, d_qlat=1536, q_nope=FAKE, ws_bytes=1 << 40):
        if folded:
            return B.LIB.mla_q_project_folded(ctypes.byref(d), FAKE, n, 5120, d_qlat, FAKE, FAKE, FAKE, seq, FAKE,
                                              FAKE, ws_bytes, None)
        return B.LIB.mla_q_project(ctypes.byref(d), FAKE, n, 5120, d_qlat, FAKE, FAKE, FAKE, seq, q_nope, FAKE, FAKE,
                                   ws_bytes, None)

    assert q(n=0) == 0 and q(folded=True, n=0) == 0
    assert q(d_qlat=0) == 1 and q(folded=True, d_qlat=0) == 1
    assert q(q_nope=None) == 1               # the unfolded form writes q_nope
    assert q(ws_bytes=ws_q - 1) == 3 and q(folded=True, ws_bytes=ws_q - 1) == 3
    assert B.LIB.mla_fold_q_weights(ctypes.byref(d), 1536, None, FAKE, FAKE, None) == 1
    assert B.LIB.mla_fold_q_weights(ctypes.byref(d), 100, FAKE, FAKE, FAKE, None) == 1


def test_per_head_calls_validate():
    """The per-head-key calls: the supported shape only, and every rejection before any launch."""
    tiny = _dims(n_heads=16, d_head=128, d_v=128, d_latent=256, d_rope=32)
    cache = B.PagedCache(FAKE.value, 4, FAKE.value, 2, 4)
    i32p = ctypes.POINTER(ctypes.c_int32)
    seq = ctypes.cast(FAKE, i32p)

    def write(dims=tiny, n=8, lat=FAKE):
        return B.LIB.mla_cache_write_per_head(ctypes.byref(dims), ctypes.byref(cache), lat, FAKE, seq, seq, n, None)

    assert write(n=0) == 0
    assert write(dims=_dims()) == 2                           # the DeepSeek-V2 shape has no per-head kernel
    assert write(dims=_dims(n_heads=16, d_latent=256, d_rope=32, dtype=0, work_dtype=0)) == 2
    assert write(n=-1) == 1
    assert write(lat=None) == 1
    assert B.LIB.mla_last_error().decode()

    def decode(dims=tiny, lens=(100, 3), batch=None, ws=None, ws_bytes=0, q=FAKE):
        lens_host = (ctypes.c_int32 * len(lens))(*lens)
        return B.LIB.mla_decode_per_head(ctypes.byref(dims), ctypes.byref(cache), q, seq, lens_host,
                                         len(lens) if batch is None else batch, FAKE, None, ws, ws_bytes, None)

    assert decode(batch=0) == 0
    assert decode(dims=_dims()) == 2
    assert decode(q=None) == 1
    assert decode(lens=(300, 3)) == 1                          # beyond 4 pages of 64
    assert decode(lens=(1, 1, 1)) == 1                         # more rows than the block table
    lens = (ctypes.c_int32 * 2)(100, 3)
    need = B.LIB.mla_decode_workspace_size(ctypes.byref(tiny), 2, lens)
    if need:                                                   # a plan that splits needs the workspace
        assert decode(ws=FAKE, ws_bytes=need - 1) == 3

    def decode_proj(dims=tiny, lens=(100, 3), ws=None, ws_bytes=0, w_uv=FAKE, out=FAKE):
        lens_host = (ctypes.c_int32 * len(lens))(*lens)
        return B.LIB.mla_decode_per_head_proj(ctypes.byref(dims), ctypes.byref(cache), FAKE, seq, lens_host,
                                              len(lens), w_uv, out, None, ws, ws_bytes, None)

    assert decode_proj(w_uv=None) == 1
    assert decode_proj(out=None) == 1
    assert decode_proj(dims=_dims()) == 2
    assert decode_proj(dims=_dims(n_heads=16, d_head=128, d_v=64, d_latent=256, d_rope=32)) == 2
    need = B.LIB.mla_decode_proj_workspace_size(ctypes.byref(tiny), 2, lens)
    assert need > 0                                            # a partial slot per item, split or not
    assert decode_proj() == 3 and decode_proj(ws=FAKE, ws_bytes=need - 1) == 3


def test_header_compiles_as_c_and_cpp(tmp_path):
    """include/mla.h is a plain C header: it compiles as strict C99 and as C++17, warning-free."""
    import shutil
    import subprocess

    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use_header.c"
    src.write_text('#include "mla.h"\nint main(void) { mla_dims d; (void)d; return 0; }\n')
    for cc, args in (("gcc", ["-std=c99", "-pedantic"]), ("g++", ["-std=c++17", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} is not installed")
        res = subprocess.run([cc, *args, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
