"""Seeded synthetic inputs for MLA decode and causal prefill.

This module is the only code shared by the CPU oracle's tests and the GPU
tests / benchmark.  It draws random numbers, forms the *inputs* of the
five-call boundary (latent c, un-rotated k^R, content query q^C, un-rotated
q^R, the up-projection weights), rounds them to the storage dtype and lays out
pages.  It holds none of the attention arithmetic: no RoPE, no absorption, no
score, no softmax.

Every array value is exactly representable in the storage dtype and is kept
as float32, so the oracle (float64 upcast) and the GPU (bf16 / fp32 tensors)
read identical numbers.

Shapes are the pages' two worked examples:
* TINY  -- "Multi-Head Latent Attention" (talalahmed.dev), "A concrete size
  comparison": 16 heads, key/value dims 128, latent 256, RoPE 32.
* DSV2  -- "AI decoupled RoPE MLA" (operatorworld.com): 128 heads x 128,
  latent d_c = 512, RoPE d_r = 64 (576 numbers per token).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

try:  # torch is only used for the bf16 round-to-nearest-even cast
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclass(frozen=True)
class Shape:
    n_heads: int
    d_head: int
    d_v: int
    d_latent: int
    d_rope: int
    hidden: int = 0
    page_size: int = 64
    rope_base: float = 10000.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_head + self.d_rope)

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope


TINY = Shape(n_heads=16, d_head=128, d_v=128, d_latent=256, d_rope=32, hidden=2048)
DSV2 = Shape(n_heads=128, d_head=128, d_v=128, d_latent=512, d_rope=64, hidden=5120)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype (RNE) and return the values as float32."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype != "bf16":
        raise ValueError(dtype)
    if torch is not None:
        return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    u = x32.view(np.uint32).astype(np.uint64)  # pragma: no cover - torch is always present here
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


@dataclass
class Case:
    """One workload.  Token rows of sequence b start at row_offsets[b]."""

    shape: Shape
    dtype: str
    kind: str                      # "decode" or "prefill"
    seq_lens: np.ndarray           # int32 [B]: cached tokens per sequence (incl. new ones)
    row_offsets: np.ndarray        # int64 [B]
    c_rows: np.ndarray             # [sum T, d_c]
    kr_rows: np.ndarray            # [sum T, d_r], or [sum T, H, d_r] with per-head keys (un-rotated)
    qc: np.ndarray                 # [N, H, d_h]
    qr: np.ndarray                 # [N, H, d_r]   (un-rotated)
    q_pos: np.ndarray              # int32 [N]
    w_uk: np.ndarray               # [H, d_h, d_c]
    w_uv: np.ndarray               # [H, d_v, d_c]
    block_table: np.ndarray        # int32 [B, max_pages], -1 padded
    num_pages: int
    cu_q: np.ndarray | None = None     # prefill: int32 [B+1]
    q_start: np.ndarray | None = None  # prefill: int32 [B], position of each chunk's first query
    seed: int = 0
    note: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def total_tokens(self) -> int:
        return int(np.sum(self.seq_lens, dtype=np.int64))

    def kv_seq_pos(self):
        """(seq, pos) of every cached token row, in row order."""
        seqs = np.repeat(np.arange(self.batch, dtype=np.int32), self.seq_lens)
        pos = np.concatenate([np.arange(t, dtype=np.int32) for t in self.seq_lens]) \
            if self.batch else np.zeros(0, np.int32)
        return seqs, pos


def allocate_pages(seq_lens, page_size: int, rng: np.random.Generator | None, shuffle: bool):
    """Block table for a pool of exactly sum ceil(T_b / page_size) pages.

    Physical ids are a seeded permutation of the pool (or the identity),
    handed out in (sequence, logical page) order; unused entries are -1.
    """
    pages = [(int(t) + page_size - 1) // page_size for t in seq_lens]
    pool = int(sum(pages))
    ids = rng.permutation(pool).astype(np.int32) if shuffle else np.arange(pool, dtype=np.int32)
    max_pages = max(pages) if pages else 0
    table = np.full((len(pages), max(1, max_pages)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(pages):
        table[b, :n] = ids[k:k + n]
        k += n
    return table, pool


def _normal(rng, shape, dtype=np.float32):
    return rng.standard_normal(shape, dtype=dtype)


def _offsets(seq_lens):
    off = np.zeros(len(seq_lens), dtype=np.int64)
    if len(seq_lens) > 1:
        off[1:] = np.cumsum(np.asarray(seq_lens, np.int64))[:-1]
    return off


def direct_decode(shape: Shape, dtype: str, seq_lens, seed: int, shuffle: bool = False,
                  weight_seed_offset: int = 0, per_head_rope: bool = False) -> Case:
    """Decode inputs drawn directly: c, k^R, q^C, q^R ~ N(0,1); W ~ N(0,1)/sqrt(d_c).

    Draw order: c rows, k^R rows, q^C, q^R, W_UK, W_UV, then the page
    permutation.  Query b sits at position T_b - 1.  per_head_rope draws one
    position key per head and token ([sum T, H, d_r]) in place of one per token.
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    total = int(seq_lens.sum(dtype=np.int64))
    h, s = shape.n_heads, shape
    c = to_storage(_normal(rng, (total, s.d_latent)), dtype)
    kr = to_storage(_normal(rng, (total, h, s.d_rope) if per_head_rope else (total, s.d_rope)), dtype)
    qc = to_storage(_normal(rng, (len(seq_lens), h, s.d_head)), dtype)
    qr = to_storage(_normal(rng, (len(seq_lens), h, s.d_rope)), dtype)
    w_uk = to_storage(_normal(rng, (h, s.d_head, s.d_latent), np.float64) / math.sqrt(s.d_latent), dtype)
    w_uv = to_storage(_normal(rng, (h, s.d_v, s.d_latent), np.float64) / math.sqrt(s.d_latent), dtype)
    table, pool = allocate_pages(seq_lens, s.page_size, rng, shuffle)
    return Case(shape, dtype, "decode", seq_lens, _offsets(seq_lens), c, kr, qc, qr,
                np.maximum(seq_lens - 1, 0).astype(np.int32), w_uk, w_uv, table, pool, seed=seed)


def direct_prefill(shape: Shape, dtype: str, prior_lens, new_lens, seed: int,
                   shuffle: bool = False) -> Case:
    """Chunked causal prefill inputs drawn directly (values N(0,1), W ~ N(0,1)/sqrt(d_c)).

    Sequence b already holds prior_lens[b] tokens and appends new_lens[b]
    tokens whose queries sit at positions prior_lens[b] .. prior_lens[b] +
    new_lens[b] - 1.  Draw order as in ``direct_decode``.
    """
    rng = np.random.default_rng(seed)
    prior = np.asarray(prior_lens, dtype=np.int32)
    new = np.asarray(new_lens, dtype=np.int32)
    seq_lens = (prior + new).astype(np.int32)
    total = int(seq_lens.sum(dtype=np.int64))
    nq = int(new.sum(dtype=np.int64))
    h, s = shape.n_heads, shape
    c = to_storage(_normal(rng, (total, s.d_latent)), dtype)
    kr = to_storage(_normal(rng, (total, s.d_rope)), dtype)
    qc = to_storage(_normal(rng, (nq, h, s.d_head)), dtype)
    qr = to_storage(_normal(rng, (nq, h, s.d_rope)), dtype)
    w_uk = to_storage(_normal(rng, (h, s.d_head, s.d_latent), np.float64) / math.sqrt(s.d_latent), dtype)
    w_uv = to_storage(_normal(rng, (h, s.d_v, s.d_latent), np.float64) / math.sqrt(s.d_latent), dtype)
    table, pool = allocate_pages(seq_lens, s.page_size, rng, shuffle)
    cu_q = np.zeros(len(new) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(new)
    q_pos = np.concatenate([p + np.arange(n, dtype=np.int32) for p, n in zip(prior, new)]) \
        if len(new) else np.zeros(0, np.int32)
    return Case(shape, dtype, "prefill", seq_lens, _offsets(seq_lens), c, kr, qc, qr,
                q_pos.astype(np.int32), w_uk, w_uv, table, pool, cu_q=cu_q, q_start=prior, seed=seed)


def _projected(shape: Shape, dtype: str, n_seq: int, t_seq: int, seed: int, query_rows):
    """Inputs formed from a hidden state, the way the tiny configs are stated.

    h ~ N(0,1) [n_seq, T, hidden]; W_DKV [d_c, hidden], W_KR [d_r, hidden],
    W_Q [H d_h, hidden], W_QR [H d_r, hidden] ~ N(0,1)/sqrt(hidden);
    W_UK, W_UV [H, *, d_c] ~ N(0,1)/sqrt(d_c).  Draw order is that list.
    c = W_DKV h, k^R = W_KR h (one per token), q^C = W_Q h, q^R = W_QR h, all
    in float64, then rounded to the storage dtype.  These projections sit in
    front of the five-call boundary; they are input construction only.
    """
    s = shape
    rng = np.random.default_rng(seed)
    hid = rng.standard_normal((n_seq, t_seq, s.hidden))
    w_dkv = rng.standard_normal((s.d_latent, s.hidden)) / math.sqrt(s.hidden)
    w_kr = rng.standard_normal((s.d_rope, s.hidden)) / math.sqrt(s.hidden)
    w_q = rng.standard_normal((s.n_heads * s.d_head, s.hidden)) / math.sqrt(s.hidden)
    w_qr = rng.standard_normal((s.n_heads * s.d_rope, s.hidden)) / math.sqrt(s.hidden)
    w_uk = rng.standard_normal((s.n_heads, s.d_head, s.d_latent)) / math.sqrt(s.d_latent)
    w_uv = rng.standard_normal((s.n_heads, s.d_v, s.d_latent)) / math.sqrt(s.d_latent)
    flat = hid.reshape(n_seq * t_seq, s.hidden)
    c = to_storage(flat @ w_dkv.T, dtype)
    kr = to_storage(flat @ w_kr.T, dtype)
    hq = hid[:, query_rows, :].reshape(-1, s.hidden)
    qc = to_storage((hq @ w_q.T).reshape(-1, s.n_heads, s.d_head), dtype)
    qr = to_storage((hq @ w_qr.T).reshape(-1, s.n_heads, s.d_rope), dtype)
    return rng, c, kr, qc, qr, to_storage(w_uk, dtype), to_storage(w_uv, dtype)


def config1(seed: int = 1) -> Case:
    """Tiny MLA decode, fp32: one query at position 255 over 256 cached tokens."""
    rng, c, kr, qc, qr, w_uk, w_uv = _projected(TINY, "f32", 1, 256, seed, [255])
    seq_lens = np.array([256], np.int32)
    table, pool = allocate_pages(seq_lens, TINY.page_size, rng, False)
    return Case(TINY, "f32", "decode", seq_lens, _offsets(seq_lens), c, kr, qc, qr,
                np.array([255], np.int32), w_uk, w_uv, table, pool, seed=seed,
                note={"workload": "tiny MLA decode fp32, 1 x 256 tokens"})


def config2(seed: int = 2) -> Case:
    """Tiny causal prefill, bf16: 4 sequences of 1024 tokens at positions 0..1023."""
    b, t = 4, 1024
    rng, c, kr, qc, qr, w_uk, w_uv = _projected(TINY, "bf16", b, t, seed, slice(None))
    seq_lens = np.full(b, t, np.int32)
    table, pool = allocate_pages(seq_lens, TINY.page_size, rng, False)
    cu_q = np.arange(b + 1, dtype=np.int32) * t
    q_pos = np.tile(np.arange(t, dtype=np.int32), b)
    return Case(TINY, "bf16", "prefill", seq_lens, _offsets(seq_lens), c, kr, qc, qr, q_pos,
                w_uk, w_uv, table, pool, cu_q=cu_q, q_start=np.zeros(b, np.int32), seed=seed,
                note={"workload": "tiny causal prefill bf16, 4 x 1024 tokens"})


def config3(seed: int = 3) -> Case:
    """DeepSeek-V2-like decode: 64 sequences x 4096 cached tokens, bf16."""
    case = direct_decode(DSV2, "bf16", np.full(64, 4096, np.int32), seed)
    case.note["workload"] = "MLA decode bf16, n_h=128 d_c=512 d_r=64, 64 x 4096 tokens"
    return case


def config4_lengths(seed: int = 4) -> np.ndarray:
    """128 lengths uniform on the integers 512 .. 32768 inclusive."""
    return np.random.default_rng(seed).integers(512, 32768, size=128, endpoint=True).astype(np.int32)


def config4(seed: int = 4) -> Case:
    """Ragged paged decode: 128 sequences, lengths U{512..32768}, shuffled 64-token pages."""
    case = direct_decode(DSV2, "bf16", config4_lengths(seed), seed + 1000, shuffle=True)
    case.note["workload"] = "MLA ragged paged decode bf16, 128 seqs, T ~ U[512, 32768]"
    return case


def config5_decode(seed: int = 5) -> Case:
    """Long-context decode: 4 sequences x 131072 cached tokens."""
    case = direct_decode(DSV2, "bf16", np.full(4, 131072, np.int32), seed)
    case.note["workload"] = "MLA long-context decode bf16, 4 x 131072 tokens"
    return case


def config5_prefill(seed: int = 5) -> Case:
    """Chunked causal prefill: 2048 new tokens after 16384 cached ones, one sequence."""
    case = direct_prefill(DSV2, "bf16", [16384], [2048], seed + 1000)
    case.note["workload"] = "MLA chunked causal prefill bf16, 2048 new over 16384 cached"
    return case


@dataclass
class FrontCase:
    """Hidden states and the projection weights of one layer (the front of the layer).

    h [total tokens, d_model] in (sequence, position) row order; the weights
    W_DKV [d_c, d_model], W_KR [d_r, d_model], W_DQ [d_q, d_model],
    W_UQ [H, d_h, d_q], W_QR [H, d_r, d_q], W_UK [H, d_h, d_c], W_UV [H, d_v, d_c].
    """
    shape: Shape
    d_model: int
    d_qlat: int
    seq_lens: np.ndarray
    h: np.ndarray
    w_dkv: np.ndarray
    w_kr: np.ndarray
    w_dq: np.ndarray
    w_uq: np.ndarray
    w_qr: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    block_table: np.ndarray
    num_pages: int
    seed: int = 0

    @property
    def row_offsets(self) -> np.ndarray:
        return _offsets(self.seq_lens)

    def kv_seq_pos(self):
        seqs = np.repeat(np.arange(len(self.seq_lens), dtype=np.int32), self.seq_lens)
        pos = np.concatenate([np.arange(t, dtype=np.int32) for t in self.seq_lens]) \
            if len(self.seq_lens) else np.zeros(0, np.int32)
        return seqs, pos


def front_layer(shape: Shape, seq_lens, d_model: int, d_qlat: int, seed: int, shuffle: bool = True,
                dtype: str = "bf16") -> FrontCase:
    """h ~ N(0,1); every weight ~ N(0,1)/sqrt(fan_in) (fan_in = its input width).
    Draw order: h, W_DKV, W_KR, W_DQ, W_UQ, W_QR, W_UK, W_UV, then the page permutation.
    All values rounded to the storage dtype."""
    s = shape
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    rng = np.random.default_rng(seed)
    total = int(seq_lens.sum())

    def w(shape_, fan_in):
        return to_storage(rng.standard_normal(shape_) / math.sqrt(fan_in), dtype)

    h = to_storage(rng.standard_normal((total, d_model)), dtype)
    w_dkv = w((s.d_latent, d_model), d_model)
    w_kr = w((s.d_rope, d_model), d_model)
    w_dq = w((d_qlat, d_model), d_model)
    w_uq = w((s.n_heads, s.d_head, d_qlat), d_qlat)
    w_qr = w((s.n_heads, s.d_rope, d_qlat), d_qlat)
    w_uk = w((s.n_heads, s.d_head, s.d_latent), s.d_latent)
    w_uv = w((s.n_heads, s.d_v, s.d_latent), s.d_latent)
    table, pool = allocate_pages(seq_lens, s.page_size, rng, shuffle)
    return FrontCase(s, d_model, d_qlat, seq_lens, h, w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, table, pool, seed)
