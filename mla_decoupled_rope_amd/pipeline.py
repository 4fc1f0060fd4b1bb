"""Device-side state and the two hot-path pipelines built from the five C-ABI calls.

* ``LatentCache``  -- the paged [c | R k^R] cache and its block table.
* ``DecodeStep``   -- rope_absorb_q (new token + q^R + q~, one launch) -> decode
                      (split + merge) -> out_proj, with every buffer
                      preallocated so a step launches kernels only.
* ``LayerDecodeStep`` -- the same step from hidden states: kv_project (the new
                      token's cache row) -> q_project -> absorb_q (or
                      q_project_folded) -> decode -> out_proj.
* ``PrefillStep``  -- rope_absorb_q (chunk rows + q^R + q~) -> prefill ->
                      out_proj, or rope_apply -> prefill_mha (the materialised
                      form); ``choose_prefill_form`` picks between them.
"""

from __future__ import annotations

import torch

from . import binding as B


# Sustained rates measured on one MI355X (2048-token chunk after 16384 cached
# tokens, n_h = 128): the absorbed prefill attention, the materialised form's
# attention and its key/value up-projection, in flop/s.
ABSORBED_PREFILL_RATE = 1.25e15
MATERIALISED_ATTENTION_RATE = 0.92e15
UPPROJECTION_RATE = 0.57e15


def choose_prefill_form(dims: B.MLADims, cu_q_host: torch.Tensor, q_start_host: torch.Tensor,
                        workspace_limit: int = 8 << 30) -> str:
    """'materialised' or 'absorbed': the form with the smaller estimated time for this chunk.

    Both forms compute one result ("ropeabsorb" README: absorption is exact).
    The absorbed form spends 2 n_h (2 d_c + d_r) flop per visible (query, key)
    pair; the materialised form 2 n_h (d_h + d_r + d_v) per pair plus
    2 n_h (d_h + d_v) d_c per visible key to form the keys and values
    ("Multi-Head Latent Attention", the MLA dataflow).  Long chunks favour the
    materialised form, a few queries over a long prefix the absorbed one.  The
    materialised form is chosen only where mla_prefill_mha supports the shape
    and its workspace fits ``workspace_limit`` bytes.
    """
    cu = [int(x) for x in cu_q_host]
    st = [int(x) for x in q_start_host]
    pairs = keys = 0
    for b in range(len(st)):
        n = cu[b + 1] - cu[b]
        pairs += n * st[b] + n * (n + 1) // 2
        keys += st[b] + n
    if pairs == 0:
        return "absorbed"
    try:
        ws = B.prefill_mha_workspace_size(dims, cu_q_host, q_start_host)
    except B.MLAError:
        return "absorbed"
    if ws == 0 or ws > workspace_limit:
        return "absorbed"
    h, dc, dr, dh, dv = dims.n_heads, dims.d_latent, dims.d_rope, dims.d_head, dims.d_v
    t_abs = 2.0 * h * (2 * dc + dr) * pairs / ABSORBED_PREFILL_RATE
    t_mat = (2.0 * h * (dh + dr + dv) * pairs / MATERIALISED_ATTENTION_RATE
             + 2.0 * h * (dh + dv) * dc * keys / UPPROJECTION_RATE)
    return "materialised" if t_mat < t_abs else "absorbed"


class LatentCache:
    """Paged latent cache: data [num_pages, 64, d_c + d_r] and block table [num_seqs, max_pages]."""

    def __init__(self, dims: B.MLADims, block_table, num_pages: int, device="cuda", fill: float | None = None):
        self.dims = dims
        bt = torch.as_tensor(block_table, dtype=torch.int32)
        self.block_table_host = bt.contiguous()
        self.block_table = bt.to(device).contiguous()
        self.num_pages = int(num_pages)
        if fill is None:
            self.data = torch.empty((self.num_pages, dims.page_size, dims.row), dtype=dims.dtype, device=device)
        else:
            self.data = torch.full((self.num_pages, dims.page_size, dims.row), fill, dtype=dims.dtype, device=device)

    def write(self, kv_latent: torch.Tensor, k_rope: torch.Tensor, kv_seq: torch.Tensor, kv_pos: torch.Tensor):
        """Write rows [c | R_pos k^R] for (seq, pos) pairs (k^R un-rotated on input)."""
        B.rope_apply(self.dims, self.data, self.block_table, kv_latent=kv_latent, k_rope=k_rope,
                     kv_seq=kv_seq, kv_pos=kv_pos)


class DecodeStep:
    """One decode step for a fixed batch: buffers are allocated once here."""

    def __init__(self, dims: B.MLADims, cache: LatentCache, seq_lens_host: torch.Tensor, device="cuda"):
        self.dims, self.cache = dims, cache
        self.seq_lens_host = seq_lens_host.to(torch.int32).contiguous()
        self.seq_lens = self.seq_lens_host.to(device)
        n = self.seq_lens_host.numel()
        self.q_pos = (self.seq_lens - 1).clamp_min(0).to(torch.int32)
        self.q_lat = torch.empty((n, dims.n_heads, dims.row), dtype=dims.wdtype, device=device)
        self.out_latent = torch.empty((n, dims.n_heads, dims.d_latent), dtype=torch.float32, device=device)
        self.lse = torch.empty((n, dims.n_heads), dtype=torch.float32, device=device)
        self.out = torch.empty((n, dims.n_heads, dims.d_v), dtype=torch.float32, device=device)
        self.workspace = B.decode_workspace(dims, self.seq_lens_host, device)
        self.proj_ws_bytes = B.decode_proj_workspace_size(dims, self.seq_lens_host)
        self.proj_workspace = None  # allocated on the first fused call
        self.kv_seq = torch.arange(n, dtype=torch.int32, device=device)

    def run(self, q_nope, q_rope, w_uk, w_uv, new_latent=None, new_k_rope=None):
        """q_nope [B,H,d_h], q_rope [B,H,d_r] (un-rotated); optional new token rows at position T_b - 1."""
        d = self.dims
        B.rope_absorb_q(d, self.cache.data, self.cache.block_table, q_nope, w_uk, q_rope, self.q_pos, self.q_lat,
                        new_latent, new_k_rope, self.kv_seq if new_latent is not None else None,
                        self.q_pos if new_latent is not None else None)
        B.decode(d, self.cache.data, self.cache.block_table, self.q_lat, self.seq_lens, self.seq_lens_host,
                 self.out_latent, self.lse, self.workspace)
        B.out_proj(d, self.out_latent, w_uv, self.out)
        return self.out

    def attend_proj(self, w_uv):
        """mla_decode_proj over q_lat: the layer output in self.out, lse in self.lse (obar is not formed)."""
        if self.proj_workspace is None and self.proj_ws_bytes:
            self.proj_workspace = torch.empty(self.proj_ws_bytes, dtype=torch.uint8, device=self.q_lat.device)
        B.decode_proj(self.dims, self.cache.data, self.cache.block_table, self.q_lat, self.seq_lens,
                      self.seq_lens_host, w_uv, self.out, self.lse, self.proj_workspace)

    def attend_split_kv(self):
        """mla_decode_split_kv over q_lat: the first of mla_decode_proj's two launches (the split
        partials go to the fused workspace; merge_out_proj finishes the step)."""
        if self.proj_workspace is None and self.proj_ws_bytes:
            self.proj_workspace = torch.empty(self.proj_ws_bytes, dtype=torch.uint8, device=self.q_lat.device)
        B.decode_split_kv(self.dims, self.cache.data, self.cache.block_table, self.q_lat, self.seq_lens,
                          self.seq_lens_host, self.proj_workspace)

    def merge_out_proj(self, w_uv):
        """mla_merge_out_proj: the second launch, from the workspace attend_split_kv filled."""
        B.merge_out_proj(self.dims, self.seq_lens, self.seq_lens_host, w_uv, self.out, self.lse,
                         self.proj_workspace)

    def run_fused(self, q_nope, q_rope, w_uk, w_uv, new_latent=None, new_k_rope=None):
        """As run(), with attention, the split merge and the output absorption through
        mla_decode_proj: two launches after the query prologue instead of three."""
        d = self.dims
        B.rope_absorb_q(d, self.cache.data, self.cache.block_table, q_nope, w_uk, q_rope, self.q_pos, self.q_lat,
                        new_latent, new_k_rope, self.kv_seq if new_latent is not None else None,
                        self.q_pos if new_latent is not None else None)
        self.attend_proj(w_uv)
        return self.out


class PerHeadDecodeStep:
    """One decode step over a cache that keeps one position key per head (rows of
    d_latent + n_heads * d_rope): the same query path, mla_decode_per_head for
    attention.  Buffers, the cache included, are allocated once here."""

    def __init__(self, dims: B.MLADims, block_table, num_pages: int, seq_lens_host: torch.Tensor, device="cuda",
                 fill: float = 0.0):
        self.dims = dims
        self.cache = torch.full((num_pages, dims.page_size, B.per_head_row(dims)), fill, dtype=dims.dtype,
                                device=device)
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.seq_lens_host = seq_lens_host.to(torch.int32).contiguous()
        self.seq_lens = self.seq_lens_host.to(device)
        n = self.seq_lens_host.numel()
        self.q_pos = (self.seq_lens - 1).clamp_min(0).to(torch.int32)
        self.q_lat = torch.empty((n, dims.n_heads, dims.row), dtype=dims.wdtype, device=device)
        self.out_latent = torch.empty((n, dims.n_heads, dims.d_latent), dtype=torch.float32, device=device)
        self.lse = torch.empty((n, dims.n_heads), dtype=torch.float32, device=device)
        self.out = torch.empty((n, dims.n_heads, dims.d_v), dtype=torch.float32, device=device)
        self.workspace = B.decode_workspace(dims, self.seq_lens_host, device)
        self.proj_ws_bytes = B.decode_proj_workspace_size(dims, self.seq_lens_host)
        self.proj_workspace = None  # allocated on the first fused call

    def write(self, kv_latent, k_rope, kv_seq, kv_pos):
        """Cache rows [c | R_t k^R_{t,0} | ... ] for tokens (kv_seq, kv_pos); k_rope [n, H, d_r]."""
        B.cache_write_per_head(self.dims, self.cache, self.block_table, kv_latent, k_rope, kv_seq, kv_pos)

    def attend(self):
        B.decode_per_head(self.dims, self.cache, self.block_table, self.q_lat, self.seq_lens, self.seq_lens_host,
                          self.out_latent, self.lse, self.workspace)

    def attend_proj(self, w_uv):
        """mla_decode_per_head_proj over q_lat: the layer output in self.out, lse in self.lse."""
        if self.proj_workspace is None and self.proj_ws_bytes:
            self.proj_workspace = torch.empty(self.proj_ws_bytes, dtype=torch.uint8, device=self.q_lat.device)
        B.decode_per_head_proj(self.dims, self.cache, self.block_table, self.q_lat, self.seq_lens,
                               self.seq_lens_host, w_uv, self.out, self.lse, self.proj_workspace)

    def run_fused(self, q_nope, q_rope, w_uk, w_uv):
        """As run(), with attention, the split merge and the output absorption through
        mla_decode_per_head_proj."""
        B.rope_absorb_q(self.dims, None, None, q_nope, w_uk, q_rope, self.q_pos, self.q_lat)
        self.attend_proj(w_uv)
        return self.out

    def run(self, q_nope, q_rope, w_uk, w_uv):
        d = self.dims
        B.rope_absorb_q(d, None, None, q_nope, w_uk, q_rope, self.q_pos, self.q_lat)
        self.attend()
        B.out_proj(d, self.out_latent, w_uv, self.out)
        return self.out


class PrefillStep:
    """Causal chunked prefill for fixed chunk sizes: buffers are allocated once here."""

    def __init__(self, dims: B.MLADims, cache: LatentCache, cu_q_host: torch.Tensor, q_start_host: torch.Tensor,
                 device="cuda"):
        self.dims, self.cache = dims, cache
        self.cu_q_host = cu_q_host.to(torch.int32).contiguous()
        self.q_start_host = q_start_host.to(torch.int32).contiguous()
        self.cu_q = self.cu_q_host.to(device)
        self.q_start = self.q_start_host.to(device)
        n = int(self.cu_q_host[-1])
        counts = (self.cu_q_host[1:] - self.cu_q_host[:-1]).to(torch.int64)
        seq = torch.repeat_interleave(torch.arange(len(counts), dtype=torch.int32), counts)
        local = torch.arange(n, dtype=torch.int32) - self.cu_q_host[:-1].repeat_interleave(counts)
        self.q_pos = (self.q_start_host.repeat_interleave(counts) + local).to(torch.int32).to(device)
        self.kv_seq = seq.to(device)
        self.q_lat = torch.empty((n, dims.n_heads, dims.row), dtype=dims.wdtype, device=device)
        self.out_latent = torch.empty((n, dims.n_heads, dims.d_latent), dtype=torch.float32, device=device)
        self.lse = torch.empty((n, dims.n_heads), dtype=torch.float32, device=device)
        self.out = torch.empty((n, dims.n_heads, dims.d_v), dtype=torch.float32, device=device)

    def run(self, q_nope, q_rope, w_uk, w_uv, new_latent=None, new_k_rope=None):
        """Queries of the chunk at positions q_start[b] + j; optional chunk rows written to the cache first."""
        d = self.dims
        B.rope_absorb_q(d, self.cache.data, self.cache.block_table, q_nope, w_uk, q_rope, self.q_pos, self.q_lat,
                        new_latent, new_k_rope, self.kv_seq if new_latent is not None else None,
                        self.q_pos if new_latent is not None else None)
        B.prefill(d, self.cache.data, self.cache.block_table, self.q_lat, self.cu_q, self.q_start, self.cu_q_host,
                  self.q_start_host, self.out_latent, self.lse)
        B.out_proj(d, self.out_latent, w_uv, self.out)
        return self.out

    def run_best(self, q_nope, q_rope, w_uk, w_uv, new_latent=None, new_k_rope=None):
        """run() or run_materialised(), whichever choose_prefill_form picks for this chunk."""
        if getattr(self, "form", None) is None:
            self.form = choose_prefill_form(self.dims, self.cu_q_host, self.q_start_host)
        if self.form == "materialised":
            return self.run_materialised(q_nope, q_rope, w_uk, w_uv, new_latent, new_k_rope)
        return self.run(q_nope, q_rope, w_uk, w_uv, new_latent, new_k_rope)

    def run_materialised(self, q_nope, q_rope, w_uk, w_uv, new_latent=None, new_k_rope=None):
        """The same chunk through mla_prefill_mha (per-head keys and values up-projected)."""
        d = self.dims
        if new_latent is not None:
            B.rope_apply(d, self.cache.data, self.cache.block_table, q_rope=q_rope, q_pos=self.q_pos,
                         q_lat=self.q_lat, kv_latent=new_latent, k_rope=new_k_rope, kv_seq=self.kv_seq,
                         kv_pos=self.q_pos)
        else:
            B.rope_apply(d, None, None, q_rope=q_rope, q_pos=self.q_pos, q_lat=self.q_lat)
        if getattr(self, "mha_workspace", None) is None:
            self.mha_workspace = B.prefill_mha_workspace(d, self.cu_q_host, self.q_start_host,
                                                         device=self.q_lat.device)
        B.prefill_mha(d, self.cache.data, self.cache.block_table, q_nope, self.q_lat, w_uk, w_uv, self.cu_q,
                      self.q_start, self.cu_q_host, self.q_start_host, self.out, self.lse, self.mha_workspace)
        return self.out


class LayerPrefillStep:
    """Causal chunked prefill of one layer from hidden states: the chunk's cache rows
    [c | R k^R] through mla_kv_project, its queries through mla_q_project (+ mla_absorb_q)
    or mla_q_project_folded, then mla_prefill and mla_out_proj.  Positions before each
    chunk must already be in the cache."""

    def __init__(self, dims: B.MLADims, cache: LatentCache, cu_q_host: torch.Tensor, q_start_host: torch.Tensor,
                 d_model: int, d_qlat: int, folded: bool, device="cuda"):
        self.dims, self.folded = dims, folded
        self.inner = PrefillStep(dims, cache, cu_q_host, q_start_host, device)
        n = int(self.inner.cu_q_host[-1])
        self.q_nope = torch.empty((n, dims.n_heads, dims.d_head), dtype=dims.dtype, device=device)
        self.front_ws = B.front_workspace(dims, n, d_model, d_qlat, device)

    def run(self, h, w_dkv, w_kr, w_dq, w_up, w_qr, w_uk, w_uv):
        """h [n, d_model]: the chunk's tokens in (sequence, position) order; w_up is W_UQ, or the
        folded weight when the step is folded."""
        s, d = self.inner, self.dims
        B.kv_project(d, s.cache.data, s.cache.block_table, h, w_dkv, w_kr, s.kv_seq, s.q_pos, self.front_ws)
        if self.folded:
            B.q_project_folded(d, h, w_dq, w_up, w_qr, s.q_pos, s.q_lat, self.front_ws)
        else:
            B.q_project(d, h, w_dq, w_up, w_qr, s.q_pos, self.q_nope, s.q_lat, self.front_ws)
            B.absorb_q(d, self.q_nope, w_uk, s.q_lat)
        B.prefill(d, s.cache.data, s.cache.block_table, s.q_lat, s.cu_q, s.q_start, s.cu_q_host, s.q_start_host,
                  s.out_latent, s.lse)
        B.out_proj(d, s.out_latent, w_uv, s.out)
        return s.out


class LayerDecodeStep:
    """One decode step from hidden states h [B, d_model] of each sequence's newest token.

    The token sits at position seq_lens[b] - 1: kv_project writes its cache row,
    the query goes through the query latent (q_project + absorb_q, or
    q_project_folded with a pre-folded W_UK), then decode and out_proj.
    """

    def __init__(self, dims: B.MLADims, cache: LatentCache, seq_lens_host: torch.Tensor, d_model: int, d_qlat: int,
                 folded: bool = False, device="cuda"):
        self.inner = DecodeStep(dims, cache, seq_lens_host, device)
        self.dims, self.cache, self.folded = dims, cache, folded
        n = self.inner.seq_lens_host.numel()
        self.q_nope = torch.empty((n, dims.n_heads, dims.d_head), dtype=dims.dtype, device=device)
        self.front_ws = B.front_workspace(dims, n, d_model, d_qlat, device)

    def kv(self, h, w_dkv, w_kr):
        s = self.inner
        B.kv_project(self.dims, self.cache.data, self.cache.block_table, h, w_dkv, w_kr, s.kv_seq, s.q_pos,
                     self.front_ws)

    def query(self, h, w_dq, w_up, w_qr, w_uk):
        """w_up is W_UQ, or W_fold when the step is folded."""
        s = self.inner
        if self.folded:
            B.q_project_folded(self.dims, h, w_dq, w_up, w_qr, s.q_pos, s.q_lat, self.front_ws)
        else:
            B.q_project(self.dims, h, w_dq, w_up, w_qr, s.q_pos, self.q_nope, s.q_lat, self.front_ws)
            B.absorb_q(self.dims, self.q_nope, w_uk, s.q_lat)

    def attend(self, w_uv):
        s, d = self.inner, self.dims
        B.decode(d, self.cache.data, self.cache.block_table, s.q_lat, s.seq_lens, s.seq_lens_host, s.out_latent,
                 s.lse, s.workspace)
        B.out_proj(d, s.out_latent, w_uv, s.out)
        return s.out

    def run(self, h, w_dkv, w_kr, w_dq, w_up, w_qr, w_uk, w_uv):
        self.kv(h, w_dkv, w_kr)
        self.query(h, w_dq, w_up, w_qr, w_uk)
        return self.attend(w_uv)
