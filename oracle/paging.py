"""Paged latent cache addressing (plain definition, integer only).

The pages say only that the cache holds, per token, the latent c_t and the
shared position key ("Latent Attention Meets RoPE", "Two small, telling
details"; "AI decoupled RoPE MLA", decoupled-RoPE section: 512 + 64 = 576
numbers per token).  Paging itself is not on the pages; the reading used is
the usual one: a sequence's logical page k = p // page_size lives in physical
page block_table[b, k], and position p occupies row p % page_size of it.
"""

from __future__ import annotations

import numpy as np


def slot(block_table: np.ndarray, seq: int, pos: int, page_size: int) -> int:
    """Physical row index (page * page_size + offset) of (seq, pos)."""
    page = int(block_table[seq, pos // page_size])
    if page < 0:
        raise IndexError("position falls in an unallocated page")
    return page * page_size + pos % page_size


def slots(block_table: np.ndarray, seqs, positions, page_size: int) -> np.ndarray:
    """Vector of physical rows for paired (seq, pos) lists, by plain loop."""
    return np.array([slot(block_table, int(b), int(p), page_size) for b, p in zip(seqs, positions)],
                    dtype=np.int64)
