"""fp64 decode attention against a paged key/value cache.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU-baseline leg.

[WGC] lists, among its follow-up directions, combining the kernel with
PagedAttention-style key/value cache management; the pages say no more. The
reading taken here is the usual one for a paged cache: a sequence's cached
positions live in fixed-size pages of page_size positions, scattered over a
shared pool, and a per-sequence block table names the physical page that
holds the sequence's j-th logical page. Position p of sequence b is row
p % page_size of page block_table[b][p // page_size]. Layout of the pool:
k_cache, v_cache [num_pages][H][page_size][d] (one page holds every head's
rows for those positions). seq_lens[b] positions are valid; rows past them
in the last page are never read.

The paged cache is only an addressing scheme: gathering a sequence's first
seq_lens[b] positions in logical order gives the contiguous K and V of the
sequence, and the result is decode attention over those (oracle.decode,
[JJ] section 3: the Nq queries are the sequence's last Nq positions).
"""
from __future__ import annotations

import torch

from .decode import attention_decode


def gather_pages(cache, table_row, seq_len: int, page_size: int):
    """[H][seq_len][d] rows of one sequence, in logical order, from a paged pool."""
    cache = torch.as_tensor(cache)
    rows = []
    for pos0 in range(0, seq_len, page_size):
        page = int(table_row[pos0 // page_size])
        n = min(page_size, seq_len - pos0)
        rows.append(cache[page, :, :n, :])
    if not rows:
        return cache.new_zeros((cache.shape[1], 0, cache.shape[3]))
    return torch.cat(rows, dim=1)


def attention_decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float,
                           causal: bool = False):
    """q [B][H][Nq][d]; caches [P][H][page_size][d]; block_table [B][max_pages];
    seq_lens [B] (Nq <= seq_len) -> (o [B][H][Nq][d], lse [B][H][Nq]) in fp64."""
    q = torch.as_tensor(q).double()
    B, H, Nq, d = q.shape
    page_size = k_cache.shape[2]
    o = torch.empty((B, H, Nq, d), dtype=torch.float64)
    lse = torch.empty((B, H, Nq), dtype=torch.float64)
    for b in range(B):
        n = int(seq_lens[b])
        k = gather_pages(k_cache, block_table[b], n, page_size)
        v = gather_pages(v_cache, block_table[b], n, page_size)
        o[b], lse[b] = attention_decode(q[b], k, v, scale, causal)
    return o, lse
