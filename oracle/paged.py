"""Paged KV cache: block-table gather and single-query decode (fp64).

Test infrastructure (see the package docstring).

Follows "Optimizing Triton kernels for custom attention patterns on H100",
Pattern C: a pool of fixed-size pages, a per-sequence block table mapping a
logical page slot to a physical page id, and a gather that copies page
block_table[b, slot] of the pool to slot ``slot`` of a dense per-sequence
buffer (page size 16 is the default named there).

Readings:
* The page's pool is [num_pages, page_size, head_dim] for one head. With H
  heads the pool here is [num_pages, H, page_size, d]: each (page, head) slice
  is exactly the page's [page_size, head_dim] tile, and one block table per
  sequence serves all heads.
* Token t of sequence s lives in page block_table[s, t // page_size], row
  t % page_size. Only tokens t < seq_lens[s] exist.
* Decode has one new query per sequence, at position L_s - 1, so under a
  causal mask it sees every one of the L_s cached keys.
"""

import numpy as np

from .attention import attention


def gather(pool, block_table, seq_lens, page_size=16):
    """Dense per-sequence copies: list of arrays [H, L_s, d], one per sequence.

    Pure indexing: element values are copied bit for bit (dtype preserved).
    """
    pool = np.asarray(pool)
    block_table = np.asarray(block_table)
    out = []
    for s, length in enumerate(np.asarray(seq_lens).tolist()):
        t = np.arange(length)
        pages = block_table[s, t // page_size]
        rows = t % page_size
        dense = pool[pages, :, rows, :]          # [L, H, d]
        out.append(np.ascontiguousarray(dense.transpose(1, 0, 2)))
    return out


def decode(q, k_pool, v_pool, block_table, seq_lens, scale, page_size=16):
    """O[s, h] = attention of query q[s, h] (position L_s - 1) over the
    sequence's L_s gathered keys. q: [S, H, d]. Returns (O [S, H, d], LSE [S, H])."""
    q = np.asarray(q, dtype=np.float64)
    ks = gather(k_pool, block_table, seq_lens, page_size)
    vs = gather(v_pool, block_table, seq_lens, page_size)
    n_seq, n_head, d = q.shape
    o = np.zeros((n_seq, n_head, np.asarray(v_pool).shape[-1]))
    lse = np.zeros((n_seq, n_head))
    for s in range(n_seq):
        length = int(seq_lens[s])
        o_s, lse_s = attention(q[s][:, None, :], ks[s].astype(np.float64), vs[s].astype(np.float64),
                               scale, mask="causal", q_pos_offset=length - 1)
        o[s] = o_s[:, 0, :]
        lse[s] = lse_s[:, 0]
    return o, lse
