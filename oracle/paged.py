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
* Prefill over the cache (the page's "prefix caching" use): q_len new query
  rows per sequence sit at positions L_s - q_len .. L_s - 1 of a sequence
  whose L_s keys (the new rows' own included) are in the pool, and attend
  causally. Decode is the case q_len = 1.
* Block-sparse cross-attention (the page's retrieval / multi-modal use, where
  each query block reads its own set of pages): query block b of sequence s
  (rows b*q_block .. b*q_block + q_block - 1) attends, with no mask, to the
  first kv_lens[s, b] tokens of the concatenation of pages
  page_table[s, b, 0], page_table[s, b, 1], ... in list order.
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


def prefill(q, k_pool, v_pool, block_table, seq_lens, scale, page_size=16):
    """Causal attention of q [S, H, q_len, d] (rows at positions L_s - q_len ..
    L_s - 1) over each sequence's gathered keys. Returns (O [S, H, q_len, dv],
    LSE [S, H, q_len])."""
    q = np.asarray(q, dtype=np.float64)
    ks = gather(k_pool, block_table, seq_lens, page_size)
    vs = gather(v_pool, block_table, seq_lens, page_size)
    n_seq, n_head, q_len, _ = q.shape
    o = np.zeros((n_seq, n_head, q_len, np.asarray(v_pool).shape[-1]))
    lse = np.zeros((n_seq, n_head, q_len))
    for s in range(n_seq):
        length = int(seq_lens[s])
        o[s], lse[s] = attention(q[s], ks[s].astype(np.float64), vs[s].astype(np.float64), scale,
                                 mask="causal", q_pos_offset=length - q_len)
    return o, lse


def listed_keys(pool, pages, n_tokens, page_size):
    """The first n_tokens rows of the concatenation of pool[pages[0]],
    pool[pages[1]], ...: array [H, n_tokens, d] (values copied exactly)."""
    pool = np.asarray(pool)
    t = np.arange(n_tokens)
    rows = pool[np.asarray(pages)[t // page_size], :, t % page_size, :]      # [n, H, d]
    return np.ascontiguousarray(rows.transpose(1, 0, 2))


def cross(q, k_pool, v_pool, page_table, kv_lens, scale, page_size=64, q_block=128):
    """Block-sparse paged cross-attention. q: [S, H, q_len, d];
    page_table: [S, QB, max_pages]; kv_lens: [S, QB]. A query block with no
    key gets O = 0 and LSE = -inf. Returns (O [S, H, q_len, dv], LSE [S, H, q_len])."""
    q = np.asarray(q, dtype=np.float64)
    page_table = np.asarray(page_table)
    kv_lens = np.asarray(kv_lens)
    n_seq, n_head, q_len, _ = q.shape
    dv = np.asarray(v_pool).shape[-1]
    o = np.zeros((n_seq, n_head, q_len, dv))
    lse = np.full((n_seq, n_head, q_len), -np.inf)
    for s in range(n_seq):
        for b in range(-(-q_len // q_block)):
            r0, r1 = b * q_block, min(q_len, (b + 1) * q_block)
            n = int(kv_lens[s, b])
            if n == 0:
                continue
            k = listed_keys(k_pool, page_table[s, b], n, page_size).astype(np.float64)
            v = listed_keys(v_pool, page_table[s, b], n, page_size).astype(np.float64)
            o[s, :, r0:r1], lse[s, :, r0:r1] = attention(q[s, :, r0:r1], k, v, scale, mask="none")
    return o, lse
