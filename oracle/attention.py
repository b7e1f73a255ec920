"""Plain fp64 attention: the result the tiled method must reach exactly.

Test infrastructure (see the package docstring): only tests, smoke() and the
bench's cpu_baseline leg may use it.

Definition followed: "Flash MSA Attention Kernel Implementation Tutorial",
section "Why We Needed a New Attention Kernel" (form S = Q K^T, take the
softmax, multiply by V) and section "Understanding Flash MSA Core Mechanics"
(the softmax subtracts the row maximum before exponentiating and divides by
the sum of the exponentials). The caller passes the scale; the pages use
1/sqrt(head_dim) (kernel listing in "Implementation Step-by-Step with
Triton").

Visibility (which key j a query i may attend to):
  none    -- every key.
  causal  -- j <= i (a decoder mask; "Flash MSA ...", "Trade-offs and Common
             Pitfalls").
  sliding -- i - window < j <= i. "Optimizing Triton kernels for custom
             attention patterns on H100", Pattern B, describes a window of W
             neighbours; the one-sided causal window used here is the reading
             taken for causal decoders (the page's prose says +-W, two-sided).
  band    -- |i - j| <= window: the two-sided window of that same passage
             (W neighbours on each side, 2W + 1 keys away from the edges).
  prefix_lm -- j <= i or j < window: the first `window` positions form a
             prefix every query sees in full (the prefix attends to itself
             bidirectionally); the rest is causal. The page names prefix-LM
             masks among the structured masks at the end of Pattern B without
             defining them; this is the usual meaning of the term.
  document -- i and j lie in the same document. "Optimizing Triton kernels
             ...", Pattern A: doc_offsets [num_docs + 1] holds the start of
             each document (the last entry is N), position p belongs to
             document searchsorted(doc_offsets, p, side='right') - 1, and a
             key outside [doc_start, doc_end) of the query's document is
             masked. Within a document every key is visible (the page stresses
             the mask is not causal). Empty documents (equal consecutive
             offsets) hold no position.
  document_causal -- document and j <= i: variable-length causal sequences
             packed end to end (a varlen batch), each attending causally only
             to itself.

Nothing here is blocked, fused or reordered: S is materialised (in blocks of
whole rows only to bound memory, which changes no arithmetic) and the softmax
runs in two passes.
"""

import numpy as np

MASKS = ("none", "causal", "sliding", "band", "prefix_lm", "document", "document_causal")
_ROW_BLOCK = 1024


def document_of(doc_offsets, pos):
    """Document index of each position: the last d with doc_offsets[d] <= pos."""
    offs = np.asarray(doc_offsets, dtype=np.int64)
    return np.searchsorted(offs, np.asarray(pos, dtype=np.int64), side="right") - 1


def check_doc_offsets(doc_offsets, n):
    """Offsets must start at 0, end at n and never decrease."""
    offs = np.asarray(doc_offsets, dtype=np.int64)
    if offs.ndim != 1 or offs.size < 2 or offs[0] != 0 or offs[-1] != n or np.any(np.diff(offs) < 0):
        raise ValueError("doc_offsets must be [0, ..., n], non-decreasing")
    return offs


def visible(mask, n_q, n_k, window=None, q_pos=None, doc_offsets=None):
    """Boolean matrix V[i, j] = key j visible to query i.

    ``q_pos`` gives the absolute position of each query row (default
    0..n_q-1); keys sit at positions 0..n_k-1. ``window`` is the window
    (sliding, band) or prefix length (prefix_lm); ``doc_offsets`` the document
    starts (document masks, which need n_k == n_q positions of one sequence).
    """
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    i = np.arange(n_q, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    j = np.arange(n_k, dtype=np.int64)
    if mask == "none":
        return np.ones((i.size, n_k), dtype=bool)
    if mask == "band":
        if window is None or window < 0:
            raise ValueError("band mask needs window >= 0")
        return np.abs(j[None, :] - i[:, None]) <= window
    if mask in ("document", "document_causal"):
        offs = check_doc_offsets(doc_offsets, n_k)
        vis = document_of(offs, i)[:, None] == document_of(offs, j)[None, :]
        if mask == "document_causal":
            vis &= j[None, :] <= i[:, None]
        return vis
    vis = j[None, :] <= i[:, None]
    if mask == "sliding":
        if window is None or window < 1:
            raise ValueError("sliding mask needs window >= 1")
        vis &= j[None, :] > (i[:, None] - window)
    if mask == "prefix_lm":
        if window is None or window < 0:
            raise ValueError("prefix_lm mask needs a prefix length >= 0")
        vis |= (j < window)[None, :]
    return vis


def visible_pair_count(mask, n, window=None, doc_offsets=None):
    """Number of visible (i, j) pairs of an n x n mask, counted row by row."""
    total = 0
    for i in range(n):
        if mask == "none":
            total += n
        elif mask == "causal":
            total += i + 1
        elif mask == "sliding":
            total += min(i + 1, window)
        elif mask == "band":
            total += min(n - 1, i + window) - max(0, i - window) + 1
        elif mask == "prefix_lm":
            total += max(i + 1, min(window, n))
        else:
            d = int(document_of(doc_offsets, i))
            start = int(doc_offsets[d])
            total += (int(doc_offsets[d + 1]) - start) if mask == "document" else (i - start + 1)
    return total


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _one_head(q, k, v, scale, mask, window, rows, q_pos_offset, doc_offsets):
    """O and LSE for one head: q [n_q, d], k [n_k, d], v [n_k, dv]."""
    n_q = q.shape[0]
    n_k = k.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.full(rows.size, -np.inf, dtype=np.float64)
    for b0 in range(0, rows.size, _ROW_BLOCK):
        r = rows[b0:b0 + _ROW_BLOCK]
        # S = Q K^T * scale, materialised for these rows.
        s = (q[r] @ k.T) * scale
        vis = visible(mask, r.size, n_k, window, q_pos=r + q_pos_offset, doc_offsets=doc_offsets)
        s = np.where(vis, s, -np.inf)
        # Pass 1: row maximum. Pass 2: exponentials, their sum, normalise.
        m = s.max(axis=1)
        live = np.isfinite(m)          # rows with at least one visible key
        m_safe = np.where(live, m, 0.0)
        e = np.exp(s - m_safe[:, None])
        l = e.sum(axis=1)
        p = np.divide(e, l[:, None], out=np.zeros_like(e), where=live[:, None])
        out[b0:b0 + r.size] = p @ v
        lse[b0:b0 + r.size] = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
    return out, lse


def attention(q, k, v, scale, mask="none", window=None, rows=None, q_pos_offset=0, doc_offsets=None):
    """softmax(Q K^T * scale, masked) V in float64.

    q: [..., n_q, d]; k: [..., n_k, d]; v: [..., n_k, dv] (same leading dims).
    ``rows`` (optional) selects the query rows to compute; the result then has
    len(rows) rows. ``q_pos_offset`` shifts the absolute query positions (a
    decode query at position L-1 uses n_q=1 and offset L-1). ``doc_offsets``
    (document masks) applies to every head.
    A row with no visible key gets O = 0 and LSE = -inf.
    Returns (O [..., rows, dv], LSE [..., rows]) with LSE = log sum_j exp(S_ij).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    lead = q.shape[:-2]
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    n_rows = q.shape[-2] if rows is None else len(rows)
    o = np.zeros((qf.shape[0], n_rows, vf.shape[-1]))
    lse = np.zeros((qf.shape[0], n_rows))
    for h in range(qf.shape[0]):
        o[h], lse[h] = _one_head(qf[h], kf[h], vf[h], float(scale), mask, window, rows, q_pos_offset,
                                 doc_offsets)
    return o.reshape(lead + o.shape[1:]), lse.reshape(lead + lse.shape[1:])


def probabilities(q, k, scale, mask="none", window=None, doc_offsets=None):
    """The full softmax matrix P [n_q, n_k] of one head (small inputs only)."""
    q = _as_f64(q)
    k = _as_f64(k)
    s = (q @ k.T) * scale
    vis = visible(mask, q.shape[0], k.shape[0], window, doc_offsets=doc_offsets)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)
