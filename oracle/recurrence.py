"""fp64 online-softmax recurrence over tiles, and the merge of partial results.

Test infrastructure (see the package docstring).

Follows "Flash MSA Attention Kernel Implementation Tutorial":
* "Understanding Flash MSA Core Mechanics": split the sequence into tiles;
  for each Q tile walk the K/V tiles, keep a running row maximum m and a
  running row sum of exponentials l; when a tile arrives take
  m_new = max(m, tile row max), rescale what was accumulated by exp(m - m_new)
  and add the new exponentials exp(s - m_new); divide by l at the end.
* The kernel listing in "Implementation Step-by-Step with Triton" keeps m, l
  and the accumulator in fp32 with m starting at -inf and l, acc at 0; this
  model runs the same steps in fp64 with tile sizes chosen freely.
* The remark after that listing: without the exp(m - m_new) rescale the
  result is wrong once N exceeds the tile size.

Readings taken where the page is silent or its code is loose:
* The listing zero-loads keys past N but leaves their scores unmasked; here
  keys outside [0, N) simply do not exist (the last tile is ragged), which is
  the same as giving their scores -inf.
* Masked scores are -inf. While a row has seen no visible key yet, its m is
  -inf; exp(-inf - (-inf)) is undefined, so the reference point used for the
  exponentials is 0 in that case (every exponential is then exp(-inf) = 0 and
  the rescale of the zero accumulator is irrelevant).
* Splitting the keys into independent ranges and merging their (m, l, acc)
  states uses the same rescale algebra: m* = max m_i,
  l* = sum exp(m_i - m*) l_i, acc* = sum exp(m_i - m*) acc_i.
"""

import numpy as np

from .attention import visible


def _rescale_factor(m_old, m_ref):
    """exp(m_old - m_ref): how much the accumulated sums shrink when the
    reference maximum moves from m_old to m_ref."""
    return np.exp(m_old - m_ref)


def partial_state(q, k, v, scale, mask="none", window=None, bn=None, key_lo=0, key_hi=None,
                  q_pos=None, doc_offsets=None):
    """Run the recurrence for one head over keys [key_lo, key_hi) in tiles of bn.

    q: [n_q, d] with absolute query positions ``q_pos`` (default 0..n_q-1);
    k, v: [n_k, d] / [n_k, dv] (full key range; only [key_lo, key_hi) is read).
    Returns the un-normalised state (m, l, acc): m [n_q], l [n_q], acc [n_q, dv].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q = q.shape[0]
    n_k = k.shape[0]
    key_hi = n_k if key_hi is None else key_hi
    bn = max(1, key_hi - key_lo) if bn is None else bn
    q_pos = np.arange(n_q) if q_pos is None else np.asarray(q_pos)
    vis_all = visible(mask, n_q, n_k, window, q_pos=q_pos, doc_offsets=doc_offsets)
    m = np.full(n_q, -np.inf)
    l = np.zeros(n_q)
    acc = np.zeros((n_q, v.shape[1]))
    for n0 in range(key_lo, key_hi, bn):
        n1 = min(n0 + bn, key_hi)
        s = (q @ k[n0:n1].T) * scale
        s = np.where(vis_all[:, n0:n1], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = _rescale_factor(m, m_ref)
        p = np.exp(s - m_ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[n0:n1]
        m = m_new
    return m, l, acc


def _finish(l, acc):
    """acc / l, with rows that saw no visible key set to 0."""
    live = l > 0
    return np.divide(acc, l[:, None], out=np.zeros_like(acc), where=live[:, None])


def tiled_attention(q, k, v, scale, mask="none", window=None, bm=None, bn=None, doc_offsets=None):
    """Flash-style forward for one head: Q tiles of bm rows, K/V tiles of bn keys.

    Every K tile is visited (masked ones contribute nothing). Returns O [n_q, dv].
    """
    q = np.asarray(q, dtype=np.float64)
    n_q = q.shape[0]
    bm = n_q if bm is None else bm
    out = np.zeros((n_q, np.asarray(v).shape[1]))
    for m0 in range(0, n_q, bm):
        m1 = min(m0 + bm, n_q)
        _, l, acc = partial_state(q[m0:m1], k, v, scale, mask, window, bn,
                                  q_pos=np.arange(m0, m1), doc_offsets=doc_offsets)
        out[m0:m1] = _finish(l, acc)
    return out


def merge_partials(states):
    """Combine (m, l, acc) states computed over disjoint key ranges."""
    ms = np.stack([s[0] for s in states])
    m_star = ms.max(axis=0)
    m_ref = np.where(np.isfinite(m_star), m_star, 0.0)
    l_star = np.zeros_like(m_star)
    acc_star = np.zeros_like(states[0][2])
    for m_i, l_i, acc_i in states:
        w = _rescale_factor(m_i, m_ref)
        l_star = l_star + w * l_i
        acc_star = acc_star + w[:, None] * acc_i
    return m_star, l_star, acc_star


def split_attention(q, k, v, scale, mask="none", window=None, bounds=(), bn=None, q_pos=None,
                    doc_offsets=None):
    """Attention of one head computed as independent key ranges, then merged.

    ``bounds`` are interior split points of [0, n_k) (any order, duplicates
    allowed: empty ranges are skipped). Returns O [n_q, dv].
    """
    n_k = np.asarray(k).shape[0]
    cuts = sorted(set([0, n_k] + [int(b) for b in bounds if 0 < b < n_k]))
    states = [partial_state(q, k, v, scale, mask, window, bn, a, b, q_pos=q_pos, doc_offsets=doc_offsets)
              for a, b in zip(cuts[:-1], cuts[1:])]
    _, l, acc = merge_partials(states)
    return _finish(l, acc)
