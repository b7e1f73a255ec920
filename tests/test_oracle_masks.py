"""Pins for the oracle's structured masks: document (block-diagonal, Pattern A
of "Optimizing Triton kernels for custom attention patterns on H100"), its
causal variant for packed variable-length sequences, the two-sided window and
the prefix-LM mask (end of Pattern B).

Each mask matrix is checked against a construction that does not use the
oracle's formula (blocks placed one document at a time, numpy's band
constructors, unions of already-pinned masks); attention under a document mask
is checked against running the already-pinned plain attention on each document
separately; pair counts against closed forms."""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _partition(n, rng, empty=True):
    """Random document offsets [0, ..., n] (possibly with empty documents)."""
    k = int(rng.integers(0, max(1, n // 2) + 1))
    cuts = sorted(rng.integers(0 if empty else 1, n + (1 if empty else 0), size=k).tolist())
    if not empty:
        cuts = sorted(set(c for c in cuts if 0 < c < n))
    return np.array([0] + cuts + [n], dtype=np.int64)


def _blocks(offs, n, causal):
    """The document mask built one diagonal block at a time."""
    m = np.zeros((n, n), dtype=bool)
    for s, e in zip(offs[:-1], offs[1:]):
        blk = np.ones((e - s, e - s), dtype=bool)
        m[s:e, s:e] = np.tril(blk) if causal else blk
    return m


DOC_CASES = [
    np.array([0, 29]),
    np.array([0, 1, 2, 3, 29]),
    np.array([0, 7, 7, 20, 29]),      # an empty document
    np.array([0, 0, 14, 29, 29]),     # empty first and last documents
    np.array(list(range(30))[:-1] + [29]),  # every position its own document
]


# ----------------------------------------------------------------- mask matrices

def test_document_masks_are_the_diagonal_blocks():
    rng = np.random.default_rng(11)
    for n in range(1, 41):
        for _ in range(6):
            offs = _partition(n, rng)
            for causal, name in ((False, "document"), (True, "document_causal")):
                got = oracle.visible(name, n, n, doc_offsets=offs)
                assert np.array_equal(got, _blocks(offs, n, causal)), (n, offs, name)


def test_document_mask_special_cases():
    for n in (1, 5, 17):
        one = np.array([0, n])
        assert np.array_equal(oracle.visible("document", n, n, doc_offsets=one), oracle.visible("none", n, n))
        assert np.array_equal(oracle.visible("document_causal", n, n, doc_offsets=one),
                              oracle.visible("causal", n, n))
        singles = np.arange(n + 1)
        assert np.array_equal(oracle.visible("document", n, n, doc_offsets=singles), np.eye(n, dtype=bool))
    with pytest.raises(ValueError):
        oracle.visible("document", 4, 4, doc_offsets=np.array([0, 3]))       # does not end at n
    with pytest.raises(ValueError):
        oracle.visible("document", 4, 4, doc_offsets=np.array([0, 3, 2, 4]))  # decreasing


def test_band_mask_is_numpy_band_and_union_of_one_sided_windows():
    for n in range(1, 30):
        ones = np.ones((n, n), dtype=bool)
        for w in range(0, n + 2):
            got = oracle.visible("band", n, n, w)
            assert np.array_equal(got, np.triu(np.tril(ones, w), -w))
            one_sided = oracle.visible("sliding", n, n, w + 1)
            assert np.array_equal(got, one_sided | one_sided.T)
        assert np.array_equal(oracle.visible("band", n, n, n), ones)


def test_prefix_lm_mask_is_prefix_block_plus_causal():
    for n in range(1, 30):
        causal = oracle.visible("causal", n, n)
        assert np.array_equal(oracle.visible("prefix_lm", n, n, 0), causal)
        assert np.array_equal(oracle.visible("prefix_lm", n, n, 1), causal)
        assert np.array_equal(oracle.visible("prefix_lm", n, n, n), np.ones((n, n), dtype=bool))
        for p in range(0, n + 3):
            want = causal.copy()
            want[:, :min(p, n)] = True
            assert np.array_equal(oracle.visible("prefix_lm", n, n, p), want)


def test_structured_pair_counts_match_closed_forms():
    rng = np.random.default_rng(12)
    for n in (1, 2, 7, 64, 300):
        for w in (0, 1, 3, n // 2, n, n + 4):
            # |i-j| <= w: n rows of 2w+1 keys minus the two clipped corners
            ww = min(w, n - 1)
            closed = (2 * ww + 1) * n - ww * (ww + 1)
            assert oracle.visible_pair_count("band", n, w) == closed
            assert int(oracle.visible("band", n, n, w).sum()) == closed
            p = min(w, n)
            closed = p * p + (n * (n + 1) - p * (p + 1)) // 2
            assert oracle.visible_pair_count("prefix_lm", n, w) == closed
            assert int(oracle.visible("prefix_lm", n, n, w).sum()) == closed
        for _ in range(4):
            offs = _partition(n, rng)
            lens = np.diff(offs)
            assert oracle.visible_pair_count("document", n, doc_offsets=offs) == int((lens * lens).sum())
            assert oracle.visible_pair_count("document_causal", n, doc_offsets=offs) == \
                int((lens * (lens + 1) // 2).sum())
            assert int(oracle.visible("document", n, n, doc_offsets=offs).sum()) == int((lens * lens).sum())


# ----------------------------------------------------------------- attention under the masks

@pytest.mark.parametrize("offs", DOC_CASES, ids=lambda o: "-".join(map(str, o[:5])))
def test_document_attention_is_per_document_attention(offs):
    """A packed batch of documents equals each document attended on its own."""
    n, d = 29, 6
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((2, n, d)) * 2 for _ in range(3))
    for name, inner in (("document", "none"), ("document_causal", "causal")):
        o, lse = oracle.attention(q, k, v, 0.7, name, doc_offsets=offs)
        for s, e in zip(offs[:-1], offs[1:]):
            if e == s:
                continue
            o_ref, lse_ref = oracle.attention(q[:, s:e], k[:, s:e], v[:, s:e], 0.7, inner)
            assert np.max(np.abs(o[:, s:e] - o_ref)) <= 1e-12
            assert np.max(np.abs(lse[:, s:e] - lse_ref)) <= 1e-12


def test_equal_scores_give_the_document_mean():
    n, d = 23, 4
    rng = np.random.default_rng(14)
    q = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    k = np.zeros((n, d))
    offs = np.array([0, 5, 6, 6, 17, 23])
    o, _ = oracle.attention(q, k, v, 0.5, "document", doc_offsets=offs)
    oc, _ = oracle.attention(q, k, v, 0.5, "document_causal", doc_offsets=offs)
    for s, e in zip(offs[:-1], offs[1:]):
        for i in range(s, e):
            assert np.max(np.abs(o[i] - v[s:e].mean(axis=0))) <= 1e-13
            assert np.max(np.abs(oc[i] - v[s:i + 1].mean(axis=0))) <= 1e-13
    w = 3
    ob, _ = oracle.attention(q, k, v, 0.5, "band", w)
    op, _ = oracle.attention(q, k, v, 0.5, "prefix_lm", 6)
    for i in range(n):
        assert np.max(np.abs(ob[i] - v[max(0, i - w):i + w + 1].mean(axis=0))) <= 1e-13
        assert np.max(np.abs(op[i] - v[:max(i + 1, 6)].mean(axis=0))) <= 1e-13


STRUCT_CASES = [("band", 0, None), ("band", 2, None), ("band", 9, None), ("prefix_lm", 0, None),
                ("prefix_lm", 5, None), ("prefix_lm", 30, None), ("document", None, DOC_CASES[2]),
                ("document", None, DOC_CASES[4]), ("document_causal", None, DOC_CASES[3])]


@pytest.mark.parametrize("mask,window,offs", STRUCT_CASES)
def test_structured_masks_match_torch_sdpa_and_logsumexp(mask, window, offs):
    n, d = 29, 5
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, 0.9, mask, window, doc_offsets=offs)
    if mask == "band":
        vis = np.triu(np.tril(np.ones((n, n), dtype=bool), window), -window)
    elif mask == "prefix_lm":
        vis = np.tril(np.ones((n, n), dtype=bool))
        vis[:, :window] = True
    else:
        vis = _blocks(offs, n, mask == "document_causal")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(vis), scale=0.9)
    assert np.max(np.abs(o - ref.numpy())) <= 1e-12
    s = (q @ k.T) * 0.9
    s[~vis] = -np.inf
    assert np.max(np.abs(lse - logsumexp(s, axis=1))) <= 1e-12


@pytest.mark.parametrize("mask,window,offs", STRUCT_CASES)
def test_recurrence_with_structured_masks(mask, window, offs):
    """Tiles that are empty, full or cut by a document edge all reduce to the two-pass result."""
    n, d = 29, 3
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    ref = oracle.attention(q, k, v, 0.8, mask, window, doc_offsets=offs)[0]
    for bn in (1, 3, 4, 8, 29, 30):
        for bm in (1, 5, 16, 29):
            got = oracle.tiled_attention(q, k, v, 0.8, mask, window, bm=bm, bn=bn, doc_offsets=offs)
            assert np.max(np.abs(got - ref)) <= 1e-12, (bm, bn)
    for bounds in [(), (7, 14, 21), tuple(range(1, n))]:
        got = oracle.split_attention(q, k, v, 0.8, mask, window, bounds=bounds, bn=4, doc_offsets=offs)
        assert np.max(np.abs(got - ref)) <= 1e-12
