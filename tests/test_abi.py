"""The C-ABI library loads and exports what include/attn.h declares; argument
checks return the documented status without touching the device; the host
tile planner agrees with the oracle's mask. No kernel is launched here."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from tiled_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x10000            # 16-byte aligned dummy address; never dereferenced (calls fail validation)
FAKE_MIS = 0x10004        # misaligned dummy


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared) <= exported
    assert set(_lib.symbols()) == set(declared)
    assert _lib.attn_abi_version() == 2


def test_status_strings():
    for code in range(5):
        s = _lib.attn_status_str(code)
        assert s.startswith("ATTN_")
    assert "unknown" in _lib.attn_status_str(99)


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=1, N=8, d=64, ind=1, outd=1, scale=0.125,
                mask=0, window=0, doc=None, nd=0, lse=None, stream=None)
    args.update(kw)
    return _lib.load().attn_fwd(args["q"], args["k"], args["v"], args["o"], args["B"], args["H"], args["N"],
                                args["d"], args["ind"], args["outd"], args["scale"], args["mask"],
                                args["window"], args["doc"], args["nd"], args["lse"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(o=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(k=FAKE_MIS), _lib.ATTN_ERR_INVALID_ARG),
    (dict(N=0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(d=0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(ind=2), _lib.ATTN_ERR_INVALID_ARG),
    (dict(outd=7), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=7), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=2, window=0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=3, window=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=4, window=-2), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=5, doc=None, nd=2), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=6, doc=FAKE, nd=0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(mask=5, doc=FAKE + 2, nd=1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(scale=-0.125), _lib.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.ATTN_ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 16, N=1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), _lib.ATTN_ERR_INVALID_ARG),
])
def test_attn_fwd_rejects(kw, status):
    assert _fwd(**kw) == status


def test_attn_fwd_fp8_rejects():
    f = _lib.load().attn_fwd_fp8
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 128, 128, 0.1, 1, 0, None, 0, None, None]
    bad = list(ok); bad[1] = None
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[10] = 64
    assert f(*bad) == _lib.ATTN_ERR_UNSUPPORTED
    bad = list(ok); bad[9] = 96
    assert f(*bad) == _lib.ATTN_ERR_UNSUPPORTED
    bad = list(ok); bad[12] = 2; bad[13] = 0
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[2] = FAKE_MIS
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[12] = 5
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    for scale in (0.0, -0.1, float("inf"), float("nan")):
        bad = list(ok); bad[11] = scale
        assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG


def test_quant_rejects():
    f = _lib.load().attn_quant_fp8_block
    assert f(None, FAKE, FAKE, 1, 1, 128, 128, 128, None) == _lib.ATTN_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 1, 1, 128, 128, 64, None) == _lib.ATTN_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 1, 1, 0, 128, 128, None) == _lib.ATTN_ERR_INVALID_ARG


def test_paged_rejects_and_workspace_size():
    lib = _lib.load()
    ws = lib.attn_decode_paged_workspace_size(64, 32, 128, 512, 16)
    assert ws == 64 * 32 * 8 * (128 + 2) * 4             # 8 ranges of 64 pages per sequence
    # 64-token pages: four 16-token units each, so four times the ranges per table row
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 128, 64) == ws
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 512, 32) == 0
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 16, 8, 20, 0.1, None, FAKE, 10 ** 9, None]
    assert lib.attn_decode_paged(*[None] + ok[1:]) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[9] = 32
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_UNSUPPORTED
    bad = list(ok); bad[9] = 64; bad[15] = lib.attn_decode_paged_workspace_size(2, 4, 128, 8, 64) - 1
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_WORKSPACE
    bad = list(ok); bad[15] = 16
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_WORKSPACE
    bad = list(ok); bad[14] = FAKE_MIS
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[8] = 80
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_UNSUPPORTED
    bad = list(ok); bad[11] = 0
    assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_INVALID_ARG
    for scale in (0.0, -0.1, float("inf")):
        bad = list(ok); bad[12] = scale
        assert lib.attn_decode_paged(*bad) == _lib.ATTN_ERR_INVALID_ARG
    g = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 16, 8, 20, _lib.ATTN_BF16, None]
    bad = list(g); bad[12] = _lib.ATTN_FP8_E4M3
    assert lib.attn_gather_paged(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(g); bad[4] = None
    assert lib.attn_gather_paged(*bad) == _lib.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["attn_prefill_paged", "attn_cross_paged"])
def test_paged_prefill_rejects(name):
    f = getattr(_lib.load(), name)
    # q, k_pool, v_pool, table, lens, o, S, H, q_len, d, page, max_pages, num_pages, out, scale, lse, stream
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 300, 128, 64, 8, 20, _lib.ATTN_BF16, 0.1, None, None]
    for i in (0, 1, 2, 3, 4, 5):
        bad = list(ok); bad[i] = None
        assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    for page in (8, 32, 128):
        bad = list(ok); bad[10] = page
        assert f(*bad) == _lib.ATTN_ERR_UNSUPPORTED      # pages of 16 or 64 tokens only
    bad = list(ok); bad[10] = 0
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[11] = 4097
    assert f(*bad) == _lib.ATTN_ERR_UNSUPPORTED          # list longer than the on-chip staging
    bad = list(ok); bad[9] = 96
    assert f(*bad) == _lib.ATTN_ERR_UNSUPPORTED
    bad = list(ok); bad[8] = 0
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[13] = _lib.ATTN_FP8_E4M3
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[3] = FAKE + 2
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    bad = list(ok); bad[1] = FAKE_MIS
    assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG
    for scale in (float("nan"), 0.0, -0.1, float("inf")):
        bad = list(ok); bad[14] = scale
        assert f(*bad) == _lib.ATTN_ERR_INVALID_ARG


def _expected_class(vis, N, m0, m1, n0, n1):
    """EMPTY / PARTIAL / FULL of a tile from the oracle's visibility matrix."""
    rows = [i for i in range(m0, min(m1, N))]
    keys = [j for j in range(n0, min(n1, N))]
    if not rows or not keys:
        return 0
    block = vis[np.ix_(rows, keys)]
    if not block.any():
        return 0
    if block.all() and n1 <= N:
        return 2
    return 1


def _doc_sets(N):
    """Document offsets exercised at length N: one document, single positions,
    seeded random cuts with and without empty documents."""
    rng = np.random.default_rng(N)
    sets = [[0, N], list(range(N + 1))]
    for k in (1, 3, max(1, N // 7)):
        cuts = sorted(rng.integers(0, N + 1, size=k).tolist())
        sets.append([0] + cuts + [N])
        sets.append(sorted(set([0] + cuts + [N])))
    return sets


MASK_PLANS = [("none", 0), ("causal", 0), ("sliding", 1), ("sliding", 3), ("sliding", 16), ("sliding", 40),
              ("band", 0), ("band", 2), ("band", 13), ("band", 70), ("prefix_lm", 0), ("prefix_lm", 7),
              ("prefix_lm", 33), ("prefix_lm", 200), ("document", 0), ("document_causal", 0)]


def _plans(mask, window, N):
    """(oracle visibility, host offsets or None) for every offsets set of the mask."""
    if mask in _lib.DOC_MASKS:
        return [(oracle.visible(mask, N, N, doc_offsets=np.array(o)), o) for o in _doc_sets(N)]
    return [(oracle.visible(mask, N, N, None if mask in ("none", "causal") else window), None)]


@pytest.mark.parametrize("mask,window", MASK_PLANS)
def test_tile_class_and_range_match_oracle_mask(mask, window):
    for N in (1, 5, 17, 40, 64):
        for vis, offs in _plans(mask, window, N):
            for bm in (1, 3, 8, 32):
                for bn in (1, 4, 16, 64):
                    for m0 in range(0, N, bm):
                        m1 = m0 + bm
                        lo, hi = _lib.attn_k_tile_range(mask, window, N, m0, m1, bn, offs)
                        nt = -(-N // bn)
                        assert 0 <= lo <= hi <= nt
                        for t in range(nt):
                            n0, n1 = t * bn, t * bn + bn
                            want = _expected_class(vis, N, m0, m1, n0, n1)
                            got = _lib.attn_tile_class(mask, window, N, m0, m1, n0, n1, offs)
                            assert got == want, (N, offs, bm, bn, m0, t)
                            # outside the range every tile is EMPTY, inside none is
                            assert (want != 0) == (lo <= t < hi), (N, offs, bm, bn, m0, t)


@pytest.mark.parametrize("mask,window", MASK_PLANS)
def test_full_tile_range_is_exactly_the_full_tiles(mask, window):
    """The kernels' FULL range equals the set of tiles whose every pair is visible."""
    for N in (1, 5, 17, 40, 64, 100):
        for vis, offs in _plans(mask, window, N):
            for bm in (1, 3, 8, 32):
                for bn in (1, 4, 16, 64):
                    for m0 in range(0, N, bm):
                        lo, hi = _lib.attn_full_tile_range(mask, window, N, m0, m0 + bm, bn, offs)
                        assert 0 <= lo <= hi
                        for t in range(-(-N // bn)):
                            full = _expected_class(vis, N, m0, m0 + bm, t * bn, t * bn + bn) == 2
                            assert full == (lo <= t < hi), (N, offs, bm, bn, m0, t, lo, hi)


def test_planner_rejects_bad_host_offsets():
    for offs in ([1, 8], [0, 7], [0, 5, 3, 8]):
        assert _lib.attn_tile_class("document", 0, 8, 0, 4, 0, 4, offs) == -1
        with pytest.raises(ValueError):
            _lib.attn_k_tile_range("document", 0, 8, 0, 4, 4, offs)
    with pytest.raises(ValueError):
        _lib.attn_full_tile_range("document_causal", 0, 8, 0, 4, 4, None)


def test_tile_counts_at_workload_sizes():
    """Tile pairs visited per head at BM=128, BN=64 (the MFMA kernel's tiles)."""
    def pairs(mask, window, N):
        total = 0
        for m0 in range(0, N, 128):
            lo, hi = _lib.attn_k_tile_range(mask, window, N, m0, m0 + 128, 64)
            total += sum(1 for t in range(lo, hi)
                         if _lib.attn_tile_class(mask, window, N, m0, m0 + 128, t * 64, t * 64 + 64) != 0)
        return total
    assert pairs("causal", 0, 2048) == 272
    assert pairs("sliding", 4096, 8192) == 3168
    assert pairs("causal", 0, 16384) == 16512
    assert pairs("none", 0, 256) == 8
