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


def _expected_ranks(costs):
    """Heaviest first, ties by index: the rank of g is the number of groups
    with a larger cost, or an equal cost and a lower index."""
    order = sorted(range(len(costs)), key=lambda g: (-costs[g], g))
    ranks = [0] * len(costs)
    for r, g in enumerate(order):
        ranks[g] = r
    return ranks


def test_dispatch_ranks_are_the_heaviest_first_permutation_for_every_group_count():
    """The device ranking's code (shared with this host copy) reads only the
    keys it wrote, padded to whole rounds of sixteen, and its ranks are a
    permutation for every group count 1..256: a bound that counted keys past
    the written ones once left order slots unset on the GPU."""
    rng = np.random.default_rng(7)
    for g in range(1, 257):
        for costs in (rng.integers(0, 64, size=g), rng.integers(0, 1 << 23, size=g), np.zeros(g, dtype=int),
                      np.full(g, (1 << 23) - 1)):
            costs = [int(c) for c in costs]
            ranks = _lib.attn_dispatch_ranks(costs)
            assert sorted(ranks) == list(range(g)), g
            assert ranks == _expected_ranks(costs), g


def test_dispatch_ranks_reject_bad_arguments():
    lib = _lib.load()
    arr = (ctypes.c_int32 * 300)()
    out = (ctypes.c_int32 * 300)()
    assert lib.attn_dispatch_ranks(arr, 0, out) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_dispatch_ranks(arr, 257, out) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_dispatch_ranks(None, 4, out) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_dispatch_ranks(arr, 4, None) == _lib.ATTN_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        _lib.attn_dispatch_ranks([1, -1])
    with pytest.raises(ValueError):
        _lib.attn_dispatch_ranks([1 << 23])


# ------------------------------------------------ binding argument validation

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _binding_cases():
    """(name, call, bad argument) triples: each call has exactly one tensor of
    the wrong shape or dtype, which the binding must refuse before the library
    sees it (no kernel is launched: these are host tensors)."""
    import torch
    f32, bf16, u8, i32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32
    B, H, N, d = 1, 2, 130, 64
    q = _t((B, H, N, d), bf16)
    cases = []

    def fwd(**kw):
        a = dict(q=q, k=q, v=q, o=_t((B, H, N, d), f32), lse=None)
        a.update(kw)
        return lambda: _lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], 0.1, "causal", lse=a["lse"])
    cases += [("attn_fwd ok", fwd(), None),
              ("lse shape", fwd(lse=_t((B, H), f32)), "lse"),
              ("lse dtype", fwd(lse=_t((B, H, N), bf16)), "lse"),
              ("k shape", fwd(k=_t((B, H, N + 1, d), bf16)), "k"),
              ("v dtype", fwd(v=_t((B, H, N, d), f32)), "v"),
              ("o shape", fwd(o=_t((B, H, N, 2 * d), f32)), "o")]
    cases.append(("doc offsets dtype",
                  lambda: _lib.attn_fwd(q, q, q, q, 0.1, "document", doc_offsets=_t((3,), torch.int64)),
                  "doc_offsets"))

    nb = 2
    def fp8(**kw):
        a = dict(q8=_t((B, H, N, d), u8), sq=_t((B, H, nb), f32), k8=_t((B, H, N, d), u8), sk=_t((B, H, nb), f32),
                 v=q, o=_t((B, H, N, d), bf16), lse=None, v8=None, sv=None)
        a.update(kw)
        if a["v8"] is not None:
            return lambda: _lib.attn_fwd_fp8_full(a["q8"], a["sq"], a["k8"], a["sk"], a["v8"], a["sv"], a["o"], 0.1,
                                                  "causal", lse=a["lse"])
        return lambda: _lib.attn_fwd_fp8(a["q8"], a["sq"], a["k8"], a["sk"], a["v"], a["o"], 0.1, "causal",
                                         lse=a["lse"])
    cases += [("fp8 ok", fp8(), None),
              ("q_scale shape", fp8(sq=_t((B, H, nb + 1), f32)), "q_scale"),
              ("k_scale dtype", fp8(sk=_t((B, H, nb), bf16)), "k_scale"),
              ("k8 dtype", fp8(k8=_t((B, H, N, d), bf16)), "k8"),
              ("fp8 lse", fp8(lse=_t((B, H, N, 1), f32)), "lse"),
              ("fp8 full ok", fp8(v8=_t((B, H, N, d), u8), sv=_t((B, H, nb), f32)), None),
              ("v_scale shape", fp8(v8=_t((B, H, N, d), u8), sv=_t((B, H), f32)), "v_scale"),
              ("v8 dtype", fp8(v8=_t((B, H, N, d), bf16), sv=_t((B, H, nb), f32)), "v8")]

    x = _t((B, H, N, d), f32)
    cases += [("quant ok", lambda: _lib.attn_quant_fp8_block(x, _t((B, H, N, d), u8), _t((B, H, nb), f32)), None),
              ("quant codes", lambda: _lib.attn_quant_fp8_block(x, _t((B, H, N, d), f32), _t((B, H, nb), f32)),
               "codes"),
              ("quant scales", lambda: _lib.attn_quant_fp8_block_pow2(x, _t((B, H, N, d), u8), _t((B, H, 1), f32)),
               "scales")]

    S, P, pg, mp = 3, 10, 16, 4
    pool = _t((P, H, pg, d), bf16)
    def dec(**kw):
        a = dict(q=_t((S, H, d), bf16), kp=pool, vp=pool, bt=_t((S, mp), i32), lens=_t((S,), i32),
                 o=_t((S, H, d), bf16), lse=None)
        a.update(kw)
        return lambda: _lib.attn_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["lens"], a["o"], 0.1,
                                              lse=a["lse"])
    cases += [("decode ok", dec(), None),
              ("decode lse", dec(lse=_t((S,), f32)), "lse"),
              ("decode table dtype", dec(bt=_t((S, mp), torch.int64)), "block_table"),
              ("decode table rows", dec(bt=_t((S + 1, mp), i32)), "block_table"),
              ("decode lens", dec(lens=_t((S, 1), i32)), "seq_lens"),
              ("decode pool heads", dec(kp=_t((P, H + 1, pg, d), bf16)), "k_pool"),
              ("decode v pool", dec(vp=_t((P, H, pg, d), f32)), "v_pool")]

    ql = 200
    qb = 2
    def pre(cross=False, **kw):
        a = dict(q=_t((S, H, ql, d), bf16), kp=pool, vp=pool,
                 t=_t((S, qb, mp) if cross else (S, mp), i32), l=_t((S, qb) if cross else (S,), i32),
                 o=_t((S, H, ql, d), bf16), lse=None)
        a.update(kw)
        fn = _lib.attn_cross_paged if cross else _lib.attn_prefill_paged
        return lambda: fn(a["q"], a["kp"], a["vp"], a["t"], a["l"], a["o"], 0.1, lse=a["lse"])
    cases += [("prefill ok", pre(), None),
              ("prefill lse", pre(lse=_t((S, H), f32)), "lse"),
              ("prefill table", pre(t=_t((S, qb, mp), i32)), "block_table"),
              ("cross ok", pre(cross=True), None),
              ("cross decode-style table", pre(cross=True, t=_t((S, mp), i32)), "page_table"),
              ("cross lens", pre(cross=True, l=_t((S,), i32)), "kv_lens"),
              ("cross o dtype", pre(cross=True, o=_t((S, H, ql, d), u8)), "o")]

    def gat(**kw):
        a = dict(kp=pool, vp=pool, bt=_t((S, mp), i32), lens=_t((S,), i32), ko=_t((S, H, mp * pg, d), bf16),
                 vo=_t((S, H, mp * pg, d), bf16))
        a.update(kw)
        return lambda: _lib.attn_gather_paged(a["kp"], a["vp"], a["bt"], a["lens"], a["ko"], a["vo"])
    cases += [("gather ok", gat(), None),
              ("gather out rows", gat(ko=_t((S, H, mp * pg - 1, d), bf16)), "k_out"),
              ("gather out dtype", gat(vo=_t((S, H, mp * pg, d), f32)), "v_out")]
    return cases


@pytest.mark.parametrize("case", _binding_cases(), ids=lambda c: c[0])
def test_binding_checks_every_tensor_argument(case):
    name, call, bad = case
    if bad is None:
        # every shape and dtype is right: only the device check remains
        with pytest.raises(ValueError, match="GPU tensors"):
            call()
    else:
        with pytest.raises(ValueError, match=rf"^{bad} must"):
            call()


def test_noalloc_decode_rejects_work_beyond_its_array():
    """attn_decode_paged_noalloc holds its partial states in a fixed 16 MiB
    device array: a size whose workspace would exceed it is refused before
    anything runs (FAKE pointers: nothing is dereferenced)."""
    lib = _lib.load()
    big = lib.attn_decode_paged_workspace_size(256, 32, 128, 2048, 16)
    assert big > (16 << 20)
    st = lib.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 32, 128, 16, 2048, 10000, 0.1,
                                       None, None)
    assert st == _lib.ATTN_ERR_WORKSPACE
    assert lib.attn_decode_paged_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, 16, 8, 100, 0.1, None,
                                         None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, 32, 8, 100, 0.1, None,
                                         None) == _lib.ATTN_ERR_UNSUPPORTED
    # the benchmark's decode fits
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 512, 16) <= (16 << 20)


def test_split_workspace_size_and_rejects():
    """attn_fwd_split_workspace_size: B*H * split tiles * 2 * 128 * (d + 1) * 4
    bytes when the plan splits (causal N = 8192, 4 heads: the 32 costliest of 64
    tiles), 0 otherwise; attn_fwd_split refuses a missing or short workspace
    before anything runs (FAKE pointers: nothing is dereferenced)."""
    lib = _lib.load()
    causal, prefix, none = _lib.MASKS["causal"], _lib.MASKS["prefix_lm"], _lib.MASKS["none"]
    bf16, f32 = _lib.ATTN_BF16, _lib.ATTN_F32
    assert lib.attn_fwd_split_workspace_size(1, 4, 8192, 64, bf16, causal, 0) == 4 * 32 * 2 * 128 * 65 * 4
    assert lib.attn_fwd_split_workspace_size(1, 16, 4096, 128, bf16, causal, 0) == 16 * 16 * 2 * 128 * 129 * 4
    # 2500 rows in 20 tiles of 2, 4, .., 40 key tiles (the last ragged): the 10 costliest split
    assert lib.attn_fwd_split_workspace_size(1, 4, 2500, 64, bf16, causal, 0) == 4 * 10 * 2 * 128 * 65 * 4
    assert lib.attn_fwd_split_workspace_size(1, 8, 2048, 128, bf16, prefix, 512) > 0
    for args in [(4, 16, 2048, 64, bf16, causal, 0),      # two tiles per slot: not split
                 (1, 16, 4096, 64, bf16, causal, 0),      # one tile per slot, loops too short to pay
                 (1, 2, 300, 64, bf16, causal, 0),        # tiles too cheap
                 (1, 4, 8192, 64, f32, causal, 0),        # fp32 path
                 (1, 4, 8192, 64, bf16, none, 0),         # equal-cost tiles
                 (1, 1, 64, 64, bf16, causal, 0),         # one tile of one key tile
                 (1, 1, 4096, 96, bf16, causal, 0)]:      # unsupported d
        assert lib.attn_fwd_split_workspace_size(*args) == 0, args
    need = lib.attn_fwd_split_workspace_size(1, 4, 8192, 64, bf16, causal, 0)
    base = (FAKE, FAKE, FAKE, FAKE, 1, 4, 8192, 64, bf16, bf16, 0.125, causal, 0, None, 0, None)
    assert lib.attn_fwd_split(*base, None, 0, None) == _lib.ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_split(*base, FAKE, need - 1, None) == _lib.ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_split(*base, FAKE_MIS, need, None) == _lib.ATTN_ERR_INVALID_ARG
    bad = (FAKE, FAKE, FAKE, FAKE, 1, 4, 8192, 64, bf16, bf16, 0.0, causal, 0, None, 0, None)
    assert lib.attn_fwd_split(*bad, FAKE, need, None) == _lib.ATTN_ERR_INVALID_ARG
