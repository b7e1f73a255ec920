"""Closed-form properties of the GPU path, checked without the oracle.

The oracle is pinned to these same properties; here they are asserted on the
kernels directly, as a second check that does not go through the oracle.
The attention the pages define ("Flash MSA Attention Kernel Implementation
Tutorial", "Understanding Flash MSA Core Mechanics": softmax of the scaled
scores times V, computed with an online softmax) implies:
- with every score equal (all keys zero, so every score is 0), softmax
  weights are uniform: a row's output is the mean of the V rows it sees and
  its LSE is the log of their count, for any Q and under every mask;
- a single dominant score returns that key's V row;
- under a causal mask the first row sees only key 0, so O[0] = V[0] exactly;
- weights sum to one, so a V whose rows are all one vector c gives O = c.
Expected values are written out here from V alone (prefix sums in float64).
"""

import math

import numpy as np
import pytest
import torch

from parity import half_ulp_bf16, say
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def visible(mask, N, window=0, offs=None):
    """Boolean [N, N] visibility of key j to query i, from the masks' definitions."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if mask == "none":
        return np.ones((N, N), dtype=bool)
    if mask == "causal":
        return j <= i
    if mask == "sliding":
        return (j <= i) & (j > i - window)
    if mask == "band":
        return np.abs(i - j) <= window
    if mask == "prefix_lm":
        return (j <= i) | (j < window)
    doc = np.searchsorted(offs, np.arange(N), side="right") - 1
    same = doc[:, None] == doc[None, :]
    return same & (j <= i) if mask == "document_causal" else same


def uniform_mean(v64, vis):
    """Mean of the visible V rows for every query row: [.., N, d]."""
    cnt = vis.sum(axis=1).astype(np.float64)
    return np.einsum("ij,...jd->...id", vis.astype(np.float64), v64) / cnt[:, None], cnt


def dense(B, H, N, d, seed, dtype):
    q, k, v = wl.dense_inputs(B, H, N, d, seed=seed)
    if dtype == "bf16":
        q, k, v = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    else:
        q, k, v = (torch.from_numpy(x) for x in (q, k, v))
    return q.cuda(), k.cuda(), v.cuda()


CASES = [
    # mask, window, N, d, dtype
    ("none", 0, 300, 64, "bf16"),
    ("causal", 0, 300, 64, "bf16"),
    ("causal", 0, 4100, 128, "bf16"),
    ("sliding", 100, 700, 128, "bf16"),
    ("band", 70, 520, 64, "bf16"),
    ("prefix_lm", 150, 450, 128, "bf16"),
    ("document", 0, 900, 128, "bf16"),
    ("document_causal", 0, 900, 64, "bf16"),
    ("causal", 0, 300, 64, "f32"),
    ("sliding", 33, 260, 128, "f32"),
    ("document", 0, 500, 64, "f32"),
]


@pytest.mark.parametrize("mask,window,N,d,dtype", CASES)
def test_equal_scores_give_mean_of_visible_values(mask, window, N, d, dtype):
    say(f"equal scores: {mask} w={window} N={N} d={d} {dtype}")
    B, H = 2, 2
    q, k, v = dense(B, H, N, d, seed=N + d, dtype=dtype)
    k = torch.zeros_like(k)
    offs = wl.document_offsets(N, 1, 200, seed=N) if mask.startswith("document") else None
    doc = None if offs is None else torch.from_numpy(offs).cuda()
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_fwd(q, k, v, o, 1.0 / math.sqrt(d), mask, window, doc_offsets=doc, lse=lse)
    torch.cuda.synchronize()
    vis = visible(mask, N, window, offs)
    ref, cnt = uniform_mean(v.double().cpu().numpy(), vis)
    err = np.abs(o.double().cpu().numpy() - ref).max()
    # every weight is exactly one; only the fp32 sums round
    assert err <= 1e-5, err
    assert np.abs(lse.double().cpu().numpy() - np.log(cnt)).max() <= 1e-5


@pytest.mark.parametrize("mask", ["causal", "none", "sliding"])
@pytest.mark.parametrize("d", [64, 128])
def test_dominant_score_returns_its_value_row(mask, d):
    say(f"dominant score: {mask} d={d}")
    B, H, N, window = 1, 2, 333, 90
    rng = np.random.default_rng(d)
    _, k, v = wl.dense_inputs(B, H, N, d, seed=5 * d)
    vis = visible(mask, N, window)
    # row i's target: a random visible key t(i); Q[i] = 16 K[t(i)] (exact in
    # bf16) puts that score tens of nats above every other one
    target = np.array([rng.choice(np.flatnonzero(vis[i])) for i in range(N)])
    kb = wl.to_bf16(k)
    q = 16.0 * kb.float()[:, :, target, :]
    qb, vb = q.to(torch.bfloat16), wl.to_bf16(v)
    k64, q64 = kb.double().numpy(), qb.double().numpy()
    s = np.einsum("bhid,bhjd->bhij", q64, k64)
    s[:, :, ~vis] = -np.inf
    gap = s[:, :, np.arange(N), target] - np.sort(s, axis=-1)[..., -2]
    assert gap.min() / math.sqrt(d) > 20.0  # the target dominates by > 20 nats
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    A.attn_fwd(qb.cuda(), kb.cuda(), vb.cuda(), o, 1.0 / math.sqrt(d), mask, window)
    torch.cuda.synchronize()
    ref = vb.double().numpy()[:, :, target, :]
    err = np.abs(o.double().cpu().numpy() - ref)
    assert np.all(err <= half_ulp_bf16(ref) + 1e-6), err.max()


@pytest.mark.parametrize("d", [64, 128])
def test_causal_first_rows_are_exact_value_rows(d):
    """Row 0 under CAUSAL, and each document's first row under
    DOCUMENT_CAUSAL, see one key: O is that V row, bit for bit."""
    B, H, N = 2, 3, 777
    q, k, v = dense(B, H, N, d, seed=9 + d, dtype="bf16")
    o = torch.empty_like(q)
    A.attn_fwd(q, k, v, o, 1.0 / math.sqrt(d), "causal")
    offs = wl.document_offsets(N, 1, 150, seed=d)
    o2 = torch.empty_like(q)
    A.attn_fwd(q, k, v, o2, 1.0 / math.sqrt(d), "document_causal", doc_offsets=torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))
    starts = torch.from_numpy(offs[:-1][np.diff(offs) > 0].astype(np.int64)).cuda()
    assert torch.equal(o2[:, :, starts].view(torch.int16), v[:, :, starts].view(torch.int16))


@pytest.mark.parametrize("mask", ["causal", "none", "document"])
def test_constant_value_rows_are_returned(mask):
    """V rows all equal to one vector c: the weights sum to one, so O = c. The
    MFMA kernels weight V by P rounded to bf16 but normalise by the sum of the
    unrounded P, so O = c only within 2^-8 relative; the fp32 kernel to fp32
    rounding. Large scores exercise the running-reference moves."""
    B, H, N, d = 1, 4, 1000, 128
    offs = wl.document_offsets(N, 1, 300, seed=3) if mask == "document" else None
    doc = None if offs is None else torch.from_numpy(offs).cuda()
    c = np.random.default_rng(2).standard_normal(d).astype(np.float32)
    for dtype, rel in (("bf16", 2.0 ** -8), ("f32", 1e-5)):
        q, k, _ = dense(B, H, N, d, seed=17, dtype=dtype)
        q = q * 6.0                              # scores spread over many nats
        vc = torch.from_numpy(np.broadcast_to(c, (B, H, N, d)).copy()).to(q.dtype).cuda()
        o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        A.attn_fwd(q, k, vc, o, 1.0 / math.sqrt(d), mask, doc_offsets=doc)
        torch.cuda.synchronize()
        cref = vc[0, 0, 0].double().cpu().numpy()
        err = np.abs(o.double().cpu().numpy() - cref)
        assert np.all(err <= rel * np.abs(cref) + 1e-6), (dtype, err.max())


@pytest.mark.parametrize("v8", [False, True])
def test_fp8_equal_scores_give_mean_of_values(v8):
    say(f"fp8 equal scores v8={v8}")
    B, H, N, d = 1, 2, 1100, 128
    q, k, v = wl.dense_inputs(B, H, N, d, seed=41)
    nb = -(-N // 128)
    codes = [torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(3)]
    scales = [torch.empty((B, H, nb), dtype=torch.float32, device="cuda") for _ in range(3)]
    A.attn_quant_fp8_block(torch.from_numpy(q).cuda(), codes[0], scales[0])
    # zero keys: all-zero blocks quantise to code 0 with scale 1
    A.attn_quant_fp8_block(torch.zeros((B, H, N, d), device="cuda"), codes[1], scales[1])
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    if v8:
        A.attn_quant_fp8_block_pow2(torch.from_numpy(v).cuda(), codes[2], scales[2])
        A.attn_fwd_fp8_full(codes[0], scales[0], codes[1], scales[1], codes[2], scales[2], o, 0.125, "causal")
        torch.cuda.synchronize()
        # V as the kernel sees it: E4M3FN codes decoded by torch, times the block scale
        vals = codes[2].cpu().view(torch.float8_e4m3fn).double().numpy()
        v64 = vals * np.repeat(scales[2].double().cpu().numpy(), 128, axis=-1)[..., :N, None]
    else:
        vb = wl.to_bf16(v)
        A.attn_fwd_fp8(codes[0], scales[0], codes[1], scales[1], vb.cuda(), o, 0.125, "causal")
        torch.cuda.synchronize()
        v64 = vb.double().numpy()
    ref, _ = uniform_mean(v64, visible("causal", N))
    err = np.abs(o.double().cpu().numpy() - ref)
    assert np.all(err <= half_ulp_bf16(ref) + 1e-5), err.max()


@pytest.mark.parametrize("page", [16, 64])
def test_paged_equal_scores_give_mean_of_sequence(page):
    """Decode and paged prefill over a pool of zero keys: the mean of the V
    rows the block table maps, gathered here by plain indexing."""
    S, H, d, q_rows = 5, 2, 128, 40
    inp = wl.paged_inputs(S, H, d, 45, 900, seed=page, spare=3, page_size=page, q_rows=q_rows)
    vpool = inp.v_pool.double().numpy()
    bt, lens = inp.block_table.numpy(), inp.seq_lens.numpy()
    kp, vp, btd, lensd = (x.cuda() for x in (inp.k_pool, inp.v_pool, inp.block_table, inp.seq_lens))
    kp = torch.zeros_like(kp)
    q_dec = inp.q[:, :, -1].contiguous().cuda()
    o_dec = torch.empty((S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
    A.attn_decode_paged(q_dec, kp, vp, btd, lensd, o_dec, 0.1, lse=lse)
    o_pre = torch.empty((S, H, q_rows, d), dtype=torch.bfloat16, device="cuda")
    A.attn_prefill_paged(inp.q.cuda(), kp, vp, btd, lensd, o_pre, 0.1)
    torch.cuda.synchronize()
    for s in range(S):
        L = int(lens[s])
        t = np.arange(L)
        rows = vpool[bt[s, t // page], :, t % page, :]          # [L, H, d]
        pref = np.cumsum(rows, axis=0) / (t + 1)[:, None, None]
        ref_dec = pref[L - 1]
        err = np.abs(o_dec[s].double().cpu().numpy() - ref_dec)
        assert np.all(err <= half_ulp_bf16(ref_dec) + 1e-5), (s, err.max())
        assert np.abs(lse[s].double().cpu().numpy() - math.log(L)).max() <= 1e-5
        ref_pre = pref[L - q_rows:].transpose(1, 0, 2)              # [H, q_rows, d]
        err = np.abs(o_pre[s].double().cpu().numpy() - ref_pre)
        assert np.all(err <= half_ulp_bf16(ref_pre) + 1e-5), (s, err.max())
