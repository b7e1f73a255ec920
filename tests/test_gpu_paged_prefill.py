"""GPU parity of the fused paged prefill and block-sparse paged
cross-attention ("Optimizing Triton kernels for custom attention patterns on
H100", Pattern C) against the oracle, element by element on small ragged
cases (64-token pages, and the decode's 16-token pages, four to a K tile) and
on sampled rows at the full workload sizes. The pools hold NaN in every row
no sequence or list owns, so a read past a list shows up."""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_lse, LSE_TOL_MFMA, check_close, cuda, sample_rows, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _prefill(inp, q_len, out_dtype, scale):
    q = inp.q.cuda()
    S, H, _, d = q.shape
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((S, H, q_len), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_prefill_paged(q, inp.k_pool.cuda(), inp.v_pool.cuda(), inp.block_table.cuda(), inp.seq_lens.cuda(), o,
                         scale, lse=lse)
    torch.cuda.synchronize()
    return o, lse


# (S, H, q_len, d, l_min, l_max): ragged lengths, q_len from one row to several blocks
PREFILL = [(3, 2, 1, 128, 1, 200), (2, 3, 100, 64, 100, 700), (4, 2, 300, 128, 300, 1500),
           (2, 1, 129, 64, 129, 129), (3, 2, 512, 128, 512, 2000), (1, 2, 64, 64, 64, 64),
           (5, 1, 33, 128, 40, 900)]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("page", [64, 16])
def test_prefill_paged_small_elementwise(case, out, page):
    S, H, q_len, d, l_min, l_max = case
    say(f"paged prefill {case} out={out} page={page}")
    inp = wl.paged_inputs(S, H, d, l_min, l_max, seed=41 + q_len + d, page_size=page, spare=5, q_rows=q_len)
    scale = 1.0 / math.sqrt(d)
    o, lse = _prefill(inp, q_len, torch.float32 if out == "f32" else torch.bfloat16, scale)
    ref, ref_lse = oracle.prefill(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                  inp.block_table.numpy(), inp.seq_lens.numpy(), scale, page_size=page)
    check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse)


def _cross(inp, out_dtype, scale):
    q = inp.q.cuda()
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    A.attn_cross_paged(q, inp.k_pool.cuda(), inp.v_pool.cuda(), inp.page_table.cuda(), inp.kv_lens.cuda(), o,
                       scale, lse=lse)
    torch.cuda.synchronize()
    return o, lse


# (S, H, q_len, d, pool pages, pages per block)
CROSS = [(2, 2, 300, 64, 9, 4), (1, 3, 128, 128, 40, 17), (3, 1, 1, 128, 5, 1), (2, 2, 700, 128, 64, 40),
         (1, 1, 257, 64, 3, 3)]


@pytest.mark.parametrize("case", CROSS, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("page", [64, 16])
def test_cross_paged_small_elementwise(case, out, page):
    S, H, q_len, d, pool, per = case
    say(f"paged cross {case} out={out} page={page}")
    inp = wl.paged_cross_inputs(S, H, d, q_len, pool, per, seed=43 + q_len, page_size=page, spare=3)
    if S * (-(-q_len // 128)) > 1:
        inp.kv_lens[0, -1] = 0                 # one block with no keys: O = 0, LSE = -inf
    scale = 1.0 / math.sqrt(d)
    o, lse = _cross(inp, torch.float32 if out == "f32" else torch.bfloat16, scale)
    ref, ref_lse = oracle.cross(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                inp.page_table.numpy(), inp.kv_lens.numpy(), scale, page_size=page)
    check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse, what=str(case))


@pytest.mark.parametrize("key", [11, 14])
def test_prefill_paged_full_size_sampled(key):
    w = wl.WORKLOADS[key]
    seed = wl.default_seed(key)
    say(f"{w.name}: generating inputs (seed {seed})")
    inp = wl.paged_inputs(w.n_seq, w.H, w.d, w.l_min, w.l_max, seed=seed, page_size=w.page_size,
                          spare=w.spare_pages, q_rows=w.q_len)
    say(f"{w.name}: running attn_prefill_paged")
    o, lse = _prefill(inp, w.q_len, torch.bfloat16, w.scale)
    o32, _ = _prefill(inp, w.q_len, torch.float32, w.scale)
    assert torch.isfinite(o).all() and torch.isfinite(o32).all()
    kp, vp = inp.k_pool.float().numpy(), inp.v_pool.float().numpy()
    table, lens = inp.block_table.numpy(), inp.seq_lens.numpy()
    for s, h in [(0, 0), (7, 31), (15, 12)]:
        rows = sample_rows(w.q_len, seed + s)
        L = int(lens[s])
        k = oracle.gather(kp, table[s:s + 1], lens[s:s + 1], page_size=w.page_size)[0][h]
        v = oracle.gather(vp, table[s:s + 1], lens[s:s + 1], page_size=w.page_size)[0][h]
        ref, ref_lse = oracle.attention(wl.bf16_to_f64(inp.q[s, h]), k, v, w.scale, "causal", rows=rows,
                                        q_pos_offset=L - w.q_len)
        check_close(to_np(o32[s, h][rows]), ref, False, what=f"{w.name} f32 {(s, h)}")
        check_close(to_np(o[s, h][rows]), ref, True, what=f"{w.name} bf16 {(s, h)}")
        check_lse(to_np(lse[s, h][rows]), ref_lse)
    say(f"{w.name}: sampled rows match")


def test_cross_paged_full_size_sampled():
    w = wl.WORKLOADS[12]
    seed = wl.default_seed(12)
    say(f"{w.name}: generating inputs (seed {seed})")
    inp = wl.paged_cross_inputs(w.n_seq, w.H, w.d, w.q_len, w.pool_pages, w.pages_per_block, seed=seed,
                                page_size=w.page_size, spare=w.spare_pages)
    say(f"{w.name}: running attn_cross_paged")
    o, lse = _cross(inp, torch.bfloat16, w.scale)
    o32, _ = _cross(inp, torch.float32, w.scale)
    assert torch.isfinite(o).all() and torch.isfinite(o32).all()
    kp, vp = inp.k_pool.float().numpy(), inp.v_pool.float().numpy()
    for s, h, b in [(0, 0, 0), (3, 17, 5), (7, 31, 7)]:
        rows = [r for r in sample_rows(128, seed + s + b, extra=8) if r < 128]
        n = int(inp.kv_lens[s, b])
        k = oracle.listed_keys(kp, inp.page_table[s, b].numpy(), n, 64)[h].astype(np.float64)
        v = oracle.listed_keys(vp, inp.page_table[s, b].numpy(), n, 64)[h].astype(np.float64)
        qrows = [128 * b + r for r in rows]
        ref, ref_lse = oracle.attention(wl.bf16_to_f64(inp.q[s, h]), k, v, w.scale, "none", rows=qrows)
        check_close(to_np(o32[s, h][qrows]), ref, False, what=f"{w.name} f32 {(s, h, b)}")
        check_close(to_np(o[s, h][qrows]), ref, True, what=f"{w.name} bf16 {(s, h, b)}")
        check_lse(to_np(lse[s, h][qrows]), ref_lse)
    say(f"{w.name}: sampled rows match")


@pytest.mark.parametrize("page", [64, 16])
def test_cross_paged_repeats_long_lists_and_page_order(page):
    """A list is a multiset of keys, so the kernel may visit its whole pages
    in any order (it sorts them by id): lists that repeat pages, lists longer
    than the part that is reordered (300 pages of 16 tokens), and lengths
    that end inside the list or inside a page, against the oracle; and a
    permutation of each list's whole pages (the partial last page left in
    place) gives the same output bit for bit."""
    S, H, q_len, d, pool = 2, 2, 256, 128, 40
    per = 300 if page == 16 else 70
    base = wl.paged_cross_inputs(S, H, d, q_len, pool, 8, seed=71 + page, page_size=page, spare=3)
    rng = np.random.default_rng(72 + page)
    nqb = -(-q_len // 128)
    table = rng.integers(0, pool, size=(S, nqb, per)).astype(np.int32)
    lens = np.array([[per * page, per * page - page // 2], [37 * page + 5, 3 * page]], dtype=np.int32)
    for s in range(S):
        for b in range(nqb):
            used = -(-int(lens[s, b]) // page)
            table[s, b, used:] = pool + rng.integers(0, 3, size=per - used)   # NaN pages, never read
    inp = wl.CrossInputs(q=base.q, k_pool=base.k_pool, v_pool=base.v_pool, page_table=torch.from_numpy(table),
                         kv_lens=torch.from_numpy(lens), page_size=page, q_block=128)
    scale = 1.0 / math.sqrt(d)
    o, lse = _cross(inp, torch.float32, scale)
    ref, ref_lse = oracle.cross(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                table, lens, scale, page_size=page)
    check_close(to_np(o), ref, False, what=f"repeats page={page}")
    check_lse(to_np(lse), ref_lse)
    perm = table.copy()
    for s in range(S):
        for b in range(nqb):
            full = int(lens[s, b]) // page
            perm[s, b, :full] = rng.permutation(perm[s, b, :full])
    inp2 = wl.CrossInputs(q=base.q, k_pool=base.k_pool, v_pool=base.v_pool, page_table=torch.from_numpy(perm),
                          kv_lens=torch.from_numpy(lens), page_size=page, q_block=128)
    o2, lse2 = _cross(inp2, torch.float32, scale)
    # the kernel orders the first 256 entries of a list; past them the order
    # is the caller's, so only lists of at most 256 whole pages match exactly
    for s in range(S):
        for b in range(nqb):
            rows = slice(128 * b, min(q_len, 128 * (b + 1)))
            if int(lens[s, b]) // page <= 256:
                assert torch.equal(o2[s, :, rows], o[s, :, rows]), (s, b)
                assert torch.equal(lse2[s, :, rows], lse[s, :, rows]), (s, b)
            else:
                check_close(to_np(o2[s, :, rows]), ref[s, :, rows], False, what=f"permuted long list {(s, b)}")


def test_prefill_paged_one_row_matches_decode():
    """q_len = 1 is a decode: the fused prefill kernel and the decode oracle agree."""
    inp = wl.paged_inputs(4, 2, 128, 1, 3000, seed=47, page_size=64, spare=2, q_rows=1)
    o, _ = _prefill(inp, 1, torch.float32, 1 / math.sqrt(128))
    ref, _ = oracle.decode(wl.bf16_to_f64(inp.q[:, :, 0]), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                           inp.block_table.numpy(), inp.seq_lens.numpy(), 1 / math.sqrt(128), page_size=64)
    check_close(to_np(o[:, :, 0]), ref, False, what="q_len=1")


def test_prefill_and_decode_share_a_16_token_pool():
    """One pool of the decode's 16-token pages serves both paths: the fused
    prefill's last row of each sequence and the decode of that row both match
    the decode oracle (the prefill rounds P to bf16, the decode does not)."""
    S, H, d = 5, 4, 128
    inp = wl.paged_inputs(S, H, d, 200, 5000, seed=53, page_size=16, spare=7, q_rows=96)
    scale = 1 / math.sqrt(d)
    o, lse = _prefill(inp, 96, torch.float32, scale)
    q_last = inp.q[:, :, -1].contiguous().cuda()
    od = torch.full((S, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")   # the decode writes bf16
    lsed = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_decode_paged(q_last, inp.k_pool.cuda(), inp.v_pool.cuda(), inp.block_table.cuda(), inp.seq_lens.cuda(),
                        od, scale, lse=lsed)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(wl.bf16_to_f64(inp.q[:, :, -1]), inp.k_pool.float().numpy(),
                                 inp.v_pool.float().numpy(), inp.block_table.numpy(), inp.seq_lens.numpy(), scale,
                                 page_size=16)
    check_close(to_np(o[:, :, -1]), ref, False, what="prefill's last row on the shared pool")
    check_close(to_np(od), ref, True, what="decode on the shared pool")
    check_lse(to_np(lse[:, :, -1]), ref_lse)
    check_lse(to_np(lsed), ref_lse)


def test_paged_prefill_rejects():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    pool32 = torch.zeros(4, 1, 32, 64, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    lens = torch.full((1,), 8, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):            # 32-token pages: unsupported
        A.attn_prefill_paged(q, pool32, pool32, table, lens, o, 0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)


@pytest.mark.parametrize("page", [64, 16])
def test_two_stage_route_equals_fused(page):
    """The two-stage route of "Optimizing Triton kernels ...", Pattern C --
    gather every sequence's pages into a dense copy, then attend over it --
    gives the fused kernel's output bit for bit: both visit the same keys in
    the same 64-key tiles, one reading pages, the other the copy (read as
    contiguous 64-token pages through an identity table). Rows of the copy
    past each sequence's length are NaN-poisoned and never read."""
    import bench
    S, H, q_len, d = 3, 4, 300, 128
    inp = wl.paged_inputs(S, H, d, 300, 1500, seed=77 + page, page_size=page, spare=5, q_rows=q_len,
                          max_pages=1536 // page)
    scale = 1.0 / math.sqrt(d)
    kp, vp, bt, lens = inp.k_pool.cuda(), inp.v_pool.cuda(), inp.block_table.cuda(), inp.seq_lens.cuda()
    q = inp.q.cuda()
    fused = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    A.attn_prefill_paged(q, kp, vp, bt, lens, fused, scale)
    T = bt.shape[1] * page
    assert T % 64 == 0                     # table rows of 1536 tokens: 24 pages of 64 or 96 of 16
    k_out = torch.full((S, H, T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_out = torch.full_like(k_out, float("nan"))
    A.attn_gather_paged(kp, vp, bt, lens, k_out, v_out)
    two = bench.two_stage_views(q, k_out, v_out, lens, H)
    o2 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    A.attn_prefill_paged(two["q"], two["k"], two["v"], two["table"], two["lens"], o2.view(two["q"].shape), scale)
    torch.cuda.synchronize()
    assert torch.isfinite(fused.float()).all()
    assert torch.equal(o2.view(torch.int16), fused.view(torch.int16))


@pytest.mark.parametrize("page", [64, 16])
def test_cross_out_of_contract_lists_stay_in_bounds(page):
    """Page ids outside [0, num_pages) and lengths outside [0, max_pages *
    page] break the caller's contract; the kernel clamps both (before it
    orders a list's pages), so the call completes (results unspecified there)
    and a valid block beside the broken ones gives its exact result."""
    S, H, q_len, d, pool, per = 2, 2, 384, 128, 30, 12
    inp = wl.paged_cross_inputs(S, H, d, q_len, pool, per, seed=91 + page, page_size=page, spare=3)
    table, lens = inp.page_table.clone(), inp.kv_lens.clone()
    num_pages = inp.k_pool.shape[0]
    table[0, 1, 0] = -1                        # an id below the pool
    table[0, 2, :] = num_pages + 7             # every id past the pool
    lens[0, 2] = per * page + 100              # ... and a length past its list
    lens[1, 1] = -3                            # a negative length
    o = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
    A.attn_cross_paged(cuda(inp.q), cuda(inp.k_pool), cuda(inp.v_pool), cuda(table), cuda(lens), o, 0.1)
    torch.cuda.synchronize()
    ref, _ = oracle.cross(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                          inp.page_table.numpy(), inp.kv_lens.numpy(), 0.1, page_size=page)
    check_close(to_np(o[1, :, 0:128]), ref[1, :, 0:128], False, what="valid block beside broken ones")
