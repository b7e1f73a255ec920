"""Sizes at the limits, against the oracle on sampled rows.

One head of 2^18 keys makes a K loop of 4096 tiles per Q tile; 128 heads of
2^17 rows at d = 128 make tensors of 2^31 elements (4 GiB each), so the last
heads sit past every 32-bit element and byte offset; the decode case walks a
131072-token sequence through its block table (8192 pages of 16 tokens, or
2048 of 64).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_lse, LSE_TOL_MFMA, check_close, cuda, sample_rows, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,mask", [(128, "causal"), (64, "none")])
def test_long_sequence_bf16_sampled(d, mask):
    N = 1 << 18
    seed = 500 + d
    say(f"long bf16: N={N} d={d} {mask}: generating inputs")
    q, k, v = wl.dense_inputs(1, 1, N, d, seed=seed)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    del q, k, v
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = cuda(qb), cuda(kb), cuda(vb)
    o = torch.empty((1, 1, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    say("long bf16: running attn_fwd")
    A.attn_fwd(qd, kd, vd, o, scale, mask, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    rows = sample_rows(N, seed, extra=12)
    say(f"long bf16: oracle on {len(rows)} rows")
    ref, ref_lse = oracle.attention(wl.bf16_to_f64(qb[0, 0]), wl.bf16_to_f64(kb[0, 0]), wl.bf16_to_f64(vb[0, 0]),
                                    scale, mask, rows=rows)
    err = check_close(to_np(o[0, 0][rows]), ref, False, what=f"N={N} d={d} {mask}")
    check_lse(to_np(lse[0, 0][rows]), ref_lse)
    say(f"long bf16: sampled max abs err {err:.3g}")


def test_tensors_past_32_bit_offsets():
    B, H, N, d = 1, 128, 1 << 17, 128
    say(f"large tensors: [{B},{H},{N},{d}] bf16 drawn on the device")
    qd, kd, vd = wl.dense_inputs_device(B, H, N, d, seed=4242)
    assert qd.numel() == 1 << 31
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    say("large tensors: running attn_fwd (causal)")
    A.attn_fwd(qd, kd, vd, o, 1.0 / math.sqrt(d), "causal", lse=lse)
    torch.cuda.synchronize()
    for h in (0, 77, H - 1):
        rows = sample_rows(N, h, extra=6)
        qh, kh, vh = (wl.bf16_to_f64(x[0, h].cpu()) for x in (qd, kd, vd))
        ref, ref_lse = oracle.attention(qh, kh, vh, 1.0 / math.sqrt(d), "causal", rows=rows)
        err = check_close(to_np(o[0, h][rows]), ref, True, what=f"head {h}")
        check_lse(to_np(lse[0, h][rows]), ref_lse)
        say(f"large tensors: head {h} sampled max abs err {err:.3g}")


def test_long_sequence_f32_causal_sampled():
    N, d = 1 << 16, 64
    q, k, v = (torch.from_numpy(x) for x in wl.dense_inputs(1, 1, N, d, seed=77))
    o = torch.empty((1, 1, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    A.attn_fwd(cuda(q), cuda(k), cuda(v), o, 0.125, "causal", lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(N, 77, extra=12)
    ref, ref_lse = oracle.attention(q[0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy(), 0.125, "causal", rows=rows)
    err = check_close(to_np(o[0, 0][rows]), ref, False, what="fp32 long causal")
    assert err <= 1e-4
    check_lse(to_np(lse[0, 0][rows]), ref_lse, tol=1e-4)


@pytest.mark.parametrize("page", [16, 64])
def test_long_decode(page):
    L = 1 << 17
    say(f"long decode: L={L} page={page}: generating pool")
    inp = wl.paged_inputs(n_seq=2, H=2, d=128, l_min=L - 40, l_max=L, seed=page, spare=7, page_size=page)
    S, H, d = inp.q.shape
    bt, lens = cuda(inp.block_table), cuda(inp.seq_lens)
    kp, vp = cuda(inp.k_pool), cuda(inp.v_pool)
    o = torch.empty((S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(A.attn_decode_paged_workspace_size(S, H, d, bt.shape[1], page), dtype=torch.uint8,
                     device="cuda")
    A.attn_decode_paged(cuda(inp.q), kp, vp, bt, lens, o, 1.0 / math.sqrt(d), workspace=ws, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                 inp.block_table.numpy(), inp.seq_lens.numpy(), 1.0 / math.sqrt(d), page_size=page)
    check_close(to_np(o), ref, True, what=f"decode L={L} page={page}")
    check_lse(to_np(lse), ref_lse)


def test_head_of_more_than_2gib_of_bytes():
    """One head of 2^23 + 77 keys at d = 128: K and V hold more than 2^31
    bytes per head, so the byte count a K/V tile stream has left from the
    first tiles does not fit 32 bits. A one-sided 100-key window keeps the
    work small; rows near the start (where that count is largest), the middle
    and the end are checked against the oracle on the keys their window
    covers."""
    N, d, W = (1 << 23) + 77, 128, 100
    say(f"2 GiB head: [1,1,{N},{d}] bf16 drawn on the device, window {W}")
    qd, kd, vd = wl.dense_inputs_device(1, 1, N, d, seed=9191)
    o = torch.empty_like(qd)
    A.attn_fwd(qd, kd, vd, o, 1.0 / math.sqrt(d), "sliding", W)
    torch.cuda.synchronize()
    say("2 GiB head: checking rows")
    worst = 0.0
    for r0 in (0, 191, N // 2 - 64, N - 300):
        r1 = min(r0 + 300, N)
        a = max(0, r0 - W + 1)
        qh, kh, vh = (wl.bf16_to_f64(x[0, 0, lo:r1].cpu()) for x, lo in ((qd, r0), (kd, a), (vd, a)))
        ref, _ = oracle.attention(qh, kh, vh, 1.0 / math.sqrt(d), "sliding", W, q_pos_offset=r0 - a)
        worst = max(worst, check_close(to_np(o[0, 0, r0:r1]), ref, True, what=f"rows {r0}..{r1}"))
    say(f"2 GiB head: max abs err {worst:.3g}")
