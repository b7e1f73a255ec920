"""Launches captured in a HIP graph (as the benchmark replays them) give, on
every replay, the eager result bit for bit. Between replays the program does
its own eager work (other attention calls, elementwise ops, synchronisation)
and poisons the outputs, so each replay must rewrite them. The captured
calls launch kernels only: no memset or allocation is recorded."""

import math

import pytest
import torch

from parity import cuda, say
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _replays_match(run, outputs, disturb, n=3):
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outputs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run()
        torch.cuda.synchronize()
        for i in range(n):
            for t in outputs:
                t.fill_(float("nan"))
            disturb()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for t, r in zip(outputs, ref):
                assert torch.equal(t, r), f"replay {i} differs from the eager result"
        del g


def test_graph_replay_attn_fwd():
    say("graph: attn_fwd causal bf16")
    q, k, v = (wl.to_bf16(x).cuda() for x in wl.dense_inputs(2, 4, 700, 64, seed=61))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    q2, k2, v2 = (wl.to_bf16(x).cuda() for x in wl.dense_inputs(1, 2, 300, 128, seed=62))
    o2 = torch.empty_like(q2)

    def disturb():
        A.attn_fwd(q2, k2, v2, o2, 1 / math.sqrt(128), "sliding", 50)
        q2.mul_(1.0)

    _replays_match(lambda: A.attn_fwd(q, k, v, o, 0.125, "causal", lse=lse), [o, lse], disturb)


def test_graph_replay_decode_and_paged_prefill():
    say("graph: split-KV decode and paged prefill on one 16-token pool")
    S, H, d = 3, 2, 128
    inp = wl.paged_inputs(S, H, d, 100, 2000, seed=63, page_size=16, spare=4, q_rows=70)
    kp, vp, bt, lens = cuda(inp.k_pool), cuda(inp.v_pool), cuda(inp.block_table), cuda(inp.seq_lens)
    q = cuda(inp.q)
    q_last = q[:, :, -1].contiguous()
    o = torch.empty_like(q)
    od = torch.empty_like(q_last)
    ws = torch.empty(A.attn_decode_paged_workspace_size(S, H, d, bt.shape[1]), dtype=torch.uint8, device="cuda")
    scale = 1 / math.sqrt(d)

    def run():
        A.attn_prefill_paged(q, kp, vp, bt, lens, o, scale)
        A.attn_decode_paged(q_last, kp, vp, bt, lens, od, scale, workspace=ws)

    def disturb():
        ws.zero_()
        A.attn_decode_paged(q_last, kp, vp, bt, lens, torch.empty_like(od), scale)

    _replays_match(run, [o, od], disturb)


def test_graph_replay_cross_split_fp8_and_noalloc_decode():
    """The paged cross-attention (page lists ordered in the kernel), the
    split-key prefill (forward kernel, then its combine), the all-fp8 forward
    and the decode that keeps its partial states in the library's own device
    array (the entry point meant for callers under graph capture)."""
    say("graph: cross, split-key prefill, all-fp8, no-allocation decode")
    cin = wl.paged_cross_inputs(2, 2, 128, 300, 20, 9, seed=64, page_size=64, spare=2)
    cq, ckp, cvp = cuda(cin.q), cuda(cin.k_pool), cuda(cin.v_pool)
    ctab, clen = cuda(cin.page_table), cuda(cin.kv_lens)
    co = torch.empty_like(cq)
    sq, sk, sv = (wl.to_bf16(x).cuda() for x in wl.dense_inputs(1, 4, 8192, 64, seed=65))
    so = torch.empty_like(sq)
    ws_bytes = A.attn_fwd_split_workspace_size(1, 4, 8192, 64, "bf16", "causal", 0)
    assert ws_bytes > 0
    sws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fq, fk, fv = wl.dense_inputs(1, 2, 500, 128, seed=66)
    codes, scales = [], []
    for x, pow2 in ((fq, False), (fk, False), (fv, True)):
        c = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        s_ = torch.empty((1, 2, -(-500 // 128)), dtype=torch.float32, device="cuda")
        (A.attn_quant_fp8_block_pow2 if pow2 else A.attn_quant_fp8_block)(cuda(torch.from_numpy(x)), c, s_)
        codes.append(c)
        scales.append(s_)
    fo = torch.empty((1, 2, 500, 128), dtype=torch.bfloat16, device="cuda")
    din = wl.paged_inputs(3, 2, 128, 100, 3000, seed=67, page_size=16, spare=4)
    dq, dkp, dvp = cuda(din.q), cuda(din.k_pool), cuda(din.v_pool)
    dbt, dlen = cuda(din.block_table), cuda(din.seq_lens)
    do = torch.empty_like(dq)

    def run():
        A.attn_cross_paged(cq, ckp, cvp, ctab, clen, co, 1 / math.sqrt(128))
        A.attn_fwd_split(sq, sk, sv, so, 0.125, "causal", 0, workspace=sws)
        A.attn_fwd_fp8_full(codes[0], scales[0], codes[1], scales[1], codes[2], scales[2], fo, 1 / math.sqrt(128),
                            "causal")
        A.attn_decode_paged_noalloc(dq, dkp, dvp, dbt, dlen, do, 1 / math.sqrt(128))

    def disturb():
        sws.fill_(255)
        A.attn_decode_paged_noalloc(dq, dkp, dvp, dbt, dlen, torch.empty_like(do), 0.3)

    _replays_match(run, [co, so, fo, do], disturb)
