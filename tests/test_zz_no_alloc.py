"""attn_decode_paged_noalloc (the decode with its partial states in the
library's fixed device array) gives exactly attn_decode_paged's split-path
result, on two calls in a row, the second smaller than the first (so the
array still holds the first call's states when the second runs)."""

import math

import pytest
import torch

from parity import cuda, say
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(key=None, **kw):
    if key is not None:
        w = wl.WORKLOADS[key]
        return wl.paged_inputs(w.n_seq, w.H, w.d, w.l_min, w.l_max, seed=wl.default_seed(key),
                               page_size=w.page_size, spare=w.spare_pages)
    return wl.paged_inputs(**kw)


def _both(inp):
    S, H, d = inp.q.shape
    q, kp, vp = cuda(inp.q), cuda(inp.k_pool), cuda(inp.v_pool)
    bt, lens = cuda(inp.block_table), cuda(inp.seq_lens)
    scale = 1.0 / math.sqrt(d)
    o_ws = torch.full((S, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_ws = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(A.attn_decode_paged_workspace_size(S, H, d, bt.shape[1], kp.shape[2]), dtype=torch.uint8,
                     device="cuda")
    A.attn_decode_paged(q, kp, vp, bt, lens, o_ws, scale, workspace=ws, lse=l_ws)
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    A.attn_decode_paged_noalloc(q, kp, vp, bt, lens, o_na, scale, lse=l_na)
    torch.cuda.synchronize()
    return (o_ws, l_ws), (o_na, l_na)


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    cases = [("workload 4 (64 sequences, 16-token pages)", _inputs(4)),
             ("6 sequences of 1..700 tokens, d = 64, 64-token pages",
              _inputs(n_seq=6, H=4, d=64, l_min=1, l_max=700, seed=123, page_size=64, spare=3))]
    for name, inp in cases:
        say(f"no-alloc decode: {name}")
        (o_ws, l_ws), (o_na, l_na) = _both(inp)
        assert torch.isfinite(o_na.float()).all()
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), name
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), name
