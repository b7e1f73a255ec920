"""A seeded sweep of random small paged problems against the oracle: the
split-KV decode (with and without a workspace), the fused paged prefill and
block-sparse paged cross-attention, over 16- and 64-token pages, d = 64 and
128, random sequence counts, heads, lengths and list sizes. The pools hold NaN
in every page no sequence or list owns. The shapes are drawn once from a fixed
seed, so a failure names a case that can be run again. ATTN_SWEEP_SCALE=k
draws k times as many cases from the same seeds (the default cases come
first)."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_lse, cuda, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCALE = max(1, int(os.environ.get("ATTN_SWEEP_SCALE", "1")))


def _decode_cases():
    rng = np.random.default_rng(31337)
    cases = []
    for i in range(30 * SCALE):
        S, H = int(rng.integers(1, 10)), int(rng.integers(1, 5))
        d, page = int(rng.choice([64, 128])), int(rng.choice([16, 64]))
        lo = int(rng.integers(1, 3000))
        hi = int(rng.integers(lo, 3001))
        cases.append((i, S, H, d, page, lo, hi, bool(rng.random() < 0.5)))
    return cases


def _prefill_cases():
    rng = np.random.default_rng(4242)
    cases = []
    for i in range(30 * SCALE):
        S, H = int(rng.integers(1, 6)), int(rng.integers(1, 4))
        d, page = int(rng.choice([64, 128])), int(rng.choice([16, 64]))
        q_len = int(rng.integers(1, 400))
        lo = q_len + int(rng.integers(0, 1500))
        hi = lo + int(rng.integers(0, 600))
        cases.append((i, S, H, d, page, q_len, lo, hi, bool(rng.random() < 0.5)))
    return cases


def _cross_cases():
    rng = np.random.default_rng(777)
    cases = []
    for i in range(30 * SCALE):
        S, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        d, page = int(rng.choice([64, 128])), int(rng.choice([16, 64]))
        q_len = int(rng.integers(1, 520))
        pool = int(rng.integers(1, 70))
        per = int(rng.integers(1, min(pool, 45) + 1))
        cases.append((i, S, H, d, page, q_len, pool, per, bool(rng.random() < 0.5)))
    return cases


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_decode(case):
    i, S, H, d, page, lo, hi, use_ws = case
    say(f"random decode {case}")
    inp = wl.paged_inputs(n_seq=S, H=H, d=d, l_min=lo, l_max=hi, seed=500 + i, spare=3, page_size=page)
    bt, lens = cuda(inp.block_table), cuda(inp.seq_lens)
    kp, vp = cuda(inp.k_pool), cuda(inp.v_pool)
    o = torch.full((S, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    if use_ws:
        ws = torch.empty(A.attn_decode_paged_workspace_size(S, H, d, bt.shape[1], page), dtype=torch.uint8,
                         device="cuda")
    scale = 1.0 / math.sqrt(d)
    A.attn_decode_paged(cuda(inp.q), kp, vp, bt, lens, o, scale, workspace=ws, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                 inp.block_table.numpy(), inp.seq_lens.numpy(), scale, page_size=page)
    check_close(to_np(o), ref, True, what=str(case))
    check_lse(to_np(lse), ref_lse, what=str(case))


@pytest.mark.parametrize("case", _prefill_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_prefill(case):
    i, S, H, d, page, q_len, lo, hi, out_f32 = case
    say(f"random prefill {case}")
    inp = wl.paged_inputs(S, H, d, lo, hi, seed=600 + i, page_size=page, spare=3, q_rows=q_len)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((S, H, q_len, d), float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16,
                   device="cuda")
    lse = torch.full((S, H, q_len), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_prefill_paged(cuda(inp.q), cuda(inp.k_pool), cuda(inp.v_pool), cuda(inp.block_table),
                         cuda(inp.seq_lens), o, scale, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                  inp.block_table.numpy(), inp.seq_lens.numpy(), scale, page_size=page)
    check_close(to_np(o), ref, not out_f32, what=str(case))
    check_lse(to_np(lse), ref_lse, what=str(case))


@pytest.mark.parametrize("case", _cross_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_cross(case):
    i, S, H, d, page, q_len, pool, per, out_f32 = case
    say(f"random cross {case}")
    inp = wl.paged_cross_inputs(S, H, d, q_len, pool, per, seed=700 + i, page_size=page, spare=2)
    if i % 3 == 0:
        inp.kv_lens[S - 1, -1] = 0                  # a block with no keys: O = 0, LSE = -inf
    scale = 1.0 / math.sqrt(d)
    o = torch.full(inp.q.shape, float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    lse = torch.full(inp.q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    A.attn_cross_paged(cuda(inp.q), cuda(inp.k_pool), cuda(inp.v_pool), cuda(inp.page_table), cuda(inp.kv_lens), o,
                       scale, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.cross(wl.bf16_to_f64(inp.q), inp.k_pool.float().numpy(), inp.v_pool.float().numpy(),
                                inp.page_table.numpy(), inp.kv_lens.numpy(), scale, page_size=page)
    check_close(to_np(o), ref, not out_f32, what=str(case))
    check_lse(to_np(lse), ref_lse, what=str(case))
