"""A seeded sweep of random small fp8 problems against the oracle run on the
dequantised inputs (codes times block scales, exact in fp64): attn_fwd_fp8
(e4m3 Q and K, bf16 V) and attn_fwd_fp8_full (V in e4m3 too), under every
mask kind, d = 64 and 128, lengths that are not block multiples, random
windows and document layouts, with the outlier inputs of the fp8 workloads.
The bars are those of the fixed-shape fp8 tests: relative RMSE at most 1e-2
with bf16 P and 2e-2 with P rounded to e4m3, and the fp8 LSE bound.
ATTN_SWEEP_SCALE=k draws k times as many cases from the same seed."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import check_lse_fp8, cuda, rel_rmse, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

MASK_KINDS = ["none", "causal", "sliding", "band", "prefix_lm", "document", "document_causal"]
SCALE = max(1, int(os.environ.get("ATTN_SWEEP_SCALE", "1")))


def _cases():
    rng = np.random.default_rng(8080)
    out = []
    for i in range(28 * SCALE):
        mask = MASK_KINDS[i % len(MASK_KINDS)]
        N = int(rng.integers(1, 1100))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        window = 0
        if mask == "sliding":
            window = int(rng.integers(1, N + 40))
        elif mask in ("band", "prefix_lm"):
            window = int(rng.integers(0, N + 40))
        out.append((i, B, H, N, d, mask, window, bool(i % 2)))
    return out


def _quant(x, pow2):
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    B, H, N, _ = x.shape
    scales = torch.empty((B, H, -(-N // 128)), dtype=torch.float32, device="cuda")
    (A.attn_quant_fp8_block_pow2 if pow2 else A.attn_quant_fp8_block)(cuda(torch.from_numpy(x)), codes, scales)
    return codes, scales


def _offsets(N, seed):
    rng = np.random.default_rng(seed)
    cuts = sorted(set(rng.integers(0, N + 1, size=int(rng.integers(0, 6))).tolist()))
    return np.array([0] + cuts + [N], dtype=np.int32)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_fp8(case):
    i, B, H, N, d, mask, window, full = case
    say(f"random fp8 {case}")
    seed = 8100 + i
    q, k, v = wl.dense_inputs(B, H, N, d, seed=seed, outlier_p=0.01, outlier_scale=20.0)
    q8, sq = _quant(q, False)
    k8, sk = _quant(k, False)
    offs = _offsets(N, seed) if mask.startswith("document") else None
    doc = None if offs is None else torch.from_numpy(offs).cuda()
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    if full:
        v8, sv = _quant(v, True)
        A.attn_fwd_fp8_full(q8, sq, k8, sk, v8, sv, o, scale, mask, window, doc_offsets=doc, lse=lse)
        vh = oracle.dequantize_blocks(v8.cpu().numpy(), sv.cpu().numpy())
    else:
        vb = wl.to_bf16(v)
        A.attn_fwd_fp8(q8, sq, k8, sk, cuda(vb), o, scale, mask, window, doc_offsets=doc, lse=lse)
        vh = wl.bf16_to_f64(vb)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    qh = oracle.dequantize_blocks(q8.cpu().numpy(), sq.cpu().numpy())
    kh = oracle.dequantize_blocks(k8.cpu().numpy(), sk.cpu().numpy())
    win = window if mask in ("sliding", "band", "prefix_lm") else None
    ref, ref_lse = oracle.attention(qh, kh, vh, scale, mask, win, doc_offsets=offs)
    rr = rel_rmse(to_np(o), ref)
    say(f"  rel RMSE vs dequantised oracle {rr:.3g}")
    assert rr <= (2e-2 if full else 1e-2), f"{case}: rel RMSE {rr:.3g}"
    check_lse_fp8(to_np(lse), ref_lse)
