"""GPU parity of attn_fwd (bf16 MFMA path and fp32 path) against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_lse, LSE_TOL_MFMA, check_close, cuda, sample_rows, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run(q, k, v, scale, mask, window, out_dtype, with_lse=True):
    q, k, v = cuda(q), cuda(k), cuda(v)
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    A.attn_fwd(q, k, v, o, scale, mask, window, lse=lse)
    torch.cuda.synchronize()
    return o, lse


# (B, H, N, d, mask, window): every case spans several tiles or a ragged tail
SMALL = [
    (1, 2, 1, 64, "none", 0), (1, 2, 1, 128, "causal", 0), (1, 1, 1, 64, "sliding", 1),
    (1, 2, 7, 128, "causal", 0), (2, 3, 100, 64, "none", 0), (1, 2, 129, 128, "causal", 0),
    (1, 2, 257, 64, "sliding", 5), (1, 1, 300, 128, "sliding", 64), (2, 2, 384, 64, "causal", 0),
    (1, 2, 1000, 128, "sliding", 100), (1, 1, 700, 64, "sliding", 703), (1, 1, 513, 128, "sliding", 1),
    (1, 2, 640, 64, "none", 0), (1, 1, 555, 128, "none", 0), (3, 1, 200, 128, "sliding", 130),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fwd_bf16_small_elementwise(case, out):
    B, H, N, d, mask, window = case
    say(f"fwd bf16 {case} out={out}")
    q, k, v = wl.dense_inputs(B, H, N, d, seed=7 + N + d)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(qb, kb, vb, scale, mask, window, torch.float32 if out == "f32" else torch.bfloat16)
    ref, ref_lse = oracle.attention(wl.bf16_to_f64(qb), wl.bf16_to_f64(kb), wl.bf16_to_f64(vb), scale, mask,
                                    window if mask == "sliding" else None)
    check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("case", [(1, 1, 256, 64, "none", 0), (1, 2, 77, 64, "causal", 0),
                                  (2, 1, 300, 128, "sliding", 33), (1, 1, 1, 64, "none", 0),
                                  (1, 3, 130, 128, "none", 0)], ids=lambda c: "-".join(map(str, c)))
def test_fwd_f32_elementwise(case):
    """fp32 in/out (the single-head fp32 workload and ragged/masked variants)."""
    B, H, N, d, mask, window = case
    say(f"fwd f32 {case}")
    q, k, v = (torch.from_numpy(x) for x in wl.dense_inputs(B, H, N, d, seed=11 + N))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, scale, mask, window, torch.float32)
    ref, ref_lse = oracle.attention(q.numpy(), k.numpy(), v.numpy(), scale, mask,
                                    window if mask == "sliding" else None)
    err = check_close(to_np(o), ref, False, what=str(case))
    assert err <= 1e-4, err            # fp32 throughout: far inside the 1e-2 bar
    check_lse(to_np(lse), ref_lse, tol=1e-4)


@pytest.mark.parametrize("case", [(2, 8, 4096, 64, "causal"), (1, 16, 2100, 128, "none")],
                         ids=lambda c: "-".join(map(str, c)))
def test_fwd_f32_large_grid_sampled(case):
    """Grids of at least one 128-row workgroup per CU take the 128-row fp32
    layout (smaller ones split the key tiles over the waves of 32-row
    workgroups); sampled rows of two heads against the oracle."""
    B, H, N, d, mask = case
    say(f"fwd f32 large grid {case}")
    q, k, v = (torch.from_numpy(x) for x in wl.dense_inputs(B, H, N, d, seed=13 + N))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, scale, mask, 0, torch.float32)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = sample_rows(N, 13 + h)
        ref, ref_lse = oracle.attention(q[b, h].numpy(), k[b, h].numpy(), v[b, h].numpy(), scale, mask, rows=rows)
        err = check_close(to_np(o[b, h][rows]), ref, False, what=f"{case} {(b, h)}")
        assert err <= 1e-4, err
        check_lse(to_np(lse[b, h][rows]), ref_lse, tol=1e-4)


def test_fwd_f32_workload_1_full():
    w = wl.WORKLOADS[1]
    q, k, v = (torch.from_numpy(x) for x in wl.dense_inputs(w.B, w.H, w.N, w.d, seed=wl.default_seed(1)))
    o, _ = _run(q, k, v, w.scale, w.mask, 0, torch.float32, with_lse=False)
    ref, _ = oracle.attention(q.numpy(), k.numpy(), v.numpy(), w.scale, w.mask)
    err = check_close(to_np(o), ref, False, what=w.name)
    say(f"{w.name}: max abs err {err:.3g}")
    assert err <= 1e-4


def _sampled_full_size(key, heads, seed):
    w = wl.WORKLOADS[key]
    say(f"{w.name}: generating inputs (seed {seed})")
    q, k, v = wl.dense_inputs(w.B, w.H, w.N, w.d, seed=seed)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    del q, k, v
    window = w.window if w.mask == "sliding" else 0
    say(f"{w.name}: running attn_fwd")
    o_bf, lse = _run(qb, kb, vb, w.scale, w.mask, window, torch.bfloat16)
    o32, _ = _run(qb, kb, vb, w.scale, w.mask, window, torch.float32, with_lse=False)
    assert torch.isfinite(o_bf).all() and torch.isfinite(o32).all()
    worst = 0.0
    for (b, h) in heads:
        rows = sample_rows(w.N, seed + 31 * b + h)
        ref, ref_lse = oracle.attention(wl.bf16_to_f64(qb[b, h]), wl.bf16_to_f64(kb[b, h]),
                                        wl.bf16_to_f64(vb[b, h]), w.scale, w.mask,
                                        window or None, rows=rows)
        worst = max(worst, check_close(to_np(o32[b, h][rows]), ref, False, what=f"{w.name} f32 {(b, h)}"))
        check_close(to_np(o_bf[b, h][rows]), ref, True, what=f"{w.name} bf16 {(b, h)}")
        check_lse(to_np(lse[b, h][rows]), ref_lse)
    say(f"{w.name}: sampled max abs err (fp32 out) {worst:.3g}")
    return qb, kb, vb, o_bf


def test_fwd_workload_2_causal_full_size_sampled():
    w = wl.WORKLOADS[2]
    qb, kb, vb, o1 = _sampled_full_size(2, [(0, 0), (1, 5), (3, 15), (2, 9)], wl.default_seed(2))
    # a repeated run is bitwise identical
    o2, _ = _run(qb, kb, vb, w.scale, w.mask, 0, torch.bfloat16, with_lse=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_fwd_workload_3_sliding_full_size_sampled():
    _sampled_full_size(3, [(0, 0), (1, 31), (0, 17)], wl.default_seed(3))


def test_fwd_second_seed_causal():
    _sampled_full_size(2, [(2, 3)], wl.default_seed(2) + 100)


def test_fwd_rejects_misaligned_and_leaves_output():
    q = torch.zeros(1, 1, 65, 64, dtype=torch.bfloat16, device="cuda")
    flat = torch.zeros(1 * 1 * 64 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:1 + 64 * 64].view(1, 1, 64, 64)      # 2-byte offset
    o = torch.full((1, 1, 64, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        A.attn_fwd(mis, mis, mis, o, 0.125, "none")
    with pytest.raises(ValueError):
        A.attn_fwd(q[:, :, :64], q[:, :, :64], q[:, :, :64], o, 0.125, "sliding", 0)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
