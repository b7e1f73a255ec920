"""GPU parity of attn_fwd under the structured masks -- documents and packed
variable-length causal sequences ("Optimizing Triton kernels for custom
attention patterns on H100", Pattern A), the two-sided window and the
prefix-LM mask (end of Pattern B) -- against the oracle, element by element
on small ragged cases and on sampled rows at the full workload sizes."""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_lse, FP8_REL_RMSE, LSE_TOL_MFMA, check_close, cuda, rel_rmse, sample_rows, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _docs(N, kind, seed=0):
    """Host document offsets [0, ..., N] of a named layout."""
    rng = np.random.default_rng(seed + N)
    if kind == "one":
        return np.array([0, N])
    if kind == "singles":                      # every position its own document
        return np.arange(N + 1)
    if kind == "aligned":                      # boundaries on 64- and 128-key tile edges
        return np.array(sorted(set([0, N] + [c for c in (64, 128, 384, 448, 1024) if c < N])))
    if kind == "empty":                        # empty documents, including first and last
        cuts = sorted(rng.integers(1, N, size=5).tolist()) if N > 1 else []
        return np.array([0, 0] + sorted(cuts + cuts[:2]) + [N, N])
    if kind == "small":                        # many short documents (multi-level search)
        lens = rng.integers(1, 9, size=N)
        offs = np.concatenate([[0], np.cumsum(lens)])
        return np.concatenate([offs[offs < N], [N]])
    if kind == "random":
        return wl.document_offsets(N, 5, max(6, N // 3), seed)
    raise ValueError(kind)


def _run(q, k, v, scale, mask, window, out_dtype, offs=None, with_lse=True):
    q, k, v = cuda(q), cuda(k), cuda(v)
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    doc = None if offs is None else torch.from_numpy(np.asarray(offs, dtype=np.int32)).cuda()
    A.attn_fwd(q, k, v, o, scale, mask, window, doc_offsets=doc, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def _ref(qb, kb, vb, scale, mask, window, offs, rows=None):
    win = window if mask in ("sliding", "band", "prefix_lm") else None
    return oracle.attention(wl.bf16_to_f64(qb), wl.bf16_to_f64(kb), wl.bf16_to_f64(vb), scale, mask, win,
                            rows=rows, doc_offsets=None if offs is None else np.asarray(offs))


# (B, H, N, d, mask, window, document layout)
SMALL = [
    (1, 2, 300, 64, "band", 0, None), (1, 1, 257, 128, "band", 5, None), (2, 1, 700, 64, "band", 100, None),
    (1, 2, 1000, 128, "band", 999, None), (1, 1, 130, 64, "band", 64, None),
    (1, 2, 300, 128, "prefix_lm", 0, None), (1, 1, 513, 64, "prefix_lm", 1, None),
    (2, 1, 700, 128, "prefix_lm", 200, None), (1, 1, 200, 64, "prefix_lm", 500, None),
    (1, 2, 1, 64, "document", 0, "one"), (1, 2, 333, 128, "document", 0, "one"),
    (1, 1, 200, 64, "document", 0, "singles"), (1, 2, 1100, 128, "document", 0, "aligned"),
    (1, 1, 777, 64, "document", 0, "empty"), (1, 2, 1000, 128, "document", 0, "small"),
    (2, 2, 900, 64, "document", 0, "random"), (1, 1, 5000, 64, "document", 0, "singles"),
    (1, 2, 333, 64, "document_causal", 0, "one"), (1, 1, 1100, 64, "document_causal", 0, "aligned"),
    (1, 2, 777, 128, "document_causal", 0, "empty"), (1, 1, 1000, 64, "document_causal", 0, "small"),
    (2, 1, 900, 128, "document_causal", 0, "random"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_masks_bf16_small_elementwise(case, out):
    B, H, N, d, mask, window, layout = case
    say(f"mask bf16 {case} out={out}")
    offs = None if layout is None else _docs(N, layout)
    q, k, v = wl.dense_inputs(B, H, N, d, seed=17 + N + d)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(qb, kb, vb, scale, mask, window, torch.float32 if out == "f32" else torch.bfloat16, offs)
    ref, ref_lse = _ref(qb, kb, vb, scale, mask, window, offs)
    check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse)


@pytest.mark.parametrize("case", [(1, 1, 256, 64, "band", 3, None), (1, 2, 300, 128, "prefix_lm", 40, None),
                                  (1, 1, 500, 64, "document", 0, "random"),
                                  (1, 2, 300, 128, "document_causal", 0, "empty"),
                                  (1, 1, 200, 64, "document", 0, "singles")],
                         ids=lambda c: "-".join(map(str, c)))
def test_masks_f32_elementwise(case):
    """fp32 in/out path under the structured masks."""
    B, H, N, d, mask, window, layout = case
    say(f"mask f32 {case}")
    offs = None if layout is None else _docs(N, layout)
    q, k, v = (torch.from_numpy(x) for x in wl.dense_inputs(B, H, N, d, seed=23 + N))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, scale, mask, window, torch.float32, offs)
    win = window if mask in ("band", "prefix_lm") else None
    ref, ref_lse = oracle.attention(q.numpy(), k.numpy(), v.numpy(), scale, mask, win,
                                    doc_offsets=None if offs is None else np.asarray(offs))
    err = check_close(to_np(o), ref, False, what=str(case))
    assert err <= 1e-4, err
    check_lse(to_np(lse), ref_lse, tol=1e-4)


def test_document_masks_fp8():
    """fp8 Q/K with documents: relative RMSE against the oracle on the dequantised inputs."""
    B, H, N, d = 1, 2, 1000, 128
    q, k, v = wl.dense_inputs(B, H, N, d, seed=29, outlier_p=0.01, outlier_scale=20.0)
    offs = _docs(N, "random")
    doc = torch.from_numpy(offs.astype(np.int32)).cuda()
    vb = wl.to_bf16(v)
    codes, scales = [], []
    for x in (q, k):
        c = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
        s = torch.empty((B, H, -(-N // 128)), dtype=torch.float32, device="cuda")
        A.attn_quant_fp8_block(cuda(torch.from_numpy(x)), c, s)
        codes.append(c)
        scales.append(s)
    for mask in ("document", "document_causal"):
        say(f"fp8 {mask}")
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        A.attn_fwd_fp8(codes[0], scales[0], codes[1], scales[1], cuda(vb), o, 1 / math.sqrt(d), mask,
                       doc_offsets=doc)
        torch.cuda.synchronize()
        qh = oracle.dequantize_blocks(codes[0].cpu().numpy(), scales[0].cpu().numpy())
        kh = oracle.dequantize_blocks(codes[1].cpu().numpy(), scales[1].cpu().numpy())
        ref, _ = oracle.attention(qh, kh, wl.bf16_to_f64(vb), 1 / math.sqrt(d), mask, doc_offsets=offs)
        rr = rel_rmse(to_np(o), ref)
        say(f"fp8 {mask}: rel RMSE vs dequantised oracle {rr:.3g}")
        assert rr <= min(FP8_REL_RMSE, 1e-2)


def _sampled_full_size(key, heads):
    w = wl.WORKLOADS[key]
    seed = wl.default_seed(key)
    say(f"{w.name}: generating inputs (seed {seed})")
    q, k, v = wl.dense_inputs(w.B, w.H, w.N, w.d, seed=seed)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    del q, k, v
    offs = wl.document_offsets(w.N, w.l_min, w.l_max, seed) if w.mask in A.DOC_MASKS else None
    say(f"{w.name}: running attn_fwd")
    o_bf, lse = _run(qb, kb, vb, w.scale, w.mask, w.window, torch.bfloat16, offs)
    o32, _ = _run(qb, kb, vb, w.scale, w.mask, w.window, torch.float32, offs, with_lse=False)
    assert torch.isfinite(o_bf).all() and torch.isfinite(o32).all()
    worst = 0.0
    for b, h in heads:
        rows = sample_rows(w.N, seed + 31 * b + h)
        if offs is not None:          # the first and last rows of every document too
            rows = sorted(set(rows) | set(int(x) for x in offs[:-1]) | set(int(x) - 1 for x in offs[1:]))
        ref, ref_lse = _ref(qb[b, h], kb[b, h], vb[b, h], w.scale, w.mask, w.window, offs, rows=rows)
        worst = max(worst, check_close(to_np(o32[b, h][rows]), ref, False, what=f"{w.name} f32 {(b, h)}"))
        check_close(to_np(o_bf[b, h][rows]), ref, True, what=f"{w.name} bf16 {(b, h)}")
        check_lse(to_np(lse[b, h][rows]), ref_lse)
    say(f"{w.name}: sampled max abs err (fp32 out) {worst:.3g}")


@pytest.mark.parametrize("key,heads", [(6, [(0, 0), (0, 15)]), (7, [(0, 3), (0, 12)]), (8, [(0, 0), (0, 9)]),
                                       (9, [(0, 0), (1, 15)]), (10, [(0, 0), (0, 11)])])
def test_structured_workloads_full_size_sampled(key, heads):
    _sampled_full_size(key, heads)


def test_document_equals_per_document_dense_runs():
    """A packed document batch gives, row for row, the output of attending each
    document on its own with no mask (the same kernel, one launch per document)."""
    H, N, d = 2, 1500, 128
    offs = _docs(N, "random", seed=5)
    q, k, v = (wl.to_bf16(x) for x in wl.dense_inputs(1, H, N, d, seed=31))
    packed, _ = _run(q, k, v, 1 / math.sqrt(d), "document", 0, torch.float32, offs, with_lse=False)
    for s, e in zip(offs[:-1], offs[1:]):
        if e == s:
            continue
        one, _ = _run(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], 1 / math.sqrt(d), "none", 0, torch.float32,
                      with_lse=False)
        assert torch.max(torch.abs(packed[:, :, s:e] - one)).item() <= 2e-3


def test_document_mask_rejects_bad_arguments():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q, o, 0.125, "document")                 # no offsets
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q, o, 0.125, "document", doc_offsets=torch.zeros(3, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q, o, 0.125, "band", -1)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
