"""GPU parity of attn_fwd_split (the costliest query tiles' key ranges split
in two, the parts merged by a second kernel) against the oracle, element by
element, for causal and prefix-LM grids with few query tiles per workgroup
slot, both layouts of the d = 64 kernel, d = 128, ragged lengths and both
output types; and the unsplit case equal to attn_fwd bit for bit."""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_lse, cuda, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

# (B, H, N, d, mask, window): all split (few tiles per slot)
CASES = [
    (1, 4, 4096, 64, "causal", 0),        # key-split layout (N >= 4096)
    (1, 2, 4173, 64, "prefix_lm", 2000),  # key-split layout, ragged last tile
    (1, 4, 2500, 64, "causal", 0),        # 32-row layout, ragged
    (2, 2, 2200, 64, "causal", 0),
    (1, 2, 2048, 128, "causal", 0),
    (1, 3, 1500, 128, "prefix_lm", 700),
    (1, 1, 4096, 64, "prefix_lm", 5000),  # window past N: every tile costs the same, all split
    (1, 1, 8192, 128, "causal", 0),       # one head
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_split_elementwise(case, out):
    B, H, N, d, mask, window = case
    ws_bytes = A.attn_fwd_split_workspace_size(B, H, N, d, "bf16", mask, window)
    assert ws_bytes > 0, "this shape must take the split path"
    say(f"split {case} out={out}: workspace {ws_bytes} B")
    seed = 41 + N + d
    q, k, v = wl.dense_inputs(B, H, N, d, seed=seed)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                   device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")    # NaN-poisoned partials
    A.attn_fwd_split(cuda(qb), cuda(kb), cuda(vb), o, scale, mask, window, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    win = window if mask == "prefix_lm" else None
    ref, ref_lse = oracle.attention(wl.bf16_to_f64(qb), wl.bf16_to_f64(kb), wl.bf16_to_f64(vb), scale, mask, win)
    err = check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse)
    say(f"split {case} out={out}: max abs err {err:.3g}")


@pytest.mark.parametrize("case", [(4, 16, 2048, 64, "causal", 0), (1, 16, 4096, 64, "causal", 0),
                                  (1, 2, 700, 128, "none", 0)],
                         ids=lambda c: "-".join(map(str, c)))
def test_unsplit_shapes_equal_attn_fwd(case):
    """With a workspace size of 0 the call is attn_fwd: same bytes out."""
    B, H, N, d, mask, window = case
    assert A.attn_fwd_split_workspace_size(B, H, N, d, "bf16", mask, window) == 0
    qd, kd, vd = wl.dense_inputs_device(B, H, N, d, seed=43)
    o1, o2 = torch.empty_like(qd), torch.empty_like(qd)
    A.attn_fwd(qd, kd, vd, o1, 1 / math.sqrt(d), mask, window)
    A.attn_fwd_split(qd, kd, vd, o2, 1 / math.sqrt(d), mask, window, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_split_without_lse_and_repeated():
    """No LSE asked for (the parts still keep theirs); two calls in a row on one
    workspace give the same bytes."""
    B, H, N, d = 1, 4, 3000, 64
    ws = torch.empty(A.attn_fwd_split_workspace_size(B, H, N, d, "bf16", "causal"), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() > 0
    qd, kd, vd = wl.dense_inputs_device(B, H, N, d, seed=47)
    o1, o2 = torch.empty_like(qd), torch.empty_like(qd)
    A.attn_fwd_split(qd, kd, vd, o1, 0.125, "causal", workspace=ws)
    A.attn_fwd_split(qd, kd, vd, o2, 0.125, "causal", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    rows = np.array([0, 1, 127, 128, 1500, 2047, 2048, 2999])
    ref, _ = oracle.attention(wl.bf16_to_f64(qd[0, 2].cpu()), wl.bf16_to_f64(kd[0, 2].cpu()),
                              wl.bf16_to_f64(vd[0, 2].cpu()), 0.125, "causal", rows=rows)
    check_close(to_np(o1[0, 2][rows]), ref, True, what="split, head 2")
