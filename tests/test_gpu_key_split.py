"""GPU parity of the bf16 d = 64 key-split layout (sequences of 4096 keys and
more: each wave takes 64 rows and one 32-key half of every K/V tile, and the
two waves that share rows merge their partial states at the end) against the
oracle, element by element, under every mask kind, with ragged lengths and
both output types."""

import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, check_lse, cuda, say, to_np
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

# (N, mask, window, document layout)
CASES = [
    (4096, "none", 0, None), (4173, "causal", 0, None), (4096, "causal", 0, None),
    (4100, "sliding", 300, None), (4096, "sliding", 1, None), (4133, "band", 200, None),
    (4096, "prefix_lm", 1000, None), (4150, "document", 0, "random"),
    (4096, "document_causal", 0, "random"), (4097, "document", 0, "empty"),
    (4096, "document_causal", 0, "singles"),
]


def _offsets(N, layout, seed):
    if layout is None:
        return None
    if layout == "random":
        return wl.document_offsets(N, 5, N // 3, seed)
    if layout == "singles":
        return np.arange(N + 1)
    rng = np.random.default_rng(seed)                     # "empty": empty documents, first and last too
    cuts = sorted(rng.integers(1, N, size=6).tolist())
    return np.array([0, 0] + sorted(cuts + cuts[:2]) + [N, N])


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_key_split_elementwise(case, out):
    N, mask, window, layout = case
    B, H, d = 1, 2, 64
    say(f"key split {case} out={out}")
    seed = 31 + N
    q, k, v = wl.dense_inputs(B, H, N, d, seed=seed)
    qb, kb, vb = wl.to_bf16(q), wl.to_bf16(k), wl.to_bf16(v)
    offs = _offsets(N, layout, seed)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                   device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    doc = None if offs is None else torch.from_numpy(offs.astype(np.int32)).cuda()
    A.attn_fwd(cuda(qb), cuda(kb), cuda(vb), o, scale, mask, window, doc_offsets=doc, lse=lse)
    torch.cuda.synchronize()
    win = window if mask in ("sliding", "band", "prefix_lm") else None
    ref, ref_lse = oracle.attention(wl.bf16_to_f64(qb), wl.bf16_to_f64(kb), wl.bf16_to_f64(vb), scale, mask, win,
                                    doc_offsets=offs)
    err = check_close(to_np(o), ref, out == "bf16", what=str(case))
    check_lse(to_np(lse), ref_lse)
    say(f"key split {case} out={out}: max abs err {err:.3g}")
