"""Seeded synthetic workloads for the attention forward path.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic. It is the one module that both the GPU path's
callers (tests, bench, smoke) and the CPU oracle's callers use, so that both
sides see the same bytes.

Shapes follow the workloads the pages discuss: seq 8192 / d 128 / 32 heads
("Flash MSA Attention Kernel Implementation Tutorial", "Performance
Benchmarks"), a 4096-token window ("Optimizing Triton kernels for custom
attention patterns on H100", Pattern B), 16-token KV pages (same page,
Pattern C) and 128-row fp8 blocks with outliers ("FlashAttention-3 ...",
"FP8 Block Quantization").

Recipe (all draws from ``numpy.random.default_rng(seed)``):
* dense: Q, K, V drawn in that order, ``standard_normal(shape, float32)``.
  With outliers, then three masks ``random(shape) < p`` (for Q, K, V in that
  order) scale the chosen entries by ``outlier_scale``.
* paged: the sequence lengths ``integers(l_min, l_max, endpoint=True)``, then
  Q [S, H, d] (or [S, H, q_len, d] for a prefill of the last q_len
  positions), then per sequence K_s and V_s [H, L_s, d], then a permutation
  of the P = sum ceil(L_s/16) + spare page ids, handed out in (sequence, slot)
  order. Unused rows of last pages and spare pages hold NaN; block-table
  entries past a sequence's last page hold -1.
* paged cross-attention: Q [S, H, q_len, d], the K pool, the V pool, then for
  each (sequence, 128-row query block) ``choice(pool_pages, pages_per_block,
  replace=False)`` and a cut ``integers(0, page_size)`` of tokens dropped from
  the end of its list; spare pages past the pool hold NaN, and no list names
  them.
* documents: document lengths ``integers(l_min, l_max, endpoint=True)`` from
  ``numpy.random.default_rng([seed, 1])`` (a stream apart from Q, K, V), drawn
  until they cover N; the last document is cut at N. The offsets are the
  running sums, starting at 0 and ending at N.
* bf16 values are the fp32 draws rounded to nearest-even once, on the host
  (``torch.Tensor.to(torch.bfloat16)``), before either side sees them.
"""

from dataclasses import dataclass, field
import hashlib

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    kind: str                      # "dense" | "paged" | "fp8"
    B: int = 1
    H: int = 1
    N: int = 1
    d: int = 64
    dtype: str = "bf16"            # input dtype of Q/K/V for dense
    out_dtype: str = "bf16"
    mask: str = "none"
    window: int = 0
    n_seq: int = 0
    l_min: int = 0
    l_max: int = 0
    page_size: int = 16
    spare_pages: int = 64
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    qk_block: int = 128
    q_len: int = 0                 # paged prefill / cross: query rows per sequence
    pool_pages: int = 0            # paged cross: pages in the pool
    pages_per_block: int = 0       # paged cross: pages each query block lists
    extra: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    1: Workload(1, "dense_f32_b1_h1_n256_d64", "dense", B=1, H=1, N=256, d=64,
                dtype="f32", out_dtype="f32", mask="none"),
    2: Workload(2, "causal_bf16_b4_h16_n2048_d64", "dense", B=4, H=16, N=2048, d=64,
                mask="causal"),
    3: Workload(3, "sliding4096_bf16_b2_h32_n8192_d128", "dense", B=2, H=32, N=8192, d=128,
                mask="sliding", window=4096),
    4: Workload(4, "paged_decode_bf16_s64_h32_d128_p16_l512to8192", "paged", H=32, d=128,
                n_seq=64, l_min=512, l_max=8192),
    5: Workload(5, "fp8_causal_b1_h16_n16384_d128", "fp8", B=1, H=16, N=16384, d=128,
                mask="causal", outlier_p=0.01, outlier_scale=20.0),
    # structured masks ("Optimizing Triton kernels ...", Patterns A and B):
    # documents of 256..4096 tokens packed into 16K positions, the same as a
    # packed batch of causal sequences, a +-4096 window over 32K positions,
    # a 2048-token prefix, and the unmasked 16K shape the document kernel is
    # compared with
    6: Workload(6, "document_bf16_b1_h16_n16384_d128_docs256to4096", "dense", B=1, H=16, N=16384, d=128,
                mask="document", l_min=256, l_max=4096),
    7: Workload(7, "varlen_causal_bf16_b1_h16_n16384_d128_seqs256to4096", "dense", B=1, H=16, N=16384,
                d=128, mask="document_causal", l_min=256, l_max=4096),
    8: Workload(8, "band4096_bf16_b1_h16_n32768_d128", "dense", B=1, H=16, N=32768, d=128,
                mask="band", window=4096),
    9: Workload(9, "prefix_lm2048_bf16_b2_h16_n8192_d128", "dense", B=2, H=16, N=8192, d=128,
                mask="prefix_lm", window=2048),
    10: Workload(10, "dense_bf16_b1_h16_n16384_d128", "dense", B=1, H=16, N=16384, d=128, mask="none"),
    # paged K/V with 64-token pages ("Optimizing Triton kernels ...", Pattern
    # C): the last 512 positions of 16 cached sequences of 1K..8K tokens, and
    # 8 x 8 query blocks each reading 32 pages picked from a 1024-page pool
    11: Workload(11, "paged_prefill_bf16_s16_h32_d128_p64_q512_l1024to8192", "paged_prefill", H=32, d=128,
                 n_seq=16, l_min=1024, l_max=8192, page_size=64, q_len=512),
    12: Workload(12, "paged_cross_bf16_s8_h32_d128_p64_q1024_32of1024pages", "paged_cross", H=32, d=128,
                 n_seq=8, page_size=64, q_len=1024, pool_pages=1024, pages_per_block=32, spare_pages=16),
    # the fp8 causal shape with V in fp8 too (power-of-two block scales) and P
    # rounded to fp8 for the second product
    13: Workload(13, "fp8_full_causal_b1_h16_n16384_d128", "fp8_full", B=1, H=16, N=16384, d=128,
                 mask="causal", outlier_p=0.01, outlier_scale=20.0),
    # the paged prefill of workload 11 over the decode's 16-token pages
    14: Workload(14, "paged_prefill_bf16_s16_h32_d128_p16_q512_l1024to8192", "paged_prefill", H=32, d=128,
                 n_seq=16, l_min=1024, l_max=8192, page_size=16, q_len=512),
    # the decode of workload 4 over 64-token pages
    15: Workload(15, "paged_decode_bf16_s64_h32_d128_p64_l512to8192", "paged", H=32, d=128,
                 n_seq=64, l_min=512, l_max=8192, page_size=64),
}


def default_seed(key):
    return 1000 + int(key)


def to_bf16(x):
    """fp32 numpy array -> torch bfloat16 tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f64(t):
    """Exact upcast of a bf16 torch tensor to a float64 numpy array."""
    return t.to(torch.float32).numpy().astype(np.float64)


def dense_inputs(B, H, N, d, seed, outlier_p=0.0, outlier_scale=1.0):
    """Q, K, V fp32 arrays [B, H, N, d]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if outlier_p > 0:
        for x in (q, k, v):
            sel = rng.random(shape) < outlier_p
            x[sel] *= np.float32(outlier_scale)
    return q, k, v


def dense_inputs_device(B, H, N, d, seed, device="cuda"):
    """Q, K, V bf16 [B, H, N, d], N(0,1) drawn on the device by a seeded torch
    generator, for tensors too large to draw on the host. The kernels read
    them there; the oracle reads host copies of some heads of the same
    tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return tuple(torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
                 for _ in range(3))


def document_offsets(N, l_min, l_max, seed):
    """Document start offsets int32 [num_docs + 1] covering N positions."""
    rng = np.random.default_rng([seed, 1])
    offs = [0]
    while offs[-1] < N:
        offs.append(min(N, offs[-1] + int(rng.integers(l_min, l_max, endpoint=True))))
    return np.array(offs, dtype=np.int32)


@dataclass
class PagedInputs:
    q: torch.Tensor               # [S, H, d] bf16
    k_pool: torch.Tensor          # [P, H, page, d] bf16
    v_pool: torch.Tensor
    block_table: torch.Tensor     # [S, max_pages] int32, -1 padded
    seq_lens: torch.Tensor        # [S] int32
    page_size: int
    k_dense: list = None          # per sequence [H, L_s, d] bf16 (if kept)
    v_dense: list = None


def paged_inputs(n_seq, H, d, l_min, l_max, seed, page_size=16, spare=64, max_pages=None,
                 keep_dense=False, q_rows=None):
    """A shuffled paged KV pool with per-sequence block tables. Q is [S, H, d]
    (one decode query per sequence), or [S, H, q_rows, d] for a prefill of the
    last q_rows positions."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(l_min, l_max, size=n_seq, endpoint=True).astype(np.int64)
    q = rng.standard_normal((n_seq, H, d) if q_rows is None else (n_seq, H, q_rows, d), dtype=np.float32)
    pages_per_seq = (lens + page_size - 1) // page_size
    if max_pages is None:
        max_pages = -(-l_max // page_size)
    n_pages = int(pages_per_seq.sum()) + spare
    k_pool = torch.full((n_pages, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    v_pool = torch.full((n_pages, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    k_dense, v_dense = [], []
    for s in range(n_seq):
        ks = rng.standard_normal((H, int(lens[s]), d), dtype=np.float32)
        vs = rng.standard_normal((H, int(lens[s]), d), dtype=np.float32)
        k_dense.append(to_bf16(ks))
        v_dense.append(to_bf16(vs))
    perm = rng.permutation(n_pages)
    table = np.full((n_seq, max_pages), -1, dtype=np.int32)
    cursor = 0
    for s in range(n_seq):
        np_s = int(pages_per_seq[s])
        ids = perm[cursor:cursor + np_s]
        cursor += np_s
        table[s, :np_s] = ids
        length = int(lens[s])
        for src, pool in ((k_dense[s], k_pool), (v_dense[s], v_pool)):
            padded = torch.full((H, np_s * page_size, d), float("nan"), dtype=torch.bfloat16)
            padded[:, :length] = src
            pool[torch.from_numpy(ids.astype(np.int64))] = padded.view(H, np_s, page_size, d).transpose(0, 1)
    out = PagedInputs(q=to_bf16(q), k_pool=k_pool, v_pool=v_pool,
                      block_table=torch.from_numpy(table), seq_lens=torch.from_numpy(lens.astype(np.int32)),
                      page_size=page_size)
    if keep_dense:
        out.k_dense, out.v_dense = k_dense, v_dense
    return out


@dataclass
class CrossInputs:
    q: torch.Tensor               # [S, H, q_len, d] bf16
    k_pool: torch.Tensor          # [P, H, page, d] bf16
    v_pool: torch.Tensor
    page_table: torch.Tensor      # [S, QB, max_pages] int32, -1 padded
    kv_lens: torch.Tensor         # [S, QB] int32
    page_size: int
    q_block: int


def paged_cross_inputs(n_seq, H, d, q_len, pool_pages, pages_per_block, seed, page_size=64, q_block=128,
                       spare=16, ragged=True):
    """Block-sparse paged cross-attention inputs: a pool of pool_pages pages of
    random keys/values (plus `spare` NaN-poisoned pages no list names), and for
    each query block of each sequence a list of pages_per_block distinct pages
    drawn without replacement; with `ragged`, the block attends to all but the
    last 0..page_size-1 tokens of its list. Draw order: Q, K pool, V pool, then
    per (sequence, block) the page choice and the cut."""
    rng = np.random.default_rng(seed)
    n_qb = -(-q_len // q_block)
    q = rng.standard_normal((n_seq, H, q_len, d), dtype=np.float32)
    kp = rng.standard_normal((pool_pages, H, page_size, d), dtype=np.float32)
    vp = rng.standard_normal((pool_pages, H, page_size, d), dtype=np.float32)
    k_pool = torch.full((pool_pages + spare, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    v_pool = torch.full((pool_pages + spare, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    k_pool[:pool_pages] = to_bf16(kp)
    v_pool[:pool_pages] = to_bf16(vp)
    table = np.full((n_seq, n_qb, pages_per_block), -1, dtype=np.int32)
    lens = np.zeros((n_seq, n_qb), dtype=np.int32)
    for s in range(n_seq):
        for b in range(n_qb):
            table[s, b] = rng.choice(pool_pages, size=pages_per_block, replace=False)
            cut = int(rng.integers(0, page_size)) if ragged else 0
            lens[s, b] = pages_per_block * page_size - cut
    return CrossInputs(q=to_bf16(q), k_pool=k_pool, v_pool=v_pool, page_table=torch.from_numpy(table),
                       kv_lens=torch.from_numpy(lens), page_size=page_size, q_block=q_block)


def tensor_digest(*tensors):
    """Short hash of the raw bytes of the given CPU tensors / arrays."""
    h = hashlib.sha256()
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t = t.contiguous().view(torch.uint8).numpy() if t.dtype != torch.uint8 else t.contiguous().numpy()
        h.update(np.ascontiguousarray(t).tobytes())
    return h.hexdigest()[:16]
