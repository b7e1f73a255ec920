"""The seeded generators are deterministic and lay data out as documented."""

import numpy as np
import torch

from tiled_attention_amd import workloads as wl


def test_dense_inputs_deterministic_per_seed():
    a = wl.dense_inputs(1, 2, 33, 8, seed=5)
    b = wl.dense_inputs(1, 2, 33, 8, seed=5)
    c = wl.dense_inputs(1, 2, 33, 8, seed=6)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    assert wl.tensor_digest(*a) == wl.tensor_digest(*b)
    assert all(x.dtype == np.float32 and x.shape == (1, 2, 33, 8) for x in a)


def test_outlier_fraction():
    q, k, v = wl.dense_inputs(1, 4, 1024, 64, seed=9, outlier_p=0.01, outlier_scale=20.0)
    base_q, _, _ = wl.dense_inputs(1, 4, 1024, 64, seed=9)
    ratio = np.abs(q) / np.maximum(np.abs(base_q), 1e-30)
    frac = np.mean(np.isclose(ratio, 20.0))
    assert 0.008 < frac < 0.012


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -3.0000001], dtype=np.float32)
    got = wl.to_bf16(x).view(torch.int16).numpy().astype(np.uint16)
    # 1+2^-8 is a tie between 0x3F80 and 0x3F81 -> even 0x3F80; 1+3*2^-8 ties -> 0x3F82
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F80, 0xC040]
    assert np.array_equal(wl.bf16_to_f64(wl.to_bf16(x)), wl.to_bf16(x).float().numpy())


def test_paged_inputs_deterministic():
    a = wl.paged_inputs(3, 2, 8, 5, 50, seed=1, spare=2)
    b = wl.paged_inputs(3, 2, 8, 5, 50, seed=1, spare=2)
    assert wl.tensor_digest(a.q, a.k_pool, a.v_pool, a.block_table, a.seq_lens) == \
        wl.tensor_digest(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens)
    assert a.block_table.dtype == torch.int32 and a.seq_lens.dtype == torch.int32
    assert a.block_table.shape == (3, 4)          # ceil(50 / 16)
    assert a.k_pool.shape[1:] == (2, 16, 8)


def test_workload_table():
    assert set(wl.WORKLOADS) == set(range(1, 16))
    assert wl.WORKLOADS[14].page_size == 16 and wl.WORKLOADS[11].page_size == 64
    w = wl.WORKLOADS[3]
    assert (w.B, w.H, w.N, w.d, w.mask, w.window) == (2, 32, 8192, 128, "sliding", 4096)
    assert abs(wl.WORKLOADS[2].scale - 0.125) == 0


def test_document_offsets_recipe():
    """Offsets start at 0, end at N, every document but the last has a length
    drawn from [l_min, l_max], and the draw is deterministic per seed."""
    for N, lo, hi, seed in ((16384, 256, 4096, 1006), (100, 1, 7, 3), (5, 10, 20, 1)):
        o = wl.document_offsets(N, lo, hi, seed)
        assert o.dtype == np.int32 and o[0] == 0 and o[-1] == N
        lens = np.diff(o)
        assert np.all(lens[:-1] >= lo) and np.all(lens <= hi) and lens[-1] >= 1
        assert np.array_equal(o, wl.document_offsets(N, lo, hi, seed))
