"""Calls enqueue on the stream they are given and keep no state between
calls: launches on two streams at once, and from two host threads at once,
give each call's single-stream result bit for bit."""

import math
import threading

import pytest
import torch

from parity import say
from tiled_attention_amd import _lib as A
from tiled_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _cases():
    """Three calls of different kinds and sizes: causal d=64, sliding d=128, decode."""
    q, k, v = (wl.to_bf16(x).cuda() for x in wl.dense_inputs(2, 4, 1500, 64, seed=3))
    q2, k2, v2 = (wl.to_bf16(x).cuda() for x in wl.dense_inputs(1, 8, 3000, 128, seed=4))
    inp = wl.paged_inputs(n_seq=8, H=4, d=128, l_min=100, l_max=3000, seed=5)
    kp, vp, bt, lens, qd = (x.cuda() for x in (inp.k_pool, inp.v_pool, inp.block_table, inp.seq_lens, inp.q))
    ws = torch.empty(A.attn_decode_paged_workspace_size(8, 4, 128, bt.shape[1], 16), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty_like(q), torch.empty_like(q2), torch.empty_like(qd)]

    def run(i, stream):
        if i == 0:
            A.attn_fwd(q, k, v, outs[0], 0.125, "causal", stream=stream)
        elif i == 1:
            A.attn_fwd(q2, k2, v2, outs[1], 1.0 / math.sqrt(128), "sliding", 700, stream=stream)
        else:
            A.attn_decode_paged(qd, kp, vp, bt, lens, outs[2], 1.0 / math.sqrt(128), workspace=ws, stream=stream)
    return run, outs


def _references(run, outs):
    refs = []
    for i in range(len(outs)):
        run(i, None)
        torch.cuda.synchronize()
        refs.append(outs[i].clone())
    return refs


def test_concurrent_streams_match_single_stream():
    run, outs = _cases()
    refs = _references(run, outs)
    streams = [torch.cuda.Stream() for _ in outs]
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                run(i, s)
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, refs)):
            assert torch.equal(t.view(torch.int16), r.view(torch.int16)), f"call {i}, repetition {rep}"
    say("three calls on three streams: bit-identical to single-stream runs")


def test_calls_from_two_host_threads():
    run, outs = _cases()
    refs = _references(run, outs)
    for t in outs:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    errors = []

    def worker(indices):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in indices:
                    run(i, s)
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=([0, 2],)), threading.Thread(target=worker, args=([1],))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not any(th.is_alive() for th in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (t, r) in enumerate(zip(outs, refs)):
        assert torch.equal(t.view(torch.int16), r.view(torch.int16)), f"call {i}"
