#!/usr/bin/env python3
"""Benchmark of the flash-attention forward path on one MI355X.

A step is one attn_fwd call over the causal bf16 prefill workload
(B=4, H=16, N=2048, d=64, fp32 accumulate, bf16 out) with inputs resident in
HBM. `value` is algorithmic TFLOP/s over the K timed steps (wall clock,
synchronised on both sides); the flop count is 4*d per visible (query, key)
pair, so masked pairs the method skips are not counted. The JSON line also
carries:
  roofline     -- the attention kernel's average launch time from HIP events
                  on its stream around the timed steps, as achieved TFLOP/s
                  against the dense bf16 MFMA peak (and the spread of
                  launches timed one by one between their own events), plus
                  measured HBM traffic when the committed counter summary
                  matches the current kernel source;
  cpu_baseline -- the fp64 CPU oracle timed on a bounded sample of the same
                  workload, on this host's cores;
  workloads    -- the other workloads (fp32 single head, sliding window,
                  paged decode in GB/s, fp8 causal, documents, packed causal
                  sequences, two-sided window, prefix-LM and the unmasked
                  shape the document masks are compared with), each timed
                  with HIP events.
With --sweep it instead prints one JSON line of bf16 prefill rates over
sequence length (causal and unmasked, d = 64 and 128, 16 heads), for context
beside the fixed workloads. One GPU only: --gpus above 1 exits with a message.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # fp32 vector
PEAK_HBM_GBS = 8000.0          # HBM3E
METRIC = "attention fwd TFLOPS and % of MI355X MFMA peak; paged decode GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock.json")
KERNEL_SOURCES = ["tiled_attention_amd/csrc/fwd_mfma.hip", "tiled_attention_amd/csrc/attn_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(mask, n, window, offs=None):
    """Visible (query, key) pairs of one n x n head (closed forms per mask)."""
    if mask == "none":
        return n * n
    if mask == "causal" or (mask == "sliding" and window >= n):
        return n * (n + 1) // 2
    if mask == "sliding":
        return window * (window + 1) // 2 + (n - window) * window
    if mask == "band":
        w = min(window, n - 1)
        return (2 * w + 1) * n - w * (w + 1)
    if mask == "prefix_lm":
        p = min(window, n)
        return p * p + (n * (n + 1) - p * (p + 1)) // 2
    lens = [int(b) - int(a) for a, b in zip(offs[:-1], offs[1:])]
    if mask == "document":
        return sum(x * x for x in lens)
    return sum(x * (x + 1) // 2 for x in lens)     # document_causal


class Dense:
    """An attn_fwd workload (any mask) with device-resident inputs."""

    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        self.w = w = wl.WORKLOADS[key]
        self.seed = seed
        q, k, v = wl.dense_inputs(w.B, w.H, w.N, w.d, seed=seed)
        if w.dtype == "f32":
            self.q, self.k, self.v = (torch.from_numpy(x).cuda() for x in (q, k, v))
        else:
            self.q, self.k, self.v = (wl.to_bf16(x).cuda() for x in (q, k, v))
        self.o = torch.empty(self.q.shape, dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16,
                             device="cuda")
        self.offs = wl.document_offsets(w.N, w.l_min, w.l_max, seed) if w.mask in A.DOC_MASKS else None
        self.doc = None if self.offs is None else torch.from_numpy(self.offs).cuda()
        self.flops = 4.0 * w.d * visible_pairs(w.mask, w.N, w.window, self.offs) * w.B * w.H
        lib = A.load()
        dt = A.ATTN_F32 if w.dtype == "f32" else A.ATTN_BF16
        odt = A.ATTN_F32 if w.out_dtype == "f32" else A.ATTN_BF16
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = (ctypes.c_void_p(self.q.data_ptr()), ctypes.c_void_p(self.k.data_ptr()),
                ctypes.c_void_p(self.v.data_ptr()), ctypes.c_void_p(self.o.data_ptr()),
                w.B, w.H, w.N, w.d, dt, odt, w.scale, A.MASKS[w.mask], w.window,
                None if self.doc is None else ctypes.c_void_p(self.doc.data_ptr()),
                0 if self.offs is None else len(self.offs) - 1, None, stream)
        fn = lib.attn_fwd

        def step():
            st = fn(*args)
            if st != 0:
                raise RuntimeError(A.attn_status_str(st))
        self.step = step

    def describe(self):
        w = self.w
        d = {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N, "head_dim": w.d,
             "mask": w.mask, "window": w.window or None, "in_dtype": w.dtype, "out_dtype": w.out_dtype,
             "seed": self.seed}
        if self.offs is not None:
            d["documents"] = len(self.offs) - 1
            d["document_lengths"] = [w.l_min, w.l_max]
        return d


class Fp8:
    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        self.w = w = wl.WORKLOADS[key]
        self.seed = seed
        q, k, v = wl.dense_inputs(w.B, w.H, w.N, w.d, seed=seed, outlier_p=w.outlier_p,
                                  outlier_scale=w.outlier_scale)
        nb = -(-w.N // 128)
        self.q8 = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
        self.k8 = torch.empty_like(self.q8)
        self.sq = torch.empty((w.B, w.H, nb), dtype=torch.float32, device="cuda")
        self.sk = torch.empty_like(self.sq)
        A.attn_quant_fp8_block(torch.from_numpy(q).cuda(), self.q8, self.sq)
        A.attn_quant_fp8_block(torch.from_numpy(k).cuda(), self.k8, self.sk)
        self.v = wl.to_bf16(v).cuda()
        self.o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        self.flops = 4.0 * w.d * visible_pairs(w.mask, w.N, w.window) * w.B * w.H

        def step():
            A.attn_fwd_fp8(self.q8, self.sq, self.k8, self.sk, self.v, self.o, w.scale, w.mask)
        self.step = step

    def describe(self):
        w = self.w
        return {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N, "head_dim": w.d,
                "mask": w.mask, "qk": "e4m3fn, fp32 scale per 128 rows", "v": "bf16", "seed": self.seed}


class Fp8Full(Fp8):
    """attn_fwd_fp8_full: V in fp8 as well (power-of-two block scales)."""

    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        super().__init__(key, seed)
        w = self.w
        v = wl.dense_inputs(w.B, w.H, w.N, w.d, seed=seed, outlier_p=w.outlier_p, outlier_scale=w.outlier_scale)[2]
        self.v8 = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
        self.sv = torch.empty_like(self.sq)
        A.attn_quant_fp8_block_pow2(torch.from_numpy(v).cuda(), self.v8, self.sv)
        torch.cuda.synchronize()

        def step():
            A.attn_fwd_fp8_full(self.q8, self.sq, self.k8, self.sk, self.v8, self.sv, self.o, w.scale, w.mask)
        self.step = step

    def describe(self):
        d = super().describe()
        d["v"] = "e4m3fn, power-of-two scale per 128 rows"
        d["p"] = "e4m3fn"
        return d


class Paged:
    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        self.w = w = wl.WORKLOADS[key]
        self.seed = seed
        inp = wl.paged_inputs(w.n_seq, w.H, w.d, w.l_min, w.l_max, seed=seed, page_size=w.page_size,
                              spare=w.spare_pages)
        self.q = inp.q.cuda()
        self.kp, self.vp = inp.k_pool.cuda(), inp.v_pool.cuda()
        self.bt, self.lens = inp.block_table.cuda(), inp.seq_lens.cuda()
        self.o = torch.empty(self.q.shape, dtype=torch.bfloat16, device="cuda")
        nbytes = A.attn_decode_paged_workspace_size(w.n_seq, w.H, w.d, self.bt.shape[1], w.page_size)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        lens = inp.seq_lens.numpy().astype(int)
        self.tokens = int(lens.sum())
        pages = int(((lens + w.page_size - 1) // w.page_size).sum())
        # compulsory bytes: every cached K and V element once, Q and O once, the page ids used, the lengths
        self.bytes = (2.0 * self.tokens * w.H * w.d * 2 + 2.0 * w.n_seq * w.H * w.d * 2 + pages * 4 + w.n_seq * 4)
        self.flops = 4.0 * w.d * self.tokens * w.H

        def step():
            A.attn_decode_paged(self.q, self.kp, self.vp, self.bt, self.lens, self.o, w.scale, workspace=self.ws)
        self.step = step

    def describe(self):
        w = self.w
        return {"workload": w.name, "sequences": w.n_seq, "heads": w.H, "head_dim": w.d,
                "page_size": w.page_size, "kv_len": [w.l_min, w.l_max], "kv_tokens": self.tokens,
                "seed": self.seed}


class PagedPrefill:
    """attn_prefill_paged over a paged pool (16- or 64-token pages); also times
    the page gather a two-stage (gather, then attend) route would add."""

    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        self.w = w = wl.WORKLOADS[key]
        self.seed = seed
        inp = wl.paged_inputs(w.n_seq, w.H, w.d, w.l_min, w.l_max, seed=seed, page_size=w.page_size,
                              spare=w.spare_pages, q_rows=w.q_len)
        self.q = inp.q.cuda()
        self.kp, self.vp = inp.k_pool.cuda(), inp.v_pool.cuda()
        self.bt, self.lens = inp.block_table.cuda(), inp.seq_lens.cuda()
        self.o = torch.empty(self.q.shape, dtype=torch.bfloat16, device="cuda")
        lens = inp.seq_lens.numpy().astype(int)
        self.tokens = int(lens.sum())
        # visible pairs: row i of sequence s sees L_s - q_len + i + 1 keys
        pairs = sum(w.q_len * (L - w.q_len) + w.q_len * (w.q_len + 1) // 2 for L in lens)
        self.flops = 4.0 * w.d * pairs * w.H
        max_tok = self.bt.shape[1] * w.page_size
        self.k_out = torch.empty((w.n_seq, w.H, max_tok, w.d), dtype=torch.bfloat16, device="cuda")
        self.v_out = torch.empty_like(self.k_out)
        self.gather_bytes = 2.0 * 2 * self.tokens * w.H * w.d * 2      # K and V, read and written

        def step():
            A.attn_prefill_paged(self.q, self.kp, self.vp, self.bt, self.lens, self.o, w.scale)

        def gather():
            A.attn_gather_paged(self.kp, self.vp, self.bt, self.lens, self.k_out, self.v_out)
        # the two-stage route's attention: the gathered copies read as a pool
        # of contiguous 64-token pages with one head per (sequence, head)
        # slice and an identity block table
        two = two_stage_views(self.q, self.k_out, self.v_out, self.lens, w.H)
        self.o2 = torch.empty_like(self.o)

        def attend_gathered():
            A.attn_prefill_paged(two["q"], two["k"], two["v"], two["table"], two["lens"], self.o2.view(two["q"].shape),
                                 w.scale)

        def two_stage():
            gather()
            attend_gathered()
        self.step = step
        self.gather = gather
        self.attend_gathered = attend_gathered
        self.two_stage = two_stage

    def describe(self):
        w = self.w
        return {"workload": w.name, "sequences": w.n_seq, "heads": w.H, "head_dim": w.d, "page_size": w.page_size,
                "q_len": w.q_len, "kv_len": [w.l_min, w.l_max], "kv_tokens": self.tokens, "seed": self.seed}


def two_stage_views(q, k_out, v_out, lens, H):
    """Views that let the paged prefill read the gather's dense output: the
    copies [S, H, T, d] are a pool of S*H*T/64 contiguous 64-token pages with
    one head, sequence-head j owns pages j*T/64 .. (j+1)*T/64 - 1 (an identity
    table), Q is [S*H, 1, q_len, d] and each sequence-head keeps its
    sequence's length."""
    import torch
    S, _, T, d = k_out.shape
    per = T // 64
    pages = S * H * per
    table = torch.arange(pages, dtype=torch.int32, device=k_out.device).view(S * H, per)
    return {"q": q.view(S * H, 1, q.shape[2], d), "k": k_out.view(pages, 1, 64, d), "v": v_out.view(pages, 1, 64, d),
            "table": table, "lens": lens.repeat_interleave(H).contiguous()}


class PagedCross:
    """attn_cross_paged: every 128-row query block over its own page list."""

    def __init__(self, key, seed):
        import torch
        from tiled_attention_amd import _lib as A
        from tiled_attention_amd import workloads as wl
        self.w = w = wl.WORKLOADS[key]
        self.seed = seed
        inp = wl.paged_cross_inputs(w.n_seq, w.H, w.d, w.q_len, w.pool_pages, w.pages_per_block, seed=seed,
                                    page_size=w.page_size, spare=w.spare_pages)
        self.q = inp.q.cuda()
        self.kp, self.vp = inp.k_pool.cuda(), inp.v_pool.cuda()
        self.table, self.lens = inp.page_table.cuda(), inp.kv_lens.cuda()
        self.o = torch.empty(self.q.shape, dtype=torch.bfloat16, device="cuda")
        lens = inp.kv_lens.numpy().astype(int)
        rows = [min(128, w.q_len - 128 * b) for b in range(lens.shape[1])]
        self.flops = 4.0 * w.d * w.H * sum(int(lens[s, b]) * rows[b] for s in range(lens.shape[0])
                                            for b in range(lens.shape[1]))

        def step():
            A.attn_cross_paged(self.q, self.kp, self.vp, self.table, self.lens, self.o, w.scale)
        self.step = step

    def describe(self):
        w = self.w
        return {"workload": w.name, "sequences": w.n_seq, "heads": w.H, "head_dim": w.d, "page_size": w.page_size,
                "q_len": w.q_len, "pool_pages": w.pool_pages, "pages_per_query_block": w.pages_per_block,
                "seed": self.seed}


def event_time_ms(step, reps, warmup=3, settle_ms=30.0):
    """Average, median, minimum and 90th-percentile duration (ms) of one step
    from HIP events on the launch stream, after `warmup` calls and then
    enough further calls to keep the GPU busy for about settle_ms (at most
    300): a workload's first launches run slower (clock ramp, first touches
    of its buffers)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(min(300, int(settle_ms / max(one_ms, 1e-3)))):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    times = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(times) / len(times), times[len(times) // 2], times[0], times[min(len(times) - 1, (9 * len(times)) // 10)]


def environment():
    """ROCm, HIP and torch versions and the device name."""
    import torch
    env = {"torch": torch.__version__, "hip": torch.version.hip, "device": torch.cuda.get_device_name(0)}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    return env


def smi_snapshot():
    """The GPUs' current clocks and power as rocm-smi reports them ({card:
    {field: value}} for the fields naming a clock or power), or the reason
    they could not be read. Read-only; runs rocm-smi as a child process."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:  # no rocm-smi, no JSON, or a time-out: say so in the line
        return {"error": f"{type(e).__name__}: {str(e)[:160]}"}
    out = {}
    for card, fields in data.items():
        if isinstance(fields, dict):
            keep = {k: v for k, v in fields.items() if any(t in k.lower() for t in ("sclk", "mclk", "fclk", "power"))}
            if keep:
                out[card] = keep
    return out


def batch_time_ms(step, reps, groups=10, warmup=3, settle_ms=30.0):
    """Average, median, minimum and 90th-percentile time (ms) per launch,
    from `groups` groups of back-to-back launches, each group between one
    pair of HIP events on the launch stream (so the events' own time is
    spread over the group), after the same settling as event_time_ms."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(min(300, int(settle_ms / max(one_ms, 1e-3)))):
        step()
    torch.cuda.synchronize()
    n = max(1, reps // groups)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(groups)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(groups)]
    for g in range(groups):
        starts[g].record()
        for _ in range(n):
            step()
        ends[g].record()
    torch.cuda.synchronize()
    times = sorted(s_.elapsed_time(e) / n for s_, e in zip(starts, ends))
    return sum(times) / len(times), times[len(times) // 2], times[0], times[min(len(times) - 1, (9 * len(times)) // 10)]


def _threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def cpu_baseline(wk, budget_s=12.0):
    """The oracle, untouched, on a bounded sample (whole heads) of a dense workload."""
    import numpy as np
    import oracle
    w = wk.w
    q = wk.q.float().cpu().numpy().reshape(-1, w.N, w.d).astype(np.float64)
    k = wk.k.float().cpu().numpy().reshape(-1, w.N, w.d).astype(np.float64)
    v = wk.v.float().cpu().numpy().reshape(-1, w.N, w.d).astype(np.float64)
    heads, t0 = 0, time.perf_counter()
    while True:          # whole heads, in order, wrapping around, until the budget is spent
        h = heads % q.shape[0]
        oracle.attention(q[h], k[h], v[h], w.scale, w.mask, w.window or None, doc_offsets=wk.offs)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * visible_pairs(w.mask, w.N, w.window, wk.offs) * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{heads} head evaluations (heads of {w.name} in order, {q.shape[0]} per pass), "
                      f"fp64, {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_fp8(wk, budget_s=12.0):
    """The oracle on the fp8 workload: dequantise a head's Q and K codes (times
    their block scales) and attend in fp64, whole heads until the budget."""
    import numpy as np
    import oracle
    w = wk.w
    q8, k8 = wk.q8.cpu().numpy().reshape(-1, w.N, w.d), wk.k8.cpu().numpy().reshape(-1, w.N, w.d)
    sq, sk = wk.sq.cpu().numpy().reshape(q8.shape[0], -1), wk.sk.cpu().numpy().reshape(q8.shape[0], -1)
    v = wk.v.float().cpu().numpy().reshape(-1, w.N, w.d).astype(np.float64)
    heads, t0 = 0, time.perf_counter()
    while True:
        h = heads % q8.shape[0]
        qh = oracle.dequantize_blocks(q8[h], sq[h])
        kh = oracle.dequantize_blocks(k8[h], sk[h])
        oracle.attention(qh, kh, v[h], w.scale, w.mask)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * visible_pairs(w.mask, w.N, w.window) * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{heads} head evaluations of {w.name} (dequantise Q and K, then attend), fp64, {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_decode(wk, budget_s=12.0):
    """The oracle's decode, whole sequences in order until the budget; GB/s on
    the same algorithmic bytes as the GPU line (the pools' upcast to host
    arrays is input preparation, outside the timed region)."""
    import numpy as np
    import oracle
    w = wk.w
    q = wk.q.float().cpu().numpy().astype(np.float64)
    kp, vp = wk.kp.float().cpu().numpy(), wk.vp.float().cpu().numpy()
    bt, lens = wk.bt.cpu().numpy(), wk.lens.cpu().numpy()
    seqs, nbytes, t0 = 0, 0.0, time.perf_counter()
    while True:
        s = seqs % q.shape[0]
        oracle.decode(q[s:s + 1], kp, vp, bt[s:s + 1], lens[s:s + 1], w.scale, page_size=w.page_size)
        L = int(lens[s])
        nbytes += 2.0 * L * w.H * w.d * 2 + 2.0 * w.H * w.d * 2 + -(-L // w.page_size) * 4 + 4
        seqs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{seqs} sequences of {w.name} in order (all {w.H} heads each), fp64, {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def settle(step, ms=40.0):
    """Untimed launches until about `ms` of back-to-back GPU work has run:
    the clock rises over the first milliseconds of load (a 50 us kernel's
    first 100-200 launches run about 15% slower)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < ms * 1e-3:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def traffic_for(digest):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def clock_for(digest):
    """Shader clock (GHz) of the main kernel under load, as (lower, upper)
    bounds from a committed counter pass: busy cycles per shader engine over
    the dispatch time, and the counting window's cycles per XCD over the
    dispatch time. None once the kernel source has changed."""
    try:
        with open(CLOCK_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != digest or "clock_ghz" not in t:
        return None
    return t["clock_ghz"], t.get("clock_ghz_upper", t["clock_ghz"])


def wl_keys():
    from tiled_attention_amd import workloads as wl
    return wl.WORKLOADS.keys()


def seq_len_sweep(torch, A):
    """bf16 prefill over N = 1K..32K: B = 4*2048^2/N^2 (at least 1) by 16
    heads, so N <= 2048 carries the causal workload's work per launch.
    Inputs N(0,1) drawn on the device (seeded); each line is timed with HIP
    events after settling launches."""
    rows = []
    for d in (64, 128):
        for mask in ("causal", "none"):
            for N in (1024, 2048, 4096, 8192, 16384, 32768):
                B, H = max(1, (4 * 2048 * 2048) // (N * N)), 16
                g = torch.Generator(device="cuda")
                g.manual_seed(N + d)
                q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
                           for _ in range(3))
                o = torch.empty_like(q)
                step = lambda: A.attn_fwd(q, k, v, o, 1.0 / math.sqrt(d), mask)
                ms = batch_time_ms(step, 40 if N <= 8192 else 10, groups=5)[0]
                pairs = N * (N + 1) / 2 if mask == "causal" else N * N
                tf = 4.0 * d * B * H * pairs / ms / 1e9
                rows.append({"d": d, "mask": mask, "N": N, "B": B, "H": H, "ms": round(ms, 5),
                             "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
                log(f"sweep: d={d} {mask} N={N}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
                del q, k, v, o
    # few-tile causal grids: attn_fwd against attn_fwd_split (the costliest
    # tiles' key ranges split in two, merged by a second kernel)
    split_rows = []
    for (B, H, N, d) in ((1, 4, 8192, 64), (1, 8, 4096, 64), (1, 16, 4096, 64), (1, 16, 2048, 128),
                         (1, 16, 4096, 128), (1, 8, 8192, 128)):
        g = torch.Generator(device="cuda")
        g.manual_seed(N + d + H)
        q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        nb = A.attn_fwd_split_workspace_size(B, H, N, d, "bf16", "causal")
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        ms_f = batch_time_ms(lambda: A.attn_fwd(q, k, v, o, 1.0 / math.sqrt(d), "causal"), 40, groups=5)[0]
        ms_s = batch_time_ms(lambda: A.attn_fwd_split(q, k, v, o, 1.0 / math.sqrt(d), "causal", workspace=ws), 40, groups=5)[0]
        fl = 4.0 * d * B * H * N * (N + 1) / 2
        split_rows.append({"B": B, "H": H, "N": N, "d": d, "workspace_bytes": nb, "fwd_ms": round(ms_f, 5),
                           "split_ms": round(ms_s, 5), "fwd_frac": round(fl / ms_f / 1e9 / PEAK_BF16_TFLOPS, 4),
                           "split_frac": round(fl / ms_s / 1e9 / PEAK_BF16_TFLOPS, 4),
                           "speedup": round(ms_f / ms_s, 3)})
        log(f"sweep: split B={B} H={H} N={N} d={d}: {ms_f * 1e3:.1f} -> {ms_s * 1e3:.1f} us")
        del q, k, v, o, ws
    return {"sweep": "bf16 prefill TFLOP/s over sequence length", "rows": rows, "split_rows": split_rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the clock settles after about 200 back-to-back launches of the 50 us
    # kernel (10 ms); the untimed warmup covers that
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--only-main", action="store_true", help="time only the causal prefill workload")
    ap.add_argument("--workload", type=int, default=2, choices=sorted(wl_keys()),
                    help="workload for --only-main runs (profiling); the JSON line always reports 2 otherwise")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="print bf16 prefill TFLOP/s over sequence length instead of the benchmark line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (attention shards by "
              "head or by sequence with no exchange, so one GPU's throughput is the per-GPU figure)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_attention_amd import workloads as wl
    from tiled_attention_amd import _lib as A
    A.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.sweep:
        print(json.dumps(seq_len_sweep(torch, A)))
        return

    def make(key):
        seed = args.seed if args.seed is not None else wl.default_seed(key)
        w = wl.WORKLOADS[key]
        return {"paged": Paged, "fp8": Fp8, "fp8_full": Fp8Full, "paged_prefill": PagedPrefill,
                "paged_cross": PagedCross}.get(
            w.kind, Dense)(key, seed)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {args.copy_calibration_mib} MiB three times (calibration)")
        del src, dst

    main_key = args.workload if args.only_main else 2
    log(f"bench: preparing workload {main_key}")
    wk = make(main_key)
    smi_before = smi_snapshot()
    settled = settle(wk.step)
    for _ in range(args.warmup):
        wk.step()
    torch.cuda.synchronize()
    # HIP events on the launch stream (torch's current stream, which the
    # steps launch on) around the timed region: their interval over the steps
    # is the average launch duration the roofline uses
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        wk.step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    smi_after = smi_snapshot()
    ms_step = wall * 1e3 / args.steps
    region_ms = ev0.elapsed_time(ev1) / args.steps
    # each launch between its own pair of events, for the spread (the events
    # add their own time to every interval)
    avg_ms, med_ms, min_ms, p90_ms = event_time_ms(wk.step, max(args.steps, 20))
    log(f"bench: workload {main_key}: wall {ms_step:.4f} ms/step, events over the timed region {region_ms:.4f} ms "
        f"per launch, events around each launch {avg_ms:.4f} ms")

    if isinstance(wk, Paged):
        value, unit = wk.bytes / (ms_step * 1e-3) / 1e9, "GB/s"
        achieved, peak, runit, bound = wk.bytes / (region_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        value, unit = wk.flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        achieved, runit = wk.flops / (region_ms * 1e-3) / 1e12, "TFLOP/s"
        if isinstance(wk, Fp8):
            peak, bound = PEAK_FP8_TFLOPS, "mfma"
        elif wk.w.dtype == "f32":
            peak, bound = PEAK_FP32_VALU_TFLOPS, "alu"
        else:
            peak, bound = PEAK_BF16_TFLOPS, "mfma"
    digest = kernel_source_digest()
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4), "traffic": traffic_for(digest) if main_key == 2 else None,
            "kernel": ("fwd_mfma_kernel<64, false, false, 0, false, false> (d=64, bf16 in and out, causal)"
                       if main_key == 2 else f"workload {main_key}"),
            "kernel_avg_ms": round(region_ms, 5),
            "per_launch_events": {"avg_ms": round(avg_ms, 5), "median_ms": round(med_ms, 5), "min_ms": round(min_ms, 5),
                                  "p90_ms": round(p90_ms, 5), "frac": round(achieved * region_ms / avg_ms / peak, 4)},
            "algorithmic_flops_per_launch": wk.flops, "kernel_source_digest": digest}
    ghz = clock_for(digest) if main_key == 2 else None
    if ghz:
        # the same rate against the peak scaled to the clock the kernel ran at
        # (between the two bounds; the lower one is close)
        roof["clock_ghz_measured"] = list(ghz)
        roof["frac_at_measured_clock"] = [round(achieved / (peak * g / 2.4), 4) for g in ghz]

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3" if isinstance(wk, Fp8Full) else "fp8e4m3+bf16" if isinstance(wk, Fp8) else "bf16",
        "data": "synthetic", "config": wk.describe(), "roofline": roof,
        "settle_launches": settled,
        # versions, and rocm-smi's clocks and power before the settling
        # launches and right after the timed steps
        "environment": dict(environment(), smi_before=smi_before, smi_after_timed=smi_after),
    }

    if not args.only_main:
        # the oracle beside the other workloads of the stated configurations
        # (about 10 s each on the host's cores)
        cpu_legs = {1: lambda o: cpu_baseline(o, budget_s=3.0), 3: lambda o: cpu_baseline(o, budget_s=10.0),
                    4: lambda o: cpu_baseline_decode(o, budget_s=10.0), 5: lambda o: cpu_baseline_fp8(o, budget_s=10.0)}
        others = {}
        for key, reps in ((1, 200), (3, 20), (4, 20), (5, 20), (6, 20), (7, 20), (8, 10), (9, 20), (10, 20),
                          (11, 20), (12, 20), (13, 20), (14, 20), (15, 20)):
            log(f"bench: workload {key}")
            o = make(key)
            avg, med, mn, p90 = batch_time_ms(o.step, reps)
            entry = {"config": o.describe(), "ms_avg": round(avg, 5), "ms_median": round(med, 5),
                     "ms_min": round(mn, 5), "ms_p90": round(p90, 5)}
            if isinstance(o, Paged):
                gbs = o.bytes / (avg * 1e-3) / 1e9
                entry.update({"value": round(gbs, 1), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                              "algorithmic_bytes": o.bytes})
            else:
                tf = o.flops / (avg * 1e-3) / 1e12
                entry.update({"value": round(tf, 2), "unit": "TFLOP/s", "algorithmic_flops": o.flops})
                if isinstance(o, Fp8Full):
                    entry.update({"frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)})
                elif isinstance(o, Fp8):
                    half = o.flops / 2
                    blended_s = half / (PEAK_FP8_TFLOPS * 1e12) + half / (PEAK_BF16_TFLOPS * 1e12)
                    entry.update({"frac_of_blended_peak": round(blended_s / (avg * 1e-3), 4),
                                  "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                                  "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
                elif getattr(o.w, "dtype", "") == "f32" and o.w.kind == "dense":
                    entry["frac_of_fp32_valu_peak"] = round(tf / PEAK_FP32_VALU_TFLOPS, 6)
                else:
                    entry["frac_of_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            if isinstance(o, PagedPrefill):
                # "Optimizing Triton kernels ...", Pattern C: gather, then
                # attend over the dense copy, against the fused kernel
                g_avg = batch_time_ms(o.gather, reps)[0]
                a_avg = batch_time_ms(o.attend_gathered, reps)[0]
                t_avg = batch_time_ms(o.two_stage, reps)[0]
                entry["two_stage_gather_ms"] = round(g_avg, 5)
                entry["two_stage_gather_GBps"] = round(o.gather_bytes / (g_avg * 1e-3) / 1e9, 1)
                entry["two_stage_attend_ms"] = round(a_avg, 5)
                entry["two_stage_total_ms"] = round(t_avg, 5)
                entry["fused_over_two_stage_speedup"] = round(t_avg / avg, 3)
            others[o.w.name] = entry
            del o
            torch.cuda.empty_cache()
        # Pattern A of the structured-mask page compares a document-masked
        # kernel with plain attention on the same shape
        dense = others.get(wl.WORKLOADS[10].name)
        for key in (6, 7):
            e = others.get(wl.WORKLOADS[key].name)
            if dense and e:
                e["ratio_to_unmasked_same_shape"] = round(e["value"] / dense["value"], 4)
        # the oracle legs run after every GPU timing, so the idle GPU's clock
        # drop does not reach the timed lines
        if not args.no_cpu_baseline:
            for key, leg in cpu_legs.items():
                log(f"bench: cpu baseline (oracle) of workload {key}")
                o = make(key)
                others[o.w.name]["cpu_baseline"] = leg(o)
                del o
                torch.cuda.empty_cache()
        result["workloads"] = others

    if not args.no_cpu_baseline and not isinstance(wk, (Paged, Fp8)):
        log("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wk)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
