"""ctypes binding of libattn.so (argument marshalling only).

Every function has the name of the C entry point it calls (see
include/attn.h). Tensors are torch tensors on the GPU; their data pointers and
the current HIP stream are passed through unchanged. A non-OK status raises
ValueError (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE) or
RuntimeError (ATTN_ERR_LAUNCH). There is no fallback: if the library is not
built, loading fails loudly.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_LAUNCH = range(5)
ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3 = range(3)
MASKS = {"none": 0, "causal": 1, "sliding": 2, "band": 3, "prefix_lm": 4, "document": 5, "document_causal": 6}
DOC_MASKS = ("document", "document_causal")

# symbol -> (restype, argtypes)
_c_int, _c_float, _p, _size = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_PROTOS = {
    "attn_fwd": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                          _c_int, _c_int, _p, _c_int, _p, _p]),
    "attn_fwd_split_workspace_size": (_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_fwd_split": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                _c_int, _c_int, _p, _c_int, _p, _p, _size, _p]),
    "attn_fwd_fp8": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                              _c_int, _c_int, _p, _c_int, _p, _p]),
    "attn_fwd_fp8_full": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_float, _c_int, _c_int, _p, _c_int, _p, _p]),
    "attn_quant_fp8_block": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p]),
    "attn_quant_fp8_block_pow2": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p]),
    "attn_decode_paged_workspace_size": (_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_decode_paged": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_float, _p, _p, _size, _p]),
    "attn_decode_paged_noalloc": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                           _c_int, _c_float, _p, _p]),
    "attn_prefill_paged": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_float, _p, _p]),
    "attn_cross_paged": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _c_int, _c_float, _p, _p]),
    "attn_gather_paged": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _p]),
    "attn_tile_class": (_c_int, [_c_int, _c_int, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_k_tile_range": (_c_int, [_c_int, _c_int, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "attn_full_tile_range": (_c_int, [_c_int, _c_int, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "attn_dispatch_ranks": (_c_int, [_p, _c_int, _p]),
    "attn_status_str": (ctypes.c_char_p, [_c_int]),
    "attn_abi_version": (_c_int, []),
}

_lib = None


def load():
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m tiled_attention_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def symbols():
    return list(_PROTOS)


def _check(status):
    if status == ATTN_OK:
        return
    msg = load().attn_status_str(status).decode()
    if status in (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE):
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        if t is not None:
            _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous GPU tensors")


def _spec(t, name, shape, dtypes, optional=False):
    """t has exactly this shape and one of these dtypes (None allowed when optional).
    Shapes and dtypes are checked before anything reaches the library: a
    mis-sized tensor would otherwise become a device access outside it."""
    if t is None:
        _require(optional, f"{name} is required")
        return
    _require(tuple(t.shape) == tuple(int(x) for x in shape),
             f"{name} must have shape {list(int(x) for x in shape)}, got {list(t.shape)}")
    _require(t.dtype in dtypes, f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _dtypes():
    import torch
    return torch.float32, torch.bfloat16, torch.uint8, torch.int32


def _docs(mask, doc_offsets):
    """(pointer, num_docs) of a device int32 offsets tensor; (None, 0) when unused."""
    _require(mask in MASKS, f"unknown mask {mask!r}")
    if mask not in DOC_MASKS:
        return None, 0
    _require(doc_offsets is not None, f"mask {mask!r} needs doc_offsets")
    import torch
    _require(doc_offsets.dtype == torch.int32 and doc_offsets.dim() == 1 and doc_offsets.numel() >= 2,
             "doc_offsets must be int32 [num_docs + 1] with num_docs >= 1")
    _dev(doc_offsets)
    return _ptr(doc_offsets), doc_offsets.numel() - 1


def _nblocks(n, block):
    return -(-int(n) // int(block)) if int(block) > 0 else 0


def attn_fwd(q, k, v, o, scale, mask="none", window=0, doc_offsets=None, lse=None, stream=None):
    """O = softmax(Q K^T * scale, mask) V for q, k, v, o of shape [B, H, N, d].

    doc_offsets: device int32 [num_docs + 1] for the document masks."""
    f32, bf16, _, _ = _dtypes()
    _require(q.dim() == 4, "q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _spec(q, "q", q.shape, (f32, bf16))
    _spec(k, "k", q.shape, (q.dtype,))
    _spec(v, "v", q.shape, (q.dtype,))
    _spec(o, "o", q.shape, (f32, bf16))
    _spec(lse, "lse", (B, H, N), (f32,), optional=True)
    dp, nd = _docs(mask, doc_offsets)
    _dev(q, k, v, o, lse)
    _check(load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, _dtype_code(q), _dtype_code(o),
                           float(scale), MASKS[mask], int(window), dp, nd, _ptr(lse), _stream(stream)))
    return o


def attn_fwd_split_workspace_size(B, H, N, d, dtype="bf16", mask="causal", window=0):
    """Bytes of workspace attn_fwd_split needs (0: the launch is not split)."""
    _require(mask in MASKS, f"unknown mask {mask!r}")
    _require(dtype in ("bf16", "f32"), "dtype is 'bf16' or 'f32'")
    return int(load().attn_fwd_split_workspace_size(int(B), int(H), int(N), int(d),
                                                     ATTN_BF16 if dtype == "bf16" else ATTN_F32,
                                                     MASKS[mask], int(window)))


def attn_fwd_split(q, k, v, o, scale, mask="causal", window=0, doc_offsets=None, lse=None, workspace=None,
                   stream=None):
    """attn_fwd with the costliest query tiles' key ranges split in two; workspace:
    a device uint8 tensor of attn_fwd_split_workspace_size(...) bytes (None
    when that size is 0)."""
    f32, bf16, u8, _ = _dtypes()
    _require(q.dim() == 4, "q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _spec(q, "q", q.shape, (f32, bf16))
    _spec(k, "k", q.shape, (q.dtype,))
    _spec(v, "v", q.shape, (q.dtype,))
    _spec(o, "o", q.shape, (f32, bf16))
    _spec(lse, "lse", (B, H, N), (f32,), optional=True)
    dp, nd = _docs(mask, doc_offsets)
    if workspace is not None:
        _require(workspace.dtype == u8 and workspace.dim() == 1, "workspace must be a 1-D uint8 tensor")
    _dev(q, k, v, o, lse, workspace)
    _check(load().attn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, _dtype_code(q), _dtype_code(o),
                                 float(scale), MASKS[mask], int(window), dp, nd, _ptr(lse), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(stream)))
    return o


def _fp8_specs(q8, q_scale, k8, k_scale, o, lse, qk_block):
    f32, bf16, u8, _ = _dtypes()
    _require(q8.dim() == 4, "q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    nb = _nblocks(N, qk_block)
    _spec(q8, "q8", q8.shape, (u8,))
    _spec(k8, "k8", q8.shape, (u8,))
    _spec(q_scale, "q_scale", (B, H, nb), (f32,))
    _spec(k_scale, "k_scale", (B, H, nb), (f32,))
    _spec(o, "o", q8.shape, (bf16,))
    _spec(lse, "lse", (B, H, N), (f32,), optional=True)
    return B, H, N, d, nb


def attn_fwd_fp8(q8, q_scale, k8, k_scale, v, o, scale, mask="none", window=0, doc_offsets=None, qk_block=128,
                 lse=None, stream=None):
    """fp8 block-scaled Q, K (uint8 E4M3FN codes + fp32 block scales), bf16 V and O."""
    B, H, N, d, _ = _fp8_specs(q8, q_scale, k8, k_scale, o, lse, qk_block)
    _spec(v, "v", q8.shape, (_dtypes()[1],))
    dp, nd = _docs(mask, doc_offsets)
    _dev(q8, q_scale, k8, k_scale, v, o, lse)
    _check(load().attn_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), _ptr(o),
                               B, H, N, d, int(qk_block), float(scale), MASKS[mask], int(window), dp, nd,
                               _ptr(lse), _stream(stream)))
    return o


def attn_fwd_fp8_full(q8, q_scale, k8, k_scale, v8, v_scale, o, scale, mask="none", window=0, doc_offsets=None,
                      qk_block=128, lse=None, stream=None):
    """Q, K and V all fp8 (uint8 E4M3FN codes + fp32 block scales; V's scales powers of two), bf16 O."""
    B, H, N, d, nb = _fp8_specs(q8, q_scale, k8, k_scale, o, lse, qk_block)
    _spec(v8, "v8", q8.shape, (_dtypes()[2],))
    _spec(v_scale, "v_scale", (B, H, nb), (_dtypes()[0],))
    dp, nd = _docs(mask, doc_offsets)
    _dev(q8, q_scale, k8, k_scale, v8, v_scale, o, lse)
    _check(load().attn_fwd_fp8_full(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                                    _ptr(o), B, H, N, d, int(qk_block), float(scale), MASKS[mask], int(window), dp,
                                    nd, _ptr(lse), _stream(stream)))
    return o


def _quant_specs(x, codes, scales, block):
    f32, _, u8, _ = _dtypes()
    _require(x.dim() == 4, "x must be [B, H, N, d]")
    B, H, N, d = x.shape
    _spec(x, "x", x.shape, (f32,))
    _spec(codes, "codes", x.shape, (u8,))
    _spec(scales, "scales", (B, H, _nblocks(N, block)), (f32,))
    _dev(x, codes, scales)
    return B, H, N, d


def attn_quant_fp8_block_pow2(x, codes, scales, block=128, stream=None):
    """As attn_quant_fp8_block with power-of-two block scales (for V of attn_fwd_fp8_full)."""
    B, H, N, d = _quant_specs(x, codes, scales, block)
    _check(load().attn_quant_fp8_block_pow2(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, int(block),
                                            _stream(stream)))
    return codes, scales


def attn_quant_fp8_block(x, codes, scales, block=128, stream=None):
    """Per-block E4M3FN quantisation of x [B, H, N, d] fp32 into codes (uint8) and scales (fp32)."""
    B, H, N, d = _quant_specs(x, codes, scales, block)
    _check(load().attn_quant_fp8_block(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, int(block),
                                       _stream(stream)))
    return codes, scales


def attn_decode_paged_workspace_size(S, H, d, max_pages, page_size=16):
    return int(load().attn_decode_paged_workspace_size(S, H, d, max_pages, page_size))


def _pool_specs(k_pool, v_pool, H, d, dtypes):
    _require(k_pool.dim() == 4, "k_pool must be [num_pages, H, page_size, d]")
    num_pages, _, page_size, _ = k_pool.shape
    _spec(k_pool, "k_pool", (num_pages, H, page_size, d), dtypes)
    _spec(v_pool, "v_pool", k_pool.shape, (k_pool.dtype,))
    return num_pages, page_size


def attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, scale, workspace=None, lse=None,
                      stream=None):
    """Single-token decode over a paged KV pool; workspace None -> one pass per (sequence, head)."""
    f32, bf16, _, i32 = _dtypes()
    _require(q.dim() == 3, "q must be [S, H, d]")
    S, H, d = q.shape
    _spec(q, "q", q.shape, (bf16,))
    _spec(o, "o", q.shape, (bf16,))
    num_pages, page_size = _pool_specs(k_pool, v_pool, H, d, (bf16,))
    _require(block_table.dim() == 2, "block_table must be [S, max_pages]")
    max_pages = block_table.shape[1]
    _spec(block_table, "block_table", (S, max_pages), (i32,))
    _spec(seq_lens, "seq_lens", (S,), (i32,))
    _spec(lse, "lse", (S, H), (f32,), optional=True)
    _dev(q, k_pool, v_pool, block_table, seq_lens, o, workspace, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().attn_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(o), S, H, d, page_size, max_pages, num_pages, float(scale), _ptr(lse),
                                    _ptr(workspace), ws_bytes, _stream(stream)))
    return o


def attn_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, o, scale, lse=None, stream=None):
    """attn_decode_paged's split path with the library's fixed device array in
    place of a workspace (allocates nothing); calls overlapping on one GPU race."""
    f32, bf16, _, i32 = _dtypes()
    _require(q.dim() == 3, "q must be [S, H, d]")
    S, H, d = q.shape
    _spec(q, "q", q.shape, (bf16,))
    _spec(o, "o", q.shape, (bf16,))
    num_pages, page_size = _pool_specs(k_pool, v_pool, H, d, (bf16,))
    _require(block_table.dim() == 2, "block_table must be [S, max_pages]")
    max_pages = block_table.shape[1]
    _spec(block_table, "block_table", (S, max_pages), (i32,))
    _spec(seq_lens, "seq_lens", (S,), (i32,))
    _spec(lse, "lse", (S, H), (f32,), optional=True)
    _dev(q, k_pool, v_pool, block_table, seq_lens, o, lse)
    _check(load().attn_decode_paged_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                            _ptr(seq_lens), _ptr(o), S, H, d, page_size, max_pages, num_pages,
                                            float(scale), _ptr(lse), _stream(stream)))
    return o


def _paged_fwd(fn, causal, q, k_pool, v_pool, table, lens, o, scale, lse, stream):
    f32, bf16, _, i32 = _dtypes()
    _require(q.dim() == 4, "q must be [S, H, q_len, d]")
    S, H, q_len, d = q.shape
    _spec(q, "q", q.shape, (bf16,))
    _spec(o, "o", q.shape, (f32, bf16))
    num_pages, page_size = _pool_specs(k_pool, v_pool, H, d, (bf16,))
    max_pages = table.shape[-1]
    if causal:
        _spec(table, "block_table", (S, max_pages), (i32,))
        _spec(lens, "seq_lens", (S,), (i32,))
    else:
        qb = _nblocks(q_len, 128)
        _spec(table, "page_table", (S, qb, max_pages), (i32,))
        _spec(lens, "kv_lens", (S, qb), (i32,))
    _spec(lse, "lse", (S, H, q_len), (f32,), optional=True)
    _dev(q, k_pool, v_pool, table, lens, o, lse)
    _check(fn(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(table), _ptr(lens), _ptr(o), S, H, q_len, d, page_size,
              max_pages, num_pages, _dtype_code(o), float(scale), _ptr(lse), _stream(stream)))
    return o


def attn_prefill_paged(q, k_pool, v_pool, block_table, seq_lens, o, scale, lse=None, stream=None):
    """Causal prefill of the last q_len positions of each paged sequence (16- or 64-token pages)."""
    return _paged_fwd(load().attn_prefill_paged, True, q, k_pool, v_pool, block_table, seq_lens, o, scale, lse,
                      stream)


def attn_cross_paged(q, k_pool, v_pool, page_table, kv_lens, o, scale, lse=None, stream=None):
    """Block-sparse cross-attention: query block b of sequence s over its own page list."""
    return _paged_fwd(load().attn_cross_paged, False, q, k_pool, v_pool, page_table, kv_lens, o, scale, lse,
                      stream)


def attn_gather_paged(k_pool, v_pool, block_table, seq_lens, k_out, v_out, stream=None):
    """Dense copies k_out/v_out [S, H, max_pages*page, d] of each sequence's pages."""
    f32, bf16, _, i32 = _dtypes()
    _require(k_pool.dim() == 4, "k_pool must be [num_pages, H, page_size, d]")
    num_pages, H, page_size, d = k_pool.shape
    _pool_specs(k_pool, v_pool, H, d, (f32, bf16))
    _require(block_table.dim() == 2, "block_table must be [S, max_pages]")
    S, max_pages = block_table.shape
    _spec(block_table, "block_table", (S, max_pages), (i32,))
    _spec(seq_lens, "seq_lens", (S,), (i32,))
    _spec(k_out, "k_out", (S, H, max_pages * page_size, d), (k_pool.dtype,))
    _spec(v_out, "v_out", (S, H, max_pages * page_size, d), (k_pool.dtype,))
    _dev(k_pool, v_pool, block_table, seq_lens, k_out, v_out)
    _check(load().attn_gather_paged(_ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(k_out),
                                    _ptr(v_out), S, H, d, page_size, max_pages, num_pages,
                                    _dtype_code(k_pool), _stream(stream)))
    return k_out, v_out


def _host_docs(doc_offsets):
    """(ctypes int32 array, num_docs) of host offsets (any int sequence), or (None, 0)."""
    if doc_offsets is None:
        return None, 0
    vals = [int(x) for x in doc_offsets]
    return (ctypes.c_int32 * len(vals))(*vals), len(vals) - 1


def attn_tile_class(mask, window, N, m0, m1, n0, n1, doc_offsets=None):
    """Tile class (0 EMPTY, 1 PARTIAL, 2 FULL; -1 invalid). doc_offsets: host offsets for document masks."""
    arr, nd = _host_docs(doc_offsets)
    return int(load().attn_tile_class(MASKS[mask], window, arr, nd, N, m0, m1, n0, n1))


def attn_k_tile_range(mask, window, N, m0, m1, bn, doc_offsets=None):
    arr, nd = _host_docs(doc_offsets)
    lo, hi = _c_int(), _c_int()
    _check(load().attn_k_tile_range(MASKS[mask], window, arr, nd, N, m0, m1, bn, ctypes.byref(lo),
                                    ctypes.byref(hi)))
    return lo.value, hi.value


def attn_full_tile_range(mask, window, N, m0, m1, bn, doc_offsets=None):
    arr, nd = _host_docs(doc_offsets)
    lo, hi = _c_int(), _c_int()
    _check(load().attn_full_tile_range(MASKS[mask], window, arr, nd, N, m0, m1, bn, ctypes.byref(lo),
                                       ctypes.byref(hi)))
    return lo.value, hi.value


def attn_dispatch_ranks(costs):
    """Heaviest-first ranks (host) of a list of group costs, as the kernels rank them."""
    vals = [int(c) for c in costs]
    arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    out = (ctypes.c_int32 * max(1, len(vals)))()
    _check(load().attn_dispatch_ranks(arr, len(vals), out))
    return [int(x) for x in out[:len(vals)]]


def attn_status_str(status):
    return load().attn_status_str(status).decode()


def attn_abi_version():
    return int(load().attn_abi_version())
