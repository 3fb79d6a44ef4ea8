"""MI355X (gfx950) lightning indexer + top-k token selector.

Thin Python binding over libdsaidx.so (include/dsaidx.h).  Every step of the
computation runs in the library's HIP kernels; this module only checks
tensor shapes, allocates outputs and workspace with torch on the inputs'
device, and passes pointers and the current HIP stream.

    indexer_prefill(q, k, w, topk, q_scale=None, k_scale=None, want_scores=False)
    indexer_decode_paged(q, w, k_cache, k_scale, block_table, context_lens, topk, max_context_len=None)
    topk_select(scores, topk, row_len=None)

Input formats: fp32 tensors; bf16 as torch.bfloat16 or int16/uint16 bit
patterns; OCP FP8 E4M3 as torch.float8_e4m3fn or uint8 codes with fp32
per-row scales.
"""
from __future__ import annotations

import torch

from . import _lib

F32, BF16, FP8_E4M3 = 0, 1, 2

__all__ = ["indexer_prefill", "indexer_prefill_noalloc", "indexer_decode_paged", "topk_select", "kcache_append", "topk_gather",
           "topk_gather_layers",
           "prefill_chunk_paged", "prefill_chunk_varlen", "dtype_code", "F32", "BF16", "FP8_E4M3"]


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need(t, name: str, *dtypes) -> None:
    """Index and table tensors must be int32, weights and scales fp32: the
    library reads them as such, so any other element type would be read as
    garbage (an int64 block table as pairs of int32 page ids)."""
    if t is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


_I32 = torch.int32
_F32 = torch.float32
_CODES = (torch.uint8, torch.float8_e4m3fn)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def indexer_prefill(q, k, w, topk: int, q_scale=None, k_scale=None, want_scores: bool = False,
                    want_topk_score: bool = True):
    """Top-k causal history positions of every token of B sequences.

    q [B,L,H,D], k [B,L,D], w [B,L,H] fp32 (+ q_scale [B,L,H], k_scale [B,L]
    fp32 for fp8).  Returns (idx int32 [B,L,topk], score fp32 [B,L,topk] or
    None, scores fp32 [B,L,L] or None)."""
    lib = _lib.load()
    B, L, H, D = q.shape
    if tuple(k.shape) != (B, L, D) or tuple(w.shape) != (B, L, H):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} w{tuple(w.shape)}")
    dt = dtype_code(q)
    if dtype_code(k) != dt:
        raise ValueError("q and k must share a format")
    _need(w, "w", _F32)
    _need(q_scale, "q_scale", _F32)
    _need(k_scale, "k_scale", _F32)
    for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None:
            _dev(t, name)
    dev = q.device
    idx = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
    val = torch.empty((B, L, topk), dtype=torch.float32, device=dev) if want_topk_score else None
    scores = torch.empty((B, L, L), dtype=torch.float32, device=dev) if want_scores else None
    nws = lib.indexer_prefill_workspace_bytes(B, L, H, D, topk, dt, 1 if want_scores else 0)
    ws = _workspace(nws, dev)
    st = lib.indexer_prefill(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), dt, _ptr(w), B, L, H, D, topk,
                             _ptr(idx), _ptr(val), _ptr(scores), _ptr(ws), nws, _stream(dev))
    _lib.check(st, "indexer_prefill")
    return idx, val, scores


def indexer_prefill_noalloc(q, k, w, topk: int, q_scale=None, k_scale=None, want_scores: bool = False,
                            want_topk_score: bool = True, out=None):
    """indexer_prefill through the library entry point that allocates
    nothing (its scratch is a fixed device array inside the library).  The
    outputs are allocated here unless ``out`` = (idx, score or None, scores or
    None) gives them.  Returns the same triple as indexer_prefill."""
    lib = _lib.load()
    B, L, H, D = q.shape
    if tuple(k.shape) != (B, L, D) or tuple(w.shape) != (B, L, H):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} w{tuple(w.shape)}")
    dt = dtype_code(q)
    if dtype_code(k) != dt:
        raise ValueError("q and k must share a format")
    _need(w, "w", _F32)
    _need(q_scale, "q_scale", _F32)
    _need(k_scale, "k_scale", _F32)
    for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None:
            _dev(t, name)
    dev = q.device
    if out is not None:
        idx, val, scores = out
        _need(idx, "idx", _I32)
        if tuple(idx.shape) != (B, L, topk) or (val is not None and tuple(val.shape) != (B, L, topk)) or \
                (scores is not None and tuple(scores.shape) != (B, L, L)):
            raise ValueError("output shapes do not match the call")
    else:
        idx = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
        val = torch.empty((B, L, topk), dtype=torch.float32, device=dev) if want_topk_score else None
        scores = torch.empty((B, L, L), dtype=torch.float32, device=dev) if want_scores else None
    st = lib.indexer_prefill_noalloc(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), dt, _ptr(w), B, L, H, D, topk,
                                     _ptr(idx), _ptr(val), _ptr(scores), _stream(dev))
    _lib.check(st, "indexer_prefill_noalloc")
    return idx, val, scores


def indexer_decode_paged(q, w, k_cache, k_scale, block_table, context_lens, topk: int,
                         max_context_len: int | None = None, want_topk_score: bool = True,
                         workspace: torch.Tensor | None = None):
    """Top-k context positions of B decode queries over a paged fp8 cache.

    q [B,H,D] bf16, w [B,H] fp32, k_cache [P,page,D] fp8 codes, k_scale
    [P,page] fp32, block_table [B,max_pages] int32, context_lens [B] int32.
    ``max_context_len`` bounds context_lens (default: max_pages * page).
    Returns (idx int32 [B,topk], score fp32 [B,topk] or None)."""
    lib = _lib.load()
    B, H, D = q.shape
    P, page, Dk = k_cache.shape
    if Dk != D or tuple(k_scale.shape) != (P, page) or tuple(w.shape) != (B, H):
        raise ValueError("shape mismatch")
    if block_table.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_table / context_lens shape mismatch")
    _need(w, "w", _F32)
    _need(k_cache, "k_cache", *_CODES)
    _need(k_scale, "k_scale", _F32)
    _need(block_table, "block_table", _I32)
    _need(context_lens, "context_lens", _I32)
    for name, t in (("q", q), ("w", w), ("k_cache", k_cache), ("k_scale", k_scale),
                    ("block_table", block_table), ("context_lens", context_lens)):
        _dev(t, name)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages]")
    mpp = block_table.shape[1]
    mcl = mpp * page if max_context_len is None else int(max_context_len)
    dev = q.device
    idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
    val = torch.empty((B, topk), dtype=torch.float32, device=dev) if want_topk_score else None
    nws = lib.indexer_decode_paged_workspace_bytes(B, mcl, H, D, topk)
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, dev)
    st = lib.indexer_decode_paged(_ptr(q), dtype_code(q), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                                  _ptr(block_table), mpp, _ptr(context_lens), mcl, B, H, D, page, P, topk,
                                  _ptr(idx), _ptr(val), _ptr(ws), nws, _stream(dev))
    _lib.check(st, "indexer_decode_paged")
    return idx, val


def decode_workspace_bytes(B: int, max_context_len: int, H: int, D: int, topk: int) -> int:
    return _lib.load().indexer_decode_paged_workspace_bytes(B, max_context_len, H, D, topk)


def topk_select(scores, topk: int, row_len=None, want_values: bool = True):
    """Top-k of each row of a [rows, cols] fp32 matrix (row r valid up to
    row_len[r]).  Returns (idx int32 [rows,topk], values fp32 or None)."""
    lib = _lib.load()
    if scores.dim() != 2 or scores.dtype != torch.float32:
        raise ValueError("scores must be a 2-D fp32 tensor")
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    rows, cols = scores.shape
    dev = scores.device
    if row_len is not None:
        _need(row_len, "row_len", _I32)
        _dev(row_len, "row_len")
        if tuple(row_len.shape) != (rows,):
            raise ValueError("row_len must hold one length per row")
    idx = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    val = torch.empty((rows, topk), dtype=torch.float32, device=dev) if want_values else None
    nws = lib.topk_select_workspace_bytes(rows, cols, topk)
    ws = _workspace(nws, dev)
    st = lib.topk_select(_ptr(scores), rows, cols, scores.stride(0), _ptr(row_len), topk, _ptr(idx), _ptr(val),
                         _ptr(ws), nws, _stream(dev))
    _lib.check(st, "topk_select")
    return idx, val


def kcache_append(k, seq_ids, positions, block_table, k_cache, k_scale):
    """Quantise T new keys to FP8 and write them into the paged cache in place.

    k [T,D] bf16 or fp32, seq_ids [T] int32 (outside [0, B): skipped),
    positions [T] int32, block_table [B,max_pages] int32, k_cache [P,page,D]
    uint8 E4M3FN codes, k_scale [P,page] fp32.  Returns nothing: k_cache and
    k_scale are updated on the current stream."""
    lib = _lib.load()
    T, D = k.shape
    P, page, Dk = k_cache.shape
    if Dk != D or tuple(k_scale.shape) != (P, page):
        raise ValueError("k_cache / k_scale shape mismatch")
    if tuple(seq_ids.shape) != (T,) or tuple(positions.shape) != (T,):
        raise ValueError("seq_ids / positions must have one entry per key")
    if k_cache.dtype != torch.uint8 or k_scale.dtype != torch.float32:
        raise ValueError("k_cache must be uint8 codes and k_scale fp32")
    _need(seq_ids, "seq_ids", _I32)
    _need(positions, "positions", _I32)
    _need(block_table, "block_table", _I32)
    for name, t in (("k", k), ("seq_ids", seq_ids), ("positions", positions), ("block_table", block_table),
                    ("k_cache", k_cache), ("k_scale", k_scale)):
        _dev(t, name)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages]")
    B, mpp = block_table.shape
    st = lib.indexer_kcache_append(_ptr(k), dtype_code(k), _ptr(seq_ids), _ptr(positions), _ptr(block_table),
                                   B, mpp, _ptr(k_cache), _ptr(k_scale), P, T, D, page, _stream(k.device))
    _lib.check(st, "indexer_kcache_append")


def topk_gather(latent_cache, block_table, topk_idx):
    """Rows of a paged latent cache at each query's selected positions.

    latent_cache [P,page,E] (any element type; E * element size a multiple of
    16 bytes), block_table [B,max_pages] int32, topk_idx [B,K] int32 (-1 or
    outside the table: a zero row).  Returns out [B,K,E] of the cache's dtype."""
    lib = _lib.load()
    P, page, E = latent_cache.shape
    B, K = topk_idx.shape
    if block_table.shape[0] != B or topk_idx.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("block_table [B, max_pages] and topk_idx [B, K] must be int32 with matching B")
    for name, t in (("latent_cache", latent_cache), ("block_table", block_table), ("topk_idx", topk_idx)):
        _dev(t, name)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages]")
    out = torch.empty((B, K, E), dtype=latent_cache.dtype, device=latent_cache.device)
    st = lib.indexer_topk_gather(_ptr(latent_cache), E * latent_cache.element_size(), _ptr(block_table),
                                 block_table.shape[1], P, page, _ptr(topk_idx), B, K, _ptr(out),
                                 _stream(latent_cache.device))
    _lib.check(st, "indexer_topk_gather")
    return out


def topk_gather_layers(latent_caches, block_table, topk_idx, outs=None):
    """Index Share: one selection gathered from several layers' latent
    caches in one launch.  latent_caches: a sequence of [P,page,E] tensors of
    one shape and dtype (at most 64); block_table, topk_idx as topk_gather.
    Returns a list of [B,K,E] tensors, one per layer (or fills `outs`)."""
    import ctypes

    lib = _lib.load()
    caches = list(latent_caches)
    if not caches:
        raise ValueError("latent_caches is empty")
    P, page, E = caches[0].shape
    for i, c in enumerate(caches):
        if c.shape != caches[0].shape or c.dtype != caches[0].dtype:
            raise ValueError(f"latent_caches[{i}] differs in shape or dtype from latent_caches[0]")
        _dev(c, f"latent_caches[{i}]")
    B, K = topk_idx.shape
    _need(block_table, "block_table", _I32)
    _need(topk_idx, "topk_idx", _I32)
    for name, t in (("block_table", block_table), ("topk_idx", topk_idx)):
        _dev(t, name)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages] with the B of topk_idx")
    if outs is None:
        outs = [torch.empty((B, K, E), dtype=caches[0].dtype, device=caches[0].device) for _ in caches]
    else:
        outs = list(outs)
        if len(outs) != len(caches):
            raise ValueError("one output per layer")
        for i, o in enumerate(outs):
            if o.shape != (B, K, E) or o.dtype != caches[0].dtype:
                raise ValueError(f"outs[{i}] must be [B, K, E] of the caches' dtype")
            _dev(o, f"outs[{i}]")
    n = len(caches)
    cp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in caches])
    op = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    st = lib.indexer_topk_gather_layers(cp, op, n, E * caches[0].element_size(), _ptr(block_table),
                                        block_table.shape[1], P, page, _ptr(topk_idx), B, K,
                                        _stream(caches[0].device))
    _lib.check(st, "indexer_topk_gather_layers")
    return outs


def probe_mfma(kind: int, blocks: int, iters: int, device="cuda"):
    """Measurement probe: blocks x 4 waves x iters x 8 MFMAs of one shape
    (0: fp8 16x16x128 scaled, 1: bf16 16x16x32, 2: f16 16x16x32).  Returns
    the (meaningless) output tensor; time the call with events."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    _lib.check(_lib.load().dsaidx_probe_mfma(kind, blocks, iters, _ptr(out), _stream(out.device)),
               "dsaidx_probe_mfma")
    return out


def probe_page_read(k_cache, k_scale, page_ids, blocks: int, out=None):
    """Measurement probe: reads the pages page_ids of a paged fp8 key cache
    (8448 bytes each) with the decode scan's load layout."""
    _need(k_cache, "k_cache", *_CODES)
    _need(k_scale, "k_scale", _F32)
    _need(page_ids, "page_ids", _I32)
    for name, t in (("k_cache", k_cache), ("k_scale", k_scale), ("page_ids", page_ids)):
        _dev(t, name)
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=k_cache.device)
    _lib.check(_lib.load().dsaidx_probe_page_read(_ptr(k_cache), _ptr(k_scale), _ptr(page_ids), page_ids.numel(),
                                                  blocks, _ptr(out), _stream(k_cache.device)),
               "dsaidx_probe_page_read")
    return out


def prefill_chunk_varlen(q, q_scale, w, cu_seqlens_q, q_start, k_cache, k_scale, block_table, topk: int,
                         max_kv_len: int, want_topk_score: bool = True, workspace: torch.Tensor | None = None):
    """Top-k of the query rows of B sequences' chunks (packed one after
    another) against the paged fp8 key cache: row cu_seqlens_q[b] + i is
    position q_start[b] + i of sequence b and sees keys 0 .. that position.

    q [T,H,D] fp8 codes (uint8) with q_scale [T,H] fp32, or bf16 with
    q_scale None; w [T,H] fp32,
    cu_seqlens_q [B+1] int32 (device), q_start [B] int32 (device), k_cache
    [P,page,D] uint8, k_scale [P,page] fp32, block_table [B,max_pages] int32;
    ``max_kv_len`` bounds q_start[b] + rows of b (host value).  Returns (idx
    int32 [T,topk] of absolute positions, score fp32 [T,topk] or None)."""
    lib = _lib.load()
    T, H, D = q.shape
    P, page, Dk = k_cache.shape
    B = q_start.shape[0]
    if Dk != D or tuple(k_scale.shape) != (P, page) or tuple(w.shape) != (T, H):
        raise ValueError("shape mismatch")
    fp8_q = dtype_code(q) == FP8_E4M3
    if fp8_q != (q_scale is not None):
        raise ValueError("q_scale [T, H] goes with fp8 queries, None with bf16 queries")
    if q_scale is not None and tuple(q_scale.shape) != (T, H):
        raise ValueError("q_scale must be [T, H]")
    if tuple(cu_seqlens_q.shape) != (B + 1,) or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("cu_seqlens_q [B+1], q_start [B] and block_table [B, max_pages] must agree on B")
    _need(q, "q", *_CODES, torch.bfloat16, torch.int16, torch.uint16)
    _need(q_scale, "q_scale", _F32)
    _need(w, "w", _F32)
    _need(k_cache, "k_cache", *_CODES)
    _need(k_scale, "k_scale", _F32)
    _need(block_table, "block_table", _I32)
    _need(cu_seqlens_q, "cu_seqlens_q", _I32)
    _need(q_start, "q_start", _I32)
    for name, t in (("q", q), ("q_scale", q_scale), ("w", w), ("cu_seqlens_q", cu_seqlens_q), ("q_start", q_start),
                    ("k_cache", k_cache), ("k_scale", k_scale), ("block_table", block_table)):
        if t is not None:
            _dev(t, name)
    dev = q.device
    idx = torch.empty((T, topk), dtype=torch.int32, device=dev)
    val = torch.empty((T, topk), dtype=torch.float32, device=dev) if want_topk_score else None
    nws = lib.indexer_prefill_chunk_paged_workspace_bytes(B, T, int(max_kv_len), dtype_code(q))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, dev)
    st = lib.indexer_prefill_chunk_paged(_ptr(q), _ptr(q_scale), dtype_code(q), _ptr(w), _ptr(cu_seqlens_q),
                                         _ptr(q_start), _ptr(k_cache), _ptr(k_scale), _ptr(block_table),
                                         block_table.shape[1], P, B, T, int(max_kv_len), H, D, page, topk,
                                         _ptr(idx), _ptr(val), _ptr(ws), nws, _stream(dev))
    _lib.check(st, "indexer_prefill_chunk_paged")
    return idx, val


def prefill_chunk_paged(q, q_scale, w, k_cache, k_scale, block_table, q0: int, topk: int,
                        want_topk_score: bool = True, workspace: torch.Tensor | None = None):
    """Top-k of a chunk of Lq query tokens per sequence, all at positions q0
    .. q0+Lq-1, against a paged fp8 key cache that holds keys 0 .. q0+Lq-1
    (prefill_chunk_varlen with equal chunks).

    q [B,Lq,H,D] fp8 codes (uint8) with q_scale [B,Lq,H] fp32, or bf16 with
    q_scale None; w [B,Lq,H] fp32, k_cache [P,page,D] uint8, k_scale [P,page]
    fp32, block_table [B,max_pages] int32.  Returns (idx int32 [B,Lq,topk] of
    absolute positions, score fp32 or None)."""
    B, Lq, H, D = q.shape
    if tuple(w.shape) != (B, Lq, H) or block_table.shape[0] != B:
        raise ValueError("w / block_table shape mismatch")
    if q_scale is not None and tuple(q_scale.shape) != (B, Lq, H):
        raise ValueError("q_scale must be [B, Lq, H]")
    dev = q.device
    cu = torch.arange(0, (B + 1) * Lq, Lq, dtype=torch.int32, device=dev)
    qs = torch.full((B,), int(q0), dtype=torch.int32, device=dev)
    qsc = None if q_scale is None else q_scale.reshape(B * Lq, H)
    idx, val = prefill_chunk_varlen(q.reshape(B * Lq, H, D), qsc, w.reshape(B * Lq, H), cu, qs,
                                    k_cache, k_scale, block_table, topk, int(q0) + Lq,
                                    want_topk_score=want_topk_score, workspace=workspace)
    return idx.view(B, Lq, topk), None if val is None else val.view(B, Lq, topk)
