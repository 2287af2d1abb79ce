"""torch-facing calls of the paged decode library.

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, then their pointers and the current HIP stream go to libpa.so.
Every step of the computation runs in the library's HIP kernels; there is
no fallback path.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

_BF16 = torch.bfloat16


class PagedAttentionError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libpa error {code}: {message}")
        self.code = code


def _check(rc: int) -> None:
    if rc != _lib.PA_OK:
        raise PagedAttentionError(rc, _lib.last_error())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor) -> _lib.KVCacheDesc:
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != _BF16 or t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor "
                             "[num_blocks, block_size, num_kv_heads, head_size]")
    if k_cache.shape != v_cache.shape or k_cache.device != v_cache.device:
        raise ValueError("k_cache and v_cache must have the same shape and device")
    nb, bs, hkv, d = k_cache.shape
    return _lib.KVCacheDesc(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, d,
                            _lib.PA_DTYPE_BF16)


def _need(t, name, dtype, shape, device):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


_workspaces: dict = {}


def _workspace(device, nbytes: int) -> torch.Tensor:
    """A scratch buffer per (device, stream), grown on demand.

    One buffer per stream keeps calls that share it ordered; its contents
    need no initialisation.
    """
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def decode_workspace_bytes(k_cache, num_seqs, num_q_heads, max_blocks_per_seq) -> int:
    desc = _cache_desc(k_cache, k_cache)
    return int(_lib.lib().pa_decode_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                   max_blocks_per_seq))


def decode_multi_workspace_bytes(k_cache, num_seqs, q_len, num_q_heads, max_blocks_per_seq) -> int:
    desc = _cache_desc(k_cache, k_cache)
    return int(_lib.lib().pa_decode_multi_workspace_bytes(ctypes.byref(desc), num_seqs, q_len, num_q_heads,
                                                         max_blocks_per_seq))


def decode_shared_workspace_bytes(k_cache, num_seqs, num_q_heads, max_blocks_per_seq, num_groups) -> int:
    desc = _cache_desc(k_cache, k_cache)
    return int(_lib.lib().pa_decode_shared_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                          max_blocks_per_seq, num_groups))


def decode_shared_tree_workspace_bytes(k_cache, num_seqs, num_q_heads, max_blocks_per_seq) -> int:
    desc = _cache_desc(k_cache, k_cache)
    return int(_lib.lib().pa_decode_shared_tree_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                               max_blocks_per_seq))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, workspace=None):
    """Paged decode attention; returns ``out`` (bf16 ``[num_seqs, num_q_heads, head_size]``).

    ``block_tables`` int32 ``[num_seqs, max_blocks_per_seq]``, ``context_lens``
    int32 ``[num_seqs]`` (newest token included). Runs on the current stream.
    """
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_workspace_bytes(ctypes.byref(desc), S, hq, mb))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode(ctypes.byref(desc), _ptr(q), _ptr(block_tables), _ptr(context_lens), S, hq,
                         mb, float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_step(q, k, v, k_cache, v_cache, block_tables, context_lens, scale, out=None, workspace=None):
    """One decode step in one call: each sequence's new token (``k``, ``v``:
    bf16 ``[num_seqs, num_kv_heads, head_size]``) is attended at position
    ``context_lens[s] - 1`` and written to the slot its block table names
    there; returns ``out``. Equal to ``reshape_and_cache`` with those slots
    followed by ``decode``."""
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    _need(k, "k", _BF16, (S, k_cache.shape[2], k_cache.shape[3]), dev)
    _need(v, "v", _BF16, (S, k_cache.shape[2], k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_step_workspace_bytes(ctypes.byref(desc), S, hq, mb))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(block_tables),
                              _ptr(context_lens), S, hq, mb, float(scale), _ptr(out), _ptr(workspace), ws_bytes,
                              _stream(dev)))
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out):
    """``decode`` through the entry point that allocates nothing
    (``pa_decode_noalloc``): the partial results go to the library's static
    device scratch, so ``out`` must be given. Calls on one GPU that overlap
    in time race on that scratch; keep them on one stream."""
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    _need(out, "out", _BF16, (S, hq, d), dev)
    _check(_lib.lib().pa_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(block_tables), _ptr(context_lens), S,
                                        hq, mb, float(scale), _ptr(out), _stream(dev)))
    return out


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, workspace=None):
    """Causal attention of several new tokens per sequence; returns ``out``.

    ``q``: bf16 ``[num_seqs, q_len, num_q_heads, head_size]``; new token j of
    a sequence with context length n attends over positions 0..n-q_len+j.
    The new tokens must be in the cache already (``reshape_and_cache``).
    """
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, ql, hq, d = q.shape
    _need(q, "q", _BF16, (S, ql, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, ql, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_multi_workspace_bytes(ctypes.byref(desc), S, ql, hq, mb))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_multi(ctypes.byref(desc), _ptr(q), _ptr(block_tables), _ptr(context_lens), S, ql, hq,
                               mb, float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_shared(q, k_cache, v_cache, block_tables, context_lens, group_starts, shared_blocks, scale,
                  out=None, workspace=None):
    """Decode attention for groups of sequences that share leading blocks.

    ``group_starts`` int32 ``[G + 1]`` and ``shared_blocks`` int32 ``[G]`` on
    the cache's device: group g is sequences ``group_starts[g]`` ..
    ``group_starts[g+1]-1`` and their tables agree on the first
    ``shared_blocks[g]`` entries. Other arguments as ``decode``.
    """
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    G = shared_blocks.shape[0] if shared_blocks.dim() == 1 else -1
    _need(shared_blocks, "shared_blocks", torch.int32, (G,), dev)
    _need(group_starts, "group_starts", torch.int32, (G + 1,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_shared_workspace_bytes(ctypes.byref(desc), S, hq, mb, G))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_shared(ctypes.byref(desc), _ptr(q), _ptr(block_tables), _ptr(context_lens), S, hq, mb,
                                _ptr(group_starts), _ptr(shared_blocks), G, float(scale), _ptr(out),
                                _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_shared_tree(q, k_cache, v_cache, block_tables, context_lens, shared_prev, scale, out=None,
                       workspace=None):
    """Decode attention for sequences that form a tree of shared prefixes,
    listed depth first.

    ``shared_prev`` int32 ``[num_seqs]`` on the cache's device: sequence i's
    table agrees with sequence i-1's on its first ``shared_prev[i]`` entries
    (entry 0 is ignored). Other arguments as ``decode``.
    """
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    _need(shared_prev, "shared_prev", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_shared_tree_workspace_bytes(ctypes.byref(desc), S, hq, mb))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_shared_tree(ctypes.byref(desc), _ptr(q), _ptr(block_tables), _ptr(context_lens), S, hq,
                                     mb, _ptr(shared_prev), float(scale), _ptr(out), _ptr(workspace), ws_bytes,
                                     _stream(dev)))
    return out


def share_plan(k_cache, context_lens, num_q_heads, max_blocks_per_seq, group_starts=None, shared_blocks=None,
               shared_prev=None, plan=None):
    """The plan of a sharing-aware decode (segments and member records),
    from the context lengths and the declaration: groups (``group_starts``,
    ``shared_blocks``) or, with ``shared_prev``, a chain. Returns the plan
    (a uint8 tensor on the cache's device), reusable by
    ``decode_shared_planned`` for every layer that decodes the same batch."""
    desc = _cache_desc(k_cache, k_cache)
    dev = k_cache.device
    S = context_lens.shape[0]
    _need(context_lens, "context_lens", torch.int32, (S,), dev)
    G = 0
    if shared_prev is not None:
        _need(shared_prev, "shared_prev", torch.int32, (S,), dev)
    elif shared_blocks is not None:
        G = shared_blocks.shape[0]
        _need(shared_blocks, "shared_blocks", torch.int32, (G,), dev)
        _need(group_starts, "group_starts", torch.int32, (G + 1,), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_share_plan_bytes(ctypes.byref(desc), S, num_q_heads, max_blocks_per_seq))
    if plan is None:
        plan = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check(lib.pa_share_plan(ctypes.byref(desc), _ptr(context_lens), S, num_q_heads, max_blocks_per_seq,
                             _ptr(group_starts) if shared_prev is None else None,
                             _ptr(shared_blocks) if shared_prev is None else None, G, _ptr(shared_prev), _ptr(plan),
                             plan.numel(), _stream(dev)))
    return plan


def decode_shared_planned(q, k_cache, v_cache, block_tables, plan, scale, out=None, workspace=None):
    """Sharing-aware decode on a plan from ``share_plan`` (made for the same
    sizes and context lengths). Other arguments as ``decode``."""
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    S, hq, d = q.shape
    _need(q, "q", _BF16, (S, hq, k_cache.shape[3]), dev)
    mb = block_tables.shape[1] if block_tables.dim() == 2 else -1
    _need(block_tables, "block_tables", torch.int32, (S, mb), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, (S, hq, d), dev)
    lib = _lib.lib()
    nbytes = int(lib.pa_decode_shared_planned_workspace_bytes(ctypes.byref(desc), S, hq, mb))
    if workspace is None and nbytes:
        workspace = _workspace(dev, nbytes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_shared_planned(ctypes.byref(desc), _ptr(q), _ptr(block_tables), S, hq, mb, _ptr(plan),
                                        float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping) -> None:
    """Scatter new tokens' K/V (bf16 ``[T, num_kv_heads, head_size]``) into
    their slots (int64 ``[T]``; negative = skip), in place, on the current stream."""
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    T = k.shape[0]
    _need(k, "k", _BF16, (T,) + tuple(k_cache.shape[2:]), dev)
    _need(v, "v", _BF16, (T,) + tuple(k_cache.shape[2:]), dev)
    _need(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    _check(_lib.lib().pa_reshape_and_cache(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping),
                                           T, _stream(dev)))


def copy_blocks(k_cache, v_cache, src_dst_pairs) -> None:
    """Copy-on-write: block ``dst`` becomes a copy of block ``src`` for every
    row of ``src_dst_pairs`` (int64 ``[P, 2]``, device), K and V, in place."""
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    P = src_dst_pairs.shape[0]
    _need(src_dst_pairs, "src_dst_pairs", torch.int64, (P, 2), dev)
    _check(_lib.lib().pa_copy_blocks(ctypes.byref(desc), _ptr(src_dst_pairs), P, _stream(dev)))


def swap_blocks(k_cache, v_cache, host_k, host_v, src_dst_pairs, direction: str) -> None:
    """Move whole blocks between the device cache and a host cache.

    ``host_k``/``host_v``: pinned CPU bf16 tensors ``[host_blocks, block_size,
    num_kv_heads, head_size]`` (the device cache's block shape). ``src_dst_pairs``: int64 ``[P, 2]`` on the
    cache's device. ``direction`` "out": host block dst <- device block src;
    "in": device block dst <- host block src. Asynchronous on the current
    stream (synchronize before reading swapped-out blocks on the host).
    """
    desc = _cache_desc(k_cache, v_cache)
    dev = k_cache.device
    shape = (host_k.shape[0],) + tuple(k_cache.shape[1:])
    for name, t in (("host_k", host_k), ("host_v", host_v)):
        if t.dtype != _BF16 or tuple(t.shape) != shape or not t.is_contiguous() or t.is_cuda or not t.is_pinned():
            raise ValueError(f"{name}: expected a contiguous pinned CPU bf16 tensor {shape}")
    P = src_dst_pairs.shape[0]
    _need(src_dst_pairs, "src_dst_pairs", torch.int64, (P, 2), dev)
    d = {"out": _lib.PA_SWAP_OUT, "in": _lib.PA_SWAP_IN}[direction]
    _check(_lib.lib().pa_swap_blocks(ctypes.byref(desc), _ptr(host_k), _ptr(host_v), shape[0],
                                     _ptr(src_dst_pairs), P, d, _stream(dev)))


def probe_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Plain 16-byte-vector copy of ``src`` into ``dst`` (measurement helper)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(_lib.lib().pa_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device)))


def probe_read_sink_bytes() -> int:
    """Bytes of the sink buffer pa_probe_read folds its loads into."""
    return int(_lib.lib().pa_probe_read_sink_bytes())


def probe_read(src: torch.Tensor, sink: torch.Tensor = None) -> torch.Tensor:
    """Read all of ``src`` with 16-byte vector loads (measurement helper);
    returns the sink buffer the probe folds its loads into."""
    lib = _lib.lib()
    need = int(lib.pa_probe_read_sink_bytes())
    if sink is None:
        sink = torch.empty(need, dtype=torch.uint8, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check(lib.pa_probe_read(_ptr(src), nbytes, _ptr(sink), sink.numel() * sink.element_size(),
                             _stream(src.device)))
    return sink
