"""Python binding of libdiagattn: argument marshalling only.

Each function takes torch tensors that live on the GPU, passes their
pointers and the current HIP stream to the C entry point of the same name
(``da_<name>`` in include/diagattn.h) and returns the output tensors.
PyTorch supplies device memory and streams; every step of the computation
runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from ctypes import c_int64 as ctypes_i64

from ._native import DaKvCache, DaMask, check, load

DENSE, BAND, ROWDIAG = 0, 1, 2
_DTYPE = {torch.float32: 0, torch.bfloat16: 1}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_cuda(name: str, *ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: every tensor must be on the GPU")


def mask(mode: int, W: int, B: int, G: int, causal: bool = True) -> DaMask:
    return DaMask(int(mode), int(W), int(B), int(G), int(bool(causal)))


def keep_count(m: DaMask, pos: int, prompt_len: int, n_keys: int = 0) -> int:
    r = load().da_keep_count(m, pos, prompt_len, n_keys)
    check(0 if r >= 0 else int(r), "da_keep_count")
    return int(r)


def keep_cap(m: DaMask, max_pos: int, max_prompt: int, n_keys: int = 0, head_wb=None) -> int:
    """Bound on keep-set sizes (sizes ``cap``).  With per-head masks
    ``head_wb`` (host [hq, 2] (W, B) pairs), the bound of the widest head's
    mask: a kv group reads the keep-set of its widest (W, B)."""
    if head_wb is not None:
        wb = [(max(int(w), 0), max(int(b), 0)) for w, b in head_wb]
        m = DaMask(m.mode, max(w for w, _ in wb), max(b for _, b in wb), m.G, m.causal)
    r = load().da_keep_cap(m, max_pos, max_prompt, n_keys)
    check(0 if r >= 0 else int(r), "da_keep_cap")
    return int(r)


def keepset_build(m: DaMask, pos: torch.Tensor, prompt_len: torch.Tensor, cap: int,
                  n_keys: int = 0, max_runs: int = 0, count=None, idx=None,
                  n_runs=None, runs=None, head_wb=None):
    """Returns (count [n_q], idx [n_q, cap], n_runs [n_q] or None,
    runs [n_q, max_runs, 2] or None), all int32 on pos.device.  With
    ``head_wb`` (device int32 [n_heads, 2] (W, B) per head) one list per
    (query, head): count [n_q, n_heads], idx [n_q, n_heads, cap], ..."""
    return _keepset_build(m, pos, prompt_len, cap, n_keys, max_runs, count, idx, n_runs, runs,
                          0, 0, None, None, head_wb)[:4]


def keepset_tiles(m: DaMask, pos: torch.Tensor, prompt_len: torch.Tensor, cap: int, tile: int,
                  cap_tiles: int, n_keys: int = 0, tiles=None, n_tiles=None, head_wb=None):
    """keepset_build with the split-KV tile list: returns (count, idx,
    tiles [cap_tiles, 2] int32 (list, first entry), n_tiles [1] int64); a
    list is a query, or with ``head_wb`` a (query, head) pair q*n_heads + h."""
    if tile < 1:
        raise ValueError("keepset_tiles: tile must be >= 1")
    count, idx, _, _, tiles, n_tiles = _keepset_build(m, pos, prompt_len, cap, n_keys, 0, None,
                                                      None, None, None, tile, cap_tiles, tiles,
                                                      n_tiles, head_wb)
    return count, idx, tiles, n_tiles


def _keepset_build(m, pos, prompt_len, cap, n_keys, max_runs, count, idx, n_runs, runs,
                   tile, cap_tiles, tiles, n_tiles, head_wb=None):
    _need_cuda("keepset_build", pos, prompt_len)
    n_q = pos.numel()
    dev = pos.device
    if head_wb is not None:
        if head_wb.dtype != torch.int32 or not head_wb.is_contiguous() or head_wb.dim() != 2 or \
                head_wb.shape[1] != 2 or head_wb.shape[0] < 1 or head_wb.device != dev:
            raise ValueError("keepset_build: head_wb must be a contiguous int32 [n_heads, 2] tensor "
                             "on the device of pos")
        nh, lead = head_wb.shape[0], (n_q, head_wb.shape[0])
    else:
        nh, lead = 1, (n_q,)
    if count is None:
        count = torch.empty(lead, dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty(lead + (cap,), dtype=torch.int32, device=dev)
    if max_runs > 0:
        if n_runs is None:
            n_runs = torch.empty(lead, dtype=torch.int32, device=dev)
        if runs is None:
            runs = torch.empty(lead + (max_runs, 2), dtype=torch.int32, device=dev)
    for t in (pos, prompt_len, count, idx, n_runs, runs, tiles):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError("keepset_build: int32 contiguous tensors expected")
    if pos.numel() != n_q or prompt_len.numel() != n_q or count.numel() < n_q * nh or \
            idx.numel() < n_q * nh * cap or \
            (n_runs is not None and (n_runs.numel() < n_q * nh or runs.numel() < n_q * nh * max_runs * 2)):
        raise ValueError("keepset_build: pos, prompt_len [n_q], count [n_q(, n_heads)] and "
                         "idx [n_q(, n_heads), cap] expected")
    if tile > 0:
        if tiles is None:
            tiles = torch.empty((max(cap_tiles, 0), 2), dtype=torch.int32, device=dev)
        if n_tiles is None:
            n_tiles = torch.empty(1, dtype=torch.int64, device=dev)
        if tiles.numel() < 2 * cap_tiles or n_tiles.dtype != torch.int64 or n_tiles.numel() < 1:
            raise ValueError("keepset_build: tiles int32 [cap_tiles, 2], n_tiles int64 [1] expected")
    else:
        tiles = n_tiles = None
    check(load().da_keepset_build(m, n_q, _ptr(pos), _ptr(prompt_len), n_keys, nh, _ptr(head_wb), cap,
                                  _ptr(count), _ptr(idx), max_runs, _ptr(n_runs), _ptr(runs),
                                  int(tile), _ptr(tiles), int(cap_tiles), _ptr(n_tiles),
                                  _stream(pos)),
          "da_keepset_build")
    return count, idx, n_runs, runs, tiles, n_tiles


def kv_cache(k: torch.Tensor, v: torch.Tensor,
             block_table: Optional[torch.Tensor] = None) -> DaKvCache:
    """Descriptor for a contiguous [n_seq, hkv, Lmax, hd] cache (no block
    table) or a paged [n_pages, hkv, page_size, hd] cache with a
    [n_seq, pages_per_seq] int32 block table."""
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v caches must share shape, strides and dtype")
    if k.dim() != 4 or k.stride(3) != 1:
        raise ValueError("cache must be 4-D with a contiguous head_dim")
    d = DaKvCache()
    d.k, d.v = k.data_ptr(), v.data_ptr()
    d.page_stride, d.head_stride, d.slot_stride = k.stride(0), k.stride(1), k.stride(2)
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [n_seq, pages] tensor")
        d.page_size = k.shape[2]
        d.bt_stride = block_table.shape[1]
        d.block_table = block_table.data_ptr()
        d.n_seq = block_table.shape[0]
        d.n_pages = k.shape[0]
        d.max_len = block_table.shape[1] * k.shape[2]
    else:
        d.page_size, d.bt_stride, d.block_table = 0, 0, None
        d.n_seq = d.n_pages = k.shape[0]
        d.max_len = k.shape[2]
    return d


def decode_workspace_bytes(n_q: int, hq: int, head_dim: int, cap: int, split: int) -> int:
    r = load().da_decode_workspace_bytes(n_q, hq, head_dim, cap, split)
    check(0 if r >= 0 else int(r), "da_decode_workspace_bytes")
    return int(r)


def decode_workspace(n_q: int, hq: int, head_dim: int, cap: int, split: int,
                     device) -> Optional[torch.Tensor]:
    """A decode workspace of the right size (None when none is needed)."""
    need = decode_workspace_bytes(n_q, hq, head_dim, cap, split)
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device=device)


def sparse_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       seq: torch.Tensor, count: torch.Tensor, idx: torch.Tensor, *,
                       split: int, block_table: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, out=None, lse=None,
                       want_lse: bool = False, workspace=None):
    """q [n_q, hq, hd]; caches as in ``kv_cache``; seq [n_q] int32; one list
    per query, count [n_q] and idx [n_q, cap] int32, or one per kv head,
    count [n_q, hkv] and idx [n_q, hkv, cap] (``keepset_build`` with a
    [hkv, 2] ``head_wb``).  ``workspace``: from ``decode_workspace``
    (reusable across calls on one stream); allocated per call when omitted.
    Returns (out [n_q, hq, hd], lse [n_q, hq] or None)."""
    _need_cuda("sparse_decode_attn", q, k_cache, v_cache, seq, count, idx, block_table)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [n_q, hq, hd] tensor")
    if q.dtype not in _DTYPE or q.dtype != k_cache.dtype:
        raise ValueError("q and the caches must share dtype fp32 or bf16")
    n_q, hq, hd = q.shape
    hkv = k_cache.shape[1]
    lh = hkv if idx.dim() == 3 else 1
    if idx.dim() not in (2, 3) or idx.shape[0] != n_q or (lh > 1 and idx.shape[1] != hkv) or \
            not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be a contiguous int32 [n_q, cap] or [n_q, hkv, cap] tensor")
    if seq.dtype != torch.int32 or not seq.is_contiguous() or seq.numel() != n_q:
        raise ValueError("seq must be a contiguous int32 [n_q] tensor")
    if count.dtype != torch.int32 or not count.is_contiguous() or count.numel() != n_q * lh:
        raise ValueError("count must be a contiguous int32 tensor of n_q (or n_q * hkv) entries")
    cap = idx.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((n_q, hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(n_q, hq, hd, cap, split, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    kv = kv_cache(k_cache, v_cache, block_table)
    check(load().da_sparse_decode_attn(_ptr(q), _DTYPE[q.dtype], n_q, hq, hkv, hd, float(scale),
                                       kv, _ptr(seq), _ptr(count), _ptr(idx), cap, lh, split,
                                       _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                       _stream(q)),
          "da_sparse_decode_attn")
    return out, lse


def sparse_decode_attn_masked(m: DaMask, q: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                              prompt_len: torch.Tensor, *, cap: int, split: int,
                              block_table: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None, out=None, lse=None,
                              want_lse: bool = False, workspace=None, count=None, idx=None,
                              want_lists: bool = False, k_new=None, v_new=None, head_wb=None):
    """Decode with the keep-set computed in the kernel from (pos, prompt_len,
    mask) -- one launch for build + attention.  q [n_q, hq, hd]; caches as in
    ``kv_cache``; seq/pos/prompt_len [n_q] int32.  With ``want_lists`` (or
    given count/idx) the lists keepset_build would write are written too.
    k_new/v_new [n_q, hkv, hd]: the new token's K/V rows, appended to the
    cache at pos before attention (one query per request).  head_wb
    [hq, 2] int32 on the device: a (W, B) per query head.
    Returns (out, lse or None, count or None, idx or None)."""
    return _decode_masked(m, q, k_cache, v_cache, seq, pos, prompt_len, cap, split, block_table,
                          scale, out, lse, want_lse, workspace, count, idx, want_lists, k_new,
                          v_new, head_wb, noalloc=False)


def sparse_decode_attn_masked_noalloc(m: DaMask, q: torch.Tensor, k_cache: torch.Tensor,
                                      v_cache: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                                      prompt_len: torch.Tensor, *, cap: int, split: int, out,
                                      block_table: Optional[torch.Tensor] = None,
                                      scale: Optional[float] = None, lse=None, count=None,
                                      idx=None, k_new=None, v_new=None, head_wb=None):
    """``sparse_decode_attn_masked`` through the allocation-free entry point:
    no workspace (the library's per-GPU scratch array serves instead) and no
    output allocation (``out``, and ``lse``/``count``/``idx`` when wanted,
    are the caller's).  Returns (out, lse, count, idx)."""
    if out is None:
        raise ValueError("sparse_decode_attn_masked_noalloc: pass `out` (nothing is allocated)")
    return _decode_masked(m, q, k_cache, v_cache, seq, pos, prompt_len, cap, split, block_table,
                          scale, out, lse, False, None, count, idx, False, k_new, v_new, head_wb,
                          noalloc=True)


def decode_scratch_bytes() -> int:
    """Scratch bytes behind the allocation-free decode entry point."""
    return int(load().da_decode_scratch_bytes())


def _decode_masked(m, q, k_cache, v_cache, seq, pos, prompt_len, cap, split, block_table, scale,
                   out, lse, want_lse, workspace, count, idx, want_lists, k_new, v_new, head_wb,
                   noalloc):
    _need_cuda("sparse_decode_attn_masked", q, k_cache, v_cache, seq, pos, prompt_len, block_table,
               k_new, v_new, head_wb, out, lse, count, idx)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [n_q, hq, hd] tensor")
    if q.dtype not in _DTYPE or q.dtype != k_cache.dtype:
        raise ValueError("q and the caches must share dtype fp32 or bf16")
    n_q, hq, hd = q.shape
    hkv = k_cache.shape[1]
    for t in (seq, pos, prompt_len):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != n_q:
            raise ValueError("seq, pos and prompt_len must be contiguous int32 [n_q] tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((n_q, hq), dtype=torch.float32, device=q.device)
    if want_lists and count is None:
        count = torch.empty(n_q, dtype=torch.int32, device=q.device)
        idx = torch.empty((n_q, cap), dtype=torch.int32, device=q.device)
    if (count is None) != (idx is None):
        raise ValueError("count and idx go together")
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous() or
                            tuple(idx.shape) != (n_q, cap) or count.dtype != torch.int32):
        raise ValueError("idx must be a contiguous int32 [n_q, cap] tensor, count int32 [n_q]")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if head_wb is not None and (head_wb.dtype != torch.int32 or not head_wb.is_contiguous() or
                                tuple(head_wb.shape) != (hq, 2)):
        raise ValueError("head_wb must be a contiguous int32 [hq, 2] tensor")
    for t in (k_new, v_new):
        if t is not None and (t.dtype != q.dtype or not t.is_contiguous() or
                              tuple(t.shape) != (n_q, hkv, hd)):
            raise ValueError("k_new and v_new must be contiguous [n_q, hkv, hd] tensors of q's dtype")
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or
                            tuple(lse.shape) != (n_q, hq)):
        raise ValueError("lse must be a contiguous fp32 [n_q, hq] tensor")
    kv = kv_cache(k_cache, v_cache, block_table)
    if noalloc:
        check(load().da_sparse_decode_attn_masked_noalloc(
                  m, _ptr(q), _DTYPE[q.dtype], n_q, hq, hkv, hd, float(scale), kv, _ptr(seq),
                  _ptr(pos), _ptr(prompt_len), _ptr(head_wb), _ptr(k_new), _ptr(v_new), cap, split,
                  _ptr(count), _ptr(idx), _ptr(out), _ptr(lse), _stream(q)),
              "da_sparse_decode_attn_masked_noalloc")
        return out, lse, count, idx
    if workspace is None:
        workspace = decode_workspace(n_q, hq, hd, cap, split, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().da_sparse_decode_attn_masked(m, _ptr(q), _DTYPE[q.dtype], n_q, hq, hkv, hd,
                                              float(scale), kv, _ptr(seq), _ptr(pos),
                                              _ptr(prompt_len), _ptr(head_wb), _ptr(k_new), _ptr(v_new),
                                              cap, split, _ptr(count), _ptr(idx),
                                              _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                              _stream(q)),
          "da_sparse_decode_attn_masked")
    return out, lse, count, idx


def ring_pages(m: DaMask, prompt_len: int, max_len: int, page_size: int) -> int:
    """KV pages one request needs when rows older than the live window are
    recycled (prompt pages plus a ring of window pages)."""
    r = load().da_ring_pages(m, int(prompt_len), int(max_len), int(page_size))
    check(r if r < 0 else 0, "da_ring_pages")
    return int(r)


def ring_block_table(m: DaMask, prompt_len, max_len: int, page_size: int, first_page: int = 0):
    """Static block table whose window pages form a ring per request.
    prompt_len: host ints [n_seq].  Returns (int32 CPU tensor [n_seq,
    ceil(max_len / page_size)], total pages)."""
    p = torch.as_tensor(prompt_len, dtype=torch.int32).contiguous()
    n_seq = p.numel()
    stride = -(-int(max_len) // int(page_size))
    bt = torch.empty((n_seq, stride), dtype=torch.int32)
    total = ctypes.c_int64(0)
    check(load().da_ring_block_table(m, n_seq, p.data_ptr(), int(max_len), int(page_size),
                                     int(first_page), stride, bt.data_ptr(), ctypes.byref(total)),
          "da_ring_block_table")
    return bt, int(total.value)


def decode_schedule(cost, wg_per_query: int, n_cu: int = 0) -> torch.Tensor:
    """Batch order balancing the decode step over the compute units: cost
    = host per-query work (e.g. keep_count of each query), wg_per_query =
    workgroups a query launches (hkv).  Returns an int32 CPU tensor: the
    query for each batch slot."""
    c = torch.as_tensor(cost, dtype=torch.int64).contiguous()
    order = torch.empty(c.numel(), dtype=torch.int32)
    check(load().da_decode_schedule(c.data_ptr(), c.numel(), int(wg_per_query), int(n_cu),
                                    order.data_ptr()),
          "da_decode_schedule")
    return order


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, grid: int,
                   nbytes: Optional[int] = None, offset: int = 0, loads_in_flight: int = 8) -> None:
    """Streams `nbytes` bytes of `buf` starting at byte `offset` (measurement)."""
    _need_cuda("hbm_read_probe", buf, sink)
    total = buf.numel() * buf.element_size()
    nbytes = total - offset if nbytes is None else nbytes
    if offset < 0 or offset + nbytes > total or sink.numel() < grid or sink.element_size() != 4:
        raise ValueError("hbm_read_probe: range outside the buffer or sink too small")
    check(load().da_hbm_read_probe(buf.data_ptr() + offset, nbytes, sink.data_ptr(), grid,
                                   int(loads_in_flight), _stream(buf)),
          "da_hbm_read_probe")


def kept_row_offsets(k_cache: torch.Tensor, seq: torch.Tensor, count: torch.Tensor, idx: torch.Tensor,
                     block_table: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Byte offsets (int64, device) from the cache's base of the K (and V)
    rows a decode step keeps: every kv head of every listed entry of the
    per-query lists count [n_q], idx [n_q, cap], in (query, kv head, entry)
    order, addressed as ``kv_cache`` describes the cache.  Measurement
    set-up for ``gather_read_probe``, computed with torch ops."""
    kv = kv_cache(k_cache, k_cache, block_table)
    esz = k_cache.element_size()
    n_q, cap = idx.shape
    hkv = k_cache.shape[1]
    dev = idx.device
    valid = torch.arange(cap, device=dev)[None, :] < count.long()[:, None]
    j = idx.long().clamp(0, kv.max_len - 1)
    sq = seq.long()[:, None]
    if block_table is not None:
        page = block_table.long()[sq.clamp(0, kv.n_seq - 1), j // kv.page_size].clamp(0, kv.n_pages - 1)
        row = page * kv.page_stride + (j % kv.page_size) * kv.slot_stride
    else:
        row = sq.clamp(0, kv.n_pages - 1) * kv.page_stride + j * kv.slot_stride
    off = row[:, None, :] + torch.arange(hkv, device=dev)[None, :, None] * kv.head_stride
    return (off[valid[:, None, :].expand(n_q, hkv, cap)] * esz).contiguous()


def gather_read_probe(k_cache: torch.Tensor, v_cache: torch.Tensor, offsets: torch.Tensor,
                      sink: torch.Tensor, grid: int, *, loads_in_flight: int = 2) -> None:
    """Reads the K and V rows at the byte ``offsets`` (``kept_row_offsets``)
    and nothing else (measurement); sink [grid] int32 receives one XOR a
    workgroup."""
    _need_cuda("gather_read_probe", k_cache, v_cache, offsets, sink)
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or \
            not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("gather_read_probe: k and v must be contiguous and alike")
    if offsets.dtype != torch.int64 or not offsets.is_contiguous():
        raise ValueError("gather_read_probe: offsets must be contiguous int64")
    if sink.numel() < grid or sink.element_size() != 4:
        raise ValueError("gather_read_probe: sink needs grid 32-bit words")
    row_bytes = k_cache.shape[-1] * k_cache.element_size()
    span = k_cache.numel() * k_cache.element_size()
    check(load().da_gather_read_probe(_ptr(k_cache), _ptr(v_cache), _ptr(offsets), offsets.numel(),
                                      int(row_bytes), int(span), _ptr(sink), int(grid), int(loads_in_flight),
                                      _stream(offsets)),
          "da_gather_read_probe")


def prefill_tiles_build(m: DaMask, prompt_len: torch.Tensor, n: int, tiles=None) -> torch.Tensor:
    """Tile lists of the keep-set for prefill of len(prompt_len) sequences of
    n tokens (uint8 device buffer in the layout of include/diagattn.h)."""
    _need_cuda("prefill_tiles_build", prompt_len)
    if prompt_len.dtype != torch.int32 or not prompt_len.is_contiguous():
        raise ValueError("prompt_len must be contiguous int32")
    bsz = prompt_len.numel()
    nbytes = int(load().da_prefill_tiles_bytes(bsz, n))
    check(0 if nbytes >= 0 else nbytes, "da_prefill_tiles_bytes")
    if tiles is None:
        tiles = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=prompt_len.device)
    check(load().da_prefill_tiles_build(m, bsz, n, _ptr(prompt_len), _ptr(tiles),
                                        tiles.numel(), _stream(prompt_len)),
          "da_prefill_tiles_build")
    return tiles


def band_prefill_attn(m: DaMask, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      prompt_len: torch.Tensor, *, tiles: Optional[torch.Tensor] = None,
                      scale: Optional[float] = None, out=None, lse=None,
                      want_lse: bool = False):
    """q [batch, heads, n, hd], k/v [batch, kv_heads, n, hd] bf16 (head_dim
    contiguous); prompt_len [batch] int32; tiles from ``prefill_tiles_build``
    (built here when omitted).  Returns (out, lse or None)."""
    _need_cuda("band_prefill_attn", q, k, v, prompt_len, tiles)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [batch, heads, n, hd] and k, v [batch, kv_heads, n, hd]")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("band_prefill_attn takes bf16 tensors")
    bsz, heads, n, hd = q.shape
    if k.shape[0] != bsz or k.shape[2] != n or k.shape[3] != hd:
        raise ValueError("k/v shape does not match q")
    if prompt_len.dtype != torch.int32 or prompt_len.numel() != bsz:
        raise ValueError("prompt_len must be int32 [batch]")
    if tiles is None:
        tiles = prefill_tiles_build(m, prompt_len, n)
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((bsz, heads, n), dtype=torch.float32, device=q.device)
    for t in (q, k, v, out):
        if t.stride(3) != 1:
            raise ValueError("head_dim must be contiguous")
    st = (ctypes_i64 * 12)(*[t.stride(d) for t in (q, k, v, out) for d in (0, 1, 2)])
    check(load().da_band_prefill_attn(m, 1, bsz, heads, k.shape[1], n, hd, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(out), st, _ptr(prompt_len), _ptr(tiles),
                                      tiles.numel() * tiles.element_size(), float(scale), _ptr(lse),
                                      _stream(q)),
          "da_band_prefill_attn")
    return out, lse
