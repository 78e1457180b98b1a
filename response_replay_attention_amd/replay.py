"""Replay driver: the prompt's paged K/V with its device page table, and the
calls that replay one response (forward, LSE merge, response-only backward)
or a whole group of responses one after another, and the chunked capture
that writes the prompt's pages in the first place.

The group loop follows the pages' serial suffix replay: the shared prompt is
captured once and each response branch is replayed, back-propagated and freed
before the next one, so peak memory follows the longest response rather than
the group size (DeepRead summary page, "Method"; LongStraw review page,
section 2, item 3).  Everything here is allocation and argument marshalling;
the arithmetic runs in libls_replay.so.
"""
from __future__ import annotations

import contextlib
import functools
import inspect
import math
from dataclasses import dataclass
from typing import Iterable, List, Optional

import numpy as np
import torch

from . import binding as B


def _on_stream(fn):
    """Run a driver with ``stream`` (a ``torch.cuda.Stream``, a raw handle or
    None for the current stream) as torch's current stream, so that every
    buffer the driver allocates belongs to the stream its kernels run on and
    the caching allocator never hands it to other work while they may still
    read it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapped(*args, **kw):
        stream = sig.bind_partial(*args, **kw).arguments.get("stream")
        if stream is None:
            ctx = contextlib.nullcontext()
        elif isinstance(stream, int):
            ctx = torch.cuda.stream(torch.cuda.ExternalStream(stream))
        else:
            ctx = torch.cuda.stream(stream)
        with ctx:
            return fn(*args, **kw)
    return wrapped


def _upload(arr, dev: torch.device) -> torch.Tensor:
    """A host int32 array on ``dev`` without a host synchronisation: staged
    through pinned memory and copied on the current stream (a plain copy from
    pageable memory waits for all earlier work on the stream, which leaves the
    GPU idle while the host prepares the next launches)."""
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dev.type != "cuda":
        return t.to(dev)
    return t.pin_memory().to(dev, non_blocking=True)


class PromptCache:
    """A detached prompt: bf16 K/V pools ``[num_phys, Hkv, 256, d]`` (never
    written by this package) and the page table that maps its logical pages to
    pool slots and deals them to ``num_splits`` emulated context-parallel
    ranks."""

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, prompt_len: int,
                 l2p=None, num_splits: int = 1, policy: int = B.LS_SPLIT_CONTIGUOUS,
                 block_pages: int = 1, owner=None):
        if k_pool.shape != v_pool.shape or k_pool.dim() != 4:
            raise ValueError("k_pool and v_pool must both be [num_phys, Hkv, 256, d]")
        self.k_pool, self.v_pool = k_pool, v_pool
        self.prompt_len = int(prompt_len)
        self.num_phys = int(k_pool.shape[0])
        self.hkv = int(k_pool.shape[1])
        self.head_dim = int(k_pool.shape[3])
        self.num_pages = (self.prompt_len + B.PAGE_SIZE - 1) // B.PAGE_SIZE
        self.num_splits = int(num_splits)
        l2p_np = (np.arange(self.num_pages, dtype=np.int32) if l2p is None
                  else np.asarray(l2p.cpu() if isinstance(l2p, torch.Tensor) else l2p, dtype=np.int32))
        order, offs = B.ls_kv_page_table(self.num_pages, B.PAGE_SIZE, self.prompt_len, l2p_np,
                                         self.num_phys, self.num_splits, policy, block_pages, owner)
        dev = k_pool.device
        self.l2p = l2p_np
        self.order = order
        self.split_offsets_host = np.ascontiguousarray(offs)  # kept alive: the table points at it
        self._l2p_dev = _upload(l2p_np, dev)
        self._order_dev = _upload(order, dev)
        self._offs_dev = _upload(self.split_offsets_host.copy(), dev)
        # the uploads run on the stream current here; table() orders the
        # stream a driver runs on after them
        self._ready = None
        if dev.type == "cuda":
            self._ready = torch.cuda.Event()
            self._ready.record(torch.cuda.current_stream(dev))
        self.pt = B.PageTable(
            self._l2p_dev.data_ptr() if self.num_pages else 0,
            self._order_dev.data_ptr() if self.num_pages else 0,
            self._offs_dev.data_ptr(), self.split_offsets_host.ctypes.data,
            self.num_pages, self.num_splits, self.num_phys)

    def table(self) -> "B.PageTable":
        """The page table for a launch on the current stream: the stream waits
        for the table's upload, and the table's device buffers are marked as
        used by it (so the caching allocator keeps them until its work is done)."""
        if self._ready is not None:
            s = torch.cuda.current_stream(self.k_pool.device)
            s.wait_event(self._ready)
            for t in (self._l2p_dev, self._order_dev, self._offs_dev):
                t.record_stream(s)
        return self.pt

    def shape(self, q: torch.Tensor, scale: Optional[float] = None, q_offset: int = 0,
              kv_rows: int = 0, flags: int = 0) -> B.AttnShape:
        hq, r, d = q.shape
        if d != self.head_dim:
            raise ValueError("head_dim mismatch between q and the pools")
        s = 1.0 / math.sqrt(d) if scale is None else float(scale)
        return B.make_shape(hq, self.hkv, d, self.prompt_len, r, s, q_offset=q_offset,
                            kv_rows=kv_rows, flags=flags)


@dataclass
class ForwardResult:
    o: torch.Tensor        # bf16 [Hq, R, d]
    lse: torch.Tensor      # fp32 [Hq, R]
    part_o: torch.Tensor   # fp32 [S+1, Hq, R, d]
    part_m: torch.Tensor   # fp32 [S+1, Hq, R]
    part_l: torch.Tensor


@_on_stream
def replay_forward(cache: PromptCache, q, k_resp, v_resp, scale=None, stream=None,
                   q_offset: int = 0) -> ForwardResult:
    """Partial attention per split + the causal response block, then the exact
    LSE merge.  With ``q_offset`` the rows of ``q`` are response tokens
    ``q_offset ..`` of a response whose K/V ``[Hkv, kv_rows, d]`` hold at least
    its first ``q_offset + R`` tokens."""
    sh = cache.shape(q, scale, q_offset, int(k_resp.shape[1]))
    hq, r, d = q.shape
    dev = q.device
    nparts = cache.num_splits + 1
    part_o = torch.empty(nparts, hq, r, d, dtype=torch.float32, device=dev)
    part_m = torch.empty(nparts, hq, r, dtype=torch.float32, device=dev)
    part_l = torch.empty(nparts, hq, r, dtype=torch.float32, device=dev)
    wsb = B.ls_replay_attn_fwd_workspace(sh, cache.pt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
    B.ls_replay_attn_fwd(sh, cache.table(), q, cache.k_pool, cache.v_pool, k_resp, v_resp,
                         part_o, part_m, part_l, ws, stream)
    o = torch.empty(hq, r, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(hq, r, dtype=torch.float32, device=dev)
    B.ls_lse_merge(nparts, hq * r, d, part_o, part_m, part_l, o, lse, stream)
    del ws
    return ForwardResult(o, lse, part_o, part_m, part_l)


@_on_stream
def score_group(cache: PromptCache, members: Iterable["Member"], scale=None, stream=None) -> List:
    """Forward-only scoring of a whole group in one pass over the prompt: the
    members' queries and response K/V are stacked along the response axis, the
    prompt splits are computed once for all of them (every K/V block serves
    every member's rows), the response block keeps each member to its own
    keys, and the merge yields every member's O and LSE.  Returns one
    ``(o, lse)`` pair per member (views into the stacked outputs)."""
    members = list(members)
    lens = [int(m.q.shape[1]) for m in members]
    offs = np.zeros(len(members) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(lens)
    q = torch.cat([m.q for m in members], dim=1).contiguous()
    k_resp = torch.cat([m.k_resp for m in members], dim=1).contiguous()
    v_resp = torch.cat([m.v_resp for m in members], dim=1).contiguous()
    sh = cache.shape(q, scale)
    hq, r, d = q.shape
    dev = q.device
    nparts = cache.num_splits + 1
    part_o = torch.empty(nparts, hq, r, d, dtype=torch.float32, device=dev)
    part_m = torch.empty(nparts, hq, r, dtype=torch.float32, device=dev)
    part_l = torch.empty(nparts, hq, r, dtype=torch.float32, device=dev)
    wsb = B.ls_replay_attn_fwd_workspace(sh, cache.pt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
    offs_dev = _upload(offs, dev) if len(members) > 1 else None
    B.ls_replay_attn_fwd_members(sh, cache.table(), offs, offs_dev, q, cache.k_pool, cache.v_pool,
                                 k_resp, v_resp, part_o, part_m, part_l, ws, stream)
    o = torch.empty(hq, r, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(hq, r, dtype=torch.float32, device=dev)
    B.ls_lse_merge(nparts, hq * r, d, part_o, part_m, part_l, o, lse, stream)
    del ws, part_o, part_m, part_l
    return [(o[:, offs[k]:offs[k + 1]], lse[:, offs[k]:offs[k + 1]]) for k in range(len(members))]


@_on_stream
def replay_backward(cache: PromptCache, q, k_resp, v_resp, o, lse, d_o, scale=None, stream=None,
                    q_offset: int = 0, dk=None, dv=None):
    """Response-only backward: returns ``(dq, dk_resp, dv_resp)`` in fp32.
    The prompt pools get no gradient.  ``dk``/``dv`` (fp32 ``[Hkv, kv_rows, d]``,
    ``kv_rows`` = the rows of ``k_resp``), when given, receive the
    contribution of these rows added to what they hold; otherwise fresh
    tensors of ``k_resp``'s row count are returned, rows past
    ``q_offset + R`` left zero."""
    hq, r, d = q.shape
    kv_rows = int(k_resp.shape[1])
    accumulate = dk is not None
    if accumulate != (dv is not None):
        raise ValueError("give both dk and dv, or neither")
    sh = cache.shape(q, scale, q_offset, kv_rows, B.LS_ACCUMULATE_KV if accumulate else 0)
    dev = q.device
    dq = torch.empty(hq, r, d, dtype=torch.float32, device=dev)
    if not accumulate:
        dk = torch.empty(cache.hkv, kv_rows, d, dtype=torch.float32, device=dev)
        dv = torch.empty(cache.hkv, kv_rows, d, dtype=torch.float32, device=dev)
        if kv_rows > q_offset + r:
            dk[:, q_offset + r:].zero_()
            dv[:, q_offset + r:].zero_()
    wsb = B.ls_replay_attn_bwd_workspace(sh, cache.pt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    B.ls_replay_attn_bwd(sh, cache.table(), q, cache.k_pool, cache.v_pool, k_resp, v_resp, o, lse, d_o,
                         dq, dk, dv, ws, stream)
    del ws
    return dq, dk, dv


@dataclass
class Member:
    """One response branch of a group: its queries, its own K/V and the
    upstream gradient of its attention output."""
    q: torch.Tensor
    k_resp: torch.Tensor
    v_resp: torch.Tensor
    d_o: torch.Tensor


@_on_stream
def replay_member(cache: PromptCache, m: Member, scale=None, stream=None):
    """Forward, merge and backward of one member.  Returns
    ``(ForwardResult, dq, dk_resp, dv_resp)``."""
    fwd = replay_forward(cache, m.q, m.k_resp, m.v_resp, scale, stream)
    dq, dk, dv = replay_backward(cache, m.q, m.k_resp, m.v_resp, fwd.o, fwd.lse, m.d_o, scale, stream)
    return fwd, dq, dk, dv


@_on_stream
def replay_group(cache: PromptCache, members: Iterable[Member], consume=None, scale=None,
                 stream=None) -> List:
    """Serial replay of a group against one shared prompt.  Each member's
    partials, outputs and gradients are handed to ``consume(index, fwd, dq,
    dk, dv)`` (if given) and then released before the next member starts, so
    at most one member's buffers are alive at a time.  Returns whatever
    ``consume`` returned, per member."""
    out = []
    for i, m in enumerate(members):
        fwd, dq, dk, dv = replay_member(cache, m, scale, stream)
        out.append(consume(i, fwd, dq, dk, dv) if consume is not None else None)
        del fwd, dq, dk, dv
    return out


@dataclass
class CaptureResult:
    cache: PromptCache   # the captured prompt: every page written, one page table
    outputs: List        # per chunk: (o bf16 [Hq, Tc, d], lse fp32 [Hq, Tc]) or consume's value


@_on_stream
def capture_prefill(chunks: Iterable, k_pool: torch.Tensor, v_pool: torch.Tensor, slots,
                    num_splits: int = 1, policy: int = B.LS_SPLIT_CONTIGUOUS,
                    block_pages: int = 1, scale=None, consume=None, stream=None) -> CaptureResult:
    """Capture of one full-attention layer of the shared prompt: a no-grad
    prefill, chunk by chunk, that keeps only the layer's K/V, as compact pages
    (DeepRead summary page, "Method"; LongStraw review page, section 2, items 1
    and 2; 4096-token chunks, same page, section 3).

    ``chunks`` yields ``(q [Hq, Tc, d], k [Hkv, Tc, d], v [Hkv, Tc, d])``, bf16
    and contiguous, for consecutive spans of the prompt; every chunk but the
    last is a whole number of 256-token pages.  ``slots`` (int32, one per page
    of the whole prompt) names the pool slot of each logical page.  Chunk
    ``[c0, c1)`` attends to the pages already captured (positions ``< c0``,
    dealt to ``num_splits`` splits like any prompt) and causally to itself, as
    the response block of one forward; its K/V pages are then appended.  The
    chunk's attention output goes to ``consume(index, o, lse)`` when given
    (and is released after it), else it is kept.  Returns the final
    :class:`PromptCache` over the pools and the per-chunk results."""
    slots_np = np.ascontiguousarray(
        np.asarray(slots.cpu() if isinstance(slots, torch.Tensor) else slots, dtype=np.int32))
    num_phys = int(k_pool.shape[0])
    if slots_np.ndim != 1 or np.unique(slots_np).size != slots_np.size:
        raise ValueError("slots must be a 1-D list of distinct pool slots")
    if slots_np.size and (slots_np.min() < 0 or slots_np.max() >= num_phys):
        raise ValueError("slots must lie in [0, num_phys_pages)")
    dev = k_pool.device
    slots_dev = _upload(slots_np.copy(), dev)
    outputs: List = []
    c0 = 0
    for i, (q, k, v) in enumerate(chunks):
        if c0 % B.PAGE_SIZE:
            raise ValueError("only the last chunk may end inside a page")
        tc = int(k.shape[1])
        p0, p1 = c0 // B.PAGE_SIZE, (c0 + tc + B.PAGE_SIZE - 1) // B.PAGE_SIZE
        if p1 > slots_np.size:
            raise ValueError(f"slots name {slots_np.size} pages; chunk {i} needs {p1}")
        cache = PromptCache(k_pool, v_pool, c0, slots_np[:p0], num_splits, policy, block_pages)
        fwd = replay_forward(cache, q, k, v, scale, stream)
        B.ls_kv_page_append(k, v, slots_np[p0:p1], slots_dev[p0:p1], k_pool, v_pool, stream)
        if consume is not None:
            outputs.append(consume(i, fwd.o, fwd.lse))
        else:
            outputs.append((fwd.o, fwd.lse))
        del fwd, cache
        c0 += tc
    npages = (c0 + B.PAGE_SIZE - 1) // B.PAGE_SIZE
    cache = PromptCache(k_pool, v_pool, c0, slots_np[:npages], num_splits, policy, block_pages)
    return CaptureResult(cache, outputs)


def block_bounds(resp_len: int, blocks: int) -> List[tuple]:
    """``blocks`` consecutive token blocks covering ``[0, resp_len)``, sizes
    differing by at most one (longer first)."""
    if blocks < 1 or blocks > resp_len:
        raise ValueError("need 1 <= blocks <= resp_len")
    base, extra = divmod(resp_len, blocks)
    out, s = [], 0
    for b in range(blocks):
        e = s + base + (1 if b < extra else 0)
        out.append((s, e))
        s = e
    return out


@_on_stream
def replay_token_blocks(cache: PromptCache, block_inputs: Iterable, k_resp, v_resp, scale=None,
                        consume=None, stream=None):
    """Reverse token-block replay of one response (the pages replay a response
    in four blocks, in reverse: LongStraw review page, section 7 mind map;
    read here as blocks of response tokens).  ``block_inputs`` lists, in
    response order, ``(q_b [Hq, Rb, d], d_o_b [Hq, Rb, d])`` for consecutive
    token blocks; ``k_resp``/``v_resp`` ``[Hkv, R, d]`` hold the whole
    response.  Blocks are replayed last first: forward and merge of the
    block's rows over the prompt and the response tokens up to each row, then
    the backward, whose dK_r/dV_r contributions are added into one fp32
    ``[Hkv, R, d]`` pair.  Each block's ``(index, fwd, dq)`` goes to
    ``consume`` (if given) and is released before the next block.  Returns
    ``(dk, dv, outputs)`` with ``outputs`` in response order."""
    blocks = list(block_inputs)
    hkv, R, d = (int(x) for x in k_resp.shape)
    offs = [0]
    for q_b, _ in blocks:
        offs.append(offs[-1] + int(q_b.shape[1]))
    if offs[-1] != R:
        raise ValueError(f"blocks cover {offs[-1]} rows, the response has {R}")
    dev = k_resp.device
    dk = torch.zeros(hkv, R, d, dtype=torch.float32, device=dev)
    dv = torch.zeros(hkv, R, d, dtype=torch.float32, device=dev)
    outputs: List = [None] * len(blocks)
    for b in reversed(range(len(blocks))):
        q_b, d_o_b = blocks[b]
        fwd = replay_forward(cache, q_b, k_resp, v_resp, scale, stream, q_offset=offs[b])
        dq, _, _ = replay_backward(cache, q_b, k_resp, v_resp, fwd.o, fwd.lse, d_o_b, scale, stream,
                                   q_offset=offs[b], dk=dk, dv=dv)
        outputs[b] = consume(b, fwd, dq) if consume is not None else (fwd, dq)
        del fwd, dq
    return dk, dv, outputs
