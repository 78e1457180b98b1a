"""Seeded synthetic inputs for response-replay attention.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds no attention arithmetic: it only draws random numbers, rounds them to
bf16, lays them out in the paged pool, and gathers the pool back into logical
order (pure indexing).

Workload shapes follow the pages' Qwen3.6-27B full-attention layer (24 query
heads, 4 KV heads, head_dim 256; "LongStraw" review page, section 3 "models and
compute") and the prompt lengths the pages report (2,097,152 and 4,456,448
positions; same page, section 3 results table). The pages publish no dataset:
their workloads are synthetic responses with deterministic rewards (DeepRead
summary page, "Strengths & Weaknesses"), so these generators are the inputs,
not stand-ins for a suite.

Recipe
------
* every tensor is drawn as float32 N(0, 1) and rounded to bf16 with
  round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``);
* the prompt K/V live in a pool ``[num_phys_pages, Hkv, page_size, d]``; logical
  page ``p`` sits in physical slot ``l2p[p]`` where ``l2p`` is a seeded random
  injection into ``range(num_phys_pages)`` (so the page table is really used);
* slots that no logical page maps to, and positions past ``prompt_len`` in the
  last logical page, hold random junk (not zero) so that a kernel reading them
  by mistake produces a visible error;
* seeds: one ``torch.Generator`` per tensor, seeded ``seed * 16 + tensor_id``.
  Generation happens on ``device``; CPU and GPU generators give different bits
  for the same seed, so a comparison always feeds both sides the same tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

PAGE_SIZE = 256

# tensor ids for per-tensor generator streams
_T_Q, _T_KR, _T_VR, _T_DO, _T_KP, _T_VP, _T_PERM = range(7)

SPLIT_CONTIGUOUS = 0
SPLIT_BLOCK_CYCLIC = 1
SPLIT_EXPLICIT = 2


@dataclasses.dataclass(frozen=True)
class ReplayShape:
    """One replay-attention problem: a response of ``resp_len`` rows attending
    to a ``prompt_len``-position paged prompt plus itself (causal)."""

    name: str
    hq: int
    hkv: int
    head_dim: int
    prompt_len: int
    resp_len: int
    num_splits: int
    policy: int = SPLIT_CONTIGUOUS
    block_pages: int = 1
    page_size: int = PAGE_SIZE
    extra_phys_pages: int = 0

    @property
    def num_pages(self) -> int:
        return (self.prompt_len + self.page_size - 1) // self.page_size

    @property
    def num_phys_pages(self) -> int:
        return self.num_pages + self.extra_phys_pages

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to float32 (the value both sides use)."""
        return float(torch.tensor(1.0 / math.sqrt(self.head_dim), dtype=torch.float32))

    def with_(self, **kw) -> "ReplayShape":
        return dataclasses.replace(self, **kw)


# The five workloads (tiny; one CP8 share of 2M; the full 2M prefix; the G=8
# group over 2M; the 4.46M stress prefix).
TINY = ReplayShape("tiny_6x1_d128_p2048_r128", 6, 1, 128, 2048, 128, 8)
SHARD_256K = ReplayShape("shard_24x4_d256_p262144_r1024", 24, 4, 256, 262_144, 1024, 1)
FULL_2M = ReplayShape("prefix_24x4_d256_p2097152_r1024_s8", 24, 4, 256, 2_097_152, 1024, 8)
GROUP_2M_RESP_LENS = (512, 768, 1024, 1536, 2048, 2560, 3072, 4096)
GROUP_2M = FULL_2M.with_(name="group8_24x4_d256_p2097152")
STRESS_4M = ReplayShape("stress_24x4_d256_p4456448_r2048_s16", 24, 4, 256, 4_456_448, 2048, 16)

WORKLOADS = {s.name: s for s in (TINY, SHARD_256K, FULL_2M, GROUP_2M, STRESS_4M)}


@dataclasses.dataclass(frozen=True)
class CaptureShape:
    """Chunked capture of one full-attention layer: ``total_len`` prompt
    positions prefilled ``chunk`` at a time (the pages' chunks are 4096
    tokens), each chunk attending to the pages before it, dealt to
    ``num_splits`` splits, and causally to itself."""

    name: str
    hq: int
    hkv: int
    head_dim: int
    total_len: int
    chunk: int
    num_splits: int
    policy: int = SPLIT_CONTIGUOUS
    block_pages: int = 1
    extra_phys_pages: int = 3

    @property
    def num_pages(self) -> int:
        return (self.total_len + PAGE_SIZE - 1) // PAGE_SIZE

    @property
    def num_phys_pages(self) -> int:
        return self.num_pages + self.extra_phys_pages

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def spans(self) -> List[tuple]:
        return [(s, min(self.total_len, s + self.chunk)) for s in range(0, self.total_len, self.chunk)]


CAPTURE_256K = CaptureShape("capture_24x4_d256_p262144_c4096_s8", 24, 4, 256, 262_144, 4096, 8,
                            SPLIT_BLOCK_CYCLIC, 1)
CAPTURE_2M = CaptureShape("capture_24x4_d256_p2097152_c4096_s8", 24, 4, 256, 2_097_152, 4096, 8,
                          SPLIT_BLOCK_CYCLIC, 1)
CAPTURE_WORKLOADS = {c.name: c for c in (CAPTURE_256K, CAPTURE_2M)}


def make_capture_inputs(shape: CaptureShape, seed: int, device="cpu") -> Dict[str, object]:
    """Draw one capture problem: the whole prompt's projections ``q [Hq,T,d]``,
    ``k/v [Hkv,T,d]`` (bf16) cut into contiguous per-chunk tensors
    (``chunks``: list of ``(q, k, v)``), junk-filled pools
    ``[num_phys, Hkv, 256, d]`` and ``slots`` (int32 CPU, a seeded injection of
    the prompt's logical pages into the pool slots)."""
    H, Hk, d, T = shape.hq, shape.hkv, shape.head_dim, shape.total_len
    dev = torch.device(device)
    full = {"q": _randn_bf16((H, T, d), _gen(seed, _T_Q, dev), dev),
            "k": _randn_bf16((Hk, T, d), _gen(seed, _T_KR, dev), dev),
            "v": _randn_bf16((Hk, T, d), _gen(seed, _T_VR, dev), dev)}
    chunks = []
    for s, e in shape.spans():
        chunks.append(tuple(full[n][:, s:e].contiguous() for n in ("q", "k", "v")))
    del full
    pool_shape = (shape.num_phys_pages, Hk, PAGE_SIZE, d)
    g = _gen(seed, _T_PERM, "cpu")
    slots = torch.randperm(shape.num_phys_pages, generator=g)[: shape.num_pages].to(torch.int32)
    return {"chunks": chunks,
            "k_pool": _randn_bf16(pool_shape, _gen(seed, _T_KP, dev), dev),
            "v_pool": _randn_bf16(pool_shape, _gen(seed, _T_VP, dev), dev),
            "slots": slots.contiguous()}


def whole_prompt(chunks, index: int) -> torch.Tensor:
    """Concatenate one projection (0 = q, 1 = k, 2 = v) of every chunk back into
    ``[H, T, d]`` along the token axis.  Pure indexing."""
    return torch.cat([c[index] for c in chunks], dim=1)


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 16 + tid)
    return g


def _randn_bf16(shape, gen, device, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """N(0,1) float32 rounded to bf16, drawn in chunks so that huge pools never
    hold a float32 copy in full."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def page_permutation(shape: ReplayShape, seed: int) -> torch.Tensor:
    """Seeded injection logical page -> physical slot (int32, CPU)."""
    g = _gen(seed, _T_PERM, "cpu")
    perm = torch.randperm(shape.num_phys_pages, generator=g)
    return perm[: shape.num_pages].to(torch.int32).contiguous()


def make_inputs(shape: ReplayShape, seed: int, device="cpu", *,
                q_zero: bool = False, v_const: Optional[float] = None,
                q_mult: float = 1.0, identity_pages: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one problem.  Returns bf16 tensors
    ``q [Hq,R,d]``, ``k_resp/v_resp [Hkv,R,d]``, ``d_o [Hq,R,d]``,
    ``k_pool/v_pool [num_phys,Hkv,page,d]`` and int32 ``l2p [num_pages]`` (CPU).

    ``q_zero``: Q = 0 (closed-form case: softmax is uniform over visible keys).
    ``v_const``: every V entry (prompt and response) equals this bf16 value.
    ``q_mult``: Q scaled by this power of two before rounding ("peaked" scores).
    """
    H, Hk, d, R = shape.hq, shape.hkv, shape.head_dim, shape.resp_len
    dev = torch.device(device)
    out: Dict[str, torch.Tensor] = {}
    if q_zero:
        out["q"] = torch.zeros(H, R, d, dtype=torch.bfloat16, device=dev)
    else:
        q = _randn_bf16((H, R, d), _gen(seed, _T_Q, dev), dev)
        if q_mult != 1.0:
            q = (q.float() * q_mult).to(torch.bfloat16)
        out["q"] = q
    out["k_resp"] = _randn_bf16((Hk, R, d), _gen(seed, _T_KR, dev), dev)
    out["v_resp"] = _randn_bf16((Hk, R, d), _gen(seed, _T_VR, dev), dev)
    out["d_o"] = _randn_bf16((H, R, d), _gen(seed, _T_DO, dev), dev)
    pool_shape = (shape.num_phys_pages, Hk, shape.page_size, d)
    out["k_pool"] = _randn_bf16(pool_shape, _gen(seed, _T_KP, dev), dev)
    out["v_pool"] = _randn_bf16(pool_shape, _gen(seed, _T_VP, dev), dev)
    if v_const is not None:
        c = torch.tensor(v_const, dtype=torch.bfloat16)
        out["v_pool"].fill_(c)
        out["v_resp"].fill_(c)
    if identity_pages:
        out["l2p"] = torch.arange(shape.num_pages, dtype=torch.int32)
    else:
        out["l2p"] = page_permutation(shape, seed)
    return out


def plant_late_dominant_keys(inp: Dict[str, torch.Tensor], shape: ReplayShape, seed: int,
                             kv: int = 0, n: int = 64) -> None:
    """Turn a problem drawn by :func:`make_inputs` into one whose last ``n``
    prompt keys of KV head ``kv`` dominate every query row of that head, late
    in the last split (in place).

    Every query row becomes ``u + 0.1 q`` for one seeded direction ``u``
    (``|u|^2 ~ d``), and keys ``P - n .. P - 1`` of KV head ``kv`` become
    ``3u + 2 z`` (``z`` seeded N(0, 1)): with scale ``1/sqrt(d)`` they score
    about ``3 sqrt(d)`` natural units, spread by about 2, while every other
    key scores about N(0, 1).  The prompt must end on a page boundary and
    ``n <= 256``.  Pure data generation: no attention arithmetic."""
    d, P = shape.head_dim, shape.prompt_len
    assert P % shape.page_size == 0 and 0 < n <= shape.page_size
    g = _gen(seed, 14, "cpu")
    u = torch.randn(d, generator=g).to(torch.bfloat16).float()
    z = torch.randn(n, d, generator=g)
    dev = inp["q"].device
    inp["q"] = (u[None, None, :].to(dev) + 0.1 * inp["q"].float()).to(torch.bfloat16)
    last = int(inp["l2p"][shape.num_pages - 1])          # pool slot of the last logical page
    inp["k_pool"][last, kv, shape.page_size - n:] = (3.0 * u[None, :] + 2.0 * z).to(torch.bfloat16).to(dev)


def make_response(shape: ReplayShape, seed: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Only the response side of a problem (``q``, ``k_resp``, ``v_resp``,
    ``d_o``), drawn exactly as :func:`make_inputs` draws them: used for the
    members of a group that share one prompt pool."""
    H, Hk, d, R = shape.hq, shape.hkv, shape.head_dim, shape.resp_len
    dev = torch.device(device)
    return {
        "q": _randn_bf16((H, R, d), _gen(seed, _T_Q, dev), dev),
        "k_resp": _randn_bf16((Hk, R, d), _gen(seed, _T_KR, dev), dev),
        "v_resp": _randn_bf16((Hk, R, d), _gen(seed, _T_VR, dev), dev),
        "d_o": _randn_bf16((H, R, d), _gen(seed, _T_DO, dev), dev),
    }


def logical_prompt(pool: torch.Tensor, l2p: torch.Tensor, prompt_len: int,
                   kv_heads: Optional[List[int]] = None) -> torch.Tensor:
    """Gather the pool back into logical order: ``[Hkv, prompt_len, d]`` (same
    dtype and device as ``pool``).  Pure indexing."""
    num_pages, hk, page, d = l2p.numel(), pool.shape[1], pool.shape[2], pool.shape[3]
    heads = list(range(hk)) if kv_heads is None else list(kv_heads)
    idx = l2p.to(device=pool.device, dtype=torch.long)
    out = torch.empty(len(heads), num_pages * page, d, dtype=pool.dtype, device=pool.device)
    for n, kv in enumerate(heads):
        out[n] = pool[idx, kv].reshape(num_pages * page, d)
    return out[:, :prompt_len]


def scatter_prompt(k_logical: torch.Tensor, l2p: torch.Tensor, num_phys_pages: int,
                   page_size: int = PAGE_SIZE, fill: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Inverse of :func:`logical_prompt`: place a logical ``[Hkv, P, d]`` sequence
    into a pool.  Unused slots and the tail of the last page are taken from
    ``fill`` (a pool-shaped tensor) or left as zeros."""
    hk, P, d = k_logical.shape
    num_pages = l2p.numel()
    pool = (fill.clone() if fill is not None else
            torch.zeros(num_phys_pages, hk, page_size, d, dtype=k_logical.dtype, device=k_logical.device))
    for p in range(num_pages):
        s, e = p * page_size, min(P, (p + 1) * page_size)
        pool[int(l2p[p]), :, : e - s] = k_logical[:, s:e]
    return pool


def sample_rows(shape: ReplayShape, per_head: int, seed: int) -> torch.Tensor:
    """Seeded sample of response rows per query head, always containing rows
    0 and R-1.  Returns an int64 tensor ``[Hq, n]`` of row indices (sorted)."""
    R = shape.resp_len
    g = _gen(seed, 15, "cpu")
    rows = []
    for _ in range(shape.hq):
        if per_head >= R:
            r = torch.arange(R)
        else:
            r = torch.randperm(R - 2, generator=g)[: max(0, per_head - 2)] + 1
            r = torch.cat([torch.tensor([0, R - 1]), r])
        rows.append(torch.sort(r).values)
    return torch.stack(rows)
