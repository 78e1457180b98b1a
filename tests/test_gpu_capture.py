"""GPU checks of the capture-side page writer: the chunked no-grad prefill of
one full-attention layer that appends each chunk's K/V as pages of the pool
and attends the chunk to the pages before it plus itself (causal).

* the pool after capture, read back through the slots, equals the prompt's
  K/V bit for bit, and nothing outside the written rows changes (unused slots
  and the tail of the last page keep their junk);
* every chunk's O and LSE match the float64 oracle's causal attention over
  the whole sequence (the oracle's forward with no prompt and the sequence as
  the response): all rows on small shapes, sampled rows that include every
  chunk's first and last row on a 24x4-head d=256 shape with 4096-token
  chunks;
* the 262,144-position capture with Q = 0: softmax is uniform over the visible
  keys, so row t has LSE = ln(t + 1) and O = mean of v_0..v_t, for every row
  of every chunk (a chunk that missed a page, or saw one too many, breaks it).

Outputs of the first rows average only a few keys and are O(1), so O is held
to the relative bounds of tests/parity.py; LSE to its usual bound.
"""
import numpy as np
import pytest
import torch

import oracle
from replay_inputs import (CAPTURE_256K, SPLIT_BLOCK_CYCLIC, SPLIT_CONTIGUOUS, CaptureShape,
                           logical_prompt, make_capture_inputs, whole_prompt)
from response_replay_attention_amd import capture_prefill, ls_kv_page_append
from tests.parity import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

SMALL = [
    CaptureShape("cap_d128_4x2_c1024_ragged_cyclic", 4, 2, 128, 3 * 1024 + 77, 1024, 2,
                 SPLIT_BLOCK_CYCLIC, 1),
    CaptureShape("cap_d256_2x1_c256_pages", 2, 1, 256, 700, 256, 3),
    CaptureShape("cap_d128_6x1_one_chunk", 6, 1, 128, 300, 4096, 1),
]
SAMPLED = CaptureShape("cap_d256_24x4_c4096_s3", 24, 4, 256, 2 * 4096 + 300, 4096, 3,
                       SPLIT_CONTIGUOUS)


def _capture(shape, inp, **kw):
    return capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], inp["slots"],
                           shape.num_splits, shape.policy, shape.block_pages, shape.scale, **kw)


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_capture_pages_bit_exact(shape):
    print(f"case {shape.name} pages", flush=True)
    inp = make_capture_inputs(shape, seed=31, device="cuda")
    k0, v0 = inp["k_pool"].clone(), inp["v_pool"].clone()
    res = _capture(shape, inp)
    torch.cuda.synchronize()
    T, slots = shape.total_len, inp["slots"]
    assert res.cache.prompt_len == T and res.cache.num_pages == shape.num_pages
    for pool, before, idx in ((inp["k_pool"], k0, 1), (inp["v_pool"], v0, 2)):
        want = whole_prompt(inp["chunks"], idx)
        assert torch.equal(logical_prompt(pool, slots, T), want)
        # everything the capture must not touch
        unused = sorted(set(range(shape.num_phys_pages)) - set(slots.tolist()))
        assert torch.equal(pool[unused], before[unused])
        tail = T % 256
        if tail:
            last = int(slots[-1])
            assert torch.equal(pool[last, :, tail:], before[last, :, tail:])


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_capture_matches_oracle(shape):
    print(f"case {shape.name} attention", flush=True)
    inp = make_capture_inputs(shape, seed=32, device="cuda")
    res = _capture(shape, inp)
    torch.cuda.synchronize()
    q, k, v = (whole_prompt(inp["chunks"], i).cpu() for i in range(3))
    empty = k[:, :0]
    o_r, lse_r = oracle.replay_forward(q, empty, empty, k, v, shape.scale)
    assert len(res.outputs) == len(shape.spans())
    for (s, e), (o, lse) in zip(shape.spans(), res.outputs):
        assert o.shape == (shape.hq, e - s, shape.head_dim)
        assert_close(f"O [{s},{e})", o, o_r[:, s:e], contract=False)
        assert_lse_close(f"LSE [{s},{e})", lse, lse_r[:, s:e])


def test_capture_matches_oracle_sampled_rows():
    shape = SAMPLED
    print(f"case {shape.name} sampled rows", flush=True)
    inp = make_capture_inputs(shape, seed=33, device="cuda")
    res = _capture(shape, inp)
    torch.cuda.synchronize()
    q, k, v = (whole_prompt(inp["chunks"], i).cpu() for i in range(3))
    T = shape.total_len
    g = np.random.default_rng(7)
    edges = sorted({t for s, e in shape.spans() for t in (s, s + 1, e - 2, e - 1)})
    rest = np.setdiff1d(np.arange(T), edges)
    rows = np.stack([np.sort(np.concatenate([edges, g.choice(rest, 24, replace=False)]))
                     for _ in range(shape.hq)])
    empty = k[:, :0]
    o_r, lse_r = oracle.replay_forward(q, empty, empty, k, v, shape.scale, rows=rows)
    o_all = torch.cat([o for o, _ in res.outputs], dim=1)
    lse_all = torch.cat([lse for _, lse in res.outputs], dim=1)
    idx = torch.from_numpy(rows).to(o_all.device)
    o_s = torch.gather(o_all, 1, idx[:, :, None].expand(-1, -1, shape.head_dim))
    lse_s = torch.gather(lse_all, 1, idx)
    assert_close("O sampled", o_s, o_r, contract=False)
    assert_lse_close("LSE sampled", lse_s, lse_r)


def test_capture_zero_query_full_size():
    shape = CAPTURE_256K
    print(f"case {shape.name} Q=0", flush=True)
    inp = make_capture_inputs(shape, seed=34, device="cuda")
    for q, _, _ in inp["chunks"]:
        q.zero_()
    g = shape.hq // shape.hkv
    csum = torch.cumsum(whole_prompt(inp["chunks"], 2).double(), dim=1)  # [Hkv, T, d]
    bad = []

    def check(i, o, lse):
        s, e = shape.spans()[i]
        n = torch.arange(s, e, device=o.device, dtype=torch.float64) + 1
        want_o = csum[:, s:e] / n[None, :, None]
        ln = torch.log(n)[None]
        lse_err = float(((lse.double() - ln).abs() / ln.clamp(min=1.0)).max())
        o_err = float((o.double() - want_o.repeat_interleave(g, 0)).abs().max())
        if lse_err > 1e-4 or o_err > 2e-2:
            bad.append((i, lse_err, o_err))
        return o_err

    res = _capture(shape, inp, consume=check)
    torch.cuda.synchronize()
    assert not bad, f"chunks off the closed form: {bad[:5]}"
    assert len(res.outputs) == len(shape.spans())


def test_page_append_direct_two_chunks():
    """The C entry point alone: two appends into the same pool, the second
    ragged, land where the slots say."""
    print("case page_append direct", flush=True)
    shape = CaptureShape("append_d256_4kv", 4, 4, 256, 512 + 130, 512, 1)
    inp = make_capture_inputs(shape, seed=35, device="cuda")
    slots = inp["slots"]
    dev_slots = slots.cuda()
    c0, c1 = inp["chunks"]
    ls_kv_page_append(c0[1], c0[2], slots[:2], dev_slots[:2], inp["k_pool"], inp["v_pool"])
    ls_kv_page_append(c1[1], c1[2], slots[2:], dev_slots[2:], inp["k_pool"], inp["v_pool"])
    torch.cuda.synchronize()
    T = shape.total_len
    assert torch.equal(logical_prompt(inp["k_pool"], slots, T), whole_prompt(inp["chunks"], 1))
    assert torch.equal(logical_prompt(inp["v_pool"], slots, T), whole_prompt(inp["chunks"], 2))
