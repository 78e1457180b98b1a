"""Host check of the chunked capture driver's sequencing (no GPU): the two
library calls it makes per chunk are stood in for by the float64 oracle and
plain indexing, so what is tested is the driver itself -- that chunk
[c0, c1) is given exactly the pages of positions < c0 as its prompt, itself
as the causal block, and that its pages land in the slots named for them.
The result must then equal the oracle's causal attention over the whole
sequence; a chunk shown one page too many or too few breaks it."""
import numpy as np
import pytest
import torch

import oracle
from replay_inputs import (SPLIT_BLOCK_CYCLIC, CaptureShape, logical_prompt, make_capture_inputs,
                           whole_prompt)
from response_replay_attention_amd import replay as RP


def _fake_forward(calls):
    def fwd(cache, q, k, v, scale=None, stream=None):
        calls.append((cache.prompt_len, cache.num_pages, cache.num_splits))
        l2p = torch.from_numpy(np.asarray(cache.l2p, dtype=np.int32))
        kp = logical_prompt(cache.k_pool, l2p, cache.prompt_len)
        vp = logical_prompt(cache.v_pool, l2p, cache.prompt_len)
        o, lse = oracle.replay_forward(q, kp, vp, k, v, scale if scale else q.shape[2] ** -0.5)
        return RP.ForwardResult(torch.from_numpy(o), torch.from_numpy(lse), None, None, None)
    return fwd


def _fake_append(k, v, slots, slots_dev, k_pool, v_pool, stream=None):
    assert np.array_equal(np.asarray(slots), slots_dev.numpy())
    for p, sl in enumerate(np.asarray(slots)):
        s, e = p * 256, min(k.shape[1], (p + 1) * 256)
        k_pool[int(sl), :, : e - s] = k[:, s:e]
        v_pool[int(sl), :, : e - s] = v[:, s:e]


@pytest.mark.parametrize("shape", [
    CaptureShape("host_c512_ragged", 4, 2, 128, 4 * 512 + 33, 512, 3, SPLIT_BLOCK_CYCLIC, 1),
    CaptureShape("host_c256_exact", 2, 1, 128, 1024, 256, 1),
], ids=lambda s: s.name)
def test_capture_driver_sequencing(shape, monkeypatch):
    calls = []
    monkeypatch.setattr(RP, "replay_forward", _fake_forward(calls))
    monkeypatch.setattr(RP.B, "ls_kv_page_append", _fake_append)
    inp = make_capture_inputs(shape, seed=5)
    res = RP.capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], inp["slots"],
                             shape.num_splits, shape.policy, shape.block_pages, shape.scale)
    spans = shape.spans()
    assert calls == [(s, s // 256, shape.num_splits) for s, _ in spans]
    q, k, v = (whole_prompt(inp["chunks"], i) for i in range(3))
    empty = k[:, :0]
    o_r, lse_r = oracle.replay_forward(q, empty, empty, k, v, shape.scale)
    for (s, e), (o, lse) in zip(spans, res.outputs):
        np.testing.assert_allclose(o.numpy(), o_r[:, s:e], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse.numpy(), lse_r[:, s:e], rtol=0, atol=1e-12)
    assert res.cache.prompt_len == shape.total_len
    assert torch.equal(logical_prompt(inp["k_pool"], inp["slots"], shape.total_len), k)


def test_capture_driver_rejects_bad_input(monkeypatch):
    monkeypatch.setattr(RP, "replay_forward", _fake_forward([]))
    monkeypatch.setattr(RP.B, "ls_kv_page_append", _fake_append)
    shape = CaptureShape("host_bad", 2, 1, 128, 600, 300, 1)   # chunk not page-aligned
    inp = make_capture_inputs(shape, seed=6)
    with pytest.raises(ValueError):
        RP.capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], inp["slots"])
    good = CaptureShape("host_bad2", 2, 1, 128, 512, 256, 1)
    inp = make_capture_inputs(good, seed=6)
    with pytest.raises(ValueError):                             # a slot named twice
        RP.capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], [0, 0])
    with pytest.raises(ValueError):                             # too few slots
        RP.capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], [0])
