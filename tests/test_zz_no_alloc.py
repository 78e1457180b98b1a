"""The allocation-free forward (ls_replay_attn_fwd_noalloc, through the C ABI)
against the forward with a caller workspace (ls_replay_attn_fwd): two calls in
a row, the second on a smaller problem, each compared bit for bit on the
partials and, after the merge, with the float64 oracle."""
import pytest
import torch

import oracle
from replay_inputs import ReplayShape, logical_prompt, make_inputs
from response_replay_attention_amd import PromptCache
from response_replay_attention_amd import binding as B
from tests.parity import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

CASES = [
    # one split of 64 pages: the plan sub-splits it, so the scratch holds the
    # chunk partials as well as the resolved page list
    ReplayShape("noalloc_chunked_d128", 6, 1, 128, 64 * 256, 128, 1),
    # smaller: ragged last page, three block-cyclic splits, spare pool slots
    ReplayShape("noalloc_ragged_d256", 24, 4, 256, 5 * 256 + 77, 45, 3, 1, 1, extra_phys_pages=2),
]


def _partials(shape, dev):
    n = shape.num_splits + 1
    return [torch.full(s, float("nan"), dtype=torch.float32, device=dev)
            for s in ((n, shape.hq, shape.resp_len, shape.head_dim), (n, shape.hq, shape.resp_len),
                      (n, shape.hq, shape.resp_len))]


def test_noalloc_forward_matches_forward_on_two_calls():
    dev = torch.device("cuda")
    for i, shape in enumerate(CASES):
        print(f"case {shape.name}", flush=True)
        inp = make_inputs(shape, seed=40 + i, device=dev)
        cache = PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"],
                            shape.num_splits, shape.policy, shape.block_pages)
        sh = cache.shape(inp["q"], shape.scale)
        pt = cache.table()
        wsb = B.ls_replay_attn_fwd_workspace(sh, pt)
        if i == 0:
            assert wsb > (shape.num_pages * 4 + 255) // 256 * 256, "the plan uses chunk partials"
        assert wsb <= B.LS_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        ref = _partials(shape, dev)
        B.ls_replay_attn_fwd(sh, pt, inp["q"], cache.k_pool, cache.v_pool, inp["k_resp"],
                             inp["v_resp"], *ref, ws)
        got = _partials(shape, dev)
        B.ls_replay_attn_fwd_noalloc(sh, pt, inp["q"], cache.k_pool, cache.v_pool, inp["k_resp"],
                                     inp["v_resp"], *got)
        torch.cuda.synchronize()
        # both plans fit the scratch, so they are the same plan: same bits
        for name, a, b in zip(("part_o", "part_m", "part_l"), got, ref):
            assert torch.equal(a, b), name
            assert not torch.isnan(a).any(), f"{name}: not every element written"
        nparts, rows = shape.num_splits + 1, shape.hq * shape.resp_len
        o = torch.empty(shape.hq, shape.resp_len, shape.head_dim, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(shape.hq, shape.resp_len, dtype=torch.float32, device=dev)
        B.ls_lse_merge(nparts, rows, shape.head_dim, *got, o, lse)
        torch.cuda.synchronize()
        kp = logical_prompt(inp["k_pool"], inp["l2p"], shape.prompt_len).cpu()
        vp = logical_prompt(inp["v_pool"], inp["l2p"], shape.prompt_len).cpu()
        o_r, lse_r = oracle.replay_forward(inp["q"].cpu(), kp, vp, inp["k_resp"].cpu(),
                                           inp["v_resp"].cpu(), shape.scale)
        assert_close("O", o, o_r)
        assert_lse_close("LSE", lse, lse_r)
