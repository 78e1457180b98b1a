"""GPU parity of group scoring: the forward of every member of a group in one
pass over the prompt (members stacked along the response axis), through the
C ABI, against the float64 oracle's forward of each member on its own.

* small shapes, every row: ragged prompts, block-cyclic splits, a one-row
  member, no prompt, 128-row and 256-row tiles that straddle members and
  query heads;
* the G = 8 group over the 2,097,152-position prefix with Q = 0: every row of
  every member must see exactly the prompt and its own response keys up to
  itself, so LSE_i = ln(P + i + 1) with i the row's index inside its member
  (a member that saw a neighbour's keys would break it).
"""
import numpy as np
import pytest
import torch

import oracle
from replay_inputs import (GROUP_2M, GROUP_2M_RESP_LENS, SPLIT_BLOCK_CYCLIC, ReplayShape,
                           logical_prompt, make_inputs, make_response)
from response_replay_attention_amd import Member, PromptCache, score_group
from tests.parity import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

CASES = [
    (ReplayShape("members_d128_ragged_cyclic", 6, 1, 128, 9 * 256 + 1, 1, 4, SPLIT_BLOCK_CYCLIC, 2,
                 extra_phys_pages=2), (1, 45, 200, 31)),
    (ReplayShape("members_d256_gqa24x4_s8", 24, 4, 256, 16 * 256, 1, 8), (64, 96, 160)),
    (ReplayShape("members_no_prompt", 12, 2, 256, 0, 1, 2), (33, 7, 90)),
]
RELATIVE_ONLY = {"members_no_prompt"}  # outputs far from the workloads' scale


def _members(shape, lens, seed):
    return [make_response(shape.with_(resp_len=r), seed + i, device="cuda")
            for i, r in enumerate(lens)]


def _cache(shape, inp):
    return PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"],
                       shape.num_splits, shape.policy, shape.block_pages)


@pytest.mark.parametrize("shape,lens", CASES, ids=[c[0].name for c in CASES])
def test_group_scoring_matches_oracle(shape, lens):
    print(f"case {shape.name} members {lens}", flush=True)
    inp = make_inputs(shape, seed=21, device="cuda")  # the prompt pool and its page map
    resp = _members(shape, lens, seed=300)
    out = score_group(_cache(shape, inp),
                      [Member(r["q"], r["k_resp"], r["v_resp"], r["d_o"]) for r in resp], shape.scale)
    torch.cuda.synchronize()
    kp = logical_prompt(inp["k_pool"], inp["l2p"], shape.prompt_len).cpu()
    vp = logical_prompt(inp["v_pool"], inp["l2p"], shape.prompt_len).cpu()
    contract = shape.name not in RELATIVE_ONLY
    assert len(out) == len(lens)
    for k, (r, (o, lse)) in enumerate(zip(resp, out)):
        assert o.shape == (shape.hq, lens[k], shape.head_dim)
        o_r, lse_r = oracle.replay_forward(r["q"].cpu(), kp, vp, r["k_resp"].cpu(),
                                           r["v_resp"].cpu(), shape.scale)
        assert_close(f"O member {k}", o, o_r, contract)
        assert_lse_close(f"LSE member {k}", lse, lse_r)


def test_group_scoring_zero_query_full_size():
    shape = GROUP_2M
    P, g = shape.prompt_len, shape.hq // shape.hkv
    inp = make_inputs(shape.with_(resp_len=GROUP_2M_RESP_LENS[0]), seed=20260004, device="cuda")
    resp = _members(shape, GROUP_2M_RESP_LENS, seed=400)
    for r in resp:
        r["q"].zero_()
    print(f"case group8 Q=0 members {GROUP_2M_RESP_LENS}", flush=True)
    out = score_group(_cache(shape, inp),
                      [Member(r["q"], r["k_resp"], r["v_resp"], r["d_o"]) for r in resp], shape.scale)
    torch.cuda.synchronize()
    psum = [logical_prompt(inp["v_pool"], inp["l2p"], P, kv_heads=[kv])[0].double().sum(0)
            for kv in range(shape.hkv)]
    for k, (r, (o, lse)) in enumerate(zip(resp, out)):
        R = GROUP_2M_RESP_LENS[k]
        n = torch.arange(R, device="cuda", dtype=torch.float64) + P + 1
        want_lse = torch.log(n).cpu().numpy()
        for kv in range(shape.hkv):
            csum = psum[kv][None, :] + torch.cumsum(r["v_resp"][kv].double(), 0)
            want_o = (csum / n[:, None]).cpu().numpy()
            for h in range(kv * g, (kv + 1) * g):
                assert_lse_close(f"LSE member {k} h{h}", lse[h], want_lse)
                assert_close(f"O member {k} h{h}", o[h], want_o)
