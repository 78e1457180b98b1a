"""GPU parity of token-block replay: a response replayed as consecutive token
blocks, last block first, each block's rows at their offset inside the
response (q_offset), against the float64 oracle of the whole response.

* every block's O, LSE and dQ equal the oracle's rows of that block, and the
  dK_r/dV_r the blocks add into one buffer equal the whole response's;
* one block through the C ABI on its own: with kv_rows = R its dK_r/dV_r rows
  past q_offset + R_b are left as they were, the rows before hold the oracle's
  contribution of exactly that block's rows, and LS_ACCUMULATE_KV adds that
  contribution to what the buffers held;
* blocks that do not start on a 32-row tile, a block of one row, and no
  prompt;
* the 2,097,152-position prefix in four blocks with Q = 0, against the closed
  form of every row's O and LSE and of the summed dV_r (dK_r must be 0).
"""
import numpy as np
import pytest
import torch

import oracle
from replay_inputs import SPLIT_BLOCK_CYCLIC, ReplayShape, logical_prompt, make_inputs
from response_replay_attention_amd import (LS_ACCUMULATE_KV, PromptCache, block_bounds,
                                           replay_forward, replay_token_blocks)
from response_replay_attention_amd import binding as B
from tests.parity import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

CASES = [
    (ReplayShape("tb_d128_6x1_ragged_s3", 6, 1, 128, 3 * 256 + 17, 300, 3), 4),
    (ReplayShape("tb_d256_24x4_cyclic", 24, 4, 256, 8 * 256, 296, 2, SPLIT_BLOCK_CYCLIC, 1,
                 extra_phys_pages=2), 4),
    (ReplayShape("tb_no_prompt", 12, 2, 256, 0, 200, 1), 3),
    (ReplayShape("tb_d128_one_row_blocks", 6, 2, 128, 2 * 256, 5, 2), 5),
]
RELATIVE_ONLY = {"tb_no_prompt"}


def _cache(shape, inp):
    return PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"],
                       shape.num_splits, shape.policy, shape.block_pages)


def _oracle(shape, inp, rows=None):
    kp = logical_prompt(inp["k_pool"], inp["l2p"], shape.prompt_len).cpu()
    vp = logical_prompt(inp["v_pool"], inp["l2p"], shape.prompt_len).cpu()
    return oracle.replay_backward(inp["q"].cpu(), kp, vp, inp["k_resp"].cpu(), inp["v_resp"].cpu(),
                                  inp["d_o"].cpu(), shape.scale, rows=rows)


@pytest.mark.parametrize("shape,nblocks", CASES, ids=[c[0].name for c in CASES])
def test_reverse_token_blocks_match_oracle(shape, nblocks):
    print(f"case {shape.name} blocks {nblocks}", flush=True)
    inp = make_inputs(shape, seed=41, device="cuda")
    bounds = block_bounds(shape.resp_len, nblocks)
    blocks = [(inp["q"][:, s:e].contiguous(), inp["d_o"][:, s:e].contiguous()) for s, e in bounds]
    order = []

    def keep(b, fwd, dq):
        order.append(b)
        return fwd.o, fwd.lse, dq

    dk, dv, outs = replay_token_blocks(_cache(shape, inp), blocks, inp["k_resp"], inp["v_resp"],
                                       shape.scale, consume=keep)
    torch.cuda.synchronize()
    assert order == list(reversed(range(nblocks)))
    dq_r, dk_r, dv_r, o_r, lse_r = _oracle(shape, inp)
    contract = shape.name not in RELATIVE_ONLY
    for (s, e), (o, lse, dq) in zip(bounds, outs):
        assert_close(f"O [{s},{e})", o, o_r[:, s:e], contract)
        assert_lse_close(f"LSE [{s},{e})", lse, lse_r[:, s:e])
        assert_close(f"dQ [{s},{e})", dq, dq_r[:, s:e], contract)
    assert_close("dK_r summed over blocks", dk, dk_r, contract)
    assert_close("dV_r summed over blocks", dv, dv_r, contract)


def _bwd_block(shape, inp, cache, s, e, dk, dv, flags):
    """One block straight through the C ABI, kv_rows = R."""
    q = inp["q"][:, s:e].contiguous()
    d_o = inp["d_o"][:, s:e].contiguous()
    fwd = replay_forward(cache, q, inp["k_resp"], inp["v_resp"], shape.scale, q_offset=s)
    sh = cache.shape(q, shape.scale, q_offset=s, kv_rows=shape.resp_len, flags=flags)
    dq = torch.empty(shape.hq, e - s, shape.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ls_replay_attn_bwd_workspace(sh, cache.pt), dtype=torch.uint8, device="cuda")
    B.ls_replay_attn_bwd(sh, cache.pt, q, cache.k_pool, cache.v_pool, inp["k_resp"], inp["v_resp"],
                         fwd.o, fwd.lse, d_o, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dq


def test_one_block_contribution_and_untouched_rows():
    shape = ReplayShape("tb_single_d256_24x4", 24, 4, 256, 6 * 256 + 100, 333, 2)
    print(f"case {shape.name} block [150, 260)", flush=True)
    inp = make_inputs(shape, seed=42, device="cuda")
    cache = _cache(shape, inp)
    s, e = 150, 260
    rows = np.tile(np.arange(s, e), (shape.hq, 1))
    dq_r, dk_r, dv_r, _, _ = _oracle(shape, inp, rows=rows)  # contribution of rows [s, e)

    fill = 7.0
    dk = torch.full((shape.hkv, shape.resp_len, shape.head_dim), fill, device="cuda")
    dv = torch.full_like(dk, fill)
    dq = _bwd_block(shape, inp, cache, s, e, dk, dv, 0)
    assert_close("dQ block", dq, dq_r)
    assert_close("dK_r block", dk[:, :e], dk_r[:, :e])
    assert_close("dV_r block", dv[:, :e], dv_r[:, :e])
    assert bool((dk[:, e:] == fill).all()) and bool((dv[:, e:] == fill).all())

    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    base_k = torch.randn(dk.shape, generator=g, device="cuda")
    base_v = torch.randn(dk.shape, generator=g, device="cuda")
    dk2, dv2 = base_k.clone(), base_v.clone()
    _bwd_block(shape, inp, cache, s, e, dk2, dv2, LS_ACCUMULATE_KV)
    bk, bv = base_k.cpu().double().numpy(), base_v.cpu().double().numpy()
    assert_close("dK_r accumulated", dk2[:, :e], bk[:, :e] + dk_r[:, :e])
    assert_close("dV_r accumulated", dv2[:, :e], bv[:, :e] + dv_r[:, :e])
    assert torch.equal(dk2[:, e:], base_k[:, e:]) and torch.equal(dv2[:, e:], base_v[:, e:])


def test_token_blocks_zero_query_full_size():
    """The 2,097,152-position prefix, R = 1024 as four blocks replayed in
    reverse, Q = 0: every visible key has weight 1/n_i with n_i = P + i + 1
    (i = the row's index in the whole response), so for every row of every
    block LSE = ln n_i and O = (sum of visible values) / n_i; dK_r = 0 exactly
    (every term carries a factor of q), and dV_r[j] = sum over heads h of the
    group and rows i >= j of dO[h, i] / n_i, summed over the blocks."""
    from replay_inputs import FULL_2M
    shape = FULL_2M
    P, R, g = shape.prompt_len, shape.resp_len, shape.hq // shape.hkv
    print(f"case {shape.name} 4 token blocks, Q=0", flush=True)
    inp = make_inputs(shape, seed=20260044, device="cuda", q_zero=True)
    bounds = block_bounds(R, 4)
    blocks = [(inp["q"][:, s:e].contiguous(), inp["d_o"][:, s:e].contiguous()) for s, e in bounds]
    dk, dv, outs = replay_token_blocks(_cache(shape, inp), blocks, inp["k_resp"], inp["v_resp"],
                                       shape.scale, consume=lambda b, fwd, dq: (fwd.o, fwd.lse))
    torch.cuda.synchronize()
    n = torch.arange(R, device="cuda", dtype=torch.float64) + P + 1
    for kv in range(shape.hkv):
        psum = logical_prompt(inp["v_pool"], inp["l2p"], P, kv_heads=[kv])[0].double().sum(0)
        want_o = (psum[None, :] + torch.cumsum(inp["v_resp"][kv].double(), 0)) / n[:, None]
        for (s, e), (o, lse) in zip(bounds, outs):
            for h in range(kv * g, (kv + 1) * g):
                assert_lse_close(f"LSE [{s},{e}) h{h}", lse[h], torch.log(n[s:e]).cpu().numpy())
                assert_close(f"O [{s},{e}) h{h}", o[h], want_o[s:e].cpu().numpy())
        w = (inp["d_o"][kv * g:(kv + 1) * g].double() / n[None, :, None]).sum(0)   # [R, d]
        want_dv = torch.flip(torch.cumsum(torch.flip(w, [0]), 0), [0])             # sum over i >= j
        assert_close(f"dV_r kv{kv}", dv[kv], want_dv.cpu().numpy())
    assert bool((dk == 0).all()), "dK_r must vanish when Q = 0"
