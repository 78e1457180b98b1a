"""Parity at the full workload sizes.

* the 262,144-position shard (one CP8 share of 2M), one split;
* the 2,097,152-position prefix over 8 splits;
* the G = 8 group replayed serially over that prefix (R = 512 ... 4096);
* the 4,456,448-position stress prefix over 16 splits.

The 262,144-position shard is also checked on every row of every head and on
every key of dK_r and dV_r (about 15 s of host time on 16 threads), and with
LS_ORACLE_FULL=1 the 2,097,152-position prefix too (about 3 minutes).

The float64 oracle computes sampled rows of every query head it checks (row 0,
row R-1 and seeded others) plus the last TAIL rows of every head of the
checked KV groups, which makes dK_r and dV_r exact for the last TAIL keys.  The
Q = 0 closed form checks every row at full size at no oracle cost.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from replay_inputs import (FULL_2M, GROUP_2M, GROUP_2M_RESP_LENS, SHARD_256K, STRESS_4M,
                           logical_prompt, make_inputs, make_response)
from response_replay_attention_amd import Member, PromptCache, replay_backward, replay_forward, replay_group
from tests.parity import assert_close, assert_lse_close, to_np

pytestmark = pytest.mark.gpu

TAIL = 4


def pick_rows(R, n_random, seed, tail=TAIL):
    """Row 0, n_random seeded rows from [1, R - tail), and the last `tail` rows."""
    g = np.random.default_rng(seed)
    mid = g.choice(np.arange(1, R - tail), size=n_random, replace=False)
    return np.concatenate([[0], np.sort(mid), np.arange(R - tail, R)]).astype(np.int64)


def prompt_f64(inp, P, kv):
    kp = logical_prompt(inp["k_pool"], inp["l2p"], P, kv_heads=[kv]).cpu()
    vp = logical_prompt(inp["v_pool"], inp["l2p"], P, kv_heads=[kv]).cpu()
    return oracle.as_f64(kp), oracle.as_f64(vp)


def check_group(shape, inp, resp, fwd, dq, dk, dv, kv, heads, rows, prompt=None, tail_keys=True):
    """Compare the given query heads of KV group kv on `rows`, and (if all heads
    of the group are given and `tail_keys`) dK_r / dV_r of the last TAIL keys."""
    g = shape.hq // shape.hkv
    kp, vp = prompt if prompt is not None else prompt_f64(inp, shape.prompt_len, kv)
    hs = list(heads)
    sel = np.tile(rows, (len(hs), 1))
    q = resp["q"][hs].cpu()
    do = resp["d_o"][hs].cpu()
    kr = resp["k_resp"][kv:kv + 1].cpu()
    vr = resp["v_resp"][kv:kv + 1].cpu()
    # the oracle sees exactly these heads as one group of len(hs) heads on one KV head
    dq_r, dk_r, dv_r, o_r, lse_r = oracle.replay_backward(q, kp[None] if kp.ndim == 2 else kp,
                                                          vp[None] if vp.ndim == 2 else vp,
                                                          kr, vr, do, shape.scale, rows=sel)
    ridx = torch.from_numpy(rows).to(fwd.o.device)
    for n, h in enumerate(hs):
        assert_close(f"O h{h}", fwd.o[h].index_select(0, ridx), o_r[n])
        assert_lse_close(f"LSE h{h}", fwd.lse[h].index_select(0, ridx), lse_r[n])
        assert_close(f"dQ h{h}", dq[h].index_select(0, ridx), dq_r[n])
    if tail_keys and len(hs) == g:
        R = shape.resp_len
        assert_close(f"dK_r kv{kv} tail", dk[kv, R - TAIL:], dk_r[0, R - TAIL:])
        assert_close(f"dV_r kv{kv} tail", dv[kv, R - TAIL:], dv_r[0, R - TAIL:])


def run(shape, inp, resp=None):
    resp = resp or inp
    cache = PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"], shape.num_splits,
                        shape.policy, shape.block_pages)
    fwd = replay_forward(cache, resp["q"], resp["k_resp"], resp["v_resp"], shape.scale)
    dq, dk, dv = replay_backward(cache, resp["q"], resp["k_resp"], resp["v_resp"], fwd.o, fwd.lse,
                                 resp["d_o"], shape.scale)
    torch.cuda.synchronize()
    for t in (fwd.o, fwd.lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    return cache, fwd, dq, dk, dv


@pytest.mark.parametrize("shape,kv_heads,n_random", [
    (SHARD_256K, (0, 1, 2, 3), 3),
    (FULL_2M, (0, 3), 3),
    (STRESS_4M, (1, 2), 2),
], ids=["shard_262k", "prefix_2m_s8", "stress_4m_s16"])
def test_full_size_sampled_rows(shape, kv_heads, n_random):
    print(f"case {shape.name}", flush=True)
    inp = make_inputs(shape, seed=20260001, device="cuda")
    _, fwd, dq, dk, dv = run(shape, inp)
    g = shape.hq // shape.hkv
    for kv in kv_heads:
        rows = pick_rows(shape.resp_len, n_random, seed=kv)
        check_group(shape, inp, inp, fwd, dq, dk, dv, kv, range(kv * g, (kv + 1) * g), rows)
        print(f"  kv head {kv} ok", flush=True)


@pytest.mark.parametrize("shape", [FULL_2M, STRESS_4M], ids=["prefix_2m_s8", "stress_4m_s16"])
def test_full_size_zero_query_closed_form(shape):
    """Q = 0 at full size: every row, every head.  LSE_i = ln(P + i + 1) and
    O_i = mean of the P + i + 1 visible values."""
    inp = make_inputs(shape, seed=20260003, device="cuda", q_zero=True)
    _, fwd, *_ = run(shape, inp)
    P, R, g = shape.prompt_len, shape.resp_len, shape.hq // shape.hkv
    n = torch.arange(R, device="cuda", dtype=torch.float64) + P + 1
    want_lse = torch.log(n)
    for kv in range(shape.hkv):
        vp = logical_prompt(inp["v_pool"], inp["l2p"], P, kv_heads=[kv])[0]
        psum = vp.double().sum(0)
        csum = psum[None, :] + torch.cumsum(inp["v_resp"][kv].double(), 0)
        want_o = (csum / n[:, None]).cpu().numpy()
        for h in range(kv * g, (kv + 1) * g):
            assert_lse_close(f"LSE h{h}", fwd.lse[h], want_lse.cpu().numpy())
            assert_close(f"O h{h}", fwd.o[h], want_o)


def _group_members(shape, lens, seed0):
    return [make_response(shape.with_(resp_len=r), seed0 + i, device="cuda") for i, r in enumerate(lens)]


@pytest.mark.parametrize("half", [0, 1])
def test_group_replay_parity(half):
    """G = 8 over the shared 2M prefix, replayed serially; each member checked
    on sampled rows of two query heads (rotating KV groups), the smallest and
    largest members also on the exact tail dK_r/dV_r of one full KV group."""
    shape = GROUP_2M
    inp = make_inputs(shape, seed=20260004, device="cuda")
    lens = GROUP_2M_RESP_LENS[4 * half: 4 * half + 4]
    members = _group_members(shape, lens, 100 + 4 * half)
    g = shape.hq // shape.hkv
    got = {}

    def keep(i, fwd, dq, dk, dv):
        got[i] = (fwd, dq, dk, dv)   # kept for checking after the loop (test only)

    cache = PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"], shape.num_splits)
    replay_group(cache, [Member(m["q"], m["k_resp"], m["v_resp"], m["d_o"]) for m in members],
                 consume=keep, scale=shape.scale)
    torch.cuda.synchronize()
    prompts = {}
    for i, (r, m) in enumerate(zip(lens, members)):
        ms = shape.with_(resp_len=r)
        fwd, dq, dk, dv = got[i]
        kv = (i + 2 * half) % shape.hkv
        if kv not in prompts:
            prompts[kv] = prompt_f64(inp, shape.prompt_len, kv)
        full = (half == 0 and i == 0) or (half == 1 and i == 3)
        heads = range(kv * g, (kv + 1) * g) if full else (kv * g, kv * g + g - 1)
        rows = pick_rows(r, 2, seed=r)
        check_group(ms, inp, m, fwd, dq, dk, dv, kv, heads, rows, prompt=prompts[kv])
        print(f"  member R={r} kv {kv} ok", flush=True)


def test_group_peak_memory_follows_longest_member():
    """Serial replay: the peak over the whole group is the peak of its longest
    member alone (no member's buffers outlive it)."""
    shape = GROUP_2M
    inp = make_inputs(shape, seed=20260005, device="cuda")
    cache = PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"], shape.num_splits)
    members = _group_members(shape, GROUP_2M_RESP_LENS, 300)
    mem = [Member(m["q"], m["k_resp"], m["v_resp"], m["d_o"]) for m in members]
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    replay_group(cache, mem[-1:], scale=shape.scale)
    torch.cuda.synchronize()
    peak_longest = torch.cuda.max_memory_allocated() - base
    torch.cuda.reset_peak_memory_stats()
    replay_group(cache, mem, scale=shape.scale)
    torch.cuda.synchronize()
    peak_group = torch.cuda.max_memory_allocated() - base
    assert torch.cuda.memory_allocated() == base
    print(f"peak longest {peak_longest / 2**20:.1f} MiB, group {peak_group / 2**20:.1f} MiB", flush=True)
    assert peak_group <= peak_longest + (1 << 20)


_FULL_2M_OPT_IN = pytest.mark.skipif(
    os.environ.get("LS_ORACLE_FULL") != "1",
    reason="every row at 2M takes about 3 minutes of host time; set LS_ORACLE_FULL=1")


@pytest.mark.timeout(3000)
@pytest.mark.parametrize("shape", [SHARD_256K, pytest.param(FULL_2M, marks=_FULL_2M_OPT_IN)],
                         ids=["shard_262k", "prefix_2m_s8"])
def test_full_size_every_row(shape):
    """The whole output against the whole oracle: O, LSE and dQ of every row of
    every query head, dK_r and dV_r of every response key of every KV head.

    The oracle runs as one task per (query head, block of rows) on host
    threads (numpy releases the GIL in its array loops and BLAS calls); each
    task returns its rows' dQ, O, LSE and its rows' contribution to dK_r and
    dV_r, and a KV head's dK_r / dV_r is the sum of those contributions over
    the heads of its group and all their rows."""
    print(f"case {shape.name} every row", flush=True)
    inp = make_inputs(shape, seed=20260001, device="cuda")
    _, fwd, dq, dk, dv = run(shape, inp)
    g, P, R = shape.hq // shape.hkv, shape.prompt_len, shape.resp_len
    got = {k: t.cpu() for k, t in (("o", fwd.o), ("lse", fwd.lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    prompts = [(oracle.as_f64(logical_prompt(inp["k_pool"], inp["l2p"], P, kv_heads=[kv])),
                oracle.as_f64(logical_prompt(inp["v_pool"], inp["l2p"], P, kv_heads=[kv])))
               for kv in range(shape.hkv)]
    resp = {k: oracle.as_f64(inp[k]) for k in ("q", "d_o", "k_resp", "v_resp")}
    del inp, fwd, dq, dk, dv
    torch.cuda.empty_cache()
    rows_per_task = 256   # each task copies its KV head's prompt once: keep the tasks few
    tasks = [(h, r0) for h in range(shape.hq) for r0 in range(0, R, rows_per_task)]
    t_start = time.time()

    def task(t):
        h, r0 = t
        kv = h // g
        rows = np.arange(r0, min(R, r0 + rows_per_task), dtype=np.int64)[None]
        out = oracle.replay_backward(resp["q"][h:h + 1], prompts[kv][0], prompts[kv][1],
                                     resp["k_resp"][kv:kv + 1], resp["v_resp"][kv:kv + 1],
                                     resp["d_o"][h:h + 1], shape.scale, rows=rows)
        print(f"  oracle head {h} rows [{r0}, {r0 + rows.shape[1]}): {time.time() - t_start:.0f} s",
              flush=True)
        return out

    # one BLAS thread per task (several BLAS pools spinning at once stall each
    # other), and no more tasks at once than ~150 GB of host memory holds: each
    # concatenates its KV head's prompt and response keys and values, and
    # holds a few [64, P + R] float64 temporaries
    per_task = 2 * (P + R) * shape.head_dim * 8 + 6 * 64 * (P + R) * 8
    workers = int(os.environ.get("LS_ORACLE_THREADS", "0")) or max(
        1, min(len(os.sched_getaffinity(0)), 16, (150 << 30) // per_task))
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(task, tasks))
    print(f"  oracle host time {time.time() - t_start:.0f} s on {workers} threads", flush=True)
    o_r = np.zeros((shape.hq, R, shape.head_dim))
    dq_r = np.zeros_like(o_r)
    lse_r = np.zeros((shape.hq, R))
    dk_r = np.zeros((shape.hkv, R, shape.head_dim))
    dv_r = np.zeros_like(dk_r)
    for (h, r0), (dq_t, dk_t, dv_t, o_t, lse_t) in zip(tasks, results):
        n = o_t.shape[1]
        o_r[h, r0:r0 + n], dq_r[h, r0:r0 + n], lse_r[h, r0:r0 + n] = o_t[0], dq_t[0], lse_t[0]
        dk_r[h // g] += dk_t[0]
        dv_r[h // g] += dv_t[0]
    m = {"O": assert_close("O", got["o"], o_r),
         "dQ": assert_close("dQ", got["dq"], dq_r),
         "dK_r": assert_close("dK_r", got["dk"], dk_r),
         "dV_r": assert_close("dV_r", got["dv"], dv_r)}
    lse_rel = assert_lse_close("LSE", got["lse"], lse_r)
    print(f"  LSE rel {lse_rel:.2e}; "
          + "; ".join(f"{k} max_abs {v['max_abs']:.2e} rel_l2 {v['rel_l2']:.2e}" for k, v in m.items()),
          flush=True)
