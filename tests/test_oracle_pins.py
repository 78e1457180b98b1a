"""Pins for the float64 oracle, independent of the oracle's own code.

Each test checks the oracle against something the mathematics fixes: a library
routine on a differently formed problem (one causal softmax attention over the
concatenated [prompt; response] sequence, torch's scaled_dot_product_attention
and autograd in float64), closed forms, central finite differences, exact
invariances of the split/merge composition, and identities of the gradient.
The pages print no worked example, so there is no printed value to pin to.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
from oracle import attention as oatt

RNG = np.random.default_rng(1234)


def _problem(hq=6, hkv=2, d=32, p=300, r=20, seed=0, qmul=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, r, d)) * qmul
    kp = rng.standard_normal((hkv, p, d))
    vp = rng.standard_normal((hkv, p, d))
    kr = rng.standard_normal((hkv, r, d))
    vr = rng.standard_normal((hkv, r, d))
    do = rng.standard_normal((hq, r, d))
    return q, kp, vp, kr, vr, do


def _full_sequence_sdpa(q, kp, vp, kr, vr, scale, grad=False, prompt_grad=False):
    """One causal attention over the whole concatenated sequence, done by torch.

    Prompt query rows are filled with zeros (they are discarded); the response
    rows are the last R rows.  GQA by repeat_interleave (contiguous groups)."""
    hq, r, d = q.shape
    hkv, p, _ = kp.shape
    g = hq // hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=grad)
    tkp = torch.tensor(kp, dtype=torch.float64, requires_grad=prompt_grad)
    tvp = torch.tensor(vp, dtype=torch.float64, requires_grad=prompt_grad)
    tkr = torch.tensor(kr, dtype=torch.float64, requires_grad=grad)
    tvr = torch.tensor(vr, dtype=torch.float64, requires_grad=grad)
    qfull = torch.cat([torch.zeros(hq, p, d, dtype=torch.float64), tq], dim=1)
    kfull = torch.cat([tkp, tkr], dim=1).repeat_interleave(g, dim=0)
    vfull = torch.cat([tvp, tvr], dim=1).repeat_interleave(g, dim=0)
    n = p + r
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    out = F.scaled_dot_product_attention(qfull[None], kfull[None], vfull[None],
                                         attn_mask=mask, scale=scale)[0]
    return out[:, p:], (tq, tkp, tvp, tkr, tvr)


def _full_sequence_lse(q, kp, kr, scale):
    hq, r, d = q.shape
    hkv, p, _ = kp.shape
    g = hq // hkv
    lse = np.zeros((hq, r))
    for h in range(hq):
        kfull = np.concatenate([kp[h // g], kr[h // g]])
        x = scale * (q[h] @ kfull.T)
        for i in range(r):
            lse[h, i] = logsumexp(x[i, : p + i + 1])
    return lse


@pytest.mark.parametrize("hq,hkv,d,p,r", [(6, 1, 16, 40, 9), (6, 2, 32, 300, 20), (4, 4, 8, 0, 7), (8, 2, 24, 1, 33)])
def test_forward_equals_full_sequence_causal_sdpa(hq, hkv, d, p, r):
    q, kp, vp, kr, vr, _ = _problem(hq, hkv, d, p, r, seed=hq * 100 + p)
    s = 1 / math.sqrt(d)
    o, lse = oracle.replay_forward(q, kp, vp, kr, vr, s)
    ref, _ = _full_sequence_sdpa(q, kp, vp, kr, vr, s)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _full_sequence_lse(q, kp, kr, s), rtol=1e-13, atol=1e-13)


def test_forward_sampled_rows_match_all_rows():
    q, kp, vp, kr, vr, _ = _problem(6, 2, 16, 100, 31, seed=5)
    s = 0.25
    o, lse = oracle.replay_forward(q, kp, vp, kr, vr, s)
    rows = np.array([[0, 3, 30]] * 6)
    os_, ls_ = oracle.replay_forward(q, kp, vp, kr, vr, s, rows=rows, row_block=2)
    np.testing.assert_allclose(os_, o[:, [0, 3, 30]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ls_, lse[:, [0, 3, 30]], rtol=0, atol=1e-13)


def test_forward_closed_form_zero_query():
    """Q = 0: every visible key has the same score, so LSE = ln(#visible) and
    O is the plain mean of the visible values."""
    q, kp, vp, kr, vr, _ = _problem(6, 2, 16, 257, 12, seed=7)
    q[:] = 0
    o, lse = oracle.replay_forward(q, kp, vp, kr, vr, 1 / 4)
    p = kp.shape[1]
    for h in range(6):
        for i in range(12):
            n = p + i + 1
            assert abs(lse[h, i] - math.log(n)) < 1e-12
            mean = (vp[h // 3].sum(0) + vr[h // 3, : i + 1].sum(0)) / n
            np.testing.assert_allclose(o[h, i], mean, rtol=0, atol=1e-13)


def test_forward_constant_values():
    q, kp, vp, kr, vr, _ = _problem(6, 3, 8, 50, 10, seed=9, qmul=3.0)
    vp[:] = 0.75
    vr[:] = 0.75
    o, _ = oracle.replay_forward(q, kp, vp, kr, vr, 1.0)
    np.testing.assert_allclose(o, 0.75, rtol=0, atol=1e-13)


def test_first_row_sees_prompt_and_own_key_only():
    """Row 0 of the response sees the prompt plus response key 0: changing any
    later response key or value must not move it (causality)."""
    q, kp, vp, kr, vr, _ = _problem(6, 2, 16, 30, 8, seed=11)
    o1, l1 = oracle.replay_forward(q, kp, vp, kr, vr, 0.3)
    kr2, vr2 = kr.copy(), vr.copy()
    kr2[:, 1:] += 5.0
    vr2[:, 1:] -= 3.0
    o2, l2 = oracle.replay_forward(q, kp, vp, kr2, vr2, 0.3)
    np.testing.assert_array_equal(o1[:, 0], o2[:, 0])
    np.testing.assert_array_equal(l1[:, 0], l2[:, 0])
    assert np.abs(o1[:, 1:] - o2[:, 1:]).min() > 0


@pytest.mark.parametrize("hq,hkv,d,p,r", [(6, 1, 16, 40, 9), (6, 2, 32, 70, 16), (4, 2, 8, 0, 6)])
def test_backward_equals_autograd_with_detached_prompt(hq, hkv, d, p, r):
    q, kp, vp, kr, vr, do = _problem(hq, hkv, d, p, r, seed=d + p)
    s = 1 / math.sqrt(d)
    dq, dkr, dvr, o, lse = oracle.replay_backward(q, kp, vp, kr, vr, do, s)
    out, (tq, _, _, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True)
    (out * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dkr, tkr.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dvr, tvr.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-12)


def test_response_gradients_do_not_depend_on_prompt_requiring_grad():
    """The stopgrad drops only the prompt K/V gradient: dQ, dK_r, dV_r are the
    same whether or not the prompt K/V carry gradient; the dropped prompt
    gradient itself is non-zero."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 50, 12, seed=3)
    s = 0.25
    dq, dkr, dvr, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, s)
    out, (tq, tkp, tvp, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True, prompt_grad=True)
    (out * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dkr, tkr.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dvr, tvr.grad.numpy(), atol=1e-11, rtol=0)
    assert np.abs(tkp.grad.numpy()).max() > 1e-3
    assert np.abs(tvp.grad.numpy()).max() > 1e-3


def test_backward_finite_differences():
    """Central differences of L = <dO, O> through the oracle's forward."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 8, 23, 6, seed=21)
    s = 0.4
    dq, dkr, dvr, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, s)

    def loss(q_, kr_, vr_):
        o, _ = oracle.replay_forward(q_, kp, vp, kr_, vr_, s)
        return float(np.sum(o * do))

    eps = 1e-5
    rng = np.random.default_rng(0)
    for _ in range(12):
        idx = tuple(int(rng.integers(0, n)) for n in q.shape)
        a, b = q.copy(), q.copy()
        a[idx] += eps
        b[idx] -= eps
        fd = (loss(a, kr, vr) - loss(b, kr, vr)) / (2 * eps)
        assert abs(fd - dq[idx]) <= 1e-6 * max(1.0, abs(fd))
    for target, grad in ((1, dkr), (2, dvr)):
        base = kr if target == 1 else vr
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            a, b = base.copy(), base.copy()
            a[idx] += eps
            b[idx] -= eps
            la = loss(q, a, vr) if target == 1 else loss(q, kr, a)
            lb = loss(q, b, vr) if target == 1 else loss(q, kr, b)
            fd = (la - lb) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd))


def test_dq_vanishes_for_constant_keys():
    """Softmax shift invariance: sum_j dS_ij = 0, so with every key equal to
    one vector c, dQ = s * c * sum_j dS_ij = 0."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 40, 10, seed=13)
    kp[:] = 0.3
    kr[:] = 0.3
    dq, _, _, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, 0.5)
    assert np.abs(dq).max() < 1e-12


def test_dv_identity_without_prompt():
    """With no prompt, sum_j dV_r[kv, j] = sum_{h in group, i} dO[h, i]
    (every softmax row sums to one).  With a prompt the response share is
    strictly smaller: the rest is the detached prompt's dV."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 0, 14, seed=17)
    _, _, dvr, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, 0.25)
    for kv in range(2):
        np.testing.assert_allclose(dvr[kv].sum(0), do[kv * 3:(kv + 1) * 3].sum((0, 1)), atol=1e-12, rtol=0)
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 64, 14, seed=17)
    _, _, dvr, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, 0.25)
    gap = dvr[0].sum(0) - do[0:3].sum((0, 1))
    assert np.abs(gap).max() > 1e-3


def test_subset_rows_give_exact_tail_key_gradients():
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 33, 20, seed=19)
    _, dkr, dvr, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, 0.25)
    rows = np.tile(np.arange(15, 20), (6, 1))
    _, dkr2, dvr2, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, 0.25, rows=rows)
    np.testing.assert_allclose(dkr2[:, 15:], dkr[:, 15:], atol=1e-13, rtol=0)
    np.testing.assert_allclose(dvr2[:, 15:], dvr[:, 15:], atol=1e-13, rtol=0)


def test_row_block_contributions_match_masked_autograd():
    """A token block's rows alone (the oracle's rows= subset, as the token-block
    replay uses it) give what autograd gives for <dO, O> with dO zero outside
    the block: rows with dO = 0 have dP = 0 and D = 0, so they add nothing.
    The blocks' contributions then sum to the whole response's gradient."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 37, 23, seed=29)
    s = 0.25
    _, dkr_all, dvr_all, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, s)
    dk_sum, dv_sum = np.zeros_like(dkr_all), np.zeros_like(dvr_all)
    for b0, b1 in ((0, 6), (6, 13), (13, 23)):
        rows = np.tile(np.arange(b0, b1), (6, 1))
        dq_b, dk_b, dv_b, _, _ = oracle.replay_backward(q, kp, vp, kr, vr, do, s, rows=rows)
        out, (tq, _, _, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True)
        mask = np.zeros_like(do)
        mask[:, b0:b1] = 1.0
        (out * torch.tensor(do * mask)).sum().backward()
        np.testing.assert_allclose(dk_b, tkr.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv_b, tvr.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dq_b, tq.grad.numpy()[:, b0:b1], atol=1e-11, rtol=0)
        assert not dk_b[:, b1:].any() and not dv_b[:, b1:].any()   # keys after the block
        dk_sum += dk_b
        dv_sum += dv_b
    np.testing.assert_allclose(dk_sum, dkr_all, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv_sum, dvr_all, atol=1e-12, rtol=0)


@pytest.mark.parametrize("hq,hkv,d,p,r", [(6, 1, 16, 40, 9), (6, 2, 32, 70, 16), (4, 2, 8, 0, 6),
                                         (8, 2, 24, 1, 33)])
def test_response_kv_grads_from_statistics_equal_autograd(hq, hkv, d, p, r):
    """dK_r, dV_r from the statistics alone: with LSE from scipy's logsumexp of
    the full causal score rows and D from torch's SDPA output, they equal
    autograd's response-key gradients of the full-sequence attention with the
    prompt detached."""
    q, kp, vp, kr, vr, do = _problem(hq, hkv, d, p, r, seed=7 * d + p)
    s = 1 / math.sqrt(d)
    out, (_, _, _, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True)
    (out * torch.tensor(do)).sum().backward()
    lse = _full_sequence_lse(q, kp, kr, s)
    dvals = (out.detach().numpy() * do).sum(-1)
    dk, dv = oracle.response_kv_grads(q, kr, vr, do, lse, dvals, s)
    np.testing.assert_allclose(dk, tkr.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tvr.grad.numpy(), rtol=0, atol=1e-11)


def test_response_kv_grads_of_token_blocks_equal_masked_autograd():
    """A token block's rows at q_offset, with the statistics of the whole
    response, give autograd's response-key gradients of <dO, O> with dO zero
    outside the block; keys after the block get nothing, and the blocks sum to
    the whole response's gradient."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 37, 23, seed=41)
    s = 0.25
    out, _ = _full_sequence_sdpa(q, kp, vp, kr, vr, s)
    lse = _full_sequence_lse(q, kp, kr, s)
    dvals = (out.detach().numpy() * do).sum(-1)
    dk_all, dv_all = oracle.response_kv_grads(q, kr, vr, do, lse, dvals, s)
    dk_sum, dv_sum = np.zeros_like(dk_all), np.zeros_like(dv_all)
    for b0, b1 in ((0, 6), (6, 13), (13, 23)):
        out, (_, _, _, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True)
        mask = np.zeros_like(do)
        mask[:, b0:b1] = 1.0
        (out * torch.tensor(do * mask)).sum().backward()
        dk_b, dv_b = oracle.response_kv_grads(q[:, b0:b1], kr, vr, do[:, b0:b1], lse[:, b0:b1],
                                              dvals[:, b0:b1], s, q_offset=b0)
        assert dk_b.shape == (2, b1, 16)
        np.testing.assert_allclose(dk_b, tkr.grad.numpy()[:, :b1], atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv_b, tvr.grad.numpy()[:, :b1], atol=1e-11, rtol=0)
        assert not tkr.grad.numpy()[:, b1:].any()
        dk_sum[:, :b1] += dk_b
        dv_sum[:, :b1] += dv_b
    np.testing.assert_allclose(dk_sum, dk_all, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv_sum, dv_all, atol=1e-12, rtol=0)


def test_response_kv_grads_planted_mistakes_are_caught(monkeypatch):
    """The autograd pin above fails when the causal mask of the response keys
    is wrong (diagonal dropped, or one key too many)."""
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 30, 11, seed=43)
    s = 0.25
    out, (_, _, _, tkr, tvr) = _full_sequence_sdpa(q, kp, vp, kr, vr, s, grad=True)
    (out * torch.tensor(do)).sum().backward()
    lse = _full_sequence_lse(q, kp, kr, s)
    dvals = (out.detach().numpy() * do).sum(-1)

    def pin_holds():
        dk, dv = oracle.response_kv_grads(q, kr, vr, do, lse, dvals, s)
        return (np.abs(dk - tkr.grad.numpy()).max() < 1e-11
                and np.abs(dv - tvr.grad.numpy()).max() < 1e-11)

    good = oatt._resp_visible
    assert pin_holds()
    for bad in (lambda tok, rk: good(tok - 1, rk), lambda tok, rk: good(tok + 1, rk)):
        monkeypatch.setattr(oatt, "_resp_visible", bad)
        assert not pin_holds()
    monkeypatch.setattr(oatt, "_resp_visible", good)
    assert pin_holds()


def _split_parts(q, kp, vp, kr, vr, s, order, offsets):
    """Per-split statistics for every (head,row), the response block last."""
    hq, r, d = q.shape
    g = hq // kp.shape[0]
    ns = len(offsets) - 1
    m = np.zeros((ns + 1, hq * r))
    l_ = np.zeros((ns + 1, hq * r))
    o = np.zeros((ns + 1, hq * r, d))
    for h in range(hq):
        kv = h // g
        sl = slice(h * r, (h + 1) * r)
        for c in range(ns):
            keys = np.array(order[offsets[c]:offsets[c + 1]], dtype=np.int64)
            m[c, sl], l_[c, sl], o[c, sl] = oracle.partial_stats(q[h], kp[kv][keys], vp[kv][keys], s)
        vis = np.arange(r)[None, :] <= np.arange(r)[:, None]
        m[ns, sl], l_[ns, sl], o[ns, sl] = oracle.partial_stats(q[h], kr[kv], vr[kv], s, visible=vis)
    return m, l_, o


@pytest.mark.parametrize("kind", ["contiguous", "cyclic", "random", "single", "with_empty", "permuted"])
def test_merge_of_any_key_partition_is_exact(kind):
    q, kp, vp, kr, vr, _ = _problem(6, 2, 16, 96, 11, seed=23, qmul=2.0)
    p = kp.shape[1]
    rng = np.random.default_rng(len(kind))
    if kind == "contiguous":
        order, offsets = list(range(p)), [0, 30, 61, 96]
    elif kind == "cyclic":
        order = [j for c in range(8) for j in range(c, p, 8)]
        offsets = [12 * c for c in range(9)]
    elif kind == "random":
        owner = rng.integers(0, 5, p)
        order = [j for c in range(5) for j in range(p) if owner[j] == c]
        offsets = [0] + list(np.cumsum([int((owner == c).sum()) for c in range(5)]))
    elif kind == "single":
        order, offsets = list(range(p)), [0, p]
    elif kind == "with_empty":
        order, offsets = list(range(p)), [0, 0, 50, 50, 96, 96]
    else:
        perm = list(rng.permutation(p))
        order, offsets = perm, [0, 40, 96]
    s = 0.25
    m, l_, o = _split_parts(q, kp, vp, kr, vr, s, order, offsets)
    if kind == "permuted":
        idx = rng.permutation(m.shape[0])
        m, l_, o = m[idx], l_[idx], o[idx]
    om, lm = oracle.lse_merge(m, l_, o)
    of, lf = oracle.replay_forward(q, kp, vp, kr, vr, s)
    np.testing.assert_allclose(om, of.reshape(-1, of.shape[-1]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lm, lf.reshape(-1), rtol=1e-14, atol=1e-13)


def test_partial_stats_of_empty_split():
    m, l_, o = oracle.partial_stats(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(np.isneginf(m)) and np.all(l_ == 0) and np.all(o == 0)


def test_merge_drops_nothing():
    """Dropping one split changes the LSE by ln of the remaining weight:
    the merge is exact, not an approximation."""
    q, kp, vp, kr, vr, _ = _problem(6, 2, 16, 64, 5, seed=29)
    m, l_, o = _split_parts(q, kp, vp, kr, vr, 0.25, list(range(64)), [0, 32, 64])
    _, lse_all = oracle.lse_merge(m, l_, o)
    _, lse_less = oracle.lse_merge(m[1:], l_[1:], o[1:])
    w0 = l_[0] * np.exp(m[0] - lse_all)
    np.testing.assert_allclose(lse_less, lse_all + np.log1p(-w0), atol=1e-12, rtol=0)


# -- planted mistakes: each must break at least one pin above ------------------

def _sdpa_pin_holds(monkeypatch_target=None):
    q, kp, vp, kr, vr, do = _problem(6, 2, 16, 40, 9, seed=31)
    s = 0.25
    o, lse = oracle.replay_forward(q, kp, vp, kr, vr, s)
    ref, _ = _full_sequence_sdpa(q, kp, vp, kr, vr, s)
    return np.abs(o - ref.detach().numpy()).max() < 1e-12 and \
        np.abs(lse - _full_sequence_lse(q, kp, kr, s)).max() < 1e-12


def test_planted_mistakes_are_caught(monkeypatch):
    assert _sdpa_pin_holds()
    good = oatt._score_rows

    def no_diagonal(qb, kp, kr, ib, scale):
        x = good(qb, kp, kr, ib, scale)
        p = kp.shape[0]
        for a, i in enumerate(ib):
            x[a, p + i] = -np.inf
        return x

    def unscaled_prompt(qb, kp, kr, ib, scale):
        x = good(qb, kp, kr, ib, scale)
        x[:, : kp.shape[0]] /= scale
        return x

    def off_by_one_mask(qb, kp, kr, ib, scale):
        return good(qb, kp, kr, ib + 1, scale)

    for bad in (no_diagonal, unscaled_prompt, off_by_one_mask):
        monkeypatch.setattr(oatt, "_score_rows", bad)
        assert not _sdpa_pin_holds(), bad.__name__
    monkeypatch.setattr(oatt, "_score_rows", good)
    assert _sdpa_pin_holds()


def _golden_hand_example():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_example.json")
    g = json.load(open(path))
    env = {"ln": math.log}

    def val(x):
        return float(eval(x, {"__builtins__": {}}, env)) if isinstance(x, str) else float(x)

    def arr(x):
        return np.array([[val(e) for e in row] for row in x]) if isinstance(x[0], list) else np.array([val(e) for e in x])
    inp = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    exp = {k: arr(v) for k, v in g["expected"].items()}
    return inp, val(g["scale"]), exp


def test_hand_worked_example():
    """The oracle against a replay worked by hand (tests/golden)."""
    inp, s, exp = _golden_hand_example()
    q, do = inp["q"][None], inp["d_o"][None]
    kp, vp = inp["k_prompt"][None], inp["v_prompt"][None]
    kr, vr = inp["k_resp"][None], inp["v_resp"][None]
    dq, dkr, dvr, o, lse = oracle.replay_backward(q, kp, vp, kr, vr, do, s)
    np.testing.assert_allclose(o[0], exp["o"], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse[0], exp["lse"], atol=1e-14, rtol=0)
    np.testing.assert_allclose(dq[0], exp["dq"], atol=1e-14, rtol=0)
    np.testing.assert_allclose(dkr[0], exp["dk_resp"], atol=1e-14, rtol=0)
    np.testing.assert_allclose(dvr[0], exp["dv_resp"], atol=1e-14, rtol=0)
