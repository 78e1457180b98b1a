"""Float64 oracle of replay attention (forward, merge, response-only backward).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation: ``Hq`` query heads, ``Hkv`` KV heads, ``g = Hq / Hkv``, ``d`` head
dim, ``P`` prompt positions, ``R`` response rows, ``s`` softmax scale.

What is computed (LongStraw abstract, cortexa.online: "exact attention
composition", response-only objective with detached prompt state; LongStraw
review page, section 2, item 2 "Qwen3.6-27B": full-attention layers keep every
prompt token's K/V in pages):

  For query head h and response row i, with kv = h // g:
    x_j     = s * <Q[h,i], Kp[kv,j]>      for prompt keys   j in [0, P)
    x_{P+j} = s * <Q[h,i], Kr[kv,j]>      for response keys j in [0, i]
    LSE     = max(x) + ln sum exp(x - max(x))
    p       = exp(x - LSE)
    O[h,i]  = sum_j p_j V_j

  Backward of L = <dO, O> with the prompt K/V detached (DeepRead summary,
  "Method": stopgrad on stored prompt state; review page section 2: the 8-card
  attention backward all-reduces only the query gradient):
    D     = <dO[h,i], O[h,i]>
    dP_j  = <dO[h,i], V_j>,   dS_j = p_j (dP_j - D)
    dQ[h,i]    = s * sum_j dS_j K_j           over prompt AND response keys
    dKr[kv,j]  = s * sum_{h in group kv} sum_{i >= j} dS * Q[h,i]
    dVr[kv,j]  =     sum_{h in group kv} sum_{i >= j} p  * dO[h,i]
    no prompt dK/dV is formed.

Readings where the pages are silent:
  * the response follows the whole prompt: every prompt key is visible to
    every response row, and the mask inside the response is causal including
    the diagonal;
  * GQA grouping is contiguous: query head h uses KV head h // g;
  * Q and K arrive already position-encoded (RoPE, norms and gates lie outside
    this operator);
  * LSE is reported in natural-log units.

The score row is materialised in full and normalised in two passes: this is
the textbook definition, deliberately not the split/online algorithm the GPU
runs, so that the two share no structure beyond the definition itself.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def as_f64(x) -> np.ndarray:
    """Widen a torch tensor (any float dtype, any device) or array to a float64
    numpy array.  bf16 -> float32 -> float64 is exact."""
    try:
        import torch  # local import: numpy inputs need no torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _rows_or_all(rows, hq: int, r: int) -> np.ndarray:
    if rows is None:
        return np.tile(np.arange(r, dtype=np.int64), (hq, 1))
    rows = np.asarray(rows, dtype=np.int64)
    assert rows.ndim == 2 and rows.shape[0] == hq
    return rows


def _score_rows(qb: np.ndarray, kp: np.ndarray, kr: np.ndarray, ib: np.ndarray,
                scale: float) -> np.ndarray:
    """Full score rows for response rows ``ib`` (queries ``qb [n,d]``):
    ``[n, P + R]``; response keys j > i are set to -inf (masked)."""
    xp = scale * (qb @ kp.T)                       # [n, P]
    xr = scale * (qb @ kr.T)                       # [n, R]
    j = np.arange(kr.shape[0])[None, :]
    xr = np.where(j <= ib[:, None], xr, -np.inf)  # causal, diagonal included
    return np.concatenate([xp, xr], axis=1)


def _softmax_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass softmax of full rows: returns (p, lse)."""
    m = np.max(x, axis=1, keepdims=True)
    z = np.sum(np.exp(x - m), axis=1, keepdims=True)
    lse = m + np.log(z)
    return np.exp(x - lse), lse[:, 0]


def replay_forward(q, k_prompt, v_prompt, k_resp, v_resp, scale: float,
                   rows=None, row_block: int = 64):
    """Exact forward of the response rows.

    q ``[Hq,R,d]``; k_prompt, v_prompt ``[Hkv,P,d]`` in logical prompt order;
    k_resp, v_resp ``[Hkv,R,d]``.  ``rows``: ``None`` (all rows) or an int
    array ``[Hq, n]`` of response rows per head.
    Returns ``O [Hq,n,d]`` and ``LSE [Hq,n]`` (float64).
    """
    q, kp, vp, kr, vr = (as_f64(t) for t in (q, k_prompt, v_prompt, k_resp, v_resp))
    hq, r, d = q.shape
    hkv = kp.shape[0]
    g = hq // hkv
    rows = _rows_or_all(rows, hq, r)
    n = rows.shape[1]
    o = np.zeros((hq, n, d))
    lse = np.zeros((hq, n))
    for kv in range(hkv):
        vcat = np.concatenate([vp[kv], vr[kv]], axis=0)
        for h in range(kv * g, (kv + 1) * g):
            for s0 in range(0, n, row_block):
                ib = rows[h, s0:s0 + row_block]
                x = _score_rows(q[h, ib], kp[kv], kr[kv], ib, scale)
                p, l_ = _softmax_rows(x)
                o[h, s0:s0 + len(ib)] = p @ vcat
                lse[h, s0:s0 + len(ib)] = l_
    return o, lse


def replay_backward(q, k_prompt, v_prompt, k_resp, v_resp, d_o, scale: float,
                    rows=None, row_block: int = 64):
    """Response-only backward of ``L = <dO, O>`` with prompt K/V detached.

    Returns ``dQ [Hq,n,d]`` for the requested rows, and ``dK_r, dV_r
    [Hkv,R,d]`` summed over the contributions of the requested rows only (with
    ``rows=None`` these are the full gradients; with a subset, key ``j`` is
    exact when every row ``i >= j`` of every head is in the subset).  Also
    returns the oracle's own ``O`` and ``LSE`` for those rows.
    There is no prompt dK/dV: the prompt state is detached.
    """
    q, kp, vp, kr, vr, do = (as_f64(t) for t in (q, k_prompt, v_prompt, k_resp, v_resp, d_o))
    hq, r, d = q.shape
    hkv, p_len = kp.shape[0], kp.shape[1]
    g = hq // hkv
    rows = _rows_or_all(rows, hq, r)
    n = rows.shape[1]
    dq = np.zeros((hq, n, d))
    dkr = np.zeros((hkv, r, d))
    dvr = np.zeros((hkv, r, d))
    o_all = np.zeros((hq, n, d))
    lse_all = np.zeros((hq, n))
    for kv in range(hkv):
        kcat = np.concatenate([kp[kv], kr[kv]], axis=0)
        vcat = np.concatenate([vp[kv], vr[kv]], axis=0)
        for h in range(kv * g, (kv + 1) * g):
            for s0 in range(0, n, row_block):
                ib = rows[h, s0:s0 + row_block]
                qb, dob = q[h, ib], do[h, ib]
                x = _score_rows(qb, kp[kv], kr[kv], ib, scale)
                p, l_ = _softmax_rows(x)
                o = p @ vcat
                dd = np.sum(dob * o, axis=1, keepdims=True)      # D = <dO, O>
                dp = dob @ vcat.T                                # dP_j = <dO, V_j>
                ds = p * (dp - dd)                               # masked keys: p = 0
                dq[h, s0:s0 + len(ib)] = scale * (ds @ kcat)
                dkr[kv] += scale * (ds[:, p_len:].T @ qb)
                dvr[kv] += p[:, p_len:].T @ dob
                o_all[h, s0:s0 + len(ib)] = o
                lse_all[h, s0:s0 + len(ib)] = l_
    return dq, dkr, dvr, o_all, lse_all


def partial_stats(q, keys, values, scale: float, visible: Optional[np.ndarray] = None):
    """Per-split statistics over a key subset, from the plain definition.

    q ``[n,d]``, keys/values ``[m,d]``, ``visible`` optional bool ``[n,m]``.
    Returns ``(mx [n], l [n], o [n,d])`` with ``mx = max_j x_j``,
    ``l = sum_j exp(x_j - mx)`` and ``o = sum_j exp(x_j - mx) v_j / l``.
    A row that sees no key gets ``(-inf, 0, 0)``.
    """
    q, k, v = as_f64(q), as_f64(keys), as_f64(values)
    n, d = q.shape
    x = scale * (q @ k.T) if k.shape[0] else np.zeros((n, 0))
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    mx = np.full(n, -np.inf)
    l_ = np.zeros(n)
    o = np.zeros((n, d))
    for a in range(n):
        row = x[a]
        if row.size == 0 or not np.isfinite(row).any():
            continue
        mx[a] = np.max(row)
        w = np.exp(row - mx[a])
        l_[a] = np.sum(w)
        o[a] = (w @ v) / l_[a]
    return mx, l_, o


def lse_merge(mx, l_, o):
    """Exact composition of split statistics (the pages' global LSE/output
    merge; LongStraw review page, section 7 mind map, "global LSE softmax
    recomposition").

    ``mx, l [S,n]``, ``o [S,n,d]``.  With ``M = max_c mx_c`` and
    ``w_c = l_c exp(mx_c - M)``: ``O = sum_c w_c o_c / sum_c w_c`` and
    ``LSE = M + ln sum_c w_c``.  Returns ``(O [n,d], LSE [n])``.
    """
    mx, l_, o = as_f64(mx), as_f64(l_), as_f64(o)
    big = np.max(mx, axis=0)
    w = np.where(l_ > 0, l_ * np.exp(mx - np.where(np.isfinite(big), big, 0.0)[None]), 0.0)
    tot = np.sum(w, axis=0)
    safe = np.where(tot > 0, tot, 1.0)
    out = np.einsum("sn,snd->nd", w, o) / safe[:, None]
    lse = np.where(tot > 0, big + np.log(safe), -np.inf)
    return out, lse


def _resp_visible(tok: np.ndarray, rk: int) -> np.ndarray:
    """``[n, rk]`` visibility of response keys ``0..rk-1`` to response tokens
    ``tok`` (causal, diagonal included)."""
    return np.arange(rk)[None, :] <= tok[:, None]


def response_kv_grads(q, k_resp, v_resp, d_o, lse, dvals, scale: float, q_offset: int = 0):
    """dK_r and dV_r of the response keys from given softmax statistics.

    The prompt enters the response-key gradients only through each row's LSE
    (the softmax normaliser) and D = <dO, O>; given those two, the gradient of
    the response keys is a sum over response rows and response keys alone
    (the backward of the pages' response-only objective with the prompt state
    detached; LongStraw abstract, cortexa.online; DeepRead summary, "Method").

    q, d_o ``[Hq, R, d]`` are rows ``q_offset .. q_offset+R-1`` of the
    response; k_resp, v_resp ``[Hkv, >= q_offset+R, d]`` (the first
    ``q_offset + R`` rows are the keys); lse, dvals ``[Hq, R]`` (natural-log
    LSE and D).  For query head h, kv = h // g, row i (token t = q_offset + i)
    and response key j <= t:
        p_ij  = exp(s <Q[h,i], Kr[kv,j]> - LSE[h,i])
        dS_ij = p_ij (<dO[h,i], Vr[kv,j]> - D[h,i])
        dVr[kv,j] = sum_h sum_i p_ij dO[h,i]
        dKr[kv,j] = s sum_h sum_i dS_ij Q[h,i]
    Returns ``dK_r, dV_r [Hkv, q_offset + R, d]`` (float64): the contribution
    of these rows (all of it for a whole response).
    """
    q, kr, vr, do = (as_f64(t) for t in (q, k_resp, v_resp, d_o))
    lse, dvals = as_f64(lse), as_f64(dvals)
    hq, r, d = q.shape
    hkv = kr.shape[0]
    g = hq // hkv
    rk = q_offset + r
    kr, vr = kr[:, :rk], vr[:, :rk]
    vis = _resp_visible(q_offset + np.arange(r), rk)          # [R, rk]
    dk = np.zeros((hkv, rk, d))
    dv = np.zeros((hkv, rk, d))
    for h in range(hq):
        kv = h // g
        x = scale * (q[h] @ kr[kv].T)                           # [R, rk]
        p = np.where(vis, np.exp(np.where(vis, x, 0.0) - lse[h][:, None]), 0.0)
        dp = do[h] @ vr[kv].T                                   # <dO_i, V_j>
        ds = p * (dp - dvals[h][:, None])
        dv[kv] += p.T @ do[h]
        dk[kv] += scale * (ds.T @ q[h])
    return dk, dv
