"""CPU ORACLE for the backward pass of the routed and shared attention.  TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the HIP library never does, and the two share no code.

What it differentiates (GQE study note, dimensionstp.github.io, §3-2 (3); GQA tutorial, GQA 核心原理与计算流程
step 4): for batch b and group g the routed query rows q_r, r = t·k + j (the j-th kept expert of token t),
attend the group's single K/V head; with causal masking row r sees keys 0..t.  The shared rows (one per token)
attend KV head 0 in the same way.  Each row's output is o_r = softmax(q_r K^T / sqrt(d_head)) V, and it is the
row's slot: hard slot g·k + j of token t for a routed row, the last slot for a shared row.  Given the gradient
of those slots (dO), this module returns the gradients of the loss L = sum(dO * O) with respect to the query
rows, K and V, by float64 autograd of that definition.  The weighted slot is not an input here: its share of
the hard slots' gradient is already in the hard-slot gradient the routing backward returns.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(a):
    if isinstance(a, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    return a.detach().to("cpu", torch.float64)


def head_backward(q, K, V, dO, kk, causal=True):
    """One head: q [R, d] query rows (row r at position r // kk), K, V [T, d], dO [R, d].

    Returns dict of float64 numpy arrays dq [R, d], dk [T, d], dv [T, d], and the forward's P [R, T] and
    the score gradient dS = dL/dS [R, T] (S = q K^T / sqrt(d)), for error bounds."""
    q = _f64(q).requires_grad_(True)
    K = _f64(K).requires_grad_(True)
    V = _f64(V).requires_grad_(True)
    dO = _f64(dO)
    R, d = q.shape
    T = K.shape[0]
    S = (q @ K.T) / np.sqrt(d)
    S.retain_grad()
    if causal:
        pos = torch.arange(R) // kk
        S_m = S.masked_fill(torch.arange(T)[None, :] > pos[:, None], float("-inf"))
    else:
        S_m = S
    P = torch.softmax(S_m, dim=-1)
    O = P @ V
    (dO * O).sum().backward()
    g = lambda t: (t.grad if t.grad is not None else torch.zeros_like(t)).detach().numpy()  # noqa: E731
    return dict(dq=g(q), dk=g(K), dv=g(V), P=P.detach().numpy(), dS=g(S))


def attention_backward(w, q_routed, q_shared, K, V, d_hard, dout, heads=None):
    """Whole layer.  q_routed [B, G, T*k, d]; q_shared [B, T, d] or None; K, V [B, G, T, d];
    d_hard [B*T, G*k, d] the hard slots' gradient; dout [B*T, S, d] (its last slot is the shared slot's
    gradient; None without a shared head).  ``heads``: optional list of (b, h) to compute, h = G for the
    shared head (default all).

    Returns dict: dq_routed [B, G, T*k, d], dq_shared [B, T, d] or None, dk, dv [B, G, T, d] (float64; heads
    not computed are NaN, and dk/dv of a KV head are complete only when every head that reads it is)."""
    B, G, T, d = K.shape
    k = w.k
    shared = q_shared is not None and w.n_shared
    qr = _f64(q_routed).reshape(B, G, T * k, d)
    dh = _f64(d_hard).reshape(B, T, G, k, d)
    dq_r = np.full((B, G, T * k, d), np.nan)
    dq_s = np.full((B, T, d), np.nan) if shared else None
    dk = np.zeros((B, G, T, d))
    dv = np.zeros((B, G, T, d))
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(G + (1 if shared else 0))]
    Kd, Vd = _f64(K), _f64(V)
    for b, h in heads:
        if h < G:
            dO = dh[b, :, h].reshape(T * k, d)      # row t*k + j <- hard slot h*k + j of token t
            r = head_backward(qr[b, h], Kd[b, h], Vd[b, h], dO, k, w.causal)
            dq_r[b, h] = r["dq"]
            kvh = h
        else:
            dO = _f64(dout).reshape(B, T, -1, d)[b, :, -1]
            r = head_backward(_f64(q_shared).reshape(B, T, d)[b], Kd[b, 0], Vd[b, 0], dO, 1, w.causal)
            dq_s[b] = r["dq"]
            kvh = 0
        dk[b, kvh] += r["dk"]
        dv[b, kvh] += r["dv"]
    return dict(dq_routed=dq_r, dq_shared=dq_s, dk=dk, dv=dv)


def row_lse2(q, K, kk, causal=True):
    """The base-2 log of each row's softmax denominator (GQE study note §1-1 attention equation):
    lse[r] = log2 sum_s exp(q_r . K_s / sqrt(d)) over the keys row r sees (r // kk >= s when causal), which is
    the statistic that turns a row's scores into its softmax, P[r, s] = 2^(q_r . K_s log2(e) / sqrt(d) - lse[r]).
    q [R, d], K [T, d].  Returns float64 numpy [R]."""
    q, K = _f64(q), _f64(K)
    R, d = q.shape
    T = K.shape[0]
    S = (q @ K.T) / np.sqrt(d)
    if causal:
        pos = torch.arange(R) // kk
        S = S.masked_fill(torch.arange(T)[None, :] > pos[:, None], float("-inf"))
    return (torch.logsumexp(S, dim=-1) / np.log(2.0)).numpy()


__all__ = ["head_backward", "attention_backward", "row_lse2"]
