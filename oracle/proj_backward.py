"""CPU ORACLE for the backward pass of the query, key and value projections.  TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the HIP library never does, and the two share no code.

What it differentiates (GQE study note, dimensionstp.github.io, §3-2 (2) and (5): each kept expert is its own
query projection of x_t and the shared head another, unselected experts are not projected; GQA tutorial,
GQA 核心原理与计算流程 step 2: K and V are linear projections of x): for token t of sequence b and group g,
  q_routed[b, g, t, j] = R_t W_q[g E + S_j] x_t,   q_shared[b, t] = R_t W_q[N] x_t,
  k[b, h, t] = R_t W_k[h] x_t,                       v[b, h, t] = W_v[h] x_t,
with the kept sets S fixed and R_t the rotary embedding at position t (identity when rope_base is 0; the
pages give no positional encoding, so its form is the reading stated with oracle.rope).  Given the gradients
of those outputs, it returns the gradients of the loss L = sum(dq * q) + sum(dk * k) + sum(dv * v) with
respect to x and the three weights, by float64 autograd of that definition.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    return a.detach().to("cpu", torch.float64)


def rotate(rows, pos, base):
    """Rotary embedding of rows [..., n, d] at positions pos [n] (torch float64, differentiable): pair
    (c, c + d/2) turned by pos * base^(-2c/d)."""
    d = rows.shape[-1]
    h = d // 2
    freq = torch.tensor(base, dtype=torch.float64) ** (-2.0 * torch.arange(h, dtype=torch.float64) / d)
    ang = pos.to(torch.float64)[:, None] * freq[None, :]
    cs, sn = torch.cos(ang), torch.sin(ang)
    u, w = rows[..., :h], rows[..., h:]
    return torch.cat([u * cs - w * sn, w * cs + u * sn], dim=-1)


def qkv_proj_backward(w, x, w_q, w_k, w_v, sel, dq_routed, dq_shared, dk=None, dv=None, positions=None,
                      rope_base=0.0):
    """w: the workload (B, T, G = H_kv, E, k, d_head, n_shared); x [B*T, d_model]; w_q [N + n_shared, d, d_model];
    w_k, w_v [H_kv, d, d_model]; sel [B*T, G, k]; dq_routed [B, G, T*k, d]; dq_shared [B, T, d]; dk, dv
    [B, H_kv, T, d] or None; positions [B*T] or None (t).  Returns float64 numpy dict dw_q, dw_k, dw_v (None
    without dk), dx."""
    B, T, G, E, k, D = w.B, w.T, w.G, w.E, w.k, w.d_head
    N = G * E
    X = _f64(x).reshape(B * T, -1).requires_grad_(True)
    Wq = _f64(w_q).requires_grad_(True)
    has_kv = dk is not None
    Wk = _f64(w_k).requires_grad_(True) if has_kv else None
    Wv = _f64(w_v).requires_grad_(True) if has_kv else None
    sel_t = torch.as_tensor(np.asarray(sel), dtype=torch.long).reshape(B * T, G, k)
    pos = torch.as_tensor(np.asarray(positions) if positions is not None else np.arange(B * T) % T, dtype=torch.long)
    rope = rope_base > 0

    q_all = torch.einsum("tm,ndm->tnd", X, Wq)                  # every head of every token
    expert = torch.arange(G)[None, :, None] * E + sel_t          # [BT, G, k] global expert index
    q_r = q_all[torch.arange(B * T)[:, None, None], expert]      # [BT, G, k, D]
    if rope:
        q_r = rotate(q_r.reshape(B * T, G * k, D).transpose(0, 1), pos, rope_base).transpose(0, 1)
        q_r = q_r.reshape(B * T, G, k, D)
    dqr = _f64(dq_routed).reshape(B, G, T, k, D).permute(0, 2, 1, 3, 4).reshape(B * T, G, k, D)
    loss = (q_r * dqr).sum()
    if w.n_shared:
        q_s = q_all[:, N]
        if rope:
            q_s = rotate(q_s, pos, rope_base)
        loss = loss + (q_s * _f64(dq_shared).reshape(B * T, D)).sum()
    if has_kv:
        Hk = Wk.shape[0]
        kk = torch.einsum("tm,hdm->htd", X, Wk)                   # [H, BT, D]
        if rope:
            kk = rotate(kk, pos, rope_base)
        vv = torch.einsum("tm,hdm->htd", X, Wv)
        dk_t = _f64(dk).reshape(B, Hk, T, D).permute(1, 0, 2, 3).reshape(Hk, B * T, D)
        dv_t = _f64(dv).reshape(B, Hk, T, D).permute(1, 0, 2, 3).reshape(Hk, B * T, D)
        loss = loss + (kk * dk_t).sum() + (vv * dv_t).sum()
    loss.backward()
    return dict(dw_q=Wq.grad.numpy(), dw_k=Wk.grad.numpy() if has_kv else None,
                dw_v=Wv.grad.numpy() if has_kv else None, dx=X.grad.numpy())
