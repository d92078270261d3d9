"""CPU ORACLE for the backward pass through slot assembly and routing.  TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the HIP library never does, and the two share no code.

What it differentiates (GQE study note, dimensionstp.github.io, §3-2 (2) and (4)): for every token t and
group g, router scores s = W_router x_t + b, p = softmax over the group's E experts, the kept set S_{t,g}
(given: a discrete choice, held fixed), p~_j = p_{S_j} / sum_i p_{S_i}, and the output slots

    hard slots   h_{g,j} = o_{t,g,S_j}                      (given attention outputs, the leaves)
    route_mode 0 w       = sum_g sum_j p~_{g,j} h_{g,j}     (one weighted slot)
    route_mode 1 w_g     = sum_j p~_{g,j} h_{g,j}           (one per group)
    route_mode 2         no weighted slot
    shared slot          passes through (not differentiated here)

The study note's point about the weighted slot is that it is the router's differentiable learning path: the
hard slots alone carry no gradient back to p~.  Given an upstream gradient dout of every slot, this module
returns the gradients of L = sum(dout * slots) with respect to the hard slots, the router scores, W_router,
b_router and x (through the router only), by autograd of that definition in float64.
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


def route_assemble_backward(w, x, w_router, b_router, sel, hard, dout):
    """w: a workload (B, T, d_model, H_q, H_kv, k, d_head, n_shared, route_mode).

    x [B*T, d_model], w_router [N, d_model], b_router [N] or None, sel [B*T, G, k] (ascending expert
    index), hard [B*T, G*k, d_head] the hard slots, dout [B*T, S, d_head] the upstream gradient.
    Returns dict of float64 numpy arrays: d_hard [B*T, G*k, d_head], d_logits [B*T, N],
    dw_router [N, d_model], db_router [N], dx [B*T, d_model].
    """
    G, k, E, dh = w.H_kv, w.k, w.H_q // w.H_kv, w.d_head
    BT = w.B * w.T
    xs = _f64(x).reshape(BT, w.d_model).requires_grad_(True)
    wr = _f64(w_router).requires_grad_(True)
    br = (_f64(b_router) if b_router is not None else torch.zeros(G * E, dtype=torch.float64)).requires_grad_(True)
    hd = _f64(hard).reshape(BT, G * k, dh).requires_grad_(True)
    go = _f64(dout).reshape(BT, -1, dh)
    s_idx = torch.as_tensor(np.asarray(sel), dtype=torch.int64).reshape(BT, G, k)

    logits = xs @ wr.T + br                                    # [BT, N]   §3-2 (2) router
    logits.retain_grad()
    p = torch.softmax(logits.reshape(BT, G, E), dim=-1)        # softmax over the group's experts
    q = torch.gather(p, 2, s_idx)                              # probabilities of the kept experts
    pt = q / q.sum(-1, keepdim=True)                           # §3-2 (4) renormalised over the kept k
    hard_g = hd.reshape(BT, G, k, dh)
    kG = G * k
    loss = (go[:, :kG] * hd).sum()
    if w.route_mode == 0:
        wsum = (pt[..., None] * hard_g).sum(dim=(1, 2))        # [BT, dh]
        loss = loss + (go[:, kG] * wsum).sum()
    elif w.route_mode == 1:
        wg = (pt[..., None] * hard_g).sum(dim=2)               # [BT, G, dh]
        loss = loss + (go[:, kG:kG + G] * wg).sum()
    loss.backward()

    def grad(t):   # route mode 2 leaves the router without a path to the loss: zero gradient
        return (t.grad if t.grad is not None else torch.zeros_like(t)).detach().numpy()

    return dict(d_hard=grad(hd), d_logits=grad(logits), dw_router=grad(wr), db_router=grad(br), dx=grad(xs))


__all__ = ["route_assemble_backward"]
