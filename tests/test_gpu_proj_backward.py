"""GPU parity of the projections' backward (gqe_qkv_proj_backward) against the fp64 autograd oracle
(oracle/proj_backward.py, itself pinned to finite differences of the C oracle's projections).

Both sides take the GPU's own routing (the backward holds the kept sets fixed) and the same seeded
gradients of q, K and V.  The GPU rounds each incoming gradient to bf16 (relative 2^-8; x and the weights
are exact bf16) and accumulates K products in fp32, so every element is held to
(2^-8 + (K + 2) 2^-24) times the sum of the absolute values of its terms (with the rotation's pair mixing
counted by taking |u| + |w| for both members of a pair), plus 1e-30.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_parity_util import say
from oracle.proj_backward import qkv_proj_backward
import sparse_routed_query_amd.gqe as G

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="pb_small", B=2, T=300, d_model=128, H_q=8, H_kv=2, k=2, d_head=64, dtype="bf16", seed=31,
                act_std=1.0, w_std=0.02)
    base.update(kw)
    return W.Workload(**base)


def pair_abs(a):
    """|u| + |w| on both members of every rotation pair (last axis)."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    h = a.shape[-1] // 2
    s = a[..., :h] + a[..., h:]
    return np.concatenate([s, s], axis=-1)


def run_case(w, rope_base=0.0, given_pos=False, with_kv=True, seed=5, use_workspace=True):
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(-1, w.d_model).to(dev)
    r = G.route(d, x, inp["w_router"].to(dev), inp["b_router"].to(dev) if inp["b_router"] is not None else None)
    gen = torch.Generator().manual_seed(seed)
    B, T, Gk, D = w.B, w.T, w.G, w.d_head
    dqr = torch.randn((B, Gk, T * w.k, D), generator=gen)
    dqs = torch.randn((B, T, D), generator=gen)
    dk = torch.randn((B, Gk, T, D), generator=gen) if with_kv else None
    dv = torch.randn((B, Gk, T, D), generator=gen) if with_kv else None
    pos = torch.randint(0, 40000, (B * T,), dtype=torch.int32, generator=gen) if given_pos else None
    tod = lambda t: t.to(dev) if t is not None else None  # noqa: E731
    out = G.qkv_proj_backward(d, x, inp["w_q"].to(dev), wk.to(dev), wv.to(dev), r, tod(dqr), tod(dqs), tod(dk), tod(dv),
                              tod(pos), rope_base, use_workspace)
    torch.cuda.synchronize()
    sel = r["sel"].cpu().numpy()
    xn, wq = inp["x"].reshape(B * T, -1).double().numpy(), inp["w_q"].double().numpy()
    wkn, wvn = wk.double().numpy(), wv.double().numpy()
    posn = pos.numpy() if given_pos else None
    n = lambda t: t.numpy() if t is not None else None  # noqa: E731
    ref = qkv_proj_backward(w, xn, wq, wkn, wvn, sel, n(dqr), n(dqs), n(dk), n(dv), posn, rope_base)
    mag = qkv_proj_backward(w, np.abs(xn), np.abs(wq), np.abs(wkn), np.abs(wvn), sel, pair_abs(n(dqr)),
                            pair_abs(n(dqs)), pair_abs(n(dk)) if with_kv else None, np.abs(n(dv)) if with_kv else None,
                            posn, 0.0)
    counts = r["counts"].cpu().numpy()
    n_dx = (w.k * w.G + w.n_shared + (2 * w.G if with_kv else 0)) * D
    for name in ("dw_q", "dw_k", "dw_v", "dx"):
        if ref[name] is None:
            assert out[name] is None
            continue
        got = out[name].cpu().double().numpy()
        if name == "dw_q":
            K = np.concatenate([counts, [B * T] * w.n_shared]).reshape(-1, 1, 1)
        elif name == "dx":
            K = n_dx
        else:
            K = B * T
        bound = (2.0 ** -8 + (K + 2) * 2.0 ** -24) * mag[name] + 1e-30
        err = np.abs(got - ref[name])
        ratio = float((err / bound).max())
        rel = float(np.linalg.norm(got - ref[name]) / max(np.linalg.norm(ref[name]), 1e-30))
        say(f"[{w.name}] {name}: max-abs={err.max():.3e} max err/bound={ratio:.3f} rel rms={rel:.2e} "
            f"finite={np.isfinite(got).all()}")
        assert np.isfinite(got).all()
        assert ratio <= 1.0


CASES = [
    (small(), 0.0, False, True),
    (small(name="rope_t"), 10000.0, False, True),
    (small(name="rope_pos", d_head=32), 10000.0, True, True),
    (small(name="d128_rope", d_head=128, k=1), 500000.0, True, True),
    (small(name="zipf_no_kv", H_q=16, H_kv=4, zipf_s=1.2), 0.0, False, False),
    (small(name="no_shared_ragged_cols", n_shared=0, d_model=320), 10000.0, False, True),
    (small(name="kE", H_q=8, H_kv=4, k=2, T=129), 0.0, False, True),
    (small(name="main_shape_quarter", B=1, T=4096, d_model=1024, H_q=16, H_kv=8, k=1, seed=1), 10000.0, False, True),
]


@pytest.mark.parametrize("w,base,given,kv", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_projection_backward(w, base, given, kv):
    run_case(w, base, given, kv)


@pytest.mark.parametrize("w", [small(name="one_chunk"), small(name="one_chunk_d128", d_head=128, k=1)],
                         ids=lambda w: w.name)
def test_projection_backward_without_workspace(w):
    """Without a workspace the weight gradient sums each head's rows in one chunk: the same bound holds."""
    run_case(w, 10000.0, True, True, use_workspace=False)


def test_projection_backward_is_deterministic():
    w = small(name="det")
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    d = G.desc_from(w)
    x = inp["x"].reshape(-1, w.d_model).cuda()
    r = G.route(d, x, inp["w_router"].cuda())
    gen = torch.Generator().manual_seed(2)
    dqr = torch.randn((w.B, w.G, w.T * w.k, w.d_head), generator=gen).cuda()
    dqs = torch.randn((w.B, w.T, w.d_head), generator=gen).cuda()
    dk = torch.randn((w.B, w.G, w.T, w.d_head), generator=gen).cuda()
    dv = torch.randn((w.B, w.G, w.T, w.d_head), generator=gen).cuda()
    a = G.qkv_proj_backward(d, x, inp["w_q"].cuda(), wk.cuda(), wv.cuda(), r, dqr, dqs, dk, dv, None, 10000.0)
    b = G.qkv_proj_backward(d, x, inp["w_q"].cuda(), wk.cuda(), wv.cuda(), r, dqr, dqs, dk, dv, None, 10000.0)
    torch.cuda.synchronize()
    for name in ("dw_q", "dw_k", "dw_v", "dx"):
        assert torch.equal(a[name], b[name]), name
