"""GPU parity of the backward through slot assembly and routing (gqe_route_backward).

The weighted slot is the router's differentiable learning path (GQE study note §3-2 (4)); the oracle
differentiates the definition by autograd in float64 (oracle/backward.py).  Both sides take the GPU's own
routing (sel, p~) and slots, and the same seeded upstream gradient.  All GPU arithmetic is fp32, so every
output is checked element by element against the rounding bound of the sums that form it, relative to
the sum of the absolute values of their terms (results that cancel to zero, as the score gradient does
when a group's kept experts produce equal outputs, are judged on the scale of what cancelled):
  d_hard    dout_h + p~ dout_w: 3 roundings, plus the GPU's fp32 p~ (2e-6 relative)
  d_logits  p~_j (dp~_j - sum_i p~_i dp~_i): the d_head-term dot products and the k-term sum, plus p~;
            experts that were not kept are exactly 0
  dw, db    sums over 256-token blocks, then the blocks added, plus the d_logits bounds carried through
  dx        N-term sums, plus the d_logits bounds carried through
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_parity_util import gpu_prefill, say
from oracle.backward import route_assemble_backward
import sparse_routed_query_amd.gqe as G

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def small(**kw):
    base = dict(name="rb_small", B=2, T=300, d_model=128, H_q=8, H_kv=2, k=2, d_head=64, dtype="bf16", seed=31,
                act_std=1.0, w_std=0.02)
    base.update(kw)
    return W.Workload(**base)


def check_bound(name, got, ref, bound):
    # (an absolute floor of 1e-10: the oracle's own float64 rounding, where the exact value is 0)
    err = np.abs(got - ref)
    r = float((err / (bound + 1e-10)).max())
    say(f"  {name}: max-abs={err.max():.3e} max err/bound={r:.3f}")
    assert np.isfinite(got).all() and r <= 1.0


def run_case(w):
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    BT, S, D, kG = w.B * w.T, d.S, w.d_head, w.k * w.G
    Gn, k, E = w.G, w.k, w.H_q // w.H_kv
    rng = np.random.default_rng(w.seed)
    dout = torch.from_numpy(rng.standard_normal((BT, S, D)).astype(np.float32))
    out = gpu["out"].reshape(BT, S, D)
    x = inp["x"].reshape(BT, w.d_model)
    res = G.route_backward(d, dout.cuda(), out.cuda(), gpu["sel"].cuda(), gpu["p_tilde"].cuda(), x.cuda(),
                           inp["w_router"].cuda())
    torch.cuda.synchronize()
    ref = route_assemble_backward(w, x, inp["w_router"], inp["b_router"], gpu["sel"].numpy(), out[:, :kG].numpy(),
                                  dout.numpy())
    say(f"[{w.name}] route backward ({BT} tokens)")
    dn, on = dout.double().numpy(), out.double().numpy()
    pt = gpu["p_tilde"].double().numpy().reshape(BT, Gn, k)
    sel = gpu["sel"].numpy().reshape(BT, Gn, k).astype(np.int64)
    if w.route_mode == 2:
        dw = np.zeros((BT, Gn, D))
    elif w.route_mode == 0:
        dw = np.repeat(dn[:, kG:kG + 1], Gn, axis=1)
    else:
        dw = dn[:, kG:kG + Gn]
    hard = on[:, :kG].reshape(BT, Gn, k, D)
    # d_hard = dout_h + p~ dout_w
    ptw = np.abs(pt[..., None] * dw[:, :, None, :])
    bound_h = 3 * U * (np.abs(dn[:, :kG]).reshape(BT, Gn, k, D) + ptw) + 2e-6 * ptw
    check_bound("d_hard", res["d_hard"].cpu().numpy(), ref["d_hard"], bound_h.reshape(BT, kG, D))
    # d_logits on the scale of p~_j (|dp~_j|_abs + sum_i p~_i |dp~_i|_abs)
    A = np.abs(hard * dw[:, :, None, :]).sum(-1)                       # [BT, G, k] absolute dot products
    scale = pt * (A + (pt * A).sum(-1, keepdims=True))
    dl_bound = np.zeros((BT, Gn, E))
    np.put_along_axis(dl_bound, sel, ((D + k + 8) * U + 2e-6) * scale, -1)
    dl_bound = dl_bound.reshape(BT, Gn * E)
    kept = np.zeros((BT, Gn, E), dtype=bool)
    np.put_along_axis(kept, sel, True, -1)
    got_dl = res["d_logits"].cpu().numpy()
    assert not got_dl[~kept.reshape(BT, -1)].any(), "experts that were not kept must get exactly 0"
    check_bound("d_logits", got_dl, ref["d_logits"], dl_bound)
    dl = np.abs(ref["d_logits"])
    xa = np.abs(x.double().numpy())
    eps = (256 + -(-BT // 256)) * U
    check_bound("dw_router", res["dw_router"].cpu().numpy(), ref["dw_router"], eps * (dl.T @ xa) + dl_bound.T @ xa)
    check_bound("db_router", res["db_router"].cpu().numpy(), ref["db_router"], eps * dl.sum(0) + dl_bound.sum(0))
    wa = np.abs(inp["w_router"].double().numpy())
    check_bound("dx", res["dx"].cpu().numpy(), ref["dx"], (w.H_q + 2) * U * (dl @ wa) + dl_bound @ wa)
    return res, ref


@pytest.mark.parametrize("w", [
    small(), small(route_mode=1, name="per_group"), small(route_mode=2, name="hard_only"),
    small(H_q=16, H_kv=4, k=3, zipf_s=1.2, name="E4k3_bias"), small(k=1, H_q=4, H_kv=2, name="top1"),
    small(d_head=32, name="d32"), small(d_head=128, name="d128"), small(dtype="f32", T=100, d_model=96, name="f32"),
    small(B=1, T=1, name="T1"), small(d_model=192, H_q=48, H_kv=4, k=3, name="N48_C192"),
    small(dtype="f32", T=50, d_model=100, H_q=48, H_kv=4, k=2, name="f32_N48"), small(d_head=32, H_q=32, H_kv=2, k=4, T=513, name="N32_d32"),
    W.WORKLOADS["main_250m"],
    W.WORKLOADS["main_250m"].replace(k=2, name="main_250m_k2"),   # full size with a router gradient
    W.WORKLOADS["wide_zipf"],   # full size: 32 experts (two MFMA row tiles), d_model 4096, k = 2, d_head 128
], ids=lambda w: f"{w.name}-{w.dtype}")
def test_route_backward(w):
    res, ref = run_case(w)
    if w.k == 1 or w.route_mode == 2:   # no learning signal reaches the router
        assert not res["d_logits"].any() and not res["dw_router"].any() and not res["dx"].any()


def test_route_backward_is_deterministic():
    w = small(T=700, name="det")
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    BT = w.B * w.T
    dout = torch.randn((BT, d.S, w.d_head), generator=torch.Generator().manual_seed(2)).cuda()
    args = (d, dout, gpu["out"].reshape(BT, d.S, w.d_head).cuda(), gpu["sel"].cuda(), gpu["p_tilde"].cuda(),
            inp["x"].reshape(BT, w.d_model).cuda(), inp["w_router"].cuda())
    a = G.route_backward(*args)
    b = G.route_backward(*args)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("w", [
    small(), small(H_q=16, H_kv=4, k=3, zipf_s=1.2, name="E4k3_bias"), small(H_q=64, H_kv=2, k=4, name="N64"),
    small(B=1, T=1, name="T1"), W.WORKLOADS["main_250m"], W.WORKLOADS["wide_zipf"],
], ids=lambda w: w.name)
def test_route_stats_importance(w):
    # per-expert importance (sum over tokens of the in-group softmax) from the GPU router's fp64 scores, against
    # the oracle end to end.  The router's scores are within 5e-7 of the oracle's, which moves each token's
    # probability by at most ~2.5e-7: the sums stay within 1e-6 BT, plus fp32 rounding of the result.
    import oracle
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    BT, Gn, E = w.B * w.T, w.H_kv, w.H_q // w.H_kv
    imp = G.route_stats(d, gpu["logits"].cuda()).cpu().double().numpy()
    od = oracle.desc(w)
    ref = oracle.expert_importance(od, oracle.route(od, inp["x"], inp["w_router"], inp["b_router"])["probs"])
    err = np.abs(imp - ref).max()
    say(f"[{w.name}] importance max err {err:.3e} (BT = {BT})")
    assert err <= 1e-6 * BT + 2.0 ** -24 * np.abs(ref).max()
    np.testing.assert_allclose(imp.reshape(Gn, E).sum(-1), BT, rtol=E * 2.0 ** -23)
    again = G.route_stats(d, gpu["logits"].cuda()).cpu().double().numpy()
    assert np.array_equal(imp, again)
