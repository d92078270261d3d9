"""GPU parity of the attention backward (gqe_attn_backward) against the fp64 oracle (oracle/attn_backward.py).

Both sides take the GPU forward's own query rows (bf16, as the projection wrote them), K and V, and the same
seeded slot gradients.  The GPU rounds dO, P and dS to bf16 for its matrix products (8 significand bits: a
relative error of at most 2^-8 each) and accumulates in fp32; it also takes Delta = <dO, O> from the forward's
output O rather than recomputing it.  Every term of a gradient therefore carries at most about three such
roundings, and each element is held to c = 2^-6 times the sum of the absolute values of its terms, with the
terms that cancel inside dS = P o (dP - Delta) counted at their own size:
  A      = P o (|dO| |V|^T + sum_d |dO| |O|)
  dq     : c (A |K|) / sqrt(d)        dK : c (A^T |q|) / sqrt(d)        dV : c (P^T |dO|)
(a result that cancels to zero -- with one key dq = 0 exactly -- is judged on the scale of what cancelled).
The normalised errors max|err|/max|ref| and the relative rms are printed as well.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_parity_util import gpu_prefill, say
from oracle.attn_backward import head_backward, row_lse2
import sparse_routed_query_amd.gqe as G

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="ab_small", B=2, T=300, d_model=128, H_q=8, H_kv=2, k=2, d_head=64, dtype="bf16", seed=41,
                act_std=1.0, w_std=0.05)
    base.update(kw)
    return W.Workload(**base)


C = 2.0 ** -6


def check(name, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), name
    err = np.abs(got - ref)
    r = float((err / (bound + 1e-30)).max())
    emax = err.max() / max(np.abs(ref).max(), 1e-30)
    erms = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {name}: max err/bound {r:.3f}  max-err/max-ref {emax:.2e}  rms {erms:.2e}")
    assert r <= 1.0, name


def forward_lse(w, inp, gpu, split=True):
    """gqe_attn_prefill_heads_lse on the forward's own queries: checks that its slots are gqe_attn_prefill_heads'
    bit for bit (same workspace choice) and returns the row statistics (device tensor)."""
    d = G.desc_from(w)
    qr = gpu["q_routed"].cuda()
    qs = gpu["q_shared"].cuda() if w.n_shared else None
    k, v = inp["k"].cuda(), inp["v"].cuda()
    shape = (w.B * w.T, d.S, w.d_head)
    out_a = torch.full(shape, float("nan"), device="cuda")
    out_b = out_a.clone()
    lse = torch.full((G.lse_rows(d),), float("nan"), device="cuda")
    nws = G.gqe_attn_prefill_workspace_bytes(d) if split else 0
    ws = torch.zeros(max(nws, 256), dtype=torch.uint8, device="cuda") if nws else None
    G.gqe_attn_prefill_heads(d, qr, qs, k, v, out_a, ws)
    G.gqe_attn_prefill_heads_lse(d, qr, qs, k, v, out_b, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(out_a, nan=0.0), torch.nan_to_num(out_b, nan=0.0))
    return lse


def check_lse(w, inp, gpu, lse, heads):
    """The forward's row statistics against the oracle's (base-2 log of each row's softmax denominator): the
    GPU forms the scores in fp32 from the bf16 rows, so 2e-4 absolute."""
    B, T, Gn, k = w.B, w.T, w.H_kv, w.k
    got = lse.cpu().double().numpy()
    nr = B * Gn * T * k
    Kf = inp["k"].double().numpy()
    worst = 0.0
    for b, h in heads:
        if h < Gn:
            q = gpu["q_routed"].double().numpy().reshape(B, Gn, T * k, -1)[b, h]
            ref = row_lse2(q, Kf[b, h], k, w.causal)
            g = got[(b * Gn + h) * T * k:(b * Gn + h + 1) * T * k]
        else:
            q = gpu["q_shared"].double().numpy().reshape(B, T, -1)[b]
            ref = row_lse2(q, Kf[b, 0], 1, w.causal)
            g = got[nr + b * T:nr + (b + 1) * T]
        assert np.isfinite(g).all()
        worst = max(worst, float(np.abs(g - ref).max()))
    say(f"[{w.name}] forward row statistics: max-abs error {worst:.2e} over {len(heads)} heads")
    assert worst <= 2e-4


def run_case(w, heads=None, use_lse=False):
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    B, T, Gn, k, D = w.B, w.T, w.H_kv, w.k, w.d_head
    BT, S, kG = B * T, d.S, k * Gn
    rng = np.random.default_rng(w.seed + 17)
    d_hard = torch.from_numpy(rng.standard_normal((BT, kG, D)).astype(np.float32))
    dout = torch.from_numpy(rng.standard_normal((BT, S, D)).astype(np.float32))
    qs = gpu["q_shared"] if w.n_shared else None
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Gn + (1 if w.n_shared else 0))]
    lse = None
    if use_lse:
        lse = forward_lse(w, inp, gpu)
        check_lse(w, inp, gpu, lse, heads)
    say(f"[{w.name}] attention backward (B={B}, T={T}, G={Gn}, k={k}, d={D}, causal={w.causal}, "
        f"forward statistics given={use_lse})")
    res = G.attn_backward(d, gpu["q_routed"].cuda(), qs.cuda() if qs is not None else None, inp["k"].cuda(),
                          inp["v"].cuda(), gpu["out"].reshape(BT, S, D).cuda(), d_hard.cuda(), dout.cuda(), lse=lse)
    torch.cuda.synchronize()
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in res.items()}
    Kf, Vf = inp["k"].double().numpy(), inp["v"].double().numpy()
    qr = gpu["q_routed"].double().numpy().reshape(B, Gn, T * k, D)
    out = gpu["out"].double().numpy().reshape(B, T, S, D)
    dh, do = d_hard.double().numpy().reshape(B, T, kG, D), dout.double().numpy().reshape(B, T, S, D)
    kv = {}   # (b, g) -> [dk_ref, dv_ref, dk_bound, dv_bound, readers seen]
    for b, h in heads:
        if h < Gn:   # row t*k + j: hard slot h*k + j of token t
            q, kvh, kk = qr[b, h], h, k
            dO = dh[b, :, h * k:(h + 1) * k].reshape(T * k, D)
            O = out[b, :, h * k:(h + 1) * k].reshape(T * k, D)
        else:
            q, kvh, kk = qs.double().numpy().reshape(B, T, D)[b], 0, 1
            dO, O = do[b, :, S - 1], out[b, :, S - 1]
        r = head_backward(q, Kf[b, kvh], Vf[b, kvh], dO, kk, w.causal)
        P = r["P"]
        A = P * (np.abs(dO) @ np.abs(Vf[b, kvh]).T + (np.abs(dO) * np.abs(O)).sum(-1, keepdims=True))
        bq = C * (A @ np.abs(Kf[b, kvh])) / np.sqrt(D)
        got = res["dq_routed"][b, h] if h < Gn else res["dq_shared"][b]
        check(f"dq[{b},{h}]", got, r["dq"], bq)
        e = kv.setdefault((b, kvh), [0.0, 0.0, 0.0, 0.0, 0])
        e[0] = e[0] + r["dk"]
        e[1] = e[1] + r["dv"]
        e[2] = e[2] + C * (A.T @ np.abs(q)) / np.sqrt(D)
        e[3] = e[3] + C * (P.T @ np.abs(dO))
        e[4] += 1
    for (b, g), (dk, dv, bk, bv, n) in kv.items():
        if n == 1 + (1 if (g == 0 and w.n_shared) else 0):   # every head reading this KV head was computed
            check(f"dk[{b},{g}]", res["dk"][b, g], dk, bk)
            check(f"dv[{b},{g}]", res["dv"][b, g], dv, bv)
    return res


@pytest.mark.parametrize("w", [
    small(), small(causal=0, name="noncausal"), small(n_shared=0, name="no_shared"),
    small(d_head=32, name="d32"), small(d_head=128, name="d128"), small(H_q=16, H_kv=4, k=3, name="E4k3"),
    small(k=1, name="top1", T=129), small(B=1, T=1, name="T1"), small(B=1, T=65, name="T65"),
    small(route_mode=1, name="per_group", T=200), small(route_mode=2, name="hard_only", T=200),
], ids=lambda w: w.name)
def test_attention_backward(w):
    run_case(w)


@pytest.mark.parametrize("w", [
    small(), small(causal=0, name="noncausal"), small(n_shared=0, name="no_shared"),
    small(d_head=32, name="d32"), small(d_head=128, name="d128"), small(H_q=16, H_kv=4, k=3, name="E4k3"),
    small(B=1, T=1, name="T1"), small(B=1, T=2304, H_q=4, H_kv=1, k=1, name="split_tiles"),
], ids=lambda w: w.name)
def test_attention_backward_given_the_forward_statistics(w):
    """gqe_attn_prefill_heads_lse's row statistics against the oracle's, its slots equal to
    gqe_attn_prefill_heads', then gqe_attn_backward_lse against fp64 autograd at the same bounds."""
    run_case(w, use_lse=True)


def test_attention_backward_full_size_given_the_forward_statistics():
    w = W.WORKLOADS["main_250m"]
    run_case(w, heads=[(0, 0), (0, w.H_kv), (2, 5)], use_lse=True)


def test_backward_with_and_without_the_forward_statistics_agree():
    """The two entry points differ only by the rounding of the statistics (recomputed or the forward's)."""
    w = small(T=700, name="lse_vs_recompute")
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    BT, S, D = w.B * w.T, d.S, w.d_head
    g = torch.Generator().manual_seed(5)
    d_hard = torch.randn((BT, w.k * w.H_kv, D), generator=g).cuda()
    dout = torch.randn((BT, S, D), generator=g).cuda()
    lse = forward_lse(w, inp, gpu)
    args = (d, gpu["q_routed"].cuda(), gpu["q_shared"].cuda(), inp["k"].cuda(), inp["v"].cuda(),
            gpu["out"].reshape(BT, S, D).cuda(), d_hard, dout)
    a, b = G.attn_backward(*args), G.attn_backward(*args, lse=lse)
    torch.cuda.synchronize()
    for key in a:
        rel = float((a[key] - b[key]).norm() / a[key].norm())
        say(f"  {key}: relative rms difference {rel:.2e}")
        assert rel <= 1e-3, key


def test_attention_backward_full_size_sampled_heads():
    # main_250m: routed head (0, 0) and the shared head of batch 0 (the two readers of KV head 0), routed (3, 7)
    w = W.WORKLOADS["main_250m"]
    run_case(w, heads=[(0, 0), (0, w.H_kv), (3, w.H_kv - 1)])


def test_attention_backward_is_deterministic():
    w = small(T=400, name="det")
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    d = G.desc_from(w)
    BT, S, D = w.B * w.T, d.S, w.d_head
    g = torch.Generator().manual_seed(3)
    d_hard = torch.randn((BT, w.k * w.H_kv, D), generator=g).cuda()
    dout = torch.randn((BT, S, D), generator=g).cuda()
    args = (d, gpu["q_routed"].cuda(), gpu["q_shared"].cuda(), inp["k"].cuda(), inp["v"].cuda(),
            gpu["out"].reshape(BT, S, D).cuda(), d_hard, dout)
    a, b = G.attn_backward(*args), G.attn_backward(*args)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
