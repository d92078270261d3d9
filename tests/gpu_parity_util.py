"""Helpers for the GPU-vs-oracle parity tests.

Comparison rules:
  * routing (sel) is bit-exact except where the oracle flags a tie (the k-th
    and (k+1)-th logits closer than 1e-6); there the GPU's choice is accepted
    and substituted into the oracle's later steps;
  * compaction (counts, offsets, rows) is bit-exact given the agreed selection;
  * p~ within 1e-6; router logits within 5e-7 of the fp64 oracle;
  * bf16 attention outputs: max-abs <= 2e-2 and mean-abs <= 2e-3 over all
    slots; fp32: max-abs <= 1e-5 * max|ref| and mean-abs <= 1e-6 * max|ref|;
  * bf16 query projections: |d| <= 2^-8 |ref| + 1e-4 (bf16 rounding of an fp32
    accumulator); fp32: |d| <= 1e-5 * max|ref|.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_routed_query_amd.gqe as G
import workloads as W

TIE_MARGIN = 1e-6
LOGIT_TOL = 5e-7
PT_TOL = 1e-6
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX_REL, F32_MEAN_REL = 1e-5, 1e-6


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp: dict, dev) -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_prefill(w: W.Workload, inp: dict, dev="cuda") -> dict:
    d = G.desc_from(w)
    di = to_dev(inp, dev)
    res = G.prefill(d, di["x"].reshape(-1, w.d_model), di["w_router"], di["b_router"], di["w_q"], di["k"], di["v"],
                    logits=True)
    torch.cuda.synchronize()
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}


def agreed_routing(w: W.Workload, orc: dict, gpu_sel: np.ndarray):
    """Oracle selection with the GPU's choice substituted where the oracle flags a tie."""
    osel = orc["sel"]
    mism = (gpu_sel != osel).any(-1)
    bad = mism & ~orc["tie"]
    assert not bad.any(), f"{int(bad.sum())} routing mismatches outside the tie margin"
    sel = osel.copy()
    pt = orc["ptilde"].copy()
    if mism.any():
        sel[mism] = gpu_sel[mism]
        probs = orc["probs"].reshape(-1, w.G, w.E)
        p = np.take_along_axis(probs, sel.astype(np.int64), -1)
        # route mode 3 keeps the group softmax of the kept experts; the others renormalise it
        pt[mism] = (p if w.route_mode == 3 else p / p.sum(-1, keepdims=True))[mism]
    return sel, pt, int(mism.sum())


def check_route(w: W.Workload, inp: dict, gpu: dict) -> dict:
    d = oracle.desc(w)
    orc = oracle.route(d, inp["x"], inp["w_router"], inp["b_router"])
    gsel = gpu["sel"].numpy()
    sel, pt, n_sub = agreed_routing(w, orc, gsel)
    dlog = float(np.abs(gpu["logits"].numpy() - orc["logits"]).max()) if gpu.get("logits") is not None else 0.0
    dpt = float(np.abs(gpu["p_tilde"].numpy().astype(np.float64) - pt).max()) if pt.size else 0.0
    say(f"[{w.name}] route: tie-substituted={n_sub} ties={int(orc['tie'].sum())} max|dlogit|={dlog:.3e} "
        f"max|dp~|={dpt:.3e}")
    assert dlog < LOGIT_TOL
    assert dpt <= PT_TOL
    c = oracle.compact(d, sel)
    assert np.array_equal(gpu["counts"].numpy(), c["counts"]), "expert counts differ"
    assert np.array_equal(gpu["offsets"].numpy(), c["offsets"]), "expert offsets differ"
    assert np.array_equal(gpu["rows"].numpy(), c["rows"]), "compacted rows differ"
    return dict(sel=sel, ptilde=pt, counts=c["counts"])


def check_qproj(w: W.Workload, inp: dict, gpu: dict, agreed: dict, tok: np.ndarray):
    d = oracle.desc(w)
    qr, qs = oracle.qproj_rows(d, inp["x"], inp["w_q"], agreed["sel"], tok)
    b, t = tok // w.T, tok % w.T
    g_qr = gpu["q_routed"].double().numpy()[b, :, t]            # [n, G, k, dh]
    checks = [(g_qr, qr)]
    if w.n_shared:
        checks.append((gpu["q_shared"].double().numpy()[b, t], qs))
    for got, ref in checks:
        err = np.abs(got - ref)
        if w.dtype == "bf16":
            lim = 2.0 ** -8 * np.abs(ref) + 1e-4
        else:
            lim = F32_MAX_REL * max(1e-30, np.abs(ref).max())
        assert (err <= lim).all(), f"q projection off by {err.max():.3e}"
    say(f"[{w.name}] qproj: {len(tok)} tokens ok")


def check_out(w: W.Workload, got: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(got.astype(np.float64) - ref)
    mx, mean, ref_max = float(err.max()), float(err.mean()), float(np.abs(ref).max())
    say(f"[{w.name}] {what}: max-abs={mx:.3e} mean-abs={mean:.3e} max|ref|={ref_max:.3e} finite={np.isfinite(got).all()}")
    assert np.isfinite(got).all()
    if w.dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN
    else:
        assert mx <= F32_MAX_REL * ref_max and mean <= F32_MEAN_REL * ref_max


def check_prefill(w: W.Workload, inp: dict, gpu: dict, agreed: dict, tok: np.ndarray):
    d = oracle.desc(w)
    ref = oracle.prefill_rows(d, inp["x"], inp["w_q"], inp["k"], inp["v"], agreed["sel"], agreed["ptilde"], tok)
    got = gpu["out"].reshape(w.B * w.T, -1, w.d_head).numpy()[tok]
    check_out(w, got, ref, f"prefill out ({len(tok)} tokens)")


def check_prefill_given_q(w: W.Workload, inp: dict, gpu: dict, agreed: dict, tok: np.ndarray):
    """Attention and slots against the oracle's attention of the query rows the GPU's projection returned
    (their bf16 values taken exactly), so that only the attention's own arithmetic is compared: the
    kernel multiplies those rows unchanged and applies the scale 1/sqrt(d) in fp32 to the scores."""
    d = oracle.desc(w)
    b, t = tok // w.T, tok % w.T
    qr = gpu["q_routed"][b, :, t].double().numpy()                     # [n, G, k, dh]
    qs = gpu["q_shared"][b, t].double().numpy() if w.n_shared else None
    ref = oracle.attend_rows(d, qr, qs, inp["k"], inp["v"], agreed["ptilde"], tok)
    got = gpu["out"].reshape(w.B * w.T, -1, w.d_head).numpy()[tok]
    check_out(w, got, ref, f"prefill out given the GPU's queries ({len(tok)} tokens)")


def full_prefill_check(w: W.Workload, n_sample: int = 0):
    say(f"case {w}")
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    agreed = check_route(w, inp, gpu)
    tok = W.stratified_rows(w, n_sample).numpy() if n_sample else np.arange(w.B * w.T)
    check_qproj(w, inp, gpu, agreed, tok)
    check_prefill(w, inp, gpu, agreed, tok)
    return inp, gpu, agreed


def gpu_decode(w: W.Workload, inp: dict, dev="cuda") -> dict:
    d = G.desc_from(w)
    di = to_dev(inp, dev)
    res = G.decode(d, di["x"].reshape(w.B, w.d_model), di["w_router"], di["b_router"], di["w_q"], di["k_cache"],
                   di["v_cache"], di["lens"])
    torch.cuda.synchronize()
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}


def full_decode_check(w: W.Workload, inp: dict | None = None):
    say(f"case {w}")
    inp = inp if inp is not None else W.make_inputs(w)
    gpu = gpu_decode(w, inp)
    d = oracle.desc(w)
    orc = oracle.decode(d, inp["x"], inp["w_router"], inp["b_router"], inp["w_q"], inp["k_cache"], inp["v_cache"],
                        inp["lens"])
    gsel = gpu["sel"].numpy()
    mism = (gsel != orc["sel"]).any(-1)
    assert not (mism & ~orc["tie"]).any(), "decode routing differs outside the tie margin"
    ref = orc["out"]
    if mism.any():
        # at a flagged tie the GPU's choice is accepted: the oracle attends with the agreed selection
        sel, pt = orc["sel"].copy(), orc["ptilde"].copy()
        sel[mism] = gsel[mism]
        probs = oracle.route(d, inp["x"].reshape(w.B, w.d_model), inp["w_router"], inp["b_router"])["probs"]
        p = np.take_along_axis(probs.reshape(w.B, w.G, w.E), sel.astype(np.int64), -1)
        pt[mism] = (p if w.route_mode == 3 else p / p.sum(-1, keepdims=True))[mism]
        ref = oracle.decode(d, inp["x"], inp["w_router"], inp["b_router"], inp["w_q"], inp["k_cache"],
                            inp["v_cache"], inp["lens"], routing=dict(sel=sel, ptilde=pt))["out"]
    say(f"[{w.name}] decode: tie-substituted={int(mism.sum())}")
    check_out(w, gpu["out"].numpy(), ref, f"decode out ({w.B} sequences)")
    return inp, gpu


def gpu_out_proj(w: W.Workload, out_slots: torch.Tensor, p_tilde: torch.Tensor, w_o: torch.Tensor,
                 write_weighted: bool = True, dev="cuda", packed: bool = False):
    """gqe_out_proj (packed: gqe_out_proj_pack, then gqe_out_proj_packed) on the given slots [B*T, S, d_head]
    with the weighted slot(s) set to NaN first, so that a read of them would show in y.  Returns (y, slots
    after the call) on the CPU."""
    d = G.desc_from(w)
    kG, nr = w.k * w.G, (1, w.G, 0, 0)[w.route_mode]
    o = out_slots.reshape(w.B * w.T, d.S, w.d_head).clone()
    o[:, kG:kG + nr] = float("nan")
    od = o.to(dev)
    wd = w_o.to(dev)
    wp = G.out_proj_pack(d, wd) if packed else None
    y = G.out_proj(d, od, p_tilde.reshape(w.B * w.T, w.G, w.k).to(dev), wd, write_weighted=write_weighted,
                   w_packed=wp)
    torch.cuda.synchronize()
    return y.cpu(), od.cpu()


def check_out_proj(w: W.Workload, slots: torch.Tensor, p_tilde: torch.Tensor, w_o: torch.Tensor,
                   y: torch.Tensor, tok: np.ndarray):
    """y of tokens ``tok`` against the oracle's projection of the same hard and shared slots (its own
    fp64 weighted sum), element by element within the bound the arithmetic gives: bf16 rounding of each
    slot value (relative 2^-8: bf16 keeps 8 significand bits), fp32 accumulation over the K = S*d_head terms and the fp32 weighted sum
    (K + kG + 1 roundings of 2^-24), each relative to sum_i |h_i| |W_o[c, i]|."""
    d = oracle.desc(w)
    S = oracle.num_slots(d)
    h_gpu = slots.reshape(-1, S, w.d_head)[tok].double().numpy()
    pt = p_tilde.reshape(-1, w.G, w.k)[tok].double().numpy()
    if w.route_mode == 3:
        # no weighted slot to form: the slots (scaled hard slots, as gqe_attn_prefill leaves them) are projected
        h, h_abs = h_gpu, np.abs(h_gpu)
    else:
        h = oracle.assemble_rows(d, h_gpu, pt)
        h_abs = oracle.assemble_rows(d, np.abs(h_gpu), pt)    # weighted part: sum p~ |hard| bounds its error too
    y_ref = oracle.out_proj_rows(d, h, w_o)
    mag = h_abs.reshape(len(tok), -1) @ np.abs(w_o.double().numpy()).T
    K = S * w.d_head
    eps = (2.0 ** -8 if w.dtype == "bf16" else 0.0) + (K + w.k * w.G + 1) * 2.0 ** -24
    got = y.reshape(-1, w.d_model)[tok].double().numpy()
    err = np.abs(got - y_ref)
    ratio = float((err / (eps * mag + 1e-30)).max())
    say(f"[{w.name}] out_proj ({len(tok)} tokens): max-abs={err.max():.3e} mean-abs={err.mean():.3e} "
        f"max|ref|={np.abs(y_ref).max():.3e} max err/bound={ratio:.3f}")
    assert np.isfinite(got).all()
    assert ratio <= 1.0
