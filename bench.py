"""Benchmark of the GQE attention forward on one MI355X.

A step is one pass of the whole prefill path on the main 250M-scale layer
shape (B=4, T=4096, d_model=1024, H_q=16, H_kv=8, k=1, shared head,
d_head=64, bf16): router + compaction (gqe_route), routed and shared query
projection (gqe_qproj), causal attention (gqe_attn_prefill_heads) and slot
assembly (gqe_assemble) -- together the work of gqe_attn_prefill -- with
every input already resident in HBM.

Printed value: routed prefill throughput in TFLOP/s counted over active
heads only (attention FLOPs 4*d*B*H_act*T(T+1)/2 with H_act = k*G + 1,
divided by the whole step's time).  The same JSON line carries:
  roofline      the attention kernel alone (the one kernel of
                gqe_attn_prefill_heads) timed with HIP events on the stream it
                is launched on, against the bf16 MFMA peak;
  decode        the one-token decode step on the decode workload (B=64 cache
                lengths in [4096, 8192]): gqe_attn_decode timed alone, bytes of
                K/V it must read over its time, against the HBM peak; the step
                is that plus gqe_decode_route_qproj (routing and query
                projection in one launch);
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  long_context  T=32768 GQE vs all-active GQA on the same inputs, every call
                timed, attention and projection as fractions of the bf16 peak;
  wide_zipf     the wider expert pool with skewed routing (B=2, T=16384,
                d_model=4096, H_q=32, H_kv=8, k=2, d_head=128), the same;
  ceilings      a sustained dense bf16 MFMA loop with the clock it ran at,
                and a streaming HBM read: measured ceilings of this chip;
  out_proj      the next step after the path, outside the timed step: the
                output projection over the kG+2 slots fused with slot assembly
                (gqe_out_proj) on the step's own slots, against the bf16 peak;
  kv_proj       the step before it, also outside: the K and V projections
                (gqe_kv_proj) of the step's x, against the bf16 peak;
  route_backward  the backward through slot assembly and routing
                (gqe_route_backward) on the step's outputs, GB/s against HBM;
  attn_backward the attention backward (gqe_attn_backward) on the step's
                query rows and slots, TFLOP/s against the bf16 peak;
  proj_backward the projections' backward (gqe_qkv_proj_backward: dW_q,
                dW_k, dW_v, dx) on the step's routing, against the bf16 peak.

--graph also times the step replayed from one HIP graph of the four calls
(on this stack replaying is not faster than launching them one by one).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--graph] [--no-cpu] [--no-context] [--no-decode]
       python bench.py --only {step,prefill,prefill_wide,prefill_long,qproj,qproj_wide,outproj,decode,copy}
                       --steps K   (profiler runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "routed prefill TFLOP/s (active heads) + %MFMA peak; decode GB/s + %HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU needs ~30 ms of load to reach its steady clock")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-context", action="store_true", help="skip the long-context GQE vs dense leg")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--graph", action="store_true", help="also time the step replayed from one HIP graph")
    ap.add_argument("--only", choices=["step", "prefill", "outproj", "decode", "copy", "qproj", "prefill_wide",
                                       "qproj_wide", "prefill_long", "attn_bwd"], default=None,
                    help="run just one call --steps times (for profiler counter runs) and print nothing else")
    return ap.parse_args()


class Prefill:
    """Preallocated buffers and the C-ABI calls of one prefill step."""

    def __init__(self, w, inp, dev):
        import torch
        import sparse_routed_query_amd.gqe as G
        self.G, self.w = G, w
        self.d = G.desc_from(w)
        self.x = inp["x"].reshape(-1, w.d_model).to(dev)
        self.wr = inp["w_router"].to(dev)
        self.br = inp["b_router"].to(dev) if inp["b_router"] is not None else None
        self.wq = inp["w_q"].to(dev)
        self.k = inp["k"].to(dev)
        self.v = inp["v"].to(dev)
        self.r = G.alloc_route(self.d, dev)
        self.q = G.alloc_qproj(self.d, dev)
        self.out = torch.empty((w.B, w.T, self.d.S, w.d_head), dtype=torch.float32, device=dev)
        n_ws = G.gqe_attn_prefill_workspace_bytes(self.d)   # zeroed once; every call leaves it zeroed
        self.ws = torch.zeros(n_ws, dtype=torch.uint8, device=dev) if n_ws else None

    def route(self):
        r = self.r
        self.G.gqe_route(self.d, self.x, self.wr, self.br, r["sel"], r["p_tilde"], r["counts"], r["offsets"],
                         r["rows"], None, r["workspace"])

    def qproj(self):
        r, q = self.r, self.q
        self.G.gqe_qproj(self.d, self.x, self.wq, r["sel"], r["counts"], r["offsets"], r["rows"], q["q_routed"],
                         q["q_shared"])

    def attn(self):
        """Attention only (hard and shared slots): the dominant kernel."""
        self.G.gqe_attn_prefill_heads(self.d, self.q["q_routed"], self.q["q_shared"], self.k, self.v, self.out,
                                      self.ws)

    def assemble(self):
        self.G.gqe_assemble(self.d, self.r["p_tilde"], self.out)

    def step(self):
        self.route()
        self.qproj()
        self.attn()
        self.assemble()


def warm(fns, torch, ms=30.0, min_calls=3):
    """Run the calls until at least `ms` of wall time has passed: the first
    tens of milliseconds of load run at a lower clock than the steady state.
    Returns (rounds of the calls, milliseconds)."""
    t0 = time.perf_counter()
    i = 0
    while i < min_calls or (time.perf_counter() - t0) * 1e3 < ms:
        for fn in fns:
            fn()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i, (time.perf_counter() - t0) * 1e3


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def time_calls(fn_list, n, torch, queue_ahead=False):
    """Average ms per call of each function, timed with events on the current stream.  queue_ahead: a
    spin kernel of a few milliseconds goes first, so that the host enqueues every timed call while the
    GPU is still busy and the events time the calls back to back on the device, without the host's
    per-call issue time (which exceeds a small kernel's own)."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fn_list]
          for _ in range(n)]
    if queue_ahead:
        torch.cuda._sleep(int(4e5 * n * len(fn_list)))   # ~0.2 ms of spinning per call at ~2 GHz
    for i in range(n):
        for j, fn in enumerate(fn_list):
            ev[i][j][0].record()
            fn()
            ev[i][j][1].record()
    torch.cuda.synchronize()
    return [sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(n)) / n for j in range(len(fn_list))]


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_routed_query_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str):
    """HBM bytes per launch from committed PMC counters, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    e = data.get(kernel_key)
    if not e or e.get("source_hash") != source_hash(*e.get("source_files", [])):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, inp, target_s: float):
    """The oracle as it stands on a stratified sample of the workload's tokens: the attention and slots of
    those tokens (oracle.attend_rows) timed alone, over the same attention FLOPs as the GPU's figure; the
    routing and query projection of the sample run first, untimed, and their time is reported beside it."""
    import numpy as np
    import oracle
    import workloads as W
    d = oracle.desc(w)
    x = inp["x"].reshape(-1, w.d_model)

    def run(tok):
        t0 = time.perf_counter()
        r = oracle.route(d, x[tok], inp["w_router"], inp["b_router"])
        sel_full = np.zeros((w.B * w.T, w.G, w.k), dtype=np.int32)
        pt_full = np.zeros((w.B * w.T, w.G, w.k))
        sel_full[tok], pt_full[tok] = r["sel"], r["ptilde"]
        qr, qs = oracle.qproj_rows(d, inp["x"], inp["w_q"], sel_full, tok)
        t1 = time.perf_counter()
        oracle.attend_rows(d, qr, qs, inp["k"], inp["v"], pt_full[tok], tok)
        return time.perf_counter() - t1, t1 - t0

    def flops(tok):
        t = tok % w.T
        return float(np.sum(4.0 * w.d_head * w.h_active * (t + 1)))

    probe = W.stratified_rows(w, 128, seed=7).numpy()
    tp, _ = run(probe)
    n = int(min(w.B * w.T, max(128, 128 * target_s / max(tp, 1e-3))))
    tok = W.stratified_rows(w, n, seed=8).numpy()
    dt, dt_pre = run(tok)
    return {"value": flops(tok) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(tok)} of {w.B * w.T} tokens of {w.name}, stratified over position: the causal attention "
                      f"and slots of those tokens (oracle.attend_rows), {dt:.1f} s wall; their routing and query "
                      f"projection ran before, untimed ({dt_pre:.2f} s)",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "routing_and_projection_s": dt_pre, "attention_s": dt}


def decode_leg(torch, dev, steps):
    import sparse_routed_query_amd.gqe as G
    import workloads as W
    w = W.WORKLOADS["decode_b64"]
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    x = inp["x"].reshape(w.B, w.d_model).to(dev)
    wr, wq, lens = inp["w_router"].to(dev), inp["w_q"].to(dev), inp["lens"].to(dev)
    # two cache copies used alternately, so the 256 MB last-level cache cannot serve a step from the previous one
    caches = [(inp["k_cache"].to(dev), inp["v_cache"].to(dev))]
    caches.append((caches[0][0].clone(), caches[0][1].clone()))
    r = G.alloc_route(d, dev)
    q = G.alloc_qproj(d, dev)
    out = torch.empty((w.B, d.S, w.d_head), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gqe_decode_workspace_bytes(d, w.L_max), dtype=torch.uint8, device=dev)

    def route():
        G.gqe_route(d, x, wr, None, r["sel"], r["p_tilde"], r["counts"], r["offsets"], r["rows"], None,
                    r["workspace"])

    def qp():
        G.gqe_qproj(d, x, wq, r["sel"], r["counts"], r["offsets"], r["rows"], q["q_routed"], q["q_shared"])

    def pre():
        # the decode step's own preamble: routing and query projection in one launch, no compaction
        G.gqe_decode_route_qproj(d, x, wr, None, wq, None, 0.0, r["sel"], r["p_tilde"], q["q_routed"],
                                 q["q_shared"])

    it = [0]

    def attn():
        kc, vc = caches[it[0] & 1]
        it[0] += 1
        G.gqe_attn_decode(d, q["q_routed"], q["q_shared"], kc, vc, lens, r["p_tilde"], out, ws)

    # the same caches in pages of 16 positions, stored in a random order (two copies alternated as above)
    PAGE = 16
    pages = [W.make_paged_cache(w, inp, PAGE, seed=s) for s in (w.seed, w.seed + 1)]
    pages = [{k: v.to(dev) for k, v in pg.items()} for pg in pages]
    ws_p = torch.empty(G.gqe_decode_workspace_bytes(d, pages[0]["block_table"].shape[1] * PAGE), dtype=torch.uint8,
                       device=dev)

    def attn_paged():
        pg = pages[it[0] & 1]
        it[0] += 1
        G.gqe_attn_decode_paged(d, q["q_routed"], q["q_shared"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                lens, r["p_tilde"], out, ws_p)

    def step():
        pre()
        attn()

    warm([route, qp, pre, attn, attn_paged], torch)
    t_route, t_qp, t_pre, t_attn, t_paged = time_calls([route, qp, pre, attn, attn_paged], steps, torch,
                                                       queue_ahead=True)
    t_step, = time_calls([step], steps, torch, queue_ahead=True)
    nbytes = W.decode_kv_bytes(w, inp["lens"])
    gbs = nbytes / (t_attn * 1e-3) / 1e9
    return {"workload": w.name, "value": gbs, "unit": "GB/s", "metric": "decode attention GB/s (K/V bytes read once)",
            "attn_us": t_attn * 1e3, "step_us": t_step * 1e3,
            "preamble_us": t_pre * 1e3, "composed_step_us": (t_route + t_qp + t_attn) * 1e3,
            "paged16_attn_us": t_paged * 1e3, "paged16_gbs": nbytes / (t_paged * 1e-3) / 1e9,
            "route_us": t_route * 1e3, "qproj_us": t_qp * 1e3,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic_for("decode"),
                         "algorithmic_bytes": nbytes, "kernel": "gqe_attn_decode (split KV chunks + merge)"}}


def out_proj_leg(p, torch, steps):
    """The attention output projection fused with slot assembly on the step's own slots: y = W_o h over the
    S = kG+2 concatenated slots, bf16 MFMA with fp32 accumulation, from W_o packed once into fragment order
    (gqe_out_proj_packed; the row-major call gqe_out_proj timed beside it).  Timed beside them, for context
    only, hipBLASLt's plain bf16 GEMM (torch.mm) of slots that were already assembled and cast to bf16, with
    a bf16 result: it does neither the assembly nor the fp32 output."""
    import workloads as W
    w, G = p.w, p.G
    wo = W.make_w_o(w).to(p.x.device)
    wp = G.out_proj_pack(p.d, wo)
    BT = w.B * w.T
    y = torch.empty((BT, w.d_model), dtype=torch.float32, device=p.x.device)
    slots = p.out.view(BT, -1)

    def op_packed():
        G.gqe_out_proj_packed(p.d, p.out, p.r["p_tilde"], wp, y, False)

    def op():
        G.gqe_out_proj(p.d, p.out, p.r["p_tilde"], wo, y, False)

    hb = slots.to(torch.bfloat16)
    wt = wo.t()

    def lib():
        torch.mm(hb, wt)

    warm([op_packed, op, lib], torch)
    t_pk, t_op, t_lib = time_calls([op_packed, op, lib], steps, torch)
    fl = W.out_proj_flops(w)
    tf = fl / (t_pk * 1e-3) / 1e12
    # HBM floor of the call: the fp32 hard and shared slots read once, y written once (fp32)
    hbm_bytes = BT * (p.d.S - (1 if w.route_mode == 0 else w.G if w.route_mode == 1 else 0)) * w.d_head * 4 \
        + BT * w.d_model * 4
    return {"workload": w.name, "kernel": f"out_proj_tile_kernel<{w.d_head}, packed> (gqe_out_proj_packed)",
            "us": t_pk * 1e3, "tflops": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS, "flops": fl,
            "shape_mnk": [BT, w.d_model, slots.shape[1]], "row_major_weights_us": t_op * 1e3,
            "hbm_floor_bytes": hbm_bytes, "hbm_floor_us_at_8tbs": hbm_bytes / 8e12 * 1e6,
            "context_torch_mm_bf16_us": t_lib * 1e3}


def kv_proj_leg(p, torch, steps):
    """The K and V projections ahead of the path (gqe_kv_proj) on the step's x: 2 * B*T * d_model * 2 *
    H_kv * d_head FLOPs, bf16 MFMA with fp32 accumulation, outside the timed step; and the whole Q/K/V
    preamble in one launch (gqe_qkv_proj: kept experts, shared head, K and V from one read of x), without
    and with the rotary embedding, against gqe_qproj + gqe_kv_proj."""
    import workloads as W
    w, G = p.w, p.G
    wk, wv = (t.to(p.x.device) for t in W.make_w_kv(w))
    k = torch.empty_like(p.k)
    v = torch.empty_like(p.v)
    q = G.alloc_qproj(p.d, p.x.device)
    r = p.r

    def kv():
        G.gqe_kv_proj(p.d, p.x, wk, wv, k, v)

    def qkv():
        G.gqe_qkv_proj(p.d, p.x, p.wq, wk, wv, r["sel"], r["counts"], r["offsets"], r["rows"], None, 0.0,
                       q["q_routed"], q["q_shared"], k, v)

    def qkv_rope():
        G.gqe_qkv_proj(p.d, p.x, p.wq, wk, wv, r["sel"], r["counts"], r["offsets"], r["rows"], None, 10000.0,
                       q["q_routed"], q["q_shared"], k, v)

    warm([kv, p.qproj, qkv, qkv_rope], torch)
    t, t_qp, t_qkv, t_rope = time_calls([kv, p.qproj, qkv, qkv_rope], steps, torch)
    fl = 2.0 * w.B * w.T * w.d_model * 2 * w.H_kv * w.d_head
    fl_all = fl + W.qproj_flops(w)
    tf = fl / (t * 1e-3) / 1e12
    return {"workload": w.name, "kernel": f"kv_dense_kernel<{w.d_head}> (gqe_kv_proj)",
            "us": t * 1e3, "tflops": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS, "flops": fl,
            "qkv_proj_us": t_qkv * 1e3, "qkv_proj_rope_us": t_rope * 1e3, "qproj_plus_kv_proj_us": (t + t_qp) * 1e3,
            "qkv_proj_tflops": fl_all / (t_qkv * 1e-3) / 1e12, "qkv_proj_flops": fl_all}


def route_backward_leg(p, torch, steps):
    """The backward through slot assembly and routing (gqe_route_backward) on the step's own slots and
    routing with a seeded upstream gradient: memory-bound, so bytes it must move over its time against the
    HBM peak (reads dout, the hard slots and x; writes d_hard, the score gradient and dx; W_router and
    dW_router are small)."""
    w, G = p.w, p.G
    BT, S, D, kG, N = w.B * w.T, p.d.S, w.d_head, w.k * w.G, w.H_q
    gen = torch.Generator(device="cpu").manual_seed(5)
    dout = torch.randn((BT, S, D), generator=gen).to(p.x.device)
    out = p.out.view(BT, S, D)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=p.x.device)  # noqa: E731
    d_hard, d_logits, dw, db, dx = f32(BT, kG, D), f32(BT, N), f32(N, w.d_model), f32(N), f32(BT, w.d_model)
    ws = torch.empty(G.gqe_route_backward_workspace_bytes(p.d), dtype=torch.uint8, device=p.x.device)

    def bwd():
        G.gqe_route_backward(p.d, dout, out, p.r["sel"], p.r["p_tilde"], p.x, p.wr, d_hard, d_logits, dw, db, dx, ws)

    warm([bwd], torch)
    (t,) = time_calls([bwd], steps, torch)
    nbytes = 4.0 * BT * (S * D + kG * D) + 2.0 * BT * w.d_model + 4.0 * BT * (kG * D + N + w.d_model)
    gbs = nbytes / (t * 1e-3) / 1e9
    return {"workload": w.name, "kernel": "route_bwd token, dW partial + final, dx kernels (gqe_route_backward)",
            "us": t * 1e3, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS, "bytes": nbytes}


def attn_backward_leg(p, torch, steps):
    """The attention backward on the step's own query rows, K, V and slots with seeded slot gradients, given
    the forward's row statistics (gqe_attn_backward_lse; the forward that keeps them, and the backward that
    recomputes them, timed beside it).  Algorithmic work: the four products dV = P^T dO, dP = dO V^T,
    dq = dS K, dK = dS^T q over the causal scores, twice the forward's attention FLOPs (recomputing S, which
    the implementation does in both kernels, is not counted); against the bf16 peak."""
    import workloads as W
    w, G = p.w, p.G
    BT, S, D, kG = w.B * w.T, p.d.S, w.d_head, w.k * w.G
    gen = torch.Generator(device="cpu").manual_seed(9)
    d_hard = torch.randn((BT, kG, D), generator=gen).to(p.x.device)
    dout = torch.randn((BT, S, D), generator=gen).to(p.x.device)
    out = p.out.view(BT, S, D)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=p.x.device)  # noqa: E731
    dqr, dqs = f32(w.B, w.G, w.T * w.k, D), f32(w.B, w.T, D)
    dk, dv = f32(w.B, w.G, w.T, D), f32(w.B, w.G, w.T, D)
    ws = torch.empty(G.gqe_attn_backward_workspace_bytes(p.d), dtype=torch.uint8, device=p.x.device)
    # the forward's row statistics, from the statistics-keeping attention call on the same rows
    lse = torch.empty(G.lse_rows(p.d), dtype=torch.float32, device=p.x.device)
    slots = torch.empty_like(out)
    G.gqe_attn_prefill_heads_lse(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, slots, lse, p.ws)

    def bwd():
        G.gqe_attn_backward(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, out, d_hard, dout, dqr, dqs, dk, dv, ws)

    def bwd_lse():
        G.gqe_attn_backward_lse(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, out, d_hard, dout, lse, dqr, dqs, dk,
                                dv, ws)

    def fwd_lse():
        G.gqe_attn_prefill_heads_lse(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, slots, lse, p.ws)

    warm([bwd, bwd_lse, fwd_lse], torch)
    t, t_lse, t_fwd = time_calls([bwd, bwd_lse, fwd_lse], steps, torch)
    fl = 2.0 * W.attention_flops(w)
    tf = fl / (t_lse * 1e-3) / 1e12
    return {"workload": w.name,
            "kernel": "attn_bwd_dq_kernel<%d> + attn_bwd_dkdv_kernel<%d> (gqe_attn_backward_lse)" % (D, D),
            "us": t_lse * 1e3, "tflops": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS, "flops": fl,
            "recompute_statistics_us": t * 1e3, "forward_keeping_statistics_us": t_fwd * 1e3}


def ceilings_leg(torch, dev):
    """What this chip reaches under sustained load with nothing but dense bf16 MFMAs (every SIMD two waves,
    each four independent chains of v_mfma_f32_32x32x16_bf16), the shader clock that loop ran at (from the
    s_memtime and s_memrealtime counters of one wave), and a streaming read of 2 GiB with non-temporal
    16-byte loads: measured ceilings beside the published peaks the fractions are quoted against."""
    import sparse_routed_query_amd.calib as C
    blocks, iters = 512, 40000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)

    def mf():
        C.mfma(sink, clk, blocks, iters)

    warm([mf], torch, ms=60.0)
    (t_mfma,) = time_calls([mf], 10, torch)
    ticks = clk.cpu().tolist()
    fl = blocks * 4.0 * 4 * iters * 32768
    src = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    rsink = torch.empty(256 * 8, dtype=torch.int32, device=dev)

    def rd():
        C.read(src, rsink, 256 * 8)

    warm([rd], torch)
    (t_read,) = time_calls([rd], 10, torch)
    del src
    torch.cuda.empty_cache()
    tf = fl / (t_mfma * 1e-3) / 1e12
    gbs = (2 << 30) / (t_read * 1e-3) / 1e9
    return {"mfma_bf16_tflops": tf, "mfma_frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS,
            "mfma_loop_clock_ghz": ticks[0] / ticks[1] * 0.1 if ticks[1] > 0 else None,
            "mfma_loop_ms": t_mfma, "stream_read_gbs": gbs, "stream_read_frac_of_peak": gbs / HBM_PEAK_GBS,
            "kernels": "calib_mfma_kernel, calib_read_kernel (libgqe_calib.so)"}


def prefill_leg(w, inp, torch, dev, steps, traffic_key=None):
    """Every call of the step on one workload, each timed alone with events (after warming the clock),
    and the step as a whole: attention TFLOP/s and projection TFLOP/s against the bf16 peak."""
    import workloads as W
    p = Prefill(w, inp, dev)
    warm([p.step], torch)
    t_route, t_qp, t_attn, t_asm = time_calls([p.route, p.qproj, p.attn, p.assemble], steps, torch)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        p.step()
    ev1.record()
    torch.cuda.synchronize()
    t_step = ev0.elapsed_time(ev1) / steps
    fl, fq = W.attention_flops(w), W.qproj_flops(w)
    at, qt = fl / (t_attn * 1e-3) / 1e12, fq / (t_qp * 1e-3) / 1e12
    counts = p.r["counts"].cpu().tolist()
    del p
    torch.cuda.empty_cache()
    return {"workload": w.name, "B": w.B, "T": w.T, "d_model": w.d_model, "H_q": w.H_q, "H_kv": w.H_kv, "k": w.k,
            "d_head": w.d_head, "active_heads": w.h_active,
            "route_us": t_route * 1e3, "qproj_us": t_qp * 1e3, "attn_us": t_attn * 1e3, "assemble_us": t_asm * 1e3,
            "step_us": t_step * 1e3, "attn_flops": fl, "attn_tflops": at, "attn_frac": at / MFMA_BF16_PEAK_TFLOPS,
            "qproj_flops": fq, "qproj_tflops": qt, "qproj_frac": qt / MFMA_BF16_PEAK_TFLOPS,
            "step_attn_tflops": fl / (t_step * 1e-3) / 1e12,
            "attn_kernel": f"prefill_bf16_kernel<{w.d_head}>", "qproj_kernel": f"qproj_bf16_kernel<{w.d_head}, 64>",
            "attn_traffic": traffic_for(traffic_key) if traffic_key else None,
            "expert_rows": counts}


def proj_backward_leg(p, torch, steps):
    """The projections' backward (gqe_qkv_proj_backward) on the step's routing and x with seeded gradients of
    q, K and V: dW_q, dW_k, dW_v and dx, each 2 * d_head * d_model * B*T * (k*G + 1 + 2*H_kv) FLOPs
    (unselected experts cost nothing), against the bf16 peak."""
    import workloads as W
    w, G = p.w, p.G
    dev = p.x.device
    wk, wv = (t.to(dev) for t in W.make_w_kv(w))
    gen = torch.Generator(device="cpu").manual_seed(13)
    B, T, D = w.B, w.T, w.d_head
    dqr = torch.randn((B, w.G, T * w.k, D), generator=gen).to(dev)
    dqs = torch.randn((B, T, D), generator=gen).to(dev)
    dk = torch.randn((B, w.G, T, D), generator=gen).to(dev)
    dv = torch.randn((B, w.G, T, D), generator=gen).to(dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    dwq, dwk, dwv, dx = f32(*p.wq.shape), f32(*wk.shape), f32(*wv.shape), f32(B * T, w.d_model)
    nws = G.gqe_qkv_proj_backward_workspace_bytes(p.d, True)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    r = p.r

    def bwd():
        G.gqe_qkv_proj_backward(p.d, p.x, p.wq, wk, wv, r["sel"], r["counts"], r["offsets"], r["rows"], None, 0.0,
                                dqr, dqs, dk, dv, dwq, dwk, dwv, dx, ws)

    def bwd_dw():
        G.gqe_qkv_proj_backward(p.d, p.x, p.wq, wk, wv, r["sel"], r["counts"], r["offsets"], r["rows"], None, 0.0,
                                dqr, dqs, dk, dv, dwq, dwk, dwv, None, ws)

    warm([bwd, bwd_dw], torch)
    t, t_dw = time_calls([bwd, bwd_dw], steps, torch)
    fl_one = 2.0 * D * w.d_model * B * T * (w.k * w.G + w.n_shared + 2 * w.G)
    tf = 2 * fl_one / (t * 1e-3) / 1e12
    return {"workload": w.name, "kernel": f"pb_dw_kernel<{D}>{f' + pb_dw2_kernel<{D}>' if D <= 64 else ''} + "
                      f"{'pb_dx64_kernel' if D == 64 else f'pb_dx_kernel<{D}>'} (gqe_qkv_proj_backward)",
            "us": t * 1e3, "dw_us": t_dw * 1e3, "dx_us": (t - t_dw) * 1e3, "tflops": tf,
            "frac": tf / MFMA_BF16_PEAK_TFLOPS, "flops": 2 * fl_one}


def long_context_leg(torch, dev, steps):
    import workloads as W
    w = W.WORKLOADS["long_32k"]
    inp = W.make_inputs(w)
    res = {"gqe": prefill_leg(w, inp, torch, dev, steps, "prefill_long"),
           "dense": prefill_leg(W.dense_variant(w), inp, torch, dev, steps)}
    res["speedup_attn"] = res["dense"]["attn_us"] / res["gqe"]["attn_us"]
    res["speedup_step"] = res["dense"]["step_us"] / res["gqe"]["step_us"]
    res["ideal_flop_ratio"] = 16 / 9
    return res


def wide_leg(torch, dev, steps):
    import workloads as W
    w = W.WORKLOADS["wide_zipf"]
    return prefill_leg(w, W.make_inputs(w), torch, dev, steps, "prefill_wide")


def only(args, torch):
    """One call repeated, for rocprofv3 counter runs: the whole prefill step, the
    prefill attention and assembly calls on the main shape, the decode step
    (one-launch preamble and attention), the attention backward given the forward's statistics (main shape), or
    a plain 256 MiB device copy (the calibration kernel for FETCH_SIZE / WRITE_SIZE)."""
    import workloads as W
    import sparse_routed_query_amd.gqe as G
    dev = "cuda:0"
    if args.only == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
    elif args.only == "step":
        w = W.WORKLOADS["main_250m"]
        p = Prefill(w, W.make_inputs(w), dev)
        for _ in range(args.steps):
            p.step()
    elif args.only in ("prefill", "prefill_wide", "prefill_long"):
        w = W.WORKLOADS[{"prefill": "main_250m", "prefill_wide": "wide_zipf", "prefill_long": "long_32k"}[args.only]]
        p = Prefill(w, W.make_inputs(w), dev)
        p.route()
        p.qproj()
        for _ in range(args.steps):
            p.attn()
            p.assemble()
    elif args.only in ("qproj", "qproj_wide"):
        w = W.WORKLOADS["main_250m" if args.only == "qproj" else "wide_zipf"]
        p = Prefill(w, W.make_inputs(w), dev)
        p.route()
        for _ in range(args.steps):
            p.qproj()
    elif args.only == "attn_bwd":
        # gqe_attn_backward_lse on main_250m's own rows, K, V and slots, given the forward's statistics
        w = W.WORKLOADS["main_250m"]
        p = Prefill(w, W.make_inputs(w), dev)
        p.step()
        BT, S, D = w.B * w.T, p.d.S, w.d_head
        gen = torch.Generator(device="cpu").manual_seed(9)
        d_hard = torch.randn((BT, w.k * w.G, D), generator=gen).to(dev)
        dout = torch.randn((BT, S, D), generator=gen).to(dev)
        lse = torch.empty(G.lse_rows(p.d), dtype=torch.float32, device=dev)
        slots = torch.empty_like(p.out)
        G.gqe_attn_prefill_heads_lse(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, slots, lse, p.ws)
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
        grads = (f32(w.B, w.G, w.T * w.k, D), f32(w.B, w.T, D), f32(w.B, w.G, w.T, D), f32(w.B, w.G, w.T, D))
        ws = torch.empty(G.gqe_attn_backward_workspace_bytes(p.d), dtype=torch.uint8, device=dev)
        for _ in range(args.steps):
            G.gqe_attn_backward_lse(p.d, p.q["q_routed"], p.q["q_shared"], p.k, p.v, p.out.view(BT, S, D), d_hard,
                                    dout, lse, *grads, ws)
    elif args.only == "outproj":
        w = W.WORKLOADS["main_250m"]
        p = Prefill(w, W.make_inputs(w), dev)
        p.step()
        wp = G.out_proj_pack(p.d, W.make_w_o(w).to(dev))
        y = torch.empty((w.B * w.T, w.d_model), dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            G.gqe_out_proj_packed(p.d, p.out, p.r["p_tilde"], wp, y, False)
    else:
        w = W.WORKLOADS["decode_b64"]
        inp = W.make_inputs(w)
        d = G.desc_from(w)
        x = inp["x"].reshape(w.B, w.d_model).to(dev)
        wr, wq = inp["w_router"].to(dev), inp["w_q"].to(dev)
        kc, vc, lens = inp["k_cache"].to(dev), inp["v_cache"].to(dev), inp["lens"].to(dev)
        out = torch.empty((w.B, d.S, w.d_head), dtype=torch.float32, device=dev)
        ws = torch.empty(G.gqe_decode_workspace_bytes(d, w.L_max), dtype=torch.uint8, device=dev)
        r, q = G.alloc_route(d, dev), G.alloc_qproj(d, dev)
        for _ in range(args.steps):
            G.gqe_decode_route_qproj(d, x, wr, None, wq, None, 0.0, r["sel"], r["p_tilde"], q["q_routed"],
                                     q["q_shared"])
            G.gqe_attn_decode(d, q["q_routed"], q["q_shared"], kc, vc, lens, r["p_tilde"], out, ws)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is a design note, "
              f"not a measured path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.only:
        only(args, torch)
        return
    w = W.WORKLOADS["main_250m"]
    inp = W.make_inputs(w)
    p = Prefill(w, inp, dev)
    for _ in range(args.warmup):
        p.step()
    torch.cuda.synchronize()
    # then at least 30 ms more of the same step, so the timed steps run at the steady clock (the first
    # tens of milliseconds of load run slower whatever the step count)
    clock_warm_steps, clock_warm_ms = warm([p.step], torch)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n, time.perf_counter() - t0

    ms_step, wall = timed(p.step, args.steps)
    ms_graph = None
    if args.graph:
        # the four calls captured once into a HIP graph and replayed (the
        # library never allocates or syncs, so the step is capturable)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            p.step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            p.step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ms_graph, _ = timed(graph.replay, args.steps)
    fl = W.attention_flops(w)
    value = fl / (ms_step * 1e-3) / 1e12

    # per-call split, measured in a separate pass with events around each call
    t_route, t_qp, t_attn, t_asm = time_calls([p.route, p.qproj, p.attn, p.assemble], max(10, args.steps), torch)
    attn_tflops = fl / (t_attn * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "d_model": w.d_model, "H_q": w.H_q, "H_kv": w.H_kv,
                   "k": w.k, "n_shared": w.n_shared, "d_head": w.d_head, "causal": w.causal,
                   "active_heads": w.h_active, "attention_flops_per_step": fl, "parallelism": "single GPU"},
        "ms_per_step_hip_graph": ms_graph,
        "step_split_us": {"route": t_route * 1e3, "qproj": t_qp * 1e3, "attn_prefill_heads": t_attn * 1e3,
                          "assemble": t_asm * 1e3},
        "wall_s_timed": wall,
        "clock_warm": {"steps": clock_warm_steps, "ms": clock_warm_ms,
                       "note": "untimed steps run after the --warmup steps and before the timed ones"},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_for("prefill"),
                     "kernel": f"prefill_bf16_kernel<{w.d_head}> (the one kernel of gqe_attn_prefill_heads)",
                     "algorithmic_flops_per_launch": fl},
    }
    line["out_proj"] = out_proj_leg(p, torch, max(10, args.steps))
    line["kv_proj"] = kv_proj_leg(p, torch, max(10, args.steps))
    line["route_backward"] = route_backward_leg(p, torch, max(10, args.steps))
    line["attn_backward"] = attn_backward_leg(p, torch, max(10, args.steps))
    line["proj_backward"] = proj_backward_leg(p, torch, max(10, args.steps))
    del p
    torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = decode_leg(torch, dev, max(10, args.steps // 2))
        torch.cuda.empty_cache()
    if not args.no_context:
        line["long_context"] = long_context_leg(torch, dev, 10)
        torch.cuda.empty_cache()
        line["wide_zipf"] = wide_leg(torch, dev, 10)
        torch.cuda.empty_cache()
    if not args.no_context:
        line["ceilings"] = ceilings_leg(torch, dev)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
