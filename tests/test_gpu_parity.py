"""GPU-vs-oracle parity of the whole GQE path through the C ABI (MI355X only).

Full-size workloads are compared on a stratified sample of tokens (routing
and compaction on every token); the small shapes below span several tiles
with ragged tails and the method's degenerate cases, compared on every token.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_parity_util import (LOGIT_TOL, PT_TOL, agreed_routing, check_out, check_prefill_given_q, check_qproj,
                             check_route, full_decode_check,
                             full_prefill_check, gpu_decode, gpu_prefill, say)
import sparse_routed_query_amd.gqe as G

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="small", B=2, T=300, d_model=128, H_q=8, H_kv=2, k=2, d_head=64, dtype="bf16", seed=11,
                act_std=1.0, w_std=0.02)
    base.update(kw)
    return W.Workload(**base)


# ---------------------------------------------------------------- the five workloads

def test_tiny_fp32_both_route_modes():
    w = W.WORKLOADS["tiny_fp32"]
    full_prefill_check(w)
    full_prefill_check(w.replace(route_mode=0, name="tiny_fp32_mode0"))


def test_main_250m():
    full_prefill_check(W.WORKLOADS["main_250m"], n_sample=192)


def test_long_32k_gqe_and_dense():
    w = W.WORKLOADS["long_32k"]
    full_prefill_check(w, n_sample=96)
    full_prefill_check(W.dense_variant(w), n_sample=48)


def test_wide_zipf():
    w = W.WORKLOADS["wide_zipf"]
    inp, gpu, agreed = full_prefill_check(w, n_sample=96)
    c = agreed["counts"]
    say(f"[{w.name}] per-expert rows min={c.min()} max={c.max()} mean={c.mean():.0f}")
    assert c.max() > 1.3 * c.mean()     # the Zipf bias makes the load visibly uneven


def test_decode_b64():
    inp, gpu = full_decode_check(W.WORKLOADS["decode_b64"])
    assert np.isfinite(gpu["out"].numpy()).all()   # NaN-poisoned cache tails were never read


# ---------------------------------------------------------------- small shapes, every token

EDGE = [
    small(),                                            # 5 query tiles per head, ragged tail
    small(T=1), small(T=2), small(T=63), small(T=64), small(T=65), small(B=1, T=257),
    small(H_q=4, H_kv=4, k=1, name="E1_mha"),           # one expert per group
    small(H_q=8, H_kv=2, k=4, name="k_eq_E"),           # every expert kept = dense GQA
    small(H_q=4, H_kv=1, k=2, name="G1_mqa"),           # one group
    small(d_head=32, name="d32"), small(d_head=128, name="d128"),
    small(causal=0, name="noncausal"),
    small(n_shared=0, name="no_shared"),
    small(route_mode=1, name="per_group_slots"),
    small(route_mode=2, name="hard_only"), small(route_mode=2, n_shared=0, k=1, name="hard_only_no_shared"),
    small(route_mode=3, name="weighted_concat"), small(route_mode=3, n_shared=0, zipf_s=1.2, name="weighted_concat_ns"),
    small(dtype="f32", T=90, route_mode=3, name="f32_weighted_concat"),
    small(H_q=16, H_kv=4, k=2, zipf_s=1.2, name="zipf"),
    small(dtype="f32", T=100, d_model=96, name="f32_d64"),
    small(dtype="f32", T=70, d_head=128, d_model=64, k=1, name="f32_d128"),
    small(dtype="f32", T=50, causal=0, route_mode=1, name="f32_noncausal"),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: f"{w.name}-T{w.T}-d{w.d_head}-{w.dtype}")
def test_small_shapes_every_token(w):
    full_prefill_check(w)


# Sweeps of the expert pool E and of k (the study note's E/k sweeps; k chosen at inference is just a
# descriptor value), every token, both with the summed and the per-group weighted slots.
EK = [(2, 1), (4, 1), (4, 2), (4, 3), (8, 2), (8, 5), (16, 4), (16, 8)]


@pytest.mark.parametrize("E,k", EK, ids=lambda v: str(v))
def test_expert_pool_and_k_sweep(E, k):
    G = 64 // E if E > 4 else 4
    w = small(B=1, T=200, H_q=G * E, H_kv=G, k=k, route_mode=int(E % 2 == 0 and k % 2 == 1), name=f"E{E}k{k}")
    full_prefill_check(w)


def test_empty_batch():
    w = small(B=0, name="empty")
    d = G.desc_from(w)
    dev = "cuda"
    r = G.alloc_route(d, dev)
    r["counts"].fill_(7)
    r["offsets"].fill_(7)
    x = torch.empty((0, w.d_model), dtype=torch.bfloat16, device=dev)
    G.route(d, x, torch.zeros((w.N, w.d_model), dtype=torch.bfloat16, device=dev), bufs=r)
    q = G.qproj(d, x, torch.zeros((w.N + 1, w.d_head, w.d_model), dtype=torch.bfloat16, device=dev), r)
    kv = torch.empty((0, w.H_kv, w.T, w.d_head), dtype=torch.bfloat16, device=dev)
    out = G.attn_prefill(d, q, kv, kv, r["p_tilde"])
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert (r["counts"].cpu() == 0).all() and (r["offsets"].cpu() == 0).all()


def test_zero_router_ties_break_to_lowest_index_exactly():
    w = small(H_q=16, H_kv=4, k=2)
    inp = W.make_inputs(w)
    inp["w_router"] = torch.zeros_like(inp["w_router"])
    gpu = gpu_prefill(w, inp)
    assert (gpu["sel"] == torch.arange(w.k, dtype=torch.int32)).all()
    assert (gpu["p_tilde"] == 1.0 / w.k).all()
    check_route(w, inp, gpu)


def test_repeat_runs_are_bitwise_identical():
    w = W.WORKLOADS["main_250m"]
    inp = W.make_inputs(w)
    a = gpu_prefill(w, inp)
    b = gpu_prefill(w, inp)
    for key in ("sel", "p_tilde", "counts", "offsets", "rows", "q_routed", "q_shared", "out"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("BT,H_q,k", [(33000, 64, 2), (4097, 16, 1), (31, 64, 8)], ids=lambda v: str(v))
def test_route_compaction_both_paths(BT, H_q, k):
    """Routing and compaction, bit-exact after tie substitution, for block tables on both sides of the
    single-pass limit (33000 tokens x 64 experts takes the scan + scatter pair)."""
    w = W.Workload("route_only", B=1, T=BT, d_model=64, H_q=H_q, H_kv=8, k=k, d_head=32, dtype="bf16", seed=31,
                   act_std=1.0, w_std=0.05)   # score std 0.4, inside the range the tie margin is set for
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    x = inp["x"].reshape(-1, w.d_model).cuda()
    r = G.route(d, x, inp["w_router"].cuda(), None, logits=True)
    torch.cuda.synchronize()
    check_route(w, inp, {key: (v.cpu() if isinstance(v, torch.Tensor) else v) for key, v in r.items()})


# ---------------------------------------------------------------- split query tiles

SPLIT = [
    small(B=1, T=2500, name="split_k2"),                # E = 4, k = 2: 5000 routed rows per head, ragged tail
    small(B=2, T=2200, H_q=4, H_kv=2, k=1, d_head=32, name="split_d32"),
    small(B=1, T=2300, H_q=4, H_kv=4, k=1, d_head=128, route_mode=1, name="split_d128_mode1"),
    small(B=1, T=3000, k=3, H_q=8, H_kv=2, n_shared=0, name="split_k3_noshared"),
]


@pytest.mark.parametrize("w", SPLIT, ids=lambda w: w.name)
def test_split_tiles_every_token(w):
    """Query tiles whose key range is cut in two and merged by the later half, on every token."""
    d = G.desc_from(w)
    plan = G.gqe_attn_prefill_plan(d, True)
    assert G.gqe_attn_prefill_workspace_bytes(d) > 0 and (plan[:, 3] >= 0).any()
    full_prefill_check(w)


def prefill_inputs_on_gpu(w):
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    di = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    x = di["x"].reshape(-1, w.d_model)
    r = G.route(d, x, di["w_router"], di["b_router"])
    q = G.qproj(d, x, di["w_q"], r)
    return d, di, r, q


def test_split_merge_is_deterministic_and_resets_its_counters():
    w = SPLIT[0]
    d, di, r, q = prefill_inputs_on_gpu(w)
    n_pairs = int((G.gqe_attn_prefill_plan(d, True)[:, 3] >= 0).sum()) // 2
    ws = torch.zeros(G.gqe_attn_prefill_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    ctr = ws[: n_pairs * 4].view(torch.int32)              # one counter per split pair
    run = lambda w_: G.attn_prefill(d, q, di["k"], di["v"], r["p_tilde"], split=False) if w_ is None else (  # noqa
        G.gqe_attn_prefill(d, q["q_routed"], q["q_shared"], di["k"], di["v"], r["p_tilde"], out, w_))
    out = torch.empty((w.B, w.T, d.S, w.d_head), dtype=torch.float32, device="cuda")
    run(ws)
    a = out.clone()
    torch.cuda.synchronize()
    assert (ctr == 0).all(), "counters not reset"
    ctr.copy_(2 * torch.arange(n_pairs, dtype=torch.int32, device="cuda"))   # any even start works
    run(ws)
    torch.cuda.synchronize()
    assert torch.equal(out, a), "split result depends on the run"
    assert (ctr == 0).all()
    whole = run(None)
    torch.cuda.synchronize()
    err = (whole - a).abs()
    say(f"[{w.name}] split vs whole: max-abs={float(err.max()):.3e} mean-abs={float(err.mean()):.3e}")
    assert float(err.max()) <= 1e-2 and float(err.mean()) <= 1e-4


@pytest.mark.parametrize("w", [small(), small(route_mode=1, name="small_mode1"), small(route_mode=2, name="small_mode2"),
                               small(dtype="f32", d_head=32),
                               SPLIT[0]], ids=lambda w: f"{w.name}-{w.dtype}")
def test_heads_then_assemble_equals_attn_prefill(w):
    """gqe_attn_prefill_heads + gqe_assemble give exactly gqe_attn_prefill's output (same workspace)."""
    d, di, r, q = prefill_inputs_on_gpu(w)
    ref = G.attn_prefill(d, q, di["k"], di["v"], r["p_tilde"])
    out = torch.full_like(ref, float("nan"))
    G.gqe_attn_prefill_heads(d, q["q_routed"], q["q_shared"], di["k"], di["v"], out, G.prefill_workspace(d, "cuda"))
    kG = w.k * w.G
    n_w = (1, w.G, 0, 0)[w.route_mode]
    torch.cuda.synchronize()
    assert torch.isnan(out[:, :, kG:kG + n_w]).all(), "heads call wrote the weighted slots"
    G.gqe_assemble(d, r["p_tilde"], out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("T", [700, 2500])
def test_graph_replay_matches_eager(T):
    """The four prefill calls captured into a HIP graph give the eager results on every replay
    (T = 2500 splits its longest query tiles: the merge counters reset themselves)."""
    w = small(B=2, T=T, k=1, name="graph")
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    di = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    x = di["x"].reshape(-1, w.d_model)
    r = G.alloc_route(d, x.device)
    q = G.alloc_qproj(d, x.device)
    out = torch.empty((w.B, w.T, d.S, w.d_head), dtype=torch.float32, device=x.device)
    ws = G.prefill_workspace(d, x.device)
    assert (ws is not None) == (T > 2176)

    def step():
        G.gqe_route(d, x, di["w_router"], di["b_router"], r["sel"], r["p_tilde"], r["counts"], r["offsets"],
                    r["rows"], None, r["workspace"])
        G.gqe_qproj(d, x, di["w_q"], r["sel"], r["counts"], r["offsets"], r["rows"], q["q_routed"], q["q_shared"])
        G.gqe_attn_prefill_heads(d, q["q_routed"], q["q_shared"], di["k"], di["v"], out, ws)
        G.gqe_assemble(d, r["p_tilde"], out)

    step()
    torch.cuda.synchronize()
    bufs = dict(sel=r["sel"], p_tilde=r["p_tilde"], counts=r["counts"], offsets=r["offsets"], rows=r["rows"],
                q_routed=q["q_routed"], q_shared=q["q_shared"], out=out)
    ref = {k: v.clone() for k, v in bufs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for v in bufs.values():                 # eager work between replays
            v.fill_(-7 if v.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager run"


# ---------------------------------------------------------------- decode edges

def decode_case(**kw):
    base = dict(name="dec", B=5, T=1, d_model=128, H_q=8, H_kv=2, k=1, d_head=64, dtype="bf16", seed=21,
                act_std=1.0, w_std=0.02, decode=True, L_lo=1, L_hi=700, L_max=700)
    base.update(kw)
    return W.Workload(**base)


@pytest.mark.parametrize("w", [
    decode_case(),
    decode_case(k=2, route_mode=1, name="dec_k2_mode1"),
    decode_case(k=2, route_mode=2, name="dec_k2_hard_only"),
    decode_case(k=2, route_mode=3, name="dec_k2_weighted_concat"),
    decode_case(d_head=128, H_q=12, H_kv=3, k=3, name="dec_d128_dense"),
    decode_case(d_head=32, n_shared=0, name="dec_d32_noshared"),
    decode_case(dtype="f32", name="dec_f32"),
    decode_case(dtype="f32", d_head=128, L_hi=300, L_max=300, name="dec_f32_d128"),
    # up to 33 chunks of 128 keys: more than the merge holds in registers at d_head 128
    decode_case(d_head=128, H_q=8, H_kv=4, L_lo=1500, L_hi=4200, L_max=4200, name="dec_d128_long"),
], ids=lambda w: w.name)
def test_decode_shapes(w):
    drawn = W.make_inputs(w)["lens"]
    lens = drawn.clone()
    lens[0], lens[1] = 1, w.L_max               # a one-entry cache and a full cache
    full_decode_check(w, W.make_inputs(w, lens=lens))


def test_decode_lengths_outside_the_range_stay_in_bounds():
    """A sequence whose length is 0 or negative gets NaN slots and one longer than L_max is read as L_max;
    the other sequences are unaffected: their slots equal, bit for bit, those of the same call with every
    length in range (the workspace and the cache past each length hold NaN, so a stray read would show)."""
    w = decode_case(B=6, name="dec_bad_lens")
    good = torch.tensor([5, 700, 300, 1, 700, 64], dtype=torch.int32)
    bad = torch.tensor([0, 700, -4, 1, 900, 64], dtype=torch.int32)
    inp = W.make_inputs(w, lens=good)            # cache positions >= good[b] hold NaN
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(w.B, w.d_model).to(dev)
    r = G.route(d, x, inp["w_router"].to(dev))
    q = G.qproj(d, x, inp["w_q"].to(dev), r)
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    ws = torch.full((G.gqe_decode_workspace_bytes(d, w.L_max) // 4,), float("nan"), dtype=torch.float32, device=dev)
    ref = G.attn_decode(d, q, kc, vc, good.to(dev), r["p_tilde"], workspace=ws).cpu()
    ws.fill_(float("nan"))
    got = G.attn_decode(d, q, kc, vc, bad.to(dev), r["p_tilde"], workspace=ws).cpu()
    torch.cuda.synchronize()
    say(f"[{w.name}] lengths {bad.tolist()}: NaN rows {torch.isnan(got).all(-1).all(-1).tolist()}")
    assert torch.isnan(got[0]).all() and torch.isnan(got[2]).all()
    for b in (1, 3, 4, 5):                      # 900 > L_max = 700 reads as 700
        assert torch.equal(got[b], ref[b]), f"sequence {b} changed"


def test_decode_matches_last_prefill_row():
    """Decode of position L-1 equals prefill row L-1 computed by the GPU."""
    w = small(B=3, T=200, k=1, H_q=8, H_kv=4)
    inp = W.make_inputs(w)
    pre = gpu_prefill(w, inp)
    lens = torch.tensor([200, 37, 1], dtype=torch.int32)
    dw = w.replace(T=1, decode=True, L_max=200)
    dinp = dict(x=inp["x"][torch.arange(3), lens.long() - 1].reshape(3, 1, -1), w_router=inp["w_router"],
                b_router=None, w_q=inp["w_q"], k_cache=inp["k"], v_cache=inp["v"], lens=lens)
    dec = gpu_decode(dw, dinp)
    ref = pre["out"][torch.arange(3), lens.long() - 1]
    check_out(dw, dec["out"].numpy(), ref.double().numpy(), "decode vs prefill row")
    assert torch.equal(dec["sel"], pre["sel"].reshape(3, 200, w.G, w.k)[torch.arange(3), lens.long() - 1])



def test_two_stream_step_matches_one_stream():
    """The shared head projected and attended on a side stream (calls with q_routed = NULL) while the main
    stream routes and handles the kept experts (calls with q_shared = NULL), sharing one workspace, gives the
    one-stream results bit for bit."""
    w = small(B=2, T=2500, k=1, name="two_streams")
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    di = {key: (v.cuda() if v is not None else None) for key, v in inp.items()}
    x = di["x"].reshape(-1, w.d_model)
    ws = G.prefill_workspace(d, "cuda")
    assert ws is not None
    r = G.route(d, x, di["w_router"], di["b_router"])
    q1 = G.qproj(d, x, di["w_q"], r)
    out1 = torch.full((w.B, w.T, d.S, w.d_head), float("nan"), device="cuda")
    G.gqe_attn_prefill_heads(d, q1["q_routed"], q1["q_shared"], di["k"], di["v"], out1, ws)
    G.gqe_assemble(d, r["p_tilde"], out1)
    q2 = G.alloc_qproj(d, "cuda")
    out2 = torch.full_like(out1, float("nan"))
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            G.gqe_qproj(d, x, di["w_q"], None, None, None, None, None, q2["q_shared"])
            G.gqe_attn_prefill_heads(d, None, q2["q_shared"], di["k"], di["v"], out2, ws)
        G.gqe_qproj(d, x, di["w_q"], r["sel"], r["counts"], r["offsets"], r["rows"], q2["q_routed"], None)
        G.gqe_attn_prefill_heads(d, q2["q_routed"], None, di["k"], di["v"], out2, ws)
        G.gqe_assemble(d, r["p_tilde"], out2)
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(q2["q_routed"], q1["q_routed"]) and torch.equal(q2["q_shared"], q1["q_shared"])
        assert torch.equal(out2, out1), f"round {rep}: two-stream result differs"


def test_large_scores_move_the_softmax_reference():
    """Scores spread over tens of log2 units and growing along the keys, so new row maxima keep arriving:
    the lazy softmax reference moves on the first tile, on the first and on the second 32-key block of
    later tiles, and across the two halves of split query tiles (T = 2500), on every token.  With scores
    this large (|s| up to ~40 log2 units) the projection's bf16 rounding of the query alone moves outputs
    by up to ~0.1, so the attention is compared with the oracle's attention of the query rows the
    projection returned (their exact bf16 values), at the same 2e-2 / 2e-3 bar; the rows themselves are
    checked against the oracle's projection first."""
    w = small(B=1, T=2500, k=1, w_std=0.35, name="large_scores")
    inp = W.make_inputs(w)
    ramp = 1.0 + 3.0 * torch.arange(w.T, dtype=torch.float32) / w.T
    inp["k"] = (inp["k"].float() * ramp[None, None, :, None]).to(inp["k"].dtype)
    # router scores back to the spread the routing tolerances are set for (std ~0.4)
    inp["w_router"] = (inp["w_router"].float() * 0.1).to(inp["w_router"].dtype)
    gpu = gpu_prefill(w, inp)
    agreed = check_route(w, inp, gpu)
    tok = np.arange(w.B * w.T)
    check_qproj(w, inp, gpu, agreed, tok)
    check_prefill_given_q(w, inp, gpu, agreed, tok)


# ---------------------------------------------------------------- decode: routing + query projection, one launch

def decode_pre(w, inp, positions=None, base=0.0):
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(w.B, w.d_model).to(dev)
    br = inp["b_router"].to(dev) if inp["b_router"] is not None else None
    pos = positions.to(dev) if positions is not None else None
    res = G.decode_route_qproj(d, x, inp["w_router"].to(dev), br, inp["w_q"].to(dev), pos, base, logits=True)
    torch.cuda.synchronize()
    return {k: (v.cpu() if v is not None else None) for k, v in res.items()}


def check_decode_pre(w, inp, got, positions=None, base=0.0):
    """Routing against oracle.route (GPU choice accepted only at a flagged tie), logits and p~ within the
    routing tolerances, query rows against the oracle's projection of the agreed selection (rotated by
    oracle.rope when base > 1)."""
    od = oracle.desc(w)
    orc = oracle.route(od, inp["x"].reshape(w.B, w.d_model), inp["w_router"], inp["b_router"])
    sel, pt, n_sub = agreed_routing(w, orc, got["sel"].numpy())
    dlog = float(np.abs(got["logits"].numpy() - orc["logits"]).max())
    dpt = float(np.abs(got["p_tilde"].numpy().astype(np.float64) - pt).max())
    say(f"[{w.name}] decode preamble route: tie-substituted={n_sub} max|dlogit|={dlog:.3e} max|dp~|={dpt:.3e}")
    assert dlog < LOGIT_TOL and dpt <= PT_TOL
    tok = np.arange(w.B)
    qr, qs = oracle.qproj_rows(od, inp["x"], inp["w_q"], sel, tok)
    pos = positions.numpy() if positions is not None else None
    check_rotated(w, got["q_routed"][:, :, 0], qr, pos, base, "decode preamble q_routed")
    if w.n_shared:
        check_rotated(w, got["q_shared"][:, 0], qs, pos, base, "decode preamble q_shared")


DEC_PRE = [decode_case(), decode_case(k=2, route_mode=1, name="dec_k2_mode1"),
           decode_case(k=2, route_mode=2, name="dec_k2_hard_only"),
           decode_case(k=2, route_mode=3, name="dec_k2_weighted_concat"),
           decode_case(d_head=128, H_q=12, H_kv=3, k=3, name="dec_d128"),
           decode_case(d_head=32, n_shared=0, name="dec_d32_noshared"),
           decode_case(H_q=64, H_kv=1, k=8, d_model=320, name="dec_e64_k8"),
           decode_case(dtype="f32", name="dec_f32"),
           decode_case(dtype="f32", d_model=90, d_head=128, H_q=12, H_kv=4, k=2, name="dec_f32_dm90"),
           decode_case(B=300, d_model=1024, H_q=16, H_kv=8, name="dec_b300"),
           W.WORKLOADS["decode_b64"]]


@pytest.mark.parametrize("w", DEC_PRE, ids=lambda w: w.name)
def test_decode_route_qproj_against_the_oracle(w):
    inp = W.make_inputs(w)
    check_decode_pre(w, inp, decode_pre(w, inp))


@pytest.mark.parametrize("w", [decode_case(name="dec_rope"), decode_case(d_head=128, k=2, name="dec_rope_d128"),
                               decode_case(dtype="f32", d_head=32, name="dec_rope_f32")], ids=lambda w: w.name)
def test_decode_route_qproj_rotary_against_the_oracle(w):
    inp = W.make_inputs(w)
    pos = (inp["lens"] - 1).to(torch.int32)
    pos[0] = 65535          # a large position: the angle's rounding grows with it
    for base in (10000.0, 500000.0):
        check_decode_pre(w, inp, decode_pre(w, inp, pos, base), pos, base)


@pytest.mark.parametrize("w", [decode_case(dtype="f32", name="dec_f32"),
                               decode_case(dtype="f32", k=2, route_mode=3, name="dec_f32_mode3")],
                         ids=lambda w: w.name)
def test_decode_route_qproj_fp32_routing_is_gqe_routes_bit_for_bit(w):
    """fp32 scores take gqe_route's own fp64 FMA chain, so logits, selection and p~ agree to the bit."""
    inp = W.make_inputs(w)
    got = decode_pre(w, inp)
    dev = "cuda"
    r = G.route(G.desc_from(w), inp["x"].reshape(w.B, w.d_model).to(dev), inp["w_router"].to(dev),
                inp["b_router"].to(dev) if inp["b_router"] is not None else None, logits=True)
    torch.cuda.synchronize()
    for key in ("logits", "sel", "p_tilde"):
        assert torch.equal(got[key], r[key].cpu()), key


def test_fused_and_composed_decode_steps_agree():
    """G.decode's one-launch preamble and gqe_route + gqe_qproj give the same slots (same selection; query
    rows within one bf16 rounding of each other, so the slots within the decode tolerance)."""
    w = W.WORKLOADS["decode_b64"]
    inp = W.make_inputs(w)
    d = G.desc_from(w)
    di = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (d, di["x"].reshape(w.B, w.d_model), di["w_router"], di["b_router"], di["w_q"], di["k_cache"],
            di["v_cache"], di["lens"])
    a, b = G.decode(*args), G.decode(*args, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(a["sel"], b["sel"])
    check_out(w, a["out"].cpu().numpy(), b["out"].cpu().double().numpy(), "fused vs composed decode")


def test_decode_route_qproj_empty_batch():
    w = decode_case(B=0, name="dec_empty")
    d = G.desc_from(w)
    res = G.decode_route_qproj(d, torch.empty((0, w.d_model), dtype=torch.bfloat16, device="cuda"),
                               torch.zeros((w.H_q, w.d_model), dtype=torch.bfloat16, device="cuda"), None,
                               torch.zeros((w.H_q + 1, w.d_head, w.d_model), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert res["sel"].numel() == 0 and res["q_routed"].numel() == 0


# ---------------------------------------------------------------- paged decode

def paged_and_dense(w, page_size):
    """gqe_attn_decode over the dense cache and gqe_attn_decode_paged over the same cache cut into pages
    stored in a random order (unused pages and positions NaN), with the same routing and queries."""
    inp = W.make_inputs(w)
    pg = W.make_paged_cache(w, inp, page_size)
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(w.B, w.d_model).to(dev)
    br = inp["b_router"].to(dev) if inp["b_router"] is not None else None
    r = G.route(d, x, inp["w_router"].to(dev), br)
    q = G.qproj(d, x, inp["w_q"].to(dev), r)
    lens = inp["lens"].to(dev)
    dense = G.attn_decode(d, q, inp["k_cache"].to(dev), inp["v_cache"].to(dev), lens, r["p_tilde"])
    out = torch.full_like(dense, float("nan"))
    L_cap = pg["block_table"].shape[1] * page_size
    ws = torch.empty(G.gqe_decode_workspace_bytes(d, L_cap), dtype=torch.uint8, device=dev)
    G.gqe_attn_decode_paged(d, q["q_routed"], q["q_shared"], pg["k_pages"].to(dev), pg["v_pages"].to(dev),
                            pg["block_table"].to(dev), lens, r["p_tilde"], out, ws)
    torch.cuda.synchronize()
    return inp, r, dense.cpu(), out.cpu()


@pytest.mark.parametrize("w,page_size", [
    (decode_case(), 8), (decode_case(), 64), (decode_case(), 4096),
    (decode_case(k=2, route_mode=1, name="dec_k2_mode1"), 16),
    (decode_case(d_head=128, H_q=12, H_kv=3, k=3, name="dec_d128"), 32),
    (decode_case(dtype="f32", name="dec_f32"), 16),
    (W.WORKLOADS["decode_b64"], 16), (W.WORKLOADS["decode_b64"], 256),
], ids=lambda v: v.name if isinstance(v, W.Workload) else f"page{v}")
def test_paged_decode_equals_dense(w, page_size):
    """Only where K and V live differs, so the outputs are the dense call's, bit for bit."""
    _, _, dense, paged = paged_and_dense(w, page_size)
    assert torch.isfinite(paged).all()          # no NaN page row or spare page was read
    assert torch.equal(paged, dense)


def test_paged_decode_against_the_oracle():
    w = decode_case(B=7, L_lo=1, L_hi=300, L_max=300, name="dec_paged_oracle")
    inp, r, _, paged = paged_and_dense(w, 32)
    orc = oracle.decode(oracle.desc(w), inp["x"].reshape(w.B, w.d_model), inp["w_router"], inp["b_router"],
                        inp["w_q"], inp["k_cache"], inp["v_cache"], inp["lens"])
    assert np.array_equal(r["sel"].cpu().numpy(), orc["sel"]) or orc["tie"].any()
    check_out(w, paged.numpy(), orc["out"], "paged decode out")


def test_decode_and_out_proj_graph_replay_and_repeat():
    """A decode step on a paged cache followed by the output projection, captured into one HIP graph,
    gives the eager results on every replay; and repeated eager calls give the same bits."""
    w = decode_case(B=6, L_lo=1, L_hi=500, L_max=500, name="dec_graph")
    inp = W.make_inputs(w)
    pg = {k: v.cuda() for k, v in W.make_paged_cache(w, inp, 32).items()}
    d = G.desc_from(w)
    x = inp["x"].reshape(w.B, w.d_model).cuda()
    wr, wq, lens = inp["w_router"].cuda(), inp["w_q"].cuda(), inp["lens"].cuda()
    wo = W.make_w_o(w).cuda()
    r = G.alloc_route(d, x.device)
    q = G.alloc_qproj(d, x.device)
    out = torch.empty((w.B, d.S, w.d_head), dtype=torch.float32, device=x.device)
    y = torch.empty((w.B, w.d_model), dtype=torch.float32, device=x.device)
    ws = torch.empty(G.gqe_decode_workspace_bytes(d, pg["block_table"].shape[1] * 32), dtype=torch.uint8,
                     device=x.device)

    def step():
        G.gqe_route(d, x, wr, None, r["sel"], r["p_tilde"], r["counts"], r["offsets"], r["rows"], None,
                    r["workspace"])
        G.gqe_qproj(d, x, wq, r["sel"], r["counts"], r["offsets"], r["rows"], q["q_routed"], q["q_shared"])
        G.gqe_attn_decode_paged(d, q["q_routed"], q["q_shared"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                lens, r["p_tilde"], out, ws)
        G.gqe_out_proj(d, out, r["p_tilde"], wo, y, True)

    step()
    torch.cuda.synchronize()
    ref = {"out": out.clone(), "y": y.clone()}
    for _ in range(2):                           # repeated eager calls: the same bits
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref["out"]) and torch.equal(y, ref["y"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        out.fill_(float("nan"))                  # eager work between replays
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref["out"]), f"replay {rep}: out differs from the eager run"
        assert torch.equal(y, ref["y"]), f"replay {rep}: y differs from the eager run"


# ---------------------------------------------------------------- K / V projection ahead of the path

@pytest.mark.parametrize("w", [small(), small(d_head=32, name="d32"), small(d_head=128, T=100, name="d128"),
                               small(B=1, T=1, name="T1"), small(dtype="f32", T=100, d_model=96, name="f32"),
                               W.WORKLOADS["main_250m"]], ids=lambda w: f"{w.name}-{w.dtype}")
def test_kv_projection(w):
    """K and V against the oracle element by element: bf16 output rounding (relative 2^-8 of the value)
    plus fp32 accumulation over d_model terms (d_model 2^-24 of sum |x| |w|)."""
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    d = G.desc_from(w)
    x = inp["x"].reshape(-1, w.d_model)
    k, v = G.kv_proj(d, x.cuda(), wk.cuda(), wv.cuda())
    torch.cuda.synchronize()
    od = oracle.desc(w)
    xa = np.abs(x.double().numpy())
    for name, got, wt in (("k", k, wk), ("v", v, wv)):
        ref = oracle.kv_proj(od, x, wt)
        mag = np.einsum("tm,hdm->htd", xa, np.abs(wt.double().numpy())).reshape(w.H_kv, w.B, w.T, w.d_head)
        mag = mag.transpose(1, 0, 2, 3)
        eps_out = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
        bound = eps_out * np.abs(ref) + (w.d_model + 2) * 2.0 ** -24 * mag * 1.01 + 1e-30
        err = np.abs(got.cpu().double().numpy() - ref)
        say(f"[{w.name}] kv_proj {name}: max-abs={err.max():.3e} max err/bound={(err / bound).max():.3f}")
        assert (err <= bound).all()


def test_layer_from_x_kv_projection_feeds_attention():
    """K/V projected on the GPU feed the prefill path; the attention matches the oracle's on those K/V."""
    w = small(B=2, T=300, name="layer")
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    d = G.desc_from(w)
    k, v = G.kv_proj(d, inp["x"].reshape(-1, w.d_model).cuda(), wk.cuda(), wv.cuda())
    torch.cuda.synchronize()
    inp = dict(inp, k=k.cpu(), v=v.cpu())
    gpu = gpu_prefill(w, inp)
    agreed = check_route(w, inp, gpu)
    tok = np.arange(w.B * w.T)
    check_qproj(w, inp, gpu, agreed, tok)
    check_prefill_given_q(w, inp, gpu, agreed, tok)


def test_decode_input_audit_counts_bad_lengths_and_page_ids():
    """gqe_check_decode_inputs counts what the decode calls would clamp: lengths outside 1..L_max and
    page ids outside the pool in the table columns a sequence uses (unused columns are not counted)."""
    w = decode_case(B=8, name="audit")
    d = G.desc_from(w)
    lens = torch.tensor([1, 700, 0, 701, -3, 350, 64, 65], dtype=torch.int32)
    assert G.check_decode_inputs(d, lens.cuda(), 700) == (3, 0)
    assert G.check_decode_inputs(d, torch.tensor([5] * 8, dtype=torch.int32).cuda(), 700) == (0, 0)
    P, max_pages, num_pages = 64, 11, 40
    table = torch.randint(0, num_pages, (8, max_pages), dtype=torch.int32, generator=torch.Generator().manual_seed(1))
    good = lens.clamp(1, 700)
    assert G.check_decode_inputs(d, good.cuda(), max_pages * P, table.cuda(), num_pages, P) == (0, 0)
    table[0, 0] = -1          # used (length 1)
    table[1, 10] = num_pages  # used (length 700 reaches column 10)
    table[6, 0] = 10 ** 6     # used (length 64 fills column 0 only)
    table[6, 1] = -5          # not used by a length of 64
    table[7, 1] = num_pages + 3   # used (length 65 reaches column 1)
    assert G.check_decode_inputs(d, good.cuda(), max_pages * P, table.cuda(), num_pages, P) == (0, 4)


# ---------------------------------------------------------------- fused Q/K/V preamble, rotary embedding

def qkv_case(w, rope_base=0.0, positions=None):
    """gqe_route, then gqe_qkv_proj on the workload's x, W_q and seeded W_k / W_v."""
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(-1, w.d_model).to(dev)
    br = inp["b_router"].to(dev) if inp["b_router"] is not None else None
    r = G.route(d, x, inp["w_router"].to(dev), br)
    pos = positions.to(dev) if positions is not None else None
    out = G.qkv_proj(d, x, inp["w_q"].to(dev), wk.to(dev), wv.to(dev), r, pos, rope_base)
    torch.cuda.synchronize()
    return inp, wk, wv, d, r, {k: v.cpu() for k, v in out.items()}


@pytest.mark.parametrize("w", [small(), small(d_head=32, name="d32"), small(d_head=128, name="d128"),
                               small(dtype="f32", T=90, name="f32")], ids=lambda w: w.name)
def test_qkv_proj_without_rotation_equals_separate_projections(w):
    """One launch of every projection gives, bit for bit, what gqe_qproj and gqe_kv_proj give."""
    inp, wk, wv, d, r, out = qkv_case(w)
    dev = "cuda"
    x = inp["x"].reshape(-1, w.d_model).to(dev)
    q = G.qproj(d, x, inp["w_q"].to(dev), r)
    k, v = G.kv_proj(d, x, wk.to(dev), wv.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(out["q_routed"], q["q_routed"].cpu()) and torch.equal(out["q_shared"], q["q_shared"].cpu())
    assert torch.equal(out["k"], k.cpu()) and torch.equal(out["v"], v.cpu())


def check_rotated(w, got, ref_plain, pos, base, what):
    """got (GPU, rotated) against the oracle's rotation of the oracle's unrotated projection ref_plain
    (float64, [..., d_head]): bf16 rounding of the result (2^-8 relative), the fp32 rotation and angle
    (1e-5 of the pair's magnitude) and 1e-4 absolute; fp32 1e-5 of max|ref|."""
    ref = oracle.rope(ref_plain, pos, base) if base else ref_plain
    g = got.double().numpy()
    err = np.abs(g - ref)
    h = w.d_head // 2
    pair = np.abs(ref_plain[..., :h]) + np.abs(ref_plain[..., h:])
    mag = np.concatenate([pair, pair], axis=-1)
    if w.dtype == "bf16":
        lim = 2.0 ** -8 * np.abs(ref) + 1e-5 * mag + 1e-4
    else:
        lim = 1e-5 * max(1e-30, np.abs(ref).max()) + 1e-6 * mag
    say(f"[{w.name}] {what}: max-abs={err.max():.3e} max err/bound={(err / lim).max():.3f}")
    assert (err <= lim).all()


@pytest.mark.parametrize("w,base,given", [
    (small(), 10000.0, False), (small(d_head=32, name="d32"), 10000.0, True),
    (small(d_head=128, k=1, name="d128"), 500000.0, False), (small(T=64, name="short_base"), 10.0, True),
    (small(dtype="f32", T=90, name="f32"), 10000.0, True),
], ids=lambda v: getattr(v, "name", str(v)))
def test_qkv_proj_rotary_against_the_oracle(w, base, given):
    """Routed and shared queries and K rotated by position (given, or t), V not rotated, against the
    oracle's projections rotated by oracle.rope."""
    positions = None
    if given:
        positions = torch.randint(0, 70000, (w.B * w.T,), dtype=torch.int32, generator=torch.Generator().manual_seed(4))
    inp, wk, wv, d, r, out = qkv_case(w, base, positions)
    agreed = check_route(w, inp, dict(sel=r["sel"].cpu(), p_tilde=r["p_tilde"].cpu(), counts=r["counts"].cpu(),
                                      offsets=r["offsets"].cpu(), rows=r["rows"].cpu()))
    od = oracle.desc(w)
    tok = np.arange(w.B * w.T)
    pos = positions.numpy() if given else tok % w.T
    qr, qs = oracle.qproj_rows(od, inp["x"], inp["w_q"], agreed["sel"], tok)
    b, t = tok // w.T, tok % w.T
    check_rotated(w, out["q_routed"][b, :, t], qr, pos, base, "q_routed")
    check_rotated(w, out["q_shared"][b, t], qs, pos, base, "q_shared")
    kp = oracle.kv_proj(od, inp["x"], wk)                         # [B, H_kv, T, d_head]
    kpos = pos.reshape(w.B, 1, w.T)
    check_rotated(w, out["k"], kp, np.broadcast_to(kpos, kp.shape[:-1]), base, "k")
    check_rotated(w, out["v"], oracle.kv_proj(od, inp["x"], wv), None, 0.0, "v")


def test_rotary_layer_prefill_and_decode():
    """x -> route -> rotated Q/K/V (one launch) -> attention: the slots against the oracle's attention of the
    GPU's rotated queries and keys; and a decode step at position L-1 (T = 1, positions = L - 1) against the
    cache of those rotated keys equals prefill row L-1."""
    w = small(B=2, T=300, name="rope_layer")
    base = 10000.0
    inp, wk, wv, d, r, out = qkv_case(w, base)
    dev = "cuda"
    slots = G.attn_prefill(d, {"q_routed": out["q_routed"].to(dev), "q_shared": out["q_shared"].to(dev)},
                           out["k"].to(dev), out["v"].to(dev), r["p_tilde"])
    torch.cuda.synchronize()
    gpu = dict(q_routed=out["q_routed"], q_shared=out["q_shared"], out=slots.cpu())
    agreed = dict(ptilde=r["p_tilde"].cpu().double().numpy())
    check_prefill_given_q(w, dict(inp, k=out["k"], v=out["v"]), gpu, agreed, np.arange(w.B * w.T))
    lens = torch.tensor([300, 41], dtype=torch.int32)
    dw = w.replace(T=1, decode=True, L_max=300, name="rope_decode")
    dd = G.desc_from(dw)
    xs = inp["x"][torch.arange(2), lens.long() - 1].reshape(2, -1).to(dev)
    rd = G.route(dd, xs, inp["w_router"].to(dev))
    qd = G.qkv_proj(dd, xs, inp["w_q"].to(dev), wk.to(dev), wv.to(dev), rd, (lens - 1).to(dev), base)
    dec = G.attn_decode(dd, qd, out["k"].to(dev), out["v"].to(dev), lens.to(dev), rd["p_tilde"])
    torch.cuda.synchronize()
    ref = slots.cpu().reshape(2, 300, d.S, w.d_head)[torch.arange(2), lens.long() - 1]
    # the decode step's rotated K of the new token equals the prefill's at that position
    assert torch.equal(qd["k"].cpu()[:, :, 0], out["k"][torch.arange(2), :, lens.long() - 1])
    check_out(dw, dec.cpu().numpy(), ref.double().numpy(), "rotary decode vs prefill row")
