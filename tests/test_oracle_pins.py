"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes one step of the oracle to a library routine (torch CPU in
float64), a closed form, an invariant, brute force on tiny inputs, or the
counts printed in the GQE study note, so that a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle fails at least one test.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))

def wl(**kw):
    base = dict(name="pin", B=2, T=29, d_model=24, H_q=6, H_kv=3, k=1, d_head=8, dtype="f32",
                seed=7, act_std=1.0, w_std=0.3)
    base.update(kw)
    return W.Workload(**base)

def torch_q(w, inp):
    """All H_q (+ shared) query projections with torch: [B, H, T, d_head], float64."""
    x = inp["x"].double()                              # [B, T, dm]
    wq = inp["w_q"].double()                           # [H, dh, dm]
    return torch.einsum("btm,hdm->bhtd", x, wq)

def torch_sdpa(q, k, v, causal):
    return F.scaled_dot_product_attention(q, k, v, is_causal=bool(causal))

# ---------------------------------------------------------------- steps 1-4

def test_router_logits_and_group_softmax_match_torch():
    w = wl(H_q=12, H_kv=3, k=2, zipf_s=1.2)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"], inp["b_router"])
    s = inp["x"].double().reshape(-1, w.d_model) @ inp["w_router"].double().T + inp["b_router"].double()
    np.testing.assert_allclose(r["logits"], s.numpy(), rtol=1e-12, atol=1e-12)
    p = torch.softmax(s.view(-1, w.G, w.E), dim=-1).reshape(-1, w.N)
    np.testing.assert_allclose(r["probs"], p.numpy(), rtol=1e-12, atol=1e-14)

@pytest.mark.parametrize("E,k", [(2, 1), (4, 2), (4, 3), (3, 1)])
def test_zero_router_gives_exact_ties_broken_to_lowest_index(E, k):
    w = wl(H_q=2 * E, H_kv=2, k=k)
    inp = W.make_inputs(w)
    r = oracle.route(oracle.desc(w), inp["x"], torch.zeros_like(inp["w_router"]))
    assert (r["sel"] == np.arange(k, dtype=np.int32)).all()
    assert (r["ptilde"] == 1.0 / k).all()
    assert r["tie"].all() == (k < E) and r["tie"].any() == (k < E)

def test_uniform_shift_of_a_groups_logits_changes_nothing():
    w = wl(H_q=12, H_kv=3, k=2)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    a = oracle.route(d, inp["x"], inp["w_router"])
    shift = torch.tensor([0.7, -3.0, 11.0], dtype=torch.float64).repeat_interleave(w.E)
    b = oracle.route(d, inp["x"], inp["w_router"], shift)
    assert (a["sel"] == b["sel"]).all()
    np.testing.assert_allclose(a["ptilde"], b["ptilde"], rtol=1e-12)

@pytest.mark.parametrize("E,k", [(4, 2), (5, 2), (5, 3), (3, 1), (4, 4)])
def test_topk_against_subset_enumeration_with_exact_ties(E, k):
    # Integer-valued logits make exact ties common; the kept set must maximise
    # the logit sum and, among maximisers, be the lexicographically smallest.
    w = wl(H_q=2 * E, H_kv=2, k=k, d_model=3, T=64)
    g = torch.Generator().manual_seed(E * 10 + k)
    x = torch.randint(-1, 2, (w.B, w.T, w.d_model), generator=g).double()
    wr = torch.randint(-2, 3, (w.N, w.d_model), generator=g).double()
    r = oracle.route(oracle.desc(w), x, wr)
    s = (x.reshape(-1, w.d_model) @ wr.T).view(-1, w.G, w.E).numpy()
    n_ties = 0
    for t in range(s.shape[0]):
        for gg in range(w.G):
            best = max(itertools.combinations(range(E), k), key=lambda c: (sum(s[t, gg, list(c)]), [-i for i in c]))
            assert tuple(r["sel"][t, gg]) == best
            srt = np.sort(s[t, gg])[::-1]
            tie = k < E and (srt[k - 1] - srt[k]) < 1e-6
            assert bool(r["tie"][t, gg]) == tie
            n_ties += tie
    assert k == E or n_ties > 0

def test_renormalised_weights_closed_forms():
    for E, k in [(4, 1), (4, 2), (4, 4), (2, 2)]:
        w = wl(H_q=2 * E, H_kv=2, k=k)
        inp = W.make_inputs(w)
        r = oracle.route(oracle.desc(w), inp["x"], inp["w_router"])
        np.testing.assert_allclose(r["ptilde"].sum(-1), 1.0, rtol=0, atol=1e-15)
        p = r["probs"].reshape(-1, w.G, E)
        if k == 1:
            assert (r["ptilde"] == 1.0).all()
        if k == E:
            assert (r["sel"] == np.arange(E)).all()
            np.testing.assert_allclose(r["ptilde"], p, rtol=1e-15, atol=1e-16)
        # p~ = p[S] / sum p[S], with the softmax taken by torch
        s = inp["x"].double().reshape(-1, w.d_model) @ inp["w_router"].double().T
        pt = torch.softmax(s.view(-1, w.G, E), -1).gather(-1, torch.as_tensor(r["sel"]).long())
        pt = pt / pt.sum(-1, keepdim=True)
        np.testing.assert_allclose(r["ptilde"], pt.numpy(), rtol=1e-12)

# ---------------------------------------------------------------- step 5

def test_compaction_brute_force_and_invariants():
    w = wl(H_q=12, H_kv=3, k=2, B=3, T=50)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"])
    c = oracle.compact(d, r["sel"])
    BT = w.B * w.T
    buckets = {n: [] for n in range(w.N)}
    for t in range(BT):
        for g in range(w.G):
            for e in r["sel"][t, g]:
                buckets[g * w.E + int(e)].append(t)
    assert [len(buckets[n]) for n in range(w.N)] == c["counts"].tolist()
    assert c["offsets"][0] == 0 and c["offsets"][-1] == BT * w.G * w.k
    for n in range(w.N):
        seg = c["rows"][c["offsets"][n]:c["offsets"][n + 1]].tolist()
        assert seg == buckets[n]
        assert all(a < b for a, b in zip(seg, seg[1:]))
    for g in range(w.G):
        assert c["counts"][g * w.E:(g + 1) * w.E].sum() == BT * w.k

# ---------------------------------------------------------------- step 6

def test_routed_and_shared_projection_match_torch():
    w = wl(H_q=12, H_kv=3, k=2)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"])
    qr, qs = oracle.qproj_rows(d, inp["x"], inp["w_q"], r["sel"])
    qall = torch_q(w, inp).permute(0, 2, 1, 3).reshape(w.B * w.T, w.N + 1, w.d_head)  # [BT, H, dh]
    n = torch.as_tensor(r["sel"]).long() + (torch.arange(w.G) * w.E).view(1, w.G, 1)
    exp = qall.gather(1, n.reshape(-1, w.G * w.k, 1).expand(-1, -1, w.d_head)).reshape(-1, w.G, w.k, w.d_head)
    np.testing.assert_allclose(qr, exp.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(qs, qall[:, w.N].numpy(), rtol=1e-12, atol=1e-13)
    # a token subset gives the same rows
    tok = np.array([5, 0, 31, 57])
    qr2, qs2 = oracle.qproj_rows(d, inp["x"], inp["w_q"], r["sel"], tok)
    assert np.array_equal(qr2, qr[tok]) and np.array_equal(qs2, qs[tok])

# ---------------------------------------------------------------- step 7-8

def test_attention_given_queries_equals_prefill_rows_and_torch():
    """attend_rows (steps 7-8 from given query rows) is prefill_rows on the oracle's own projection, bit for
    bit, and on other queries (rounded ones) each hard and shared slot is torch's causal attention of that query."""
    w = wl(H_q=12, H_kv=3, k=2, route_mode=1)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"])
    tok = np.array([0, 3, 28, 29, 57, 40])
    qr, qs = oracle.qproj_rows(d, inp["x"], inp["w_q"], r["sel"], tok)
    ref = oracle.prefill_rows(d, inp["x"], inp["w_q"], inp["k"], inp["v"], r["sel"], r["ptilde"], tok)
    assert np.array_equal(oracle.attend_rows(d, qr, qs, inp["k"], inp["v"], r["ptilde"], tok), ref)
    qr2, qs2 = np.round(qr * 8) / 8, np.round(qs * 8) / 8
    got = oracle.attend_rows(d, qr2, qs2, inp["k"], inp["v"], r["ptilde"], tok)
    K, V = inp["k"].double(), inp["v"].double()
    for i, t in enumerate(tok):
        b, tt = divmod(int(t), w.T)
        def att(q, h):
            sc = (torch.as_tensor(q) @ K[b, h, : tt + 1].T) / np.sqrt(w.d_head)
            return (torch.softmax(sc, -1) @ V[b, h, : tt + 1]).numpy()
        for g in range(w.G):
            for j in range(w.k):
                np.testing.assert_allclose(got[i, g * w.k + j], att(qr2[i, g, j], g), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got[i, -1], att(qs2[i], 0), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("route_mode", [0, 1])
def test_all_experts_kept_is_dense_gqa(causal, route_mode):
    """k = E: hard slots are GQA (repeat_interleave + SDPA), weighted slot is sum p*o."""
    w = wl(H_q=8, H_kv=2, k=4, causal=causal, route_mode=route_mode, n_shared=1)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    res = oracle.prefill(d, inp)
    q = torch_q(w, inp)
    kx = inp["k"].double().repeat_interleave(w.E, dim=1)
    vx = inp["v"].double().repeat_interleave(w.E, dim=1)
    dense = torch_sdpa(q[:, :w.N], kx, vx, causal)                  # [B, H_q, T, dh]
    dense = dense.permute(0, 2, 1, 3).reshape(w.B * w.T, w.N, w.d_head)
    out = res["out"]
    np.testing.assert_allclose(out[:, :w.N], dense.numpy(), rtol=1e-10, atol=1e-12)
    s = inp["x"].double().reshape(-1, w.d_model) @ inp["w_router"].double().T
    p = torch.softmax(s.view(-1, w.G, w.E), -1)                      # [BT, G, E]
    per_group = (p.unsqueeze(-1) * dense.view(-1, w.G, w.E, w.d_head)).sum(2)   # [BT, G, dh]
    if route_mode == 0:
        np.testing.assert_allclose(out[:, w.N], per_group.sum(1).numpy(), rtol=1e-10, atol=1e-12)
    else:
        np.testing.assert_allclose(out[:, w.N:w.N + w.G], per_group.numpy(), rtol=1e-10, atol=1e-12)
    shared = torch_sdpa(q[:, w.N:w.N + 1], inp["k"].double()[:, :1], inp["v"].double()[:, :1], causal)
    np.testing.assert_allclose(out[:, -1], shared[:, 0].reshape(-1, w.d_head).numpy(), rtol=1e-10, atol=1e-12)

def test_one_query_head_per_group_is_mha_and_one_group_is_mqa():
    # E = 1 (H_kv = H_q): multi-head attention, every head kept, p~ = 1.
    w = wl(H_q=4, H_kv=4, k=1)
    inp = W.make_inputs(w)
    out = oracle.prefill(oracle.desc(w), inp)["out"]
    mha = torch_sdpa(torch_q(w, inp)[:, :4], inp["k"].double(), inp["v"].double(), 1)
    mha = mha.permute(0, 2, 1, 3).reshape(-1, 4, w.d_head)
    np.testing.assert_allclose(out[:, :4], mha.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out[:, 4], mha.sum(1).numpy(), rtol=1e-10, atol=1e-12)
    # G = 1 (H_kv = 1), all kept: multi-query attention.
    w = wl(H_q=4, H_kv=1, k=4)
    inp = W.make_inputs(w)
    out = oracle.prefill(oracle.desc(w), inp)["out"]
    mqa = torch_sdpa(torch_q(w, inp)[:, :4], inp["k"].double().expand(-1, 4, -1, -1),
                     inp["v"].double().expand(-1, 4, -1, -1), 1)
    np.testing.assert_allclose(out[:, :4], mqa.permute(0, 2, 1, 3).reshape(-1, 4, w.d_head).numpy(),
                               rtol=1e-10, atol=1e-12)

def test_causal_prefix_invariance():
    w = wl(H_q=8, H_kv=2, k=2, T=40)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    a = oracle.prefill(d, inp)
    cut = 23
    pert = dict(inp)
    g = torch.Generator().manual_seed(99)
    for key in ("x",):
        t = inp[key].clone(); t[:, cut:] = torch.randn(t[:, cut:].shape, generator=g); pert[key] = t
    for key in ("k", "v"):
        t = inp[key].clone(); t[:, :, cut:] = torch.randn(t[:, :, cut:].shape, generator=g); pert[key] = t
    b = oracle.prefill(d, pert)
    keep = np.array([bb * w.T + t for bb in range(w.B) for t in range(cut)])
    assert np.array_equal(a["out"][keep], b["out"][keep])
    assert np.array_equal(a["sel"][keep], b["sel"][keep])
    later = np.array([bb * w.T + t for bb in range(w.B) for t in range(cut, w.T)])
    assert not np.allclose(a["out"][later], b["out"][later])

def test_attention_closed_forms():
    w = wl(H_q=6, H_kv=3, k=2, T=17)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    hard = slice(0, w.G * w.k)
    # position 0 attends only itself: o = v_0 exactly
    out = oracle.prefill(d, inp)["out"].reshape(w.B, w.T, -1, w.d_head)
    for b in range(w.B):
        for g in range(w.G):
            for j in range(w.k):
                assert np.array_equal(out[b, 0, g * w.k + j], inp["v"][b, g, 0].double().numpy())
        assert np.array_equal(out[b, 0, -1], inp["v"][b, 0, 0].double().numpy())
    # constant V gives that constant everywhere
    c = torch.randn(w.d_head, dtype=torch.float64)
    cst = dict(inp, v=c.expand_as(inp["v"]).clone())
    out = oracle.prefill(d, cst)["out"]
    np.testing.assert_allclose(out[:, hard], np.broadcast_to(c.numpy(), out[:, hard].shape), rtol=1e-13, atol=1e-14)
    # zero keys: uniform weights, o_t = mean_{s<=t} v_s
    zk = dict(inp, k=torch.zeros_like(inp["k"]))
    out = oracle.prefill(d, zk)["out"].reshape(w.B, w.T, -1, w.d_head)
    mean = torch.cumsum(inp["v"].double(), 2) / torch.arange(1, w.T + 1, dtype=torch.float64).view(1, 1, -1, 1)
    for g in range(w.G):
        for j in range(w.k):
            np.testing.assert_allclose(out[:, :, g * w.k + j], mean[:, g].numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out[:, :, -1], mean[:, 0].numpy(), rtol=1e-12, atol=1e-13)

def test_shared_slot_is_single_head_attention_on_kv0_and_ignores_router():
    w = wl(H_q=8, H_kv=4, k=1)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    a = oracle.prefill(d, inp)["out"]
    q = torch_q(w, inp)[:, w.N:w.N + 1]
    ref = torch_sdpa(q, inp["k"].double()[:, :1], inp["v"].double()[:, :1], 1)[:, 0].reshape(-1, w.d_head)
    np.testing.assert_allclose(a[:, -1], ref.numpy(), rtol=1e-10, atol=1e-12)
    other = dict(inp, w_router=torch.randn(inp["w_router"].shape))
    b = oracle.prefill(d, other)["out"]
    assert np.array_equal(a[:, -1], b[:, -1])

def test_top1_weighted_slot_is_sum_of_hard_slots():
    w = wl(H_q=8, H_kv=4, k=1)
    inp = W.make_inputs(w)
    out = oracle.prefill(oracle.desc(w), inp)["out"]
    acc = np.zeros_like(out[:, 0])
    for g in range(w.G):
        acc = acc + out[:, g]
    assert np.array_equal(out[:, w.G], acc)
    # one group, top-1: the weighted slot is exactly the single selected output
    w1 = wl(H_q=3, H_kv=1, k=1)
    inp1 = W.make_inputs(w1)
    out1 = oracle.prefill(oracle.desc(w1), inp1)["out"]
    assert np.array_equal(out1[:, 0], out1[:, 1])
    # per-group weighted slots with top-1 equal the hard slots bit for bit
    wm = w.replace(route_mode=1)
    outm = oracle.prefill(oracle.desc(wm), inp)["out"]
    assert np.array_equal(outm[:, w.G:2 * w.G], outm[:, :w.G])

def test_hard_concat_only_drops_the_weighted_slot():
    # route mode 2 ("hard concat only", [note] §5-1 ablation table): the same hard and shared slots,
    # bit for bit, and no weighted slot in between
    w = wl(H_q=12, H_kv=3, k=2)
    inp = W.make_inputs(w)
    a = oracle.prefill(oracle.desc(w), inp)["out"]
    d2 = oracle.desc(w.replace(route_mode=2))
    b = oracle.prefill(d2, inp)["out"]
    kG = w.G * w.k
    assert oracle.num_slots(d2) == kG + 1 and b.shape[1] == kG + 1
    assert np.array_equal(b[:, :kG], a[:, :kG]) and np.array_equal(b[:, kG], a[:, kG + 1])

@pytest.mark.parametrize("k", [1, 2, 4])
def test_weighted_concat_scales_each_hard_slot_by_its_group_softmax(k):
    """Route mode 3 (the "weighted concat, no renormalized slot" row of [note] §5-1, read as each hard slot times
    its kept expert's group softmax probability, no weighted-sum slot): the probabilities are torch's softmax of
    the oracle's router scores over each group's E experts (not renormalised over the kept k), the head outputs
    are mode 2's hard slots, and the slots of a group sum to (sum of the kept p) times mode 1's per-group
    weighted slot, whose weights are renormalised."""
    w = wl(H_q=12, H_kv=3, k=k, zipf_s=1.2)
    inp = W.make_inputs(w)
    d3 = oracle.desc(w.replace(route_mode=3))
    kG = w.G * k
    assert oracle.num_slots(d3) == kG + 1
    r3 = oracle.prefill(d3, inp)
    out3 = r3["out"]
    logits = torch.from_numpy(oracle.route(oracle.desc(w), inp["x"], inp["w_router"], inp["b_router"])["logits"])
    p = torch.softmax(logits.reshape(-1, w.G, w.E), dim=-1).numpy()
    p_kept = np.take_along_axis(p, r3["sel"].astype(np.int64), -1)            # [BT, G, k]
    np.testing.assert_allclose(r3["ptilde"], p_kept, rtol=1e-13, atol=1e-15)
    out2 = oracle.prefill(oracle.desc(w.replace(route_mode=2)), inp)["out"]
    np.testing.assert_allclose(out3[:, :kG], out2[:, :kG] * p_kept.reshape(-1, kG, 1), rtol=1e-13, atol=1e-15)
    assert np.array_equal(out3[:, kG], out2[:, kG])                          # the shared slot, unchanged
    out1 = oracle.prefill(oracle.desc(w.replace(route_mode=1)), inp)["out"]
    grp = out3[:, :kG].reshape(-1, w.G, k, w.d_head).sum(axis=2)
    want = out1[:, kG:kG + w.G] * p_kept.sum(-1)[..., None]
    np.testing.assert_allclose(grp, want, rtol=1e-12, atol=1e-14)
    if k == w.E:   # every expert kept: the kept probabilities sum to 1, so the sum is the weighted slot itself
        np.testing.assert_allclose(grp, out1[:, kG:kG + w.G], rtol=1e-12, atol=1e-14)


def test_weighted_concat_invariances():
    """Mode 3 with one expert per group keeps the hard slot (p = 1), and a constant added to every score of a
    group (a uniform router bias) changes no slot: the weights are a softmax over the group."""
    w1 = wl(H_q=3, H_kv=3, k=1)
    inp1 = W.make_inputs(w1)
    a = oracle.prefill(oracle.desc(w1.replace(route_mode=3)), inp1)["out"]
    b = oracle.prefill(oracle.desc(w1.replace(route_mode=2)), inp1)["out"]
    assert np.array_equal(a, b)
    w = wl(H_q=12, H_kv=3, k=2)
    inp = W.make_inputs(w)
    d3 = oracle.desc(w.replace(route_mode=3))
    base = oracle.prefill(d3, inp)["out"]
    shifted = dict(inp, b_router=torch.tensor([1.7] * 4 + [-0.9] * 4 + [3.1] * 4, dtype=torch.float32))
    np.testing.assert_allclose(oracle.prefill(d3, shifted)["out"], base, rtol=1e-12, atol=1e-14)


def test_permuting_experts_inside_a_group_keeps_weighted_and_shared_slots():
    w = wl(H_q=12, H_kv=3, k=2)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    a = oracle.prefill(d, inp)["out"]
    perm = torch.cat([g * w.E + torch.tensor([2, 0, 3, 1]) for g in range(w.G)])
    q_perm = torch.cat([perm, torch.tensor([w.N])])
    b = oracle.prefill(d, dict(inp, w_router=inp["w_router"][perm], w_q=inp["w_q"][q_perm]))["out"]
    np.testing.assert_allclose(a[:, w.G * w.k:], b[:, w.G * w.k:], rtol=1e-12, atol=1e-14)
    for g in range(w.G):   # hard slots of a group are the same set of vectors
        sa = np.sort(a[:, g * w.k:(g + 1) * w.k], axis=1)
        sb = np.sort(b[:, g * w.k:(g + 1) * w.k], axis=1)
        np.testing.assert_allclose(sa, sb, rtol=1e-12, atol=1e-14)

# ---------------------------------------------------------------- K / V projection

def test_kv_projection_closed_form_and_torch():
    # [tut] step 2: x projected to K and V, split into H_kv heads of d_head
    w = wl(B=2, T=11, d_model=8, d_head=8, H_q=6, H_kv=3)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    x = inp["x"].reshape(-1, w.d_model)
    # scaled identities: head h of K is (h + 1) * x exactly
    eye = torch.stack([torch.eye(8, dtype=torch.float64) * (h + 1) for h in range(3)])
    k = oracle.kv_proj(d, x, eye)
    for h in range(3):
        assert np.array_equal(k[:, h], (h + 1) * inp["x"].double().numpy())
    # a general W (d_model != d_head, so a transposed operand cannot pass) against torch, head h at [:, h]
    w2 = wl(B=2, T=11, d_model=24, d_head=8, H_q=6, H_kv=3)
    inp2 = W.make_inputs(w2)
    wk = torch.randn(3, 8, 24, dtype=torch.float64, generator=torch.Generator().manual_seed(4))
    got = oracle.kv_proj(oracle.desc(w2), inp2["x"], wk)
    ref = torch.einsum("btm,hdm->bhtd", inp2["x"].double(), wk)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)

# ---------------------------------------------------------------- output projection

@pytest.mark.parametrize("route_mode", [0, 1])
def test_assemble_rows_restores_the_weighted_slots(route_mode):
    # given the hard and shared slots of the prefill rows path, the weighted
    # slot(s) come back bit for bit, and equal p~-weighted sums of the hard slots
    w = wl(H_q=12, H_kv=3, k=2, route_mode=route_mode)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    ref = oracle.prefill(d, inp)
    out = ref["out"]
    G, k, dh = w.G, w.k, w.d_head
    nr = G if route_mode else 1
    garbled = out.copy()
    garbled[:, G * k:G * k + nr] = np.nan
    got = oracle.assemble_rows(d, garbled, ref["ptilde"])
    assert np.array_equal(got, out)
    hard = out[:, :G * k].reshape(-1, G, k, dh)
    per_group = np.einsum("tgj,tgjd->tgd", ref["ptilde"], hard)
    want = per_group if route_mode else per_group.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(got[:, G * k:G * k + nr], want, rtol=1e-12, atol=1e-15)

def test_output_projection_closed_forms_and_torch():
    # [tut] step 5 / [note] §3-2 (5), (7): y = concat(slots) W_o^T over S*d_head inputs
    w = wl(H_q=6, H_kv=3, k=1)                       # S = 3 hard + 1 weighted + 1 shared = 5
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    h = oracle.prefill(d, inp)["out"]
    n, S, dh = h.shape
    width = S * dh
    flat = h.reshape(n, width)
    # identity: d_model = S*d_head, W_o = I gives the concatenation back exactly
    di = oracle.desc(w, d_model=width)
    assert np.array_equal(oracle.out_proj_rows(di, h, np.eye(width)), flat)
    # a permutation matrix picks slot entries: output c is input perm[c]
    perm = np.random.default_rng(3).permutation(width)
    assert np.array_equal(oracle.out_proj_rows(di, h, np.eye(width)[perm]), flat[:, perm])
    # a block selector returns one slot (here the shared one, slot S-1)
    sel_blk = np.zeros((dh, width)); sel_blk[:, (S - 1) * dh:] = np.eye(dh)
    assert np.array_equal(oracle.out_proj_rows(oracle.desc(w, d_model=dh), h, sel_blk), h[:, S - 1])
    # a general W_o (d_model != width, so a transposed operand cannot pass) against torch
    wo = torch.randn(w.d_model, width, dtype=torch.float64, generator=torch.Generator().manual_seed(5))
    y = oracle.out_proj_rows(d, h, wo)
    ref = torch.from_numpy(flat) @ wo.T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)
    # per-group weighted slots widen the input to S = kG + G + 1
    wm = w.replace(route_mode=1)
    dm = oracle.desc(wm)
    hm = oracle.prefill(dm, inp)["out"]
    wom = torch.randn(w.d_model, hm.shape[1] * dh, dtype=torch.float64, generator=torch.Generator().manual_seed(6))
    np.testing.assert_allclose(oracle.out_proj_rows(dm, hm, wom), (torch.from_numpy(hm.reshape(n, -1)) @ wom.T).numpy(),
                               rtol=1e-12, atol=1e-13)

# ---------------------------------------------------------------- rotary embedding (next-step row, reading)

def test_rotary_embedding_pins():
    """oracle.rope (the RoFormer rotary embedding with rotate-half pairing; the pages give no positional
    encoding, so the form is a reading) against numpy's complex exponential, and its invariants: position 0
    is the identity, each pair keeps its norm, pair 0 turns by the position in radians, rotations compose by
    adding positions, and a score of a rotated query and key depends only on their relative position."""
    rng = np.random.default_rng(3)
    dh, base = 16, 10000.0
    x = rng.standard_normal((6, dh))
    pos = np.array([0, 1, 5, 100, 4095, 32767])
    y = oracle.rope(x, pos, base)
    freq = base ** (-2.0 * np.arange(dh // 2) / dh)
    z = (x[:, :dh // 2] + 1j * x[:, dh // 2:]) * np.exp(1j * pos[:, None] * freq[None, :])
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], axis=1), rtol=1e-12, atol=1e-12)
    assert np.array_equal(y[0], x[0])
    np.testing.assert_allclose(y[:, :8] ** 2 + y[:, 8:] ** 2, x[:, :8] ** 2 + x[:, 8:] ** 2, rtol=1e-12)
    e = np.zeros((1, dh)); e[0, 0] = 1.0
    r = oracle.rope(e, np.array([3]), base)
    assert abs(r[0, 0] - np.cos(3.0)) < 1e-15 and abs(r[0, dh // 2] - np.sin(3.0)) < 1e-15
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, np.full(6, 7), base), pos, base),
                               oracle.rope(x, pos + 7, base), rtol=1e-10, atol=1e-10)
    q, k = rng.standard_normal((1, dh)), rng.standard_normal((1, dh))
    for pq, pk, c in [(10, 3, 50), (0, 7, 1000), (300, 300, 12345)]:
        s1 = float((oracle.rope(q, [pq], base) * oracle.rope(k, [pk], base)).sum())
        s2 = float((oracle.rope(q, [pq + c], base) * oracle.rope(k, [pk + c], base)).sum())
        assert abs(s1 - s2) < 1e-10 * (np.abs(q).sum() * np.abs(k).sum())

# ---------------------------------------------------------------- decode

def test_decode_equals_last_prefill_row():
    w = wl(H_q=8, H_kv=2, k=1, B=3, T=20)
    inp = W.make_inputs(w)
    lens = np.array([20, 1, 13], dtype=np.int32)
    d = oracle.desc(w)
    full = oracle.route(d, inp["x"], inp["w_router"])
    tok = np.array([b * w.T + lens[b] - 1 for b in range(w.B)])
    ref = oracle.prefill_rows(d, inp["x"], inp["w_q"], inp["k"], inp["v"], full["sel"], full["ptilde"], tok)
    xs = inp["x"][torch.arange(w.B), torch.as_tensor(lens - 1).long()]
    kc, vc = inp["k"].clone(), inp["v"].clone()
    for b in range(w.B):       # positions past the length must never be read
        kc[b, :, lens[b]:] = float("nan"); vc[b, :, lens[b]:] = float("nan")
    dd = oracle.desc(w, T=1)
    dec = oracle.decode(dd, xs, inp["w_router"], None, inp["w_q"], kc, vc, lens)
    assert np.array_equal(dec["out"], ref)
    assert np.array_equal(dec["sel"], full["sel"][tok])
    # a one-entry cache returns v_0
    assert np.array_equal(dec["out"][1, 0], inp["v"][1, 0, 0].double().numpy())


def test_decode_with_a_given_selection_equals_that_prefill_row():
    """decode(routing=...) attends with the selection it is given: with another valid selection (the
    next expert after the one the oracle kept, k = 1 of E = 4) it equals the prefill rows of that selection at each
    sequence's last position, and with its own routing it repeats its plain result bit for bit."""
    w = wl(H_q=8, H_kv=2, k=1, B=3, T=20)
    inp = W.make_inputs(w)
    lens = np.array([20, 1, 13], dtype=np.int32)
    d = oracle.desc(w)
    full = oracle.route(d, inp["x"], inp["w_router"])
    tok = np.array([b * w.T + lens[b] - 1 for b in range(w.B)])
    other = ((full["sel"] + 1) % w.E).astype(np.int32)           # an expert not kept, in each group
    pt_other = np.ones_like(full["ptilde"])
    ref = oracle.prefill_rows(d, inp["x"], inp["w_q"], inp["k"], inp["v"], other, pt_other, tok)
    xs = inp["x"][torch.arange(w.B), torch.as_tensor(lens - 1).long()]
    dd = oracle.desc(w, T=1)
    dec = oracle.decode(dd, xs, inp["w_router"], None, inp["w_q"], inp["k"], inp["v"], lens,
                        routing=dict(sel=other[tok], ptilde=pt_other[tok]))
    assert np.array_equal(dec["out"], ref)
    assert np.array_equal(dec["sel"], full["sel"][tok])          # the reported routing is still its own
    plain = oracle.decode(dd, xs, inp["w_router"], None, inp["w_q"], inp["k"], inp["v"], lens)
    own = oracle.decode(dd, xs, inp["w_router"], None, inp["w_q"], inp["k"], inp["v"], lens,
                        routing=dict(sel=plain["sel"], ptilde=plain["ptilde"]))
    assert np.array_equal(own["out"], plain["out"])
    assert not np.allclose(dec["out"][:, :w.k * w.G], plain["out"][:, :w.k * w.G])

# ---------------------------------------------------------------- printed counts

def test_main_setting_counts_from_the_study_note():
    g = json.load(open(os.path.join(HERE, "golden", "main_setting.json")))
    w = W.WORKLOADS["main_250m"]
    assert (w.H_q, w.H_kv, w.k, w.n_shared) == (g["H_q"], g["H_kv"], g["k"], g["n_shared"])
    small = w.replace(B=1, T=5, d_model=16, d_head=8, dtype="f32", act_std=1.0, w_std=0.3)
    d = oracle.desc(small)
    assert oracle.num_slots(d) == g["output_slots"] == g["hard_slots"] + g["weighted_sum_slots"] + g["shared_slots"]
    assert oracle.num_slots(oracle.desc(W.dense_variant(small), n_shared=0, route_mode=0)) - 1 == g["dense_output_slots"]
    inp = W.make_inputs(small)
    r = oracle.route(d, inp["x"], inp["w_router"])
    qr, qs = oracle.qproj_rows(d, inp["x"], inp["w_q"], r["sel"])
    assert qs is not None and qs.shape[0] == small.T
    assert qr.shape[1] * qr.shape[2] == g["routed_active"]
    assert qr.shape[1] * qr.shape[2] + 1 == g["computed_query_attentions"]
    assert small.G * small.E == g["routed_pool"] and small.G == g["groups"] and small.E == g["experts_per_group"]
    c = oracle.compact(d, r["sel"])
    assert c["counts"].sum() == small.T * g["routed_active"]

# ---------------------------------------------------------------- backward through assembly and routing

from oracle.backward import route_assemble_backward  # noqa: E402


def _bwd_case(k, E=3, G=2, route_mode=0, seed=3):
    w = wl(B=1, T=4, d_model=5, H_q=G * E, H_kv=G, k=k, d_head=3, route_mode=route_mode, seed=seed)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"])
    rng = np.random.default_rng(seed)
    S = oracle.num_slots(d)
    hard = rng.standard_normal((w.B * w.T, G * k, w.d_head))
    dout = rng.standard_normal((w.B * w.T, S, w.d_head))
    return w, inp, r, hard, dout


def _loss(w, x, w_router, sel, hard, dout):
    """L = sum(dout * slots) with the slots assembled from p~ of the given selection (numpy, float64)."""
    G, k, E = w.H_kv, w.k, w.H_q // w.H_kv
    logits = x @ w_router.T
    p = np.exp(logits.reshape(-1, G, E) - logits.reshape(-1, G, E).max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    q = np.take_along_axis(p, sel.astype(np.int64), -1)
    pt = q / q.sum(-1, keepdims=True)
    kG = G * k
    L = (dout[:, :kG] * hard).sum()
    hg = hard.reshape(-1, G, k, hard.shape[-1])
    if w.route_mode == 0:
        L += (dout[:, kG] * (pt[..., None] * hg).sum((1, 2))).sum()
    elif w.route_mode == 1:
        L += (dout[:, kG:kG + G] * (pt[..., None] * hg).sum(2)).sum()
    return L


@pytest.mark.parametrize("route_mode", [0, 1])
def test_router_backward_matches_finite_differences(route_mode):
    w, inp, r, hard, dout = _bwd_case(k=2, route_mode=route_mode)
    x = inp["x"].double().numpy().reshape(-1, w.d_model)
    wr = inp["w_router"].double().numpy()
    g = route_assemble_backward(w, x, wr, None, r["sel"], hard, dout)
    h = 1e-6
    for n in range(wr.shape[0]):
        for c in range(wr.shape[1]):
            a, b = wr.copy(), wr.copy()
            a[n, c] += h; b[n, c] -= h
            fd = (_loss(w, x, a, r["sel"], hard, dout) - _loss(w, x, b, r["sel"], hard, dout)) / (2 * h)
            assert abs(fd - g["dw_router"][n, c]) <= 1e-6 * max(1.0, abs(fd))
    for t in range(x.shape[0]):
        for c in range(x.shape[1]):
            a, b = x.copy(), x.copy()
            a[t, c] += h; b[t, c] -= h
            fd = (_loss(w, a, wr, r["sel"], hard, dout) - _loss(w, b, wr, r["sel"], hard, dout)) / (2 * h)
            assert abs(fd - g["dx"][t, c]) <= 1e-6 * max(1.0, abs(fd))
    # the loss is linear in the hard slots: one probe per slot entry gives its gradient exactly
    e = np.zeros_like(hard); e[1, 2, 1] = 1.0
    assert np.isclose(_loss(w, x, wr, r["sel"], hard + e, dout) - _loss(w, x, wr, r["sel"], hard, dout),
                      g["d_hard"][1, 2, 1], rtol=1e-12, atol=1e-12)
    # p~ depends on a group's scores only through their differences: the score gradient sums to zero
    assert np.allclose(g["d_logits"].reshape(-1, w.G, w.E).sum(-1), 0.0, atol=1e-13)


def test_router_backward_closed_forms():
    # top-1: p~ = 1 whatever the scores, so the router gets no gradient and the hard slots get dout + dout_w
    w, inp, r, hard, dout = _bwd_case(k=1)
    x = inp["x"].double().numpy().reshape(-1, w.d_model)
    g = route_assemble_backward(w, x, inp["w_router"], None, r["sel"], hard, dout)
    assert not g["d_logits"].any() and not g["dw_router"].any() and not g["dx"].any()
    kG = w.G * w.k
    assert np.array_equal(g["d_hard"], dout[:, :kG] + dout[:, kG:kG + 1])
    # no weighted slot (route mode 2): no learning signal reaches the router ([note] §3-2 (4))
    w2, inp2, r2, hard2, dout2 = _bwd_case(k=2, route_mode=2)
    g2 = route_assemble_backward(w2, inp2["x"], inp2["w_router"], None, r2["sel"], hard2, dout2)
    assert not g2["d_logits"].any() and np.array_equal(g2["d_hard"], dout2[:, :w2.G * w2.k])
    # all experts kept: p~ = p, so d s_e = p_e (g_e - sum_e' p_e' g_e') with g_e = <dout_w, o_e>
    w3, inp3, r3, hard3, dout3 = _bwd_case(k=3, E=3)
    g3 = route_assemble_backward(w3, inp3["x"], inp3["w_router"], None, r3["sel"], hard3, dout3)
    kG3 = w3.G * w3.k
    ge = np.einsum("td,thd->th", dout3[:, kG3], hard3).reshape(-1, w3.G, 3)
    p = r3["probs"].reshape(-1, w3.G, 3)
    want = p * (ge - (p * ge).sum(-1, keepdims=True))
    np.testing.assert_allclose(g3["d_logits"].reshape(-1, w3.G, 3), want, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- attention backward (oracle/attn_backward.py)

from oracle.attn_backward import attention_backward, head_backward, row_lse2  # noqa: E402


def _attn_bwd_case(k=2, E=2, G=2, T=5, d=3, seed=11, causal=1):
    w = wl(B=1, T=T, d_model=4, H_q=G * E, H_kv=G, k=k, d_head=d, seed=seed, causal=causal)
    rng = np.random.default_rng(seed)
    n = w.B * w.T
    q_tok = rng.standard_normal((n, G, k, d))              # token-major, as attend_rows takes them
    q_sh = rng.standard_normal((n, d))
    K = rng.standard_normal((w.B, G, T, d))
    V = rng.standard_normal((w.B, G, T, d))
    S = G * k + 2
    dout = rng.standard_normal((n, S, d))
    return w, q_tok, q_sh, K, V, dout


def _q_routed(w, q_tok):
    """[B*T, G, k, d] token-major -> [B, G, T*k, d], row t*k + j."""
    G, k, d = q_tok.shape[1:]
    return q_tok.reshape(w.B, w.T, G, k, d).transpose(0, 2, 1, 3, 4).reshape(w.B, G, w.T * k, d)


def _attn_loss(w, q_tok, q_sh, K, V, dout):
    """sum over the hard and shared slots of dout * slot, the slots from the C oracle's forward."""
    d = oracle.desc(w)
    G, k = w.H_kv, w.k
    pt = np.full((w.B * w.T, G, k), 1.0 / k)
    out = oracle.attend_rows(d, q_tok, q_sh, K, V, pt)
    kG = G * k
    return float((dout[:, :kG] * out[:, :kG]).sum() + (dout[:, -1] * out[:, -1]).sum())


@pytest.mark.parametrize("causal", [1, 0])
def test_attention_backward_matches_finite_differences_of_the_forward(causal):
    # the forward here is the C oracle's attention (pinned against SDPA above), the gradient is autograd
    w, q_tok, q_sh, K, V, dout = _attn_bwd_case(causal=causal)
    G, k = w.H_kv, w.k
    g = attention_backward(w, _q_routed(w, q_tok), q_sh.reshape(w.B, w.T, -1), K, V, dout[:, :G * k], dout)
    h = 1e-6

    def fd(arr, idx):
        a, b = arr.copy(), arr.copy()
        a[idx] += h
        b[idx] -= h
        args_a = [a if x is arr else x for x in (q_tok, q_sh, K, V)]
        args_b = [b if x is arr else x for x in (q_tok, q_sh, K, V)]
        return (_attn_loss(w, *args_a, dout) - _attn_loss(w, *args_b, dout)) / (2 * h)

    dq_tok = g["dq_routed"].reshape(w.B, G, w.T, k, -1).transpose(0, 2, 1, 3, 4).reshape(q_tok.shape)
    for arr, grad in ((q_tok, dq_tok), (q_sh, g["dq_shared"].reshape(q_sh.shape)), (K, g["dk"]), (V, g["dv"])):
        for idx in itertools.product(*[range(s) for s in arr.shape]):
            f = fd(arr, idx)
            assert abs(f - grad[idx]) <= 1e-6 * max(1.0, abs(f)), (idx, f, grad[idx])


def test_row_statistic_closed_forms():
    """row_lse2 against closed forms: with every score equal to c a row over n keys has log2(n) + c log2(e);
    its 2^(s log2(e) - lse) are the softmax of the row (they sum to one and equal torch's); shifting every
    key's score by a constant shifts lse by that constant times log2(e)."""
    rng = np.random.default_rng(7)
    d, T, kk = 16, 9, 2
    q = np.zeros((T * kk, d))
    q[:, 0] = 1.0
    K = np.zeros((T, d))
    K[:, 0] = 0.75 * np.sqrt(d)                       # every score q.K/sqrt(d) = 0.75
    lse = row_lse2(q, K, kk, causal=True)
    n = np.arange(T * kk) // kk + 1
    assert np.allclose(lse, np.log2(n) + 0.75 / np.log(2.0), rtol=0, atol=1e-12)
    assert np.allclose(row_lse2(q, K, kk, causal=False), np.log2(T) + 0.75 / np.log(2.0), rtol=0, atol=1e-12)
    q = rng.standard_normal((T * kk, d))
    K = rng.standard_normal((T, d))
    lse = row_lse2(q, K, kk, causal=True)
    S = q @ K.T / np.sqrt(d)
    mask = np.arange(T)[None, :] > (np.arange(T * kk) // kk)[:, None]
    P = np.where(mask, 0.0, np.exp2(S / np.log(2.0) - lse[:, None]))
    assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    ref = torch.softmax(torch.from_numpy(np.where(mask, -np.inf, S)), dim=-1).numpy()
    assert np.allclose(P, ref, rtol=0, atol=1e-12)
    u = rng.standard_normal(d)
    shift = (q @ u) / np.sqrt(d)                      # K_s + u moves every score of row r by q_r.u/sqrt(d)
    assert np.allclose(row_lse2(q, K + u, kk, causal=True) - lse, shift / np.log(2.0), rtol=0, atol=1e-10)


def test_attention_backward_single_key():
    # one key: P = 1 whatever the scores, so no gradient reaches q or K, and V gets the sum of the rows' dO
    rng = np.random.default_rng(1)
    q, K, V, dO = rng.standard_normal((3, 4)), rng.standard_normal((1, 4)), rng.standard_normal((1, 4)), \
        rng.standard_normal((3, 4))
    r = head_backward(q, K, V, dO, kk=3)
    assert not r["dq"].any() and not r["dk"].any()
    np.testing.assert_allclose(r["dv"][0], dO.sum(0), rtol=1e-14)


@pytest.mark.parametrize("kk", [1, 2])
def test_attention_backward_uniform_scores_closed_form(kk):
    # q = 0: row r (position t = r // kk) weights keys 0..t equally, so
    #   dv_s = sum over rows with t >= s of dO_r / (t + 1),
    #   dq_r = (1/sqrt(d)) (1/(t+1)) sum_s (g_rs - mean_s g_rs) k_s,  g_rs = dO_r . v_s,   dk = 0
    rng = np.random.default_rng(2)
    T, d = 6, 5
    R = T * kk
    q = np.zeros((R, d))
    K, V, dO = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((R, d))
    r = head_backward(q, K, V, dO, kk)
    dv = np.zeros((T, d))
    dq = np.zeros((R, d))
    for row in range(R):
        t = row // kk
        for s in range(t + 1):
            dv[s] += dO[row] / (t + 1)
        gr = np.array([dO[row] @ V[s] for s in range(t + 1)])
        for s in range(t + 1):
            dq[row] += (gr[s] - gr.mean()) * K[s] / (t + 1) / np.sqrt(d)
    np.testing.assert_allclose(r["dv"], dv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dq"], dq, rtol=1e-12, atol=1e-14)
    assert np.abs(r["dk"]).max() < 1e-14


@pytest.mark.parametrize("causal", [1, 0])
def test_attention_backward_all_experts_equals_dense_gqa(causal):
    # k = E: the routed rows are every query head of the group, so the gradients are those of dense GQA,
    # here by torch's SDPA autograd on K/V repeated over each group's heads (GQA tutorial code listing)
    w, q_tok, q_sh, K, V, dout = _attn_bwd_case(k=3, E=3, G=2, T=7, d=4, causal=causal)
    G, E, T, d = w.H_kv, 3, w.T, w.d_head
    g = attention_backward(w, _q_routed(w, q_tok), q_sh.reshape(1, T, d), K, V, dout[:, :G * E], dout)
    qd = torch.tensor(q_tok.reshape(T, G * E, d).transpose(1, 0, 2)[None], requires_grad=True)   # [1, H, T, d]
    qs = torch.tensor(q_sh[None, None], requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    o = torch_sdpa(qd, Kt.repeat_interleave(E, dim=1), Vt.repeat_interleave(E, dim=1), causal)
    os_ = torch_sdpa(qs, Kt[:, :1], Vt[:, :1], causal)
    dO = torch.tensor(dout[:, :G * E].reshape(T, G * E, d).transpose(1, 0, 2)[None])
    ((o * dO).sum() + (os_ * torch.tensor(dout[:, -1][None, None])).sum()).backward()
    dq_dense = qd.grad.numpy()[0].transpose(1, 0, 2).reshape(T, G, E, d)     # [T, G, E, d]
    want_routed = dq_dense.transpose(1, 0, 2, 3).reshape(1, G, T * E, d)
    np.testing.assert_allclose(g["dq_routed"], want_routed, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dq_shared"], qs.grad.numpy()[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk"], Kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dv"], Vt.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- expert load statistics


@pytest.mark.parametrize("zipf", [0.0, 1.2])
def test_expert_importance(zipf):
    w = wl(H_q=12, H_kv=3, k=2, zipf_s=zipf)
    inp = W.make_inputs(w)
    d = oracle.desc(w)
    r = oracle.route(d, inp["x"], inp["w_router"], inp["b_router"])
    imp = oracle.expert_importance(d, r["probs"])
    BT, G, E = w.B * w.T, w.H_kv, w.H_q // w.H_kv
    # every token spreads probability 1 over each group's experts
    np.testing.assert_allclose(imp.reshape(G, E).sum(-1), BT, rtol=1e-12)
    # torch: softmax of the oracle's scores within each group, summed over tokens
    lg = torch.tensor(r["logits"]).reshape(BT, G, E)
    np.testing.assert_allclose(imp, torch.softmax(lg, -1).reshape(BT, -1).sum(0).numpy(), rtol=1e-12)
    # a zero router spreads it evenly
    r0 = oracle.route(d, inp["x"], np.zeros_like(inp["w_router"].double().numpy()))
    np.testing.assert_allclose(oracle.expert_importance(d, r0["probs"]), BT / E, rtol=1e-12)


# ---------------------------------------------------------------- projections' backward (next-step row)

def _proj_case(rope_base, k=1, H_q=6, H_kv=3):
    from oracle.proj_backward import qkv_proj_backward
    w = wl(H_q=H_q, H_kv=H_kv, k=k, B=2, T=5, d_model=8, d_head=4)
    inp = W.make_inputs(w)
    wk, wv = W.make_w_kv(w)
    sel = oracle.route(oracle.desc(w), inp["x"], inp["w_router"])["sel"]
    rng = np.random.default_rng(11)
    B, T, G, D = w.B, w.T, w.G, w.d_head
    dqr = rng.standard_normal((B, G, T * w.k, D))
    dqs = rng.standard_normal((B, T, D))
    dk, dv = rng.standard_normal((B, G, T, D)), rng.standard_normal((B, G, T, D))
    pos = rng.integers(0, 50, B * T)
    x, wq = inp["x"].double().numpy().reshape(B * T, -1), inp["w_q"].double().numpy()
    wkn, wvn = wk.double().numpy(), wv.double().numpy()
    g = qkv_proj_backward(w, x, wq, wkn, wvn, sel, dqr, dqs, dk, dv, pos, rope_base)
    d = oracle.desc(w)

    def loss(x_, wq_, wk_, wv_):
        # the forward through the C oracle's projections and its rotation
        qr, qs = oracle.qproj_rows(d, x_, wq_, sel)                    # [BT, G, k, D], [BT, D]
        K = oracle.kv_proj(d, x_, wk_)                                  # [B, H, T, D]
        V = oracle.kv_proj(d, x_, wv_)
        if rope_base:
            qr = oracle.rope(qr, pos, rope_base)
            qs = oracle.rope(qs, pos, rope_base)
            K = oracle.rope(K, np.broadcast_to(pos.reshape(B, 1, T), K.shape[:-1]), rope_base)
        dq_tok = dqr.reshape(B, G, T, w.k, D).transpose(0, 2, 1, 3, 4).reshape(B * T, G, w.k, D)
        return float((qr * dq_tok).sum() + (qs * dqs.reshape(B * T, D)).sum() + (K * dk).sum() + (V * dv).sum())

    return w, sel, x, wq, wkn, wvn, g, loss


@pytest.mark.parametrize("rope_base", [0.0, 100.0])
def test_projection_backward_matches_finite_differences(rope_base):
    """oracle.proj_backward (fp64 autograd) against central differences of the loss through the C oracle's
    projections and rotation, for entries of x and of every weight; the loss is bilinear in (x, W), so the
    differences are exact up to rounding.  Experts no token kept get exactly zero weight gradient."""
    w, sel, x, wq, wk, wv, g, loss = _proj_case(rope_base)
    h = 1e-3
    args = [x, wq, wk, wv]
    for ai, name, idx in [(0, "dx", (3, 5)), (0, "dx", (9, 0)), (1, "dw_q", (0, 1, 2)), (1, "dw_q", (4, 3, 7)),
                          (1, "dw_q", (w.N, 2, 6)), (2, "dw_k", (1, 0, 4)), (3, "dw_v", (2, 3, 1))]:
        plus = [a.copy() for a in args]; minus = [a.copy() for a in args]
        plus[ai][idx] += h; minus[ai][idx] -= h
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        assert abs(fd - g[name][idx]) <= 1e-9 * max(1.0, abs(fd)), (name, idx, fd, g[name][idx])
    kept = np.zeros(w.N, dtype=bool)
    kept[(np.arange(w.G)[None, :, None] * w.E + sel).reshape(-1)] = True
    for n in range(w.N):
        if not kept[n]:
            assert not g["dw_q"][n].any()


def test_projection_backward_all_experts_kept_is_a_plain_matmul():
    """With k = E every token keeps every expert and no rotation: dW_q[n] = dq_n^T X, dx = sum_n dq_n W_q[n]
    + the K/V terms, as plain matrix products (torch fp64)."""
    w, sel, x, wq, wk, wv, g, _ = _proj_case(0.0, k=2, H_q=6, H_kv=3)
    from oracle.proj_backward import qkv_proj_backward  # noqa: F401  (the case above already ran it)
    B, T, G, E, D = w.B, w.T, w.G, w.E, w.d_head
    rng = np.random.default_rng(11)
    dqr = rng.standard_normal((B, G, T * w.k, D))
    dqs = rng.standard_normal((B, T, D))
    dk, dv = rng.standard_normal((B, G, T, D)), rng.standard_normal((B, G, T, D))
    # with k = E the kept experts of a group, in ascending order, are all of them: j = e
    assert (np.sort(sel, axis=-1) == np.arange(E)).all()
    dq_tok = dqr.reshape(B, G, T, E, D).transpose(0, 2, 1, 3, 4).reshape(B * T, G * E, D)   # expert n = g E + e
    X = torch.from_numpy(x)
    for n in range(w.N):
        np.testing.assert_allclose(g["dw_q"][n], (torch.from_numpy(dq_tok[:, n]).T @ X).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw_q"][w.N], (torch.from_numpy(dqs.reshape(B * T, D)).T @ X).numpy(), rtol=1e-12,
                               atol=1e-12)
    dk_tok = dk.transpose(0, 2, 1, 3).reshape(B * T, G, D)
    dv_tok = dv.transpose(0, 2, 1, 3).reshape(B * T, G, D)
    dx = sum(dq_tok[:, n] @ wq[n] for n in range(w.N)) + dqs.reshape(B * T, D) @ wq[w.N]
    dx = dx + sum(dk_tok[:, h] @ wk[h] + dv_tok[:, h] @ wv[h] for h in range(G))
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-12, atol=1e-12)
