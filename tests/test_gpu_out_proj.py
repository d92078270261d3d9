"""GPU parity of the attention output projection fused with slot assembly (gqe_out_proj).

y_t = W_o h_t over the S concatenated slots (GQA tutorial, "GQA 核心原理与计算流程" step 5; GQE study
note §3-2 (5), (7)).  The GPU's own hard and shared slots are the input of both sides, so the
comparison isolates the projection: the oracle forms the weighted slot(s) in fp64 and projects in fp64;
the bound per element follows from bf16 rounding of the slots and fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_parity_util import check_out_proj, gpu_decode, gpu_out_proj, gpu_prefill, say
import sparse_routed_query_amd.gqe as G

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="op_small", B=2, T=300, d_model=128, H_q=8, H_kv=2, k=2, d_head=64, dtype="bf16", seed=21,
                act_std=1.0, w_std=0.02)
    base.update(kw)
    return W.Workload(**base)


def run_and_check(w, tok=None, packed=False):
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    wo = W.make_w_o(w)
    slots = gpu["out"].reshape(w.B * w.T, -1, w.d_head)
    y, after = gpu_out_proj(w, slots, gpu["p_tilde"], wo, packed=packed)
    # the weighted slot(s) written back are gqe_assemble's bits; the other slots are untouched
    assert torch.equal(after, slots)
    assert torch.isfinite(y).all()
    tok = np.arange(w.B * w.T) if tok is None else tok
    check_out_proj(w, slots, gpu["p_tilde"], wo, y, tok)
    return gpu, wo, slots, y


SHAPES = [
    small(),                                              # ragged token tile (600 = 4 x 128 + 88)
    small(d_model=320, name="ragged_cols"),               # a 64-wide last column tile
    small(d_head=32, name="d32"), small(d_head=128, name="d128"),
    small(route_mode=1, name="per_group_slots"),
    small(route_mode=2, name="hard_only"),
    small(route_mode=3, name="weighted_concat"),
    small(n_shared=0, name="no_shared"),
    small(H_q=16, H_kv=4, k=2, zipf_s=1.2, name="kG8"),
    small(H_q=4, H_kv=1, k=2, name="G1"),
    small(T=1, name="T1"),
    small(B=1, T=64, d_model=1024, name="d_model1024"),
    small(dtype="f32", T=100, d_model=96, name="f32"),
    small(dtype="f32", T=70, d_head=128, d_model=64, k=1, route_mode=1, name="f32_d128_mode1"),
]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: f"{w.name}-d{w.d_head}-{w.dtype}")
def test_out_proj_every_token(w):
    run_and_check(w)


@pytest.mark.parametrize("w", [x for x in SHAPES if x.dtype == "bf16"], ids=lambda w: f"{w.name}-d{w.d_head}")
def test_out_proj_packed_every_token(w):
    """The packed-weight call against the oracle at the same bound, its weighted-slot write-back equal to the
    plain call's bit for bit, and y within fp32 reordering of the plain call's."""
    gpu, wo, slots, y = run_and_check(w, packed=True)
    y2, after2 = gpu_out_proj(w, slots, gpu["p_tilde"], wo)
    _, after = gpu_out_proj(w, slots, gpu["p_tilde"], wo, packed=True)
    assert torch.equal(torch.nan_to_num(after, nan=7.0), torch.nan_to_num(after2, nan=7.0))
    rel = float((y - y2).norm() / max(float(y2.norm()), 1e-30))
    say(f"[{w.name}] packed vs plain: relative rms {rel:.2e}")
    assert rel <= 1e-5


def test_out_proj_pack_layout():
    """gqe_out_proj_pack writes W_o[64 ct + 32 cb + c][16 ks + 8 h + e] at
    ((ct K/16 + ks) 2 + cb) 512 + (32 h + c) 8 + e, the order the header defines."""
    w = small(d_model=192, name="pack_layout")
    d = G.desc_from(w)
    wo = W.make_w_o(w)
    got = G.out_proj_pack(d, wo.cuda()).cpu().reshape(-1)
    dm, K = wo.shape
    ref = wo.reshape(dm // 64, 2, 32, K // 16, 2, 8).permute(0, 3, 1, 4, 2, 5).reshape(-1)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_out_proj_packed_is_refused_where_it_has_no_form():
    wide = small(H_q=32, H_kv=8, k=2, d_head=128, name="wide_k")   # K = 18 * 128: a 64-token tile exceeds LDS
    assert G.gqe_out_proj_packed_bytes(G.desc_from(wide)) == 0
    assert G.gqe_out_proj_packed_bytes(G.desc_from(small(dtype="f32", name="f32"))) == 0
    with pytest.raises(G.GqeError):
        G.out_proj_pack(G.desc_from(wide), W.make_w_o(wide).cuda())


@pytest.mark.parametrize("packed", [False, True], ids=["plain", "packed"])
def test_out_proj_main_250m_sampled(packed):
    w = W.WORKLOADS["main_250m"]
    BT = w.B * w.T
    rng = np.random.default_rng(0)
    tok = np.unique(np.concatenate([np.arange(0, BT, BT // 256), rng.integers(0, BT, 128), [0, BT - 1]]))
    run_and_check(w, tok, packed=packed)


def test_out_proj_after_decode_and_without_write_back():
    w = W.WORKLOADS["decode_b64"]
    inp = W.make_inputs(w)
    dec = gpu_decode(w, inp)
    wo = W.make_w_o(w)
    slots = dec["out"].reshape(w.B, -1, w.d_head)
    y, after = gpu_out_proj(w, slots, dec["p_tilde"], wo)
    assert torch.equal(after, slots)
    check_out_proj(w, slots, dec["p_tilde"], wo, y, np.arange(w.B))
    # without write-back the slots stay as given (NaN where the weighted ones were) and y is the same bits
    y2, after2 = gpu_out_proj(w, slots, dec["p_tilde"], wo, write_weighted=False)
    assert torch.equal(y2, y)
    kG = w.k * w.G
    assert torch.isnan(after2[:, kG]).all()
    assert torch.equal(after2[:, :kG], slots[:, :kG]) and torch.equal(after2[:, kG + 1:], slots[:, kG + 1:])
    say(f"[{w.name}] out_proj after decode ok")


@pytest.mark.parametrize("w", [small(route_mode=1, name="combination_only"),
                               small(route_mode=1, n_shared=0, H_q=16, H_kv=4, k=2, name="combination_only_noshared")],
                         ids=lambda w: w.name)
def test_weighted_combination_only_output(w):
    # The ai-feeds summary's output: per group the router-weighted combination of its kept experts' outputs
    # (route mode 1's weighted slots), with no hard slots.  gqe_out_proj gives it when W_o's hard-slot
    # columns are zero.  Reference: that definition written out in fp64 from the GPU's hard and shared slots.
    inp = W.make_inputs(w)
    gpu = gpu_prefill(w, inp)
    wo = W.make_w_o(w).clone()
    kG, D, Gn, k = w.k * w.G, w.d_head, w.G, w.k
    wo[:, :kG * D] = 0
    y, _ = gpu_out_proj(w, gpu["out"], gpu["p_tilde"], wo)
    BT = w.B * w.T
    S = kG + Gn + w.n_shared
    h = gpu["out"].reshape(BT, S, D).double().numpy()
    pt = gpu["p_tilde"].reshape(BT, Gn, k).double().numpy()
    comb = (pt[..., None] * h[:, :kG].reshape(BT, Gn, k, D)).sum(2)            # [BT, G, d]
    wod = wo.double().numpy()
    ref = comb.reshape(BT, Gn * D) @ wod[:, kG * D:(kG + Gn) * D].T
    mag = (np.abs(pt[..., None]) * np.abs(h[:, :kG].reshape(BT, Gn, k, D))).sum(2).reshape(BT, -1) \
        @ np.abs(wod[:, kG * D:(kG + Gn) * D]).T
    if w.n_shared:
        ref = ref + h[:, S - 1] @ wod[:, (S - 1) * D:].T
        mag = mag + np.abs(h[:, S - 1]) @ np.abs(wod[:, (S - 1) * D:]).T
    eps = 2.0 ** -8 + (S * D + kG + 1) * 2.0 ** -24
    err = np.abs(y.double().numpy() - ref)
    r = float((err / (eps * mag + 1e-30)).max())
    say(f"[{w.name}] combination-only projection: max err/bound {r:.3f}")
    assert np.isfinite(y.numpy()).all() and r <= 1.0
