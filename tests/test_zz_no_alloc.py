"""gqe_attn_decode_noalloc (the decode call that keeps its split partials in the library's static device
scratch instead of a caller's workspace) against gqe_attn_decode on the same inputs, through the C ABI.

Both calls run the same kernels, so the bar is bitwise equality.  The reference call gets a NaN-filled
workspace, so a read of a partial it did not write would show as NaN there; the no-alloc call runs right
after a larger one, so the scratch still holds that call's partials.
"""
import numpy as np
import pytest
import torch

import sparse_routed_query_amd.gqe as G
import workloads as W

pytestmark = pytest.mark.gpu


def decode_both(w, lens=None):
    inp = W.make_inputs(w, lens=lens)
    d = G.desc_from(w)
    dev = "cuda"
    x = inp["x"].reshape(w.B, w.d_model).to(dev)
    br = inp["b_router"].to(dev) if inp["b_router"] is not None else None
    r = G.route(d, x, inp["w_router"].to(dev), br)
    q = G.qproj(d, x, inp["w_q"].to(dev), r)
    kc, vc, ln = inp["k_cache"].to(dev), inp["v_cache"].to(dev), inp["lens"].to(dev)
    need = G.gqe_decode_workspace_bytes(d, w.L_max)
    assert need <= G.DECODE_SCRATCH_BYTES
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
    ref = torch.empty((w.B, d.S, w.d_head), dtype=torch.float32, device=dev)
    G.gqe_attn_decode(d, q["q_routed"], q["q_shared"], kc, vc, ln, r["p_tilde"], ref, ws)
    got = torch.full_like(ref, float("nan"))
    G.gqe_attn_decode_noalloc(d, q["q_routed"], q["q_shared"], kc, vc, ln, r["p_tilde"], got)
    torch.cuda.synchronize()
    print(f"[{w.name}] B={w.B} L_max={w.L_max} scratch used {need} of {G.DECODE_SCRATCH_BYTES} bytes", flush=True)
    return ref.cpu(), got.cpu()


def test_noalloc_decode_equals_the_workspace_call_twice_in_a_row():
    big = W.WORKLOADS["decode_b64"]                            # 5.9 MB of partials
    ref, got = decode_both(big)
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref)
    small = W.Workload("dec_small", B=5, T=1, d_model=128, H_q=8, H_kv=2, k=1, d_head=64, dtype="bf16", seed=21,
                       act_std=1.0, w_std=0.02, decode=True, L_lo=1, L_hi=700, L_max=700)
    lens = W.make_inputs(small)["lens"].clone()
    lens[0], lens[1] = 1, small.L_max
    ref2, got2 = decode_both(small, lens)                      # the scratch still holds the big call's partials
    assert torch.isfinite(ref2).all()
    assert torch.equal(got2, ref2)
    wide = small.replace(name="dec_small_k2_d128", H_q=12, H_kv=3, k=2, d_head=128, route_mode=1)
    ref3, got3 = decode_both(wide)
    assert torch.isfinite(ref3).all()
    assert torch.equal(got3, ref3)
