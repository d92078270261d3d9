"""CPU tests of the input generator and the benchmark's host-side contract (no GPU needed)."""
import math
import os
import subprocess
import sys

import torch

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_zipf_bias_is_log_zipf_pmf():
    # b_e = ln Zipf(e + 1; s = 1.2, n = 4): -1.2 ln(e + 1) - ln(sum_r r^-1.2)
    b = W.zipf_log_pmf(4, 1.2).double()
    h = sum(r ** -1.2 for r in range(1, 5))
    want = torch.tensor([-1.2 * math.log(e + 1) - math.log(h) for e in range(4)], dtype=torch.float64)
    assert torch.allclose(b, want, atol=1e-6)
    assert abs(float(torch.exp(b).sum()) - 1.0) < 1e-6            # a probability distribution
    # the same bias for every group of the wide workload
    inp = W.make_inputs(W.WORKLOADS["wide_zipf"].replace(B=1, T=4, d_model=64))
    assert torch.equal(inp["b_router"], W.zipf_log_pmf(4, 1.2).repeat(8))


def test_inputs_are_seeded_and_decode_tails_are_poisoned():
    w = W.WORKLOADS["decode_b64"].replace(B=3, L_lo=5, L_hi=9, L_max=12)
    a, b = W.make_inputs(w), W.make_inputs(w)
    for key in ("x", "w_router", "w_q", "k_cache", "v_cache", "lens"):
        assert torch.equal(a[key].nan_to_num(123.0), b[key].nan_to_num(123.0)), key
    for i, n in enumerate(a["lens"].tolist()):
        assert 5 <= n <= 9
        assert torch.isnan(a["k_cache"][i, :, n:]).all() and not torch.isnan(a["k_cache"][i, :, :n]).any()
        assert torch.isnan(a["v_cache"][i, :, n:]).all() and not torch.isnan(a["v_cache"][i, :, :n]).any()


def test_dense_variant_sees_the_same_routed_weights():
    w = W.WORKLOADS["long_32k"].replace(T=8)
    a, d = W.make_inputs(w), W.make_inputs(W.dense_variant(w))
    assert torch.equal(a["w_q"][: w.N], d["w_q"])
    assert torch.equal(a["k"], d["k"]) and torch.equal(a["x"], d["x"])


def test_flop_and_byte_accounting():
    w = W.WORKLOADS["main_250m"]
    assert W.attention_flops(w) == 4 * 64 * 4 * 9 * 4096 * 4097 / 2
    dw = W.WORKLOADS["decode_b64"]
    lens = torch.tensor([4096, 8192])
    assert W.decode_kv_bytes(dw, lens) == (4096 + 8192) * 8 * 64 * 2 * 2


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
