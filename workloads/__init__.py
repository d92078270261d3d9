"""Seeded synthetic inputs for the GQE attention forward pass.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both sides of every parity check (the HIP library and
the CPU oracle) read the tensors it returns, and the benchmark uses it for its
inputs.  Everything is generated on the CPU with ``torch.Generator`` so the
same seed gives the same bits on any machine.

Problem statement followed (GQE study note, dimensionstp.github.io, §1-1 and
§3-2 (1)): H_q query heads, H_kv KV heads, G = H_kv groups, E = H_q / G query
experts per group, N = G * E routed experts; the query-head -> KV-head map is
floor(i / E) (GQA tutorial, freeguideonline, "GQA 核心原理与计算流程" step 3).

Draw order for every workload: x, W_router, W_q (N routed heads then the
shared head), K, V, then the decode cache lengths.  Values are drawn in fp32
and rounded to bf16 (round-to-nearest-even) for the bf16 workloads.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, dtype and value distribution of one synthetic workload."""

    name: str
    B: int
    T: int                 # prefill: tokens per sequence; decode: 1
    d_model: int
    H_q: int
    H_kv: int
    k: int
    d_head: int
    dtype: str             # "f32" or "bf16"
    seed: int
    act_std: float         # std of x, K, V
    w_std: float           # std of W_router, W_q
    n_shared: int = 1
    causal: int = 1
    route_mode: int = 0    # 0: one summed weighted slot; 1: one weighted slot per group; 2: none;
                           # 3: none, hard slots scaled by their group softmax probability
    zipf_s: float = 0.0    # >0: per-expert router bias ln(Zipf pmf) with this exponent
    decode: bool = False
    L_lo: int = 0          # decode: cache length drawn uniformly in [L_lo, L_hi]
    L_hi: int = 0
    L_max: int = 0         # decode: allocated cache length

    @property
    def G(self) -> int:
        return self.H_kv

    @property
    def E(self) -> int:
        return self.H_q // self.H_kv

    @property
    def N(self) -> int:
        return self.H_q

    @property
    def n_slots(self) -> int:
        return self.k * self.G + (1, self.G, 0, 0)[self.route_mode] + self.n_shared

    @property
    def h_active(self) -> int:
        return self.k * self.G + self.n_shared

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Seeds: tiny fp32 0, main 1, long-context 2, wide/skewed 3,
# decode 4.  Distributions: the tiny case draws everything from N(0, 0.02^2);
# the others draw activations (x, K, V) from N(0, 1) and weights from N(0, 0.02^2).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, T=128, d_model=64, H_q=4, H_kv=2, k=1, d_head=32,
                          dtype="f32", seed=0, act_std=0.02, w_std=0.02, route_mode=1),
    "main_250m": Workload("main_250m", B=4, T=4096, d_model=1024, H_q=16, H_kv=8, k=1, d_head=64,
                          dtype="bf16", seed=1, act_std=1.0, w_std=0.02),
    "long_32k": Workload("long_32k", B=1, T=32768, d_model=1024, H_q=16, H_kv=8, k=1, d_head=64,
                         dtype="bf16", seed=2, act_std=1.0, w_std=0.02),
    "wide_zipf": Workload("wide_zipf", B=2, T=16384, d_model=4096, H_q=32, H_kv=8, k=2, d_head=128,
                          dtype="bf16", seed=3, act_std=1.0, w_std=0.02, zipf_s=1.2),
    "decode_b64": Workload("decode_b64", B=64, T=1, d_model=1024, H_q=16, H_kv=8, k=1, d_head=64,
                           dtype="bf16", seed=4, act_std=1.0, w_std=0.02, decode=True,
                           L_lo=4096, L_hi=8192, L_max=8192),
}


def dense_variant(w: Workload) -> Workload:
    """All-active GQA on the same inputs: every expert kept (k = E), no shared head."""
    return w.replace(name=w.name + "_dense", k=w.E, n_shared=0)


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def zipf_log_pmf(E: int, s: float) -> torch.Tensor:
    """ln of the Zipf(s) probability of ranks 1..E over a support of size E."""
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    h = torch.sum(ranks ** (-s))
    return (-s * torch.log(ranks) - torch.log(h)).to(torch.float32)


def _randn(gen: torch.Generator, shape, std: float) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32) * std


def make_inputs(w: Workload, seed: Optional[int] = None, lens: Optional[torch.Tensor] = None) -> dict:
    """Draw the seeded inputs of workload ``w`` as CPU tensors.

    Returns a dict with ``x`` [B, T, d_model], ``w_router`` [N, d_model],
    ``b_router`` [N] fp32 or None, ``w_q`` [N + n_shared, d_head, d_model]
    (routed experts in global index order g*E + e, shared head last), and
    ``k``/``v`` [B, H_kv, T, d_head] for prefill.  Decode workloads return
    ``k_cache``/``v_cache`` [B, H_kv, L_max, d_head] with every position at or
    beyond a sequence's length set to NaN, and ``lens`` [B] int32 (``lens``
    replaces the drawn lengths when given; the random draws stay the same).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w)
    out = {}
    out["x"] = _randn(gen, (w.B, w.T, w.d_model), w.act_std).to(dt)
    out["w_router"] = _randn(gen, (w.N, w.d_model), w.w_std).to(dt)
    # The shared head's projection is drawn even when n_shared == 0, so that a
    # dense (k = E, no shared head) run sees exactly the same routed weights.
    out["w_q"] = _randn(gen, (w.N + 1, w.d_head, w.d_model), w.w_std).to(dt)[: w.N + w.n_shared].contiguous()
    if w.decode:
        shape = (w.B, w.H_kv, w.L_max, w.d_head)
        kc = _randn(gen, shape, w.act_std).to(dt)
        vc = _randn(gen, shape, w.act_std).to(dt)
        drawn = torch.randint(w.L_lo, w.L_hi + 1, (w.B,), generator=gen, dtype=torch.int64).to(torch.int32)
        lens = drawn if lens is None else lens.to(torch.int32).clone()
        for b in range(w.B):
            kc[b, :, int(lens[b]):, :] = float("nan")
            vc[b, :, int(lens[b]):, :] = float("nan")
        out["k_cache"], out["v_cache"], out["lens"] = kc, vc, lens
    else:
        shape = (w.B, w.H_kv, w.T, w.d_head)
        out["k"] = _randn(gen, shape, w.act_std).to(dt)
        out["v"] = _randn(gen, shape, w.act_std).to(dt)
    if w.zipf_s > 0:
        out["b_router"] = zipf_log_pmf(w.E, w.zipf_s).repeat(w.G).contiguous()
    else:
        out["b_router"] = None
    return out


def make_paged_cache(w: Workload, inp: dict, page_size: int, spare: int = 3, seed: Optional[int] = None) -> dict:
    """The decode caches of ``inp`` cut into pages of ``page_size`` positions and stored in a random order.

    Returns ``k_pages``/``v_pages`` [num_pages, H_kv, page_size, d_head] and ``block_table`` [B, max_pages]
    int32 (max_pages = L_max / page_size rounded up): page j of sequence b holds positions
    j*page_size .. (j+1)*page_size-1 of ``inp``'s cache.  Only pages that hold positions below the
    sequence's length are stored; ``spare`` more pages and the positions past each length are NaN, and
    table entries past a sequence's last page point at random pages, so a read of anything outside the
    sequence shows.  A pure rearrangement of the dense draws (generator seed + 2000003).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed((w.seed if seed is None else seed) + 2000003)
    kc, vc, lens = inp["k_cache"], inp["v_cache"], inp["lens"]
    B, H, L_max, D = kc.shape
    max_pages = -(-L_max // page_size)
    used = [-(-int(l) // page_size) for l in lens]
    num_pages = sum(used) + spare
    order = torch.randperm(num_pages, generator=gen)
    kp = torch.full((num_pages, H, page_size, D), float("nan"), dtype=kc.dtype)
    vp = torch.full_like(kp, float("nan"))
    table = torch.randint(0, num_pages, (B, max_pages), generator=gen, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for j in range(used[b]):
            pg = int(order[nxt]); nxt += 1
            table[b, j] = pg
            lo, hi = j * page_size, min((j + 1) * page_size, L_max)
            kp[pg, :, :hi - lo] = kc[b, :, lo:hi]
            vp[pg, :, :hi - lo] = vc[b, :, lo:hi]
    return dict(k_pages=kp, v_pages=vp, block_table=table)


def make_w_kv(w: Workload, seed: Optional[int] = None):
    """Draw the K and V projection weights [H_kv, d_head, d_model] of workload ``w``, N(0, w_std^2) in the
    workload dtype, from a generator of their own (seed + 3000017)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed((w.seed if seed is None else seed) + 3000017)
    shape = (w.H_kv, w.d_head, w.d_model)
    return _randn(gen, shape, w.w_std).to(torch_dtype(w)), _randn(gen, shape, w.w_std).to(torch_dtype(w))


def make_w_o(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """Draw the output-projection weight [d_model, S * d_head] of workload ``w``,
    N(0, w_std^2) in the workload dtype, from a generator of its own (seed +
    1000003), so the draws of ``make_inputs`` are unchanged."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed((w.seed if seed is None else seed) + 1000003)
    S = w.k * w.G + (1, w.G, 0, 0)[w.route_mode] + w.n_shared
    return _randn(gen, (w.d_model, S * w.d_head), w.w_std).to(torch_dtype(w))


def out_proj_flops(w: Workload, n_tok: Optional[int] = None) -> float:
    """Output-projection FLOPs: 2 * tokens * d_model * S * d_head."""
    S = w.k * w.G + (1, w.G, 0, 0)[w.route_mode] + w.n_shared
    n = w.B * w.T if n_tok is None else n_tok
    return 2.0 * n * w.d_model * S * w.d_head


def attention_flops(w: Workload, lens=None) -> float:
    """Active-head attention FLOPs (QK^T and PV multiply-adds, 2 FLOPs each).

    Prefill, causal: 4 * d_head * B * H_act * T(T+1)/2; non-causal uses T^2.
    Decode: 4 * d_head * H_act * sum(L_b).  Softmax exponentials are not counted.
    """
    if w.decode:
        total = float(sum(int(l) for l in lens))
        return 4.0 * w.d_head * w.h_active * total
    pairs = w.T * (w.T + 1) / 2 if w.causal else float(w.T) * w.T
    return 4.0 * w.d_head * w.B * w.h_active * pairs


def decode_kv_bytes(w: Workload, lens) -> float:
    """Bytes of K and V a decode step must read once: sum_b L_b * H_kv * d_head * 2 * elt."""
    elt = 4 if w.dtype == "f32" else 2
    return float(sum(int(l) for l in lens)) * w.H_kv * w.d_head * 2 * elt


def qproj_flops(w: Workload) -> float:
    return 2.0 * w.d_model * w.d_head * w.B * w.T * w.h_active


def router_flops(w: Workload) -> float:
    return 2.0 * w.d_model * w.N * w.B * w.T


def stratified_rows(w: Workload, n: int, seed: int = 1234) -> torch.Tensor:
    """A seeded sample of flat token ids b*T + t, stratified over positions t.

    Always includes the first and last position of the first and last sequence,
    so both ends of the causal range are covered.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    BT = w.B * w.T
    if n >= BT:
        return torch.arange(BT, dtype=torch.int64)
    edges = torch.linspace(0, w.T, n + 1)
    ts = []
    for i in range(n):
        lo, hi = int(edges[i]), max(int(edges[i]) + 1, int(edges[i + 1]))
        ts.append(int(torch.randint(lo, hi, (1,), generator=gen)))
    bs = torch.randint(0, w.B, (n,), generator=gen)
    ids = {int(b) * w.T + t for b, t in zip(bs.tolist(), ts)}
    ids |= {0, w.T - 1, (w.B - 1) * w.T, BT - 1}
    return torch.tensor(sorted(ids), dtype=torch.int64)


__all__ = [
    "Workload", "WORKLOADS", "dense_variant", "make_inputs", "torch_dtype", "zipf_log_pmf",
    "attention_flops", "decode_kv_bytes", "qproj_flops", "router_flops", "stratified_rows",
]
