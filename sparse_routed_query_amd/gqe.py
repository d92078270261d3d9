"""Python binding of libgqe.so: argument marshalling only.

Every function named ``gqe_*`` here calls the C entry point of the same name
with the tensors' device pointers and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  torch provides device
memory and streams.  The convenience wrappers ``route``, ``qproj``,
``attn_prefill``, ``attn_decode``, ``prefill`` and ``decode`` only allocate
outputs with ``torch.empty`` and call the entry points.

If the library is not built, loading raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqe.so")
_lib = None

GQE_F32, GQE_BF16 = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype", -3: "pointer not 16-byte aligned",
           -4: "kernel launch failed", -5: "workspace missing or too small",
           -6: "call needs more than the static scratch holds"}
DECODE_SCRATCH_BYTES = 16 << 20   # GQE_DECODE_SCRATCH_BYTES

# Every symbol the C header declares (checked by the host tests).
EXPORTS = ("gqe_num_slots", "gqe_status_string", "gqe_route_workspace_bytes", "gqe_route", "gqe_qproj",
           "gqe_attn_prefill_workspace_bytes", "gqe_attn_prefill_plan", "gqe_attn_prefill",
           "gqe_attn_prefill_heads", "gqe_assemble", "gqe_out_proj", "gqe_decode_workspace_bytes", "gqe_attn_decode",
           "gqe_attn_decode_paged", "gqe_kv_proj", "gqe_check_decode_inputs", "gqe_route_backward_workspace_bytes",
           "gqe_route_backward", "gqe_attn_backward_workspace_bytes", "gqe_attn_backward", "gqe_route_stats",
           "gqe_attn_decode_noalloc", "gqe_qkv_proj", "gqe_qkv_proj_backward",
           "gqe_qkv_proj_backward_workspace_bytes", "gqe_decode_route_qproj", "gqe_attn_prefill_heads_lse",
           "gqe_attn_backward_lse", "gqe_out_proj_packed_bytes", "gqe_out_proj_pack", "gqe_out_proj_packed")


class GqeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({_STATUS.get(status, 'unknown')})")
        self.status = status


class GqeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "d_model", "H_q", "H_kv", "k", "d_head", "n_shared", "causal", "route_mode", "dtype")]

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
    def S(self) -> int:
        return self.k * self.H_kv + (1, self.H_kv, 0, 0)[self.route_mode] + self.n_shared

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == GQE_BF16 else torch.float32


def make_desc(B, T, d_model, H_q, H_kv, k, d_head, n_shared=1, causal=1, route_mode=0, dtype="bf16") -> GqeDesc:
    dt = {"bf16": GQE_BF16, "f32": GQE_F32, torch.bfloat16: GQE_BF16, torch.float32: GQE_F32}[dtype]
    return GqeDesc(B, T, d_model, H_q, H_kv, k, d_head, n_shared, causal, route_mode, dt)


def desc_from(w, **over) -> GqeDesc:
    """Descriptor from any object with the shape attributes (e.g. a workload)."""
    f = dict(B=w.B, T=w.T, d_model=w.d_model, H_q=w.H_q, H_kv=w.H_kv, k=w.k, d_head=w.d_head,
             n_shared=w.n_shared, causal=w.causal, route_mode=w.route_mode, dtype=w.dtype)
    f.update(over)
    return make_desc(**f)


def load():
    """Load libgqe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m sparse_routed_query_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        D = ctypes.POINTER(GqeDesc)
        lib.gqe_num_slots.argtypes = [D]
        lib.gqe_num_slots.restype = I
        lib.gqe_status_string.argtypes = [I]
        lib.gqe_status_string.restype = ctypes.c_char_p
        lib.gqe_route_workspace_bytes.argtypes = [D]
        lib.gqe_route_workspace_bytes.restype = Z
        lib.gqe_route.argtypes = [D, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.gqe_route.restype = I
        lib.gqe_qproj.argtypes = [D, P, P, P, P, P, P, P, P, P]
        lib.gqe_qproj.restype = I
        lib.gqe_attn_prefill_workspace_bytes.argtypes = [D]
        lib.gqe_attn_prefill_workspace_bytes.restype = Z
        lib.gqe_attn_prefill_plan.argtypes = [D, I, P, ctypes.c_int64]
        lib.gqe_attn_prefill_plan.restype = ctypes.c_int64
        lib.gqe_attn_prefill.argtypes = [D, P, P, P, P, P, P, P, Z, P]
        lib.gqe_attn_prefill.restype = I
        lib.gqe_attn_prefill_heads.argtypes = [D, P, P, P, P, P, P, Z, P]
        lib.gqe_attn_prefill_heads.restype = I
        lib.gqe_assemble.argtypes = [D, P, P, P]
        lib.gqe_assemble.restype = I
        lib.gqe_check_decode_inputs.argtypes = [D, P, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, P, P]
        lib.gqe_check_decode_inputs.restype = I
        lib.gqe_route_backward_workspace_bytes.argtypes = [D]
        lib.gqe_route_backward_workspace_bytes.restype = Z
        lib.gqe_route_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.gqe_route_backward.restype = I
        lib.gqe_route_stats.argtypes = [D, P, P, P]
        lib.gqe_route_stats.restype = I
        lib.gqe_attn_backward_workspace_bytes.argtypes = [D]
        lib.gqe_attn_backward_workspace_bytes.restype = Z
        lib.gqe_attn_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.gqe_attn_backward.restype = I
        lib.gqe_out_proj_packed_bytes.argtypes = [D]
        lib.gqe_out_proj_packed_bytes.restype = Z
        lib.gqe_out_proj_pack.argtypes = [D, P, P, P]
        lib.gqe_out_proj_pack.restype = I
        lib.gqe_out_proj_packed.argtypes = [D, P, P, P, P, ctypes.c_int32, P]
        lib.gqe_out_proj_packed.restype = I
        lib.gqe_attn_prefill_heads_lse.argtypes = [D, P, P, P, P, P, P, P, Z, P]
        lib.gqe_attn_prefill_heads_lse.restype = I
        lib.gqe_attn_backward_lse.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.gqe_attn_backward_lse.restype = I
        lib.gqe_kv_proj.argtypes = [D, P, P, P, P, P, P]
        lib.gqe_kv_proj.restype = I
        lib.gqe_out_proj.argtypes = [D, P, P, P, P, ctypes.c_int32, P]
        lib.gqe_out_proj.restype = I
        lib.gqe_decode_workspace_bytes.argtypes = [D, ctypes.c_int32]
        lib.gqe_decode_workspace_bytes.restype = Z
        lib.gqe_attn_decode.argtypes = [D, P, P, P, P, ctypes.c_int32, P, P, P, P, Z, P]
        lib.gqe_attn_decode.restype = I
        lib.gqe_qkv_proj.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P]
        lib.gqe_qkv_proj.restype = I
        lib.gqe_qkv_proj_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P,
                                              Z, P]
        lib.gqe_qkv_proj_backward.restype = I
        lib.gqe_decode_route_qproj.argtypes = [D, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P]
        lib.gqe_decode_route_qproj.restype = I
        lib.gqe_qkv_proj_backward_workspace_bytes.argtypes = [D, ctypes.c_int32]
        lib.gqe_qkv_proj_backward_workspace_bytes.restype = Z
        lib.gqe_attn_decode_noalloc.argtypes = [D, P, P, P, P, ctypes.c_int32, P, P, P, P]
        lib.gqe_attn_decode_noalloc.restype = I
        i32 = ctypes.c_int32
        lib.gqe_attn_decode_paged.argtypes = [D, P, P, P, P, i32, i32, i32, P, P, P, P, P, Z, P]
        lib.gqe_attn_decode_paged.restype = I
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise GqeError(fn, rc)


# ---------------------------------------------------------------- entry points

def gqe_num_slots(desc: GqeDesc) -> int:
    return load().gqe_num_slots(ctypes.byref(desc))


def gqe_route_workspace_bytes(desc: GqeDesc) -> int:
    return load().gqe_route_workspace_bytes(ctypes.byref(desc))


def gqe_decode_workspace_bytes(desc: GqeDesc, L_max: int) -> int:
    return load().gqe_decode_workspace_bytes(ctypes.byref(desc), L_max)


def gqe_route(desc, x, w_router, b_router, sel, p_tilde, counts, offsets, rows, logits, workspace, stream=None):
    dt = desc.torch_dtype
    rc = load().gqe_route(ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_router, dt, "w_router"),
                          _ptr(b_router, torch.float32, "b_router"), _ptr(sel, torch.int32, "sel"),
                          _ptr(p_tilde, torch.float32, "p_tilde"), _ptr(counts, torch.int32, "counts"),
                          _ptr(offsets, torch.int32, "offsets"), _ptr(rows, torch.int32, "rows"),
                          _ptr(logits, torch.float64, "logits"), _ptr(workspace, None, "workspace"),
                          workspace.numel() * workspace.element_size() if workspace is not None else 0,
                          _stream(stream))
    _check("gqe_route", rc)


def gqe_qproj(desc, x, w_q, sel, counts, offsets, rows, q_routed, q_shared, stream=None):
    dt = desc.torch_dtype
    rc = load().gqe_qproj(ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_q, dt, "w_q"), _ptr(sel, torch.int32, "sel"),
                          _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
                          _ptr(rows, torch.int32, "rows"), _ptr(q_routed, dt, "q_routed"),
                          _ptr(q_shared, dt, "q_shared"), _stream(stream))
    _check("gqe_qproj", rc)


def gqe_attn_prefill_workspace_bytes(desc: GqeDesc) -> int:
    return int(load().gqe_attn_prefill_workspace_bytes(ctypes.byref(desc)))


def gqe_attn_prefill_plan(desc: GqeDesc, split: bool = True):
    """Work items of one bf16 prefill attention launch: int32 array [n, 5] of
    (b, head, query tile, part, pair) in launch order."""
    import numpy as np
    lib = load()
    n = lib.gqe_attn_prefill_plan(ctypes.byref(desc), int(split), None, 0)
    _check("gqe_attn_prefill_plan", min(int(n), 0))
    items = np.zeros((max(int(n), 1), 5), dtype=np.int32)
    lib.gqe_attn_prefill_plan(ctypes.byref(desc), int(split), items.ctypes.data_as(ctypes.c_void_p), int(n))
    return items[: int(n)]


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()


def gqe_attn_prefill(desc, q_routed, q_shared, k, v, p_tilde, out, workspace=None, stream=None):
    dt = desc.torch_dtype
    wp, wb = _ws(workspace)
    rc = load().gqe_attn_prefill(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"),
                                 _ptr(k, dt, "k"), _ptr(v, dt, "v"), _ptr(p_tilde, torch.float32, "p_tilde"),
                                 _ptr(out, torch.float32, "out"), wp, wb, _stream(stream))
    _check("gqe_attn_prefill", rc)


def gqe_attn_prefill_heads(desc, q_routed, q_shared, k, v, out, workspace=None, stream=None):
    dt = desc.torch_dtype
    wp, wb = _ws(workspace)
    rc = load().gqe_attn_prefill_heads(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"),
                                       _ptr(q_shared, dt, "q_shared"), _ptr(k, dt, "k"), _ptr(v, dt, "v"),
                                       _ptr(out, torch.float32, "out"), wp, wb, _stream(stream))
    _check("gqe_attn_prefill_heads", rc)


def gqe_attn_prefill_heads_lse(desc, q_routed, q_shared, k, v, out, lse, workspace=None, stream=None):
    dt = desc.torch_dtype
    wp, wb = _ws(workspace)
    rc = load().gqe_attn_prefill_heads_lse(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"),
                                           _ptr(q_shared, dt, "q_shared"), _ptr(k, dt, "k"), _ptr(v, dt, "v"),
                                           _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), wp, wb,
                                           _stream(stream))
    _check("gqe_attn_prefill_heads_lse", rc)


def lse_rows(desc) -> int:
    """Number of rows of the attention statistics: routed rows, then shared rows."""
    return desc.B * desc.H_kv * desc.T * desc.k + (desc.B * desc.T if desc.n_shared else 0)


def gqe_assemble(desc, p_tilde, out, stream=None):
    rc = load().gqe_assemble(ctypes.byref(desc), _ptr(p_tilde, torch.float32, "p_tilde"),
                             _ptr(out, torch.float32, "out"), _stream(stream))
    _check("gqe_assemble", rc)


def check_decode_inputs(desc, lens, L_max, block_table=None, num_pages=0, page_size=0, stream=None):
    """Device-side audit of decode inputs: returns (bad lengths, bad page ids) after a synchronise."""
    bad = torch.zeros(2, dtype=torch.int32, device=lens.device)
    max_pages = block_table.shape[1] if block_table is not None else 0
    rc = load().gqe_check_decode_inputs(ctypes.byref(desc), _ptr(lens, torch.int32, "lens"), int(L_max),
                                        _ptr(block_table, torch.int32, "block_table"), int(num_pages),
                                        int(page_size), int(max_pages), _ptr(bad, None, "bad"), _stream(stream))
    _check("gqe_check_decode_inputs", rc)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return int(bad[0]), int(bad[1])


def gqe_route_backward_workspace_bytes(desc: GqeDesc) -> int:
    return load().gqe_route_backward_workspace_bytes(ctypes.byref(desc))


def gqe_route_backward(desc, dout, out, sel, p_tilde, x, w_router, d_hard, d_logits, dw_router, db_router, dx,
                       workspace, stream=None):
    dt = desc.torch_dtype
    nb = workspace.numel() if workspace is not None else 0
    rc = load().gqe_route_backward(ctypes.byref(desc), _ptr(dout, torch.float32, "dout"), _ptr(out, torch.float32, "out"),
                                   _ptr(sel, torch.int32, "sel"), _ptr(p_tilde, torch.float32, "p_tilde"),
                                   _ptr(x, dt, "x"), _ptr(w_router, dt, "w_router"),
                                   _ptr(d_hard, torch.float32, "d_hard"), _ptr(d_logits, torch.float32, "d_logits"),
                                   _ptr(dw_router, torch.float32, "dw_router"), _ptr(db_router, torch.float32, "db_router"),
                                   _ptr(dx, torch.float32, "dx"), _ptr(workspace, torch.uint8, "workspace"), nb,
                                   _stream(stream))
    _check("gqe_route_backward", rc)


def route_backward(desc, dout, out, sel, p_tilde, x, w_router, want_dw=True, want_dx=True, stream=None) -> dict:
    """Gradients through slot assembly and routing (allocates its outputs and workspace)."""
    BT, G, k, N, D = desc.B * desc.T, desc.H_kv, desc.k, desc.H_q, desc.d_head
    dev = dout.device
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    res = dict(d_hard=e(BT, G * k, D), d_logits=e(BT, N), dw_router=e(N, desc.d_model) if want_dw else None,
               db_router=e(N) if want_dw else None, dx=e(BT, desc.d_model) if want_dx else None)
    nb = gqe_route_backward_workspace_bytes(desc) if want_dw else 0
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if want_dw else None
    gqe_route_backward(desc, dout, out, sel, p_tilde, x, w_router, res["d_hard"], res["d_logits"], res["dw_router"],
                       res["db_router"], res["dx"], ws, stream)
    return res


def gqe_route_stats(desc, logits, importance, stream=None):
    rc = load().gqe_route_stats(ctypes.byref(desc), _ptr(logits, torch.float64, "logits"),
                                _ptr(importance, torch.float32, "importance"), _stream(stream))
    _check("gqe_route_stats", rc)


def route_stats(desc, logits, stream=None) -> torch.Tensor:
    """Per-expert router importance [N] (fp32) from gqe_route's fp64 scores."""
    imp = torch.empty(desc.H_q, dtype=torch.float32, device=logits.device)
    gqe_route_stats(desc, logits, imp, stream)
    return imp


def gqe_attn_backward_workspace_bytes(desc: GqeDesc) -> int:
    return load().gqe_attn_backward_workspace_bytes(ctypes.byref(desc))


def gqe_attn_backward(desc, q_routed, q_shared, k, v, out, d_hard, dout, dq_routed, dq_shared, dk, dv, workspace,
                      stream=None):
    dt = desc.torch_dtype
    rc = load().gqe_attn_backward(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"),
                                  _ptr(k, dt, "k"), _ptr(v, dt, "v"), _ptr(out, torch.float32, "out"),
                                  _ptr(d_hard, torch.float32, "d_hard"), _ptr(dout, torch.float32, "dout"),
                                  _ptr(dq_routed, torch.float32, "dq_routed"),
                                  _ptr(dq_shared, torch.float32, "dq_shared"), _ptr(dk, torch.float32, "dk"),
                                  _ptr(dv, torch.float32, "dv"), _ptr(workspace, torch.uint8, "workspace"),
                                  workspace.numel(), _stream(stream))
    _check("gqe_attn_backward", rc)


def gqe_attn_backward_lse(desc, q_routed, q_shared, k, v, out, d_hard, dout, lse, dq_routed, dq_shared, dk, dv,
                          workspace, stream=None):
    dt = desc.torch_dtype
    rc = load().gqe_attn_backward_lse(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"),
                                      _ptr(q_shared, dt, "q_shared"), _ptr(k, dt, "k"), _ptr(v, dt, "v"),
                                      _ptr(out, torch.float32, "out"), _ptr(d_hard, torch.float32, "d_hard"),
                                      _ptr(dout, torch.float32, "dout"), _ptr(lse, torch.float32, "lse"),
                                      _ptr(dq_routed, torch.float32, "dq_routed"),
                                      _ptr(dq_shared, torch.float32, "dq_shared"), _ptr(dk, torch.float32, "dk"),
                                      _ptr(dv, torch.float32, "dv"), _ptr(workspace, torch.uint8, "workspace"),
                                      workspace.numel(), _stream(stream))
    _check("gqe_attn_backward_lse", rc)


def attn_backward(desc, q_routed, q_shared, k, v, out, d_hard, dout, lse=None, stream=None) -> dict:
    """Gradients of the attention: dq_routed [B, G, T*k, d], dq_shared [B, T, d] or None, dk, dv [B, H_kv, T, d]
    (fp32; allocates its outputs and workspace).  lse: the forward's row statistics
    (gqe_attn_prefill_heads_lse), which skips their recomputation."""
    B, T, G, k_, D = desc.B, desc.T, desc.H_kv, desc.k, desc.d_head
    dev = d_hard.device
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    res = dict(dq_routed=e(B, G, T * k_, D), dq_shared=e(B, T, D) if desc.n_shared else None, dk=e(B, G, T, D),
               dv=e(B, G, T, D))
    ws = torch.empty(gqe_attn_backward_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    if lse is not None:
        gqe_attn_backward_lse(desc, q_routed, q_shared if desc.n_shared else None, k, v, out, d_hard,
                              dout if desc.n_shared else None, lse, res["dq_routed"], res["dq_shared"], res["dk"],
                              res["dv"], ws, stream)
        return res
    gqe_attn_backward(desc, q_routed, q_shared if desc.n_shared else None, k, v, out, d_hard,
                      dout if desc.n_shared else None, res["dq_routed"], res["dq_shared"], res["dk"], res["dv"], ws,
                      stream)
    return res


def gqe_kv_proj(desc, x, w_k, w_v, k, v, stream=None):
    dt = desc.torch_dtype
    rc = load().gqe_kv_proj(ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_k, dt, "w_k"), _ptr(w_v, dt, "w_v"),
                            _ptr(k, dt, "k"), _ptr(v, dt, "v"), _stream(stream))
    _check("gqe_kv_proj", rc)


def kv_proj(desc, x, w_k, w_v, stream=None):
    """K and V [B, H_kv, T, d_head] from x [B*T, d_model]."""
    shape = (desc.B, desc.H_kv, desc.T, desc.d_head)
    k = torch.empty(shape, dtype=desc.torch_dtype, device=x.device)
    v = torch.empty(shape, dtype=desc.torch_dtype, device=x.device)
    gqe_kv_proj(desc, x, w_k, w_v, k, v, stream)
    return k, v


def gqe_out_proj(desc, out, p_tilde, w_o, y, write_weighted=False, stream=None):
    rc = load().gqe_out_proj(ctypes.byref(desc), _ptr(out, torch.float32, "out"), _ptr(p_tilde, torch.float32, "p_tilde"),
                             _ptr(w_o, desc.torch_dtype, "w_o"), _ptr(y, torch.float32, "y"), int(bool(write_weighted)),
                             _stream(stream))
    _check("gqe_out_proj", rc)


def gqe_out_proj_packed_bytes(desc) -> int:
    return load().gqe_out_proj_packed_bytes(ctypes.byref(desc))


def gqe_out_proj_pack(desc, w_o, w_packed, stream=None):
    rc = load().gqe_out_proj_pack(ctypes.byref(desc), _ptr(w_o, desc.torch_dtype, "w_o"),
                                  _ptr(w_packed, desc.torch_dtype, "w_packed"), _stream(stream))
    _check("gqe_out_proj_pack", rc)


def gqe_out_proj_packed(desc, out, p_tilde, w_packed, y, write_weighted=False, stream=None):
    rc = load().gqe_out_proj_packed(ctypes.byref(desc), _ptr(out, torch.float32, "out"),
                                    _ptr(p_tilde, torch.float32, "p_tilde"),
                                    _ptr(w_packed, desc.torch_dtype, "w_packed"), _ptr(y, torch.float32, "y"),
                                    int(bool(write_weighted)), _stream(stream))
    _check("gqe_out_proj_packed", rc)


def out_proj_pack(desc, w_o, stream=None) -> torch.Tensor:
    """W_o rearranged into the packed order gqe_out_proj_packed reads (a tensor of W_o's shape and dtype)."""
    if gqe_out_proj_packed_bytes(desc) == 0:
        raise GqeError("gqe_out_proj_pack", -2)
    w_packed = torch.empty_like(w_o)
    gqe_out_proj_pack(desc, w_o, w_packed, stream)
    return w_packed


def gqe_attn_decode(desc, q_routed, q_shared, k_cache, v_cache, lens, p_tilde, out, workspace, stream=None):
    dt = desc.torch_dtype
    L_max = k_cache.shape[2]
    rc = load().gqe_attn_decode(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"),
                                _ptr(k_cache, dt, "k_cache"), _ptr(v_cache, dt, "v_cache"), L_max,
                                _ptr(lens, torch.int32, "lens"), _ptr(p_tilde, torch.float32, "p_tilde"),
                                _ptr(out, torch.float32, "out"), _ptr(workspace, None, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gqe_attn_decode", rc)


def gqe_qkv_proj(desc, x, w_q, w_k, w_v, sel, counts, offsets, rows, positions, rope_base, q_routed, q_shared, k, v,
                 stream=None):
    """The Q/K/V preamble in one launch, optionally with the rotary embedding (rope_base > 1; 0 = none)."""
    dt = desc.torch_dtype
    rc = load().gqe_qkv_proj(ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_q, dt, "w_q"), _ptr(w_k, dt, "w_k"),
                             _ptr(w_v, dt, "w_v"), _ptr(sel, torch.int32, "sel"), _ptr(counts, torch.int32, "counts"),
                             _ptr(offsets, torch.int32, "offsets"), _ptr(rows, torch.int32, "rows"),
                             _ptr(positions, torch.int32, "positions"), float(rope_base),
                             _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"), _ptr(k, dt, "k"),
                             _ptr(v, dt, "v"), _stream(stream))
    _check("gqe_qkv_proj", rc)


def gqe_decode_route_qproj(desc, x, w_router, b_router, w_q, positions, rope_base, sel, p_tilde, q_routed, q_shared,
                           logits=None, stream=None):
    """Routing and query projection of one new token per sequence in one launch (desc.T == 1)."""
    dt = desc.torch_dtype
    rc = load().gqe_decode_route_qproj(ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_router, dt, "w_router"),
                                       _ptr(b_router, torch.float32, "b_router"), _ptr(w_q, dt, "w_q"),
                                       _ptr(positions, torch.int32, "positions"), float(rope_base),
                                       _ptr(sel, torch.int32, "sel"), _ptr(p_tilde, torch.float32, "p_tilde"),
                                       _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"),
                                       _ptr(logits, torch.float64, "logits"), _stream(stream))
    _check("gqe_decode_route_qproj", rc)


def decode_route_qproj(desc, x, w_router, b_router, w_q, positions=None, rope_base=0.0, logits=False,
                       stream=None) -> dict:
    """Allocating wrapper: sel, p_tilde, q_routed, q_shared (and logits) of one new token per sequence."""
    dev = x.device
    B, G, k, D = desc.B, desc.H_kv, desc.k, desc.d_head
    res = dict(sel=torch.empty((B, G, k), dtype=torch.int32, device=dev),
               p_tilde=torch.empty((B, G, k), dtype=torch.float32, device=dev),
               q_routed=torch.empty((B, G, 1, k, D), dtype=desc.torch_dtype, device=dev),
               q_shared=torch.empty((B, 1, D), dtype=desc.torch_dtype, device=dev) if desc.n_shared else None,
               logits=torch.empty((B, desc.H_q), dtype=torch.float64, device=dev) if logits else None)
    gqe_decode_route_qproj(desc, x, w_router, b_router, w_q, positions, rope_base, res["sel"], res["p_tilde"],
                           res["q_routed"], res["q_shared"], res["logits"], stream)
    return res


def gqe_qkv_proj_backward_workspace_bytes(desc, with_kv: bool) -> int:
    return load().gqe_qkv_proj_backward_workspace_bytes(ctypes.byref(desc), int(bool(with_kv)))


def gqe_qkv_proj_backward(desc, x, w_q, w_k, w_v, sel, counts, offsets, rows, positions, rope_base, dq_routed,
                          dq_shared, dk, dv, dw_q, dw_k, dw_v, dx, workspace=None, stream=None):
    """Gradients of the projection weights and of x from the gradients of q, K and V."""
    dt = desc.torch_dtype
    f = torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().gqe_qkv_proj_backward(
        ctypes.byref(desc), _ptr(x, dt, "x"), _ptr(w_q, dt, "w_q"), _ptr(w_k, dt, "w_k"), _ptr(w_v, dt, "w_v"),
        _ptr(sel, torch.int32, "sel"), _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(rows, torch.int32, "rows"), _ptr(positions, torch.int32, "positions"), float(rope_base),
        _ptr(dq_routed, f, "dq_routed"), _ptr(dq_shared, f, "dq_shared"), _ptr(dk, f, "dk"), _ptr(dv, f, "dv"),
        _ptr(dw_q, f, "dw_q"), _ptr(dw_k, f, "dw_k"), _ptr(dw_v, f, "dw_v"), _ptr(dx, f, "dx"),
        _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))
    _check("gqe_qkv_proj_backward", rc)


def qkv_proj_backward(desc, x, w_q, w_k, w_v, r: dict, dq_routed, dq_shared, dk=None, dv=None, positions=None,
                      rope_base=0.0, use_workspace=True, stream=None) -> dict:
    """Allocating wrapper: dw_q, dw_k, dw_v (with dk, dv) and dx, fp32."""
    dev = x.device
    nws = gqe_qkv_proj_backward_workspace_bytes(desc, dk is not None) if use_workspace else 0
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    f = torch.float32
    dw_q = torch.empty(tuple(w_q.shape), dtype=f, device=dev)
    dw_k = torch.empty(tuple(w_k.shape), dtype=f, device=dev) if dk is not None else None
    dw_v = torch.empty(tuple(w_v.shape), dtype=f, device=dev) if dk is not None else None
    dx = torch.empty((desc.B * desc.T, desc.d_model), dtype=f, device=dev)
    gqe_qkv_proj_backward(desc, x, w_q, w_k, w_v, r["sel"], r["counts"], r["offsets"], r["rows"], positions, rope_base,
                          dq_routed, dq_shared, dk, dv, dw_q, dw_k, dw_v, dx, ws, stream)
    return dict(dw_q=dw_q, dw_k=dw_k, dw_v=dw_v, dx=dx)


def gqe_attn_decode_noalloc(desc, q_routed, q_shared, k_cache, v_cache, lens, p_tilde, out, stream=None):
    """gqe_attn_decode with its partials in the library's static device scratch (no workspace)."""
    dt = desc.torch_dtype
    L_max = k_cache.shape[2]
    rc = load().gqe_attn_decode_noalloc(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"),
                                        _ptr(q_shared, dt, "q_shared"), _ptr(k_cache, dt, "k_cache"),
                                        _ptr(v_cache, dt, "v_cache"), L_max, _ptr(lens, torch.int32, "lens"),
                                        _ptr(p_tilde, torch.float32, "p_tilde"), _ptr(out, torch.float32, "out"),
                                        _stream(stream))
    _check("gqe_attn_decode_noalloc", rc)


def gqe_attn_decode_paged(desc, q_routed, q_shared, k_pages, v_pages, block_table, lens, p_tilde, out, workspace,
                          stream=None):
    """k_pages, v_pages [num_pages, H_kv, page_size, d_head]; block_table [B, max_pages] int32."""
    dt = desc.torch_dtype
    rc = load().gqe_attn_decode_paged(ctypes.byref(desc), _ptr(q_routed, dt, "q_routed"), _ptr(q_shared, dt, "q_shared"),
                                      _ptr(k_pages, dt, "k_pages"), _ptr(v_pages, dt, "v_pages"), k_pages.shape[0],
                                      k_pages.shape[2], block_table.shape[1], _ptr(block_table, torch.int32, "block_table"),
                                      _ptr(lens, torch.int32, "lens"), _ptr(p_tilde, torch.float32, "p_tilde"),
                                      _ptr(out, torch.float32, "out"), _ptr(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gqe_attn_decode_paged", rc)


# ---------------------------------------------------------------- allocating wrappers

def alloc_route(desc: GqeDesc, device, logits: bool = False) -> dict:
    BT, G, k, N = desc.B * desc.T, desc.G, desc.k, desc.N
    e = lambda *s, dtype: torch.empty(s, dtype=dtype, device=device)  # noqa: E731
    return dict(sel=e(BT, G, k, dtype=torch.int32), p_tilde=e(BT, G, k, dtype=torch.float32),
                counts=e(N, dtype=torch.int32), offsets=e(N + 1, dtype=torch.int32),
                rows=e(BT * G * k, dtype=torch.int32),
                logits=e(BT, N, dtype=torch.float64) if logits else None,
                workspace=e(max(1, gqe_route_workspace_bytes(desc)), dtype=torch.uint8))


def alloc_qproj(desc: GqeDesc, device) -> dict:
    dt = desc.torch_dtype
    qr = torch.empty((desc.B, desc.G, desc.T, desc.k, desc.d_head), dtype=dt, device=device)
    qs = torch.empty((desc.B, desc.T, desc.d_head), dtype=dt, device=device) if desc.n_shared else None
    return dict(q_routed=qr, q_shared=qs)


def route(desc, x, w_router, b_router=None, logits=False, bufs=None, stream=None) -> dict:
    r = bufs if bufs is not None else alloc_route(desc, x.device, logits)
    gqe_route(desc, x, w_router, b_router, r["sel"], r["p_tilde"], r["counts"], r["offsets"], r["rows"],
              r["logits"], r["workspace"], stream)
    return r


def qkv_proj(desc, x, w_q, w_k, w_v, r: dict, positions=None, rope_base=0.0, stream=None) -> dict:
    """q_routed, q_shared, k, v of x in one launch (rotary embedding when rope_base > 1)."""
    q = alloc_qproj(desc, x.device)
    shape = (desc.B, desc.H_kv, desc.T, desc.d_head)
    k = torch.empty(shape, dtype=desc.torch_dtype, device=x.device)
    v = torch.empty(shape, dtype=desc.torch_dtype, device=x.device)
    gqe_qkv_proj(desc, x, w_q, w_k, w_v, r["sel"], r["counts"], r["offsets"], r["rows"], positions, rope_base,
                 q["q_routed"], q["q_shared"], k, v, stream)
    return dict(q, k=k, v=v)


def qproj(desc, x, w_q, r: dict, bufs=None, stream=None) -> dict:
    q = bufs if bufs is not None else alloc_qproj(desc, x.device)
    gqe_qproj(desc, x, w_q, r["sel"], r["counts"], r["offsets"], r["rows"], q["q_routed"], q["q_shared"], stream)
    return q


_prefill_ws = {}


def prefill_workspace(desc: GqeDesc, device) -> Optional[torch.Tensor]:
    """A zeroed workspace for the prefill attention of `desc` on `device`, kept
    and reused (each call leaves its counters at zero), or None if the shape
    splits no query tile.  Calls that use it must not overlap in time."""
    n = gqe_attn_prefill_workspace_bytes(desc)
    if n == 0:
        return None
    dev = torch.device(device)
    ws = _prefill_ws.get(dev)
    if ws is None or ws.numel() < n:
        ws = torch.zeros(n, dtype=torch.uint8, device=dev)
        _prefill_ws[dev] = ws
    return ws


def attn_prefill(desc, q: dict, k, v, p_tilde, out=None, split=True, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((desc.B, desc.T, desc.S, desc.d_head), dtype=torch.float32, device=k.device)
    ws = prefill_workspace(desc, k.device) if split else None
    gqe_attn_prefill(desc, q["q_routed"], q["q_shared"], k, v, p_tilde, out, ws, stream)
    return out


def attn_decode(desc, q: dict, k_cache, v_cache, lens, p_tilde, out=None, workspace=None, stream=None):
    if out is None:
        out = torch.empty((desc.B, desc.S, desc.d_head), dtype=torch.float32, device=k_cache.device)
    if workspace is None:
        workspace = torch.empty(gqe_decode_workspace_bytes(desc, k_cache.shape[2]), dtype=torch.uint8,
                                device=k_cache.device)
    gqe_attn_decode(desc, q["q_routed"], q["q_shared"], k_cache, v_cache, lens, p_tilde, out, workspace, stream)
    return out


def out_proj(desc, out, p_tilde, w_o, y=None, write_weighted=False, w_packed=None, stream=None) -> torch.Tensor:
    """y = W_o h_t over the concatenated slots of every token (weighted slot(s) formed inside); with w_packed
    (out_proj_pack's result) the packed-weight call."""
    if y is None:
        y = torch.empty((desc.B * desc.T, desc.d_model), dtype=torch.float32, device=out.device)
    if w_packed is not None:
        gqe_out_proj_packed(desc, out, p_tilde, w_packed, y, write_weighted, stream)
    else:
        gqe_out_proj(desc, out, p_tilde, w_o, y, write_weighted, stream)
    return y


def prefill(desc, x, w_router, b_router, w_q, k, v, logits=False, stream=None) -> dict:
    """Whole prefill path: route -> compaction -> projection -> attention -> slots."""
    r = route(desc, x, w_router, b_router, logits=logits, stream=stream)
    q = qproj(desc, x, w_q, r, stream=stream)
    out = attn_prefill(desc, q, k, v, r["p_tilde"], stream=stream)
    return dict(r, **q, out=out)


def decode(desc, x, w_router, b_router, w_q, k_cache, v_cache, lens, positions=None, rope_base=0.0,
           fused=True, stream=None) -> dict:
    """Whole decode step for one new token per sequence (desc.T == 1): routing and query projection in one
    launch (gqe_decode_route_qproj), then the attention.  fused=False takes gqe_route + gqe_qproj instead
    (no rotary embedding there)."""
    if fused:
        r = decode_route_qproj(desc, x, w_router, b_router, w_q, positions, rope_base, logits=True, stream=stream)
        q = dict(q_routed=r.pop("q_routed"), q_shared=r.pop("q_shared"))
    else:
        if rope_base:
            raise ValueError("the rotary embedding needs the fused decode preamble")
        r = route(desc, x, w_router, b_router, logits=True, stream=stream)
        q = qproj(desc, x, w_q, r, stream=stream)
    out = attn_decode(desc, q, k_cache, v_cache, lens, r["p_tilde"], stream=stream)
    return dict(r, **q, out=out)
