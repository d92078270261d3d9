"""CPU oracle for the GQE attention forward -- TEST INFRASTRUCTURE ONLY.

A thin numpy/ctypes wrapper around ``gqe_oracle.c``: a plain, slow,
double-precision definition of every step of the Grouped Query Experts
forward (router, top-k, renormalisation, compaction, routed projection,
causal attention against the group's dense KV head, slot assembly, and the
one-token decode step).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  It imports nothing from the
HIP library's package and the library never imports it.

Inputs may be torch tensors or numpy arrays of any float dtype; they are
converted to float64, which represents bf16 and fp32 values exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

TIE_MARGIN = 1e-6


def build() -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE double arithmetic)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "d_model", "H_q", "H_kv", "k", "d_head", "n_shared", "causal", "route_mode")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.ora_route.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P, P, P]
        lib.ora_route.restype = ctypes.c_int
        lib.ora_compact.argtypes = [P, ctypes.c_int64, P, P, P, P]
        lib.ora_compact.restype = None
        lib.ora_qproj_rows.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P]
        lib.ora_qproj_rows.restype = None
        lib.ora_prefill_rows.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, P, P]
        lib.ora_prefill_rows.restype = None
        lib.ora_attend_rows.argtypes = [P, P, P, P, P, P, ctypes.c_int64, P, P]
        lib.ora_attend_rows.restype = None
        lib.ora_kv_proj.argtypes = [P, P, P, P]
        lib.ora_kv_proj.restype = None
        lib.ora_assemble_rows.argtypes = [P, P, ctypes.c_int64, P]
        lib.ora_assemble_rows.restype = None
        lib.ora_out_proj_rows.argtypes = [P, P, P, ctypes.c_int64, P]
        lib.ora_out_proj_rows.restype = None
        lib.ora_decode.argtypes = [P, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P, P]
        lib.ora_decode.restype = ctypes.c_int
        lib.ora_rope.argtypes = [ctypes.c_int64, ctypes.c_int, P, ctypes.c_double, P]
        lib.ora_rope.restype = None
        lib.ora_decode_given.argtypes = [P, P, P, P, P, ctypes.c_int32, P, P, P, P]
        lib.ora_decode_given.restype = ctypes.c_int
        lib.ora_num_slots.argtypes = [P]
        lib.ora_num_slots.restype = ctypes.c_int
        lib.ora_num_threads.argtypes = []
        lib.ora_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def desc(w, **over) -> _Desc:
    """Build the oracle's descriptor from any object with the shape attributes."""
    f = {n: int(getattr(w, n)) for n, _ in _Desc._fields_}
    f.update({k: int(v) for k, v in over.items()})
    return _Desc(**f)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().ora_num_threads()


def num_slots(d: _Desc) -> int:
    return _load().ora_num_slots(ctypes.byref(d))


def route(d: _Desc, x, w_router, b_router=None):
    """Router, softmax, top-k and renormalisation over all B*T tokens.

    Returns dict(logits [BT, N], probs [BT, N], sel [BT, G, k] int32,
    ptilde [BT, G, k], tie [BT, G] bool).
    """
    lib = _load()
    G, E, k, N = d.H_kv, d.H_q // d.H_kv, d.k, d.H_q
    x = _f64(x).reshape(-1, d.d_model)
    n_tok = x.shape[0]
    wr, br = _f64(w_router), _f64(b_router)
    logits = np.empty((n_tok, N)); probs = np.empty((n_tok, N))
    sel = np.empty((n_tok, G, k), dtype=np.int32)
    pt = np.empty((n_tok, G, k)); tie = np.empty((n_tok, G), dtype=np.uint8)
    rc = lib.ora_route(ctypes.byref(d), n_tok, _ptr(x), _ptr(wr), _ptr(br), _ptr(logits), _ptr(probs),
                       _ptr(sel), _ptr(pt), _ptr(tie))
    if rc != 0:
        raise ValueError("oracle route: invalid shape (need 1 <= k <= E <= 256)")
    return dict(logits=logits, probs=probs, sel=sel, ptilde=pt, tie=tie.astype(bool))


def expert_importance(d: _Desc, probs):
    """Per-expert router importance, the probability mass each expert receives summed over tokens:
    importance[n] = sum_t p[t, n] with p the in-group softmax (study note §3-2 (2)).  With the per-expert
    counts of kept tokens (compact's counts) these are the load statistics a balance loss is formed from
    (§4 names the loss but not its exact form).  probs [BT, N] as route() returns them."""
    return np.asarray(probs, dtype=np.float64).reshape(-1, d.H_q).sum(axis=0)


def compact(d: _Desc, sel):
    """Counting sort of kept (token, expert) pairs: counts [N], offsets [N+1], rows [BT*G*k]."""
    lib = _load()
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    n_tok = sel.shape[0]
    N = d.H_q
    counts = np.empty(N, dtype=np.int32); offsets = np.empty(N + 1, dtype=np.int32)
    rows = np.empty(n_tok * d.H_kv * d.k, dtype=np.int32)
    lib.ora_compact(ctypes.byref(d), n_tok, _ptr(sel), _ptr(counts), _ptr(offsets), _ptr(rows))
    return dict(counts=counts, offsets=offsets, rows=rows)


def qproj_rows(d: _Desc, x, w_q, sel, tok=None):
    """Routed and shared query projections for tokens ``tok`` (default: all).

    Returns (q_routed [n, G, k, d_head], q_shared [n, d_head] or None).
    """
    lib = _load()
    x = _f64(x).reshape(-1, d.d_model)
    tok = np.arange(x.shape[0], dtype=np.int64) if tok is None else np.ascontiguousarray(np.asarray(tok, dtype=np.int64))
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    wq = _f64(w_q)
    n = tok.shape[0]
    qr = np.empty((n, d.H_kv, d.k, d.d_head))
    qs = np.empty((n, d.d_head)) if d.n_shared else None
    lib.ora_qproj_rows(ctypes.byref(d), n, _ptr(tok), _ptr(x), _ptr(wq), _ptr(sel), _ptr(qr), _ptr(qs))
    return qr, qs


def prefill_rows(d: _Desc, x, w_q, K, V, sel, ptilde, tok=None):
    """Attention and slot assembly for tokens ``tok`` (flat b*T+t; default all).

    Returns out [n, S, d_head] float64.
    """
    lib = _load()
    x = _f64(x).reshape(-1, d.d_model)
    tok = np.arange(x.shape[0], dtype=np.int64) if tok is None else np.ascontiguousarray(np.asarray(tok, dtype=np.int64))
    K, V, wq = _f64(K), _f64(V), _f64(w_q)
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    pt = _f64(ptilde)
    S = num_slots(d)
    out = np.empty((tok.shape[0], S, d.d_head))
    lib.ora_prefill_rows(ctypes.byref(d), _ptr(x), _ptr(wq), _ptr(K), _ptr(V), _ptr(sel), _ptr(pt),
                         tok.shape[0], _ptr(tok), _ptr(out))
    return out


def attend_rows(d: _Desc, q_routed, q_shared, K, V, ptilde, tok=None):
    """Attention and slot assembly for tokens ``tok`` given their query rows
    (q_routed [n, G, k, d_head], q_shared [n, d_head] or None, as qproj_rows
    returns them).  Returns out [n, S, d_head] float64."""
    lib = _load()
    qr = _f64(q_routed)
    n = qr.shape[0]
    tok = np.arange(n, dtype=np.int64) if tok is None else np.ascontiguousarray(np.asarray(tok, dtype=np.int64))
    qs = _f64(q_shared) if (d.n_shared and q_shared is not None) else None
    K, V, pt = _f64(K), _f64(V), _f64(ptilde)
    out = np.empty((n, num_slots(d), d.d_head))
    lib.ora_attend_rows(ctypes.byref(d), _ptr(qr), _ptr(qs), _ptr(K), _ptr(V), _ptr(pt), n, _ptr(tok), _ptr(out))
    return out


def kv_proj(d: _Desc, x, w):
    """One of the K / V projections: x [B*T, d_model] (or [B, T, d_model]), w [H_kv, d_head, d_model].
    Returns [B, H_kv, T, d_head] float64."""
    lib = _load()
    x = _f64(x).reshape(d.B * d.T, d.d_model)
    w = _f64(w).reshape(d.H_kv, d.d_head, d.d_model)
    out = np.empty((d.B, d.H_kv, d.T, d.d_head))
    lib.ora_kv_proj(ctypes.byref(d), _ptr(x), _ptr(w), _ptr(out))
    return out


def rope(rows, positions, base: float):
    """Rotary position embedding of rows [..., d_head] at positions [...] (broadcast over the leading axes
    of rows that positions does not cover), float64: pair (c, c + d_head/2) rotated by positions *
    base^(-2c/d_head).  Returns a new array."""
    lib = _load()
    x = np.array(_f64(rows), dtype=np.float64, copy=True)
    dh = x.shape[-1]
    pos = np.asarray(positions, dtype=np.int32)
    pos = np.broadcast_to(pos.reshape(pos.shape + (1,) * (x.ndim - 1 - pos.ndim)), x.shape[:-1])
    flat = np.ascontiguousarray(x.reshape(-1, dh))
    p = np.ascontiguousarray(pos.reshape(-1))
    lib.ora_rope(flat.shape[0], dh, _ptr(p), float(base), _ptr(flat))
    return flat.reshape(x.shape)


def assemble_rows(d: _Desc, slots, ptilde):
    """The weighted slot(s) of token rows whose hard and shared slots are given.

    slots [n, S, d_head] (the weighted slot(s) are ignored), ptilde [n, G, k].
    Returns a float64 copy of ``slots`` with the weighted slot(s) filled.
    """
    lib = _load()
    out = np.array(_f64(slots), dtype=np.float64, copy=True).reshape(-1, num_slots(d), d.d_head)
    pt = _f64(ptilde).reshape(out.shape[0], d.H_kv, d.k)
    lib.ora_assemble_rows(ctypes.byref(d), _ptr(pt), out.shape[0], _ptr(out))
    return out


def out_proj_rows(d: _Desc, slots, w_o):
    """The attention output projection y = h W_o^T of token rows.

    slots [n, S, d_head] (all slots filled), w_o [d_model, S*d_head].
    Returns y [n, d_model] float64.
    """
    lib = _load()
    h = _f64(slots).reshape(-1, num_slots(d), d.d_head)
    wo = _f64(w_o).reshape(d.d_model, num_slots(d) * d.d_head)
    y = np.empty((h.shape[0], d.d_model))
    lib.ora_out_proj_rows(ctypes.byref(d), _ptr(h), _ptr(wo), h.shape[0], _ptr(y))
    return y


def prefill(d: _Desc, inputs: dict, tok=None, routing=None):
    """Full prefill forward from a dict of inputs (x, w_router, b_router, w_q, k, v).

    ``routing`` may carry an agreed selection (sel, ptilde) to attend with;
    by default the oracle's own routing is used.  Returns dict with the
    routing outputs, the compaction and ``out`` for the tokens in ``tok``.
    """
    r = route(d, inputs["x"], inputs["w_router"], inputs.get("b_router"))
    if routing is not None:
        r = dict(r, **routing)
    c = compact(d, r["sel"])
    out = prefill_rows(d, inputs["x"], inputs["w_q"], inputs["k"], inputs["v"], r["sel"], r["ptilde"], tok)
    return dict(r, **c, out=out)


def decode(d: _Desc, x, w_router, b_router, w_q, k_cache, v_cache, lens, routing=None):
    """One decode step per sequence.  x [B, d_model] (or [B, 1, d_model]).

    ``routing`` may carry an agreed selection (sel [B, G, k], ptilde [B, G, k]) to attend with, in place of
    the oracle's own; sel, ptilde and tie in the result are then still the oracle's own routing.
    Returns dict(out [B, S, d_head], sel [B, G, k], ptilde [B, G, k], tie [B, G]).
    """
    lib = _load()
    x = _f64(x).reshape(d.B, d.d_model)
    kc, vc = _f64(k_cache), _f64(v_cache)
    L_max = kc.shape[2]
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    S = num_slots(d)
    out = np.empty((d.B, S, d.d_head))
    sel = np.empty((d.B, d.H_kv, d.k), dtype=np.int32)
    pt = np.empty((d.B, d.H_kv, d.k)); tie = np.empty((d.B, d.H_kv), dtype=np.uint8)
    rc = lib.ora_decode(ctypes.byref(d), _ptr(x), _ptr(_f64(w_router)), _ptr(_f64(b_router)), _ptr(_f64(w_q)),
                        _ptr(kc), _ptr(vc), L_max, _ptr(lens), _ptr(out), _ptr(sel), _ptr(pt), _ptr(tie))
    if rc != 0:
        raise ValueError("oracle decode: invalid shape or cache length")
    if routing is not None:
        rs = np.ascontiguousarray(np.asarray(routing["sel"], dtype=np.int32).reshape(d.B, d.H_kv, d.k))
        rp = np.ascontiguousarray(np.asarray(routing["ptilde"], dtype=np.float64).reshape(d.B, d.H_kv, d.k))
        rc = lib.ora_decode_given(ctypes.byref(d), _ptr(x), _ptr(_f64(w_q)), _ptr(kc), _ptr(vc), L_max, _ptr(lens),
                                  _ptr(rs), _ptr(rp), _ptr(out))
        if rc != 0:
            raise ValueError("oracle decode: invalid cache length")
    return dict(out=out, sel=sel, ptilde=pt, tie=tie.astype(bool))


__all__ = ["build", "desc", "num_slots", "num_threads", "route", "compact", "qproj_rows", "prefill_rows", "prefill",
           "assemble_rows", "out_proj_rows", "kv_proj", "rope",
           "decode", "TIE_MARGIN"]
