"""Host-side tests of the C ABI (CPU only, no kernel is ever launched).

The library must load, export every function include/gqe.h declares, and
reject bad arguments on the host with the documented status codes before
anything is enqueued.  Every call here fails validation, so no HIP call is
made and these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import sparse_routed_query_amd.gqe as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIGN, LAUNCH, WORKSPACE = 0, -1, -2, -3, -4, -5
P = ctypes.c_void_p
A16 = P(0x10000)      # an aligned address that is never dereferenced
MIS = P(0x10008)      # 8-byte aligned only


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gqe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gqe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = G.load()
    names = declared_functions()
    assert len(names) == 10
    assert set(names) == set(G.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def main(**kw):
    d = dict(B=4, T=4096, d_model=1024, H_q=16, H_kv=8, k=1, d_head=64)
    d.update(kw)
    return G.make_desc(**d)


def route_rc(desc, x=A16, wr=A16, br=None, sel=A16, pt=A16, counts=A16, offsets=A16, rows=A16, logits=None,
             ws=A16, ws_bytes=1 << 30):
    return G.load().gqe_route(ctypes.byref(desc) if desc is not None else None, x, wr, br, sel, pt, counts,
                              offsets, rows, logits, ws, ws_bytes, None)


def test_num_slots_and_workspace_sizes():
    assert G.gqe_num_slots(main()) == 10                        # 8 hard + weighted + shared
    assert G.gqe_num_slots(main(route_mode=1)) == 17            # 8 hard + 8 per-group + shared
    assert G.gqe_num_slots(main(k=2, n_shared=0)) == 17         # dense: 16 hard + weighted
    assert G.gqe_num_slots(main(H_q=15)) == -1
    nblk = (4 * 4096 + 31) // 32
    assert G.gqe_route_workspace_bytes(main()) >= 2 * nblk * 16 * 4
    dd = main(B=64, T=1)
    ws = G.gqe_decode_workspace_bytes(dd, 8192)
    assert ws >= 64 * 8 * 2 * (8192 // 256) * 66 * 4
    assert G.gqe_decode_workspace_bytes(dd, 0) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(H_q=15), INVALID),                 # H_q not a multiple of H_kv
    (dict(k=0), INVALID),
    (dict(k=3), INVALID),                    # k > E = 2
    (dict(n_shared=2), INVALID),
    (dict(causal=5), INVALID),
    (dict(route_mode=2), INVALID),
    (dict(B=-1), INVALID),
    (dict(d_head=96), UNSUPPORTED),
    (dict(d_model=1000), UNSUPPORTED),       # bf16 needs d_model % 64 == 0
    (dict(H_q=128, H_kv=8), UNSUPPORTED),    # more experts than the router keeps
    (dict(H_q=80, H_kv=8, k=9), UNSUPPORTED),
])
def test_route_rejects_bad_descriptors(bad, code):
    assert route_rc(main(**bad)) == code


def test_route_rejects_bad_pointers():
    d = main()
    assert route_rc(None) == INVALID
    assert route_rc(d, x=None) == INVALID
    assert route_rc(d, counts=None) == INVALID
    assert route_rc(d, x=MIS) == ALIGN
    assert route_rc(d, rows=MIS) == ALIGN
    assert route_rc(d, br=MIS) == ALIGN
    assert route_rc(d, logits=MIS) == ALIGN
    assert route_rc(d, ws=None) == WORKSPACE
    assert route_rc(d, ws_bytes=G.gqe_route_workspace_bytes(d) - 1) == WORKSPACE


def test_qproj_prefill_decode_reject_bad_arguments():
    lib = G.load()
    d = main()
    by = ctypes.byref
    assert lib.gqe_qproj(by(d), None, A16, A16, A16, A16, A16, A16, A16, None) == INVALID
    assert lib.gqe_qproj(by(d), A16, A16, A16, A16, A16, A16, A16, None, None) == INVALID   # shared head needs q_shared
    assert lib.gqe_qproj(by(d), A16, MIS, A16, A16, A16, A16, A16, A16, None) == ALIGN
    assert lib.gqe_attn_prefill(by(d), A16, A16, A16, None, A16, A16, None) == INVALID
    assert lib.gqe_attn_prefill(by(main(d_head=48)), A16, A16, A16, A16, A16, A16, None) == UNSUPPORTED
    assert lib.gqe_attn_prefill(by(d), A16, A16, A16, A16, A16, MIS, None) == ALIGN
    assert lib.gqe_attn_prefill(by(d), A16, A16, A16, A16, None, A16, None) == INVALID     # p_tilde needed
    assert lib.gqe_attn_prefill_heads(by(d), A16, None, A16, A16, A16, None) == INVALID    # shared head needs q_shared
    assert lib.gqe_attn_prefill_heads(by(main(d_head=48)), A16, A16, A16, A16, A16, None) == UNSUPPORTED
    assert lib.gqe_attn_prefill_heads(by(d), A16, A16, A16, A16, MIS, None) == ALIGN
    assert lib.gqe_assemble(by(d), None, A16, None) == INVALID
    assert lib.gqe_assemble(by(d), A16, MIS, None) == ALIGN
    assert lib.gqe_assemble(by(main(H_q=15)), A16, A16, None) == INVALID
    dd = main(B=64, T=1)
    ws = G.gqe_decode_workspace_bytes(dd, 8192)
    dec = lambda desc, L=8192, lens=A16, w=A16, wb=ws: lib.gqe_attn_decode(  # noqa: E731
        by(desc), A16, A16, A16, A16, L, lens, A16, A16, w, wb, None)
    assert dec(main(B=64, T=2)) == INVALID      # decode is one token per sequence
    assert dec(dd, L=0) == INVALID
    assert dec(dd, lens=None) == INVALID
    assert dec(dd, w=None) == WORKSPACE
    assert dec(dd, wb=ws - 1) == WORKSPACE
    assert dec(dd, lens=MIS) == ALIGN


def test_python_binding_refuses_host_tensors():
    import torch
    d = main(B=1, T=4, d_model=64, H_q=4, H_kv=2, d_head=32, dtype="f32")
    with pytest.raises(ValueError):
        G.gqe_route(d, torch.zeros(4, 64), torch.zeros(4, 64), None, torch.zeros(4, 2, 1, dtype=torch.int32),
                    None, None, None, None, None, None)
