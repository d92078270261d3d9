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
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|size_t|const char\*)\s+(gqe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = G.load()
    names = declared_functions()
    assert len(names) == 31
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
    assert G.gqe_num_slots(main(route_mode=2)) == 9             # 8 hard + shared ("hard concat only")
    assert G.gqe_num_slots(main(route_mode=2, n_shared=0)) == 8
    assert G.gqe_num_slots(main(route_mode=3)) == 9             # 8 scaled hard + shared ("weighted concat")
    assert G.gqe_num_slots(main(route_mode=4)) == -1
    nblk = (4 * 4096 + 31) // 32
    assert G.gqe_route_workspace_bytes(main()) >= 2 * nblk * 16 * 4
    dd = main(B=64, T=1)
    ws = G.gqe_decode_workspace_bytes(dd, 8192)
    # (max, sum, 64 values) in fp32 per sequence, group, row (k = 1 + shared) and 384-key chunk
    assert ws >= 64 * 8 * 2 * -(-8192 // 384) * 66 * 4
    assert G.gqe_decode_workspace_bytes(dd, 0) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(H_q=15), INVALID),                 # H_q not a multiple of H_kv
    (dict(k=0), INVALID),
    (dict(k=3), INVALID),                    # k > E = 2
    (dict(n_shared=2), INVALID),
    (dict(causal=5), INVALID),
    (dict(route_mode=4), INVALID),
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
    assert lib.gqe_qproj(by(d), A16, MIS, A16, A16, A16, A16, A16, A16, None) == ALIGN
    assert lib.gqe_qproj(by(d), A16, A16, None, A16, A16, A16, A16, None, None) == INVALID   # routed part needs sel
    assert lib.gqe_qproj(by(d), A16, A16, A16, A16, A16, A16, MIS, None, None) == ALIGN
    assert lib.gqe_qproj(by(d), None, None, None, None, None, None, None, None, None) == OK  # nothing to compute
    pws = G.gqe_attn_prefill_workspace_bytes(d)
    pf = lambda desc, q=A16, qs=A16, v=A16, pt=A16, out=A16, w=A16, wb=pws: lib.gqe_attn_prefill(  # noqa: E731
        by(desc), q, qs, A16, v, pt, out, w, wb, None)
    hd = lambda desc, qs=A16, out=A16, w=A16, wb=pws: lib.gqe_attn_prefill_heads(  # noqa: E731
        by(desc), A16, qs, A16, A16, out, w, wb, None)
    assert pf(d, v=None) == INVALID
    assert pf(main(d_head=48)) == UNSUPPORTED
    assert pf(d, out=MIS) == ALIGN
    assert pf(d, pt=None) == INVALID                 # p_tilde needed
    assert pf(d, w=MIS) == ALIGN
    assert pf(d, wb=pws - 1) == WORKSPACE
    assert pf(d, q=None) == INVALID                  # the weighted slots need the routed hard slots
    assert lib.gqe_attn_prefill_heads(by(d), None, None, None, None, None, None, 0, None) == OK  # nothing to compute
    assert hd(main(d_head=48)) == UNSUPPORTED
    assert hd(d, out=MIS) == ALIGN
    assert hd(d, w=MIS) == ALIGN
    assert hd(d, wb=0) == WORKSPACE
    assert lib.gqe_assemble(by(d), None, A16, None) == INVALID
    assert lib.gqe_assemble(by(d), A16, MIS, None) == ALIGN
    assert lib.gqe_assemble(by(main(H_q=15)), A16, A16, None) == INVALID
    rws = G.load().gqe_route_backward_workspace_bytes(by(d))
    assert rws >= 64 * 16 * 1025 * 4                       # 64 blocks of 256 tokens x N x (d_model + 1)
    rb = lambda desc, dout=A16, dw=A16, db=A16, dx=A16, w=A16, wb=rws: lib.gqe_route_backward(  # noqa: E731
        by(desc), dout, A16, A16, A16, A16, A16, A16, A16, dw, db, dx, w, wb, None)
    assert rb(d, dout=None) == INVALID
    assert rb(d, dw=None, db=A16) == INVALID     # db only with dw
    assert rb(d, wb=rws - 1) == WORKSPACE
    assert rb(d, w=None) == WORKSPACE
    assert rb(d, dx=MIS) == ALIGN
    assert rb(main(B=0), dout=None, dw=None, db=None, dx=None, w=None) == OK
    rs = lambda desc, lg=A16, imp=A16: lib.gqe_route_stats(by(desc), lg, imp, None)  # noqa: E731
    assert rs(d, lg=None) == INVALID
    assert rs(d, imp=None) == INVALID
    assert rs(d, imp=MIS) == ALIGN
    assert rs(main(H_q=15)) == INVALID
    aws = G.load().gqe_attn_backward_workspace_bytes(by(d))
    assert aws == (4 * 8 * 4096 + 4 * 4096) * 8 + 256          # two floats per routed and shared row
    assert G.load().gqe_attn_backward_workspace_bytes(by(main(n_shared=0))) == 4 * 8 * 4096 * 8 + 256
    ab = lambda desc, q=A16, qs=A16, dh=A16, dq=A16, w=A16, wb=aws: lib.gqe_attn_backward(  # noqa: E731
        by(desc), q, qs, A16, A16, A16, dh, A16, dq, A16, A16, A16, w, wb, None)
    assert ab(d, q=None) == INVALID
    assert ab(d, qs=None) == INVALID             # the shared head's rows are needed with n_shared = 1
    assert ab(d, dh=MIS) == ALIGN
    assert ab(d, w=None) == WORKSPACE
    assert ab(d, wb=aws - 1) == WORKSPACE
    assert ab(main(dtype="f32")) == UNSUPPORTED  # bf16 only
    assert ab(main(d_head=48)) == UNSUPPORTED
    assert ab(main(B=0), q=None, qs=None, dh=None, dq=None, w=None) == OK
    kv = lambda desc, x=A16, wk=A16, wv=A16, k=A16, v=A16: lib.gqe_kv_proj(by(desc), x, wk, wv, k, v, None)  # noqa
    assert kv(d, x=None) == INVALID
    assert kv(d, wv=None) == INVALID
    assert kv(d, k=MIS) == ALIGN
    assert kv(main(d_head=48)) == UNSUPPORTED
    assert kv(main(B=0), x=None, wk=None, wv=None, k=None, v=None) == OK
    op = lambda desc, out=A16, pt=A16, wo=A16, y=A16, ww=0: lib.gqe_out_proj(  # noqa: E731
        by(desc), out, pt, wo, y, ww, None)
    assert op(d, out=None) == INVALID
    assert op(d, pt=None) == INVALID             # the weighted slot(s) need p~
    assert op(d, wo=None) == INVALID
    assert op(d, y=MIS) == ALIGN
    assert op(d, ww=2) == INVALID
    assert op(main(d_head=48)) == UNSUPPORTED
    assert op(main(B=0), out=None, pt=None, wo=None, y=None) == OK   # nothing to compute
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
    pws_ = G.gqe_decode_workspace_bytes(dd, 512 * 16)
    pg = lambda desc, npg=100, P=16, mp=512, bt=A16, w=A16, wb=pws_: lib.gqe_attn_decode_paged(  # noqa: E731
        by(desc), A16, A16, A16, A16, npg, P, mp, bt, A16, A16, A16, w, wb, None)
    assert pg(main(B=64, T=2)) == INVALID       # one token per sequence
    assert pg(dd, P=24) == INVALID              # page size must be a power of two ...
    assert pg(dd, P=4) == INVALID               # ... from 8
    assert pg(dd, npg=0) == INVALID
    assert pg(dd, mp=0) == INVALID
    assert pg(dd, bt=None) == INVALID
    assert pg(dd, bt=MIS) == ALIGN
    assert pg(dd, wb=pws_ - 1) == WORKSPACE     # sized for max_pages * page_size positions
    assert pg(main(B=0, T=1), bt=None, w=None) == OK
    ck = lambda desc, lens=A16, L=64, bt=None, npg=4, P=16, mp=4, bad=A16: lib.gqe_check_decode_inputs(  # noqa: E731
        by(desc), lens, L, bt, npg, P, mp, bad, None)
    assert ck(dd, lens=None) == INVALID
    assert ck(dd, bad=None) == INVALID
    assert ck(dd, L=0) == INVALID
    assert ck(dd, bt=MIS) == ALIGN
    assert ck(dd, bt=A16, mp=2) == INVALID      # the table must cover L_max positions
    assert ck(dd, bt=A16, npg=0) == INVALID


def test_python_binding_refuses_host_tensors():
    import torch
    d = main(B=1, T=4, d_model=64, H_q=4, H_kv=2, d_head=32, dtype="f32")
    with pytest.raises(ValueError):
        G.gqe_route(d, torch.zeros(4, 64), torch.zeros(4, 64), None, torch.zeros(4, 2, 1, dtype=torch.int32),
                    None, None, None, None, None, None)


# ------------------------------------------------------------- prefill schedule

def plan_reference(B, T, G_, k, n_shared, causal, split, d_head=64, split_tiles=32, slots=768):
    """Work items of the prefill attention launch, written out directly: every
    query tile of bm rows (256 at d_head 128, else 128), cut in two when it is
    causal, needs more than 32 key tiles of 64 and its first row sees key
    64*(nkv//2), provided the longest tile needs more key tiles than the average
    load of 768 workgroup slots of 128 rows (768 * 128 / bm slots of bm rows);
    sorted by item size (larger part), routed before shared, split before
    whole, tile descending, split tiles by part then head.  Then, since
    workgroup j runs on XCD j mod 8: in each run of one tile's items over a
    number of heads that is a multiple of 8, the item at position j takes the
    run's head 8*(r//8) + j%8 (r its rank in the run), so all items of a head
    run on one XCD."""
    bm = 256 if d_head == 128 else 128

    def nkv_of(i, kk):
        if not causal:
            return -(-T // 64)
        return (min(T * kk - 1, bm * (i + 1) - 1) // kk) // 64 + 1
    units = sum(nkv_of(i, k) * B * G_ for i in range(-(-T * k // bm)))
    units += sum(nkv_of(i, 1) * B for i in range(-(-T // bm))) if n_shared else 0
    split = split and causal and -(-T // 64) * slots * 128 // bm > units
    items = []
    n_pairs_r = 0
    for lst, (kk, heads) in enumerate(((k, [(b, g) for b in range(B) for g in range(G_)]),
                                       (1, [(b, G_) for b in range(B)] if n_shared else []))):
        R = T * kk
        nt = -(-R // bm)

        def nkv(i):
            if not causal:
                return -(-T // 64)
            return (min(R - 1, bm * (i + 1) - 1) // kk) // 64 + 1

        def can(i):
            return causal and nkv(i) > split_tiles and 64 * (nkv(i) // 2) <= (bm * i) // kk
        first_split = nt
        while split and first_split > 0 and can(first_split - 1):
            first_split -= 1
        base = n_pairs_r if lst else 0
        for i in range(nt):
            n = nkv(i)
            for hi in range(len(heads)):
                if i >= first_split:
                    for part in (0, 1):   # part-major: all part 0s of a tile, then all part 1s
                        items.append(((-(n - n // 2), lst, 0, -i, part, hi), (heads, hi, i, part, base, first_split)))
                else:
                    items.append(((-n, lst, 1, -i, hi, 0), (heads, hi, i, -1, base, first_split)))
        if lst == 0:
            n_pairs_r = (nt - first_split) * len(heads)
    items.sort(key=lambda it: it[0])
    out = []
    for j, (_, (heads, r, i, part, base, first_split)) in enumerate(items):
        hi = 8 * (r // 8) + j % 8 if len(heads) % 8 == 0 else r
        b, h = heads[hi]
        pair = base + (i - first_split) * len(heads) + hi if part >= 0 else -1
        out.append((b, h, i, part, pair))
    return out


@pytest.mark.parametrize("shape", [
    dict(B=4, T=4096, k=1, n_shared=1, causal=1),     # the 250M-model shape
    dict(B=1, T=32768, k=1, n_shared=1, causal=1),    # long: longest-first order is enough, nothing split
    dict(B=2, T=4000, k=3, n_shared=1, causal=1),     # ragged rows, three kept experts
    dict(B=1, T=8192, k=2, n_shared=0, causal=1),
    dict(B=3, T=2100, k=1, n_shared=1, causal=0),     # non-causal: nothing split
    dict(B=2, T=300, k=2, n_shared=1, causal=1),      # short: nothing split
    dict(B=1, T=1, k=1, n_shared=1, causal=1),
    dict(B=2, T=16384, k=2, n_shared=1, causal=1, d_head=128),   # wide_zipf's shape: 256-row tiles
    dict(B=4, T=4096, k=1, n_shared=1, causal=1, d_head=128),
    dict(B=2, T=700, k=3, n_shared=0, causal=1, d_head=128),
    dict(B=1, T=5000, k=1, n_shared=1, causal=0, d_head=32),
])
def test_prefill_plan_matches_its_definition(shape):
    dh = shape.get("d_head", 64)
    d = main(B=shape["B"], T=shape["T"], k=shape["k"], H_q=8 * max(2, shape["k"]), n_shared=shape["n_shared"],
             causal=shape["causal"], d_head=dh)
    for split in (False, True):
        got = [tuple(int(x) for x in r) for r in G.gqe_attn_prefill_plan(d, split)]
        want = plan_reference(shape["B"], shape["T"], 8, shape["k"], shape["n_shared"], shape["causal"], split, dh)
        assert got == want, (split, len(got), len(want))
    plan = G.gqe_attn_prefill_plan(d, True)
    # 8 groups per batch here, so every routed head's items (whole or either half) share one XCD, j mod 8
    assert all(j % 8 == (int(r[0]) * 8 + int(r[1])) % 8 for j, r in enumerate(plan) if r[1] < 8)
    pairs = sorted((int(r[4]), int(r[3])) for r in plan if r[3] >= 0)
    n_pairs = len(pairs) // 2
    assert pairs == [(p, part) for p in range(n_pairs) for part in (0, 1)]
    threads = 512 if dh == 128 else 256   # two per query row of a tile
    want_bytes = 0 if n_pairs == 0 else -(-n_pairs * 4 // 256) * 256 + n_pairs * 2 * threads * (dh // 2 + 2) * 4
    assert G.gqe_attn_prefill_workspace_bytes(d) == want_bytes


def test_prefill_workspace_only_for_split_shapes():
    assert G.gqe_attn_prefill_workspace_bytes(main()) > 0
    assert G.gqe_attn_prefill_workspace_bytes(main(causal=0)) == 0
    assert G.gqe_attn_prefill_workspace_bytes(main(T=2048)) == 0           # at most 32 key tiles
    assert G.gqe_attn_prefill_workspace_bytes(main(B=1, T=32768)) == 0     # balanced without splitting
    assert G.gqe_attn_prefill_workspace_bytes(main(dtype="f32")) == 0
    assert G.load().gqe_attn_prefill_plan(ctypes.byref(main(dtype="f32")), 1, None, 0) == UNSUPPORTED


def test_noalloc_decode_rejects_more_than_its_static_scratch():
    """A call whose split partials exceed GQE_DECODE_SCRATCH_BYTES returns GQE_ERR_SCRATCH on the host, before
    the scratch is looked up or anything is enqueued; bad descriptors and pointers fail as in gqe_attn_decode."""
    SCRATCH = -6
    lib = G.load()

    def rc(desc, L_max=8192, lens=A16):
        return lib.gqe_attn_decode_noalloc(ctypes.byref(desc), A16, A16, A16, A16, L_max, lens, A16, A16, None)

    big = main(B=256, T=1)                                     # 256 * 8 * 2 * 22 * 66 * 4 B = 23.8 MB
    assert G.gqe_decode_workspace_bytes(big, 8192) > G.DECODE_SCRATCH_BYTES
    assert rc(big) == SCRATCH
    assert G.gqe_decode_workspace_bytes(main(B=64, T=1), 8192) <= G.DECODE_SCRATCH_BYTES
    assert rc(main(B=64, T=2)) == INVALID                      # decode is one token per sequence
    assert rc(main(B=64, T=1), L_max=0) == INVALID
    assert rc(big, lens=None) == INVALID
    assert rc(big, lens=MIS) == ALIGN
    assert lib.gqe_status_string(SCRATCH) == b"call needs more than the static scratch holds"


def test_route_backward_rejects_the_weighted_concat_mode():
    """Route mode 3 scales hard slots by the group softmax, whose gradient reaches experts that were not kept;
    its routing backward is not built and is refused on the host."""
    lib = G.load()
    d = main(route_mode=3)
    rc = lib.gqe_route_backward(ctypes.byref(d), A16, A16, A16, A16, A16, A16, A16, A16, None, None, None, None, 0,
                                None)
    assert rc == UNSUPPORTED


def test_decode_route_qproj_rejects_prefill_shapes_bad_rope_base_and_pointers():
    lib = G.load()

    def rc(d, base=0.0, positions=None, x=A16, qs=A16, sel=A16):
        return lib.gqe_decode_route_qproj(ctypes.byref(d), x, A16, None, A16, positions, ctypes.c_float(base), sel,
                                          A16, A16, qs, None, None)

    dec = main(B=64, T=1)
    assert rc(main()) == INVALID                 # T = 4096: one token per sequence only
    assert rc(main(B=64, T=2)) == INVALID
    assert rc(dec, 10000.0) == INVALID           # rotation needs the positions
    assert rc(dec, 1.0, A16) == INVALID
    assert rc(dec, float("nan"), A16) == INVALID
    assert rc(dec, float("inf"), A16) == INVALID
    assert rc(dec, x=None) == INVALID
    assert rc(dec, sel=None) == INVALID
    assert rc(dec, qs=None) == INVALID           # the shared head is on
    assert rc(dec, 10000.0, MIS) == ALIGN
    assert rc(main(B=0, T=1), x=None) == OK      # empty batch: nothing to do, no pointer read


def test_attention_lse_entries_reject_fp32_and_missing_statistics():
    lib = G.load()
    d = main()
    f32 = main(dtype="f32")
    heads = lambda desc, lse=A16: lib.gqe_attn_prefill_heads_lse(ctypes.byref(desc), A16, A16, A16, A16, A16, lse,  # noqa: E731
                                                                None, 0, None)
    assert heads(f32) == UNSUPPORTED
    assert heads(d, None) == INVALID
    assert heads(d, MIS) == ALIGN
    bwd = lambda desc, lse=A16, ws=A16: lib.gqe_attn_backward_lse(  # noqa: E731
        ctypes.byref(desc), A16, A16, A16, A16, A16, A16, A16, lse, A16, A16, A16, A16, ws, 1 << 40, None)
    assert bwd(f32) == UNSUPPORTED
    assert bwd(d, None) == INVALID
    assert bwd(d, ws=None) == WORKSPACE


def test_out_proj_packed_sizes_and_rejects():
    lib = G.load()
    d = main()
    K = d.H_kv * d.k * d.d_head + 2 * d.d_head                   # S = kG + 2 slots of d_head
    assert G.gqe_out_proj_packed_bytes(d) == d.d_model * K * 2
    assert G.gqe_out_proj_packed_bytes(main(dtype="f32")) == 0
    assert G.gqe_out_proj_packed_bytes(main(H_q=32, H_kv=8, k=2, d_head=128)) == 0   # 64 x (2304 + 8) x 2 > 160 KiB
    assert lib.gqe_out_proj_pack(ctypes.byref(main(dtype="f32")), A16, A16, None) == UNSUPPORTED
    assert lib.gqe_out_proj_pack(ctypes.byref(d), None, A16, None) == INVALID
    assert lib.gqe_out_proj_pack(ctypes.byref(d), A16, MIS, None) == ALIGN
    op = lambda desc, wp=A16, ww=0: lib.gqe_out_proj_packed(ctypes.byref(desc), A16, A16, wp, A16, ww, None)  # noqa: E731
    assert op(main(dtype="f32")) == UNSUPPORTED
    assert op(d, ww=2) == INVALID
    assert op(d, wp=None) == INVALID
    assert op(main(B=0)) == OK


def test_qkv_proj_rejects_bad_rope_base_and_pointers():
    lib = G.load()
    d = main()

    def rc(base, positions=None, x=A16, qs=A16):
        return lib.gqe_qkv_proj(ctypes.byref(d), x, A16, A16, A16, A16, A16, A16, A16, positions, ctypes.c_float(base),
                                A16, qs, A16, A16, None)

    assert rc(1.0) == INVALID                    # base 1: every pair the same frequency
    assert rc(0.5) == INVALID
    assert rc(-3.0) == INVALID
    assert rc(float("nan")) == INVALID
    assert rc(float("inf")) == INVALID
    assert rc(10000.0, x=None) == INVALID
    assert rc(10000.0, qs=None) == INVALID       # the shared head is on
    assert rc(10000.0, positions=MIS) == ALIGN
