"""The C-ABI library loads, exports every symbol include/eta.h declares, and rejects
invalid arguments before anything is enqueued (CPU only: no valid call is made,
so no kernel is ever launched here)."""
import ctypes
import os
import re

import pytest
import torch

from long_context_decode_predict_amd import _lib
from long_context_decode_predict_amd.build import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # a 256-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    ensure_built()
    return _lib.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "eta.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(eta_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 18, names
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_defaults_and_strings(L):
    p = L.eta_default_params()
    assert (p.gate_beta, p.z, p.gate_hard, p.bound_mode, p.split_blocks) == (5.0, 4.0, 0, 0, 0)
    for st, s in [(0, "ETA_OK"), (-1, "ETA_ERR_INVALID_ARG"), (-2, "ETA_ERR_UNSUPPORTED"),
                  (-3, "ETA_ERR_WORKSPACE"), (-4, "ETA_ERR_HIP"), (7, "ETA_ERR_UNKNOWN")]:
        assert _lib.status_string(st) == s
    assert [L.eta_nblk_cap(t) for t in (0, 1, 64, 65, 256, 257, 2048, 131072)] == \
        [0, 4, 4, 4, 4, 8, 32, 2048]
    # split-KV item: 8 blocks per query head of a key/value unit unless given
    d = L.eta_default_params()
    assert [_lib.split_blocks(32, H, Hkv, 32768, d)
            for H, Hkv in ((16, 0), (16, 16), (8, 4), (32, 8), (64, 8))] == [8, 8, 16, 32, 64]
    # doubled from 2^20 unit blocks (B * H_kv * nblk_cap) on
    assert [_lib.split_blocks(B, 16, 16, T, d) for B, T in ((64, 131072), (64, 65536),
                                                          (63, 65536), (32, 65536))] == [16, 16, 8, 8]
    assert _lib.split_blocks(32, 32, 8, 32768, _lib.default_params(split_blocks=5)) == 5
    assert _lib.split_blocks(32, 32, 8, 32768, _lib.default_params(split_blocks=-1)) == 0
    assert L.eta_split_blocks(None, BY(d)) == 0
    assert L.eta_split_blocks(BY(shape(H=8, H_kv=3)), BY(d)) == 0  # invalid shape
    assert L.eta_split_blocks(BY(shape(H=24, H_kv=2)), BY(d)) == 0  # unsupported G
    assert L.eta_split_blocks(BY(shape()), None) == 0


def shape(**kw):
    s = dict(B=2, H=3, d=128, T=1000, T_cap=1024, block=64, kv_dtype=1, H_kv=0)
    s.update(kw)
    return _lib.eta_shape(**s)


def meta(T_cap=1024, **kw):
    m = dict(centroid=FAKE, var=FAKE, maxnorm=FAKE, nblk_cap=_lib.nblk_cap(T_cap))
    m.update(kw)
    return _lib.eta_meta(**m)


BY = ctypes.byref
INV, UNS, WSP = _lib.ETA_ERR_INVALID_ARG, _lib.ETA_ERR_UNSUPPORTED, _lib.ETA_ERR_WORKSPACE


@pytest.mark.parametrize("s,st", [
    (None, INV),
    (dict(d=96), UNS), (dict(d=256), UNS), (dict(block=32), UNS), (dict(kv_dtype=5), UNS),
    (dict(T=1025), INV), (dict(T=-1), INV), (dict(B=0), INV), (dict(H=0), INV),
    (dict(T_cap=0, T=0), INV), (dict(T_cap=1000, T=900), INV),
    (dict(H=6, H_kv=4), INV), (dict(H=6, H_kv=-1), INV), (dict(H=12, H_kv=1), UNS),
    (dict(H=6, H_kv=2), UNS),
])
def test_build_meta_shape_errors(L, s, st):
    sp = None if s is None else BY(shape(**s))
    assert L.eta_build_block_meta(sp, FAKE, BY(meta()), None) == st


def test_build_meta_meta_and_pointer_errors(L):
    s = BY(shape())
    assert L.eta_build_block_meta(s, FAKE, None, None) == INV
    assert L.eta_build_block_meta(s, None, BY(meta()), None) == INV
    assert L.eta_build_block_meta(s, FAKE + 2, BY(meta()), None) == INV  # misaligned K
    assert L.eta_build_block_meta(s, FAKE, BY(meta(nblk_cap=20)), None) == INV
    assert L.eta_build_block_meta(s, FAKE, BY(meta(centroid=FAKE + 4)), None) == INV
    assert L.eta_build_block_meta(s, FAKE, BY(meta(var=None)), None) == INV


def test_append_errors(L):
    s = BY(shape(T=1000))
    assert L.eta_append_meta(s, 0, FAKE, BY(meta()), None) == INV
    assert L.eta_append_meta(s, 25, FAKE, BY(meta()), None) == INV  # past T_cap
    assert L.eta_append_meta(BY(shape(d=80)), 1, FAKE, BY(meta()), None) == UNS


def test_predict_errors(L):
    assert L.eta_predict_tau(0, 4, 64, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_predict_tau(1, 0, 64, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_predict_tau(1, 4, 64, None, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_predict_tau(1, 4, 64, FAKE, FAKE, None, FAKE, None) == INV
    assert L.eta_predict_tau(1, 4, 64, FAKE, FAKE, FAKE, None, None) == INV


def params(**kw):
    return _lib.default_params(**kw)


@pytest.mark.parametrize("kw", [dict(gate_beta=0.0), dict(gate_beta=float("inf")),
                                dict(gate_beta=float("nan")), dict(z=-1.0), dict(z=float("inf")),
                                dict(bound_mode=3), dict(bound_mode=-1), dict(split_blocks=-1),
                                dict(split_blocks=5000)])
def test_screen_param_errors(L, kw):
    p = params(**kw)
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), BY(p), FAKE, FAKE, None, None) == INV


def test_centered_bound_needs_distances(L):
    """ETA_BOUND_CENTERED reads eta_meta.maxdev2: rejected before any launch when it is
    NULL or not 16-byte aligned (the other modes ignore a NULL maxdev2)."""
    p = BY(params(bound_mode=2))
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), p, FAKE, FAKE, None, None) == INV
    m = meta()
    m.maxdev2 = FAKE + 4
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(m), p, FAKE, FAKE, None, None) == INV
    assert L.eta_predict_screen(BY(shape()), FAKE, None, FAKE, BY(meta()), p, FAKE, FAKE, FAKE,
                                None, None) == INV
    assert L.eta_build_block_meta(BY(shape()), FAKE, BY(m), None) == INV


def test_screen_other_errors(L):
    p = BY(params())
    assert L.eta_screen(BY(shape()), None, FAKE, BY(meta()), p, FAKE, FAKE, None, None) == INV
    assert L.eta_screen(BY(shape()), FAKE, None, BY(meta()), p, FAKE, FAKE, None, None) == INV
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), p, None, FAKE, None, None) == INV
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), p, FAKE, None, None, None) == INV
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), None, FAKE, FAKE, None, None) == INV
    assert L.eta_screen(BY(shape()), FAKE, FAKE, BY(meta()), p, FAKE, FAKE, FAKE + 4, None) == INV
    # a hard gate does not need a finite beta
    assert L.eta_screen(BY(shape(d=32)), FAKE, FAKE, BY(meta()), BY(params(gate_hard=1, gate_beta=0.0)),
                        FAKE, FAKE, None, None) == UNS


def test_predict_screen_errors(L):
    p = BY(params())
    call = lambda **kw: L.eta_predict_screen(
        BY(shape(**kw.get("shape", {}))), kw.get("q", FAKE), kw.get("W", FAKE), kw.get("bias", FAKE),
        BY(meta()), kw.get("p", p), kw.get("tau", FAKE), kw.get("idx", FAKE), kw.get("cnt", FAKE),
        kw.get("bound", None), None)
    assert call(q=None) == INV
    assert call(bias=None) == INV
    assert call(tau=None) == INV
    assert call(idx=None) == INV
    assert call(cnt=None) == INV
    assert call(p=None) == INV
    assert call(bound=FAKE + 8) == INV
    assert call(shape=dict(d=100)) == UNS
    assert call(shape=dict(T=2000)) == INV


def test_union_errors(L):
    s = BY(shape(H=8, H_kv=2))
    assert L.eta_admit_union(s, None, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_admit_union(s, FAKE, None, FAKE, FAKE, None) == INV
    assert L.eta_admit_union(s, FAKE, FAKE, None, FAKE, None) == INV
    assert L.eta_admit_union(s, FAKE, FAKE, FAKE, None, None) == INV
    assert L.eta_admit_union(BY(shape(H=8, H_kv=3)), FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_admit_union(BY(shape(H=24, H_kv=2)), FAKE, FAKE, FAKE, FAKE, None) == UNS


def test_workspace_size(L):
    p = params()
    n1 = L.eta_decode_attn_workspace_size(BY(shape(T_cap=1024)), BY(p))
    n2 = L.eta_decode_attn_workspace_size(BY(shape(T_cap=4096, T=0)), BY(p))
    assert n1 > 0 and n2 > n1 and n1 % 256 == 0
    assert L.eta_decode_attn_workspace_size(BY(shape(d=7)), BY(p)) == 0
    assert L.eta_decode_attn_workspace_size(BY(shape()), None) == 0
    small = L.eta_decode_attn_workspace_size(BY(shape(T_cap=4096, T=0)),
                                             BY(params(split_blocks=4096)))
    assert 0 < small < n2


def test_decode_attn_errors(L):
    s = BY(shape())
    p = params()
    need = L.eta_decode_attn_workspace_size(s, BY(p))
    args = lambda **kw: dict(dict(q=FAKE, K=FAKE, V=FAKE, tau=FAKE, idx=FAKE, cnt=FAKE,
                                  out=FAKE, lse=None, ws=FAKE, ws_bytes=need), **kw)

    def call(**kw):
        a = args(**kw)
        return L.eta_decode_attn(s, a["q"], a["K"], a["V"], a["tau"], a["idx"], a["cnt"], BY(p),
                                 a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    assert call(ws_bytes=need - 1) == WSP
    assert call(ws=None) == WSP
    assert call(ws=FAKE + 128) == WSP
    assert call(out=None) == INV
    assert call(q=None) == INV
    assert call(K=FAKE + 8) == INV
    assert call(cnt=None) == INV
    # arrays read with scalar loads (wave-uniform index) must be word aligned
    for name in ("q", "tau", "idx", "cnt"):
        assert call(**{name: FAKE + 2}) == INV, name
    assert L.eta_decode_attn(BY(shape(d=48)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BY(p), FAKE,
                             None, FAKE, need, None) == UNS
    # bf16, d = 64: rows are 8-byte aligned, but grouped heads read K in 16-byte chunks
    g = BY(shape(H=4, H_kv=2, d=64))
    need_g = L.eta_decode_attn_workspace_size(g, BY(p))
    assert L.eta_decode_attn(g, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, BY(p), FAKE, None, FAKE,
                             need_g, None) == INV
    assert L.eta_decode_attn_partial(g, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, BY(p), FAKE, None,
                                     FAKE, need_g, None) == INV


def test_decode_attn_noalloc_errors(L):
    """The allocation-free variant validates everything before its first HIP call
    (the device query): invalid operands, and a shape whose workspace exceeds the
    library's per-GPU array, return without touching the runtime."""
    p = params()
    s = BY(shape())
    ok = dict(q=FAKE, K=FAKE, V=FAKE, tau=FAKE, idx=FAKE, cnt=FAKE, out=FAKE)

    def call(sh=s, **kw):
        a = dict(ok, **kw)
        return L.eta_decode_attn_noalloc(sh, a["q"], a["K"], a["V"], a["tau"], a["idx"],
                                         a["cnt"], BY(p), a["out"], None, None)
    assert call(q=None) == INV
    assert call(out=None) == INV
    assert call(cnt=None) == INV
    assert call(idx=None) == INV
    assert call(K=FAKE + 8) == INV
    assert call(tau=FAKE + 2) == INV
    assert call(cnt=FAKE + 2) == INV
    assert call(sh=BY(shape(d=48))) == UNS
    assert L.eta_decode_attn_noalloc(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                     None) == INV
    # B = 64, H = 16, T_cap = 128K fits (d = 128, default split); 4x the cache does not
    fits = BY(shape(B=64, H=16, d=128, T=0, T_cap=131072))
    big = BY(shape(B=64, H=16, d=128, T=0, T_cap=4 * 131072))
    assert 0 < L.eta_decode_attn_workspace_size(fits, BY(p)) <= _lib.NOALLOC_SCRATCH_BYTES
    assert L.eta_decode_attn_workspace_size(big, BY(p)) > _lib.NOALLOC_SCRATCH_BYTES
    assert call(sh=big) == WSP


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((1, 2, 64))
    with pytest.raises(ValueError):
        _lib.eta_predict_tau(q, None, torch.zeros(2), torch.zeros((1, 2)))


def test_layout_errors(L):
    """Paged / variable-length descriptors: a page table needs a positive pool size,
    a pool size needs a page table, and both arrays must be int32-aligned."""
    m = BY(meta())
    assert L.eta_build_block_meta(BY(shape(page_table=FAKE, num_pages=0)), FAKE, m, None) == INV
    assert L.eta_build_block_meta(BY(shape(page_table=FAKE, num_pages=-3)), FAKE, m, None) == INV
    assert L.eta_build_block_meta(BY(shape(num_pages=5)), FAKE, m, None) == INV
    assert L.eta_build_block_meta(BY(shape(seq_lens=FAKE + 2)), FAKE, m, None) == INV
    assert L.eta_build_block_meta(BY(shape(page_table=FAKE + 2, num_pages=4)), FAKE, m, None) == INV
    assert L.eta_build_block_meta(BY(shape(page_table=FAKE, num_pages=1 << 30)), FAKE, m,
                                  None) == INV  # pool offsets bounded
    p = BY(params())
    assert L.eta_screen(BY(shape(num_pages=2)), FAKE, FAKE, m, p, FAKE, FAKE, None, None) == INV
    s = BY(shape(page_table=FAKE, num_pages=0))
    assert L.eta_decode_attn_workspace_size(s, p) == 0
    # the workspace does not depend on the layout
    assert (L.eta_decode_attn_workspace_size(BY(shape(seq_lens=FAKE, page_table=FAKE,
                                                      num_pages=9)), p)
            == L.eta_decode_attn_workspace_size(BY(shape()), p))
    # the block stride: 0, or a positive multiple of 64*d, in the dense and paged layouts
    for bad in (-64 * 128, 64 * 128 + 8, 64 * 64):
        assert L.eta_build_block_meta(BY(shape(kv_block_stride=bad)), FAKE, m, None) == INV, bad
        assert L.eta_build_block_meta(BY(shape(kv_block_stride=bad, page_table=FAKE,
                                               num_pages=4)), FAKE, m, None) == INV, bad
    assert L.eta_decode_attn_workspace_size(BY(shape(kv_block_stride=128 * 128,
                                                     page_table=FAKE, num_pages=4)), p) > 0
    assert L.eta_decode_attn_workspace_size(BY(shape(kv_block_stride=100)), p) == 0
    assert (L.eta_decode_attn_workspace_size(BY(shape(kv_block_stride=128 * 128)), p)
            == L.eta_decode_attn_workspace_size(BY(shape()), p))
    assert (L.eta_decode_attn_workspace_size(BY(shape(d=64, kv_block_stride=64 * 64 * 3)), p)
            > 0)


def test_block_view_binding_checks():
    """The binding derives kv_block_stride from a 5-d block view of K/V and refuses
    views whose blocks are not whole multiples of 64*d apart, or whose units are not
    packed (host-side checks only; the tensors are never handed to the library)."""
    B, Hk, nb, d = 2, 3, 4, 64
    kv = torch.empty((B, Hk, nb, 2, 64, d), dtype=torch.bfloat16, device="meta")
    K, V = kv[:, :, :, 0], kv[:, :, :, 1]
    assert _lib.kv_block_view(K) and _lib.kv_block_stride(K) == 2 * 64 * d
    assert _lib.kv_dims(K) == (B, Hk, nb * 64, d, 0)
    assert _lib.kv_block_stride(torch.empty((B, Hk, nb * 64, d), device="meta")) == 0
    with pytest.raises(ValueError):  # a block view is a dense layout, not a pool
        _lib.kv_dims(K, _lib.KVLayout(None, torch.zeros((B, nb), dtype=torch.int32)))
    for bad in (torch.empty((B, Hk, 64, nb, d), device="meta").transpose(2, 3),  # rows apart
                torch.empty((B, Hk, nb, 64, d + 8), device="meta")[..., :d],      # padded rows
                torch.empty((Hk, B, nb, 64, d), device="meta").transpose(0, 1)):  # units apart
        with pytest.raises(ValueError, match="block view"):
            _lib._check_kv(bad)
    with pytest.raises(ValueError, match="device tensor"):  # a good view, but on the host
        _lib._check_kv(torch.empty((B, Hk, nb, 2, 64, d))[:, :, :, 0])
    # page pools given block by block: a strided 4-d view [P, H_kv, 64, d]
    P = 5
    pool = torch.empty((P, Hk, 2, 64, d), dtype=torch.bfloat16, device="meta")
    Kp = pool[:, :, 0]
    assert _lib.kv_pool_view(Kp) and _lib.kv_block_stride(Kp) == 2 * 64 * d
    table = _lib.KVLayout(None, torch.zeros((B, nb), dtype=torch.int32))
    assert _lib.kv_dims(Kp, table) == (B, Hk, nb * 64, d, P)
    with pytest.raises(ValueError, match="page-pool view"):  # strided 4-d without a table
        _lib.kv_dims(Kp)
    for bad in (torch.empty((Hk, P, 64, d), device="meta").transpose(0, 1),   # pages apart
                torch.empty((P, Hk, 64, d + 8), device="meta")[..., :d]):     # padded rows
        with pytest.raises(ValueError, match="pool view"):
            _lib._check_kv(bad)
    with pytest.raises(ValueError, match="device tensor"):
        _lib._check_kv(torch.empty((P, Hk, 2, 64, d))[:, :, 0])


def test_page_pool_round_trip():
    """The page-pool generator: every row's logical keys read back through the table,
    absent blocks carry out-of-range ids, unused pages are NaN (host only)."""
    import torch
    from long_context_decode_predict_amd import workloads as wl
    w = wl.custom("pp", B=4, H=2, d=64, T=300, kv_dtype=torch.float32, seed=5)
    d = wl.generate(w, "cpu", T_cap=320)
    lens = [300, 0, 65, 64]
    tbl, Kp, Vp = wl.page_pool(d["K"], d["V"], lens, 5, spare=2)
    P = Kp.shape[0]
    assert P == 5 + 0 + 2 + 1 + 2
    used = set()
    for b, t in enumerate(lens):
        nb = (t + 63) // 64
        row = tbl[b].tolist()
        assert all(0 <= x < P for x in row[:nb]) and all(x < 0 or x >= P for x in row[nb:])
        used |= set(row[:nb])
        for k in range(2):
            assert torch.equal(wl.gather_unit(Kp, tbl, b, k, t), d["K"][b, k, :t])
            assert torch.equal(wl.gather_unit(Vp, tbl, b, k, t), d["V"][b, k, :t])
    assert len(used) == P - 2  # distinct pages, two spares
    for x in set(range(P)) - used:
        assert torch.isnan(Kp[x]).all() and torch.isnan(Vp[x]).all()
    assert torch.isnan(Kp[tbl[2, 1], :, 1:]).all()  # past row 2's length in its last page
    lens_w = wl.row_lengths(wl.WORKLOADS["paged_b64_h16_d128_t128k_bf16"])
    assert max(lens_w) == 131072 and min(lens_w) >= 65536 and len(lens_w) == 64


def pshape(**kw):
    s = dict(B=2, H=4, H_kv=0, d=128, T_q=100, T_k=300)
    s.update(kw)
    return _lib.eta_prefill_shape(**s)


@pytest.mark.parametrize("kw,st", [
    (dict(d=96), UNS), (dict(B=0), INV), (dict(H=0), INV), (dict(T_q=-1), INV),
    (dict(T_q=400), INV), (dict(H_kv=3), INV), (dict(H=16, H_kv=1), UNS), (dict(H_kv=-2), INV),
    (dict(T_q=65535 * 128 + 1, T_k=65535 * 128 + 1), INV),
])
def test_prefill_shape_errors(L, kw, st):
    p = BY(params())
    assert L.eta_prefill_attn(BY(pshape(**kw)), FAKE, FAKE, FAKE, FAKE, p, FAKE, None, None,
                              None) == st
    assert L.eta_prefill_predict_tau(BY(pshape(**kw)), FAKE, FAKE, FAKE, FAKE, None) == st


@pytest.mark.parametrize("d,T_k", [(128, 1 << 23), (64, 1 << 24), (128, (1 << 31) - 1)])
def test_prefill_slab_limit(L, d, T_k):
    """One row's K (or V) of one head must stay under 2^31 bytes for the forward (it
    is addressed through a buffer resource); the predictor does not read K and takes
    the shape."""
    s = BY(pshape(d=d, T_q=100, T_k=T_k))
    assert L.eta_prefill_attn(s, FAKE, FAKE, FAKE, FAKE, BY(params()), FAKE, None, None,
                              None) == INV


def test_prefill_pointer_errors(L):
    s, p = BY(pshape()), BY(params())
    call = lambda **kw: L.eta_prefill_attn(s, kw.get("Q", FAKE), kw.get("K", FAKE),
                                           kw.get("V", FAKE), kw.get("tau", FAKE),
                                           kw.get("p", p), kw.get("out", FAKE), None, None, None)
    for k in ("Q", "K", "V", "tau", "out", "p"):
        assert call(**{k: None}) == INV, k
    for k in ("Q", "K", "V", "out"):
        assert call(**{k: FAKE + 8}) == INV, k  # 16-byte alignment
    assert call(p=BY(params(gate_beta=0.0))) == INV
    assert L.eta_prefill_predict_tau(s, None, FAKE, FAKE, FAKE, None) == INV
    assert L.eta_prefill_predict_tau(s, FAKE, FAKE, None, FAKE, None) == INV
    assert L.eta_prefill_predict_tau(s, FAKE, FAKE, FAKE, None, None) == INV
    assert L.eta_prefill_predict_tau(s, FAKE + 4, FAKE, FAKE, FAKE, None) == INV


def test_predict_screen_union_errors(L):
    p = BY(params())
    call = lambda sh, **kw: L.eta_predict_screen_union(
        BY(sh), kw.get("q", FAKE), FAKE, kw.get("bias", FAKE), BY(meta()), p, FAKE, FAKE, FAKE,
        kw.get("uidx", FAKE), kw.get("ucnt", FAKE), None, None)
    g = shape(H=8, H_kv=2)
    assert call(shape()) == INV  # multi-head: no union to form
    assert call(shape(H=8, H_kv=8)) == INV
    assert call(g, uidx=None) == INV
    assert call(g, ucnt=None) == INV
    assert call(g, q=None) == INV
    assert call(g, bias=None) == INV
    assert call(shape(H=8, H_kv=3)) == INV


def test_head_correlated_rows():
    """Multi-head rows with head_corr c: every query and block centroid stays
    N(0, I) per element while the heads of a row share direction c^2 (host only)."""
    import torch
    from long_context_decode_predict_amd import workloads
    w = workloads.custom("hc", B=16, H=8, d=128, T=64 * 64, kv_dtype=torch.float32,
                         head_corr=0.9, sigma=0.0, seed=3)
    data = workloads.generate(w, "cpu")
    q = data["q"].double()
    assert abs(float(q.var()) - 1.0) < 0.1
    qn = q / q.norm(dim=2, keepdim=True)
    cos = (qn[:, :, None, :] * qn[:, None, :, :]).sum(-1)  # [B, H, H]
    off = cos[:, ~torch.eye(w.H, dtype=torch.bool)]
    assert abs(float(off.mean()) - 0.81) < 0.1
    K = data["K"].double().view(w.B, w.H, -1, 64, w.d)[:, :, :, 0]  # sigma 0: keys = centroids
    assert abs(float(K.var()) - 1.0) < 0.05
    kc = (K[:, 0] * K[:, 1]).sum(-1) / (K[:, 0].norm(dim=-1) * K[:, 1].norm(dim=-1))
    assert abs(float(kc.mean()) - 0.81) < 0.05
    # without it the heads are independent
    w0 = workloads.custom("hc0", B=2, H=8, d=128, T=64 * 64, kv_dtype=torch.float32, seed=3)
    q0 = workloads.generate(w0, "cpu")["q"].double()
    q0n = q0 / q0.norm(dim=2, keepdim=True)
    assert abs(float((q0n[:, 0] * q0n[:, 1]).sum(-1).mean())) < 0.2
