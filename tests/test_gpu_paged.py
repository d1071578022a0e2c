"""GPU parity of the paged / variable-length cache layouts.

Rows hold their own token counts (including 0, 1, whole blocks and ragged
tails) and K/V live in a pool of 64-token pages assigned in a shuffled order;
pages no block uses and the rows past a row's length in its last page are NaN,
so any read the layout does not allow shows up. Every case is checked against
the fp64 oracle on each row's logical keys, and the paged run must equal the
dense run with the same lengths bitwise (only addresses differ). Runs on an
MI355X only."""
import numpy as np
import pytest
import torch

from gpu_util import Case, compare_gqa_units, compare_units, kv_host
from long_context_decode_predict_amd import _lib, workloads
from long_context_decode_predict_amd.build import ensure_built
from long_context_decode_predict_amd.decode import DecodeStep
from oracle import oracle as oracle_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ensure_built()
    _lib.lib()
    yield
    torch.cuda.empty_cache()


def _announce(name):
    print(f"\n[case] {name}", flush=True)


def _results(case):
    s = case.step
    return {"tau": s.tau, "cnt": s.adm_cnt, "idx": s.adm_idx, "ucnt": s.uni_cnt,
            "uidx": s.uni_idx, "out": s.out, "lse": s.lse, "U": s.bounds,
            "c": case.meta.centroid, "v": case.meta.var, "m": case.meta.maxnorm,
            "d": case.meta.maxdev2}


def _assert_same(a, b, case):
    """Bitwise equality of two runs on the parts every layout defines."""
    for k in ("tau", "cnt", "ucnt", "out", "lse"):
        assert torch.equal(a[k], b[k]), k
    for bi in range(case.w.B):
        nb = (case.row_len(bi) + 63) // 64
        for k in ("c",):
            assert torch.equal(a[k][bi, ..., :nb], b[k][bi, ..., :nb]), (k, bi)
        for k in ("v", "m", "U") + (("d",) if a["d"] is not None else ()):
            assert torch.equal(a[k][bi, :, :nb], b[k][bi, :, :nb]), (k, bi)
        for k, ck in (("idx", "cnt"), ("uidx", "ucnt")):
            for h in range(a[k].shape[1]):
                n = int(a[ck][bi, h])
                assert torch.equal(a[k][bi, h, :n], b[k][bi, h, :n]), (k, bi, h)


MHA = [
    # name, workload kwargs, row lengths, params
    ("bf16_d128_mixed", dict(B=6, H=4, d=128, T=4100, kv_dtype=torch.bfloat16, seed=201),
     [0, 1, 64, 4100, 2049, 777], {}),
    ("f32_d64_mixed", dict(B=4, H=3, d=64, T=2048, kv_dtype=torch.float32, seed=202),
     [130, 0, 2048, 63], {}),
    ("bf16_d64_split1_hard", dict(B=3, H=2, d=64, T=3000, kv_dtype=torch.bfloat16, seed=203),
     [3000, 129, 1500], {"split_blocks": 1, "gate_hard": 1}),
    ("bf16_d128_two_passes", dict(B=2, H=1, d=128, T=300_000, kv_dtype=torch.bfloat16,
                                  seed=204), [300_000, 170_001], {}),
    ("bf16_d128_centered", dict(B=3, H=2, d=128, T=3000, kv_dtype=torch.bfloat16, seed=205),
     [3000, 65, 1900], {"bound_mode": 2}),
]


@pytest.mark.parametrize("name,kw,lens,pkw", MHA, ids=[c[0] for c in MHA])
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_varlen_and_paged_parity(name, kw, lens, pkw, fused):
    w = workloads.custom(name, **kw)
    _announce(f"varlen {name} lens={lens} fused={fused}")
    params = _lib.default_params(**pkw)
    dense = Case(w, params=params, seq_lens=lens, fused=fused).run()
    st = compare_units(dense, range(w.B * w.H))
    assert st["units"] == w.B * w.H
    assert st["band_mismatch_units"] <= max(1, st["units"] // 50), st
    for b, t in enumerate(lens):
        if t == 0:  # an empty row attends to nothing
            assert torch.all(dense.step.adm_cnt[b] == 0)
            assert torch.all(dense.step.out[b] == 0) and torch.all(torch.isneginf(dense.step.lse[b]))
    ref = {k: (v.clone() if v is not None else None) for k, v in _results(dense).items()}
    dense.free()

    _announce(f"paged {name}")
    paged = Case(w, params=params, seq_lens=lens, paged=True, fused=fused).run()
    assert not torch.isnan(paged.step.out).any()
    _assert_same(ref, _results(paged), paged)
    paged.free()


GQA = [
    ("g4_bf16_d128", dict(B=4, H=16, H_kv=4, d=128, T=5000, kv_dtype=torch.bfloat16,
                          group_corr=0.9, seed=211), [5000, 0, 1234, 64], {}),
    ("g2_f32_d128_hard", dict(B=3, H=4, H_kv=2, d=128, T=1000, kv_dtype=torch.float32,
                              seed=212), [999, 1000, 1], {"gate_hard": 1}),
    ("g8_bf16_d64", dict(B=2, H=16, H_kv=2, d=64, T=2600, kv_dtype=torch.bfloat16,
                         group_corr=0.8, seed=213), [2600, 1900], {}),
    ("g4_bf16_d128_centered", dict(B=2, H=8, H_kv=2, d=128, T=2000, kv_dtype=torch.bfloat16,
                                   group_corr=0.9, seed=214), [2000, 700], {"bound_mode": 2}),
]


@pytest.mark.parametrize("name,kw,lens,pkw", GQA, ids=[c[0] for c in GQA])
def test_grouped_varlen_and_paged_parity(name, kw, lens, pkw):
    w = workloads.custom(name, **kw)
    _announce(f"gqa varlen {name} G={w.G} lens={lens}")
    params = _lib.default_params(**pkw)
    dense = Case(w, params=params, seq_lens=lens, fused=True).run()
    st = compare_gqa_units(dense, range(w.B * w.kv_heads))
    assert st["kv_units"] == w.B * w.kv_heads
    assert st["band_mismatch_units"] <= 1, st
    ref = {k: (v.clone() if v is not None else None) for k, v in _results(dense).items()}
    dense.free()
    paged = Case(w, params=params, seq_lens=lens, paged=True, fused=True).run()
    _assert_same(ref, _results(paged), paged)
    paged.free()


@pytest.mark.parametrize("paged", [False, True], ids=["dense", "paged"])
def test_varlen_append_equals_rebuild_bitwise(paged):
    """Appends with per-row lengths (every row receives the same n_new tokens at its
    own end) equal a rebuild at the grown lengths, in both layouts."""
    _announce(f"varlen append paged={paged}")
    w = workloads.custom("vap", B=4, H=2, d=128, T=3000, kv_dtype=torch.bfloat16, seed=221)
    lens0 = [1000, 0, 63, 2017]
    case = Case(w, seq_lens=lens0, paged=paged, all_pages=True, T_cap=3072)
    K = case.kv()[0]
    tbl = case.layout.page_table
    grown = _lib.Meta.alloc(w.B, w.H, w.d, 3072)
    built = _lib.Meta.alloc(w.B, w.H, w.d, 3072)
    lens = list(lens0)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    _lib.eta_build_block_meta(K, max(lens), grown, layout=_lib.KVLayout(lt, tbl))
    for n in [1, 1, 64, 5, 200, 1]:
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        _lib.eta_append_meta(K, max(lens), n, grown, layout=_lib.KVLayout(lt, tbl))
        lens = [t + n for t in lens]
        lt2 = torch.tensor(lens, dtype=torch.int32, device="cuda")
        _lib.eta_build_block_meta(K, max(lens), built, layout=_lib.KVLayout(lt2, tbl))
        torch.cuda.synchronize()
        for b in range(w.B):
            nb = (lens[b] + 63) // 64
            assert torch.equal(built.centroid[b, ..., :nb], grown.centroid[b, ..., :nb]), (b, lens)
            assert torch.equal(built.var[b, :, :nb], grown.var[b, :, :nb]), (b, lens)
            assert torch.equal(built.maxnorm[b, :, :nb], grown.maxnorm[b, :, :nb]), (b, lens)
    # and the grown metadata matches the oracle on the logical keys
    O = oracle_mod.default()
    for b in range(w.B):
        for h in range(w.H):
            c, v, m = O.block_meta(kv_host(case.data["K"][b, h]), lens[b])
            nb = len(v)
            assert np.max(np.abs(grown.centroid[b, h, :, :nb].cpu().numpy().T - c)) <= 1e-5
            assert np.all(np.abs(grown.var[b, h, :nb].cpu().numpy() - v) <= 1e-5 * v + 1e-12)
            assert np.all(np.abs(grown.maxnorm[b, h, :nb].cpu().numpy() - m) <= 1e-5 * m + 1e-12)
    case.free()


def test_out_of_range_page_is_skipped():
    """A present block whose page id is out of range gets zero metadata and adds no
    token: with tau = -inf (every block admitted) the row's output is the oracle's
    attention over the other blocks; the other rows are untouched."""
    _announce("bad page id")
    w = workloads.custom("bp", B=2, H=2, d=128, T=1000, kv_dtype=torch.bfloat16, seed=231)
    case = Case(w, tau_mode="neg_inf", paged=True)
    bad = 3
    case.layout.page_table[0, bad] = -7
    case.run()
    assert torch.all(case.meta.centroid[0, :, :, bad] == 0)
    assert torch.all(case.meta.var[0, :, bad] == 0) and torch.all(case.meta.maxnorm[0, :, bad] == 0)
    O = oracle_mod.default()
    q = case.data["q"].cpu().numpy()
    nblk = (w.T + 63) // 64
    for b in range(w.B):
        for h in range(w.H):
            idx = np.array([j for j in range(nblk) if b != 0 or j != bad], dtype=np.int32)
            out_o, lse_o = O.attend(q[b, h], kv_host(case.data["K"][b, h]),
                                    kv_host(case.data["V"][b, h]), w.T, -np.inf, idx)
            assert int(case.step.adm_cnt[b, h]) == nblk
            err = float(np.max(np.abs(case.step.out[b, h].cpu().numpy() - out_o)))
            assert err <= 2e-3, (b, h, err)
            assert abs(float(case.step.lse[b, h]) - lse_o) <= 1e-4
    case.free()


def test_paged_graph_follows_layout_updates():
    """A captured step reads the lengths and the page table at replay time: after
    the lengths shrink in place (and the metadata is rebuilt eagerly), a replay
    equals an eager step on the new lengths, bitwise."""
    _announce("paged graph")
    w = workloads.custom("pg", B=4, H=8, d=128, T=6000, kv_dtype=torch.bfloat16, seed=241)
    lens = [6000, 4100, 77, 3000]
    case = Case(w, seq_lens=lens, paged=True, fused=True).run()
    d = case.data
    K, V = case.kv()
    graph = case.step.capture(d["q"], K, V, w.T, case.meta, case.W, case.bias, fused=True)
    for new in ([6000, 4100, 77, 3000], [5000, 64, 0, 2999]):
        case.layout.seq_lens.copy_(torch.tensor(new, dtype=torch.int32))
        case.build_meta()
        case.step(d["q"], K, V, w.T, case.meta, case.W, case.bias, fused=True)
        torch.cuda.synchronize()
        ref = (case.step.out.clone(), case.step.lse.clone(), case.step.adm_cnt.clone())
        for r in range(3):
            case.step.out.zero_()
            case.step.lse.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(case.step.out, ref[0]), (new, r)
            assert torch.equal(case.step.lse, ref[1]), (new, r)
            assert torch.equal(case.step.adm_cnt, ref[2]), (new, r)
    case.row_T = [5000, 64, 0, 2999]
    st = compare_units(case, range(w.B * w.H))
    assert st["band_mismatch_units"] <= 1
    del graph
    case.free()


@pytest.mark.parametrize("G", [1, 4])
def test_interleaved_pages_in_one_buffer(G):
    """K and V pools may share one allocation with their pages interleaved: K page p
    at even page 2p, V page p right after it (V pointer = K pointer + one page, page
    ids doubled). The metadata, the screen and the attention read through the same
    page table, so every result equals the separate-pool run bitwise."""
    _announce(f"interleaved pool pages G={G}")
    w = workloads.custom("ip", B=3, H=4 * G, H_kv=4, d=128, T=5000, kv_dtype=torch.bfloat16,
                         seed=251 + G)
    lens = [5000, 1, 3333]
    case = Case(w, seq_lens=lens, paged=True, fused=True).run()
    ref = {k: (v.clone() if v is not None else None) for k, v in _results(case).items()}
    Kp, Vp = case.kv()
    P = Kp.shape[0]
    buf = torch.empty((2 * P + 1,) + tuple(Kp.shape[1:]), dtype=Kp.dtype, device="cuda")
    buf[0:2 * P:2] = Kp
    buf[1:2 * P:2] = Vp
    buf[2 * P] = float("nan")
    tab = case.layout.page_table
    case.layout = _lib.KVLayout(case.layout.seq_lens,
                                torch.where(tab >= 0, tab * 2, tab).to(torch.int32).contiguous())
    case.data["Kp"], case.data["Vp"] = buf[0:2 * P], buf[1:2 * P + 1]
    case.meta = _lib.Meta.alloc(w.B, w.kv_heads, w.d, case.T_cap)
    case.step = DecodeStep(w.B, w.H, w.d, case.T_cap, w.kv_dtype, case.params, with_bounds=True,
                           H_kv=w.kv_heads, layout=case.layout)
    case.run()
    _assert_same(ref, _results(case), case)
    case.free()


@pytest.mark.parametrize("name,kw,lens", [
    ("mha_bf16_d128_varlen", dict(B=3, H=4, d=128, T=5000, kv_dtype=torch.bfloat16), [5000, 64, 2999]),
    ("mha_f32_d64", dict(B=2, H=3, d=64, T=3000, kv_dtype=torch.float32), None),
    ("gqa4_bf16_d128", dict(B=2, H=16, H_kv=4, d=128, T=4100, kv_dtype=torch.bfloat16), None),
    ("gqa2_f32_d128_varlen", dict(B=2, H=8, H_kv=4, d=128, T=3000, kv_dtype=torch.float32),
     [3000, 1]),
])
def test_block_interleaved_dense_layout(name, kw, lens):
    """K and V interleaved block by block in one allocation (kv [B,H_kv,T_cap/64,2,64,d],
    passed as the block views kv[..., 0, :, :] and kv[..., 1, :, :], kv_block_stride =
    128*d): the metadata, the screen and the attention equal the run on separate
    [B,H_kv,T_cap,d] buffers bitwise, and an append equals a rebuild."""
    _announce(f"block-interleaved {name}")
    w = workloads.custom(name, seed=261, **kw)
    case = Case(w, seq_lens=lens, fused=True).run()
    ref = {k: (v.clone() if v is not None else None) for k, v in _results(case).items()}
    K, V = case.data["K"], case.data["V"]
    B, Hk, Tc, d = K.shape
    nb = Tc // 64
    kv = torch.empty((B, Hk, nb, 2, 64, d), dtype=K.dtype, device="cuda")
    kv[:, :, :, 0] = K.view(B, Hk, nb, 64, d)
    kv[:, :, :, 1] = V.view(B, Hk, nb, 64, d)
    K5, V5 = kv[:, :, :, 0], kv[:, :, :, 1]
    assert _lib.kv_block_stride(K5) == 128 * d
    case.data["Kp"], case.data["Vp"] = K5, V5  # the K, V the library reads
    for t in (case.step.out, case.step.lse, case.meta.centroid, case.meta.var, case.meta.maxnorm):
        t.zero_()
    case.run()
    _assert_same(ref, _results(case), case)
    # and the allocation-free entry point (same kernels and split)
    s = case.step
    out, lse = torch.full_like(s.out, float("nan")), torch.full_like(s.lse, float("nan"))
    _lib.eta_decode_attn_noalloc(case.data["q"], K5, V5, case.T, s.tau, s.uni_idx, s.uni_cnt,
                                 case.params, out, lse, layout=case.layout)
    torch.cuda.synchronize()
    assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
    # the block view also serves appends: every row n tokens shorter, then n more
    n_new = 77 if lens is None else min(lens)
    grown = _lib.Meta.alloc(B, Hk, d, Tc)
    lay = case.layout
    if lay is not None:
        lay.seq_lens.copy_(torch.tensor([t - n_new for t in lens], dtype=torch.int32))
    _lib.eta_build_block_meta(K5, w.T - n_new, grown, layout=lay)
    _lib.eta_append_meta(K5, w.T - n_new, n_new, grown, layout=lay)
    torch.cuda.synchronize()
    for bi in range(B):
        n = (case.row_len(bi) + 63) // 64
        assert torch.equal(grown.centroid[bi, ..., :n], case.meta.centroid[bi, ..., :n]), bi
        assert torch.equal(grown.var[bi, :, :n], case.meta.var[bi, :, :n]), bi
        assert torch.equal(grown.maxnorm[bi, :, :n], case.meta.maxnorm[bi, :, :n]), bi
    case.free()


@pytest.mark.parametrize("G,dtype", [(1, torch.bfloat16), (4, torch.bfloat16), (2, torch.float32)])
def test_block_interleaved_page_pool(G, dtype):
    """A page pool with each (page, head) block's K rows and V rows side by side in one
    allocation ([P,H_kv,2,64,d], passed as the strided views [:, :, 0] and [:, :, 1],
    kv_block_stride = 128*d) gives the separate pools' results bitwise, also through
    the allocation-free entry point; unused pages are NaN in both."""
    _announce(f"block-interleaved pool G={G} {dtype}")
    w = workloads.custom("bip", B=3, H=4 * G, H_kv=4, d=128, T=4500, kv_dtype=dtype,
                         seed=271 + G)
    lens = [4500, 65, 2000]
    case = Case(w, seq_lens=lens, paged=True, fused=True).run()
    ref = {k: (v.clone() if v is not None else None) for k, v in _results(case).items()}
    table, Kp, Vp = workloads.page_pool(case.data["K"], case.data["V"], lens, w.seed,
                                        interleaved=True)
    assert torch.equal(table, case.layout.page_table)
    assert _lib.kv_pool_view(Kp) and _lib.kv_block_stride(Kp) == 128 * w.d
    case.data["Kp"], case.data["Vp"] = Kp, Vp
    for t in (case.step.out, case.step.lse, case.meta.centroid, case.meta.var, case.meta.maxnorm):
        t.zero_()
    case.run()
    _assert_same(ref, _results(case), case)
    s = case.step
    out, lse = torch.full_like(s.out, float("nan")), torch.full_like(s.lse, float("nan"))
    _lib.eta_decode_attn_noalloc(case.data["q"], Kp, Vp, case.T, s.tau, s.uni_idx, s.uni_cnt,
                                 case.params, out, lse, layout=case.layout)
    torch.cuda.synchronize()
    assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
    case.free()
