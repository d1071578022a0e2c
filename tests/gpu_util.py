"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI, run
the fp64 oracle on chosen (batch, head) units, and compare.

Criteria (tolerances written here, used by every GPU test):
  * admitted-block mask: bit-exact against the oracle for every block whose fp64
    bound lies farther than BAND = 1e-5 from the oracle's fp64 tau; a block
    inside the band may go either way (fp32 vs fp64 rounding of the bound);
  * out: max-abs error <= 2e-3 for bf16 K/V, <= 1e-5 for fp32 K/V;
  * lse: abs error <= 1e-4 (fp32 logits of magnitude <= ~15 and an fp32 sum of
    at most 2^19 terms: the rounding error is below 1e-5; 1e-4 leaves margin);
  * tau: abs error <= 1e-5 (fp32 dot of length H*d <= 2048 of O(0.1) terms);
  * block metadata: centroid abs <= 1e-5, var and maxnorm rel <= 1e-5;
  * bound: abs <= 1e-5 * max(1, |U|).
A unit whose GPU mask differs from the oracle's inside the band (its admitted
set legitimately differs) is compared on out/lse against the oracle run over
the GPU's own admitted list, so every compared unit gets an output check; the
count of such units is returned and kept small by the callers.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from long_context_decode_predict_amd import _lib, calibrate, workloads
from long_context_decode_predict_amd.decode import DecodeStep
from oracle import oracle as oracle_mod

BAND = 1e-5
OUT_TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}
LSE_TOL = 1e-4
TAU_TOL = 1e-5


def kv_host(t: torch.Tensor) -> np.ndarray:
    """A device K/V slab as numpy: float32, or the uint16 bit patterns of bf16."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


class Case:
    """A workload instance on the GPU plus the library's results for one step."""

    def __init__(self, w: workloads.Workload, tau_mode="predictor", params=None, T=None,
                 T_cap=None, bias=None, fused=False, seq_lens=None, paged=None,
                 all_pages=False):
        self.fused = fused
        self.w = w
        self.T_cap = T_cap if T_cap is not None else w.T_cap
        self.T = T if T is not None else w.T
        self.params = params if params is not None else _lib.default_params()
        self.data = workloads.generate(w, "cuda", T_cap=self.T_cap)
        d = self.data
        self.W = d["W"] if tau_mode == "predictor" else None
        if bias is not None:
            self.bias = bias.to("cuda", torch.float32)
        elif tau_mode in ("predictor", "static"):
            z = (calibrate.centered_z(w.d) if self.params.bound_mode == _lib.ETA_BOUND_CENTERED
                 else self.params.z)
            self.bias = calibrate.bias_for(w, d["q"], d["W"], z=z)
        else:
            val = {"neg_inf": -math.inf, "pos_inf": math.inf, "nan": math.nan}[tau_mode]
            self.bias = torch.full((w.H,), val, dtype=torch.float32, device="cuda")
        # optional per-row lengths and page pool (the dense K/V stay for the oracle)
        if seq_lens is None and w.var_len > 0:
            seq_lens = workloads.row_lengths(w)
        self.row_T = None if seq_lens is None else [int(t) for t in seq_lens]
        paged = w.paged if paged is None else paged
        self.layout = None
        if self.row_T is not None or paged:
            lens = (None if self.row_T is None else
                    torch.tensor(self.row_T, dtype=torch.int32, device="cuda"))
            table = None
            if paged:
                table, d["Kp"], d["Vp"] = workloads.page_pool(
                    d["K"], d["V"], self.row_T or [self.T] * w.B, w.seed, all_blocks=all_pages)
            self.layout = _lib.KVLayout(lens, table)
        self.meta = _lib.Meta.alloc(w.B, w.kv_heads, w.d, self.T_cap,
                                    centered=self.params.bound_mode == _lib.ETA_BOUND_CENTERED)
        self.step = DecodeStep(w.B, w.H, w.d, self.T_cap, w.kv_dtype, self.params,
                               with_bounds=True, H_kv=w.kv_heads, layout=self.layout)

    def kv(self):
        """The K, V the library reads: the page pools of a paged case, else the cache."""
        d = self.data
        return (d["Kp"], d["Vp"]) if d.get("Kp") is not None else (d["K"], d["V"])

    def row_len(self, b: int) -> int:
        return self.T if self.row_T is None else self.row_T[b]

    def build_meta(self):
        _lib.eta_build_block_meta(self.kv()[0], self.T, self.meta, layout=self.layout)

    def run(self, build=True):
        if build:
            self.build_meta()
        d = self.data
        K, V = self.kv()
        self.step(d["q"], K, V, self.T, self.meta, self.W, self.bias, fused=self.fused)
        torch.cuda.synchronize()
        return self

    def host(self):
        s = self.step
        return {"tau": s.tau.cpu().numpy(), "idx": s.adm_idx.cpu().numpy(),
                "cnt": s.adm_cnt.cpu().numpy(), "uni_idx": s.uni_idx.cpu().numpy(),
                "uni_cnt": s.uni_cnt.cpu().numpy(), "out": s.out.cpu().numpy(),
                "lse": s.lse.cpu().numpy(), "U": s.bounds.cpu().numpy(),
                "centroid": self.meta.centroid, "var": self.meta.var,
                "maxnorm": self.meta.maxnorm, "maxdev2": self.meta.maxdev2}

    def free(self):
        for k in list(self.data):
            self.data[k] = None
        self.meta = None
        self.step = None
        torch.cuda.empty_cache()


def check_list_properties(g: dict, nblk, rows: int | None = None):
    """Every unit's list is strictly ascending, in range and exactly cnt long.
    nblk: one block count for all units, or one per batch row (rows = batch size)."""
    cnt = g["cnt"].reshape(-1)
    idx = g["idx"].reshape(cnt.shape[0], -1)
    per_unit = (np.full(cnt.shape[0], nblk) if np.isscalar(nblk)
                else np.repeat(np.asarray(nblk), cnt.shape[0] // rows))
    assert np.all(cnt >= 0) and np.all(cnt <= per_unit)
    for u in range(cnt.shape[0]):
        lst = idx[u, :cnt[u]]
        assert np.all(np.diff(lst) > 0), u
        if len(lst):
            assert lst[0] >= 0 and lst[-1] < per_unit[u], u


def _check_unit(O, p, u, b, h, T, nblk, Kh, Vh, meta_g, qv, t, U_g, idx_g, out_g, lse_g, tol):
    """The oracle side of one (row, head) unit and its comparison (host data only,
    so units can be checked on a pool of threads: the oracle's C calls release
    the interpreter lock). Returns the unit's figures; raises on a mismatch."""
    c, v, m = O.block_meta(Kh, T)
    centered = p.bound_mode == _lib.ETA_BOUND_CENTERED
    md = O.block_maxdev(Kh, T) if centered else None
    if meta_g is not None:
        cg, vg, mg = meta_g[:3]
        assert np.max(np.abs(cg - c)) <= 1e-5, (u, np.max(np.abs(cg - c)))
        assert np.all(np.abs(vg - v) <= 1e-5 * np.maximum(v, 1e-30) + 1e-12), u
        assert np.all(np.abs(mg - m) <= 1e-5 * m + 1e-12), u
        if centered:
            # fp32 squared distances from the fp32 centroid: relative 1e-5 of the
            # distance, or 1e-5 of the block's key norm when the distance is small
            dg = np.sqrt(meta_g[3].astype(np.float64))
            assert np.all(np.abs(dg - md) <= 1e-5 * md + 1e-5 * m + 1e-12), (u, np.max(np.abs(dg - md)))
    U = (O.bounds_centered(qv, c, m, md) if centered
         else O.bounds(qv, c, v, m, z=p.z, mode=p.bound_mode))
    assert np.all(np.abs(U_g - U) <= 1e-5 * np.maximum(1.0, np.abs(U))), (u, np.max(np.abs(U_g - U)))
    mask_o = U >= t
    mask_g = np.zeros(nblk, bool)
    mask_g[idx_g] = True
    outside = ~(np.abs(U - t) <= BAND)
    assert np.array_equal(mask_g[outside], mask_o[outside]), (u, np.nonzero(mask_g != mask_o))
    mismatch = not np.array_equal(mask_g, mask_o)
    # only in-band blocks can differ (asserted above); then attend over the GPU's set
    idx_o = np.nonzero(mask_g if mismatch else mask_o)[0].astype(np.int32)
    out_o, lse_o = O.attend(qv, Kh, Vh, T, t, idx_o, beta=p.gate_beta, hard=bool(p.gate_hard))
    err = float(np.max(np.abs(out_g - out_o)))
    assert err <= tol, (u, err)
    if math.isinf(lse_o):
        assert lse_g == lse_o and np.all(out_g == 0), (u, lse_g)
        lerr = 0.0
    else:
        lerr = abs(lse_g - lse_o)
        assert lerr <= LSE_TOL, (u, lse_g, lse_o)
    return {"in_band": int((~outside).sum()), "mismatch": mismatch, "err": err, "lerr": lerr,
            "density": len(idx_g) / max(nblk, 1)}


def compare_units(case: Case, units, O=None, check_meta=True, workers: int = 8):
    """Compare the library against the oracle on the given units; returns stats.
    Device-to-host copies happen here; the oracle work of the units runs on a
    pool of `workers` threads (at most 2 * workers units' host copies in flight)."""
    from concurrent.futures import ThreadPoolExecutor
    O = O or oracle_mod.default()
    w, p = case.w, case.params
    g = case.host()
    q = case.data["q"].cpu().numpy()
    W = None if case.W is None else case.W.cpu().numpy()
    bias = case.bias.cpu().numpy()
    tau_o = O.predict_tau(q, W, bias)
    rows_nblk = [(case.row_len(b) + 63) // 64 for b in range(w.B)]
    check_list_properties(g, rows_nblk, w.B)
    tau_g = g["tau"]
    fin = np.isfinite(tau_o)
    assert np.array_equal(fin, np.isfinite(tau_g))
    assert np.all(np.abs(tau_g[fin] - tau_o[fin]) <= TAU_TOL)
    stats = {"units": 0, "in_band": 0, "band_mismatch_units": 0, "out_checked": 0,
             "max_out_err": 0.0, "max_lse_err": 0.0, "density": []}
    tol = OUT_TOL[w.kv_dtype]

    def collect(fut):
        r = fut.result()
        stats["units"] += 1
        stats["in_band"] += r["in_band"]
        stats["band_mismatch_units"] += int(r["mismatch"])
        stats["density"].append(r["density"])
        stats["out_checked"] += 1
        stats["max_out_err"] = max(stats["max_out_err"], r["err"])
        stats["max_lse_err"] = max(stats["max_lse_err"], r["lerr"])

    pending = []
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for u in units:
            b, h = divmod(int(u), w.H)
            T = case.row_len(b)
            nblk = rows_nblk[b]
            Kh = kv_host(case.data["K"][b, h])
            Vh = kv_host(case.data["V"][b, h])
            meta_g = None
            if check_meta and nblk:
                meta_g = (g["centroid"][b, h, :, :nblk].cpu().numpy().T,
                          g["var"][b, h, :nblk].cpu().numpy(),
                          g["maxnorm"][b, h, :nblk].cpu().numpy())
                if g["maxdev2"] is not None:
                    meta_g += (g["maxdev2"][b, h, :nblk].cpu().numpy(),)
            cnt = int(g["cnt"][b, h])
            pending.append(pool.submit(
                _check_unit, O, p, u, b, h, T, nblk, Kh, Vh, meta_g, q[b, h],
                float(tau_o[b, h]), g["U"][b, h, :nblk], g["idx"][b, h, :cnt], g["out"][b, h],
                float(g["lse"][b, h]), tol))
            if len(pending) >= 2 * workers:
                collect(pending.pop(0))
        for fut in pending:
            collect(fut)
    return stats


def compare_gqa_units(case: Case, kv_units, O=None):
    """Grouped heads: per query head masks, the union of each key/value head's lists,
    and every query head's output over that union, against the oracle."""
    O = O or oracle_mod.default()
    w, p = case.w, case.params
    G = w.G
    g = case.host()
    q = case.data["q"].cpu().numpy()
    W = None if case.W is None else case.W.cpu().numpy()
    tau_o = O.predict_tau(q, W, case.bias.cpu().numpy())
    rows_nblk = [(case.row_len(b) + 63) // 64 for b in range(w.B)]
    check_list_properties(g, rows_nblk, w.B)
    check_list_properties({"cnt": g["uni_cnt"], "idx": g["uni_idx"]}, rows_nblk, w.B)
    fin = np.isfinite(tau_o)
    assert np.array_equal(fin, np.isfinite(g["tau"]))
    assert np.all(np.abs(g["tau"][fin] - tau_o[fin]) <= TAU_TOL)
    stats = {"kv_units": 0, "heads_checked": 0, "band_mismatch_units": 0, "max_out_err": 0.0,
             "density": [], "union_density": []}
    tol = OUT_TOL[w.kv_dtype]
    for uk in kv_units:
        b, k = divmod(int(uk), w.kv_heads)
        T = case.row_len(b)
        nblk = rows_nblk[b]
        Kh = kv_host(case.data["K"][b, k])
        Vh = kv_host(case.data["V"][b, k])
        c, v, m = O.block_meta(Kh, T)
        md = O.block_maxdev(Kh, T) if p.bound_mode == _lib.ETA_BOUND_CENTERED else None
        masks, outs = [], []
        for j in range(G):
            h = k * G + j
            U = (O.bounds_centered(q[b, h], c, m, md) if md is not None
                 else O.bounds(q[b, h], c, v, m, z=p.z, mode=p.bound_mode))
            Ug = g["U"][b, h, :nblk]
            assert np.all(np.abs(Ug - U) <= 1e-5 * np.maximum(1.0, np.abs(U)))
            t = float(tau_o[b, h])
            mask_o = U >= t
            mask_g = np.zeros(nblk, bool)
            mask_g[g["idx"][b, h, :g["cnt"][b, h]]] = True
            outside = ~(np.abs(U - t) <= BAND)
            assert np.array_equal(mask_g[outside], mask_o[outside]), (uk, j)
            masks.append(mask_o)
            outs.append(outside)
            stats["density"].append(mask_g.sum() / max(nblk, 1))
        union_o = O.union([np.nonzero(mk)[0].astype(np.int32) for mk in masks], nblk)
        union_g = g["uni_idx"][b, k, :g["uni_cnt"][b, k]]
        stats["union_density"].append(len(union_g) / max(nblk, 1))
        stats["kv_units"] += 1
        # a block's union membership is decided when some head admits it outside the
        # band, or every head rejects it outside the band
        sure_in = np.zeros(nblk, bool)
        sure_out = np.ones(nblk, bool)
        for mk, od in zip(masks, outs):
            sure_in |= mk & od
            sure_out &= (~mk) & od
        ug = np.zeros(nblk, bool)
        ug[union_g] = True
        assert np.all(ug[sure_in]) and not np.any(ug[sure_out]), uk
        if np.array_equal(union_g, union_o):
            attend_on = union_o
        else:  # only in-band decisions differ (asserted above): attend over the GPU's union
            stats["band_mismatch_units"] += 1
            attend_on = np.asarray(union_g, dtype=np.int32)
        for j in range(G):
            h = k * G + j
            out_o, lse_o = O.attend(q[b, h], Kh, Vh, T, float(tau_o[b, h]), attend_on,
                                    beta=p.gate_beta, hard=bool(p.gate_hard))
            err = float(np.max(np.abs(g["out"][b, h] - out_o)))
            assert err <= tol, (uk, j, err)
            lse_g = float(g["lse"][b, h])
            if math.isinf(lse_o):
                assert lse_g == lse_o and np.all(g["out"][b, h] == 0)
            else:
                assert abs(lse_g - lse_o) <= LSE_TOL, (uk, j, lse_g, lse_o)
            stats["heads_checked"] += 1
            stats["max_out_err"] = max(stats["max_out_err"], err)
    return stats
