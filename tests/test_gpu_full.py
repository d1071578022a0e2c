"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (default parameters, one DecodeStep): every unit's admitted list is checked
for its invariants, and units are compared with the fp64 oracle block by block
(metadata, bound, admission mask) and output by output: every unit of a
workload whose K/V fit in ALL_UNITS_BYTES of host memory (the tiny one and the
B = 32, 32K one), a seeded sample of 12 units otherwise (the first, the last and
10 drawn). The log prints how many units were checked. Runs on an MI355X only."""
import numpy as np
import pytest
import torch

from gpu_util import Case, compare_units
from long_context_decode_predict_amd import _lib, workloads
from long_context_decode_predict_amd.build import ensure_built

pytestmark = pytest.mark.gpu

N_SAMPLE = 10
ALL_UNITS_BYTES = 16 << 30  # K + V copied to the host unit by unit


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ensure_built()
    yield
    torch.cuda.empty_cache()


def sample_units(w, n=N_SAMPLE):
    rng = np.random.default_rng(w.seed)
    units = {0, w.B * w.H - 1}
    units |= set(rng.choice(w.B * w.H, size=min(n, w.B * w.H), replace=False).tolist())
    return sorted(units)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size(name):
    w = workloads.WORKLOADS[name]
    print(f"\n[full] {name} B={w.B} H={w.H} d={w.d} T={w.T} paged={w.paged} "
          f"var_len={w.var_len}", flush=True)
    mode = "static" if w.static_tau else "predictor"
    case = Case(w, tau_mode=mode, fused=True)  # the launch configuration bench.py times
    if w.append:
        # the cache is built before the last `append` tokens, which then arrive one by one
        T0 = w.T - w.append
        _lib.eta_build_block_meta(case.data["K"], T0, case.meta)
        for t in range(T0, w.T):
            _lib.eta_append_meta(case.data["K"], t, 1, case.meta)
        rebuilt = _lib.Meta.alloc(w.B, w.H, w.d, case.T_cap)
        _lib.eta_build_block_meta(case.data["K"], w.T, rebuilt)
        torch.cuda.synchronize()
        assert torch.equal(rebuilt.centroid, case.meta.centroid)
        assert torch.equal(rebuilt.var, case.meta.var)
        assert torch.equal(rebuilt.maxnorm, case.meta.maxnorm)
        del rebuilt
        case.run(build=False)
    else:
        case.run()
    if w.G > 1:
        from gpu_util import compare_gqa_units
        kv = sample_units(workloads.custom("s", B=w.B, H=w.kv_heads, T=64, seed=w.seed), n=6)
        st = compare_gqa_units(case, kv)
        per_head = float(np.mean(st["density"]))
        print(f"  per-head density {per_head:.3f}, union {np.mean(st['union_density']):.3f}, "
              f"masks checked {st['kv_units'] * w.G} of {w.B * w.H} query heads "
              f"({st['kv_units']} key/value units), heads checked {st['heads_checked']}, "
              f"max|dout| {st['max_out_err']:.2e}", flush=True)
        assert st["heads_checked"] == len(kv) * w.G
        assert abs(per_head - w.density) < 0.1
        case.free()
        return
    kv_bytes = 2 * w.B * w.H * case.T_cap * w.d * (2 if w.kv_dtype == torch.bfloat16 else 4)
    units = list(range(w.B * w.H)) if kv_bytes <= ALL_UNITS_BYTES else sample_units(w)
    st = compare_units(case, units)
    cnt = case.step.adm_cnt.cpu().numpy()
    rows_nblk = np.array([(case.row_len(b) + 63) // 64 for b in range(w.B)], dtype=np.float64)
    frac = cnt / np.maximum(rows_nblk, 1)[:, None]  # per unit admitted fraction of its row
    dens = frac.mean()
    print(f"  mean density {dens:.3f} (target {w.density if not w.static_tau else 'per head'}),"
          f" masks checked {st['units']} of {w.B * w.H} units, out checked {st['out_checked']},"
          f" in-band mismatches {st['band_mismatch_units']},"
          f" max|dout| {st['max_out_err']:.2e}, in-band blocks {st['in_band']}", flush=True)
    assert st["units"] == st["out_checked"] == len(units)
    assert st["band_mismatch_units"] <= max(1, len(units) // 50), st
    if not w.static_tau:
        assert abs(dens - w.density) < 0.1
    else:
        per_head = frac.mean(axis=0)
        assert np.all(np.abs(per_head - np.array(w.head_densities)) < 0.1), per_head
    if name == workloads.HEADLINE:
        # the dense reference on the same kernels: tau = -inf admits every block
        case.W = None
        case.bias = torch.full((w.H,), -float("inf"), device="cuda")
        case.run(build=False)
        assert int(case.step.adm_cnt.min()) == w.nblk
        st = compare_units(case, units[:4], check_meta=False)
        assert st["out_checked"] == len(units[:4])
    case.free()


@pytest.mark.parametrize("name", list(workloads.PREFILL_WORKLOADS))
def test_prefill_full_size(name):
    """The training-time forward at the benchmark's sizes and launch configuration
    (Eq. 1 per token on the GPU, then the gated forward): a seeded sample of
    (row, head, query) triples, spread over early, middle and last positions (16 of
    them among the last 2048), is
    compared with the oracle (its own Eq. 1 for tau, a one-query call over the
    query's causal window)."""
    from oracle import oracle as oracle_mod
    from statistics import NormalDist
    import math
    w = workloads.PREFILL_WORKLOADS[name]
    print(f"\n[full] {name} B={w.B} H={w.H}/{w.kv_heads} d={w.d} T={w.T_q}", flush=True)
    data = workloads.generate_prefill(w)
    params = _lib.default_params()
    bias_v = NormalDist().inv_cdf(1.0 - w.inclusion) * math.sqrt(2.0 + w.sigma ** 2)
    bias = torch.full((w.H,), bias_v, dtype=torch.float32, device="cuda")
    B, H, T, d = data["Q"].shape
    tau = torch.empty((B, H, T), device="cuda")
    out = torch.empty((B, H, T, d), device="cuda")
    lse = torch.empty((B, H, T), device="cuda")
    gs = torch.empty((B, H, T), device="cuda")
    _lib.eta_prefill_predict_tau(data["Q"], data["W"], bias, tau)
    _lib.eta_prefill_attn(data["Q"], data["K"], data["V"], tau, params, out, lse, gs)
    torch.cuda.synchronize()
    O = oracle_mod.default()
    rng = np.random.default_rng(w.seed)
    picks = [(0, 0, 0), (B - 1, H - 1, T - 1)]
    picks += [(int(rng.integers(B)), int(rng.integers(H)), int(t))
              for t in np.concatenate([rng.integers(0, 256, 4), rng.integers(256, T, 10)])]
    # the last queries see the most keys: lse there shows any rounding that grows
    # with the number of keys summed
    picks += [(int(rng.integers(B)), int(rng.integers(H)), int(t))
              for t in rng.integers(max(0, T - 2048), T, 16)]
    Wn = data["W"].cpu().numpy()
    bn = bias.cpu().numpy()
    worst = 0.0
    for b, h, t in picks:
        hk = h // w.G
        q_tok = data["Q"][b, :, t, :].float().cpu().numpy()[None]  # all heads of token t
        tau_o = float(O.predict_tau(q_tok, Wn, bn)[0, h])
        assert abs(float(tau[b, h, t]) - tau_o) <= 1e-5, (b, h, t)
        Kb = data["K"][b, hk, :t + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        Vb = data["V"][b, hk, :t + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        Qb = data["Q"][b, h, t:t + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        o_o, l_o, g_o = O.prefill(Qb, Kb, Vb, t + 1, np.array([tau_o]))
        err = float(np.max(np.abs(out[b, h, t].cpu().numpy() - o_o[0])))
        assert err <= 2e-3, (b, h, t, err)
        assert abs(float(lse[b, h, t]) - l_o[0]) <= 1e-4, (b, h, t)
        assert abs(float(gs[b, h, t]) - g_o[0]) <= 1e-4 * abs(g_o[0]) + 1e-3, (b, h, t)
        worst = max(worst, err)
    incl = float(gs.double().sum()) / (B * H * T * (T + 1) / 2)
    print(f"  sampled {len(picks)} queries, max|dout| {worst:.2e}, mean inclusion {incl:.3f}",
          flush=True)
    assert 0.05 < incl < 0.3
