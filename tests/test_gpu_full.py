"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (default parameters, one DecodeStep): every unit's admitted list is checked
for its invariants, and a seeded sample of units is compared with the fp64
oracle block by block and output by output. Runs on an MI355X only."""
import numpy as np
import pytest
import torch

from gpu_util import Case, compare_units
from long_context_decode_predict_amd import _lib, workloads
from long_context_decode_predict_amd.build import ensure_built

pytestmark = pytest.mark.gpu

N_SAMPLE = 10


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
              f"heads checked {st['heads_checked']}, max|dout| {st['max_out_err']:.2e}", flush=True)
        assert st["heads_checked"] >= (len(kv) - 1) * w.G
        assert abs(per_head - w.density) < 0.1
        case.free()
        return
    units = sample_units(w)
    st = compare_units(case, units)
    cnt = case.step.adm_cnt.cpu().numpy()
    rows_nblk = np.array([(case.row_len(b) + 63) // 64 for b in range(w.B)], dtype=np.float64)
    frac = cnt / np.maximum(rows_nblk, 1)[:, None]  # per unit admitted fraction of its row
    dens = frac.mean()
    print(f"  mean density {dens:.3f} (target {w.density if not w.static_tau else 'per head'}),"
          f" sampled units {st['units']}, out checked {st['out_checked']},"
          f" max|dout| {st['max_out_err']:.2e}, in-band blocks {st['in_band']}", flush=True)
    assert st["out_checked"] >= len(units) - 1
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
