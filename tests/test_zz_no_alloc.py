"""The allocation-free attention entry point, eta_decode_attn_noalloc, against the
entry point it varies, eta_decode_attn with a caller-allocated workspace: two
calls in a row through the C ABI, the second on a smaller cache (grouped heads,
d = 64) right after the first left its partials in the library's array. Each
result must equal eta_decode_attn's on the same lists bitwise (same kernels,
same split) and so lie within the parity bar (out 2e-3 for bf16 K/V, lse 1e-4).
Runs on an MI355X only."""
import pytest
import torch

from gpu_util import LSE_TOL, OUT_TOL, Case
from long_context_decode_predict_amd import _lib, workloads
from long_context_decode_predict_amd.build import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ensure_built()
    _lib.lib()
    yield
    torch.cuda.empty_cache()


def _both(case):
    """(out, lse) of eta_decode_attn with the step's workspace, then of the no-alloc call."""
    s, w = case.step, case.w
    K, V = case.kv()
    q = case.data["q"]
    res = []
    for noalloc in (False, True):
        out = torch.full_like(s.out, float("nan"))
        lse = torch.full_like(s.lse, float("nan"))
        if noalloc:
            _lib.eta_decode_attn_noalloc(q, K, V, case.T, s.tau, s.uni_idx, s.uni_cnt,
                                         case.params, out, lse, layout=case.layout)
        else:
            _lib.eta_decode_attn(q, K, V, case.T, s.tau, s.uni_idx, s.uni_cnt, case.params,
                                 out, lse, s.ws, layout=case.layout)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def test_noalloc_matches_workspace_entry_point():
    bf16 = torch.bfloat16
    calls = [
        # many work items (2 blocks each): the larger call fills much of the array
        (workloads.custom("na_big", B=4, H=8, d=128, T=40000, kv_dtype=bf16, seed=501),
         _lib.default_params(split_blocks=2)),
        # smaller, grouped heads on the matrix cores, default split
        (workloads.custom("na_small", B=2, H=4, H_kv=2, d=64, T=3000, kv_dtype=bf16, seed=502),
         _lib.default_params()),
    ]
    for w, params in calls:
        print(f"\n[case] noalloc {w.name} B={w.B} H={w.H} H_kv={w.kv_heads} d={w.d} T={w.T} "
              f"split={params.split_blocks}", flush=True)
        need = _lib.eta_decode_attn_workspace_size(w.B, w.H, w.d, w.T_cap, params, w.kv_dtype,
                                                   w.kv_heads if w.G > 1 else 0)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
        case = Case(w, params=params).run()
        assert int(case.step.uni_cnt.sum()) > 0
        (out_a, lse_a), (out_b, lse_b) = _both(case)
        assert not torch.isnan(out_a).any() and not torch.isnan(lse_a).any()
        err = float((out_a - out_b).abs().max())
        lfin = torch.isfinite(lse_a)
        assert torch.equal(lfin, torch.isfinite(lse_b))
        lerr = float((lse_a[lfin] - lse_b[lfin]).abs().max()) if lfin.any() else 0.0
        assert err <= OUT_TOL[w.kv_dtype] and lerr <= LSE_TOL, (w.name, err, lerr)
        assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), (w.name, err, lerr)
        print(f"  workspace {need} bytes, bitwise equal to eta_decode_attn", flush=True)
        case.free()

