"""Threshold bias for a target block density, from a closed-form density model of
the synthetic keys (no pass over K, no call into the library or the oracle).

The pages' offline calibration algorithm is not printed; what is needed here is
only an input: a predictor bias (or frozen per-head thresholds) that makes the
mean admitted fraction land near a target. Under the generator of
``workloads`` (block centroid ~ N(0, I), in-block spread sigma_h), the
combined screen bound of a block of unit u is approximately
    U ~= r_u * (a_h * g + z * sigma'_h)     g ~ N(0, 1),  r_u = |q_u| / sqrt(d),
    a_h = sqrt(1 + sigma_h^2 / 64),  sigma'_h = sigma_h * sqrt(63 / 64),
so a unit with threshold tau_u admits a fraction
    rho_u = 1 - Phi((tau_u / r_u - z * sigma'_h) / a_h)
of its blocks. With a predictor, tau_u = t_u + bias where t_u is the query's
linear term (Eq. 1 without the bias); the bias is found by bisection so that
the mean of rho_u over all units equals the target. Frozen per-head thresholds
are bisected per head over that head's units. The density actually reached is
measured and reported by the caller.
"""
from __future__ import annotations

import math
from statistics import NormalDist

import torch

from .workloads import BLOCK, Workload, head_sigmas

_PHI = NormalDist().cdf


def _unit_density(tau_over_r: float, sigma: float, z: float) -> float:
    a = math.sqrt(1.0 + sigma * sigma / BLOCK)
    se = sigma * math.sqrt((BLOCK - 1) / BLOCK)
    return 1.0 - _PHI((tau_over_r - z * se) / a)


def _bisect(f, target: float, lo=-50.0, hi=50.0, iters=200) -> float:
    """Solve f(x) = target for a decreasing f."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def centered_z(d: int) -> float:
    """The z at which the combined model above stands in for the centered bound
    s (q.c + |q| max|k - c|): under the generator a block's largest key distance
    from its centroid is about sigma (sqrt(d) + 1.7) (the largest of 64 norms of
    N(0, sigma^2 I_d) noise, whose spread is about sigma / sqrt(2)), i.e. z ~=
    sqrt(d) + 1.7 in-block standard deviations."""
    return math.sqrt(d) + 1.7


def bias_for(w: Workload, q: torch.Tensor, W, z: float = 4.0, device="cuda") -> torch.Tensor:
    """float32 [H] bias: frozen per-head thresholds for a workload without a predictor,
    else one predictor bias shared by all heads."""
    sig_kv = head_sigmas(w).tolist()
    sig = [sig_kv[h // w.G] for h in range(w.H)]  # spread of each query head's keys
    qd = q.detach().to("cpu", torch.float64)
    B, H, d = qd.shape
    r = (qd.norm(dim=2) / math.sqrt(d)).tolist()  # [B][H]
    if w.static_tau:
        vals = []
        for h in range(H):
            def mean_rho(tau_h, h=h):
                return sum(_unit_density(tau_h / r[b][h], sig[h], z) for b in range(B)) / B
            vals.append(_bisect(mean_rho, w.head_densities[h]))
        return torch.tensor(vals, dtype=torch.float32, device=device)
    t = (qd.reshape(B, H * d) @ W.detach().to("cpu", torch.float64)).tolist()  # [B][H]

    def mean_rho(bias):
        return sum(_unit_density((t[b][h] + bias) / r[b][h], sig[h], z)
                   for b in range(B) for h in range(H)) / (B * H)
    bias = _bisect(mean_rho, w.density)
    return torch.full((H,), bias, dtype=torch.float32, device=device)
