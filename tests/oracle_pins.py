"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``check_*`` takes a loaded oracle (``oracle.oracle.OracleLib``) and raises
``AssertionError`` when the oracle disagrees with what the pages print, with a
closed form, with a textbook/library routine or with a brute-force guarantee.
``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutants.py`` runs them against deliberately broken copies of the
oracle source to show that each plausible mistake is caught by at least one.

Sources pinned (pages describing arXiv:2609.20888):
  * evolve.pub review, "Methodology Assessment": Eq. 1 predictor, Eq. 2
    logistic gate with slope 3.35e-4 at 8, Eq. 3 multiplicative gating;
  * evolve.pub review, Q&A on attention sinks: a suppressed logit weighs e^0 = 1;
  * evolve.pub review, Q&A "What is ETA?": a block none of whose keys can reach
    tau is skipped (hence the bound must dominate every key's score).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str, fname: str = "gate_constants.txt"):
    """(value, abs_tol) of one named constant in a golden fixture."""
    with open(os.path.join(GOLDEN_DIR, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == name:
                return float(parts[1]), float(parts[2])
    raise KeyError(name)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sdpa(q, K, V, mask=None):
    """Library softmax attention in float64 (scale 1/sqrt(d)); returns (out, lse)."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).reshape(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    mt = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=np.float64)).reshape(1, 1, 1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mt)
    d = K.shape[1]
    logits = (Kt[0, 0] @ qt.reshape(-1)) / math.sqrt(d)
    if mt is not None:
        logits = logits + mt.reshape(-1)
    lse = torch.logsumexp(logits, dim=0)
    return out.reshape(-1).numpy(), float(lse)


def _clustered(rng, nblk, d, sigma=0.3, bs=64):
    """Tiny clustered keys: per-block centroid ~ N(0,1)^d plus N(0, sigma^2) noise."""
    cen = rng.standard_normal((nblk, 1, d))
    K = (cen + sigma * rng.standard_normal((nblk, bs, d))).reshape(nblk * bs, d)
    return K.astype(np.float32)


def _scores(q, K, idx, T, bs=64):
    """Exact scaled scores s*q.k of the tokens < T of blocks idx (numpy fp64)."""
    d = K.shape[1]
    rows = np.concatenate([np.arange(b * bs, min(T, (b + 1) * bs)) for b in idx]) if len(idx) else np.zeros(0, int)
    Kf = K[rows].astype(np.float64) if K.dtype != np.uint16 else bf16_bits_to_f64(K[rows])
    return Kf @ np.asarray(q, dtype=np.float64) / math.sqrt(d), rows


# ----------------------------------------------------------------------------------------
# Eq. 1 predictor
# ----------------------------------------------------------------------------------------
def check_predict_static_and_zero(O):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 4, 8)).astype(np.float32)
    bias = rng.standard_normal(4).astype(np.float32)
    want = np.broadcast_to(bias.astype(np.float64), (3, 4))
    assert np.array_equal(O.predict_tau(q, None, bias), want)
    W0 = np.zeros((32, 4), np.float32)
    assert np.array_equal(O.predict_tau(q, W0, bias), want)


def check_predict_single_entry(O):
    """A W with one non-zero entry at row g*d+i, column h picks out q[b,g,i] for head h
    only (catches a transposed W or a wrong index into the concatenated query)."""
    rng = np.random.default_rng(2)
    B, H, d = 2, 3, 4
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    bias = rng.standard_normal(H).astype(np.float32)
    for (g, i, h) in [(0, 0, 0), (0, 3, 2), (2, 1, 0), (1, 2, 1), (2, 3, 2)]:
        W = np.zeros((H * d, H), np.float32)
        W[g * d + i, h] = 1.5
        tau = O.predict_tau(q, W, bias)
        for b in range(B):
            for hh in range(H):
                want = float(bias[hh]) + (1.5 * float(q[b, g, i]) if hh == h else 0.0)
                assert tau[b, hh] == want, (g, i, h, b, hh, tau[b, hh], want)


def check_predict_matmul(O):
    """Against the library matrix product of the concatenated queries (Eq. 1)."""
    rng = np.random.default_rng(3)
    B, H, d = 5, 4, 16
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    W = (rng.standard_normal((H * d, H)) / math.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(H).astype(np.float32)
    want = q.reshape(B, H * d).astype(np.float64) @ W.astype(np.float64) + bias.astype(np.float64)
    np.testing.assert_allclose(O.predict_tau(q, W, bias), want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------
# Block metadata
# ----------------------------------------------------------------------------------------
def check_meta_library(O):
    """Centroid / variance / max-norm against numpy's mean, var and norm, with a ragged
    last block (T not a multiple of the block size), for float32 and bf16 keys."""
    rng = np.random.default_rng(4)
    T_cap, d, T, bs = 256, 8, 150, 64
    Kf = (rng.standard_normal((T_cap, d)) * 2 + 0.5).astype(np.float32)
    for K, Kval in [(Kf, Kf.astype(np.float64)),
                    (f32_to_bf16_bits(Kf), bf16_bits_to_f64(f32_to_bf16_bits(Kf)))]:
        c, v, m = O.block_meta(K, T, bs)
        assert c.shape == (3, d)
        for blk in range(3):
            rows = Kval[blk * bs:min(T, (blk + 1) * bs)]
            np.testing.assert_allclose(c[blk], rows.mean(axis=0), rtol=0, atol=1e-12)
            np.testing.assert_allclose(v[blk], np.var(rows - rows.mean(axis=0)), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(v[blk], np.mean(np.var(rows, axis=0)), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(m[blk], np.linalg.norm(rows, axis=1).max(), rtol=1e-13)


def check_meta_one_token_and_two_token(O):
    """A one-token block has centroid = key and variance 0; a two-token block
    {a+e, a-e} has centroid a and variance |e|^2/d (closed forms)."""
    rng = np.random.default_rng(5)
    d = 8
    K = rng.standard_normal((128, d)).astype(np.float32)
    c, v, m = O.block_meta(K, 65, 64)
    assert np.array_equal(c[1], K[64].astype(np.float64))
    assert v[1] == 0.0
    assert m[1] == np.sqrt(np.sum(K[64].astype(np.float64) ** 2))
    a = np.array([1.0, -2.0, 0.5, 4.0, 0.0, 3.0, -1.0, 2.0], np.float32)
    e = np.array([0.5, 0.25, -1.0, 2.0, 1.0, -0.5, 0.0, 0.75], np.float32)
    K2 = np.stack([a + e, a - e]).astype(np.float32)
    c, v, m = O.block_meta(K2, 2, 64)
    np.testing.assert_allclose(c[0], a.astype(np.float64), atol=1e-15)
    np.testing.assert_allclose(v[0], float(np.sum(e.astype(np.float64) ** 2)) / d, rtol=1e-14)
    want_m = max(np.linalg.norm((a + e).astype(np.float64)), np.linalg.norm((a - e).astype(np.float64)))
    np.testing.assert_allclose(m[0], want_m, rtol=1e-14)


# ----------------------------------------------------------------------------------------
# Block bounds
# ----------------------------------------------------------------------------------------
def check_bound_cauchy_schwarz(O):
    """Geometric bound: brute force on tiny inputs -- no key of a block scores above
    U_geo, so the GEO screen never skips a block holding a key with score >= tau;
    equality for a one-key block parallel to q."""
    rng = np.random.default_rng(6)
    d, nblk = 16, 12
    K = _clustered(rng, nblk, d, sigma=0.8)
    K[5 * 64 + 17] = 3.0 * rng.standard_normal(d)  # an outlier key
    meta = O.block_meta(K, nblk * 64)
    for trial in range(20):
        q = rng.standard_normal(d).astype(np.float32) * (1 + trial % 3)
        U = O.bounds(q, *meta, z=4.0, mode=1)
        for blk in range(nblk):
            S, _ = _scores(q, K, [blk], nblk * 64)
            assert S.max() <= U[blk] + 1e-12
            tau = float(S.max()) - 1e-9  # the block holds a key with score >= tau
            assert blk in O.screen(U, tau)
    q = rng.standard_normal(d).astype(np.float32)
    K1 = np.zeros((64, d), np.float32)
    K1[0] = 2.0 * q
    U = O.bounds(q, *O.block_meta(K1, 1), z=4.0, mode=1)
    S, _ = _scores(q, K1, [0], 1)
    np.testing.assert_allclose(U[0], S[0], rtol=1e-12)


def check_bound_samuelson(O):
    """Combined bound with z = sqrt((n-1) d) dominates every key (Samuelson's
    inequality); brute force on tiny clustered blocks and an outlier."""
    rng = np.random.default_rng(7)
    d, nblk = 16, 10
    K = _clustered(rng, nblk, d, sigma=0.3)
    K[3 * 64 + 9] = 4.0 * rng.standard_normal(d)
    meta = O.block_meta(K, nblk * 64)
    z = math.sqrt(63 * d)
    for trial in range(20):
        q = rng.standard_normal(d).astype(np.float32)
        U = O.bounds(q, *meta, z=z, mode=0)
        for blk in range(nblk):
            S, _ = _scores(q, K, [blk], nblk * 64)
            assert S.max() <= U[blk] + 1e-12, (trial, blk, S.max(), U[blk])


def check_bound_one_token_exact(O):
    """A one-token block has variance 0, so the probabilistic bound equals the key's
    scaled score exactly, and the combined bound takes it (it is below U_geo)."""
    rng = np.random.default_rng(8)
    d = 32
    K = rng.standard_normal((64, d)).astype(np.float32)
    for trial in range(5):
        q = rng.standard_normal(d).astype(np.float32)
        U = O.bounds(q, *O.block_meta(K, 1), z=4.0, mode=0)
        S, _ = _scores(q, K, [0], 1)
        np.testing.assert_allclose(U[0], S[0], rtol=0, atol=1e-13)


def check_bound_per_block(O):
    """The bound of a block depends on that block's metadata only (O(1) screening):
    bounds over many blocks equal the bounds of each block alone; with one-token
    blocks (block size 1) every bound is that token's exact scaled score."""
    rng = np.random.default_rng(15)
    d, nblk = 16, 9
    K = _clustered(rng, nblk, d, sigma=0.5)
    c, v, m = O.block_meta(K, nblk * 64 - 5)
    q = rng.standard_normal(d).astype(np.float32)
    for z, mode in [(4.0, 0), (1.0, 0), (4.0, 1)]:
        U = O.bounds(q, c, v, m, z=z, mode=mode)
        for blk in range(nblk):
            one = O.bounds(q, c[blk:blk + 1], v[blk:blk + 1], m[blk:blk + 1], z=z, mode=mode)
            assert U[blk] == one[0]
    c1, v1, m1 = O.block_meta(K[:20], 20, bs=1)
    U = O.bounds(q, c1, v1, m1, z=4.0, mode=0)
    S = K[:20].astype(np.float64) @ q.astype(np.float64) / math.sqrt(d)
    np.testing.assert_allclose(U, S, rtol=0, atol=1e-13)


def check_bound_worked_example(O):
    """Hand-worked d=2 block {(2,1), (0,1)}: centroid (1,1), variance 1/2, max-norm
    sqrt(5), s = 1/sqrt(2). U_geo = sqrt(5/2); U_prob = (q.c + z*sqrt(1/2))/sqrt(2)."""
    K = np.array([[2.0, 1.0], [0.0, 1.0]], np.float32)
    meta = O.block_meta(K, 2)
    r2 = math.sqrt(2.0)
    geo = math.sqrt(5.0) / r2
    cases = [((1.0, 0.0), 1.0, 0, (1 + math.sqrt(0.5)) / r2),
             ((1.0, 0.0), 4.0, 0, geo),
             ((-1.0, 0.0), 1.0, 0, (-1 + math.sqrt(0.5)) / r2),
             ((1.0, 0.0), 1.0, 1, geo),
             ((0.0, -2.0), 2.0, 0, (-2 + 2 * 2 * math.sqrt(0.5)) / r2)]
    for q, z, mode, want in cases:
        U = O.bounds(np.array(q, np.float32), *meta, z=z, mode=mode)
        np.testing.assert_allclose(U[0], want, rtol=0, atol=1e-14, err_msg=str((q, z, mode)))


def check_maxdev_library(O):
    """Largest distance from the centroid against numpy (mean, then the row norms of
    the deviations), with a ragged last block and bf16 input."""
    rng = np.random.default_rng(31)
    d, T = 24, 3 * 64 + 11
    K = (rng.standard_normal((T + 5, d)) * 2.0).astype(np.float32)
    md = O.block_maxdev(K, T)
    assert md.shape == (4,)
    for blk in range(4):
        X = K[blk * 64:min(T, blk * 64 + 64)].astype(np.float64)
        want = np.max(np.linalg.norm(X - X.mean(axis=0), axis=1))
        np.testing.assert_allclose(md[blk], want, rtol=1e-13)
    Kb = f32_to_bf16_bits(K)
    mdb = O.block_maxdev(Kb, T)
    X = bf16_bits_to_f64(Kb[:64])
    np.testing.assert_allclose(mdb[0], np.max(np.linalg.norm(X - X.mean(axis=0), axis=1)),
                               rtol=1e-13)


def check_bound_centered_guarantee(O):
    """Centered bound: brute force -- no key scores above min(U_geo, U_cen), so the
    screen keeps every block holding a key that reaches tau; never above U_geo; a
    one-token block bounds to its key's exact score; a block whose farthest key
    lies from the centroid along q is bounded exactly by that key."""
    rng = np.random.default_rng(32)
    d, nblk = 16, 12
    K = _clustered(rng, nblk, d, sigma=0.4)
    K[7 * 64 + 40] = 5.0 * rng.standard_normal(d)  # an outlier (a needle-like key)
    c, v, m = O.block_meta(K, nblk * 64)
    md = O.block_maxdev(K, nblk * 64)
    for trial in range(20):
        q = (rng.standard_normal(d) * (1 + trial % 3)).astype(np.float32)
        U = O.bounds_centered(q, c, m, md)
        Ug = O.bounds(q, c, v, m, mode=1)
        assert np.all(U <= Ug)
        for blk in range(nblk):
            S, _ = _scores(q, K, [blk], nblk * 64)
            assert S.max() <= U[blk] + 1e-12, (trial, blk)
            assert blk in O.screen(U, float(S.max()) - 1e-9)
    q = rng.standard_normal(d).astype(np.float32)
    c1, _, m1 = O.block_meta(K, 1)
    U = O.bounds_centered(q, c1, m1, O.block_maxdev(K, 1))
    S, _ = _scores(q, K, [0], 1)
    np.testing.assert_allclose(U[0], S[0], rtol=0, atol=1e-13)
    base = rng.standard_normal(d)
    qh = q.astype(np.float64) / np.linalg.norm(q.astype(np.float64))
    K2 = np.stack([base + 1.5 * qh, base - 1.5 * qh, base]).astype(np.float32)
    c2, v2, m2 = O.block_meta(K2, 3)
    U = O.bounds_centered(q, c2, m2, O.block_maxdev(K2, 3))
    S, _ = _scores(q, K2, [0], 3)
    np.testing.assert_allclose(U[0], min(S.max(), O.bounds(q, c2, v2, m2, mode=1)[0]),
                               rtol=0, atol=1e-6)


def check_bound_centered_worked_example(O):
    """Hand-worked d=2 block {(2,1), (0,1)}: centroid (1,1), both keys at distance 1
    from it, max-norm sqrt(5), s = 1/sqrt(2). q = (1,0): U_cen = (1 + 1)/sqrt(2) =
    sqrt(2), the score of (2,1) exactly, below U_geo = sqrt(5/2); q = (0,-2): U_cen =
    (-2 + 2)/sqrt(2) = 0; q = (3,0): U_cen = (3 + 3)/sqrt(2), U_geo = 3 sqrt(5/2),
    the smaller is U_cen."""
    K = np.array([[2.0, 1.0], [0.0, 1.0]], np.float32)
    c, _, m = O.block_meta(K, 2)
    md = O.block_maxdev(K, 2)
    np.testing.assert_allclose(md[0], 1.0, rtol=0, atol=1e-15)
    r2 = math.sqrt(2.0)
    for q, want in [((1.0, 0.0), r2), ((0.0, -2.0), 0.0), ((3.0, 0.0), 6.0 / r2)]:
        U = O.bounds_centered(np.array(q, np.float32), c, m, md)
        np.testing.assert_allclose(U[0], want, rtol=0, atol=1e-14, err_msg=str(q))


# ----------------------------------------------------------------------------------------
# Screen
# ----------------------------------------------------------------------------------------
def check_screen_properties(O):
    rng = np.random.default_rng(9)
    U = rng.standard_normal(300)
    U[17] = 0.25
    idx = O.screen(U, 0.25)
    assert 17 in idx  # a tie is admitted
    assert np.array_equal(idx, np.nonzero(U >= 0.25)[0])
    assert np.all(np.diff(idx) > 0)
    taus = np.sort(rng.standard_normal(6))
    prev = None
    for t in taus:  # nesting: a larger tau admits a subset
        cur = set(O.screen(U, t).tolist())
        assert len(cur) == int(np.sum(U >= t))
        if prev is not None:
            assert cur <= prev
        prev = cur
    assert len(O.screen(U, -math.inf)) == 300
    assert len(O.screen(U, math.inf)) == 0
    assert len(O.screen(U, math.nan)) == 0


def check_union(O):
    """Group union against numpy's set union (library routine); one list is its own
    union; empty lists; full coverage."""
    rng = np.random.default_rng(16)
    nblk = 300
    for g in (1, 2, 4, 8):
        lists = [np.sort(rng.choice(nblk, size=rng.integers(0, 120), replace=False)).astype(np.int32)
                 for _ in range(g)]
        want = lists[0]
        for x in lists[1:]:
            want = np.union1d(want, x)
        assert np.array_equal(O.union(lists, nblk), want.astype(np.int32))
    x = np.array([3, 9, 200], np.int32)
    assert np.array_equal(O.union([x], nblk), x)
    assert len(O.union([np.zeros(0, np.int32)] * 3, nblk)) == 0
    assert np.array_equal(O.union([np.arange(0, nblk, 2, dtype=np.int32),
                                   np.arange(1, nblk, 2, dtype=np.int32)], nblk), np.arange(nblk))


# ----------------------------------------------------------------------------------------
# Eq. 2 gate
# ----------------------------------------------------------------------------------------
def check_gate_golden(O):
    """Printed slope sigma'(8) = 3.35e-4 at the start-dense init b = -8 (beta = 1)."""
    slope, tol = golden("sigma_prime_at_8")
    b0, _ = golden("start_dense_bias")
    h = 1e-4
    num = (O.gate(h, b0, 1.0) - O.gate(-h, b0, 1.0)) / (2 * h)
    assert abs(num - slope) <= tol, num
    assert 1.0 - 1e-3 < O.gate(0.0, b0, 1.0) < 1.0  # start dense: gate ~ 1
    beta_end, _ = golden("beta_anneal_end")
    beta_start, _ = golden("beta_anneal_start")
    # the gate depends on beta*(S - tau) only
    assert abs(O.gate(8.0 / beta_end, 0.0, beta_end) - O.gate(8.0, 0.0, beta_start)) < 1e-15
    num5 = (O.gate(1.6 + h, 0.0, beta_end) - O.gate(1.6 - h, 0.0, beta_end)) / (2 * h)
    assert abs(num5 - beta_end * slope) <= beta_end * tol + 1e-8


def check_gate_shape(O):
    assert O.gate(0.3, 0.3, 5.0) == 0.5
    assert O.gate(10.0, 0.0, 5.0) >= 1 - 1e-15
    assert O.gate(-10.0, 0.0, 5.0) < 1e-20
    assert O.gate(0.3, 0.3, 5.0, hard=True) == 1.0  # tie kept
    assert O.gate(0.3 - 1e-9, 0.3, 5.0, hard=True) == 0.0
    for S in [-2.0, -0.1, 0.05, 1.7]:  # soft -> hard as beta grows (away from the tie)
        assert abs(O.gate(S, 0.0, 1e4) - O.gate(S, 0.0, 5.0, hard=True)) < 1e-12


# ----------------------------------------------------------------------------------------
# Gated softmax attention
# ----------------------------------------------------------------------------------------
def check_attend_dense_is_sdpa(O):
    """tau = -inf admits every block and the gate is 1: the result is dense softmax
    attention (library SDPA in float64), for float32 and bf16 K/V and a ragged tail."""
    rng = np.random.default_rng(10)
    d, T = 16, 300
    K = rng.standard_normal((320, d)).astype(np.float32)
    V = rng.standard_normal((320, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    idx = np.arange(5, dtype=np.int32)
    for KK, VV, Kv, Vv in [(K, V, K, V),
                           (f32_to_bf16_bits(K), f32_to_bf16_bits(V),
                            bf16_bits_to_f64(f32_to_bf16_bits(K)), bf16_bits_to_f64(f32_to_bf16_bits(V)))]:
        out, lse = O.attend(q, KK, VV, T, -math.inf, idx)
        want, want_lse = _sdpa(q, Kv[:T], Vv[:T])
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
        assert abs(lse - want_lse) < 1e-12
        step = O.unit_step(q, KK, VV, T, -math.inf, O.block_meta(KK, T))
        assert np.array_equal(step["idx"], idx)
        np.testing.assert_allclose(step["out"], want, rtol=0, atol=1e-12)


def check_attend_gated_is_sdpa(O):
    """Finite tau on a subset of blocks: softmax over S' = S * gate(S) (Eq. 3) is SDPA
    over the admitted tokens with the additive mask S' - S; soft and hard gate."""
    rng = np.random.default_rng(11)
    d, T = 16, 400
    K = _clustered(rng, 7, d)
    V = rng.standard_normal((448, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    idx = np.array([0, 2, 3, 6], np.int32)
    S, rows = _scores(q, K, idx, T)
    for tau in [float(np.median(S)), float(np.quantile(S, 0.8))]:
        for hard in (False, True):
            Sg = np.array([s * O.gate(s, tau, 5.0, hard) for s in S])
            want, want_lse = _sdpa(q, K[rows], V[rows], mask=Sg - S)
            out, lse = O.attend(q, K, V, T, tau, idx, beta=5.0, hard=hard)
            np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
            assert abs(lse - want_lse) < 1e-12


def check_attend_uniform_floor(O):
    """All admitted scores far below tau: every logit is suppressed to 0, each weight is
    e^0 = 1, so out is the plain mean of the admitted values and lse = log(n)."""
    w, _ = golden("suppressed_logit_weight")
    rng = np.random.default_rng(12)
    d, T = 16, 200
    K = rng.standard_normal((256, d)).astype(np.float32)
    V = rng.standard_normal((256, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    idx = np.array([1, 3], np.int32)
    out, lse = O.attend(q, K, V, T, 1e3, idx, beta=5.0)
    rows = np.r_[64:128, 192:200]
    np.testing.assert_allclose(out, V[rows].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)
    assert abs(lse - math.log(len(rows) * w)) < 1e-12


def check_attend_closed_forms(O):
    """Constant V rows give that row; a single admitted token gives its value and its
    gated logit as lse; an empty set gives zeros and -inf."""
    rng = np.random.default_rng(13)
    d = 16
    K = rng.standard_normal((192, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    row = rng.standard_normal(d).astype(np.float32)
    Vc = np.tile(row, (192, 1))
    out, _ = O.attend(q, K, Vc, 192, 0.1, np.array([0, 2], np.int32))
    np.testing.assert_allclose(out, row.astype(np.float64), rtol=0, atol=1e-12)
    V = rng.standard_normal((192, d)).astype(np.float32)
    out, lse = O.attend(q, K, V, 129, -0.2, np.array([2], np.int32))
    np.testing.assert_allclose(out, V[128].astype(np.float64), rtol=0, atol=1e-14)
    S = float(K[128].astype(np.float64) @ q.astype(np.float64)) / math.sqrt(d)
    assert abs(lse - S * O.gate(S, -0.2, 5.0)) < 1e-13
    out, lse = O.attend(q, K, V, 192, 0.0, np.zeros(0, np.int32))
    assert np.array_equal(out, np.zeros(d)) and lse == -math.inf


def check_attend_ignores_tail_and_order(O):
    """Rows at or beyond T are never read (NaN there changes nothing), and the result
    does not depend on the order of tokens inside the admitted blocks."""
    rng = np.random.default_rng(14)
    d, T = 16, 150
    K = rng.standard_normal((192, d)).astype(np.float32)
    V = rng.standard_normal((192, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    idx = np.array([0, 2], np.int32)
    ref, ref_lse = O.attend(q, K, V, T, 0.0, idx)
    Kn, Vn = K.copy(), V.copy()
    Kn[T:] = np.nan
    Vn[T:] = np.nan
    out, lse = O.attend(q, Kn, Vn, T, 0.0, idx)
    assert np.array_equal(out, ref) and lse == ref_lse
    perm = np.arange(192)
    perm[0:64] = rng.permutation(64)
    perm[128:T] = 128 + rng.permutation(T - 128)
    out, lse = O.attend(q, K[perm], V[perm], T, 0.0, idx)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    assert abs(lse - ref_lse) < 1e-13


def _sdpa_rows(Q, K, V, mask):
    """Library attention of many queries in float64 with an additive mask [T_q, T_k]
    (-inf hides a key); returns (out [T_q, d], lse [T_q])."""
    Qt = torch.from_numpy(np.asarray(Q, dtype=np.float64))[None, None]
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    mt = torch.from_numpy(np.asarray(mask, dtype=np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mt)
    logits = (Qt[0, 0] @ Kt[0, 0].T) / math.sqrt(K.shape[1]) + mt[0, 0]
    return out[0, 0].numpy(), torch.logsumexp(logits, dim=1).numpy()


def _causal(T_q, T_k):
    """Visibility of the training-time forward: query t sits at position T_k - T_q + t."""
    return np.arange(T_k)[None, :] <= (T_k - T_q + np.arange(T_q))[:, None]


def check_prefill_dense_is_causal_sdpa(O):
    """tau = -inf: every gate is 1, so the training-time forward is causal softmax
    attention (library SDPA in float64 with a bottom-right causal mask), for a whole
    sequence and for a chunk continuing a prefix; the gate sum counts the visible keys."""
    rng = np.random.default_rng(21)
    d = 16
    K = rng.standard_normal((150, d)).astype(np.float32)
    V = rng.standard_normal((150, d)).astype(np.float32)
    for T_q, T_k in [(130, 130), (37, 150), (1, 1), (1, 150)]:
        Q = rng.standard_normal((T_q, d)).astype(np.float32)
        vis = _causal(T_q, T_k)
        want, want_lse = _sdpa_rows(Q, K[:T_k], V[:T_k], np.where(vis, 0.0, -np.inf))
        out, lse, gs = O.prefill(Q, K, V, T_k, np.full(T_q, -np.inf))
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)
        assert np.array_equal(gs, vis.sum(axis=1).astype(np.float64))


def check_prefill_gated_is_masked_sdpa(O):
    """Finite per-token tau: the training-time forward equals SDPA with the additive
    mask S' - S on visible keys (gate from scipy's logistic function, an independent
    library routine) and -inf on hidden ones; the gate sum is the sum of those gates
    (soft) or the count of visible S >= tau (hard); bf16 K/V widened exactly."""
    from scipy.special import expit
    rng = np.random.default_rng(22)
    d, T_q, T_k = 16, 70, 200
    K32 = _clustered(rng, 4, d)[:T_k]
    V32 = rng.standard_normal((T_k, d)).astype(np.float32)
    Q = rng.standard_normal((T_q, d)).astype(np.float32)
    tau = rng.normal(0.3, 0.5, T_q)
    vis = _causal(T_q, T_k)
    for KK, VV, Kv, Vv in [(K32, V32, K32, V32),
                           (f32_to_bf16_bits(K32), f32_to_bf16_bits(V32),
                            bf16_bits_to_f64(f32_to_bf16_bits(K32)),
                            bf16_bits_to_f64(f32_to_bf16_bits(V32)))]:
        S = (Q.astype(np.float64) @ np.asarray(Kv, np.float64).T) / math.sqrt(d)
        for beta, hard in [(5.0, False), (1.0, False), (5.0, True)]:
            gate = (S >= tau[:, None]).astype(np.float64) if hard else expit(beta * (S - tau[:, None]))
            mask = np.where(vis, S * gate - S, -np.inf)
            want, want_lse = _sdpa_rows(Q, Kv, Vv, mask)
            out, lse, gs = O.prefill(Q, KK, VV, T_k, tau, beta=beta, hard=hard)
            np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)
            np.testing.assert_allclose(gs, np.where(vis, gate, 0.0).sum(axis=1), rtol=0, atol=1e-9)


def check_prefill_uniform_floor(O):
    """tau = +inf suppresses every logit to 0 (weight e^0 = 1): each query's output is
    the plain mean of its visible values, lse = log(visible count), gate sum 0."""
    rng = np.random.default_rng(23)
    d, T_q, T_k = 8, 20, 90
    K = rng.standard_normal((T_k, d)).astype(np.float32)
    V = rng.standard_normal((T_k, d)).astype(np.float32)
    Q = rng.standard_normal((T_q, d)).astype(np.float32)
    out, lse, gs = O.prefill(Q, K, V, T_k, np.full(T_q, np.inf))
    for t in range(T_q):
        n = T_k - T_q + t + 1
        np.testing.assert_allclose(out[t], V[:n].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[t] - math.log(n)) < 1e-12 and gs[t] == 0.0


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
