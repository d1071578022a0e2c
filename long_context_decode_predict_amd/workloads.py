"""Seeded synthetic decode workloads shaped like the pages' long-context setting.

Input generation only: this module draws random tensors and holds none of the
method's arithmetic. Both the HIP path and the oracle are handed the bytes it
produces (the oracle gets device-to-host copies).

Recipe (per (batch, head) unit, per 64-token block): a block centroid drawn
from N(0, 1)^d; each key = centroid + N(0, sigma^2) elementwise (clustered
keys, sigma = 0.3 unless a per-head range is given); values ~ N(0, 1); the
post-RoPE query ~ N(0, 1)^d; the predictor W is block-diagonal (head h reads
only its own query slice) with entries N(0, 1/d). Grouped heads (H_kv < H):
K/V per key/value head, and the G = H / H_kv queries of a group share a common
direction, q_h = c * q_group + sqrt(1 - c^2) * xi_h (c = group_corr), and so do
their predictor columns, as the query heads that read one key/value head tend
to in trained models. Optional "needle" keys: in a
fraction of the blocks one key at a seeded slot is replaced by
r * (0.9 * q_hat + sqrt(0.19) * u), u a random unit vector orthogonal to q_hat,
r = sqrt(d (1 + sigma^2)) -- a key aligned with the query at cosine 0.9.
Variable-length rows: row b holds T_b tokens, drawn uniformly in
[(1 - var_len) T, T] (the largest row is set to T). Paged caches: each present
64-token block of each row gets its own page of a pool [P, H_kv, 64, d], pages
assigned in a seeded random order; pages no block uses, and the rows past T_b of
a row's last page, are filled with NaN, so that any read the layout does not
allow shows in the results.
All draws use torch generators seeded per workload on the target device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 64
SEED_BASE = 20260916


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    T: int                      # tokens present at the timed step
    kv_dtype: torch.dtype
    sigma: float = 0.3          # in-block key spread
    sigma_range: tuple | None = None   # per-head spread ~ U(lo, hi) instead of sigma
    density: float = 0.38       # target mean admitted-block fraction
    head_densities: tuple | None = None  # static per-head targets (no predictor)
    needle_frac: float = 0.0
    append: int = 0             # tokens appended one by one before the step
    H_kv: int = 0               # key/value heads (0: multi-head, H_kv = H)
    group_corr: float = 0.0     # shared direction of a group's queries (grouped heads)
    head_corr: float = 0.0      # multi-head: block structure shared by a row's heads
    var_len: float = 0.0        # row lengths ~ U[(1 - var_len) T, T] (0: every row holds T)
    paged: bool = False         # K/V in a shuffled page pool with a page table
    seed: int = SEED_BASE
    note: str = field(default="", compare=False)

    @property
    def static_tau(self) -> bool:
        return self.head_densities is not None

    @property
    def kv_heads(self) -> int:
        return self.H_kv if self.H_kv else self.H

    @property
    def G(self) -> int:
        return self.H // self.kv_heads

    @property
    def T_cap(self) -> int:
        """Cache capacity: T rounded up to whole 64-token blocks (at least one)."""
        return max(BLOCK, (self.T + BLOCK - 1) // BLOCK * BLOCK)

    @property
    def nblk(self) -> int:
        return (self.T + BLOCK - 1) // BLOCK


WORKLOADS = {
    "tiny_b1_h4_d64_t2k_f32": Workload(
        "tiny_b1_h4_d64_t2k_f32", B=1, H=4, d=64, T=2048, kv_dtype=torch.float32,
        seed=SEED_BASE + 0, note="tiny single decode step, fp32 K/V"),
    "llama_b32_h16_d128_t32k_bf16": Workload(
        "llama_b32_h16_d128_t32k_bf16", B=32, H=16, d=128, T=32768, kv_dtype=torch.bfloat16,
        head_corr=0.992, seed=SEED_BASE + 1,
        note="LLaMA-style layer decode, heads of a row selecting overlapping blocks"),
    "headline_b64_h16_d128_t128k_bf16": Workload(
        "headline_b64_h16_d128_t128k_bf16", B=64, H=16, d=128, T=131072,
        kv_dtype=torch.bfloat16, needle_frac=0.01, seed=SEED_BASE + 2,
        note="headline decode with planted needle keys"),
    "sparse_b16_h16_d128_t512k_bf16": Workload(
        "sparse_b16_h16_d128_t512k_bf16", B=16, H=16, d=128, T=524288,
        kv_dtype=torch.bfloat16, density=0.16, append=128, seed=SEED_BASE + 3,
        note="sparse long context, 128 single-token appends before the step"),
    "static_b64_h16_d128_t64k_bf16": Workload(
        "static_b64_h16_d128_t64k_bf16", B=64, H=16, d=128, T=65536,
        kv_dtype=torch.bfloat16, sigma_range=(0.1, 0.6),
        head_densities=tuple(0.1 + 0.8 * h / 15 for h in range(16)), seed=SEED_BASE + 4,
        note="frozen per-head thresholds, per-head densities 10..90%"),
    "gqa_b32_h32kv8_d128_t128k_bf16": Workload(
        "gqa_b32_h32kv8_d128_t128k_bf16", B=32, H=32, d=128, T=131072,
        kv_dtype=torch.bfloat16, H_kv=8, group_corr=0.95, seed=SEED_BASE + 5,
        note="grouped heads (4 query heads per key/value head), union loading"),
    "gqa8_b16_h64kv8_d128_t128k_bf16": Workload(
        "gqa8_b16_h64kv8_d128_t128k_bf16", B=16, H=64, d=128, T=131072,
        kv_dtype=torch.bfloat16, H_kv=8, group_corr=0.95, seed=SEED_BASE + 7,
        note="eight query heads per key/value head (a 70B-class layer), union loading"),
    "paged_b64_h16_d128_t128k_bf16": Workload(
        "paged_b64_h16_d128_t128k_bf16", B=64, H=16, d=128, T=131072,
        kv_dtype=torch.bfloat16, var_len=0.5, paged=True, seed=SEED_BASE + 6,
        note="paged pool, shuffled pages, row lengths 64k..128k"),
}

HEADLINE = "headline_b64_h16_d128_t128k_bf16"


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit sizes (tests use small ragged ones)."""
    base = dict(B=1, H=2, d=128, T=300, kv_dtype=torch.bfloat16)
    base.update(kw)
    return Workload(name, **base)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def head_sigmas(w: Workload) -> torch.Tensor:
    """In-block key spread per key/value head (float32 [H_kv], on the CPU)."""
    if w.sigma_range is None:
        return torch.full((w.kv_heads,), float(w.sigma), dtype=torch.float32)
    g = _gen("cpu", w.seed + 7)
    lo, hi = w.sigma_range
    return (lo + (hi - lo) * torch.rand(w.kv_heads, generator=g)).to(torch.float32)


def generate(w: Workload, device="cuda", T_cap: int | None = None) -> dict:
    """Draw q, K, V, W for a workload on `device`.

    Returns dict(q [B,H,d] f32, K, V [B,H_kv,T_cap,d] kv_dtype, W [H*d,H] f32 or None,
    sigmas [H_kv], needles: LongTensor [n,3] of (unit, block, slot) or None)."""
    T_cap = w.T_cap if T_cap is None else T_cap
    B, H, d = w.B, w.H, w.d
    Hk = w.kv_heads
    nblk_cap = (T_cap + BLOCK - 1) // BLOCK
    g = _gen(device, w.seed)
    q = torch.randn((B, H, d), generator=g, device=device, dtype=torch.float32)
    if w.G > 1 and w.group_corr > 0:
        base = torch.randn((B, Hk, 1, d), generator=g, device=device, dtype=torch.float32)
        c = float(w.group_corr)
        q = (c * base + math.sqrt(1.0 - c * c) * q.view(B, Hk, w.G, d)).reshape(B, H, d)
    hc = float(w.head_corr) if w.G == 1 else 0.0
    if hc > 0:  # the heads of a row share a query direction (and, below, block centroids)
        base = torch.randn((B, 1, d), generator=g, device=device, dtype=torch.float32)
        q = hc * base + math.sqrt(1.0 - hc * hc) * q
    sig = head_sigmas(w).to(device)
    K = torch.empty((B, Hk, T_cap, d), dtype=w.kv_dtype, device=device)
    V = torch.empty((B, Hk, T_cap, d), dtype=w.kv_dtype, device=device)
    for b in range(B):  # one batch row at a time keeps fp32 temporaries small
        cen = torch.randn((Hk, nblk_cap, 1, d), generator=g, device=device, dtype=torch.float32)
        if hc > 0:
            shared = torch.randn((1, nblk_cap, 1, d), generator=g, device=device,
                                 dtype=torch.float32)
            cen.mul_(math.sqrt(1.0 - hc * hc)).add_(shared, alpha=hc)
            del shared
        noise = torch.randn((Hk, nblk_cap, BLOCK, d), generator=g, device=device,
                            dtype=torch.float32)
        noise.mul_(sig.view(Hk, 1, 1, 1)).add_(cen)
        K[b].copy_(noise.view(Hk, nblk_cap * BLOCK, d)[:, :T_cap])
        del noise, cen
        vb = torch.randn((Hk, T_cap, d), generator=g, device=device, dtype=torch.float32)
        V[b].copy_(vb)
        del vb
    W = None
    if not w.static_tau:
        W = torch.zeros((H * d, H), dtype=torch.float32, device=device)
        wdiag = torch.randn((H, d), generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
        if w.G > 1 and w.group_corr > 0:  # a group's predictor columns share a direction too
            wb = torch.randn((Hk, 1, d), generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
            c = float(w.group_corr)
            wdiag = (c * wb + math.sqrt(1.0 - c * c) * wdiag.view(Hk, w.G, d)).reshape(H, d)
        if hc > 0:  # and so do the heads' predictor columns
            wb = torch.randn((1, d), generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
            wdiag = hc * wb + math.sqrt(1.0 - hc * hc) * wdiag
        for h in range(H):
            W[h * d:(h + 1) * d, h] = wdiag[h]
    needles = None
    if w.needle_frac > 0:
        needles = plant_needles(w, q, K, sig, g, T_cap)
    return {"q": q, "K": K, "V": V, "W": W, "sigmas": sig, "needles": needles}


def plant_needles(w: Workload, q, K, sig, g, T_cap):
    """Replace one key in a seeded fraction of each unit's blocks by a key aligned with
    the unit's query at cosine 0.9. Returns (unit, block, slot) triples."""
    assert w.G == 1, "needles are planted for multi-head workloads only"
    B, H, d = w.B, w.H, w.d
    nblk = w.nblk
    per_unit = max(1, int(round(w.needle_frac * nblk)))
    dev = q.device
    units = B * H
    # seeded distinct blocks per unit and a slot inside each
    keys = torch.rand((units, nblk), generator=g, device=dev)
    blocks = torch.argsort(keys, dim=1)[:, :per_unit]
    slots = torch.randint(0, BLOCK, (units, per_unit), generator=g, device=dev)
    tok = blocks * BLOCK + slots
    tok = torch.minimum(tok, torch.full_like(tok, w.T - 1))
    qf = q.reshape(units, d)
    qhat = qf / qf.norm(dim=1, keepdim=True)
    u = torch.randn((units, per_unit, d), generator=g, device=dev)
    u = u - (u * qhat[:, None, :]).sum(-1, keepdim=True) * qhat[:, None, :]
    u = u / u.norm(dim=-1, keepdim=True)
    sig_u = sig.repeat(B)  # unit = b*H + h
    r = torch.sqrt(d * (1.0 + sig_u ** 2))[:, None, None]
    key = r * (0.9 * qhat[:, None, :] + math.sqrt(0.19) * u)
    Kf = K.view(units, T_cap, d)
    rows = torch.arange(units, device=dev)[:, None].expand_as(tok)
    Kf[rows.reshape(-1), tok.reshape(-1)] = key.reshape(-1, d).to(K.dtype)
    return torch.stack([rows.reshape(-1), (tok // BLOCK).reshape(-1), (tok % BLOCK).reshape(-1)], 1)


def row_lengths(w: Workload) -> list[int]:
    """Seeded tokens per row: every row holds T unless var_len > 0."""
    if w.var_len <= 0:
        return [w.T] * w.B
    g = _gen("cpu", w.seed + 11)
    lo = int(math.floor((1.0 - w.var_len) * w.T))
    lens = torch.randint(lo, w.T + 1, (w.B,), generator=g).tolist()
    lens[int(torch.randint(0, w.B, (1,), generator=g))] = w.T  # the largest row holds T
    return [int(t) for t in lens]


def page_pool(K: torch.Tensor, V: torch.Tensor, lens, seed: int, spare: int = 3,
              all_blocks: bool = False, interleaved: bool = False):
    """Scatter a dense cache [B,H_kv,T_cap,d] into a shuffled page pool.

    Returns (page_table int32 [B, T_cap/64], Kp, Vp [P,H_kv,64,d]). Block j of row b
    gets a page when j < ceil(lens[b] / 64) (every block with all_blocks); the
    table holds an out-of-range id (-1, or P + 5 on odd rows) for the others.
    Unused pages and the rows past lens[b] of a row's last page are NaN.
    interleaved: one allocation [P, H_kv, 2, 64, d] holding each (page, head) block's
    K rows then its V rows; Kp and Vp are its strided views [:, :, 0] and [:, :, 1]
    (kv_block_stride = 128*d)."""
    B, Hk, T_cap, d = K.shape
    mp = T_cap // BLOCK
    dev = K.device
    need = [mp if all_blocks else (int(t) + BLOCK - 1) // BLOCK for t in lens]
    n_used = sum(need)
    P = n_used + spare
    g = _gen("cpu", seed + 13)
    perm = torch.randperm(P, generator=g)
    table = torch.empty((B, mp), dtype=torch.int32)
    nxt = 0
    for b in range(B):
        table[b, :need[b]] = perm[nxt:nxt + need[b]].to(torch.int32)
        table[b, need[b]:] = -1 if b % 2 == 0 else P + 5
        nxt += need[b]
    if interleaved:
        pool = torch.full((P, Hk, 2, BLOCK, d), float("nan"), dtype=K.dtype, device=dev)
        Kp, Vp = pool[:, :, 0], pool[:, :, 1]
    else:
        Kp = torch.full((P, Hk, BLOCK, d), float("nan"), dtype=K.dtype, device=dev)
        Vp = torch.full((P, Hk, BLOCK, d), float("nan"), dtype=V.dtype, device=dev)
    for b in range(B):  # one row at a time: no dense-sized temporaries
        if need[b] == 0:
            continue
        pages = table[b, :need[b]].to(dev, torch.long)
        Kp[pages] = K[b, :, :need[b] * BLOCK].reshape(Hk, need[b], BLOCK, d).transpose(0, 1)
        Vp[pages] = V[b, :, :need[b] * BLOCK].reshape(Hk, need[b], BLOCK, d).transpose(0, 1)
        tail = int(lens[b]) % BLOCK
        if tail and not all_blocks:
            last = int(table[b, need[b] - 1])
            Kp[last, :, tail:] = float("nan")
            Vp[last, :, tail:] = float("nan")
    return table.to(dev), Kp, Vp


def gather_unit(pool: torch.Tensor, table: torch.Tensor, b: int, k: int, T_b: int) -> torch.Tensor:
    """The first T_b tokens [T_b, d] of key/value head k of row b, read through the table."""
    nb = (T_b + BLOCK - 1) // BLOCK
    if nb == 0:
        return pool.new_empty((0, pool.shape[-1]))
    pages = table[b, :nb].to(pool.device, torch.long)
    return pool[pages, k].reshape(nb * BLOCK, pool.shape[-1])[:T_b]


@dataclass(frozen=True)
class PrefillWorkload:
    """A training-time (prefill) forward: T_q queries at the end of T_k keys."""
    name: str
    B: int
    H: int
    d: int
    T_q: int
    T_k: int
    H_kv: int = 0
    sigma: float = 0.3           # in-block key spread, as for the decode caches
    inclusion: float = 0.15      # target mean gate (about 85 % training sparsity)
    seed: int = SEED_BASE + 100
    note: str = field(default="", compare=False)

    @property
    def kv_heads(self) -> int:
        return self.H_kv if self.H_kv else self.H

    @property
    def G(self) -> int:
        return self.H // self.kv_heads


PREFILL_WORKLOADS = {
    "prefill_b4_h16_d128_t8k_bf16": PrefillWorkload(
        "prefill_b4_h16_d128_t8k_bf16", B=4, H=16, d=128, T_q=8192, T_k=8192,
        seed=SEED_BASE + 101, note="training-time forward of 8K sequences"),
    "prefill_b1_h32kv8_d128_t32k_bf16": PrefillWorkload(
        "prefill_b1_h32kv8_d128_t32k_bf16", B=1, H=32, d=128, T_q=32768, T_k=32768, H_kv=8,
        seed=SEED_BASE + 102, note="long prefill with grouped heads"),
}


def generate_prefill(w: PrefillWorkload, device="cuda", tau_mu: float = 0.5,
                     tau_sigma: float = 0.5) -> dict:
    """Q [B,H,T_q,d], K, V [B,H_kv,T_k,d] bfloat16 (keys clustered per 64-token block
    as in the decode caches), W [H*d,H] block-diagonal N(0, 1/d), and a seeded
    per-token threshold tau ~ N(tau_mu, tau_sigma^2) [B,H,T_q] float32 that both the
    kernels and the oracle take as an input."""
    g = _gen(device, w.seed)
    B, H, Hk, d = w.B, w.H, w.kv_heads, w.d
    nblk = (w.T_k + BLOCK - 1) // BLOCK
    Q = torch.randn((B, H, w.T_q, d), generator=g, device=device).to(torch.bfloat16)
    K = torch.empty((B, Hk, w.T_k, d), dtype=torch.bfloat16, device=device)
    V = torch.empty((B, Hk, w.T_k, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        cen = torch.randn((Hk, nblk, 1, d), generator=g, device=device)
        noise = torch.randn((Hk, nblk, BLOCK, d), generator=g, device=device)
        K[b].copy_((noise * w.sigma + cen).view(Hk, nblk * BLOCK, d)[:, :w.T_k])
        V[b].copy_(torch.randn((Hk, w.T_k, d), generator=g, device=device))
        del cen, noise
    W = torch.zeros((H * d, H), dtype=torch.float32, device=device)
    wdiag = torch.randn((H, d), generator=g, device=device) / math.sqrt(d)
    for h in range(H):
        W[h * d:(h + 1) * d, h] = wdiag[h]
    tau = tau_mu + tau_sigma * torch.randn((B, H, w.T_q), generator=g, device=device)
    return {"Q": Q, "K": K, "V": V, "W": W, "tau": tau.float()}
