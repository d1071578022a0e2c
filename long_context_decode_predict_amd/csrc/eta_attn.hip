// eta_attn.hip -- block-sparse split-KV decode attention with the ETA gate.
//
// arXiv:2609.20888: only the admitted blocks are loaded (evolve.pub review,
// Q&A "What is ETA?"); each logit S = s*q.k is multiplied by the gate
// sigmoid(beta*(S - tau)) (review "Methodology Assessment", Eq. 2 and Eq. 3),
// so a sub-threshold logit tends to 0 (weight e^0 = 1) instead of -inf, which
// absorbs the tokens that coarse block selection lets in (abstract).
//
// Work decomposition. A unit's ascending admitted list is cut into work items
// of `split` blocks; the grid is (item index) x (unit), item-major, and an
// item past a unit's list exits at once. A workgroup of four waves takes one
// item; wave w walks the item's blocks w, w+4, ... in tiles of TS tokens:
//   - row r of the wave owns one token and lane c of the row the EPL = d/16
//     elements [EPL*c, EPL*c + EPL) of it, so one 16-byte load per lane covers
//     four whole token rows; every load is a uniform block base plus a fixed
//     per-lane offset plus an immediate, so no per-load address arithmetic;
//   - software pipeline per wave: the V tile of tile t and the K tile of tile
//     t+1 are in flight while tile t's logits and weighted values are formed;
//   - dot products reduce over the 16 lanes of a DPP row; the gated logits of
//     a whole tile are formed first, so the running (max, sum, weighted V)
//     state is rescaled once per tile, not per token.
// The waves' states merge in LDS. A one-item unit writes out/lse directly;
// otherwise each item stores a (max, sum, weighted V) partial and the combine
// kernel merges a unit's partials in item order with a log-sum-exp
// (deterministic; the kernel boundary orders the two, so no fences or atomics
// are needed).
//
// The K/V capacity is a whole number of blocks, so the rows of a partial last
// block past T are inside the allocation: they are loaded unclamped and masked
// (their logits become -inf and their values are zeroed before use).
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kAttnWaves = 4;

struct AttnArgs {
    int units, T, T_cap, nblk, nblk_cap, split, ws_chunks;
    float s, nbl2e;  // 1/sqrt(d), -beta*log2(e)
    const float *q;
    const void *K;
    const void *V;
    const float *tau;
    const int32_t *idx;
    const int32_t *cnt;
    float *out;
    float *lse;
    float *ws_m;
    float *ws_l;
    float *ws_o;
};

// Zero the raw bits of a row held in registers (used for rows past T).
template <typename KV, int EPL>
__device__ __forceinline__ void zero_row(RowLoad<KV, EPL> &r);
template <>
__device__ __forceinline__ void zero_row<uint16_t, 8>(RowLoad<uint16_t, 8> &r) { r.raw = make_uint4(0, 0, 0, 0); }
template <>
__device__ __forceinline__ void zero_row<uint16_t, 4>(RowLoad<uint16_t, 4> &r) { r.raw = make_uint2(0, 0); }
template <>
__device__ __forceinline__ void zero_row<float, 8>(RowLoad<float, 8> &r) {
    r.a = make_float4(0.f, 0.f, 0.f, 0.f);
    r.b = r.a;
}
template <>
__device__ __forceinline__ void zero_row<float, 4>(RowLoad<float, 4> &r) { r.a = make_float4(0.f, 0.f, 0.f, 0.f); }

template <typename KV, int D, int TS, bool HARD>
__global__ __launch_bounds__(kAttnWaves *kWave) void attn_partial_kernel(AttnArgs a) {
    constexpr int EPL = D / 16;
    constexpr int L = TS / 4;                 // row loads per lane per tile
    constexpr int TPB = kBlockTokens / TS;    // tiles per block
    constexpr int ROW = D;                    // elements per token row
    __shared__ float sm_m[kAttnWaves];
    __shared__ float sm_l[kAttnWaves];
    __shared__ float sm_o[kAttnWaves][D];

    const int u = blockIdx.x % a.units;
    const int chunk = blockIdx.x / a.units;
    const int c = a.cnt[u];
    const int nchunks = (c + a.split - 1) / a.split;
    if (chunk >= (nchunks > 1 ? nchunks : 1)) return;

    const int tid = threadIdx.x;
    if (c <= 0) {  // nothing admitted: out = 0, lse = -inf
        for (int i = tid; i < D; i += blockDim.x) a.out[(size_t)u * D + i] = 0.f;
        if (tid == 0 && a.lse) a.lse[u] = -INFINITY;
        return;
    }

    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;

    float qr[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[e] = a.q[(size_t)u * D + col * EPL + e] * a.s;
    const float t = a.tau[u];
    const float nbt = -a.nbl2e * t;  // gate exponent = nbl2e * S + nbt

    const KV *Ku = static_cast<const KV *>(a.K) + (size_t)u * a.T_cap * ROW;
    const KV *Vu = static_cast<const KV *>(a.V) + (size_t)u * a.T_cap * ROW;
    const int lane_off = row * ROW + col * EPL;  // element offset inside a 4-row group
    const int32_t *iu = a.idx + (size_t)u * a.nblk_cap;

    const int j0 = chunk * a.split;
    const int j1 = min(c, j0 + a.split);
    // this wave's blocks: j0 + wave + k*kAttnWaves < j1
    const int nb = (j1 - j0 - wave + kAttnWaves - 1) / kAttnWaves;
    const int ntiles = nb > 0 ? nb * TPB : 0;

    float m_run = -INFINITY;
    float l_run = 0.f;  // per row: sum over this row's tokens
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    auto tile_block = [&](int tt) { return iu[j0 + wave + (tt / TPB) * kAttnWaves]; };
    auto tile_base = [&](int blk, int tt) {
        return (size_t)blk * kBlockTokens * ROW + (size_t)((tt % TPB) * TS) * ROW;
    };

    RowLoad<KV, EPL> kb[L], vb[L];
    if (ntiles > 0) {
        const KV *p = Ku + tile_base(tile_block(0), 0) + lane_off;
#pragma unroll
        for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
    }
    for (int tt = 0; tt < ntiles; ++tt) {
        const int blk = tile_block(tt);
        const size_t base = tile_base(blk, tt);
        // rows of this tile below T (TS or more for every tile but a partial last block's)
        const int valid = min(a.T - blk * kBlockTokens, kBlockTokens) - (tt % TPB) * TS;
        {
            const KV *p = Vu + base + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) vb[i].load(p + i * 4 * ROW);
        }
        // gated logits of the tile
        float sg[L];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[EPL];
            kb[i].widen(x);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot += qr[e] * x[e];
            const float S = row_sum16(dot);
            float g;
            if (HARD) {
                g = S >= t ? S : 0.f;
            } else {
                g = S * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(a.nbl2e, S, nbt)));
            }
            sg[i] = g;
        }
        if (valid < TS) {  // partial last block: rows past T take no weight
#pragma unroll
            for (int i = 0; i < L; ++i)
                if (4 * i + row >= valid) sg[i] = -INFINITY;
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < L; ++i) bmax = fmaxf(bmax, sg[i]);
        // the K registers are free: start the next tile's K loads
        if (tt + 1 < ntiles) {
            const KV *p = Ku + tile_base(tile_block(tt + 1), tt + 1) + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
        }
        bmax = xrow_max(bmax);
        const float m_new = fmaxf(m_run, bmax);
        const float corr = fast_exp(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= corr;
        if (valid < TS) {
#pragma unroll
            for (int i = 0; i < L; ++i)
                if (4 * i + row >= valid) zero_row<KV, EPL>(vb[i]);
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const float p = fast_exp(sg[i] - m_new);
            l_run += p;
            float x[EPL];
            vb[i].widen(x);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] += p * x[e];
        }
        m_run = m_new;
    }

    // merge the four rows of the wave (m_run is wave-uniform)
    const float l_w = xrow_sum(l_run);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = xrow_sum(o[e]);
    if (lane == 0) {
        sm_m[wave] = m_run;
        sm_l[wave] = l_w;
    }
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_o[wave][lane * EPL + e] = o[e];
    }
    __syncthreads();

    // merge the waves of the workgroup
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w]);
    float Lsum = 0.f;
    float wgt[kAttnWaves];
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        wgt[w] = fast_exp(sm_m[w] - M);  // a wave without blocks has m = -inf: weight 0
        Lsum += sm_l[w] * wgt[w];
    }
    if (tid < D) {
        float O = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) O += sm_o[w][tid] * wgt[w];
        if (nchunks == 1) {
            a.out[(size_t)u * D + tid] = O / Lsum;
        } else {
            const size_t slot = (size_t)u * a.ws_chunks + chunk;
            a.ws_o[slot * D + tid] = O;
        }
    }
    if (tid == 0) {
        if (nchunks == 1) {
            if (a.lse) a.lse[u] = M + __logf(Lsum);
        } else {
            const size_t slot = (size_t)u * a.ws_chunks + chunk;
            a.ws_m[slot] = M;
            a.ws_l[slot] = Lsum;
        }
    }
}

// Log-sum-exp merge of the partials of every unit that has more than one item.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
    const int u = blockIdx.x;
    const int c = a.cnt[u];
    const int nchunks = (c + a.split - 1) / a.split;
    if (nchunks <= 1) return;
    const size_t s0 = (size_t)u * a.ws_chunks;
    float M = -INFINITY;
    for (int i = 0; i < nchunks; ++i) M = fmaxf(M, a.ws_m[s0 + i]);
    float Lsum = 0.f, O = 0.f;
    const int tid = threadIdx.x;
    for (int i = 0; i < nchunks; ++i) {
        const float w = fast_exp(a.ws_m[s0 + i] - M);
        Lsum += a.ws_l[s0 + i] * w;
        O += a.ws_o[(s0 + i) * D + tid] * w;
    }
    a.out[(size_t)u * D + tid] = O / Lsum;
    if (tid == 0 && a.lse) a.lse[u] = M + __logf(Lsum);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

AttnArgs make_args(const Geometry &g, const float *q, const void *K, const void *V,
                   const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                   float gate_beta, int split_blocks, int max_chunks, float *out, float *lse,
                   void *ws) {
    const AttnWorkspace w = attn_workspace_layout(g.units, max_chunks, g.d);
    char *base = static_cast<char *>(ws);
    AttnArgs a;
    a.units = g.units;
    a.T = g.T;
    a.T_cap = g.T_cap;
    a.nblk = g.nblk;
    a.nblk_cap = g.nblk_cap;
    a.split = split_blocks;
    a.ws_chunks = max_chunks;
    a.s = 1.0f / sqrtf((float)g.d);
    a.nbl2e = -gate_beta * kLog2e;
    a.q = q;
    a.K = K;
    a.V = V;
    a.tau = tau;
    a.idx = adm_idx;
    a.cnt = adm_cnt;
    a.out = out;
    a.lse = lse;
    a.ws_m = reinterpret_cast<float *>(base + w.off_m);
    a.ws_l = reinterpret_cast<float *>(base + w.off_l);
    a.ws_o = reinterpret_cast<float *>(base + w.off_o);
    return a;
}

template <typename KV, int D, int TS>
hipError_t launch_partial_t(const AttnArgs &a, bool hard, int grid_chunks, hipStream_t st) {
    const dim3 grid((unsigned)((long long)a.units * grid_chunks));
    if (hard) {
        hipLaunchKernelGGL((attn_partial_kernel<KV, D, TS, true>), grid, dim3(kAttnWaves * kWave), 0,
                           st, a);
    } else {
        hipLaunchKernelGGL((attn_partial_kernel<KV, D, TS, false>), grid, dim3(kAttnWaves * kWave),
                           0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

AttnWorkspace attn_workspace_layout(int units, int max_chunks, int d) {
    AttnWorkspace w;
    const size_t slots = (size_t)units * (size_t)max_chunks;
    w.off_m = 0;
    w.off_l = align256(w.off_m + sizeof(float) * slots);
    w.off_o = align256(w.off_l + sizeof(float) * slots);
    w.bytes = align256(w.off_o + sizeof(float) * slots * (size_t)d);
    return w;
}

hipError_t launch_attn_partial(const Geometry &g, const float *q, const void *K, const void *V,
                               const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                               float gate_beta, bool gate_hard, int split_blocks, int max_chunks,
                               float *out, float *lse, void *ws, hipStream_t st) {
    if (g.units == 0) return hipSuccess;
    const AttnArgs a = make_args(g, q, K, V, tau, adm_idx, adm_cnt, gate_beta, split_blocks,
                                 max_chunks, out, lse, ws);
    // items needed at the current length (at least one per unit for the empty list)
    int grid_chunks = (g.nblk + split_blocks - 1) / split_blocks;
    if (grid_chunks < 1) grid_chunks = 1;
    if (g.bf16) {
        return g.d == 128 ? launch_partial_t<uint16_t, 128, 64>(a, gate_hard, grid_chunks, st)
                          : launch_partial_t<uint16_t, 64, 64>(a, gate_hard, grid_chunks, st);
    }
    return g.d == 128 ? launch_partial_t<float, 128, 32>(a, gate_hard, grid_chunks, st)
                      : launch_partial_t<float, 64, 64>(a, gate_hard, grid_chunks, st);
}

hipError_t launch_attn_combine(const Geometry &g, const int32_t *adm_cnt, int split_blocks,
                               int max_chunks, float *out, float *lse, void *ws, hipStream_t st) {
    if (g.units == 0) return hipSuccess;
    const AttnArgs a = make_args(g, nullptr, nullptr, nullptr, nullptr, nullptr, adm_cnt, 1.f,
                                 split_blocks, max_chunks, out, lse, ws);
    if (g.d == 128) {
        hipLaunchKernelGGL((attn_combine_kernel<128>), dim3((unsigned)g.units), dim3(128), 0, st, a);
    } else {
        hipLaunchKernelGGL((attn_combine_kernel<64>), dim3((unsigned)g.units), dim3(64), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace eta
