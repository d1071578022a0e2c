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
// item past a unit's list exits at once. A workgroup of NW waves takes one
// item; wave w processes the item's blocks w, w+NW, ... one 64-token block at
// a time:
//   - every lane issues 16-byte loads: a wave load covers four whole token
//     rows (row r of the wave = one token, lane c = elements [EPL*c, EPL*c+EPL));
//     tokens at or beyond T are clamped to a present row and masked out;
//   - dot products reduce over the 16 lanes of a DPP row;
//   - the gated logits of the whole block are formed first, so the running
//     (max, sum, weighted V) state is rescaled once per block, not per token.
// The waves' states merge in LDS; a one-item unit writes its output directly.
// Otherwise each item stores its (max, sum, weighted V) partial, and the last
// item to finish (device-scope counter) merges all partials of the unit in item
// order with a log-sum-exp combine -- deterministic, one kernel for the whole
// attention step. A prologue kernel clears the counters, so the workspace
// needs no initialisation.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kAttnWaves = 4;

struct AttnArgs {
    int units, T, T_cap, nblk, nblk_cap, split, ws_chunks;
    float s, beta_log2e;
    int hard;
    const float *q;
    const void *K;
    const void *V;
    const float *tau;
    const int32_t *idx;
    const int32_t *cnt;
    float *out;
    float *lse;
    int *ws_count;
    float *ws_m;
    float *ws_l;
    float *ws_o;
};

__global__ void clear_counts_kernel(int *__restrict__ c, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) c[i] = 0;
}

// Gate of Eq. 2 applied multiplicatively (Eq. 3).
__device__ __forceinline__ float gated(float S, float t, float beta_log2e, int hard) {
    if (hard) return S >= t ? S : 0.f;
    const float e = __builtin_amdgcn_exp2f(-beta_log2e * (S - t));
    return S * __builtin_amdgcn_rcpf(1.f + e);
}

template <typename KV, int D, int TS>
__global__ __launch_bounds__(kAttnWaves *kWave) void decode_attn_kernel(AttnArgs a) {
    constexpr int EPL = D / 16;
    constexpr int LOADS = TS / 4;  // token rows per lane per sub-block
    __shared__ float sm_m[kAttnWaves];
    __shared__ float sm_l[kAttnWaves];
    __shared__ float sm_o[kAttnWaves][D];
    __shared__ int sm_last;

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

    const KV *Ku = static_cast<const KV *>(a.K) + (size_t)u * a.T_cap * D + col * EPL;
    const KV *Vu = static_cast<const KV *>(a.V) + (size_t)u * a.T_cap * D + col * EPL;
    const int32_t *iu = a.idx + (size_t)u * a.nblk_cap;

    float m_run = -INFINITY;
    float l_run = 0.f;  // per row: sum over this row's tokens
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    const int j0 = chunk * a.split;
    const int j1 = min(c, j0 + a.split);
    for (int j = j0 + wave; j < j1; j += kAttnWaves) {
        const int blk = iu[j];
        if ((unsigned)blk >= (unsigned)a.nblk) continue;  // not a present block: skip it
        const int tb = blk * kBlockTokens;
        const int n = min(a.T - tb, kBlockTokens);
#pragma unroll
        for (int sub = 0; sub < kBlockTokens; sub += TS) {
            RowLoad<KV, EPL> kl[LOADS], vl[LOADS];
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int tok = min(sub + 4 * i + row, n - 1);
                kl[i].load(Ku + (size_t)(tb + tok) * D);
            }
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int tok = min(sub + 4 * i + row, n - 1);
                vl[i].load(Vu + (size_t)(tb + tok) * D);
            }
            float sg[LOADS];
            float bmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                float x[EPL];
                kl[i].widen(x);
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot += qr[e] * x[e];
                const float S = row_sum16(dot);
                const float g = gated(S, t, a.beta_log2e, a.hard);
                sg[i] = (sub + 4 * i + row < n) ? g : -INFINITY;
                bmax = fmaxf(bmax, sg[i]);
            }
            bmax = xrow_max(bmax);
            const float m_new = fmaxf(m_run, bmax);
            const float corr = fast_exp(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] *= corr;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const float p = fast_exp(sg[i] - m_new);
                l_run += p;
                float x[EPL];
                vl[i].widen(x);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] += p * x[e];
            }
            m_run = m_new;
        }
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
    float L = 0.f;
    float wgt[kAttnWaves];
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        wgt[w] = fast_exp(sm_m[w] - M);  // a wave without blocks has m = -inf: weight 0
        L += sm_l[w] * wgt[w];
    }
    float O = 0.f;
    if (tid < D) {
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) O += sm_o[w][tid] * wgt[w];
    }

    if (nchunks == 1) {
        if (tid < D) a.out[(size_t)u * D + tid] = O / L;
        if (tid == 0 && a.lse) a.lse[u] = M + __logf(L);
        return;
    }

    // store this item's partial, then let the last item of the unit combine
    const size_t slot = (size_t)u * a.ws_chunks + chunk;
    if (tid < D) a.ws_o[slot * D + tid] = O;
    if (tid == 0) {
        a.ws_m[slot] = M;
        a.ws_l[slot] = L;
    }
    __threadfence();  // release the partial at device scope before counting
    __syncthreads();
    if (tid == 0) {
        const int prev = atomicAdd(&a.ws_count[u], 1);
        sm_last = (prev == nchunks - 1);
    }
    __syncthreads();
    if (!sm_last) return;
    __threadfence();  // acquire the other items' partials

    const size_t s0 = (size_t)u * a.ws_chunks;
    float Mx = -INFINITY;
    for (int i = 0; i < nchunks; ++i) Mx = fmaxf(Mx, a.ws_m[s0 + i]);
    float Lx = 0.f, Ox = 0.f;
    for (int i = 0; i < nchunks; ++i) {
        const float w = fast_exp(a.ws_m[s0 + i] - Mx);
        Lx += a.ws_l[s0 + i] * w;
        if (tid < D) Ox += a.ws_o[(s0 + i) * D + tid] * w;
    }
    if (tid < D) a.out[(size_t)u * D + tid] = Ox / Lx;
    if (tid == 0) {
        if (a.lse) a.lse[u] = Mx + __logf(Lx);
        a.ws_count[u] = 0;
    }
}

template <typename KV, int D, int TS>
hipError_t launch_attn_t(const AttnArgs &a, int grid_chunks, hipStream_t st) {
    const long long grid = (long long)a.units * grid_chunks;
    hipLaunchKernelGGL((decode_attn_kernel<KV, D, TS>), dim3((unsigned)grid),
                       dim3(kAttnWaves * kWave), 0, st, a);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

AttnWorkspace attn_workspace_layout(int units, int max_chunks, int d) {
    AttnWorkspace w;
    const size_t slots = (size_t)units * (size_t)max_chunks;
    w.off_count = 0;
    w.off_m = align256(w.off_count + sizeof(int) * (size_t)units);
    w.off_l = align256(w.off_m + sizeof(float) * slots);
    w.off_o = align256(w.off_l + sizeof(float) * slots);
    w.bytes = align256(w.off_o + sizeof(float) * slots * (size_t)d);
    return w;
}

hipError_t launch_decode_attn(const Geometry &g, const float *q, const void *K, const void *V,
                              const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                              float gate_beta, bool gate_hard, int split_blocks, int max_chunks,
                              float *out, float *lse, void *ws, hipStream_t st) {
    if (g.units == 0) return hipSuccess;
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
    a.beta_log2e = gate_beta * kLog2e;
    a.hard = gate_hard ? 1 : 0;
    a.q = q;
    a.K = K;
    a.V = V;
    a.tau = tau;
    a.idx = adm_idx;
    a.cnt = adm_cnt;
    a.out = out;
    a.lse = lse;
    a.ws_count = reinterpret_cast<int *>(base + w.off_count);
    a.ws_m = reinterpret_cast<float *>(base + w.off_m);
    a.ws_l = reinterpret_cast<float *>(base + w.off_l);
    a.ws_o = reinterpret_cast<float *>(base + w.off_o);

    hipLaunchKernelGGL(clear_counts_kernel, dim3((unsigned)((g.units + 255) / 256)), dim3(256),
                       0, st, a.ws_count, g.units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // items needed at the current length (at least one per unit for the
    // empty-list case)
    int grid_chunks = (g.nblk + split_blocks - 1) / split_blocks;
    if (grid_chunks < 1) grid_chunks = 1;
    if (g.bf16) {
        return g.d == 128 ? launch_attn_t<uint16_t, 128, 64>(a, grid_chunks, st)
                          : launch_attn_t<uint16_t, 64, 64>(a, grid_chunks, st);
    }
    return g.d == 128 ? launch_attn_t<float, 128, 32>(a, grid_chunks, st)
                      : launch_attn_t<float, 64, 64>(a, grid_chunks, st);
}

}  // namespace eta
