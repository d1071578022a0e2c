// eta_screen.hip -- O(1) per-block screen and ordered compaction.
//
// arXiv:2609.20888 abstract: each KV block is screened in constant time from a
// cached bound with a geometric and a probabilistic part; evolve.pub review,
// Q&A "What is ETA?": a block none of whose keys can reach the threshold is
// skipped. With
// s = 1/sqrt(d):
//   U_geo  = s * |q| * maxnorm                       (Cauchy-Schwarz)
//   U_prob = s * (q . centroid + z * |q| * sqrt(var))
//   U = min(U_geo, U_prob), or U_geo alone; admit iff U >= tau.
//
// Multi-head attention: one workgroup per (batch, head) unit, up to 8 waves.
// Grouped heads: one workgroup per key/value unit screens its G query heads,
// each with its own query and threshold, from one read of the shared metadata
// (screen_group_kernel, below). The centroids are
// dimension-major per unit, so lane l of a wave handles four consecutive
// blocks and every load of one dimension is a contiguous 1 KiB run across the
// wave (float4 per lane), with no cross-lane reduction. When a unit has few
// blocks, the head dimension is split across DS waves that work on the same
// 256 blocks (partial dot products meet in LDS and are added in slice order),
// so short contexts still put enough loads in flight. Admission bits are
// compacted with wave ballots plus an LDS exclusive scan over the block
// groups: the admitted list comes out ascending with no atomics.
//
// Each unit screens only the blocks of its own row (rows may hold different
// numbers of tokens); bounds past the row's last block are not written, apart
// from -inf in the float4 that holds that block.
//
// With PRED the workgroup first evaluates the threshold predictor of its unit
// (evolve.pub review, "Methodology Assessment", Eq. 1: tau = qbar . W + b over
// the concatenated queries of the batch row) and stores tau for the attention.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kScreenMaxWaves = 8;  // two workgroups fit a CU: one streams while the other syncs
constexpr int kBlocksPerLane = 4;
constexpr int kBlocksPerWave = kWave * kBlocksPerLane;
constexpr int kMaxSlices = 8;
constexpr int kDimBatch = 4;  // grouped screen: centroid dimensions loaded per batch
constexpr int kGroupMaxWaves = 8;  // grouped screen: waves per workgroup (registers for G heads)

struct ScreenArgs {
    int nblk, nblk_cap, H, G, nbg, ds;  // query heads per KV head, block groups, slices
    float s, z;
    int geo_only;
    const float *q;
    float *tau;        // read, or written with PRED
    const float *W;    // PRED: [H*d][H] or null (frozen tau = bias)
    const float *bias;
    const float *centroid;
    const float *var;
    const float *maxnorm;
    int32_t *adm_idx;
    int32_t *adm_cnt;
    float *bound_out;
    KVLayout lay;  // per-row token counts (the K/V addresses are not used here)
    int32_t *uni_idx;  // grouped heads: union per key/value unit (null: not formed here)
    int32_t *uni_cnt;
    int w_vec;         // W is 16-byte aligned and H % 4 == 0 (rows of W load as float4)
};

template <int D, bool PRED>
__global__ __launch_bounds__(kScreenMaxWaves *kWave) void screen_kernel(ScreenArgs a) {
    __shared__ float q_s[D];
    __shared__ float4 part[kScreenMaxWaves][kWave];  // partial dots, per wave and lane
    __shared__ int wave_tot[kScreenMaxWaves];
    __shared__ float red[kScreenMaxWaves];
    __shared__ float tau_s;

    const int u = blockIdx.x;
    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int grp = wave / a.ds;    // block group of this wave
    const int slice = wave % a.ds;  // dimension slice of this wave
    const int dps = D / a.ds;       // dimensions per slice

    for (int i = threadIdx.x; i < D; i += blockDim.x) q_s[i] = a.q[(size_t)u * D + i];
    if (PRED) {
        const int b = u / a.H, h = u - (u / a.H) * a.H;
        float acc = 0.f;
        if (a.W != nullptr) {
            const float *qb = a.q + (size_t)b * a.H * D;
            for (int k = threadIdx.x; k < a.H * D; k += blockDim.x) acc += qb[k] * a.W[(size_t)k * a.H + h];
        }
        acc = xrow_sum(row_sum16(acc));
        if (lane == 0) red[wave] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[w];
            const float t = a.bias[h] + sum;
            tau_s = t;
            a.tau[u] = t;
        }
    } else {
        if (threadIdx.x == 0) tau_s = a.tau[u];
    }
    __syncthreads();

    float qq = 0.f;
    for (int i = lane; i < D; i += kWave) qq += q_s[i] * q_s[i];
    const float qn = sqrtf(xrow_sum(row_sum16(qq)));
    const float t = tau_s;
    const float geo_scale = a.s * qn;
    const float z_scale = a.z * qn;

    const int nblk = (a.lay.row_len(u / a.H) + kBlockTokens - 1) / kBlockTokens;  // this row's blocks
    const int ukv = u / a.G;  // the key/value unit whose metadata this query head screens
    const float *cu = a.centroid + (size_t)ukv * D * a.nblk_cap;
    const float *vu = a.var + (size_t)ukv * a.nblk_cap;
    const float *mu = a.maxnorm + (size_t)ukv * a.nblk_cap;
    int32_t *iu = a.adm_idx + (size_t)u * a.nblk_cap;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int d0 = slice * dps;

    int base = 0;
    for (int pass0 = 0; pass0 < nblk; pass0 += a.nbg * kBlocksPerWave) {
        const int blk0 = pass0 + grp * kBlocksPerWave + lane * kBlocksPerLane;
        const bool active = blk0 < nblk;  // nblk_cap % 4 == 0: the float4 is in bounds
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        // max norms and variances first: their loads overlap the centroid rows'
        float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f), v4 = m4;
        if (slice == 0 && active) {
            m4 = ld_stream(reinterpret_cast<const float4 *>(mu + blk0));
            if (!a.geo_only) v4 = ld_stream(reinterpret_cast<const float4 *>(vu + blk0));
        }
        if (active && !a.geo_only) {
            // batches of kDimBatch dimensions (dps is a multiple of 8), the next
            // batch's loads in flight while the current one is used
            const float *cp = cu + (size_t)d0 * a.nblk_cap + blk0;
            const size_t st = a.nblk_cap;
            const int nbt = dps / kDimBatch;
            float4 cb[2][kDimBatch];
            auto load = [&](float4(&dst)[kDimBatch], int bt) {
#pragma unroll
                for (int i = 0; i < kDimBatch; ++i)
                    dst[i] = ld_stream(reinterpret_cast<const float4 *>(cp + (size_t)(bt * kDimBatch + i) * st));
            };
            auto use = [&](const float4(&src)[kDimBatch], int bt) {
#pragma unroll
                for (int i = 0; i < kDimBatch; ++i) {
                    const float qd = q_s[d0 + bt * kDimBatch + i];
                    acc[0] += qd * src[i].x;
                    acc[1] += qd * src[i].y;
                    acc[2] += qd * src[i].z;
                    acc[3] += qd * src[i].w;
                }
            };
            load(cb[0], 0);
            for (int bt = 0; bt < nbt; bt += 2) {  // nbt is even
                load(cb[1], bt + 1);
                use(cb[0], bt);
                if (bt + 2 < nbt) load(cb[0], bt + 2);
                use(cb[1], bt + 1);
            }
        }
        if (a.ds > 1) {  // add the slices' partial dots in slice order
            part[wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            __syncthreads();
            if (slice == 0) {
                float4 sum = part[wave][lane];
                for (int k = 1; k < a.ds; ++k) {
                    const float4 p = part[wave + k][lane];
                    sum.x += p.x;
                    sum.y += p.y;
                    sum.z += p.z;
                    sum.w += p.w;
                }
                acc[0] = sum.x;
                acc[1] = sum.y;
                acc[2] = sum.z;
                acc[3] = sum.w;
            }
        }

        float U[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        bool adm[4] = {false, false, false, false};
        int before = 0;
        if (slice == 0) {
            if (active) {
                const float mx[4] = {m4.x, m4.y, m4.z, m4.w};
                if (a.geo_only) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) U[j] = geo_scale * mx[j];
                } else {
                    const float vx[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float u_geo = geo_scale * mx[j];
                        const float u_prob = a.s * (acc[j] + z_scale * sqrtf(vx[j]));
                        U[j] = (u_prob < u_geo) ? u_prob : u_geo;
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (blk0 + j >= nblk) U[j] = -INFINITY;
            }
            int total = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                adm[j] = active && (blk0 + j < nblk) && (U[j] >= t);
                const uint64_t mask = __ballot(adm[j]);
                before += __popcll(mask & lanes_below);
                total += __popcll(mask);
            }
            if (lane == 0) wave_tot[grp] = total;
        }
        __syncthreads();
        int grp_base = 0, pass_total = 0;
        for (int g = 0; g < a.nbg; ++g) {
            const int c = wave_tot[g];
            grp_base += (g < grp) ? c : 0;
            pass_total += c;
        }
        if (slice == 0) {
            int pos = base + grp_base + before;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (adm[j]) iu[pos++] = blk0 + j;
            }
            if (a.bound_out != nullptr && active) {
                *reinterpret_cast<float4 *>(a.bound_out + (size_t)u * a.nblk_cap + blk0) =
                    make_float4(U[0], U[1], U[2], U[3]);
            }
        }
        base += pass_total;
        __syncthreads();  // wave_tot and part are rewritten by the next pass
    }
    if (threadIdx.x == 0) a.adm_cnt[u] = base;
}

// Grouped heads: one workgroup per key/value unit screens its G query heads
// together, so each block's metadata is read once for all of them (a query head
// of the group otherwise re-reads the same centroids). Lane l of wave w handles
// blocks 256w + 4l .. + 3 of each pass; every centroid float4 feeds 4G FMAs.
// Each head's list is compacted exactly as in screen_kernel (ballots plus an
// LDS scan over the waves), so it comes out ascending with no atomics; when
// asked, the union of the G lists is compacted the same way from the OR of the
// heads' admission bits.
template <int D, bool PRED, int G>
__global__ __launch_bounds__(kGroupMaxWaves *kWave) void screen_group_kernel(ScreenArgs a) {
    __shared__ float q_s[G][D];
    __shared__ int wave_tot[G + 1][kGroupMaxWaves];  // per head, then the union
    __shared__ float red[G][kGroupMaxWaves];
    __shared__ float tau_s[G];

    const int ukv = blockIdx.x;  // key/value unit; its query units are ukv*G + j
    const int u0 = ukv * G;
    const int b = u0 / a.H;
    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);

    for (int i = threadIdx.x; i < G * D; i += blockDim.x) q_s[i / D][i % D] = a.q[(size_t)u0 * D + i];
    if (PRED) {
        // the group's G heads are G adjacent columns of W: one pass over W's rows
        // reads each row's G entries together (one 16-byte load per 4 heads)
        const int h0 = u0 - b * a.H;
        float acc[G];
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = 0.f;
        if (a.W != nullptr) {
            const float *qb = a.q + (size_t)b * a.H * D;
            const int HD = a.H * D;
            if (G % 4 == 0 && a.w_vec) {
#pragma unroll 4
                for (int k = threadIdx.x; k < HD; k += blockDim.x) {
                    const float qv = qb[k];
                    const float4 *wr = reinterpret_cast<const float4 *>(a.W + (size_t)k * a.H + h0);
#pragma unroll
                    for (int j4 = 0; j4 < G / 4; ++j4) {
                        const float4 w4 = wr[j4];
                        acc[4 * j4 + 0] += qv * w4.x;
                        acc[4 * j4 + 1] += qv * w4.y;
                        acc[4 * j4 + 2] += qv * w4.z;
                        acc[4 * j4 + 3] += qv * w4.w;
                    }
                }
            } else {
#pragma unroll 4
                for (int k = threadIdx.x; k < HD; k += blockDim.x) {
                    const float qv = qb[k];
                    const float *wr = a.W + (size_t)k * a.H + h0;
#pragma unroll
                    for (int j = 0; j < G; ++j) acc[j] += qv * wr[j];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float r = xrow_sum(row_sum16(acc[j]));
            if (lane == 0) red[j][wave] = r;
        }
        __syncthreads();
        if (threadIdx.x < G) {
            const int j = threadIdx.x;
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[j][w];
            const float t = a.bias[h0 + j] + sum;
            tau_s[j] = t;
            a.tau[u0 + j] = t;
        }
        __syncthreads();
    } else {
        if (threadIdx.x < G) tau_s[threadIdx.x] = a.tau[u0 + threadIdx.x];
        __syncthreads();
    }

    float t[G], geo_scale[G], z_scale[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float qq = 0.f;
        for (int i = lane; i < D; i += kWave) qq += q_s[j][i] * q_s[j][i];
        const float qn = sqrtf(xrow_sum(row_sum16(qq)));
        t[j] = tau_s[j];
        geo_scale[j] = a.s * qn;
        z_scale[j] = a.z * qn;
    }

    const int nblk = (a.lay.row_len(b) + kBlockTokens - 1) / kBlockTokens;  // this row's blocks
    const float *cu = a.centroid + (size_t)ukv * D * a.nblk_cap;
    const float *vu = a.var + (size_t)ukv * a.nblk_cap;
    const float *mu = a.maxnorm + (size_t)ukv * a.nblk_cap;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    int base[G];
#pragma unroll
    for (int j = 0; j < G; ++j) base[j] = 0;
    int base_u = 0;
    const bool with_union = a.uni_idx != nullptr;
    for (int pass0 = 0; pass0 < nblk; pass0 += nw * kBlocksPerWave) {
        const int blk0 = pass0 + wave * kBlocksPerWave + lane * kBlocksPerLane;
        const bool active = blk0 < nblk;  // nblk_cap % 4 == 0: the float4 is in bounds
        float acc[G][4];
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.f;
        // max norms and variances first: their loads overlap the centroid rows'
        float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f), v4 = m4;
        if (active) {
            m4 = ld_stream(reinterpret_cast<const float4 *>(mu + blk0));
            if (!a.geo_only) v4 = ld_stream(reinterpret_cast<const float4 *>(vu + blk0));
        }
        if (active && !a.geo_only) {
            // centroid rows in batches of kDimBatch dimensions, the next batch's loads
            // in flight while the current one is used
            const float *cp = cu + blk0;
            const size_t st = a.nblk_cap;
            float4 cb[2][kDimBatch];
#pragma unroll
            for (int i = 0; i < kDimBatch; ++i) cb[0][i] = ld_stream(reinterpret_cast<const float4 *>(cp + i * st));
#pragma unroll
            for (int bt = 0; bt < D / kDimBatch; ++bt) {
                const int cur = bt & 1;
                if (bt + 1 < D / kDimBatch) {
#pragma unroll
                    for (int i = 0; i < kDimBatch; ++i)
                        cb[cur ^ 1][i] = ld_stream(reinterpret_cast<const float4 *>(
                            cp + (size_t)((bt + 1) * kDimBatch + i) * st));
                }
#pragma unroll
                for (int i = 0; i < kDimBatch; ++i) {
                    const float4 c4 = cb[cur][i];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const float qd = q_s[j][bt * kDimBatch + i];
                        acc[j][0] += qd * c4.x;
                        acc[j][1] += qd * c4.y;
                        acc[j][2] += qd * c4.z;
                        acc[j][3] += qd * c4.w;
                    }
                }
            }
        }
        const float mx[4] = {m4.x, m4.y, m4.z, m4.w};
        const float vx[4] = {v4.x, v4.y, v4.z, v4.w};
        int before[G];
        bool uadm[4] = {false, false, false, false};
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float U[4];
            bool adm[4];
            int bf = 0, total = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float u_geo = geo_scale[j] * mx[e];
                if (a.geo_only) {
                    U[e] = u_geo;
                } else {
                    const float u_prob = a.s * (acc[j][e] + z_scale[j] * sqrtf(vx[e]));
                    U[e] = (u_prob < u_geo) ? u_prob : u_geo;
                }
                if (!active || blk0 + e >= nblk) U[e] = -INFINITY;
                adm[e] = active && (blk0 + e < nblk) && (U[e] >= t[j]);
                const uint64_t mask = __ballot(adm[e]);
                bf += __popcll(mask & lanes_below);
                total += __popcll(mask);
            }
            before[j] = bf;
            if (lane == 0) wave_tot[j][wave] = total;
            if (a.bound_out != nullptr && active) {
                *reinterpret_cast<float4 *>(a.bound_out + (size_t)(u0 + j) * a.nblk_cap + blk0) =
                    make_float4(U[0], U[1], U[2], U[3]);
            }
            // the admitted blocks are rewritten after the scan below: keep the bits
#pragma unroll
            for (int e = 0; e < 4; ++e) uadm[e] = uadm[e] || adm[e];
            acc[j][0] = adm[0] ? 1.f : 0.f;
            acc[j][1] = adm[1] ? 1.f : 0.f;
            acc[j][2] = adm[2] ? 1.f : 0.f;
            acc[j][3] = adm[3] ? 1.f : 0.f;
        }
        int before_u = 0;
        if (with_union) {
            int total = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint64_t mask = __ballot(uadm[e]);
                before_u += __popcll(mask & lanes_below);
                total += __popcll(mask);
            }
            if (lane == 0) wave_tot[G][wave] = total;
        }
        __syncthreads();
        if (with_union) {
            int grp_base = 0, pass_total = 0;
            for (int w = 0; w < nw; ++w) {
                const int c = wave_tot[G][w];
                grp_base += (w < wave) ? c : 0;
                pass_total += c;
            }
            int32_t *iu = a.uni_idx + (size_t)ukv * a.nblk_cap;
            int pos = base_u + grp_base + before_u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (uadm[e]) iu[pos++] = blk0 + e;
            base_u += pass_total;
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            int grp_base = 0, pass_total = 0;
            for (int w = 0; w < nw; ++w) {
                const int c = wave_tot[j][w];
                grp_base += (w < wave) ? c : 0;
                pass_total += c;
            }
            int32_t *iu = a.adm_idx + (size_t)(u0 + j) * a.nblk_cap;
            int pos = base[j] + grp_base + before[j];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (acc[j][e] != 0.f) iu[pos++] = blk0 + e;
            base[j] += pass_total;
        }
        __syncthreads();  // wave_tot is rewritten by the next pass
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
        if ((int)threadIdx.x == j) a.adm_cnt[u0 + j] = base[j];
    if (with_union && threadIdx.x == 0) a.uni_cnt[ukv] = base_u;
}

// Block groups per pass and dimension slices: up to 8 waves; split the
// dimension when the unit has fewer than 8 x 256 blocks.
void pick_shape(int nblk, int d, int *nbg, int *ds) {
    int g = (nblk + kBlocksPerWave - 1) / kBlocksPerWave;
    g = g < 1 ? 1 : (g > kScreenMaxWaves ? kScreenMaxWaves : g);
    int pow2 = 1;
    while (pow2 < g) pow2 <<= 1;  // block groups rounded up to a power of two
    int slices = kScreenMaxWaves / pow2;
    if (slices > kMaxSlices) slices = kMaxSlices;
    while (slices > 1 && d / slices < 8) slices >>= 1;  // keep >= 8 dimensions per slice
    *nbg = pow2;
    *ds = slices < 1 ? 1 : slices;
}

template <int D>
hipError_t launch_screen_t(const Geometry &g, int H, const float *q, float *tau, const float *W,
                           const float *bias, bool predict, const float *c, const float *v,
                           const float *m, float z, bool geo_only, int32_t *idx, int32_t *cnt,
                           float *bound_out, hipStream_t st, int32_t *uni_idx, int32_t *uni_cnt) {
    ScreenArgs a;
    pick_shape(g.nblk, D, &a.nbg, &a.ds);
    a.nblk = g.nblk;
    a.nblk_cap = g.nblk_cap;
    a.H = H;
    a.G = g.G;
    a.s = 1.0f / sqrtf((float)D);
    a.z = z;
    a.geo_only = geo_only ? 1 : 0;
    a.q = q;
    a.tau = tau;
    a.W = W;
    a.bias = bias;
    a.centroid = c;
    a.var = v;
    a.maxnorm = m;
    a.adm_idx = idx;
    a.adm_cnt = cnt;
    a.bound_out = bound_out;
    a.lay = g.lay;
    a.uni_idx = g.G > 1 ? uni_idx : nullptr;
    a.uni_cnt = g.G > 1 ? uni_cnt : nullptr;
    a.w_vec = (W != nullptr && reinterpret_cast<uintptr_t>(W) % 16 == 0 && H % 4 == 0) ? 1 : 0;
    if (g.G > 1) {
        int nw = (g.nblk + kBlocksPerWave - 1) / kBlocksPerWave;
        nw = nw < 1 ? 1 : (nw > kGroupMaxWaves ? kGroupMaxWaves : nw);
        const dim3 grid((unsigned)g.kv_units), blk(nw * kWave);
#define ETA_SCREEN_GROUP(GG)                                                                   \
    if (predict) {                                                                             \
        hipLaunchKernelGGL((screen_group_kernel<D, true, GG>), grid, blk, 0, st, a);          \
    } else {                                                                                   \
        hipLaunchKernelGGL((screen_group_kernel<D, false, GG>), grid, blk, 0, st, a);         \
    }
        switch (g.G) {
            case 2: ETA_SCREEN_GROUP(2) break;
            case 4: ETA_SCREEN_GROUP(4) break;
            default: ETA_SCREEN_GROUP(8) break;
        }
#undef ETA_SCREEN_GROUP
        return hipGetLastError();
    }
    const dim3 block(a.nbg * a.ds * kWave);
    if (predict) {
        hipLaunchKernelGGL((screen_kernel<D, true>), dim3((unsigned)g.units), block, 0, st, a);
    } else {
        hipLaunchKernelGGL((screen_kernel<D, false>), dim3((unsigned)g.units), block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_screen(const Geometry &g, int H, const float *q, float *tau, const float *W,
                         const float *bias, bool predict, const float *centroid,
                         const float *var, const float *maxnorm, float z, bool geo_only,
                         int32_t *adm_idx, int32_t *adm_cnt, float *bound_out, hipStream_t st,
                         int32_t *uni_idx, int32_t *uni_cnt) {
    if (g.units == 0) return hipSuccess;
    return g.d == 128 ? launch_screen_t<128>(g, H, q, tau, W, bias, predict, centroid, var, maxnorm,
                                             z, geo_only, adm_idx, adm_cnt, bound_out, st,
                                             uni_idx, uni_cnt)
                      : launch_screen_t<64>(g, H, q, tau, W, bias, predict, centroid, var, maxnorm,
                                            z, geo_only, adm_idx, adm_cnt, bound_out, st,
                                            uni_idx, uni_cnt);
}

}  // namespace eta
