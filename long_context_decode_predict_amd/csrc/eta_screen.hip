// eta_screen.hip -- O(1) per-block screen and ordered compaction.
//
// arXiv:2609.20888 abstract: KV blocks are screened in O(1) time from cached
// geometric-probabilistic bounds; evolve.pub review, Q&A "What is ETA?": a
// block whose best possible score is below the threshold is skipped. With
// s = 1/sqrt(d):
//   U_geo  = s * |q| * maxnorm                       (Cauchy-Schwarz)
//   U_prob = s * (q . centroid + z * |q| * sqrt(var))
//   U = min(U_geo, U_prob), or U_geo alone; admit iff U >= tau.
//
// One workgroup per (batch, head) unit. The centroids are dimension-major per
// unit, so lane l of wave w handles four consecutive blocks and every load of
// one dimension is a contiguous 1 KiB run across the wave (float4 per lane);
// no cross-lane reduction is needed for the dot products. Admission bits are
// compacted with wave ballots plus an LDS exclusive scan over the waves, so
// the admitted list comes out ascending with no atomics (deterministic).
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kScreenMaxWaves = 16;
constexpr int kBlocksPerLane = 4;
constexpr int kBlocksPerWave = kWave * kBlocksPerLane;

template <int D>
__global__ __launch_bounds__(kScreenMaxWaves *kWave) void screen_kernel(
    int nblk, int nblk_cap, const float *__restrict__ q, const float *__restrict__ tau,
    const float *__restrict__ centroid, const float *__restrict__ var,
    const float *__restrict__ maxnorm, float s, float z, int geo_only,
    int32_t *__restrict__ adm_idx, int32_t *__restrict__ adm_cnt, float *__restrict__ bound_out) {
    __shared__ float q_s[D];
    __shared__ int wave_tot[kScreenMaxWaves];

    const int u = blockIdx.x;
    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);

    for (int i = threadIdx.x; i < D; i += blockDim.x) q_s[i] = q[(size_t)u * D + i];
    __syncthreads();

    float qq = 0.f;
    for (int i = lane; i < D; i += kWave) qq += q_s[i] * q_s[i];
    const float qn = sqrtf(xrow_sum(row_sum16(qq)));
    const float t = tau[u];
    const float geo_scale = s * qn;
    const float z_scale = z * qn;

    const float *cu = centroid + (size_t)u * D * nblk_cap;
    const float *vu = var + (size_t)u * nblk_cap;
    const float *mu = maxnorm + (size_t)u * nblk_cap;
    int32_t *iu = adm_idx + (size_t)u * nblk_cap;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    int base = 0;
    for (int pass0 = 0; pass0 < nblk; pass0 += nw * kBlocksPerWave) {
        const int blk0 = pass0 + wave * kBlocksPerWave + lane * kBlocksPerLane;
        const bool active = blk0 < nblk;  // nblk_cap % 4 == 0: the float4 is in bounds
        float U[kBlocksPerLane] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (active) {
            const float4 m4 = *reinterpret_cast<const float4 *>(mu + blk0);
            const float mx[4] = {m4.x, m4.y, m4.z, m4.w};
            if (geo_only) {
#pragma unroll
                for (int j = 0; j < 4; ++j) U[j] = geo_scale * mx[j];
            } else {
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
                for (int dim = 0; dim < D; ++dim) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(cu + (size_t)dim * nblk_cap + blk0);
                    const float qd = q_s[dim];
                    acc[0] += qd * c4.x;
                    acc[1] += qd * c4.y;
                    acc[2] += qd * c4.z;
                    acc[3] += qd * c4.w;
                }
                const float4 v4 = *reinterpret_cast<const float4 *>(vu + blk0);
                const float vx[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float u_geo = geo_scale * mx[j];
                    const float u_prob = s * (acc[j] + z_scale * sqrtf(vx[j]));
                    U[j] = (u_prob < u_geo) ? u_prob : u_geo;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (blk0 + j >= nblk) U[j] = -INFINITY;
        }

        bool adm[4];
        int before = 0, total = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            adm[j] = active && (blk0 + j < nblk) && (U[j] >= t);
            const uint64_t mask = __ballot(adm[j]);
            before += __popcll(mask & lanes_below);
            total += __popcll(mask);
        }
        if (lane == 0) wave_tot[wave] = total;
        __syncthreads();
        int wave_base = 0, pass_total = 0;
        for (int w = 0; w < nw; ++w) {
            const int c = wave_tot[w];
            wave_base += (w < wave) ? c : 0;
            pass_total += c;
        }
        int pos = base + wave_base + before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (adm[j]) iu[pos++] = blk0 + j;
        }
        if (bound_out != nullptr && active) {
            *reinterpret_cast<float4 *>(bound_out + (size_t)u * nblk_cap + blk0) =
                make_float4(U[0], U[1], U[2], U[3]);
        }
        base += pass_total;
        __syncthreads();  // wave_tot is rewritten by the next pass
    }
    if (threadIdx.x == 0) adm_cnt[u] = base;
}

template <int D>
hipError_t launch_screen_t(const Geometry &g, const float *q, const float *tau, const float *c,
                           const float *v, const float *m, float z, bool geo_only, int32_t *idx,
                           int32_t *cnt, float *bound_out, hipStream_t st) {
    int waves = (g.nblk + kBlocksPerWave - 1) / kBlocksPerWave;
    waves = waves < 1 ? 1 : (waves > kScreenMaxWaves ? kScreenMaxWaves : waves);
    const float s = 1.0f / sqrtf((float)D);
    hipLaunchKernelGGL((screen_kernel<D>), dim3((unsigned)g.units), dim3(waves * kWave), 0, st,
                       g.nblk, g.nblk_cap, q, tau, c, v, m, s, z, geo_only ? 1 : 0, idx, cnt,
                       bound_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_screen(const Geometry &g, const float *q, const float *tau,
                         const float *centroid, const float *var, const float *maxnorm, float z,
                         bool geo_only, int32_t *adm_idx, int32_t *adm_cnt, float *bound_out,
                         hipStream_t st) {
    if (g.units == 0) return hipSuccess;
    return g.d == 128 ? launch_screen_t<128>(g, q, tau, centroid, var, maxnorm, z, geo_only,
                                             adm_idx, adm_cnt, bound_out, st)
                      : launch_screen_t<64>(g, q, tau, centroid, var, maxnorm, z, geo_only,
                                            adm_idx, adm_cnt, bound_out, st);
}

}  // namespace eta
