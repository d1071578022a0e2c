// eta_meta.hip -- per-block key metadata (centroid, variance, max key norm).
//
// The cached block metadata is what makes the screen O(1) per block
// (arXiv:2609.20888 abstract; evolve.pub review "Summary": centroid /
// variance / max-norm). One wave computes one 64-token block entirely from
// registers (a single read of the keys); a workgroup of four waves covers 64
// consecutive blocks of one unit and writes the dimension-major centroid tile
// through LDS so that every global store is a contiguous 64-float run.
//
// The build and the incremental append launch the same kernel (only the block
// range differs), so an append is bitwise equal to a rebuild.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kMetaWaves = 4;
constexpr int kMetaBlocksPerGroup = 64;

// Statistics of block `blk` of one unit, computed by the calling wave.
// cen: the lane's EPL centroid dimensions (identical in all four rows);
// var and maxnorm are wave-uniform.
template <typename KV, int D>
__device__ __forceinline__ void block_stats(const KV *__restrict__ Ku, int blk, int T,
                                            float (&cen)[D / 16], float &var, float &maxnorm) {
    constexpr int EPL = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;
    const int t0 = blk * kBlockTokens;
    const int n = min(T - t0, kBlockTokens);  // >= 1 for a present block

    RowLoad<KV, EPL> ld[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = min(4 * i + row, n - 1);  // clamp: never read past T
        ld[i].load(Ku + (size_t)(t0 + t) * D + col * EPL);
    }

    float sum[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x[EPL];
        ld[i].widen(x);
        const bool valid = 4 * i + row < n;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sum[e] += valid ? x[e] : 0.f;
    }
    const float fn = (float)n;
#pragma unroll
    for (int e = 0; e < EPL; ++e) cen[e] = xrow_sum(sum[e]) / fn;

    float sq = 0.f;
    float nmax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x[EPL];
        ld[i].widen(x);
        const bool valid = 4 * i + row < n;
        float dev2 = 0.f, nrm2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float dd = x[e] - cen[e];
            dev2 += dd * dd;
            nrm2 += x[e] * x[e];
        }
        sq += valid ? dev2 : 0.f;
        nrm2 = row_sum16(nrm2);  // squared norm of this row's token
        nmax = valid ? fmaxf(nmax, nrm2) : nmax;
    }
    sq = xrow_sum(row_sum16(sq));
    nmax = xrow_max(nmax);
    var = sq / (fn * (float)D);
    maxnorm = sqrtf(nmax);
}

template <typename KV, int D>
__global__ __launch_bounds__(kMetaWaves *kWave) void block_meta_kernel(
    const KV *__restrict__ K, float *__restrict__ centroid, float *__restrict__ var,
    float *__restrict__ maxnorm, int T, int T_cap, int nblk_cap, int blk_begin, int blk_end,
    int groups_per_unit) {
    constexpr int EPL = D / 16;
    __shared__ float tile_c[D][kMetaBlocksPerGroup + 1];  // +1: no bank conflicts
    __shared__ float tile_v[kMetaBlocksPerGroup];
    __shared__ float tile_m[kMetaBlocksPerGroup];

    const int u = blockIdx.x / groups_per_unit;
    const int grp = blockIdx.x - u * groups_per_unit;
    const int first = blk_begin + grp * kMetaBlocksPerGroup;
    const int count = min(kMetaBlocksPerGroup, blk_end - first);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const KV *Ku = K + (size_t)u * T_cap * D;

    for (int j = wave; j < count; j += kMetaWaves) {
        float cen[EPL];
        float v, m;
        block_stats<KV, D>(Ku, first + j, T, cen, v, m);
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) tile_c[lane * EPL + e][j] = cen[e];
        }
        if (lane == 0) {
            tile_v[j] = v;
            tile_m[j] = m;
        }
    }
    __syncthreads();

    float *cu = centroid + (size_t)u * D * nblk_cap;
    for (int i = threadIdx.x; i < D * kMetaBlocksPerGroup; i += kMetaWaves * kWave) {
        const int dim = i / kMetaBlocksPerGroup;
        const int j = i - dim * kMetaBlocksPerGroup;
        if (j < count) cu[(size_t)dim * nblk_cap + first + j] = tile_c[dim][j];
    }
    for (int j = threadIdx.x; j < count; j += kMetaWaves * kWave) {
        var[(size_t)u * nblk_cap + first + j] = tile_v[j];
        maxnorm[(size_t)u * nblk_cap + first + j] = tile_m[j];
    }
}

template <typename KV, int D>
hipError_t launch_meta_t(const Geometry &g, const void *K, float *c, float *v, float *m,
                         int blk_begin, int blk_end, hipStream_t st) {
    const int groups = (blk_end - blk_begin + kMetaBlocksPerGroup - 1) / kMetaBlocksPerGroup;
    const dim3 grid((unsigned)((long long)g.kv_units * groups));
    hipLaunchKernelGGL((block_meta_kernel<KV, D>), grid, dim3(kMetaWaves * kWave), 0, st,
                       static_cast<const KV *>(K), c, v, m, g.T, g.T_cap, g.nblk_cap, blk_begin,
                       blk_end, groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_meta(const Geometry &g, const void *K, float *centroid, float *var,
                             float *maxnorm, int blk_begin, int blk_end, hipStream_t st) {
    if (blk_end <= blk_begin || g.kv_units == 0) return hipSuccess;
    if (g.bf16) {
        return g.d == 128 ? launch_meta_t<uint16_t, 128>(g, K, centroid, var, maxnorm, blk_begin, blk_end, st)
                          : launch_meta_t<uint16_t, 64>(g, K, centroid, var, maxnorm, blk_begin, blk_end, st);
    }
    return g.d == 128 ? launch_meta_t<float, 128>(g, K, centroid, var, maxnorm, blk_begin, blk_end, st)
                      : launch_meta_t<float, 64>(g, K, centroid, var, maxnorm, blk_begin, blk_end, st);
}

}  // namespace eta
