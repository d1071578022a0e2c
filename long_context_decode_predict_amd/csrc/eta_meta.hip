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
// range differs), so an append is bitwise equal to a rebuild. Rows may hold
// different numbers of tokens and their blocks may live in a page pool; the
// metadata stays indexed by logical block either way.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kMetaWaves = 4;
constexpr int kMetaBlocksPerGroup = 64;

// Statistics of the block at Kb (its first token row) holding n >= 1 tokens,
// computed by the calling wave. cen: the lane's EPL centroid dimensions
// (identical in all four rows); var and maxnorm are wave-uniform.
template <typename KV, int D, bool PART>
__device__ __forceinline__ void block_stats(const KV *__restrict__ Kb, int n,
                                            float (&cen)[D / 16], float &var, float &maxnorm) {
    constexpr int EPL = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;

    RowLoad<KV, EPL> ld[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = min(4 * i + row, n - 1);  // clamp: never read past the row's end
        ld[i].load(Kb + (size_t)t * D + col * EPL);
    }

    float sum[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x[EPL];
        ld[i].widen(x);
        const bool valid = !PART || 4 * i + row < n;
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
        const bool valid = !PART || 4 * i + row < n;
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

// One workgroup per (key/value unit, group of 64 blocks). Build (n_new = 0):
// blocks [blk_begin, blk_end) clipped to the row's blocks. Append (n_new > 0):
// the blocks touched by tokens [T_b, T_b + n_new) of row b, counted from the
// block holding token T_b. A block whose page id is out of range gets zero
// metadata.
template <typename KV, int D>
__global__ __launch_bounds__(kMetaWaves *kWave) void block_meta_kernel(
    const KV *__restrict__ K, float *__restrict__ centroid, float *__restrict__ var,
    float *__restrict__ maxnorm, KVLayout lay, int nblk_cap, int blk_begin, int blk_end,
    int n_new, int groups_per_unit) {
    constexpr int EPL = D / 16;
    __shared__ float tile_c[D][kMetaBlocksPerGroup + 1];  // +1: no bank conflicts
    __shared__ float tile_v[kMetaBlocksPerGroup];
    __shared__ float tile_m[kMetaBlocksPerGroup];

    const int u = blockIdx.x / groups_per_unit;
    const int grp = blockIdx.x - u * groups_per_unit;
    const int b = u / lay.H_kv;
    const int k = u - b * lay.H_kv;
    int len = lay.row_len(b);  // tokens of the row the statistics see
    int row_first = blk_begin, row_end = blk_end;
    if (n_new > 0) {
        row_first = len / kBlockTokens;
        len += n_new;
        row_end = (len + kBlockTokens - 1) / kBlockTokens;
    } else {
        row_end = min(row_end, (len + kBlockTokens - 1) / kBlockTokens);
    }
    const int first = row_first + grp * kMetaBlocksPerGroup;
    const int count = min(kMetaBlocksPerGroup, row_end - first);
    if (count <= 0) return;  // uniform over the workgroup
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);

    for (int j = wave; j < count; j += kMetaWaves) {
        const int blk = first + j;
        float cen[EPL];
        float v = 0.f, m = 0.f;
        const long long off = lay.block_offset(b, k, blk, D);
        if (off >= 0) {
            const int n = min(len - blk * kBlockTokens, kBlockTokens);
            if (n == kBlockTokens) {  // a whole block: no row masks
                block_stats<KV, D, false>(K + off, n, cen, v, m);
            } else {
                block_stats<KV, D, true>(K + off, n, cen, v, m);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) cen[e] = 0.f;
        }
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
                         int blk_begin, int blk_end, int n_new, hipStream_t st) {
    // blocks per row: the range, or at most ceil(n_new / 64) + 1 for an append
    const int span = n_new > 0 ? (n_new + kBlockTokens - 1) / kBlockTokens + 1 : blk_end - blk_begin;
    const int groups = (span + kMetaBlocksPerGroup - 1) / kMetaBlocksPerGroup;
    const dim3 grid((unsigned)((long long)g.kv_units * groups));
    hipLaunchKernelGGL((block_meta_kernel<KV, D>), grid, dim3(kMetaWaves * kWave), 0, st,
                       static_cast<const KV *>(K), c, v, m, g.lay, g.nblk_cap, blk_begin, blk_end,
                       n_new, groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_meta(const Geometry &g, const void *K, float *centroid, float *var,
                             float *maxnorm, int blk_begin, int blk_end, int n_new,
                             hipStream_t st) {
    if (g.kv_units == 0 || (n_new <= 0 && blk_end <= blk_begin)) return hipSuccess;
    if (g.bf16) {
        return g.d == 128 ? launch_meta_t<uint16_t, 128>(g, K, centroid, var, maxnorm, blk_begin, blk_end, n_new, st)
                          : launch_meta_t<uint16_t, 64>(g, K, centroid, var, maxnorm, blk_begin, blk_end, n_new, st);
    }
    return g.d == 128 ? launch_meta_t<float, 128>(g, K, centroid, var, maxnorm, blk_begin, blk_end, n_new, st)
                      : launch_meta_t<float, 64>(g, K, centroid, var, maxnorm, blk_begin, blk_end, n_new, st);
}

}  // namespace eta
