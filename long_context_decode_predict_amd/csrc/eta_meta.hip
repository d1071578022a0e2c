// eta_meta.hip -- per-block key metadata (centroid, variance, max key norm, and
// optionally the largest squared key distance from the centroid).
//
// The cached block metadata is what makes the screen O(1) per block
// (arXiv:2609.20888 abstract; evolve.pub review "Summary": centroid /
// variance / max-norm). One wave computes one block from a single read of its
// keys held in registers; a workgroup of 8 waves covers 256 consecutive blocks
// of one unit and writes the dimension-major centroid tile through LDS, so
// every dimension's row of the tile leaves as one contiguous 1 KiB run of
// 16-byte stores.
//
// Statistics in one pass over the keys, shifted by the block's first key k0:
// with d_j = k_j - k0, the centroid is k0 + mean(d) and
//   sum_j |k_j - c|^2 = sum_j |d_j|^2 - n |mean(d)|^2,
// which is exact algebra; the shift keeps the two terms of the difference of
// the size of the in-block spread, so fp32 loses no more than in a two-pass
// sum (the shifted-data method for the variance). Each row load is consumed
// as it arrives, so no widened copy of the block stays live. Rows of a
// partial last block past its end load token 0 again: their d is exactly 0
// and token 0's norm is already in the maximum, so no row needs a mask.
//
// The metadata stores leave with the non-temporal hint (like the key loads):
// interleaved with the key stream, cached stores of the 520 bytes per block
// slowed the build by a fifth, and longer runs per dimension (256 blocks per
// workgroup instead of 64) recovered the rest.
//
// The build and the incremental append launch the same kernel (only the block
// range differs), so an append is bitwise equal to a rebuild. Rows may hold
// different numbers of tokens and their blocks may live in a page pool; the
// metadata stays indexed by logical block either way.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

// 8 waves (each with one block's 16 KiB of key rows in flight) rather than 16:
// past ~128 KiB in flight per CU the memory system only lengthens its queues
// (5.30 vs 5.36 ms at the headline, same process; 4 waves: 6.22 ms).
constexpr int kMetaWaves = 8;
constexpr int kMetaBlocksPerGroup = 256;

typedef float f32x4_st __attribute__((ext_vector_type(4)));

// Row 0's value of x in every row of the wave: the odd rows take the even rows'
// values (16-lane swap), then the upper half of the wave takes the lower half's
// (32-lane swap).
__device__ __forceinline__ float bcast_row0(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    return __uint_as_float(b[0]);
}

// Statistics of the block at Kb (its first token row) holding n >= 1 tokens,
// computed by the calling wave. cen: the lane's EPL centroid dimensions
// (identical in all four rows); var and maxnorm are wave-uniform. With DEV the
// wave also returns maxdev2, the largest squared distance of a key from the
// centroid, from a second pass over the rows still held in registers.
template <typename KV, int D, bool DEV>
__device__ __forceinline__ void block_stats(const KV *__restrict__ Kb, int n,
                                            float (&cen)[D / 16], float &var, float &maxnorm,
                                            float &maxdev2) {
    constexpr int EPL = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;

    RowLoad<KV, EPL> ld[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 4 * i + row < n ? 4 * i + row : 0;  // past the end: token 0 again
        ld[i].load(Kb + (size_t)t * D + col * EPL);
    }

    float k0[EPL];  // token 0: row 0 of the first load
    ld[0].widen(k0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) k0[e] = bcast_row0(k0[e]);
    float s[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = 0.f;
    float q = 0.f, nmax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x[EPL];
        ld[i].widen(x);
        float dd2 = 0.f, nrm2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float dv = x[e] - k0[e];
            s[e] += dv;
            dd2 = fmaf(dv, dv, dd2);
            nrm2 = fmaf(x[e], x[e], nrm2);
        }
        q += dd2;
        nmax = fmaxf(nmax, row_sum16(nrm2));  // squared norm of this row's token
    }
    const float fn = (float)n;
    float m2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float me = xrow_sum(s[e]) / fn;  // mean of k - k0, this lane's dimensions
        cen[e] = k0[e] + me;
        m2 = fmaf(me, me, m2);
    }
    q = xrow_sum(row_sum16(q));
    m2 = row_sum16(m2);
    var = fmaxf(q - fn * m2, 0.f) / (fn * (float)D);
    maxnorm = sqrtf(xrow_max(nmax));
    if (DEV) {
        // rows past the end repeat token 0, whose distance is already among them
        float dmax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x[EPL];
            ld[i].widen(x);
            float dist2 = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float dv = x[e] - cen[e];
                dist2 = fmaf(dv, dv, dist2);
            }
            dmax = fmaxf(dmax, row_sum16(dist2));
        }
        maxdev2 = xrow_max(dmax);
    }
}

// One workgroup per (key/value unit, group of 256 blocks). Build (n_new = 0):
// blocks [blk_begin, blk_end) clipped to the row's blocks. Append (n_new > 0):
// the blocks touched by tokens [T_b, T_b + n_new) of row b, counted from the
// block holding token T_b. A block whose page id is out of range gets zero
// metadata.
template <typename KV, int D, bool DEV>
__global__ __launch_bounds__(kMetaWaves *kWave) void block_meta_kernel(
    const KV *__restrict__ K, float *__restrict__ centroid, float *__restrict__ var,
    float *__restrict__ maxnorm, float *__restrict__ maxdev2, KVLayout lay, int nblk_cap,
    int blk_begin, int blk_end, int n_new, int groups_per_unit) {
    constexpr int EPL = D / 16;
    __shared__ float tile_c[D][kMetaBlocksPerGroup + 1];  // +1: no bank conflicts
    __shared__ float tile_v[kMetaBlocksPerGroup];
    __shared__ float tile_m[kMetaBlocksPerGroup];
    __shared__ float tile_d[DEV ? kMetaBlocksPerGroup : 1];

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
        float v = 0.f, m = 0.f, dv2 = 0.f;
        const long long off = lay.block_offset(b, k, blk);
        if (off >= 0) {
            block_stats<KV, D, DEV>(K + off, min(len - blk * kBlockTokens, kBlockTokens), cen, v,
                                    m, dv2);
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
            if (DEV) tile_d[j] = dv2;
        }
    }
    __syncthreads();

    // four consecutive blocks of one dimension per thread: 16-byte stores when the
    // group starts on a multiple of 4 blocks (every build; the centroid rows are
    // 16-byte aligned since nblk_cap is a multiple of 4), else one float per store
    // (an append, which starts at the block holding its first new token)
    float *cu = centroid + (size_t)u * D * nblk_cap;
    constexpr int kQuads = kMetaBlocksPerGroup / 4;
    const bool vec = (first & 3) == 0;
    for (int i = threadIdx.x; i < D * kQuads; i += kMetaWaves * kWave) {
        const int dim = i / kQuads;
        const int j = (i - dim * kQuads) * 4;
        float *dst = cu + (size_t)dim * nblk_cap + first + j;
        if (vec && j + 4 <= count) {
            const f32x4_st v = {tile_c[dim][j], tile_c[dim][j + 1], tile_c[dim][j + 2],
                                tile_c[dim][j + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_st *>(dst));
        } else {
            for (int e = 0; j + e < count; ++e) __builtin_nontemporal_store(tile_c[dim][j + e], dst + e);
        }
    }
    for (int j = threadIdx.x; j < count; j += kMetaWaves * kWave) {
        __builtin_nontemporal_store(tile_v[j], var + (size_t)u * nblk_cap + first + j);
        __builtin_nontemporal_store(tile_m[j], maxnorm + (size_t)u * nblk_cap + first + j);
        if (DEV) __builtin_nontemporal_store(tile_d[j], maxdev2 + (size_t)u * nblk_cap + first + j);
    }
}

template <typename KV, int D>
hipError_t launch_meta_t(const Geometry &g, const void *K, float *c, float *v, float *m,
                         float *dev2, int blk_begin, int blk_end, int n_new, hipStream_t st) {
    // blocks per row: the range, or at most ceil(n_new / 64) + 1 for an append
    const int span = n_new > 0 ? (n_new + kBlockTokens - 1) / kBlockTokens + 1 : blk_end - blk_begin;
    const int groups = (span + kMetaBlocksPerGroup - 1) / kMetaBlocksPerGroup;
    const dim3 grid((unsigned)((long long)g.kv_units * groups));
    if (dev2 != nullptr) {
        hipLaunchKernelGGL((block_meta_kernel<KV, D, true>), grid, dim3(kMetaWaves * kWave), 0, st,
                           static_cast<const KV *>(K), c, v, m, dev2, g.lay, g.nblk_cap, blk_begin,
                           blk_end, n_new, groups);
    } else {
        hipLaunchKernelGGL((block_meta_kernel<KV, D, false>), grid, dim3(kMetaWaves * kWave), 0, st,
                           static_cast<const KV *>(K), c, v, m, dev2, g.lay, g.nblk_cap, blk_begin,
                           blk_end, n_new, groups);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_meta(const Geometry &g, const void *K, float *centroid, float *var,
                             float *maxnorm, float *maxdev2, int blk_begin, int blk_end,
                             int n_new, hipStream_t st) {
    if (g.kv_units == 0 || (n_new <= 0 && blk_end <= blk_begin)) return hipSuccess;
    if (g.bf16) {
        return g.d == 128 ? launch_meta_t<uint16_t, 128>(g, K, centroid, var, maxnorm, maxdev2, blk_begin, blk_end, n_new, st)
                          : launch_meta_t<uint16_t, 64>(g, K, centroid, var, maxnorm, maxdev2, blk_begin, blk_end, n_new, st);
    }
    return g.d == 128 ? launch_meta_t<float, 128>(g, K, centroid, var, maxnorm, maxdev2, blk_begin, blk_end, n_new, st)
                      : launch_meta_t<float, 64>(g, K, centroid, var, maxnorm, maxdev2, blk_begin, blk_end, n_new, st);
}

}  // namespace eta
