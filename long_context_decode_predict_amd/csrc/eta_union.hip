// eta_union.hip -- union of the admitted lists of the query heads that share
// one key/value head (grouped heads).
//
// The pages measure the fraction of KV blocks fetched when the selections of
// several heads are fetched together (evolve.pub review, Q&A on speed and
// "Summary"), and the gate's floor is what lets tokens that only ride along with
// a selected block do no harm (arXiv:2609.20888 abstract). With G query heads per key/value head,
// a block is loaded once for the key/value head when any of its G query heads
// admits it, and each query head attends over that union with its own gate.
//
// One workgroup per key/value unit. The block range is walked 8192 blocks at a
// time: the G sorted lists mark a 1 KiB LDS bitmap (OR is order-free, so the
// result is deterministic), each thread then owns one 32-bit word and the
// words' popcounts are scanned across the workgroup, so the union is written
// ascending with consecutive threads on consecutive runs of ids.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kUnionThreads = 256;
constexpr int kUnionRange = kUnionThreads * 32;  // blocks per bitmap pass
constexpr int kMaxGroup = 8;

__global__ __launch_bounds__(kUnionThreads) void union_kernel(int G, int nblk, int nblk_cap,
                                                              const int32_t *__restrict__ adm_idx,
                                                              const int32_t *__restrict__ adm_cnt,
                                                              int32_t *__restrict__ uni_idx,
                                                              int32_t *__restrict__ uni_cnt) {
    __shared__ uint32_t bits[kUnionThreads];
    __shared__ int cursor[kMaxGroup];
    __shared__ int seen[kMaxGroup];
    __shared__ int wave_sum[kUnionThreads / kWave];
    const int u = blockIdx.x;  // key/value unit; its query heads are u*G + j
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (tid < G) cursor[tid] = 0;
    int out_base = 0;
    int32_t *out = uni_idx + (size_t)u * nblk_cap;

    for (int r0 = 0; r0 < nblk; r0 += kUnionRange) {
        bits[tid] = 0u;
        if (tid < G) seen[tid] = 0;
        __syncthreads();
        for (int j = 0; j < G; ++j) {
            const int h = u * G + j;
            const int32_t *lst = adm_idx + (size_t)h * nblk_cap;
            const int cnt = min(max(adm_cnt[h], 0), nblk_cap);  // reads stay in the list row
            int mine = 0;
            for (int i = cursor[j] + tid; i < cnt; i += kUnionThreads) {
                const int b = lst[i];
                if (b >= r0 + kUnionRange) break;  // sorted: later entries are past this pass
                if (b >= r0 && b < nblk)  // an id outside [0, ceil(T / 64)) is dropped
                    atomicOr(&bits[(b - r0) >> 5], 1u << ((b - r0) & 31));
                ++mine;
            }
            if (mine) atomicAdd(&seen[j], mine);
        }
        __syncthreads();
        if (tid < G) cursor[tid] += seen[tid];

        const uint32_t word = bits[tid];
        const int n = __popc(word);
        int x = n;  // inclusive scan over the workgroup's words
#pragma unroll
        for (int k = 1; k < kWave; k <<= 1) {
            const int y = __shfl_up(x, k, kWave);
            if (lane >= k) x += y;
        }
        if (lane == kWave - 1) wave_sum[wave] = x;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kUnionThreads / kWave; ++w) {
            before += (w < wave) ? wave_sum[w] : 0;
            total += wave_sum[w];
        }
        int pos = out_base + before + x - n;
        uint32_t rest = word;
        while (rest) {
            const int bit = __ffs(rest) - 1;
            out[pos++] = r0 + tid * 32 + bit;
            rest &= rest - 1u;
        }
        out_base += total;
        __syncthreads();  // bits, seen and wave_sum are reused by the next pass
    }
    if (tid == 0) uni_cnt[u] = out_base;
}

}  // namespace

hipError_t launch_union(const Geometry &g, const int32_t *adm_idx, const int32_t *adm_cnt,
                        int32_t *uni_idx, int32_t *uni_cnt, hipStream_t st) {
    if (g.kv_units == 0) return hipSuccess;
    hipLaunchKernelGGL(union_kernel, dim3((unsigned)g.kv_units), dim3(kUnionThreads), 0, st, g.G,
                       g.nblk, g.nblk_cap, adm_idx, adm_cnt, uni_idx, uni_cnt);
    return hipGetLastError();
}

}  // namespace eta
