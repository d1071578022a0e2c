// eta_predict.hip -- per-head threshold predictor, a batched GEMV.
//
// evolve.pub review of arXiv:2609.20888, "Methodology Assessment", Eq. 1: the
// threshold of every head is a linear function (weights W, bias b) of the
// concatenation of all heads' post-RoPE queries of the same batch row. With
// no predictor (abstract: offline calibration freezes per-head constants) the
// threshold is the bias alone.
//
// One workgroup per (batch row, group of 16 heads): each thread walks a
// strided slice of the H*d concatenated query, reading contiguous 16-head
// slices of W rows (W stays L2-resident across batch rows), then the partial
// sums are reduced in a fixed order (deterministic).
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

constexpr int kPredThreads = 256;
constexpr int kPredHeads = 16;

__global__ __launch_bounds__(kPredThreads) void predict_tau_kernel(
    int H, int HD, const float *__restrict__ q, const float *__restrict__ W,
    const float *__restrict__ bias, float *__restrict__ tau, int vec) {
    __shared__ float part[kPredThreads / kWave][kPredHeads];
    const int b = blockIdx.x;
    const int h0 = blockIdx.y * kPredHeads;
    const int nh = min(kPredHeads, H - h0);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    if (W == nullptr) {
        if ((int)threadIdx.x < nh) tau[(size_t)b * H + h0 + threadIdx.x] = bias[h0 + threadIdx.x];
        return;
    }

    float acc[kPredHeads];
#pragma unroll
    for (int j = 0; j < kPredHeads; ++j) acc[j] = 0.f;
    const float *qb = q + (size_t)b * HD;
    if (vec && nh == kPredHeads) {
        // 16 whole heads and 16-byte aligned rows: four float4 loads per row slice
#pragma unroll 4
        for (int k = threadIdx.x; k < HD; k += kPredThreads) {
            const float qv = qb[k];
            const float4 *wr = reinterpret_cast<const float4 *>(W + (size_t)k * H + h0);
#pragma unroll
            for (int j4 = 0; j4 < kPredHeads / 4; ++j4) {
                const float4 w4 = wr[j4];
                acc[4 * j4 + 0] += qv * w4.x;
                acc[4 * j4 + 1] += qv * w4.y;
                acc[4 * j4 + 2] += qv * w4.z;
                acc[4 * j4 + 3] += qv * w4.w;
            }
        }
    } else {
        for (int k = threadIdx.x; k < HD; k += kPredThreads) {
            const float qv = qb[k];
            const float *wr = W + (size_t)k * H + h0;
#pragma unroll
            for (int j = 0; j < kPredHeads; ++j)
                if (j < nh) acc[j] += qv * wr[j];
        }
    }
#pragma unroll
    for (int j = 0; j < kPredHeads; ++j) {
        const float r = xrow_sum(row_sum16(acc[j]));
        if (lane == 0) part[wave][j] = r;
    }
    __syncthreads();
    if ((int)threadIdx.x < nh) {
        float t = bias[h0 + threadIdx.x];
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kPredThreads / kWave; ++w) s += part[w][threadIdx.x];
        tau[(size_t)b * H + h0 + threadIdx.x] = t + s;
    }
}

}  // namespace

hipError_t launch_predict_tau(int B, int H, int d, const float *q, const float *W,
                              const float *bias, float *tau, hipStream_t st) {
    const dim3 grid((unsigned)B, (unsigned)((H + kPredHeads - 1) / kPredHeads));
    const int vec = (H % 4 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0);
    hipLaunchKernelGGL(predict_tau_kernel, grid, dim3(kPredThreads), 0, st, H, H * d, q, W,
                       bias, tau, vec);
    return hipGetLastError();
}

}  // namespace eta
