// eta_launch.hpp -- host-side launchers behind the C ABI (internal).
// Every launcher assumes arguments already validated by eta_api.hip and only
// enqueues work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "eta_device.hpp"

namespace eta {

struct Geometry {
    int units;     // query units B * H
    int kv_units;  // key/value units B * H_kv (= units for multi-head attention)
    int G;         // query heads per key/value head (1, 2, 4 or 8)
    int d;         // 64 or 128
    int T;         // tokens present
    int T_cap;     // token capacity of K / V
    int nblk;      // ceil(T / 64)
    int nblk_cap;  // metadata / list capacity per unit (multiple of 4)
    bool bf16;     // K / V element type
    KVLayout lay;  // dense or paged rows, optional per-row lengths
};

// Metadata of blocks [blk_begin, blk_end) of every row (clipped to the row's
// length); with n_new > 0, of the blocks each row's next n_new tokens touch
// (the layout's lengths are then the lengths before those tokens). maxdev2 may be
// null (not computed).
hipError_t launch_block_meta(const Geometry &g, const void *K, float *centroid, float *var,
                             float *maxnorm, float *maxdev2, int blk_begin, int blk_end,
                             int n_new, hipStream_t st);

hipError_t launch_predict_tau(int B, int H, int d, const float *q, const float *W,
                              const float *bias, float *tau, hipStream_t st);

// Screen; with `predict` the threshold of every unit is first evaluated from
// q, W (nullable) and bias and stored to tau, otherwise tau is read.
// With grouped heads and uni_idx non-null the union per key/value unit is
// written in the same launch.
hipError_t launch_screen(const Geometry &g, int H, const float *q, float *tau, const float *W,
                         const float *bias, bool predict, const float *centroid,
                         const float *var, const float *maxnorm, float z, bool geo_only,
                         int32_t *adm_idx, int32_t *adm_cnt, float *bound_out, hipStream_t st,
                         int32_t *uni_idx = nullptr, int32_t *uni_cnt = nullptr);

// Union, per key/value unit, of the admitted lists of its G query heads.
hipError_t launch_union(const Geometry &g, const int32_t *adm_idx, const int32_t *adm_cnt,
                        int32_t *uni_idx, int32_t *uni_cnt, hipStream_t st);

// Workspace layout of the split-KV attention for `units` units with at most
// `max_chunks` work items each.
struct AttnWorkspace {
    size_t off_hdr, off_items, off_m, off_l, off_o, bytes;
};
AttnWorkspace attn_workspace_layout(int units, int max_chunks, int d);

// Split-KV partials (writes out/lse directly for units with a single item).
hipError_t launch_attn_partial(const Geometry &g, const float *q, const void *K, const void *V,
                               const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                               float gate_beta, bool gate_hard, int split_blocks, int max_chunks,
                               float *out, float *lse, void *ws, hipStream_t st);

// Log-sum-exp merge of the partials of units with more than one item.
hipError_t launch_attn_combine(const Geometry &g, const int32_t *adm_cnt, int split_blocks,
                               int max_chunks, float *out, float *lse, void *ws, hipStream_t st);

// Prefill (training-time forward): Q [B][H][T_q][d], K, V [B][Hkv][T_k][d] bf16.
struct PrefillGeometry {
    int B, H, Hkv, d, T_q, T_k;
};

// Eq. 1 per query token: tau [B][H][T_q] from the bf16 queries.
hipError_t launch_prefill_tau(const PrefillGeometry &g, const void *Q, const float *W,
                              const float *bias, float *tau, hipStream_t st);

// Dense causal gated attention (out [B][H][T_q][d], lse and gate_sum [B][H][T_q]).
hipError_t launch_prefill_attn(const PrefillGeometry &g, const void *Q, const void *K,
                               const void *V, const float *tau, float gate_beta, bool gate_hard,
                               float *out, float *lse, float *gate_sum, hipStream_t st);

}  // namespace eta
