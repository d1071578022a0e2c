// eta_attn.hip -- block-sparse split-KV decode attention with the ETA gate.
//
// arXiv:2609.20888: only the admitted blocks are loaded (evolve.pub review,
// Q&A "What is ETA?"); each logit S = s*q.k is multiplied by the gate
// sigmoid(beta*(S - tau)) (review "Methodology Assessment", Eq. 2 and Eq. 3),
// so a sub-threshold logit tends to 0 (weight e^0 = 1) instead of -inf, which
// absorbs the tokens that coarse block selection lets in (abstract).
//
// Work decomposition. A unit's ascending admitted list is cut into work items
// of `split` blocks. A plan kernel (one workgroup per 64 units) scans the
// per-unit item counts into a compacted item list (and settles empty units
// directly); a persistent grid of one workgroup per CU (two for the smallest
// tiles) then takes items from the list through a device-scope ticket counter,
// so no workgroup is launched for an absent item and the load balances itself
// whatever the per-unit densities. A workgroup of
// four waves processes one item at a time; wave w walks the item's blocks
// w, w+4, ... in tiles of TS tokens:
//   - row r of the wave owns one token and lane c of the row the EPL = d/16
//     elements [EPL*c, EPL*c + EPL) of it, so one 16-byte load per lane covers
//     four whole token rows; every load is a uniform block base plus a fixed
//     per-lane offset plus an immediate, so no per-load address arithmetic;
//   - software pipeline per wave: the V tile of tile t and the K tile of tile
//     t+1 are in flight while tile t's logits and weighted values are formed,
//     and the scalar reads that locate the tiles run ahead of them (list
//     entries two blocks ahead, page ids one block ahead);
//   - dot products reduce over the 16 lanes of a DPP row; the gated logits of
//     a whole tile are formed first, so the running (max, sum, weighted V)
//     state is rescaled once per tile, not per token.
// With grouped heads (G > 1) q.K and P.V are dense products over the G heads:
// with bf16 K/V they run on the matrix cores (attn_item_mfma); with fp32 K/V
// the per-row dot products are reduce-scattered (attn_item_dist) so each lane
// ends with whole (head, row) pairs and the gate and softmax weight are
// evaluated once per pair, not on all 16 lanes.
// The waves' states merge in LDS. A one-item unit writes out/lse directly;
// otherwise each item stores a (max, sum, weighted V) partial and the combine
// kernel merges a unit's partials in item order with a log-sum-exp
// (deterministic; the kernel boundary orders the two, so no fences or atomics
// are needed).
//
// The K/V capacity is a whole number of blocks (dense layout) and a page holds
// a whole block (paged layout), so the rows of a partial last block past the
// row's length are inside the allocation: they are loaded unclamped and masked
// (their logits become -inf and their values are zeroed before use). For a
// block whose page id is out of range, or a list entry that is not a block of
// the row (negative, or at or past ceil(T_b / 64)), no byte outside the K/V
// buffers is touched: the tiles load from the start of K/V instead and are
// masked whole, so the entry contributes nothing (a unit left with no token
// gets out = 0, lse = -inf, as an empty list does). Counts are clamped to
// [0, T_cap / 64], the most blocks a list of distinct ids can hold: no list read
// leaves the unit's row of the list, and no unit has more work items than the
// workspace is sized for (ceil(T_cap / 64 / split) per unit).
#include "eta_device.hpp"
#include "eta_launch.hpp"

#include <type_traits>

namespace eta {
namespace {

constexpr int kAttnWaves = 4;
// Persistent workgroups per CU: the memory system saturates at about 64-128 KiB
// in flight per CU, and more only lengthens its queues (a read kernel with 16
// waves x 16 KiB per CU streams ~7 % slower than 8 x 16 KiB). One workgroup of
// four waves keeps up to 4 x 32 KiB of K/V tiles in flight on the multi-head
// path, except with bf16 rows of 64, whose tile pair is 16 KiB: two workgroups
// there (B = 64, 128K: 1.96 vs 2.36 ms with one). The grouped-head path runs
// fastest with one at d = 64 and 128 alike (G = 8: 0.652 vs 0.671 ms at d = 64).
constexpr int kWorkersPerCU = 1;
constexpr int kWorkersPerCUSmallTiles = 2;

struct AttnArgs {
    int units, G, nblk, nblk_cap, split, ws_chunks;  // units: key/value units
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
    int *ws_hdr;     // [0] = number of items, [1] = ticket counter
    int2 *ws_items;  // compacted (unit, item index) list
    KVLayout lay;    // dense or paged rows, per-row lengths
};

// Admitted blocks of key/value unit u as every kernel here counts them: clamped
// to the blocks of the capacity (T_cap / 64 <= nblk_cap), so no list read leaves
// the unit's row of the list and no item index reaches past the unit's
// workspace slots.
__device__ __forceinline__ int unit_count(const AttnArgs &a, int u) {
    const int c = ld_const(a.cnt + u);
    const int cap = a.lay.max_pages;
    return c < 0 ? 0 : (c > cap ? cap : c);
}

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

template <int D, int G, bool KT = false>
struct AttnShared {
    float m[kAttnWaves][G];
    float l[kAttnWaves][G];
    float o[kAttnWaves][G][D];
    int ticket;
};
// Matrix-core path: each wave's two K tiles (the one being multiplied and the next);
// the item's merge reuses their space once every wave has left its tile loop.
template <int D, int G>
struct AttnShared<D, G, true> {
    float m[kAttnWaves][G];
    float l[kAttnWaves][G];
    union {
        float o[kAttnWaves][G][D];
        uint4 kt[kAttnWaves][2][4 * D];
    };
    int ticket;
};

// One work item (key/value unit u, item `chunk`) by the whole workgroup, for the
// G query heads u*G + j that share the unit's keys and values: every loaded
// tile of K and V serves all G heads, each with its own query, threshold and
// running softmax state. Ends with the workgroup merge (one barrier); the
// caller barriers before LDS is reused.
template <typename KV, int D, int TS, bool HARD, int G>
__device__ __forceinline__ void attn_item(const AttnArgs &a, int u, int chunk,
                                          AttnShared<D, G> &sm) {
    constexpr int EPL = D / 16;
    constexpr int L = TS / 4;                 // row loads per lane per tile
    constexpr int TPB = kBlockTokens / TS;    // tiles per block
    constexpr int ROW = D;                    // elements per token row
    const int c = unit_count(a, u);
    const int nchunks = (c + a.split - 1) / a.split;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;

    float qr[G][EPL], t[G], nbt[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const size_t uq = (size_t)u * G + j;  // query unit
#pragma unroll
        for (int e = 0; e < EPL; ++e) qr[j][e] = a.q[uq * D + col * EPL + e] * a.s;
        t[j] = ld_const(a.tau + uq);
        nbt[j] = -a.nbl2e * t[j];  // gate exponent = nbl2e * S + nbt
    }

    const KV *Kp = static_cast<const KV *>(a.K);
    const KV *Vp = static_cast<const KV *>(a.V);
    const int rb = u / a.lay.H_kv;          // batch row of the unit
    const int kh = u - rb * a.lay.H_kv;     // its key/value head
    const int Tb = a.lay.row_len(rb);       // tokens present in the row
    const int nblk_row = (Tb + kBlockTokens - 1) / kBlockTokens;  // ids past it are skipped
    const int lane_off = row * ROW + col * EPL;  // element offset inside a 4-row group
    const int32_t *iu = a.idx + (size_t)u * a.nblk_cap;

    const int j0 = chunk * a.split;
    const int j1 = min(c, j0 + a.split);
    // this wave's blocks: j0 + wave + k*kAttnWaves < j1
    const int nb = (j1 - j0 - wave + kAttnWaves - 1) / kAttnWaves;
    const int ntiles = nb > 0 ? nb * TPB : 0;

    float m_run[G], l_run[G], o[G][EPL];  // l_run per row: this row's tokens
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
    }

    // The scalar reads that locate a tile run ahead of its K loads: list entries
    // two blocks ahead, page ids one block ahead (page_of issues the read, base_of
    // first uses its value a tile later), so no scalar round trip stands between a
    // tile's logits and the next tile's K loads. blk_id: the wave's k-th block (-1
    // past its last); page_of: page id of a block (the block id itself when dense,
    // -1 outside the row's blocks); base_of: element offset of a block, -1 for a
    // bad page or an id outside the row; tile_of: offset of a tile and the number
    // of its rows below the row's length (TS or more for every tile but a partial
    // last block's; 0 when the block is bad).
    auto blk_id = [&](int k) { return k < nb ? ld_const(iu + j0 + wave + k * kAttnWaves) : -1; };
    auto page_of = [&](int blk) -> int {
        return (unsigned)blk < (unsigned)nblk_row ? a.lay.page_of(rb, blk) : -1;
    };
    auto base_of = [&](int blk, int pg) -> long long {
        return (unsigned)blk < (unsigned)nblk_row ? a.lay.page_offset(rb, kh, pg) : -1;
    };
    auto tile_of = [&](int blk, long long bo, int part, size_t &off, int &valid) {
        const int sub = part * TS;
        off = (bo < 0 ? 0 : (size_t)bo) + (size_t)sub * ROW;
        valid = bo < 0 ? 0 : min(Tb - blk * kBlockTokens, kBlockTokens) - sub;
    };

    RowLoad<KV, EPL> kb[L], vb[L];
    size_t next_off = 0;
    int next_valid = 0;
    int blk_c = -1, blk_n = -1, blk_nn = -1;  // block of the last K tile, the next two
    int pg_n = -1;
    long long bo_c = -1;
    if (ntiles > 0) {
        blk_c = blk_id(0);
        bo_c = base_of(blk_c, page_of(blk_c));
        tile_of(blk_c, bo_c, 0, next_off, next_valid);
        const KV *p = Kp + next_off + lane_off;
#pragma unroll
        for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
        blk_n = blk_id(1);
    }
    for (int tt = 0; tt < ntiles; ++tt) {
        const size_t base = next_off;
        const int valid = next_valid;
        {
            const KV *p = Vp + base + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) vb[i].load(p + i * 4 * ROW);
        }
        const bool cross = (tt + 1) % TPB == 0;  // the next K tile starts a new block
        if (cross && tt + 1 < ntiles) {
            pg_n = page_of(blk_n);
            blk_nn = blk_id((tt + 1) / TPB + 1);
        }
        // gated logits of the tile, per head
        float sg[G][L];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[EPL];
            kb[i].widen(x);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot += qr[j][e] * x[e];
                const float S = row_sum16(dot);
                float gv;
                if (HARD) {
                    gv = S >= t[j] ? S : 0.f;
                } else {
                    gv = S * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(a.nbl2e, S, nbt[j])));
                }
                sg[j][i] = gv;
            }
        }
        if (valid < TS) {  // partial last block: rows past the row's length take no weight
#pragma unroll
            for (int i = 0; i < L; ++i)
                if (4 * i + row >= valid) {
#pragma unroll
                    for (int j = 0; j < G; ++j) sg[j][i] = -INFINITY;
                }
        }
        // the K registers are free: start the next tile's K loads
        if (tt + 1 < ntiles) {
            if (cross) {
                bo_c = base_of(blk_n, pg_n);
                blk_c = blk_n;
                blk_n = blk_nn;
            }
            tile_of(blk_c, bo_c, (tt + 1) % TPB, next_off, next_valid);
            const KV *p = Kp + next_off + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
        }
        float m_new[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float bmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < L; ++i) bmax = fmaxf(bmax, sg[j][i]);
            bmax = xrow_max(bmax);
            const float mx = fmaxf(m_run[j], bmax);
            // reference for the weights; a fully masked tile before any token
            // leaves the max at -inf, and 0 then keeps the weights 0, not NaN
            m_new[j] = mx == -INFINITY ? 0.f : mx;
            const float corr = fast_exp(m_run[j] - m_new[j]);
            l_run[j] *= corr;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] *= corr;
            m_run[j] = mx;
        }
        if (valid < TS) {
#pragma unroll
            for (int i = 0; i < L; ++i)
                if (4 * i + row >= valid) zero_row<KV, EPL>(vb[i]);
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[EPL];
            vb[i].widen(x);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float p = fast_exp(sg[j][i] - m_new[j]);
                l_run[j] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] += p * x[e];
            }
        }
    }

    // merge the four rows of the wave (m_run is wave-uniform)
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float l_w = xrow_sum(l_run[j]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = xrow_sum(o[j][e]);
        if (lane == 0) {
            sm.m[wave][j] = m_run[j];
            sm.l[wave][j] = l_w;
        }
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm.o[wave][j][lane * EPL + e] = o[j][e];
        }
    }
    __syncthreads();

    // merge the waves of the workgroup, head by head
    for (int j = 0; j < G; ++j) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm.m[w][j]);
        const float Mr = M == -INFINITY ? 0.f : M;  // no token at all: weights 0, Lsum 0
        float Lsum = 0.f;
        float wgt[kAttnWaves];
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            wgt[w] = fast_exp(sm.m[w][j] - Mr);  // a wave without tokens has m = -inf: weight 0
            Lsum += sm.l[w][j] * wgt[w];
        }
        const size_t uq = (size_t)u * G + j;
        if (tid < D) {
            float O = 0.f;
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) O += sm.o[w][j][tid] * wgt[w];
            if (nchunks == 1) {
                a.out[uq * D + tid] = Lsum > 0.f ? O / Lsum : 0.f;
            } else {
                const size_t slot = ((size_t)u * a.ws_chunks + chunk) * G + j;
                a.ws_o[slot * D + tid] = O;
            }
        }
        if (tid == 0) {
            if (nchunks == 1) {
                if (a.lse) a.lse[uq] = Lsum > 0.f ? M + __logf(Lsum) : -INFINITY;
            } else {
                const size_t slot = ((size_t)u * a.ws_chunks + chunk) * G + j;
                a.ws_m[slot] = M;
                a.ws_l[slot] = Lsum;
            }
        }
    }
}

// ---- grouped heads: one gate per (token, head) instead of one per lane ----
//
// With G query heads per tile every 16-lane row holds, per lane, partial dot
// products of P = G*L (head, row-load) pairs (head-major: k = j*L + i). A
// reduce-scatter over the row (four halving steps on the same DPP patterns as
// row_sum16) leaves lane c with the full sums of the m = P/16 pairs
// k = c*m .. c*m + m - 1, all of one head j = c*m / L. The gate, the tile
// maximum and the softmax weight are then computed once per pair rather than on
// all 16 lanes of the row; the weights come back to the row with one DPP row
// broadcast per pair for the P.V products.

template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}
// Broadcast lane n (compile-time after unrolling) of each row to the row.
__device__ __forceinline__ float row_bcast_n(float x, int n) {
    switch (n) {
        case 0: return row_bcast<0>(x);
        case 1: return row_bcast<1>(x);
        case 2: return row_bcast<2>(x);
        case 3: return row_bcast<3>(x);
        case 4: return row_bcast<4>(x);
        case 5: return row_bcast<5>(x);
        case 6: return row_bcast<6>(x);
        case 7: return row_bcast<7>(x);
        case 8: return row_bcast<8>(x);
        case 9: return row_bcast<9>(x);
        case 10: return row_bcast<10>(x);
        case 11: return row_bcast<11>(x);
        case 12: return row_bcast<12>(x);
        case 13: return row_bcast<13>(x);
        case 14: return row_bcast<14>(x);
        default: return row_bcast<15>(x);
    }
}

// One halving step of the reduce-scatter: lanes whose `hi` bit is clear keep
// the first half of v (plus the partner's first half), the others the second.
template <int CTRL, int N>
__device__ __forceinline__ void rs_step(float (&v)[64], bool hi) {
#pragma unroll
    for (int t = 0; t < N / 2; ++t) {
        const float lo_sum = v[t] + dpp_for_add<CTRL>(v[t]);
        const float hi_sum = v[N / 2 + t] + dpp_for_add<CTRL>(v[N / 2 + t]);
        v[t] = hi ? hi_sum : lo_sum;
    }
}

// Maximum / sum over the aligned group of GS lanes of a row (GS = 16/G).
template <int GS>
__device__ __forceinline__ float group_max(float x) {
    if (GS >= 2) x = fmaxf(x, dpp_mov<kQuadXor1>(x));
    if (GS >= 4) x = fmaxf(x, dpp_mov<kQuadXor2>(x));
    if (GS >= 8) x = fmaxf(x, dpp_mov<kRowHalfMirror>(x));
    if (GS >= 16) x = fmaxf(x, dpp_mov<kRowMirror>(x));
    return x;
}
template <int GS>
__device__ __forceinline__ float group_sum(float x) {
    if (GS >= 2) x += dpp_for_add<kQuadXor1>(x);
    if (GS >= 4) x += dpp_for_add<kQuadXor2>(x);
    if (GS >= 8) x += dpp_for_add<kRowHalfMirror>(x);
    if (GS >= 16) x += dpp_for_add<kRowMirror>(x);
    return x;
}

// Workgroup merge of one item for G heads: every wave has left its (max, sum,
// weighted V) state per head in sm; the states are combined in wave order and
// either normalised into out/lse (a one-item unit) or stored as the item's
// partial for the combine kernel.
template <int D, int G, typename SM>
__device__ __forceinline__ void merge_heads(const AttnArgs &a, int u, int chunk, int nchunks,
                                            SM &sm) {
    const int tid = threadIdx.x;
    for (int j = 0; j < G; ++j) {
        float M_ = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M_ = fmaxf(M_, sm.m[w][j]);
        const float Mr = M_ == -INFINITY ? 0.f : M_;
        float Lsum = 0.f;
        float wgt[kAttnWaves];
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            wgt[w] = fast_exp(sm.m[w][j] - Mr);
            Lsum += sm.l[w][j] * wgt[w];
        }
        const size_t uq = (size_t)u * G + j;
        if (tid < D) {
            float O = 0.f;
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) O += sm.o[w][j][tid] * wgt[w];
            if (nchunks == 1) {
                a.out[uq * D + tid] = Lsum > 0.f ? O / Lsum : 0.f;
            } else {
                const size_t slot = ((size_t)u * a.ws_chunks + chunk) * G + j;
                a.ws_o[slot * D + tid] = O;
            }
        }
        if (tid == 0) {
            if (nchunks == 1) {
                if (a.lse) a.lse[uq] = Lsum > 0.f ? M_ + __logf(Lsum) : -INFINITY;
            } else {
                const size_t slot = ((size_t)u * a.ws_chunks + chunk) * G + j;
                a.ws_m[slot] = M_;
                a.ws_l[slot] = Lsum;
            }
        }
    }
}

template <typename KV, int D, int TS, bool HARD, int G>
__device__ __forceinline__ void attn_item_dist(const AttnArgs &a, int u, int chunk,
                                               AttnShared<D, G> &sm) {
    constexpr int EPL = D / 16;
    constexpr int L = TS / 4;               // row loads per lane per tile
    constexpr int TPB = kBlockTokens / TS;  // tiles per block
    constexpr int ROW = D;
    constexpr int P = G * L;                // (head, row-load) pairs per row
    constexpr int M = P / 16;               // pairs owned per lane
    constexpr int GS = 16 / G;              // lanes of a row that own one head
    static_assert(P >= 16 && P <= 64 && P % 16 == 0 && L % M == 0, "pair layout");
    const int c = unit_count(a, u);
    const int nchunks = (c + a.split - 1) / a.split;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & (kWave - 1);
    const int row = lane >> 4;
    const int col = lane & 15;
    const int my_j = col / GS;          // the head whose pairs this lane owns
    const int my_i0 = (col * M) % L;    // its first row-load

    float qr[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const size_t uq = (size_t)u * G + j;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qr[j][e] = a.q[uq * D + col * EPL + e] * a.s;
    }
    const float t_own = a.tau[(size_t)u * G + my_j];
    const float nbt_own = -a.nbl2e * t_own;

    const KV *Kp = static_cast<const KV *>(a.K);
    const KV *Vp = static_cast<const KV *>(a.V);
    const int rb = u / a.lay.H_kv;
    const int kh = u - rb * a.lay.H_kv;
    const int Tb = a.lay.row_len(rb);
    const int nblk_row = (Tb + kBlockTokens - 1) / kBlockTokens;  // ids past it are skipped
    const int lane_off = row * ROW + col * EPL;
    const int32_t *iu = a.idx + (size_t)u * a.nblk_cap;

    const int j0 = chunk * a.split;
    const int j1 = min(c, j0 + a.split);
    const int nb = (j1 - j0 - wave + kAttnWaves - 1) / kAttnWaves;
    const int ntiles = nb > 0 ? nb * TPB : 0;

    float m_run = -INFINITY, l_run = 0.f;  // for head my_j: l over this lane's pairs
    float o[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;

    auto tile_at = [&](int tt, size_t &off, int &valid) {
        const int blk = ld_const(iu + j0 + wave + (tt / TPB) * kAttnWaves);
        const long long bo =
            (unsigned)blk < (unsigned)nblk_row ? a.lay.block_offset(rb, kh, blk) : -1;
        const int sub = (tt % TPB) * TS;
        off = (bo < 0 ? 0 : (size_t)bo) + (size_t)sub * ROW;
        valid = bo < 0 ? 0 : min(Tb - blk * kBlockTokens, kBlockTokens) - sub;
    };

    RowLoad<KV, EPL> kb[L], vb[L];
    size_t next_off = 0;
    int next_valid = 0;
    if (ntiles > 0) {
        tile_at(0, next_off, next_valid);
        const KV *p = Kp + next_off + lane_off;
#pragma unroll
        for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
    }
    for (int tt = 0; tt < ntiles; ++tt) {
        const size_t base = next_off;
        const int valid = next_valid;
        {
            const KV *p = Vp + base + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) vb[i].load(p + i * 4 * ROW);
        }
        // partial dots of every (head, row-load) pair, head-major
        float v[64];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[EPL];
            kb[i].widen(x);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot += qr[j][e] * x[e];
                v[j * L + i] = dot;
            }
        }
        // the K registers are free: start the next tile's K loads
        if (tt + 1 < ntiles) {
            tile_at(tt + 1, next_off, next_valid);
            const KV *p = Kp + next_off + lane_off;
#pragma unroll
            for (int i = 0; i < L; ++i) kb[i].load(p + i * 4 * ROW);
        }
        // reduce-scatter over the row: lane col ends with pairs col*M .. col*M + M - 1
        rs_step<kRowMirror, P>(v, (col >> 3) & 1);
        rs_step<kRowHalfMirror, P / 2>(v, (col >> 2) & 1);
        rs_step<kQuadXor2, P / 4>(v, (col >> 1) & 1);
        rs_step<kQuadXor1, P / 8>(v, col & 1);

        // gate of the owned pairs, rows past the row's length masked
        float gv[M];
        float bmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < M; ++t) {
            const float S = v[t];
            float g;
            if (HARD) {
                g = S >= t_own ? S : 0.f;
            } else {
                g = S * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(a.nbl2e, S, nbt_own)));
            }
            if (4 * (my_i0 + t) + row >= valid) g = -INFINITY;
            gv[t] = g;
            bmax = fmaxf(bmax, g);
        }
        bmax = xrow_max(group_max<GS>(bmax));  // over the head's lanes and the 4 rows
        const float mx = fmaxf(m_run, bmax);
        const float m_ref = mx == -INFINITY ? 0.f : mx;  // nothing visible yet: weights 0
        const float corr = fast_exp(m_run - m_ref);
        m_run = mx;
        l_run *= corr;
        float pw[M];
#pragma unroll
        for (int t = 0; t < M; ++t) {
            pw[t] = fast_exp(gv[t] - m_ref);
            l_run += pw[t];
        }
        // every lane rescales and accumulates all G heads' outputs
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float cj = row_bcast_n(corr, j * GS);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] *= cj;
        }
        if (valid < TS) {
#pragma unroll
            for (int i = 0; i < L; ++i)
                if (4 * i + row >= valid) zero_row<KV, EPL>(vb[i]);
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[EPL];
            vb[i].widen(x);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int k = j * L + i;
                const float p = row_bcast_n(pw[k % M], k / M);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] += p * x[e];
            }
        }
    }

    // merge: l over the head's lanes and the rows; outputs over the rows
    const float l_head = xrow_sum(group_sum<GS>(l_run));
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = xrow_sum(o[j][e]);
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm.o[wave][j][lane * EPL + e] = o[j][e];
        }
    }
    if (lane < 16 && col % GS == 0) {  // the first lane of each head's group, row 0
        sm.m[wave][my_j] = m_run;
        sm.l[wave][my_j] = l_head;
    }
    __syncthreads();

    merge_heads<D, G>(a, u, chunk, nchunks, sm);
}

// ---- grouped heads on the matrix cores (bf16 K/V) ----
//
// With G query heads per key/value unit, q.K over a tile is a dense
// [tokens x d] x [d x G] product and P.V a [G x tokens] x [tokens x d] one, so
// both run on the 16x16x32 bf16 MFMA (A: lane l holds row l%16, k-slots
// 8*(l/16) + [0, 8); B: column l%16, the same k-slots; D: column l%16, rows
// 4*(l/16) + [0, 4)). K and V enter as stored. The fp32 operands (scaled
// queries, softmax weights) are split into a bf16 value and a bf16 residual
// (x - hi, exact in fp32), which sit in columns [0, G) and [8, 8 + G) of the
// same B operand: one MFMA forms both partial products and a DPP rotation of
// each row by 8 lanes adds them. A query keeps a third bf16 term (the residual
// of the residual, columns [0, G) of a second operand, accumulated into the
// same logits), so a logit is exact to about 2^-26 of its terms: close to fp32
// arithmetic, which the hard gate's step at tau needs; a weight's two terms
// leave about 2^-17 of it.
//
// A wave's tile is 32 tokens, in two halves of 16. Lane (g, n) = (lane/16,
// lane%16):
//   q.K: it reads 16 bytes of token 16h + n at element 32kc + 8g (A operand of
//     half h, k-step kc) from the wave's LDS copy of the K tile (loaded whole
//     rows at a time, so HBM sees full 128-byte lines per load), holds query
//     column n at the same elements (B), and receives the logits of tokens
//     16h + 4g + i (i < 4) for column n.
//   So it owns, per column, the tokens tok(g, j) = 4g + j for j < 4 and
//     16 + 4g + j - 4 for j >= 4: exactly k-slots 8g + j of the P.V product's
//     B operand, which therefore needs no data movement.
//   P.V: one MFMA per e < EPL = d/16, A row n <-> element EPL*n + e. The lane
//     loads elements [EPL*n, EPL*n + EPL) of its eight tokens (16 lanes read a
//     whole row per load), transposes them in registers with v_perm, and
//     accumulates elements EPL*(4g + i) + e of column n.
// Columns n and n + 8 hold the same head's logits after the rotation, so both
// evaluate the same gate and weight; the value lane keeps the rounded weight,
// the residual lane the remainder.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kRowRor8 = 0x128;  // DPP row_ror:8: lane n of a row reads lane (n + 8) % 16

// Round-to-nearest-even bf16 of a pair, packed (x0 in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
}
// The bf16 value of a pair (sel = 0) or its residual x - value (sel = 1).
__device__ __forceinline__ uint32_t split_pair(float x0, float x1, float sel) {
    const uint32_t h = pack_bf16(x0, x1);
    return pack_bf16(fmaf(-sel, bf16_lo(h), x0), fmaf(-sel, bf16_hi(h), x1));
}
// Three-term split of a pair: x = v + r + t to about 2^-26 |x|; `main` gets v
// (sel = 0) or r (sel = 1), `third` gets t where sel = 0 and zero elsewhere.
__device__ __forceinline__ void split3_pair(float x0, float x1, float sel, uint32_t &main,
                                            uint32_t &third) {
    const uint32_t v = pack_bf16(x0, x1);
    const float r0 = x0 - bf16_lo(v), r1 = x1 - bf16_hi(v);
    const uint32_t r = pack_bf16(r0, r1);
    main = sel != 0.f ? r : v;
    third = sel != 0.f ? 0u : pack_bf16(r0 - bf16_lo(r), r1 - bf16_hi(r));
}
// Element e of a bf16 row held in registers, as the 32-bit word holding it.
__device__ __forceinline__ uint32_t row_word(const RowLoad<uint16_t, 8> &r, int w) {
    return w == 0 ? r.raw.x : w == 1 ? r.raw.y : w == 2 ? r.raw.z : r.raw.w;
}
__device__ __forceinline__ uint32_t row_word(const RowLoad<uint16_t, 4> &r, int w) {
    return w == 0 ? r.raw.x : r.raw.y;
}

template <int D, bool HARD, int G>
__device__ __forceinline__ void attn_item_mfma(const AttnArgs &a, int u, int chunk,
                                               AttnShared<D, G, true> &sm) {
    constexpr int KC = D / 32;   // k-steps of q.K per half tile
    constexpr int EPL = D / 16;  // V elements per lane and token = P.V MFMAs per tile
    constexpr int TT = 32;       // tokens per tile
    constexpr int TPB = kBlockTokens / TT;
    static_assert(G >= 2 && G <= 8, "two operand columns per head");
    using VRow = RowLoad<uint16_t, EPL>;
    const int c = unit_count(a, u);
    const int nchunks = (c + a.split - 1) / a.split;
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4;
    const int n = lane & 15;
    const int head = n & 7;
    const bool live = head < G;
    const float sel = n >= 8 ? 1.f : 0.f;  // residual column

    bf16x8 qb[KC], qt[KC];  // query columns: value / residual, and the third terms
    {
        const float *qh = a.q + ((size_t)u * G + (live ? head : 0)) * D + 8 * g;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = live ? qh[32 * kc + e] * a.s : 0.f;
            uint4 w, t;
            split3_pair(x[0], x[1], sel, w.x, t.x);
            split3_pair(x[2], x[3], sel, w.y, t.y);
            split3_pair(x[4], x[5], sel, w.z, t.z);
            split3_pair(x[6], x[7], sel, w.w, t.w);
            qb[kc] = __builtin_bit_cast(bf16x8, w);
            qt[kc] = __builtin_bit_cast(bf16x8, t);
        }
    }
    const float t_own = live ? a.tau[(size_t)u * G + head] : 0.f;
    const float nbt_own = -a.nbl2e * t_own;

    const uint16_t *Kp = static_cast<const uint16_t *>(a.K);
    const uint16_t *Vp = static_cast<const uint16_t *>(a.V);
    const int rb = u / a.lay.H_kv;
    const int kh = u - rb * a.lay.H_kv;
    const int Tb = a.lay.row_len(rb);
    const int nblk_row = (Tb + kBlockTokens - 1) / kBlockTokens;  // ids past it are skipped
    // K tile: loaded row by row (CPR lanes per token row, TPI rows per load), kept
    // in this wave's LDS with 16-byte chunk c of token t at slot c ^ (t % CPR), and
    // read back in the A-operand layout (both directions free of bank conflicts)
    constexpr int CPR = D / 8;         // 16-byte chunks per token row
    constexpr int TPI = kWave / CPR;   // token rows per load instruction
    constexpr int NLD = TT / TPI;      // loads per tile
    const int ld_tok = lane / CPR, ld_ch = lane % CPR;
    const int k_off = ld_tok * D + ld_ch * 8;  // + TPI*D*i
    const int v_off = 4 * g * D + EPL * n;  // + (j + (j >= 4 ? 12 : 0)) * D
    const int32_t *iu = a.idx + (size_t)u * a.nblk_cap;

    const int j0 = chunk * a.split;
    const int j1 = min(c, j0 + a.split);
    const int nb = (j1 - j0 - wave + kAttnWaves - 1) / kAttnWaves;
    const int ntiles = nb > 0 ? nb * TPB : 0;

    auto tile_at = [&](int tt, size_t &off, int &valid) {
        const int blk = ld_const(iu + j0 + wave + (tt / TPB) * kAttnWaves);
        const long long bo =
            (unsigned)blk < (unsigned)nblk_row ? a.lay.block_offset(rb, kh, blk) : -1;
        const int sub = (tt % TPB) * TT;
        off = (bo < 0 ? 0 : (size_t)bo) + (size_t)sub * D;
        valid = bo < 0 ? 0 : min(Tb - blk * kBlockTokens, kBlockTokens) - sub;
    };

    float m_run = -INFINITY, l_run = 0.f;  // column n's head, over this lane's tokens
    f32x4 o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Pipeline: while tile t is multiplied from LDS buffer t % 2, the K of tile
    // t + 1 waits in registers (stored to the other buffer right after the q.K
    // products), the K loads of tile t + 2 and the V loads of tile t are in flight;
    // V of tile t + 1 is issued once tile t's P.V products have read V. Every load
    // thus has about one whole tile of work to arrive in.
    uint4 kr[NLD];
    VRow vr[8];
    auto k_load = [&](size_t off) {
        const uint16_t *p = Kp + off + k_off;
#pragma unroll
        for (int i = 0; i < NLD; ++i) kr[i] = ld_stream(reinterpret_cast<const uint4 *>(p + TPI * D * i));
    };
    auto k_store = [&](uint4 *kt) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int t = i * TPI + ld_tok;
            kt[t * CPR + (ld_ch ^ (t % CPR))] = kr[i];
        }
    };
    auto v_load = [&](size_t off) {
        const uint16_t *p = Vp + off + v_off;
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j].load(p + (j + (j >= 4 ? 12 : 0)) * D);
    };
    // One tile. NEXT: a tile t + 1 exists (store its K, issue its V); NEXT2: a tile
    // t + 2 exists (issue its K). The steady-state loop issues every load without a
    // branch, so the compiler's wait counts stay exact (a load skipped on some path
    // makes it wait for all loads in flight).
    size_t nxt_off = 0;  // tile t + 1
    int cur_valid = 0, nxt_valid = 0;
    auto tile = [&](int tt, auto NEXT, auto NEXT2) {
        const int valid = cur_valid;
        const uint4 *kt = sm.kt[wave][tt & 1];
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int c = 4 * kc + g;  // this lane's chunk of tokens n and 16 + n
            const bf16x8 k0 = __builtin_bit_cast(bf16x8, kt[n * CPR + (c ^ (n % CPR))]);
            const bf16x8 k1 = __builtin_bit_cast(bf16x8, kt[(16 + n) * CPR + (c ^ ((16 + n) % CPR))]);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[kc], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[kc], s1, 0, 0, 0);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qt[kc], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qt[kc], s1, 0, 0, 0);
        }
        // K of tile t + 1 into the other buffer (last read for tile t - 1), then the
        // K loads of tile t + 2 into the freed registers
        size_t nn_off = 0;
        int nn_valid = 0;
        if constexpr (decltype(NEXT)::value) k_store(sm.kt[wave][(tt + 1) & 1]);
        if constexpr (decltype(NEXT2)::value) {
            tile_at(tt + 2, nn_off, nn_valid);
            k_load(nn_off);
        }
        // logits of tok(g, j) for column n: value (+ third) part + residual part
        float gv[8];
        float bmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float part = j < 4 ? s0[j] : s1[j - 4];
            const float S = part + dpp_for_add<kRowRor8>(part);
            float gt;
            if (HARD) {
                gt = S >= t_own ? S : 0.f;
            } else {
                gt = S * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(a.nbl2e, S, nbt_own)));
            }
            if (4 * g + j + (j >= 4 ? 12 : 0) >= valid) gt = -INFINITY;
            gv[j] = gt;
            bmax = fmaxf(bmax, gt);
        }
        bmax = xrow_max(bmax);  // over the four lane rows: the tile's 32 tokens
        const float mx = fmaxf(m_run, bmax);
        const float m_ref = mx == -INFINITY ? 0.f : mx;  // nothing visible yet: weights 0
        const float corr = fast_exp(m_run - m_ref);
        m_run = mx;
        l_run *= corr;
        float pw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pw[j] = fast_exp(gv[j] - m_ref);
            l_run += pw[j];
        }
        const uint4 pwb = make_uint4(split_pair(pw[0], pw[1], sel), split_pair(pw[2], pw[3], sel),
                                     split_pair(pw[4], pw[5], sel), split_pair(pw[6], pw[7], sel));
        const bf16x8 pB = __builtin_bit_cast(bf16x8, pwb);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= corr;
        if (valid < TT) {  // rows past the row's length hold arbitrary bits
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (4 * g + j + (j >= 4 ? 12 : 0) >= valid) zero_row<uint16_t, EPL>(vr[j]);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint32_t sel_b = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint4 w = make_uint4(
                __builtin_amdgcn_perm(row_word(vr[1], e / 2), row_word(vr[0], e / 2), sel_b),
                __builtin_amdgcn_perm(row_word(vr[3], e / 2), row_word(vr[2], e / 2), sel_b),
                __builtin_amdgcn_perm(row_word(vr[5], e / 2), row_word(vr[4], e / 2), sel_b),
                __builtin_amdgcn_perm(row_word(vr[7], e / 2), row_word(vr[6], e / 2), sel_b));
            o[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pB, o[e],
                                                           0, 0, 0);
        }
        if constexpr (decltype(NEXT)::value) v_load(nxt_off);
        cur_valid = nxt_valid;
        nxt_off = nn_off;
        nxt_valid = nn_valid;
    };
    using yes = std::true_type;
    using no = std::false_type;
    if (ntiles > 0) {
        size_t cur_off;
        tile_at(0, cur_off, cur_valid);
        k_load(cur_off);
        k_store(sm.kt[wave][0]);
        if (ntiles > 1) {
            tile_at(1, nxt_off, nxt_valid);
            k_load(nxt_off);
            v_load(cur_off);
            int tt = 0;
            for (; tt + 2 < ntiles; ++tt) tile(tt, yes{}, yes{});
            tile(tt, yes{}, no{});
            tile(tt + 1, no{}, no{});
        } else {
            v_load(cur_off);
            tile(0, no{}, no{});
        }
    }

    // value + residual columns; then lane (g, n < G) holds elements
    // EPL*(4g + i) + e of head n
    const float l_head = xrow_sum(l_run);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[e][i] += dpp_for_add<kRowRor8>(o[e][i]);
    __syncthreads();  // sm.o shares its space with the waves' K tiles
    if (n < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm.o[wave][n][EPL * (4 * g + i) + e] = o[e][i];
        if (g == 0) {
            sm.m[wave][n] = m_run;
            sm.l[wave][n] = l_head;
        }
    }
    __syncthreads();
    merge_heads<D, G>(a, u, chunk, nchunks, sm);
}

// Persistent workers: each workgroup takes item tickets until the list is done.
template <typename KV, int D, int TS, bool HARD, int G>
__global__ __launch_bounds__(kAttnWaves *kWave, 2) void attn_partial_kernel(AttnArgs a) {
    __shared__ AttnShared<D, G, (G > 1 && sizeof(KV) == 2)> sm;
    const int total = ld_const(a.ws_hdr);
    if (threadIdx.x == 0) sm.ticket = atomicAdd(&a.ws_hdr[1], 1);
    __syncthreads();
    int ticket = uniform(sm.ticket);  // the item's unit, list and lengths: scalar loads
    while (ticket < total) {
        const int *itp = reinterpret_cast<const int *>(a.ws_items + ticket);
        const int2 it = make_int2(ld_const(itp), ld_const(itp + 1));
        int next = 0;
        if (threadIdx.x == 0) next = atomicAdd(&a.ws_hdr[1], 1);  // fetched early
        if constexpr (G > 1 && sizeof(KV) == 2) {  // grouped heads, bf16: matrix cores
            attn_item_mfma<D, HARD, G>(a, it.x, it.y, sm);
        } else if constexpr (G > 1) {  // grouped heads, fp32: reduce-scatter on the VALU
            attn_item_dist<KV, D, TS, HARD, G>(a, it.x, it.y, sm);
        } else {  // multi-head attention: the one-pass row layout
            attn_item<KV, D, TS, HARD, G>(a, it.x, it.y, sm);
        }
        if (threadIdx.x == 0) sm.ticket = next;
        __syncthreads();
        ticket = uniform(sm.ticket);
    }
}

// Compacted item list: items of unit u are (u, 0 .. ceil(cnt[u]/split) - 1),
// units in order. Units with nothing admitted get out = 0, lse = -inf here.
// Each workgroup owns kPlanUnits consecutive units: it first sums the item
// counts of all earlier units itself (a few KiB of reads, no cross-workgroup
// communication), scans its own units in one wave, and then writes each unit's
// items with one wave per unit on consecutive list entries. The last workgroup
// stores the item total; workgroup 0 resets the ticket counter.
constexpr int kPlanThreads = 256;
constexpr int kPlanUnits = 64;

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnArgs a, int D, int G) {
    __shared__ int red[kPlanThreads / kWave];
    __shared__ int excl[kPlanUnits];
    __shared__ int cnt_s[kPlanUnits];
    __shared__ int tile_total;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    static_assert(kPlanUnits == kWave, "one lane per unit of the tile");
    const int u0 = blockIdx.x * kPlanUnits;
    auto items_of = [&](int u) { return (unit_count(a, u) + a.split - 1) / a.split; };

    int before = 0;  // items of units [0, u0)
#pragma unroll 4
    for (int u = tid; u < u0; u += kPlanThreads) before += items_of(u);
#pragma unroll
    for (int k = 1; k < kWave; k <<= 1) before += __shfl_xor(before, k, kWave);
    if (lane == 0) red[wave] = before;
    if (wave == 0) {
        const int u = u0 + lane;
        const int c = u < a.units ? unit_count(a, u) : 0;
        const int n = (c + a.split - 1) / a.split;
        cnt_s[lane] = c;
        int x = n;  // inclusive scan over the tile's units
#pragma unroll
        for (int k = 1; k < kWave; k <<= 1) {
            const int y = __shfl_up(x, k, kWave);
            if (lane >= k) x += y;
        }
        excl[lane] = x - n;
        if (lane == kWave - 1) tile_total = x;
    }
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w) base += red[w];

    for (int t = wave; t < kPlanUnits; t += kPlanThreads / kWave) {
        const int u = u0 + t;
        if (u >= a.units) break;
        const int c = cnt_s[t];
        if (c <= 0) {  // nothing admitted for any of the unit's query heads
            for (int i = lane; i < D * G; i += kWave) a.out[(size_t)u * G * D + i] = 0.f;
            if (lane < G && a.lse) a.lse[(size_t)u * G + lane] = -INFINITY;
            continue;
        }
        const int n = (c + a.split - 1) / a.split;
        const int off = base + excl[t];
        for (int j = lane; j < n; j += kWave) a.ws_items[off + j] = make_int2(u, j);
    }
    if (tid == 0) {
        if (blockIdx.x == gridDim.x - 1) a.ws_hdr[0] = base + tile_total;
        if (blockIdx.x == 0) a.ws_hdr[1] = 0;
    }
}

// Log-sum-exp merge of the partials of every unit that has more than one item.
// One workgroup per unit: the item maxima, weights and sums are reduced across
// the workgroup, and thread t accumulates output dimension t % D over the items
// i = t / D, t / D + R, ... (R = threads / D), in a fixed order; the R partial
// sums are then added in LDS in a fixed order (deterministic).
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
    constexpr int R = kCombineThreads / D;
    constexpr int NW = kCombineThreads / kWave;
    __shared__ float red[NW];
    __shared__ float part[R][D];
    const int uq = blockIdx.x;     // query unit
    const int u = uq / a.G;        // its key/value unit
    const int hj = uq - u * a.G;   // head within the group
    const int c = unit_count(a, u);
    const int nchunks = (c + a.split - 1) / a.split;
    if (nchunks <= 1) return;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    const size_t s0 = (size_t)u * a.ws_chunks * a.G + hj;  // partial of item i: s0 + i * G
    const int gs = a.G;

    float mx = -INFINITY;
    for (int i = tid; i < nchunks; i += kCombineThreads) mx = fmaxf(mx, a.ws_m[s0 + (size_t)i * gs]);
    mx = xrow_max(row_max16(mx));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
    const float Mr = M == -INFINITY ? 0.f : M;  // no token in any item: weights 0
    __syncthreads();  // red is reused below

    float ls = 0.f;
    for (int i = tid; i < nchunks; i += kCombineThreads) {
        const size_t sl = s0 + (size_t)i * gs;
        ls += a.ws_l[sl] * fast_exp(a.ws_m[sl] - Mr);
    }
    ls = xrow_sum(row_sum16(ls));
    if (lane == 0) red[wave] = ls;

    const int dim = tid % D;
    const int r = tid / D;
    float O = 0.f;
#pragma unroll 4
    for (int i = r; i < nchunks; i += R) {
        const size_t sl = s0 + (size_t)i * gs;
        O += a.ws_o[sl * D + dim] * fast_exp(a.ws_m[sl] - Mr);
    }
    part[r][dim] = O;
    __syncthreads();
    if (tid < D) {
        float Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) Lsum += red[w];
        float Ot = 0.f;
#pragma unroll
        for (int k = 0; k < R; ++k) Ot += part[k][tid];
        a.out[(size_t)uq * D + tid] = Lsum > 0.f ? Ot / Lsum : 0.f;
        if (tid == 0 && a.lse) a.lse[uq] = Lsum > 0.f ? M + __logf(Lsum) : -INFINITY;
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

AttnArgs make_args(const Geometry &g, const float *q, const void *K, const void *V,
                   const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                   float gate_beta, int split_blocks, int max_chunks, float *out, float *lse,
                   void *ws) {
    const AttnWorkspace w = attn_workspace_layout(g.units, max_chunks, g.d);
    char *base = static_cast<char *>(ws);
    AttnArgs a;
    a.units = g.kv_units;
    a.G = g.G;
    a.lay = g.lay;
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
    a.ws_hdr = reinterpret_cast<int *>(base + w.off_hdr);
    a.ws_items = reinterpret_cast<int2 *>(base + w.off_items);
    return a;
}

template <typename KV, int D, int TS, int G>
hipError_t launch_partial_t(const AttnArgs &a, bool hard, int workers, hipStream_t st) {
    const dim3 grid((unsigned)workers);
    if (hard) {
        hipLaunchKernelGGL((attn_partial_kernel<KV, D, TS, true, G>), grid,
                           dim3(kAttnWaves * kWave), 0, st, a);
    } else {
        hipLaunchKernelGGL((attn_partial_kernel<KV, D, TS, false, G>), grid,
                           dim3(kAttnWaves * kWave), 0, st, a);
    }
    return hipGetLastError();
}

// Tile rows per K/V register buffer of the vector-ALU paths: smaller tiles for
// wider rows and more query heads per key/value head keep every instance but
// fp32 d = 128 with G = 2 at two or three waves per SIMD. (bf16 with grouped
// heads takes the matrix-core path, whose 32-token tile does not depend on it.)
template <typename KV, int D>
hipError_t launch_partial_g(const AttnArgs &a, bool hard, int workers, hipStream_t st) {
    constexpr bool wide = sizeof(KV) * D > 256;  // fp32 rows of 128
    constexpr bool narrow = sizeof(KV) * D < 256;  // bf16 rows of 64
    switch (a.G) {
        case 1: return launch_partial_t<KV, D, wide ? 32 : 64, 1>(a, hard, workers, st);
        case 2: return launch_partial_t<KV, D, narrow ? 64 : 32, 2>(a, hard, workers, st);
        case 4: return launch_partial_t<KV, D, narrow ? 32 : (wide ? 16 : 32), 4>(a, hard, workers, st);
        default: return launch_partial_t<KV, D, narrow ? 32 : (D == 128 ? 8 : 16), 8>(a, hard, workers, st);
    }
}

}  // namespace

AttnWorkspace attn_workspace_layout(int units, int max_chunks, int d) {
    AttnWorkspace w;
    const size_t slots = (size_t)units * (size_t)max_chunks;
    w.off_hdr = 0;
    w.off_items = align256(w.off_hdr + 2 * sizeof(int));
    w.off_m = align256(w.off_items + 2 * sizeof(int) * slots);
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
    hipLaunchKernelGGL(attn_plan_kernel,
                       dim3((unsigned)((g.kv_units + kPlanUnits - 1) / kPlanUnits)),
                       dim3(kPlanThreads), 0, st, a, g.d, g.G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // persistent workers: one or two per CU, never more than the largest possible item count
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    const bool small_tiles = g.G == 1 && g.bf16 && g.d == 64;
    long long workers = (long long)cus * (small_tiles ? kWorkersPerCUSmallTiles : kWorkersPerCU);
    const long long most = (long long)g.kv_units * ((g.nblk + split_blocks - 1) / split_blocks);
    if (workers > most) workers = most > 0 ? most : 1;
    const int wk = (int)workers;
    if (g.bf16) {
        return g.d == 128 ? launch_partial_g<uint16_t, 128>(a, gate_hard, wk, st)
                          : launch_partial_g<uint16_t, 64>(a, gate_hard, wk, st);
    }
    return g.d == 128 ? launch_partial_g<float, 128>(a, gate_hard, wk, st)
                      : launch_partial_g<float, 64>(a, gate_hard, wk, st);
}

hipError_t launch_attn_combine(const Geometry &g, const int32_t *adm_cnt, int split_blocks,
                               int max_chunks, float *out, float *lse, void *ws, hipStream_t st) {
    if (g.units == 0) return hipSuccess;
    const AttnArgs a = make_args(g, nullptr, nullptr, nullptr, nullptr, nullptr, adm_cnt, 1.f,
                                 split_blocks, max_chunks, out, lse, ws);
    if (g.d == 128) {
        hipLaunchKernelGGL((attn_combine_kernel<128>), dim3((unsigned)g.units),
                           dim3(kCombineThreads), 0, st, a);
    } else {
        hipLaunchKernelGGL((attn_combine_kernel<64>), dim3((unsigned)g.units),
                           dim3(kCombineThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace eta
