// eta_device.hpp -- device helpers shared by the ETA kernels (gfx950, wave64).
//
// Lane layout used by every kernel that walks key or value rows: a wave64 is
// four 16-lane DPP rows; row r of the wave owns one token, and lane c of the
// row owns the EPL = d/16 consecutive elements [EPL*c, EPL*c + EPL) of it.
// One wave load instruction therefore covers four whole token rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eta {

constexpr int kWave = 64;
constexpr int kBlockTokens = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- streaming loads ----
// Data one launch reads once (K/V rows, block metadata) is loaded with the
// non-temporal hint. On MI355X a plain read kernel streams about 6.2 TB/s with
// ordinary 16-byte loads and about 6.9 TB/s with this hint.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2 *p) {
    const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 ld_stream(const float4 *p) {
    const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// ---- bfloat16 -> float32: exact widening of the upper half of a binary32 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- DPP helpers (row = 16 lanes) ----
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Lane permutation for a sum: every source lane of the patterns used here lies in
// the same full row, so the zero written for an invalid source never occurs; the
// zero "old" value lets the compiler fold the move into the add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_for_add(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each row; every lane of the row receives the sum.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_for_add<kQuadXor1>(x);
    x += dpp_for_add<kQuadXor2>(x);
    x += dpp_for_add<kRowHalfMirror>(x);
    x += dpp_for_add<kRowMirror>(x);
    return x;
}

// Max over the 16 lanes of each row; every lane of the row receives it.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp_mov<kQuadXor1>(x));
    x = fmaxf(x, dpp_mov<kQuadXor2>(x));
    x = fmaxf(x, dpp_mov<kRowHalfMirror>(x));
    x = fmaxf(x, dpp_mov<kRowMirror>(x));
    return x;
}

// Combine lanes l and l ^ 16 (rows 0-1 and 2-3) or l and l ^ 32 (the two halves of
// the wave) without LDS: each swap leaves a lane's own value in one result and its
// partner's in the other, the lower row's first in both, so both partners get
// bitwise the same result (addition and max are commutative, so it also equals
// adding the partner's value to one's own).
__device__ __forceinline__ float row_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Combine the four rows of the wave (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float xrow_sum(float x) { return half_pair_sum(row_pair_sum(x)); }
__device__ __forceinline__ float xrow_max(float x) { return half_pair_max(row_pair_max(x)); }

// ---- wave-uniform values ----
// The compiler cannot tell that threadIdx.x / 64, or a value read back from LDS,
// is the same on every lane of a wave. Addresses formed from such values are then
// read with vector loads, and waiting for one of those (vmcnt counts in issue
// order) also waits for every K/V load issued before it. Passed through
// readfirstlane, the value is known to be uniform: list entries, page ids and
// lengths indexed by it are read with scalar loads, whose wait does not touch the
// vector loads in flight.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int wave_id() { return uniform((int)threadIdx.x / kWave); }
// A read of memory that no thread writes while the kernel runs (its inputs, and
// what an earlier launch on the stream wrote). Stores elsewhere in the kernel
// keep the compiler from proving that on its own; through the constant address
// space a wave-uniform address becomes a scalar load, a per-lane one stays a
// vector load.
template <typename T>
__device__ __forceinline__ T ld_const(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---- where the rows of a key/value unit live ----
// Dense: block j of unit (b, k) at ((b*H_kv + k)*T_cap/64 + j)*block_stride, its
// 64 rows of d elements back to back (block_stride = 64*d: K[(b*H_kv + k)][T_cap][d];
// 128*d with V = K + 64*d: K and V interleaved block by block). Paged: a page
// table [B][max_pages] (logical block -> page) and pools whose block of head k in
// page p sits at (p*H_kv + k)*block_stride ([num_pages][H_kv][64][d] at 64*d).
// Rows may hold different numbers of tokens (seq_lens).
struct KVLayout {
    const int32_t *seq_lens;  // null: every row holds T
    const int32_t *pages;     // null: dense layout
    int T, T_cap, H_kv, max_pages, num_pages;
    long long block_stride;   // elements from one 64-row block to the next

    __device__ __forceinline__ int row_len(int b) const {
        if (seq_lens == nullptr) return T;
        const int t = ld_const(seq_lens + b);
        return t < 0 ? 0 : (t > T ? T : t);
    }
    // Where logical block j of row b lives: its page id (paged), or j itself
    // (dense). Split from page_offset so that a caller can read the page table
    // well before it needs the address.
    __device__ __forceinline__ int page_of(int b, int j) const {
        return pages != nullptr ? ld_const(pages + (size_t)b * max_pages + j) : j;
    }
    // Element offset of key/value unit (b, k)'s block at pg (from page_of); -1
    // when the page id is out of range.
    __device__ __forceinline__ long long page_offset(int b, int k, int pg) const {
        if (pages != nullptr) {
            if ((unsigned)pg >= (unsigned)num_pages) return -1;
            return ((long long)pg * H_kv + k) * block_stride;
        }
        return ((long long)(b * H_kv + k) * (T_cap / kBlockTokens) + pg) * block_stride;
    }
    // Element offset of logical block j of key/value unit (b, k); -1 when the
    // block's page is out of range.
    __device__ __forceinline__ long long block_offset(int b, int k, int j) const {
        return page_offset(b, k, page_of(b, j));
    }
};

// ---- row loads: EPL elements of one token row, widened to float ----
// KV = float or uint16_t (bfloat16 bits). EPL = d / 16.
template <typename KV, int EPL>
struct RowLoad;

template <>
struct RowLoad<uint16_t, 8> {  // d = 128, bf16: 16 bytes per lane
    uint4 raw;
    __device__ __forceinline__ void load(const uint16_t *p) { raw = ld_stream(reinterpret_cast<const uint4 *>(p)); }
    __device__ __forceinline__ void widen(float (&x)[8]) const {
        x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
        x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
        x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
        x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
    }
};

template <>
struct RowLoad<uint16_t, 4> {  // d = 64, bf16: 8 bytes per lane
    uint2 raw;
    __device__ __forceinline__ void load(const uint16_t *p) { raw = ld_stream(reinterpret_cast<const uint2 *>(p)); }
    __device__ __forceinline__ void widen(float (&x)[4]) const {
        x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
        x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
    }
};

template <>
struct RowLoad<float, 8> {  // d = 128, fp32: 32 bytes per lane
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = ld_stream(reinterpret_cast<const float4 *>(p));
        b = ld_stream(reinterpret_cast<const float4 *>(p + 4));
    }
    __device__ __forceinline__ void widen(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

template <>
struct RowLoad<float, 4> {  // d = 64, fp32: 16 bytes per lane
    float4 a;
    __device__ __forceinline__ void load(const float *p) { a = ld_stream(reinterpret_cast<const float4 *>(p)); }
    __device__ __forceinline__ void widen(float (&x)[4]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    }
};

}  // namespace eta
