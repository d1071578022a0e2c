// eta_prefill.hip -- the training-time (prefill) forward of the ETA gate: dense
// causal attention over whole sequences with every logit S = s * q.k multiplied
// by sigmoid(beta * (S - tau_t)), tau_t the threshold of query token t
// (evolve.pub review, "Methodology Assessment": Eq. 1 per token, Eq. 2 gate,
// Eq. 3 multiplicative gating; arXiv:2609.20888 abstract: in training a logit
// under the threshold is multiplied down to zero instead of being masked out).
//
// Unlike the decode step this is a dense contraction, so both products run on
// the CDNA4 matrix cores (32x32x16 MFMA):
//   S^T = K . Q^T  bf16 x bf16 -> fp32   (M = keys, N = queries, K = head dim)
//   O^T += V^T . P^T  fp16 x fp16 -> fp32 (M = head dim, N = queries, K = keys)
// Computing the transposes keeps one query per lane: in the MFMA result layout
// lane l holds query l % 32 and 32 of the tile's 64 keys, its partner lane
// l ^ 32 the other 32, so the row softmax needs one cross-lane exchange per
// tile. The 32 gated weights of a lane are, register for register, the B
// operand of the P.V product (the product's reduction runs over keys in any
// fixed order, and both operands use the same key order), so P never leaves
// the registers. V is staged into LDS transposed and converted to fp16 (exact
// for |v| in [2^-14, 65504]). The weights enter the product rounded toward
// zero to fp16 (one conversion instruction per pair), and out is divided by
// the sum of those same rounded weights (one fp16 dot2 per pair), so the
// rounding perturbs each weight's share by at most 2^-11 around their common
// part and cannot bias the output: constant value rows come out exactly, and
// |out error| <= 2^-11 * sum_j w_j |v_j - out|, whatever the mean of V. The
// fp32 sum of the unrounded weights gives lse. Both sums (and the gate sum) are
// formed per tile first and added to the running sums once per tile, so their
// rounding stays at a few units in the last place however many keys a query
// sees (a running sum taking every weight drifted by ~1e-4 in lse at 32K keys).
// The weights are taken against a reference that may trail the running
// maximum by a bounded amount, so a tile whose maximum stays under that bound
// needs no rescaling of the output and the sums.
//
// Workgroup = 4 waves = 128 consecutive queries of one (row, head); wave w owns
// queries 32w .. 32w + 31. Key tiles of 64 are staged into LDS (K row-major by
// direct global-to-LDS loads, V^T through registers), the next tile's global
// loads are in flight while the current one is computed. Causal: query i sits at position T_k - T_q + i and sees keys at or
// before it. Grid x = (row, head), y = query block, heaviest blocks first; all
// query blocks of one head share an XCD when B * H is a multiple of 8.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kPfWaves = 4;
constexpr int kPfQ = 32 * kPfWaves;  // queries per workgroup
constexpr int kPfKeys = 64;          // keys per tile
constexpr float kPfSlack = 8.f;      // log2 units the weight reference may trail the maximum

template <int D>
struct PfShared {
    static constexpr int KCH = D / 8;       // 16-byte chunks per K row
    static constexpr int VS = kPfKeys + 4;  // fp16 per V^T row (8 bytes of padding)
    // K rows unpadded; chunk c of row r sits at chunk c ^ (r % KCH) of its row, so
    // the rows an MFMA operand read touches together hit distinct banks. Written by the
    // direct global-to-LDS loads (64 lanes x 16 contiguous bytes per instruction).
    alignas(16) uint16_t k[2][kPfKeys * D];  // double buffered: one barrier per tile
    // V^T row r keeps key k at column k ^ swz(r): 16-key groups are permuted by the
    // row's 32-dimension tile, so the transposing writes (8 bytes per lane, rows
    // 8 apart across lanes) spread over the banks; a reading wave works on one
    // 32-row tile at a time, so its reads are only shifted.
    alignas(16) uint16_t vt[2][D * VS];
};

struct PfArgs {
    int H, Hkv, G, T_q, T_k, q_off;
    float s, c_gate, c_soft;  // 1/sqrt(d), -beta*log2(e)/sqrt(d), log2(e)/sqrt(d)
    float inv_c;              // 1 / c_soft
    const uint16_t *Q;
    const uint16_t *K;
    const uint16_t *V;
    const float *tau;
    float *out;
    float *lse;
    float *gate_sum;
};

// bfloat16 element e of a 16-byte row chunk, widened to float (exact).
__device__ __forceinline__ float bf16_elem(const uint4 &r, int e) {
    const uint32_t w = e < 2 ? r.x : (e < 4 ? r.y : (e < 6 ? r.z : r.w));
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Two floats to packed fp16, rounded toward zero (exact for values representable
// in fp16).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Staging of one key tile: K rows as they are, V transposed to [d][key] in fp16.
// KPT keys x 8 dimensions of V per thread (D / 32 keys: 4 for d = 128, 2 for 64);
// each fp16 pair written to LDS holds two consecutive keys of one dimension.
template <int D>
struct StageShape {
    static constexpr int KCH = D / 8;                               // 16-byte chunks per row
    static constexpr int KLD = kPfKeys * KCH / (kPfWaves * kWave);  // K chunks per thread
    static constexpr int KPT = D / 32;                              // V keys per thread
};

// Chunk swizzle of K row r (see PfShared): the 16 rows (8 at d = 64) a reading
// lane group touches at one logical chunk land on distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return r & (D / 8 - 1); }

// Key swizzle of V^T row r (see PfShared): flips the 16-key group by r / 32.
__device__ __forceinline__ int vt_swz(int r) { return ((r >> 5) & 3) << 4; }

// Buffer resource over the rows [k0, T_k) of one (row, key/value head) slab of K or
// V: reads at or past T_k return zeros (hardware range check), so a tile that
// runs past the end needs no clamping, and the tile's base lives in scalar
// registers (lanes add only their constant 32-bit offsets). The slab is at most
// 2^31 bytes (checked on the host).
#define ETA_TILE_RSRC(slab, k0, T_k)                                                     \
    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>((slab) + (size_t)(k0) * D), \
                                      (short)0, max((T_k) - (k0), 0) * D * 2, 0x00020000)

// Byte offsets of a lane's K chunks within a tile: instruction i of wave w fills
// chunk positions (w * KLD + i) * 64 + lane of the swizzled LDS buffer.
template <int D>
__device__ __forceinline__ uint32_t k_lane_off(int wave, int lane, int i) {
    using S = StageShape<D>;
    const int p = (wave * S::KLD + i) * kWave + lane;
    const int r = p / S::KCH;
    const int c = (p % S::KCH) ^ k_swz<D>(r);
    return (uint32_t)(r * D * 2 + c * 16);
}

// K rows of one key tile straight into LDS (no registers).
template <int D>
__device__ __forceinline__ void stage_k_lds(const uint16_t *Kh, int k0, int T_k, int wave_u,
                                            const uint32_t (&koff)[StageShape<D>::KLD],
                                            uint16_t *kbuf) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-resource type exists for the device only
    using S = StageShape<D>;
    const auto rs = ETA_TILE_RSRC(Kh, k0, T_k);
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs,
            reinterpret_cast<__attribute__((address_space(3))) void *>(
                reinterpret_cast<uintptr_t>(kbuf + (wave_u * S::KLD + i) * kWave * 8)),
            16, koff[i], 0, 0, 0);
    }
#endif
}

// V rows of one key tile into registers: KPT consecutive keys x 8 dimensions per
// thread (rows past T_k read as zeros).
template <int D>
__device__ __forceinline__ void stage_load(const uint16_t *Vh, int k0, int T_k, uint32_t voff,
                                           uint4 (&vr)[StageShape<D>::KPT]) {
#if defined(__HIP_DEVICE_COMPILE__)
    using S = StageShape<D>;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const auto rs = ETA_TILE_RSRC(Vh, k0, T_k);
#pragma unroll
    for (int r = 0; r < S::KPT; ++r) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + r * D * 2, 0, 0);
        vr[r] = make_uint4(x.x, x.y, x.z, x.w);
    }
#endif
}

template <int D>
__device__ __forceinline__ void stage_store(PfShared<D> &sm, int buf,
                                            const uint4 (&vr)[StageShape<D>::KPT]) {
    using S = StageShape<D>;
    const int tid = threadIdx.x;
    const int ka = tid / S::KCH;
    const int db = tid % S::KCH;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = db * 8 + i;
        uint16_t *dst = &sm.vt[buf][row * PfShared<D>::VS + ((ka * S::KPT) ^ vt_swz(row))];
        const uint32_t p01 = pack_f16(bf16_elem(vr[0], i), bf16_elem(vr[1], i));
        if (S::KPT == 4) {
            const uint32_t p23 = pack_f16(bf16_elem(vr[2], i), bf16_elem(vr[3], i));
            *reinterpret_cast<uint2 *>(dst) = make_uint2(p01, p23);
        } else {
            *reinterpret_cast<uint32_t *>(dst) = p01;
        }
    }
}

// Gate, mask and exponent of one lane's 32 scores (acc = q.k, unscaled), in
// log2 units relative to the reference mref: t = log2(e) * S' - mref, with
// S' = S * sigmoid(beta (S - tau)) and S = s * acc. The soft gate's reciprocal
// carries the scale: rcp(inv_c * (1 + e)) = c_soft * sigmoid, so the gated
// exponent is one fma of acc with it. g_sum gains the tile's gates in those
// scaled units (the caller divides by c_soft), summed within the tile first so
// that the running sum takes one addition per tile. Returns the tile maximum.
template <bool HARD, bool GSUM, bool MASK>
__device__ __forceinline__ float gate_tile(const PfArgs &a, const float (&acc)[2][16], float t_acc,
                                           float nbt, float mref, int lim, float (&tv)[2][16],
                                           float &g_sum) {
    float mx = -INFINITY;
    float gp[4] = {0.f, 0.f, 0.f, 0.f};  // the tile's gates, four partial sums
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float x = acc[mt][j];
            float t, gate = 0.f;
            if (HARD) {
                const bool on = x >= t_acc;
                t = fmaf(on ? x : 0.f, a.c_soft, -mref);
                if (GSUM) gate = on ? 1.f : 0.f;
            } else {
                const float e = __builtin_amdgcn_exp2f(fmaf(a.c_gate, x, nbt));
                const float mc = __builtin_amdgcn_rcpf(fmaf(e, a.inv_c, a.inv_c));
                t = fmaf(x, mc, -mref);
                if (GSUM) gate = mc;
            }
            if (MASK) {
                const int off = mt * 32 + (j >> 2) * 8 + (j & 3);  // key offset minus 4*hl
                if (off > lim) {
                    t = -INFINITY;
                    gate = 0.f;
                }
            }
            if (GSUM) gp[j & 3] += gate;
            tv[mt][j] = t;
            mx = fmaxf(mx, t);
        }
    }
    if (GSUM) g_sum += (gp[0] + gp[1]) + (gp[2] + gp[3]);
    return mx;
}

template <int D, bool HARD, bool GSUM>
__global__ __launch_bounds__(kPfWaves *kWave, 2) void prefill_attn_kernel(PfArgs a) {
    __shared__ PfShared<D> sm;
    constexpr int VS = PfShared<D>::VS;
    constexpr int NKS = D / 16;  // k-steps of the S product
    constexpr int NMD = D / 32;  // head-dimension tiles of the O product

    const int bh = blockIdx.x;  // b * H + h
    const int nqb = gridDim.y;
    const int qb = nqb - 1 - (int)blockIdx.y;  // heaviest (latest) query blocks first
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int hk = h / a.G;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int hl = lane >> 5;   // lane half: which 8 of a 16-wide reduction step
    const int col = lane & 31;  // query within the wave's 32

    const int q0 = qb * kPfQ;
    const int qi = q0 + wave * 32 + col;  // this lane's query index
    const int qc = min(qi, a.T_q - 1);    // clamped for loads
    const int qpos = a.q_off + qi;        // its position among the keys
    const uint16_t *Qh = a.Q + ((size_t)bh * a.T_q) * D;
    const uint16_t *Kh = a.K + ((size_t)(b * a.Hkv + hk) * a.T_k) * D;
    const uint16_t *Vh = a.V + ((size_t)(b * a.Hkv + hk) * a.T_k) * D;

    // Q^T as the B operand of S^T = K Q^T, one 8-element slice per k-step
    bf16x8 qB[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(Qh + (size_t)qc * D + ks * 16 + hl * 8);
        qB[ks] = __builtin_bit_cast(bf16x8, raw);
    }
    const float t = a.tau[(size_t)bh * a.T_q + qc];
    const float nbt = -a.c_gate * t / a.s;  // gate exponent = c_gate * acc + nbt
    const float t_acc = t / a.s;            // the hard step in acc units

    // keys this workgroup needs: up to the position of its last query
    const int q_last = min(q0 + kPfQ, a.T_q) - 1;
    const int k_end = min(a.T_k, a.q_off + q_last + 1);
    const int ntiles = (k_end + kPfKeys - 1) / kPfKeys;
    const int wave_first_pos = a.q_off + q0 + wave * 32;  // smallest query position of the wave

    f32x16 o[NMD];
#pragma unroll
    for (int m = 0; m < NMD; ++m) o[m] = f32x16{};
    // Weights are 2^t with t taken against a reference mref (log2 units) that
    // trails the running maximum by at most kPfSlack: the first tile sets it to
    // that tile's maximum, a later tile moves it (and rescales the sums) only
    // when its own maximum lies more than kPfSlack above it. Every weight is
    // then at most 2^kPfSlack and the largest one at least 1, so the fp16
    // weights keep their full precision and the sums stay far from overflow.
    float mref = 0.f, g_sum = 0.f;
    float l_run = 0.f;   // sum of the fp32 weights: lse
    float lh_run = 0.f;  // sum of the weights as rounded to fp16 for P.V: out's divisor
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    // staging offsets of this lane (constant over the key tiles)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t koff[StageShape<D>::KLD];
#pragma unroll
    for (int i = 0; i < StageShape<D>::KLD; ++i) koff[i] = k_lane_off<D>(wave_u, lane, i);
    const uint32_t voff = (uint32_t)((tid / StageShape<D>::KCH) * StageShape<D>::KPT * D * 2 +
                                     (tid % StageShape<D>::KCH) * 16);
    uint4 vr[StageShape<D>::KPT];
    stage_k_lds<D>(Kh, 0, a.T_k, wave_u, koff, sm.k[0]);
    stage_load<D>(Vh, 0, a.T_k, voff, vr);
    stage_store<D>(sm, 0, vr);
    __builtin_amdgcn_s_waitcnt(0);  // the K rows have landed in LDS
    __syncthreads();
    for (int tt = 0; tt < ntiles; ++tt) {
        const int k0 = tt * kPfKeys;
        const int buf = tt & 1;
        // the next tile's V rows are in flight during this one (issued
        // unconditionally: past the last tile every row reads as zero, and the
        // staging registers stay out of scratch memory)
        stage_load<D>(Vh, k0 + kPfKeys, a.T_k, voff, vr);

        // S^T for keys k0 .. k0 + 63 (two 32-key tiles) against the wave's 32 queries
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int r = mt * 32 + col;
                const uint4 raw = *reinterpret_cast<const uint4 *>(
                    &sm.k[buf][r * D + (((ks * 2 + hl) ^ k_swz<D>(r)) * 8)]);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw),
                                                                qB[ks], s[mt], 0, 0, 0);
            }
        }
        // the next tile's K rows go straight into the other buffer once this tile's
        // K reads are issued (that buffer's last readers finished before the barrier
        // that ended the previous iteration)
        if (tt + 1 < ntiles) stage_k_lds<D>(Kh, k0 + kPfKeys, a.T_k, wave_u, koff, sm.k[buf ^ 1]);
        float acc[2][16];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][j] = s[mt][j];

        // gate, causal mask (diagonal and last tiles only), exponents, tile maximum
        float g[2][16];
        float mx;
        if (k0 + kPfKeys - 1 > wave_first_pos || k0 + kPfKeys > a.T_k) {
            mx = gate_tile<HARD, GSUM, true>(a, acc, t_acc, nbt, mref, qpos - k0 - hl * 4, g, g_sum);
        } else {
            mx = gate_tile<HARD, GSUM, false>(a, acc, t_acc, nbt, mref, 0, g, g_sum);
        }
        mx = half_pair_max(mx);  // the partner lane l ^ 32 holds the other 32 keys
        // the first tile holds key 0, which every query sees: its maximum is finite
        const bool move = tt == 0 || mx > kPfSlack;
        if (__any(move)) {
            const float shift = move ? mx : 0.f;
            mref += shift;
            if (tt > 0) {  // the sums so far were taken against the old reference
                const float corr = __builtin_amdgcn_exp2f(-shift);
                l_run *= corr;
                lh_run *= corr;
#pragma unroll
                for (int m = 0; m < NMD; ++m) o[m] *= corr;
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int j = 0; j < 16; ++j) g[mt][j] -= shift;
        }

        // weights, packed as the fp16 B operand of O^T += V^T P^T: k-step s (keys
        // 16s .. 16s + 15) takes registers 8(s%2) .. 8(s%2) + 7 of key tile s/2
        uint32_t pw[4][4];
        // the tile's weights summed on their own first (fp32 partial sums for lse, fp16
        // dot products for out's divisor): the running sums take one addition per tile,
        // so their rounding does not grow with the number of keys
        float lp[4] = {0.f, 0.f, 0.f, 0.f};
        float lhp[2] = {0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(g[mt][j]);
                const float p1 = __builtin_amdgcn_exp2f(g[mt][j + 1]);
                lp[(j >> 1) & 3] += p0 + p1;
                const uint32_t pk = pack_f16(p0, p1);
                lhp[(j >> 1) & 1] =
                    __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones, lhp[(j >> 1) & 1], false);
                pw[mt * 2 + j / 8][(j % 8) / 2] = pk;
            }
        }
        l_run += (lp[0] + lp[1]) + (lp[2] + lp[3]);
        lh_run += lhp[0] + lhp[1];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 pB = __builtin_bit_cast(f16x8, make_uint4(pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]));
#pragma unroll
            for (int m = 0; m < NMD; ++m) {
                const uint16_t *src = &sm.vt[buf][(m * 32 + col) * VS + ((ks ^ (m & 3)) * 16 + hl * 4)];
                const uint2 lo = *reinterpret_cast<const uint2 *>(src);
                const uint2 hi = *reinterpret_cast<const uint2 *>(src + 8);
                o[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), pB, o[m], 0, 0, 0);
            }
        }
        // next tile into the other buffer: its last readers finished before the
        // barrier that ended the previous iteration
        if (tt + 1 < ntiles) stage_store<D>(sm, buf ^ 1, vr);
        __builtin_amdgcn_s_waitcnt(0);  // the next tile's K rows have landed in LDS
        __syncthreads();
    }

    // the two halves of a query's keys meet
    const float l_tot = half_pair_sum(l_run);
    const float lh_tot = half_pair_sum(lh_run);  // >= 1 once a key is visible (its max weighs 1)
    const float gs_tot = GSUM ? (HARD ? half_pair_sum(g_sum) : half_pair_sum(g_sum) * a.inv_c) : 0.f;
    if (qi < a.T_q) {
        const size_t uq = (size_t)bh * a.T_q + qi;
        const float inv = l_tot > 0.f ? 1.f / lh_tot : 0.f;
        float *orow = a.out + uq * D;
#pragma unroll
        for (int m = 0; m < NMD; ++m) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = m * 32 + gq * 8 + hl * 4;
                *reinterpret_cast<float4 *>(orow + d0) =
                    make_float4(o[m][4 * gq] * inv, o[m][4 * gq + 1] * inv, o[m][4 * gq + 2] * inv,
                                o[m][4 * gq + 3] * inv);
            }
        }
        if (hl == 0) {
            if (a.lse) a.lse[uq] = l_tot > 0.f ? (mref + __log2f(l_tot)) * kLn2 : -INFINITY;
            if (GSUM) a.gate_sum[uq] = gs_tot;
        }
    }
}

// Eq. 1 for every query token of a prefill: tau[b, h, t] = bias[h] + sum over the
// token's queries of all heads g and dimensions i of Q[b, g, t, i] * W[g*d + i, h].
// Workgroup = 64 consecutive tokens (one per lane) x 16 waves, up to 16 output
// heads per pass; wave w sums the query heads g = w, w + 16, ... . A row of W is
// the same for every lane of a wave: it is read through the scalar cache into
// scalar registers and enters the FMAs as their scalar operand, so each query
// element costs 16 FMAs and no LDS traffic or barrier. The sixteen partial sums
// meet in LDS and are added in wave order (fixed order, deterministic), wave k
// finishing output head k. Each lane reads its own token's query rows, 16 bytes
// at a time (one row per lane, rows 2d bytes apart).
constexpr int kTauTokens = 64;
constexpr int kTauWaves = 16;
constexpr int kTauHeads = 16;

// One query head g of a token against rows W[g*d .. g*d + d)[h0 .. h0 + 16): FULL
// when all 16 columns exist and the rows are 16-byte aligned (four 16-byte scalar
// loads per row); otherwise column by column, the missing ones skipped.
template <int D, bool FULL>
__device__ __forceinline__ void tau_rows(const uint16_t *__restrict__ qrow,
                                         const float *__restrict__ wg, int H, int nh,
                                         float (&acc)[kTauHeads]) {
    for (int i0 = 0; i0 < D; i0 += 8) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(qrow + i0);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float qv = (e & 1) ? bf16_hi(w4[e >> 1]) : bf16_lo(w4[e >> 1]);
            const float *wr = wg + (size_t)(i0 + e) * H;  // wave-uniform row
            if (FULL) {
#pragma unroll
                for (int k4 = 0; k4 < kTauHeads / 4; ++k4) {
                    const float4 w = reinterpret_cast<const float4 *>(wr)[k4];
                    acc[4 * k4] = fmaf(qv, w.x, acc[4 * k4]);
                    acc[4 * k4 + 1] = fmaf(qv, w.y, acc[4 * k4 + 1]);
                    acc[4 * k4 + 2] = fmaf(qv, w.z, acc[4 * k4 + 2]);
                    acc[4 * k4 + 3] = fmaf(qv, w.w, acc[4 * k4 + 3]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < kTauHeads; ++k) {
                    if (k < nh) acc[k] = fmaf(qv, wr[k], acc[k]);
                }
            }
            // one row's scalar registers at a time (scalar loads return out of order,
            // so rows loaded ahead would only hold registers)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kTauWaves *kWave) void prefill_tau_kernel(
    const uint16_t *__restrict__ Q, const float *__restrict__ W, const float *__restrict__ bias,
    float *__restrict__ tau, int H, int T, int wvec) {
    __shared__ float part[kTauWaves][kTauHeads][kTauTokens];
    const int b = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int tok = blockIdx.x * kTauTokens + lane;
    const int tc = min(tok, T - 1);
    for (int h0 = 0; h0 < H; h0 += kTauHeads) {
        const int nh = min(kTauHeads, H - h0);
        const bool full = nh == kTauHeads && wvec;
        float acc[kTauHeads];
#pragma unroll
        for (int k = 0; k < kTauHeads; ++k) acc[k] = 0.f;
        if (W != nullptr) {
            for (int g = wave; g < H; g += kTauWaves) {
                const uint16_t *qrow = Q + (((size_t)b * H + g) * T + tc) * D;
                const float *wg = W + (size_t)g * D * H + h0;
                if (full) {
                    tau_rows<D, true>(qrow, wg, H, nh, acc);
                } else {
                    tau_rows<D, false>(qrow, wg, H, nh, acc);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kTauHeads; ++k) part[wave][k][lane] = acc[k];
        __syncthreads();
        if (wave < nh && tok < T) {
            float sum = part[0][wave][lane];
#pragma unroll
            for (int w = 1; w < kTauWaves; ++w) sum += part[w][wave][lane];
            tau[((size_t)b * H + h0 + wave) * T + tok] = bias[h0 + wave] + sum;
        }
        __syncthreads();  // part is rewritten by the next pass
    }
}

template <int D, bool HARD>
void launch_prefill_g(const PfArgs &a, dim3 grid, hipStream_t st) {
    if (a.gate_sum != nullptr) {
        hipLaunchKernelGGL((prefill_attn_kernel<D, HARD, true>), grid, dim3(kPfWaves * kWave), 0, st, a);
    } else {
        hipLaunchKernelGGL((prefill_attn_kernel<D, HARD, false>), grid, dim3(kPfWaves * kWave), 0, st, a);
    }
}

template <int D>
hipError_t launch_prefill_t(const PrefillGeometry &g, const void *Q, const void *K, const void *V,
                            const float *tau, float gate_beta, bool hard, float *out, float *lse,
                            float *gate_sum, hipStream_t st) {
    PfArgs a;
    a.H = g.H;
    a.Hkv = g.Hkv;
    a.G = g.H / g.Hkv;
    a.T_q = g.T_q;
    a.T_k = g.T_k;
    a.q_off = g.T_k - g.T_q;
    a.s = 1.0f / sqrtf((float)D);
    a.c_gate = -gate_beta * kLog2e * a.s;
    a.c_soft = kLog2e * a.s;
    a.inv_c = 1.0f / a.c_soft;
    a.Q = static_cast<const uint16_t *>(Q);
    a.K = static_cast<const uint16_t *>(K);
    a.V = static_cast<const uint16_t *>(V);
    a.tau = tau;
    a.out = out;
    a.lse = lse;
    a.gate_sum = gate_sum;
    const dim3 grid((unsigned)(g.B * g.H), (unsigned)((g.T_q + kPfQ - 1) / kPfQ));
    if (hard) {
        launch_prefill_g<D, true>(a, grid, st);
    } else {
        launch_prefill_g<D, false>(a, grid, st);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_tau(const PrefillGeometry &g, const void *Q, const float *W,
                              const float *bias, float *tau, hipStream_t st) {
    if (g.T_q == 0) return hipSuccess;
    const dim3 grid((unsigned)((g.T_q + kTauTokens - 1) / kTauTokens), (unsigned)g.B);
    // 16-byte rows of W for the four-column loads: H a multiple of 4, W 16-byte aligned
    const int wvec = (g.H % 4 == 0 && (reinterpret_cast<uintptr_t>(W) % 16) == 0) ? 1 : 0;
    if (g.d == 128) {
        hipLaunchKernelGGL((prefill_tau_kernel<128>), grid, dim3(kTauWaves * kWave), 0, st,
                           static_cast<const uint16_t *>(Q), W, bias, tau, g.H, g.T_q, wvec);
    } else {
        hipLaunchKernelGGL((prefill_tau_kernel<64>), grid, dim3(kTauWaves * kWave), 0, st,
                           static_cast<const uint16_t *>(Q), W, bias, tau, g.H, g.T_q, wvec);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillGeometry &g, const void *Q, const void *K,
                               const void *V, const float *tau, float gate_beta, bool gate_hard,
                               float *out, float *lse, float *gate_sum, hipStream_t st) {
    if (g.T_q == 0) return hipSuccess;
    return g.d == 128 ? launch_prefill_t<128>(g, Q, K, V, tau, gate_beta, gate_hard, out, lse,
                                              gate_sum, st)
                      : launch_prefill_t<64>(g, Q, K, V, tau, gate_beta, gate_hard, out, lse,
                                             gate_sum, st);
}

}  // namespace eta
