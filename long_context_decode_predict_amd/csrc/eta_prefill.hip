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
// for |v| in [2^-14, 65504]); P in fp16 keeps 11 significant bits.
//
// Workgroup = 4 waves = 128 consecutive queries of one (row, head); wave w owns
// queries 32w .. 32w + 31. Key tiles of 64 are staged into LDS (K row-major,
// V^T), the next tile's global loads are in flight while the current one is
// computed. Causal: query i sits at position T_k - T_q + i and sees keys at or
// before it. Grid x = (row, head), y = query block, heaviest blocks first; all
// query blocks of one head share an XCD when B * H is a multiple of 8.
#include "eta_device.hpp"
#include "eta_launch.hpp"

namespace eta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 4;
constexpr int kPfQ = 32 * kPfWaves;  // queries per workgroup
constexpr int kPfKeys = 64;          // keys per tile

template <int D>
struct PfShared {
    static constexpr int KS = D + 8;        // bf16 per K row (16 bytes of padding)
    static constexpr int VS = kPfKeys + 4;  // fp16 per V^T row (8 bytes of padding)
    // V^T row r keeps key k at column k ^ swz(r): 16-key groups are permuted by the
    // row's 32-dimension tile, so the transposing writes (8 bytes per lane, rows
    // 8 apart across lanes) spread over the banks; a reading wave works on one
    // 32-row tile at a time, so its reads are only shifted.
    alignas(16) uint16_t k[2][kPfKeys * KS];  // double buffered: one barrier per tile
    alignas(16) uint16_t vt[2][D * VS];
};

struct PfArgs {
    int H, Hkv, G, T_q, T_k, q_off;
    float s, c_gate, c_soft;  // 1/sqrt(d), -beta*log2(e)/sqrt(d), log2(e)/sqrt(d)
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

// Two floats to packed fp16 (exact for values representable in fp16).
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

// Key swizzle of V^T row r (see PfShared): flips the 16-key group by r / 32.
__device__ __forceinline__ int vt_swz(int r) { return ((r >> 5) & 3) << 4; }

template <int D>
__device__ __forceinline__ void stage_load(const PfArgs &a, const uint16_t *Kh, const uint16_t *Vh,
                                           int k0, uint4 (&kr)[StageShape<D>::KLD],
                                           uint4 (&vr)[StageShape<D>::KPT]) {
    using S = StageShape<D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
        const int c = tid + i * kPfWaves * kWave;
        const int row = min(k0 + c / S::KCH, a.T_k - 1);  // rows past T_k: clamped, masked later
        kr[i] = *reinterpret_cast<const uint4 *>(Kh + (size_t)row * D + (c % S::KCH) * 8);
    }
    const int ka = tid / S::KCH;  // key group
    const int db = tid % S::KCH;  // 8-dimension chunk
#pragma unroll
    for (int r = 0; r < S::KPT; ++r) {
        const int row = min(k0 + ka * S::KPT + r, a.T_k - 1);
        vr[r] = *reinterpret_cast<const uint4 *>(Vh + (size_t)row * D + db * 8);
    }
}

template <int D>
__device__ __forceinline__ void stage_store(PfShared<D> &sm, int buf,
                                            const uint4 (&kr)[StageShape<D>::KLD],
                                            const uint4 (&vr)[StageShape<D>::KPT]) {
    using S = StageShape<D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
        const int c = tid + i * kPfWaves * kWave;
        *reinterpret_cast<uint4 *>(&sm.k[buf][(c / S::KCH) * PfShared<D>::KS + (c % S::KCH) * 8]) =
            kr[i];
    }
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

// Gate, mask and tile maximum of one lane's 32 scores (acc = q.k, unscaled).
// Returns the gated values in acc units (the 1/sqrt(d) scale is folded into
// the exponent constants, and a positive scale keeps the order).
template <bool HARD, bool GSUM, bool MASK>
__device__ __forceinline__ float gate_tile(const PfArgs &a, const float (&acc)[2][16], float t_acc,
                                           float nbt, int lim, float (&g)[2][16], float &g_sum) {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float x = acc[mt][j];
            float gv, gate = 0.f;
            if (HARD) {
                const bool on = x >= t_acc;
                gv = on ? x : 0.f;
                if (GSUM) gate = on ? 1.f : 0.f;
            } else {
                const float m = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(a.c_gate, x, nbt)));
                gv = x * m;
                if (GSUM) gate = m;
            }
            if (MASK) {
                const int off = mt * 32 + (j >> 2) * 8 + (j & 3);  // key offset minus 4*hl
                if (off > lim) {
                    gv = -INFINITY;
                    gate = 0.f;
                }
            }
            if (GSUM) g_sum += gate;
            g[mt][j] = gv;
            mx = fmaxf(mx, gv);
        }
    }
    return mx;
}

template <int D, bool HARD, bool GSUM>
__global__ __launch_bounds__(kPfWaves *kWave, 2) void prefill_attn_kernel(PfArgs a) {
    __shared__ PfShared<D> sm;
    constexpr int KS = PfShared<D>::KS;
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
    float m_run = -INFINITY, l_run = 0.f, g_sum = 0.f;  // m_run in acc units

    uint4 kr[StageShape<D>::KLD], vr[StageShape<D>::KPT];
    stage_load<D>(a, Kh, Vh, 0, kr, vr);
    stage_store<D>(sm, 0, kr, vr);
    __syncthreads();
    for (int tt = 0; tt < ntiles; ++tt) {
        const int k0 = tt * kPfKeys;
        const int buf = tt & 1;
        // the next tile's loads are in flight during this one (issued unconditionally:
        // rows are clamped, so the load past the last tile stays in bounds and keeps
        // the staging registers out of scratch memory)
        stage_load<D>(a, Kh, Vh, k0 + kPfKeys, kr, vr);

        // S^T for keys k0 .. k0 + 63 (two 32-key tiles) against the wave's 32 queries
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(
                    &sm.k[buf][(mt * 32 + col) * KS + ks * 16 + hl * 8]);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw),
                                                                qB[ks], s[mt], 0, 0, 0);
            }
        }
        float acc[2][16];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][j] = s[mt][j];

        // gate, causal mask (diagonal and last tiles only), tile maximum
        float g[2][16];
        float mx;
        if (k0 + kPfKeys - 1 > wave_first_pos || k0 + kPfKeys > a.T_k) {
            mx = gate_tile<HARD, GSUM, true>(a, acc, t_acc, nbt, qpos - k0 - hl * 4, g, g_sum);
        } else {
            mx = gate_tile<HARD, GSUM, false>(a, acc, t_acc, nbt, 0, g, g_sum);
        }
        mx = half_pair_max(mx);  // the partner lane l ^ 32 holds the other 32 keys
        const float m_new = fmaxf(m_run, mx);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // nothing visible yet: weights 0
        const float corr = __builtin_amdgcn_exp2f((m_run - m_ref) * a.c_soft);
        m_run = m_new;
        l_run *= corr;
        if (__any(corr != 1.f)) {  // the running maximum moved for some query of the wave
#pragma unroll
            for (int m = 0; m < NMD; ++m) o[m] *= corr;
        }

        // weights, packed as the fp16 B operand of O^T += V^T P^T: k-step s (keys
        // 16s .. 16s + 15) takes registers 8(s%2) .. 8(s%2) + 7 of key tile s/2
        const float mref_c = m_ref * a.c_soft;
        uint32_t pw[4][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(g[mt][j], a.c_soft, -mref_c));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(g[mt][j + 1], a.c_soft, -mref_c));
                l_run += p0 + p1;
                pw[mt * 2 + j / 8][(j % 8) / 2] = pack_f16(p0, p1);
            }
        }
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
        if (tt + 1 < ntiles) stage_store<D>(sm, buf ^ 1, kr, vr);
        __syncthreads();
    }

    // the two halves of a query's keys meet
    const float l_tot = half_pair_sum(l_run);
    const float gs_tot = GSUM ? half_pair_sum(g_sum) : 0.f;
    if (qi < a.T_q) {
        const size_t uq = (size_t)bh * a.T_q + qi;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
            if (a.lse) a.lse[uq] = l_tot > 0.f ? a.s * m_run + __logf(l_tot) : -INFINITY;
            if (GSUM) a.gate_sum[uq] = gs_tot;
        }
    }
}

// Eq. 1 for every query token of a prefill: tau[b, h, t] = bias[h] + sum over the
// token's queries of all heads g and dimensions i of Q[b, g, t, i] * W[g*d + i, h].
// Workgroup = 64 consecutive tokens (one per lane) x up to 16 heads per pass;
// wave w sums the query heads g = w, w + 4, ... . In each round the workgroup
// stages the four W slices W[g*d .. g*d + d)[h0 .. h0 + 16) in LDS; a wave reads
// its slice with broadcast loads (the same address in every lane) and every
// lane does 16 FMAs per query element. The four partial sums meet in LDS and
// are added in wave order (fixed order, deterministic).
constexpr int kTauTokens = 64;
constexpr int kTauWaves = 4;
constexpr int kTauHeads = 16;

template <int D>
__global__ __launch_bounds__(kTauWaves *kWave) void prefill_tau_kernel(
    const uint16_t *__restrict__ Q, const float *__restrict__ W, const float *__restrict__ bias,
    float *__restrict__ tau, int H, int T, int vec) {
    __shared__ float4 wsl[kTauWaves][D][kTauHeads / 4];
    __shared__ float part[kTauWaves][kTauHeads][kTauTokens];
    const int b = blockIdx.y;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int tok = blockIdx.x * kTauTokens + lane;
    const int tc = min(tok, T - 1);
    for (int h0 = 0; h0 < H; h0 += kTauHeads) {
        float acc[kTauHeads];
#pragma unroll
        for (int k = 0; k < kTauHeads; ++k) acc[k] = 0.f;
        if (W != nullptr) {
            for (int g0 = 0; g0 < H; g0 += kTauWaves) {
                __syncthreads();  // the previous round's slices are consumed
                // stage W[(g0 + w)*d + i][h0 .. h0 + 16) for w < 4, i < d (zeros outside)
                for (int c = threadIdx.x; c < kTauWaves * D * (kTauHeads / 4); c += kTauWaves * kWave) {
                    const int w = c / (D * (kTauHeads / 4));
                    const int i = (c / (kTauHeads / 4)) % D;
                    const int q4 = c % (kTauHeads / 4);
                    const int g = g0 + w;
                    const int h = h0 + q4 * 4;
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (g < H) {
                        const float *src = W + (size_t)(g * D + i) * H + h;
                        if (vec && h + 4 <= H) {
                            v = *reinterpret_cast<const float4 *>(src);
                        } else {
                            v.x = h < H ? src[0] : 0.f;
                            v.y = h + 1 < H ? src[1] : 0.f;
                            v.z = h + 2 < H ? src[2] : 0.f;
                            v.w = h + 3 < H ? src[3] : 0.f;
                        }
                    }
                    wsl[w][i][q4] = v;
                }
                __syncthreads();
                const int g = g0 + wave;
                if (g < H) {
                    const uint16_t *qrow = Q + (((size_t)b * H + g) * T + tc) * D;
                    for (int i0 = 0; i0 < D; i0 += 8) {
                        const uint4 raw = *reinterpret_cast<const uint4 *>(qrow + i0);
                        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float qv = (e & 1) ? bf16_hi(w4[e >> 1]) : bf16_lo(w4[e >> 1]);
#pragma unroll
                            for (int q4 = 0; q4 < kTauHeads / 4; ++q4) {
                                const float4 wv = wsl[wave][i0 + e][q4];
                                acc[4 * q4] = fmaf(qv, wv.x, acc[4 * q4]);
                                acc[4 * q4 + 1] = fmaf(qv, wv.y, acc[4 * q4 + 1]);
                                acc[4 * q4 + 2] = fmaf(qv, wv.z, acc[4 * q4 + 2]);
                                acc[4 * q4 + 3] = fmaf(qv, wv.w, acc[4 * q4 + 3]);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kTauHeads; ++k) part[wave][k][lane] = acc[k];
        __syncthreads();
        if (wave == 0 && tok < T) {
#pragma unroll
            for (int k = 0; k < kTauHeads; ++k) {
                if (h0 + k < H) {
                    const float sum = ((part[0][k][lane] + part[1][k][lane]) + part[2][k][lane]) +
                                      part[3][k][lane];
                    tau[((size_t)b * H + h0 + k) * T + tok] = bias[h0 + k] + sum;
                }
            }
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
    // float4 slices of W rows need 16-byte aligned rows
    const int vec = (g.H % 4 == 0 && (reinterpret_cast<uintptr_t>(W) % 16) == 0) ? 1 : 0;
    if (g.d == 128) {
        hipLaunchKernelGGL((prefill_tau_kernel<128>), grid, dim3(kTauWaves * kWave), 0, st,
                           static_cast<const uint16_t *>(Q), W, bias, tau, g.H, g.T_q, vec);
    } else {
        hipLaunchKernelGGL((prefill_tau_kernel<64>), grid, dim3(kTauWaves * kWave), 0, st,
                           static_cast<const uint16_t *>(Q), W, bias, tau, g.H, g.T_q, vec);
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
