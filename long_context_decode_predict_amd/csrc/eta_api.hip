// eta_api.hip -- the extern "C" boundary declared in include/eta.h.
//
// Every entry point validates its arguments on the host before anything is
// enqueued (no HIP call happens on an invalid call), maps launch failures to
// ETA_ERR_HIP, never allocates, frees or synchronises, and keeps no state.
#include "eta.h"

#include <math.h>

#include <mutex>

#include "eta_launch.hpp"

namespace {

constexpr int kBlock = 64;
// Default split-KV item: 8 admitted blocks per query head of the key/value
// unit, i.e. 8 * G (an item carries the state and partials of G heads, so its
// fixed cost grows with G and so should its length), doubled for caches of at
// least 2^20 unit blocks, where there are items enough to keep the grid busy
// with longer ones.
constexpr int kDefaultSplitPerHead = 8;
constexpr long long kLongItemSlots = 1ll << 20;
constexpr int kMaxSplit = 4096;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Per-unit capacity of the metadata, admitted-list and bound arrays.
int nblk_cap_of(int T_cap) { return (int)(ceil_div(ceil_div(T_cap, kBlock), 4) * 4); }

int kv_heads_of(const eta_shape *s) { return s->H_kv > 0 ? s->H_kv : s->H; }

eta_status check_shape(const eta_shape *s) {
    if (s == nullptr) return ETA_ERR_INVALID_ARG;
    if (s->B < 1 || s->H < 1 || s->T < 0 || s->T_cap < 1 || s->T > s->T_cap)
        return ETA_ERR_INVALID_ARG;
    if (s->T_cap % kBlock != 0) return ETA_ERR_INVALID_ARG;  // whole blocks of capacity
    if (s->d != 64 && s->d != 128) return ETA_ERR_UNSUPPORTED;
    if (s->block != kBlock) return ETA_ERR_UNSUPPORTED;
    if (s->kv_dtype != ETA_F32 && s->kv_dtype != ETA_BF16) return ETA_ERR_UNSUPPORTED;
    const long long units = (long long)s->B * s->H;
    if (units > (1ll << 24)) return ETA_ERR_INVALID_ARG;  // grid-size headroom
    if (s->H_kv < 0) return ETA_ERR_INVALID_ARG;
    if (s->H_kv > 0) {
        if (s->H % s->H_kv != 0) return ETA_ERR_INVALID_ARG;
        const int G = s->H / s->H_kv;
        if (G != 1 && G != 2 && G != 4 && G != 8) return ETA_ERR_UNSUPPORTED;
    }
    if (s->seq_lens != nullptr && !aligned(s->seq_lens, 4)) return ETA_ERR_INVALID_ARG;
    if (s->page_table != nullptr) {
        if (!aligned(s->page_table, 4) || s->num_pages < 1) return ETA_ERR_INVALID_ARG;
        // keeps every element offset of the pool far inside 64 bits
        if ((long long)s->num_pages * kv_heads_of(s) > (1ll << 31)) return ETA_ERR_INVALID_ARG;
    } else if (s->num_pages != 0) {
        return ETA_ERR_INVALID_ARG;
    }
    if (s->kv_block_stride < 0) return ETA_ERR_INVALID_ARG;
    if (s->kv_block_stride > 0 && s->kv_block_stride % (kBlock * s->d) != 0)
        return ETA_ERR_INVALID_ARG;
    return ETA_OK;
}

eta_status check_meta(const eta_shape *s, const eta_meta *m) {
    if (m == nullptr || m->centroid == nullptr || m->var == nullptr || m->maxnorm == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (m->nblk_cap != nblk_cap_of(s->T_cap)) return ETA_ERR_INVALID_ARG;
    if (!aligned(m->centroid, 16) || !aligned(m->var, 16) || !aligned(m->maxnorm, 16) ||
        !aligned(m->maxdev2, 16))
        return ETA_ERR_INVALID_ARG;
    return ETA_OK;
}

// What a screen call reads for the bound's second term: the centered bound is the
// combined formula with z = 1 over the squared largest distance from the centroid
// (s (q.c + |q| sqrt(maxdev2)), then the minimum with the max-norm bound).
struct BoundInputs {
    const float *spread;
    float z;
    bool geo_only;
};

eta_status bound_inputs(const eta_meta *m, const eta_params *p, BoundInputs *bi) {
    if (p->bound_mode == ETA_BOUND_CENTERED) {
        if (m->maxdev2 == nullptr) return ETA_ERR_INVALID_ARG;
        *bi = {m->maxdev2, 1.0f, false};
    } else {
        *bi = {m->var, p->z, p->bound_mode == ETA_BOUND_GEO};
    }
    return ETA_OK;
}

// Alignment the row loads need: one lane reads d/16 consecutive elements.
bool kv_aligned(const eta_shape *s, const void *p) {
    const size_t elem = s->kv_dtype == ETA_BF16 ? 2 : 4;
    return aligned(p, elem * (size_t)(s->d / 16) >= 16 ? 16 : 8);
}

eta::Geometry geometry(const eta_shape *s, int nblk_cap) {
    eta::Geometry g;
    g.units = s->B * s->H;
    g.kv_units = s->B * kv_heads_of(s);
    g.G = s->H / kv_heads_of(s);
    g.d = s->d;
    g.T = s->T;
    g.T_cap = s->T_cap;
    g.nblk = (int)ceil_div(s->T, kBlock);
    g.nblk_cap = nblk_cap;
    g.bf16 = s->kv_dtype == ETA_BF16;
    g.lay.seq_lens = s->seq_lens;
    g.lay.pages = s->page_table;
    g.lay.T = s->T;
    g.lay.T_cap = s->T_cap;
    g.lay.H_kv = kv_heads_of(s);
    g.lay.max_pages = s->T_cap / kBlock;
    g.lay.num_pages = s->page_table != nullptr ? s->num_pages : 0;
    g.lay.block_stride = s->kv_block_stride > 0 ? s->kv_block_stride : (long long)kBlock * s->d;
    return g;
}

eta_status check_params(const eta_params *p) {
    if (p == nullptr) return ETA_ERR_INVALID_ARG;
    if (!p->gate_hard && !(p->gate_beta > 0.f && isfinite(p->gate_beta))) return ETA_ERR_INVALID_ARG;
    if (!(p->z >= 0.f && isfinite(p->z))) return ETA_ERR_INVALID_ARG;
    if (p->bound_mode != ETA_BOUND_COMBINED && p->bound_mode != ETA_BOUND_GEO &&
        p->bound_mode != ETA_BOUND_CENTERED)
        return ETA_ERR_INVALID_ARG;
    if (p->split_blocks < 0 || p->split_blocks > kMaxSplit) return ETA_ERR_INVALID_ARG;
    return ETA_OK;
}

int split_of(const eta_shape *s, const eta_params *p) {
    if (p->split_blocks != 0) return p->split_blocks;
    const int hkv = kv_heads_of(s);
    const int G = (hkv > 0 && hkv < s->H) ? s->H / hkv : 1;
    const long long slots = (long long)s->B * hkv * nblk_cap_of(s->T_cap);
    return kDefaultSplitPerHead * G * (slots >= kLongItemSlots ? 2 : 1);
}

eta_status from_hip(hipError_t e) { return e == hipSuccess ? ETA_OK : ETA_ERR_HIP; }

// Shared validation of the attention calls; fills the geometry and item count.
eta_status check_attn(const eta_shape *s, const eta_params *p, const int32_t *adm_cnt,
                      const float *out, void *ws, size_t ws_bytes, eta::Geometry *g,
                      int *max_chunks) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (adm_cnt == nullptr || out == nullptr || !aligned(adm_cnt, 4)) return ETA_ERR_INVALID_ARG;
    const size_t need = eta_decode_attn_workspace_size(s, p);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return ETA_ERR_WORKSPACE;
    long long mc = ceil_div(ceil_div(s->T_cap, kBlock), split_of(s, p));
    if (mc < 1) mc = 1;
    if ((long long)s->B * s->H * mc > 0x7fffffffll) return ETA_ERR_INVALID_ARG;
    *g = geometry(s, nblk_cap_of(s->T_cap));
    *max_chunks = (int)mc;
    return ETA_OK;
}

// The attention operands other than the workspace (shape already checked).
eta_status check_attn_operands(const eta_shape *s, const float *q, const void *K, const void *V,
                               const float *tau, const int32_t *adm_idx) {
    if (q == nullptr || K == nullptr || V == nullptr || tau == nullptr || adm_idx == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (!kv_aligned(s, K) || !kv_aligned(s, V)) return ETA_ERR_INVALID_ARG;
    // read with scalar loads where the index is wave-uniform: whole words only
    if (!aligned(q, 4) || !aligned(tau, 4) || !aligned(adm_idx, 4)) return ETA_ERR_INVALID_ARG;
    // grouped heads with bf16 K read whole 16-byte chunks of every row (d = 64 too)
    const bool grouped = kv_heads_of(s) < s->H;
    if (grouped && s->kv_dtype == ETA_BF16 && !aligned(K, 16)) return ETA_ERR_INVALID_ARG;
    return ETA_OK;
}

// Workspace of eta_decode_attn_noalloc: one copy per GPU, in device memory the
// code object reserves when the library's kernels are loaded on that GPU. Host
// code never uses the array's name as an address (on the host it names a
// stand-in): every use goes through the device address looked up below.
static __device__ __align__(256) unsigned char scratch[ETA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_addr[kMaxDevices] = {};  // per device, looked up once

// The current device's address of `scratch` (looked up on first use, with that
// device current); `stream`, when non-null, must belong to the same device.
eta_status scratch_for_stream(hipStream_t stream, void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ETA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ETA_ERR_UNSUPPORTED;
    if (stream != nullptr) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ETA_ERR_HIP;
        if (sdev != dev) return ETA_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ETA_ERR_HIP;
        scratch_addr[dev] = p;
    }
    *ptr = scratch_addr[dev];
    return ETA_OK;
}

eta_status check_prefill(const eta_prefill_shape *s, eta::PrefillGeometry *g) {
    if (s == nullptr) return ETA_ERR_INVALID_ARG;
    if (s->B < 1 || s->H < 1 || s->T_q < 0 || s->T_k < s->T_q || s->H_kv < 0)
        return ETA_ERR_INVALID_ARG;
    if (s->d != 64 && s->d != 128) return ETA_ERR_UNSUPPORTED;
    if ((long long)s->B * s->H > (1ll << 24)) return ETA_ERR_INVALID_ARG;
    if ((long long)s->T_q > 65535ll * 128) return ETA_ERR_INVALID_ARG;  // query blocks on grid y
    const int hkv = s->H_kv > 0 ? s->H_kv : s->H;
    if (s->H % hkv != 0) return ETA_ERR_INVALID_ARG;
    const int G = s->H / hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return ETA_ERR_UNSUPPORTED;
    g->B = s->B;
    g->H = s->H;
    g->Hkv = hkv;
    g->d = s->d;
    g->T_q = s->T_q;
    g->T_k = s->T_k;
    return ETA_OK;
}

}  // namespace

extern "C" {

eta_params eta_default_params(void) {
    eta_params p;
    p.gate_beta = 5.0f;
    p.z = 4.0f;
    p.gate_hard = 0;
    p.bound_mode = ETA_BOUND_COMBINED;
    p.split_blocks = 0;
    return p;
}

int eta_nblk_cap(int T_cap) { return T_cap < 1 ? 0 : nblk_cap_of(T_cap); }

int eta_split_blocks(const eta_shape *s, const eta_params *p) {
    if (check_shape(s) != ETA_OK || p == nullptr || p->split_blocks < 0 ||
        p->split_blocks > kMaxSplit)
        return 0;
    return split_of(s, p);
}

const char *eta_status_string(eta_status st) {
    switch (st) {
        case ETA_OK: return "ETA_OK";
        case ETA_ERR_INVALID_ARG: return "ETA_ERR_INVALID_ARG";
        case ETA_ERR_UNSUPPORTED: return "ETA_ERR_UNSUPPORTED";
        case ETA_ERR_WORKSPACE: return "ETA_ERR_WORKSPACE";
        case ETA_ERR_HIP: return "ETA_ERR_HIP";
        case ETA_STATUS_MAX_ENUM: break;  // a range guard, not a status
    }
    return "ETA_ERR_UNKNOWN";
}

eta_status eta_build_block_meta(const eta_shape *s, const void *K, const eta_meta *m,
                                hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_meta(s, m)) != ETA_OK) return st;
    if (K == nullptr || !kv_aligned(s, K)) return ETA_ERR_INVALID_ARG;
    const eta::Geometry g = geometry(s, m->nblk_cap);
    return from_hip(eta::launch_block_meta(g, K, m->centroid, m->var, m->maxnorm, m->maxdev2, 0,
                                           g.nblk, 0, stream));
}

eta_status eta_append_meta(const eta_shape *s, int n_new, const void *K, const eta_meta *m,
                           hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_meta(s, m)) != ETA_OK) return st;
    if (K == nullptr || !kv_aligned(s, K)) return ETA_ERR_INVALID_ARG;
    if (n_new < 1 || (long long)s->T + n_new > s->T_cap) return ETA_ERR_INVALID_ARG;
    // the layout keeps the lengths before the append; each row's blocks from the one
    // holding its first new token through the one holding its last are rebuilt
    const eta::Geometry g = geometry(s, m->nblk_cap);
    return from_hip(eta::launch_block_meta(g, K, m->centroid, m->var, m->maxnorm, m->maxdev2, 0, 0,
                                           n_new, stream));
}

eta_status eta_predict_tau(int B, int H, int d, const float *q, const float *W,
                           const float *bias, float *tau, hipStream_t stream) {
    if (B < 1 || H < 1 || d < 1 || q == nullptr || bias == nullptr || tau == nullptr)
        return ETA_ERR_INVALID_ARG;
    if ((long long)H * d > (1ll << 30) || B > 65535 * 1024) return ETA_ERR_INVALID_ARG;
    if ((long long)H > 65535ll * 16) return ETA_ERR_INVALID_ARG;
    return from_hip(eta::launch_predict_tau(B, H, d, q, W, bias, tau, stream));
}

eta_status eta_screen(const eta_shape *s, const float *q, const float *tau, const eta_meta *m,
                      const eta_params *p, int32_t *adm_idx, int32_t *adm_cnt, float *bound_out,
                      hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_meta(s, m)) != ETA_OK) return st;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (q == nullptr || tau == nullptr || adm_idx == nullptr || adm_cnt == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (bound_out != nullptr && !aligned(bound_out, 16)) return ETA_ERR_INVALID_ARG;
    BoundInputs bi;
    if ((st = bound_inputs(m, p, &bi)) != ETA_OK) return st;
    const eta::Geometry g = geometry(s, m->nblk_cap);
    return from_hip(eta::launch_screen(g, s->H, q, const_cast<float *>(tau), nullptr, nullptr,
                                       false, m->centroid, bi.spread, m->maxnorm, bi.z,
                                       bi.geo_only, adm_idx, adm_cnt, bound_out, stream));
}

eta_status eta_predict_screen(const eta_shape *s, const float *q, const float *W,
                              const float *bias, const eta_meta *m, const eta_params *p,
                              float *tau, int32_t *adm_idx, int32_t *adm_cnt, float *bound_out,
                              hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_meta(s, m)) != ETA_OK) return st;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (q == nullptr || bias == nullptr || tau == nullptr || adm_idx == nullptr ||
        adm_cnt == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (bound_out != nullptr && !aligned(bound_out, 16)) return ETA_ERR_INVALID_ARG;
    BoundInputs bi;
    if ((st = bound_inputs(m, p, &bi)) != ETA_OK) return st;
    const eta::Geometry g = geometry(s, m->nblk_cap);
    return from_hip(eta::launch_screen(g, s->H, q, tau, W, bias, true, m->centroid, bi.spread,
                                       m->maxnorm, bi.z, bi.geo_only, adm_idx, adm_cnt, bound_out,
                                       stream));
}

eta_status eta_predict_screen_union(const eta_shape *s, const float *q, const float *W,
                                    const float *bias, const eta_meta *m, const eta_params *p,
                                    float *tau, int32_t *adm_idx, int32_t *adm_cnt,
                                    int32_t *uni_idx, int32_t *uni_cnt, float *bound_out,
                                    hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_meta(s, m)) != ETA_OK) return st;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (q == nullptr || bias == nullptr || tau == nullptr || adm_idx == nullptr ||
        adm_cnt == nullptr || uni_idx == nullptr || uni_cnt == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (kv_heads_of(s) == s->H) return ETA_ERR_INVALID_ARG;  // grouped heads only
    if (bound_out != nullptr && !aligned(bound_out, 16)) return ETA_ERR_INVALID_ARG;
    BoundInputs bi;
    if ((st = bound_inputs(m, p, &bi)) != ETA_OK) return st;
    const eta::Geometry g = geometry(s, m->nblk_cap);
    return from_hip(eta::launch_screen(g, s->H, q, tau, W, bias, true, m->centroid, bi.spread,
                                       m->maxnorm, bi.z, bi.geo_only, adm_idx, adm_cnt, bound_out,
                                       stream, uni_idx, uni_cnt));
}

eta_status eta_admit_union(const eta_shape *s, const int32_t *adm_idx, const int32_t *adm_cnt,
                           int32_t *uni_idx, int32_t *uni_cnt, hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if (adm_idx == nullptr || adm_cnt == nullptr || uni_idx == nullptr || uni_cnt == nullptr)
        return ETA_ERR_INVALID_ARG;
    const eta::Geometry g = geometry(s, nblk_cap_of(s->T_cap));
    return from_hip(eta::launch_union(g, adm_idx, adm_cnt, uni_idx, uni_cnt, stream));
}

size_t eta_decode_attn_workspace_size(const eta_shape *s, const eta_params *p) {
    if (check_shape(s) != ETA_OK || check_params(p) != ETA_OK) return 0;
    const int split = split_of(s, p);
    long long max_chunks = ceil_div(ceil_div(s->T_cap, kBlock), split);
    if (max_chunks < 1) max_chunks = 1;
    return eta::attn_workspace_layout(s->B * s->H, (int)max_chunks, s->d).bytes;
}

eta_status eta_decode_attn_partial(const eta_shape *s, const float *q, const void *K,
                                   const void *V, const float *tau, const int32_t *adm_idx,
                                   const int32_t *adm_cnt, const eta_params *p, float *out,
                                   float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    eta::Geometry g;
    int max_chunks = 0;
    eta_status st = check_attn(s, p, adm_cnt, out, ws, ws_bytes, &g, &max_chunks);
    if (st != ETA_OK) return st;
    if ((st = check_attn_operands(s, q, K, V, tau, adm_idx)) != ETA_OK) return st;
    return from_hip(eta::launch_attn_partial(g, q, K, V, tau, adm_idx, adm_cnt, p->gate_beta,
                                             p->gate_hard != 0, split_of(s, p), max_chunks, out, lse,
                                             ws, stream));
}

eta_status eta_decode_attn_combine(const eta_shape *s, const int32_t *adm_cnt,
                                   const eta_params *p, float *out, float *lse, void *ws,
                                   size_t ws_bytes, hipStream_t stream) {
    eta::Geometry g;
    int max_chunks = 0;
    eta_status st = check_attn(s, p, adm_cnt, out, ws, ws_bytes, &g, &max_chunks);
    if (st != ETA_OK) return st;
    return from_hip(eta::launch_attn_combine(g, adm_cnt, split_of(s, p), max_chunks, out, lse, ws,
                                             stream));
}

eta_status eta_decode_attn(const eta_shape *s, const float *q, const void *K, const void *V,
                           const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                           const eta_params *p, float *out, float *lse, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
    eta_status st = eta_decode_attn_partial(s, q, K, V, tau, adm_idx, adm_cnt, p, out, lse, ws,
                                            ws_bytes, stream);
    if (st != ETA_OK) return st;
    return eta_decode_attn_combine(s, adm_cnt, p, out, lse, ws, ws_bytes, stream);
}

eta_status eta_decode_attn_noalloc(const eta_shape *s, const float *q, const void *K,
                                   const void *V, const float *tau, const int32_t *adm_idx,
                                   const int32_t *adm_cnt, const eta_params *p, float *out,
                                   float *lse, hipStream_t stream) {
    eta_status st = check_shape(s);
    if (st != ETA_OK) return st;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (adm_cnt == nullptr || out == nullptr || !aligned(adm_cnt, 4)) return ETA_ERR_INVALID_ARG;
    if ((st = check_attn_operands(s, q, K, V, tau, adm_idx)) != ETA_OK) return st;
    if (eta_decode_attn_workspace_size(s, p) > ETA_NOALLOC_SCRATCH_BYTES) return ETA_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((st = scratch_for_stream(stream, &ws)) != ETA_OK) return st;
    return eta_decode_attn(s, q, K, V, tau, adm_idx, adm_cnt, p, out, lse, ws,
                           ETA_NOALLOC_SCRATCH_BYTES, stream);
}

eta_status eta_prefill_predict_tau(const eta_prefill_shape *s, const void *Q, const float *W,
                                   const float *bias, float *tau, hipStream_t stream) {
    eta::PrefillGeometry g;
    eta_status st = check_prefill(s, &g);
    if (st != ETA_OK) return st;
    if (Q == nullptr || bias == nullptr || tau == nullptr || !aligned(Q, 16))
        return ETA_ERR_INVALID_ARG;
    return from_hip(eta::launch_prefill_tau(g, Q, W, bias, tau, stream));
}

eta_status eta_prefill_attn(const eta_prefill_shape *s, const void *Q, const void *K,
                            const void *V, const float *tau, const eta_params *p, float *out,
                            float *lse, float *gate_sum, hipStream_t stream) {
    eta::PrefillGeometry g;
    eta_status st = check_prefill(s, &g);
    if (st != ETA_OK) return st;
    // the forward addresses one (row, key/value head) slab of K or V through a
    // buffer resource with a 31-bit byte range
    if ((long long)s->T_k * s->d * 2 >= (1ll << 31)) return ETA_ERR_INVALID_ARG;
    if ((st = check_params(p)) != ETA_OK) return st;
    if (Q == nullptr || K == nullptr || V == nullptr || tau == nullptr || out == nullptr)
        return ETA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16))
        return ETA_ERR_INVALID_ARG;
    return from_hip(eta::launch_prefill_attn(g, Q, K, V, tau, p->gate_beta, p->gate_hard != 0,
                                             out, lse, gate_sum, stream));
}

}  // extern "C"
