"""ctypes binding of ``libeta.so`` (the C ABI in ``include/eta.h``).

Argument marshalling only: every function checks the torch tensors it is
handed (device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C function of the same name, and raises ``EtaError``
on a non-OK status. All arithmetic runs in the library's HIP kernels; there is
no fallback, and loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

from .build import LIB_PATH

ETA_OK = 0
ETA_ERR_INVALID_ARG = -1
ETA_ERR_UNSUPPORTED = -2
ETA_ERR_WORKSPACE = -3
ETA_ERR_HIP = -4

ETA_F32 = 0
ETA_BF16 = 1
ETA_BOUND_COMBINED = 0
ETA_BOUND_GEO = 1
ETA_BOUND_CENTERED = 2
BLOCK = 64


class EtaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class eta_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int),
                ("T", ctypes.c_int), ("T_cap", ctypes.c_int), ("block", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("H_kv", ctypes.c_int),
                ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("num_pages", ctypes.c_int), ("kv_block_stride", ctypes.c_int)]


class eta_meta(ctypes.Structure):
    _fields_ = [("centroid", ctypes.c_void_p), ("var", ctypes.c_void_p),
                ("maxnorm", ctypes.c_void_p), ("nblk_cap", ctypes.c_int),
                ("maxdev2", ctypes.c_void_p)]


class eta_prefill_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int),
                ("d", ctypes.c_int), ("T_q", ctypes.c_int), ("T_k", ctypes.c_int)]


class eta_params(ctypes.Structure):
    _fields_ = [("gate_beta", ctypes.c_float), ("z", ctypes.c_float),
                ("gate_hard", ctypes.c_int), ("bound_mode", ctypes.c_int),
                ("split_blocks", ctypes.c_int)]


_P = ctypes.POINTER
_vp = ctypes.c_void_p
_lib = None

# (restype, argtypes) of every exported symbol of include/eta.h
SIGNATURES = {
    "eta_default_params": (eta_params, []),
    "eta_nblk_cap": (ctypes.c_int, [ctypes.c_int]),
    "eta_split_blocks": (ctypes.c_int, [_P(eta_shape), _P(eta_params)]),
    "eta_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "eta_build_block_meta": (ctypes.c_int, [_P(eta_shape), _vp, _P(eta_meta), _vp]),
    "eta_append_meta": (ctypes.c_int, [_P(eta_shape), ctypes.c_int, _vp, _P(eta_meta), _vp]),
    "eta_predict_tau": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp,
                                       _vp, _vp]),
    "eta_screen": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _P(eta_meta), _P(eta_params), _vp,
                                  _vp, _vp, _vp]),
    "eta_predict_screen": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _P(eta_meta),
                                          _P(eta_params), _vp, _vp, _vp, _vp, _vp]),
    "eta_admit_union": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _vp, _vp]),
    "eta_predict_screen_union": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _P(eta_meta),
                                                _P(eta_params), _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp]),
    "eta_decode_attn_workspace_size": (ctypes.c_size_t, [_P(eta_shape), _P(eta_params)]),
    "eta_decode_attn": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _vp, _vp, _vp,
                                       _P(eta_params), _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "eta_decode_attn_partial": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _vp, _vp, _vp,
                                               _P(eta_params), _vp, _vp, _vp, ctypes.c_size_t,
                                               _vp]),
    "eta_decode_attn_combine": (ctypes.c_int, [_P(eta_shape), _vp, _P(eta_params), _vp, _vp, _vp,
                                               ctypes.c_size_t, _vp]),
    "eta_decode_attn_noalloc": (ctypes.c_int, [_P(eta_shape), _vp, _vp, _vp, _vp, _vp, _vp,
                                               _P(eta_params), _vp, _vp, _vp]),
    "eta_prefill_predict_tau": (ctypes.c_int, [_P(eta_prefill_shape), _vp, _vp, _vp, _vp, _vp]),
    "eta_prefill_attn": (ctypes.c_int, [_P(eta_prefill_shape), _vp, _vp, _vp, _vp,
                                        _P(eta_params), _vp, _vp, _vp, _vp]),
}


def lib_path() -> str:
    """The library to load: ``libeta.so`` in the package, or another build of the same
    sources named by ETA_LIB_PATH (a host-instrumented one, for instance)."""
    return os.environ.get("ETA_LIB_PATH") or LIB_PATH


def lib() -> ctypes.CDLL:
    """Load ``libeta.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "long_context_decode_predict_amd.build.build_lib()")
        L = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().eta_status_string(st).decode()


def _check(fn: str, st: int):
    if st != ETA_OK:
        raise EtaError(fn, st, status_string(st))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kv_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return ETA_BF16
    if dtype == torch.float32:
        return ETA_F32
    raise ValueError(f"K/V dtype must be bfloat16 or float32, got {dtype}")


def nblk_cap(T_cap: int) -> int:
    return int(lib().eta_nblk_cap(int(T_cap)))


def split_blocks(B: int, H: int, H_kv: int, T_cap: int, params: "eta_params") -> int:
    """The split-KV item length the library uses (eta_split_blocks)."""
    s = eta_shape(int(B), int(H), 128, 0, int(T_cap), BLOCK, 1, int(H_kv))
    return int(lib().eta_split_blocks(ctypes.byref(s), ctypes.byref(params)))


@dataclass
class KVLayout:
    """Paged and/or variable-length cache (the optional fields of eta_shape).

    seq_lens: int32 [B] tokens present in each row (each <= the call's T), or None.
    page_table: int32 [B, T_cap/64] page of each logical block, or None; with it K
    and V are pools [num_pages, H_kv, 64, d] instead of [B, H_kv, T_cap, d].
    """
    seq_lens: torch.Tensor | None = None
    page_table: torch.Tensor | None = None

    @property
    def paged(self) -> bool:
        return self.page_table is not None


def make_shape(B, H, d, T, T_cap, kv_dtype: torch.dtype, H_kv: int = 0,
               layout: KVLayout | None = None, num_pages: int = 0,
               block_stride: int = 0) -> eta_shape:
    s = eta_shape(int(B), int(H), int(d), int(T), int(T_cap), BLOCK, kv_code(kv_dtype),
                  int(H_kv))
    s.kv_block_stride = int(block_stride)
    if layout is not None:
        if layout.seq_lens is not None:
            _need(layout.seq_lens, "seq_lens", torch.int32, (B,))
            s.seq_lens = layout.seq_lens.data_ptr()
        if layout.page_table is not None:
            _need(layout.page_table, "page_table", torch.int32, (B, T_cap // BLOCK))
            s.page_table = layout.page_table.data_ptr()
            s.num_pages = int(num_pages)
    return s


def kv_block_view(K: torch.Tensor) -> bool:
    """True for a dense cache given block by block: a 5-d view [B, H_kv, T_cap/64, 64, d]
    whose 64-row blocks lie K.stride(2) elements apart (for example K = kv[..., 0, :, :]
    and V = kv[..., 1, :, :] of kv [B, H_kv, T_cap/64, 2, 64, d], K and V interleaved
    block by block in one allocation)."""
    return K.dim() == 5


def kv_pool_view(K: torch.Tensor) -> bool:
    """True for a page pool given as a strided 4-d view [P, H_kv, 64, d] whose 64-row
    blocks lie K.stride(1) elements apart (for example K = pool[:, :, 0] and
    V = pool[:, :, 1] of pool [P, H_kv, 2, 64, d], K and V interleaved block by block);
    a contiguous 4-d tensor is a dense cache or a plain pool."""
    return K.dim() == 4 and not K.is_contiguous()


def kv_block_stride(K: torch.Tensor) -> int:
    """eta_shape.kv_block_stride of a K/V tensor: 0 for a contiguous 4-d cache or pool."""
    if kv_block_view(K):
        return int(K.stride(2))
    return int(K.stride(1)) if kv_pool_view(K) else 0


def kv_dims(K: torch.Tensor, layout: KVLayout | None = None):
    """(B, H_kv, T_cap, d, num_pages) of a dense [B,H_kv,T_cap,d] cache (or its 5-d block
    view, see kv_block_view), or of a page pool [num_pages,H_kv,64,d] addressed through
    layout.page_table [B, T_cap/64]."""
    if kv_block_view(K):
        if layout is not None and layout.paged:
            raise ValueError("a block view of K/V is a dense layout; a page pool is 4-d")
        B, H_kv, nb, blk, d = K.shape
        return B, H_kv, nb * blk, d, 0
    if K.dim() != 4:
        raise ValueError("K/V must be 4-d: [B,H_kv,T_cap,d] or a page pool [P,H_kv,64,d]")
    if kv_pool_view(K) and (layout is None or not layout.paged):
        raise ValueError("a strided 4-d K/V is a page-pool view; a dense cache given "
                         "block by block is 5-d")
    if layout is not None and layout.paged:
        P, H_kv, blk, d = K.shape
        if blk != BLOCK:
            raise ValueError(f"a page holds {BLOCK} tokens, got {blk}")
        if layout.page_table.dim() != 2:
            raise ValueError("page_table must be [B, T_cap/64]")
        B, mp = layout.page_table.shape
        return B, H_kv, mp * BLOCK, d, P
    B, H_kv, T_cap, d = K.shape
    return B, H_kv, T_cap, d, 0


def shape_of(K: torch.Tensor, T: int, layout: KVLayout | None = None) -> eta_shape:
    """Shape descriptor of a multi-head K/V cache holding T tokens."""
    B, H, T_cap, d, P = kv_dims(K, layout)
    return make_shape(B, H, d, T, T_cap, K.dtype, 0, layout, P, kv_block_stride(K))


def default_params(**kw) -> eta_params:
    p = lib().eta_default_params()
    for k, v in kw.items():
        if not hasattr(p, k):
            raise KeyError(k)
        setattr(p, k, v)
    return p


@dataclass
class Meta:
    """Device buffers of the cached block metadata for one [B,H,T_cap,d] cache."""
    centroid: torch.Tensor  # [B,H,d,nblk_cap] float32
    var: torch.Tensor       # [B,H,nblk_cap] float32
    maxnorm: torch.Tensor   # [B,H,nblk_cap] float32
    nblk_cap: int
    maxdev2: Optional[torch.Tensor] = None  # [B,H,nblk_cap] float32, for the centered bound

    @staticmethod
    def alloc(B, H, d, T_cap, device="cuda", centered: bool = False) -> "Meta":
        n = nblk_cap(T_cap)
        return Meta(torch.empty((B, H, d, n), dtype=torch.float32, device=device),
                    torch.empty((B, H, n), dtype=torch.float32, device=device),
                    torch.empty((B, H, n), dtype=torch.float32, device=device), n,
                    torch.empty((B, H, n), dtype=torch.float32, device=device)
                    if centered else None)

    def c(self) -> eta_meta:
        return eta_meta(self.centroid.data_ptr(), self.var.data_ptr(), self.maxnorm.data_ptr(),
                        self.nblk_cap,
                        self.maxdev2.data_ptr() if self.maxdev2 is not None else None)


def _check_meta(meta: Meta, B, H, d, T_cap):
    n = nblk_cap(T_cap)
    _need(meta.centroid, "centroid", torch.float32, (B, H, d, n))
    _need(meta.var, "var", torch.float32, (B, H, n))
    _need(meta.maxnorm, "maxnorm", torch.float32, (B, H, n))
    if meta.maxdev2 is not None:
        _need(meta.maxdev2, "maxdev2", torch.float32, (B, H, n))


def _check_kv(K: torch.Tensor, name="K"):
    if kv_block_view(K):
        # [B, H_kv, nblk, 64, d]: rows of a block back to back, blocks of a unit S apart
        # (S a positive multiple of 64*d), units nblk*S apart
        B, H_kv, nb, blk, d = K.shape
        S = K.stride(2)
        if blk != BLOCK or K.stride(3) != d or K.stride(4) != 1 or S <= 0 \
                or S % (BLOCK * d) != 0 or K.stride(1) != nb * S or K.stride(0) != H_kv * nb * S:
            raise ValueError(f"{name} as a block view must be [B,H_kv,T_cap/64,64,d] with "
                             "blocks a multiple of 64*d elements apart and units packed")
        _need(K[0, 0, 0], name)  # device tensor
        kv_code(K.dtype)
        return
    if K.dim() != 4:
        raise ValueError(f"{name} must be [B,H,T_cap,d] (or its block view)")
    if kv_pool_view(K):
        # [P, H_kv, 64, d]: rows of a block back to back, blocks S apart (a positive
        # multiple of 64*d), pages H_kv*S apart
        P, H_kv, blk, d = K.shape
        S = K.stride(1)
        if blk != BLOCK or K.stride(2) != d or K.stride(3) != 1 or S <= 0 \
                or S % (BLOCK * d) != 0 or K.stride(0) != H_kv * S:
            raise ValueError(f"{name} as a pool view must be [P,H_kv,64,d] with blocks a "
                             "multiple of 64*d elements apart and pages packed")
        _need(K[0, 0], name)  # device tensor
        kv_code(K.dtype)
        return
    _need(K, name)
    kv_code(K.dtype)


# ------------------------------------------------------------------------------------
# The C entry points, same names
# ------------------------------------------------------------------------------------
def eta_build_block_meta(K: torch.Tensor, T: int, meta: Meta, stream=None,
                         layout: KVLayout | None = None):
    _check_kv(K)
    s = shape_of(K, T, layout)
    _check_meta(meta, s.B, s.H, s.d, s.T_cap)
    m = meta.c()
    _check("eta_build_block_meta",
           lib().eta_build_block_meta(ctypes.byref(s), K.data_ptr(), ctypes.byref(m), _stream(stream)))


def eta_append_meta(K: torch.Tensor, T_old: int, n_new: int, meta: Meta, stream=None,
                    layout: KVLayout | None = None):
    """With layout.seq_lens, those are the lengths before the append (T_old their
    maximum) and every row receives n_new tokens."""
    _check_kv(K)
    s = shape_of(K, T_old, layout)
    _check_meta(meta, s.B, s.H, s.d, s.T_cap)
    m = meta.c()
    _check("eta_append_meta",
           lib().eta_append_meta(ctypes.byref(s), int(n_new), K.data_ptr(), ctypes.byref(m),
                                 _stream(stream)))


def eta_predict_tau(q: torch.Tensor, W, bias: torch.Tensor, tau: torch.Tensor, stream=None):
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d]")
    B, H, d = q.shape
    _need(q, "q", torch.float32)
    if W is not None:
        _need(W, "W", torch.float32, (H * d, H))
    _need(bias, "bias", torch.float32, (H,))
    _need(tau, "tau", torch.float32, (B, H))
    _check("eta_predict_tau",
           lib().eta_predict_tau(B, H, d, q.data_ptr(), _ptr(W), bias.data_ptr(), tau.data_ptr(),
                                 _stream(stream)))


def eta_screen(q: torch.Tensor, tau: torch.Tensor, meta: Meta, T: int, T_cap: int,
               params: eta_params, adm_idx: torch.Tensor, adm_cnt: torch.Tensor,
               bound_out=None, kv_dtype=torch.bfloat16, stream=None, H_kv: int = 0,
               layout: KVLayout | None = None):
    """Per query head lists; with grouped heads (H_kv < H) each query head screens
    the metadata of its key/value head. Only layout.seq_lens matters here."""
    B, H, d = q.shape
    s = make_shape(B, H, d, T, T_cap, kv_dtype, H_kv, _lens_only(layout))
    n = nblk_cap(T_cap)
    _need(q, "q", torch.float32)
    _need(tau, "tau", torch.float32, (B, H))
    _check_meta(meta, B, H_kv or H, d, T_cap)
    _need(adm_idx, "adm_idx", torch.int32, (B, H, n))
    _need(adm_cnt, "adm_cnt", torch.int32, (B, H))
    if bound_out is not None:
        _need(bound_out, "bound_out", torch.float32, (B, H, n))
    m = meta.c()
    _check("eta_screen",
           lib().eta_screen(ctypes.byref(s), q.data_ptr(), tau.data_ptr(), ctypes.byref(m),
                            ctypes.byref(params), adm_idx.data_ptr(), adm_cnt.data_ptr(),
                            _ptr(bound_out), _stream(stream)))


def eta_predict_screen(q: torch.Tensor, W, bias: torch.Tensor, meta: Meta, T: int, T_cap: int,
                       params: eta_params, tau: torch.Tensor, adm_idx: torch.Tensor,
                       adm_cnt: torch.Tensor, bound_out=None, kv_dtype=torch.bfloat16,
                       stream=None, H_kv: int = 0, layout: KVLayout | None = None):
    B, H, d = q.shape
    s = make_shape(B, H, d, T, T_cap, kv_dtype, H_kv, _lens_only(layout))
    n = nblk_cap(T_cap)
    _need(q, "q", torch.float32)
    if W is not None:
        _need(W, "W", torch.float32, (H * d, H))
    _need(bias, "bias", torch.float32, (H,))
    _need(tau, "tau", torch.float32, (B, H))
    _check_meta(meta, B, H_kv or H, d, T_cap)
    _need(adm_idx, "adm_idx", torch.int32, (B, H, n))
    _need(adm_cnt, "adm_cnt", torch.int32, (B, H))
    if bound_out is not None:
        _need(bound_out, "bound_out", torch.float32, (B, H, n))
    m = meta.c()
    _check("eta_predict_screen",
           lib().eta_predict_screen(ctypes.byref(s), q.data_ptr(), _ptr(W), bias.data_ptr(),
                                    ctypes.byref(m), ctypes.byref(params), tau.data_ptr(),
                                    adm_idx.data_ptr(), adm_cnt.data_ptr(), _ptr(bound_out),
                                    _stream(stream)))


def eta_predict_screen_union(q: torch.Tensor, W, bias: torch.Tensor, meta: Meta, T: int,
                             T_cap: int, params: eta_params, tau: torch.Tensor,
                             adm_idx: torch.Tensor, adm_cnt: torch.Tensor, uni_idx: torch.Tensor,
                             uni_cnt: torch.Tensor, bound_out=None, kv_dtype=torch.bfloat16,
                             stream=None, layout: KVLayout | None = None):
    """Grouped heads: eta_predict_screen and eta_admit_union in one launch."""
    B, H, d = q.shape
    H_kv = uni_idx.shape[1]
    s = make_shape(B, H, d, T, T_cap, kv_dtype, H_kv, _lens_only(layout))
    n = nblk_cap(T_cap)
    _need(q, "q", torch.float32)
    if W is not None:
        _need(W, "W", torch.float32, (H * d, H))
    _need(bias, "bias", torch.float32, (H,))
    _need(tau, "tau", torch.float32, (B, H))
    _check_meta(meta, B, H_kv, d, T_cap)
    _need(adm_idx, "adm_idx", torch.int32, (B, H, n))
    _need(adm_cnt, "adm_cnt", torch.int32, (B, H))
    _need(uni_idx, "uni_idx", torch.int32, (B, H_kv, n))
    _need(uni_cnt, "uni_cnt", torch.int32, (B, H_kv))
    if bound_out is not None:
        _need(bound_out, "bound_out", torch.float32, (B, H, n))
    m = meta.c()
    _check("eta_predict_screen_union",
           lib().eta_predict_screen_union(ctypes.byref(s), q.data_ptr(), _ptr(W), bias.data_ptr(),
                                          ctypes.byref(m), ctypes.byref(params), tau.data_ptr(),
                                          adm_idx.data_ptr(), adm_cnt.data_ptr(),
                                          uni_idx.data_ptr(), uni_cnt.data_ptr(),
                                          _ptr(bound_out), _stream(stream)))


def eta_admit_union(adm_idx: torch.Tensor, adm_cnt: torch.Tensor, uni_idx: torch.Tensor,
                    uni_cnt: torch.Tensor, T: int, T_cap: int, d: int, kv_dtype=torch.bfloat16,
                    stream=None):
    """Union of each key/value head's query-head lists ([B,H,n] -> [B,H_kv,n])."""
    B, H, n = adm_idx.shape
    H_kv = uni_idx.shape[1]
    s = make_shape(B, H, d, T, T_cap, kv_dtype, H_kv)
    _need(adm_idx, "adm_idx", torch.int32, (B, H, nblk_cap(T_cap)))
    _need(adm_cnt, "adm_cnt", torch.int32, (B, H))
    _need(uni_idx, "uni_idx", torch.int32, (B, H_kv, nblk_cap(T_cap)))
    _need(uni_cnt, "uni_cnt", torch.int32, (B, H_kv))
    _check("eta_admit_union",
           lib().eta_admit_union(ctypes.byref(s), adm_idx.data_ptr(), adm_cnt.data_ptr(),
                                 uni_idx.data_ptr(), uni_cnt.data_ptr(), _stream(stream)))


def eta_decode_attn_workspace_size(B, H, d, T_cap, params: eta_params,
                                   kv_dtype=torch.bfloat16, H_kv: int = 0) -> int:
    s = make_shape(B, H, d, 0, T_cap, kv_dtype, H_kv)
    return int(lib().eta_decode_attn_workspace_size(ctypes.byref(s), ctypes.byref(params)))


def alloc_workspace(B, H, d, T_cap, params: eta_params, kv_dtype=torch.bfloat16,
                    device="cuda", H_kv: int = 0) -> torch.Tensor:
    n = eta_decode_attn_workspace_size(B, H, d, T_cap, params, kv_dtype, H_kv)
    if n == 0:
        raise EtaError("eta_decode_attn_workspace_size", ETA_ERR_INVALID_ARG, "invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _lens_only(layout: KVLayout | None) -> KVLayout | None:
    return None if layout is None or layout.seq_lens is None else KVLayout(layout.seq_lens)


def attn_shape(q: torch.Tensor, K: torch.Tensor, T: int,
               layout: KVLayout | None = None) -> eta_shape:
    """Shape of an attention call: H query heads from q, H_kv key/value heads from K."""
    B, H_kv, T_cap, d, P = kv_dims(K, layout)
    H = q.shape[1]
    return make_shape(B, H, d, T, T_cap, K.dtype, H_kv if H_kv != H else 0, layout, P,
                      kv_block_stride(K))


NOALLOC_SCRATCH_BYTES = 128 << 20  # ETA_NOALLOC_SCRATCH_BYTES


def _attn_checks(q, K, V, T, tau, adm_idx, adm_cnt, out, lse, ws, layout=None):
    _check_kv(K)
    _check_kv(V, "V")
    if V.shape != K.shape or V.dtype != K.dtype or V.stride() != K.stride():
        raise ValueError("K and V must have the same shape, strides and dtype")
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d]")
    s = attn_shape(q, K, T, layout)
    n = nblk_cap(s.T_cap)
    H_kv = K.shape[1]
    _need(q, "q", torch.float32, (s.B, s.H, s.d))
    _need(tau, "tau", torch.float32, (s.B, s.H))
    _need(adm_idx, "adm_idx", torch.int32, (s.B, H_kv, n))
    _need(adm_cnt, "adm_cnt", torch.int32, (s.B, H_kv))
    _need(out, "out", torch.float32, (s.B, s.H, s.d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (s.B, s.H))
    if ws is not None:
        _need(ws, "ws", torch.uint8)
    return s


def eta_decode_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, T: int,
                    tau: torch.Tensor, adm_idx: torch.Tensor, adm_cnt: torch.Tensor,
                    params: eta_params, out: torch.Tensor, lse, ws: torch.Tensor, stream=None,
                    layout: KVLayout | None = None):
    s = _attn_checks(q, K, V, T, tau, adm_idx, adm_cnt, out, lse, ws, layout)
    _check("eta_decode_attn",
           lib().eta_decode_attn(ctypes.byref(s), q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                 tau.data_ptr(), adm_idx.data_ptr(), adm_cnt.data_ptr(),
                                 ctypes.byref(params), out.data_ptr(), _ptr(lse),
                                 ws.data_ptr(), ws.numel(), _stream(stream)))


def eta_decode_attn_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, T: int,
                            tau: torch.Tensor, adm_idx: torch.Tensor, adm_cnt: torch.Tensor,
                            params: eta_params, out: torch.Tensor, lse, stream=None,
                            layout: KVLayout | None = None):
    """eta_decode_attn with the library's own per-GPU workspace (no allocation by the
    library or here). Calls that overlap in time on one GPU race."""
    s = _attn_checks(q, K, V, T, tau, adm_idx, adm_cnt, out, lse, None, layout)
    st = lib().eta_decode_attn_noalloc(ctypes.byref(s), q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                       tau.data_ptr(), adm_idx.data_ptr(), adm_cnt.data_ptr(),
                                       ctypes.byref(params), out.data_ptr(), _ptr(lse),
                                       _stream(stream))
    if st == ETA_ERR_WORKSPACE:
        need = lib().eta_decode_attn_workspace_size(ctypes.byref(s), ctypes.byref(params))
        raise EtaError("eta_decode_attn_noalloc", st,
                       f"this shape needs {need} bytes of workspace, more than the "
                       f"{NOALLOC_SCRATCH_BYTES} the library holds per GPU")
    _check("eta_decode_attn_noalloc", st)


def eta_decode_attn_partial(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, T: int,
                            tau: torch.Tensor, adm_idx: torch.Tensor, adm_cnt: torch.Tensor,
                            params: eta_params, out: torch.Tensor, lse, ws: torch.Tensor,
                            stream=None, layout: KVLayout | None = None):
    s = _attn_checks(q, K, V, T, tau, adm_idx, adm_cnt, out, lse, ws, layout)
    _check("eta_decode_attn_partial",
           lib().eta_decode_attn_partial(ctypes.byref(s), q.data_ptr(), K.data_ptr(),
                                         V.data_ptr(), tau.data_ptr(), adm_idx.data_ptr(),
                                         adm_cnt.data_ptr(), ctypes.byref(params),
                                         out.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(),
                                         _stream(stream)))


def eta_decode_attn_combine(K: torch.Tensor, T: int, adm_cnt: torch.Tensor, params: eta_params,
                            out: torch.Tensor, lse, ws: torch.Tensor, stream=None,
                            layout: KVLayout | None = None):
    _check_kv(K)
    if out.dim() != 3:
        raise ValueError("out must be [B,H,d]")
    s = attn_shape(out, K, T, layout)
    _need(adm_cnt, "adm_cnt", torch.int32, (s.B, K.shape[1]))
    _need(out, "out", torch.float32, (s.B, s.H, s.d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (s.B, s.H))
    _need(ws, "ws", torch.uint8)
    _check("eta_decode_attn_combine",
           lib().eta_decode_attn_combine(ctypes.byref(s), adm_cnt.data_ptr(),
                                         ctypes.byref(params), out.data_ptr(), _ptr(lse),
                                         ws.data_ptr(), ws.numel(), _stream(stream)))


# ------------------------------------------------------------------------------------
# Training-time (prefill) forward
# ------------------------------------------------------------------------------------
def prefill_shape(Q: torch.Tensor, K: torch.Tensor) -> eta_prefill_shape:
    """Q [B,H,T_q,d] and K [B,H_kv,T_k,d] (bfloat16) -> the C shape descriptor."""
    if Q.dim() != 4 or K.dim() != 4:
        raise ValueError("Q must be [B,H,T_q,d] and K [B,H_kv,T_k,d]")
    B, H, T_q, d = Q.shape
    B2, H_kv, T_k, d2 = K.shape
    if B2 != B or d2 != d:
        raise ValueError("Q and K disagree on B or d")
    return eta_prefill_shape(int(B), int(H), int(H_kv if H_kv != H else 0), int(d), int(T_q),
                             int(T_k))


def eta_prefill_predict_tau(Q: torch.Tensor, W, bias: torch.Tensor, tau: torch.Tensor,
                            stream=None):
    """Eq. 1 per query token from bf16 Q [B,H,T,d] -> tau float32 [B,H,T]."""
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    B, H, T, d = Q.shape
    _need(Q, "Q", torch.bfloat16)
    if W is not None:
        _need(W, "W", torch.float32, (H * d, H))
    _need(bias, "bias", torch.float32, (H,))
    _need(tau, "tau", torch.float32, (B, H, T))
    s = eta_prefill_shape(B, H, 0, d, T, T)
    _check("eta_prefill_predict_tau",
           lib().eta_prefill_predict_tau(ctypes.byref(s), Q.data_ptr(), _ptr(W), bias.data_ptr(),
                                         tau.data_ptr(), _stream(stream)))


def eta_prefill_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, tau: torch.Tensor,
                     params: eta_params, out: torch.Tensor, lse=None, gate_sum=None,
                     stream=None):
    """Dense causal gated attention: the T_q queries are the last T_q of the T_k keys."""
    s = prefill_shape(Q, K)
    _need(Q, "Q", torch.bfloat16)
    _need(K, "K", torch.bfloat16)
    _need(V, "V", torch.bfloat16, tuple(K.shape))
    _need(tau, "tau", torch.float32, (s.B, s.H, s.T_q))
    _need(out, "out", torch.float32, (s.B, s.H, s.T_q, s.d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (s.B, s.H, s.T_q))
    if gate_sum is not None:
        _need(gate_sum, "gate_sum", torch.float32, (s.B, s.H, s.T_q))
    _check("eta_prefill_attn",
           lib().eta_prefill_attn(ctypes.byref(s), Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                  tau.data_ptr(), ctypes.byref(params), out.data_ptr(), _ptr(lse),
                                  _ptr(gate_sum), _stream(stream)))
